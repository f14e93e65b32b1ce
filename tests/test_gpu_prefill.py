"""GPU parity of chunked causal (prefill) attention over the latent cache: query l of sequence b at
position pos0 + l attends to cached tokens [0, pos0 + l]. Every checked row is compared with the
oracle's decode of that row's causal prefix (the plain definition, fp64), to the same 2e-3 bar as
decode. Covers binary16, bfloat16 and mixed 4/3-bit caches, head dims 64 and 128, chunk lengths
that take every query grouping (multiples of 4, of 2 only, odd), per-sequence ragged chunks, a
peaked-attention case for the query-key product, and a 2048-query chunk on the LongChat layer."""
import numpy as np
import pytest

import oracle
import rank_kv_cache_amd as sk
from rank_kv_cache_amd import synth

from gpu_support import DeviceLayer, latent_layer, rel_err, say

pytestmark = pytest.mark.gpu
TOL = 2e-3
FRAC = 0.25


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.lib()


def _prefill(L, cache, pos0, chunk, q, bk, bv, chunk_lens=None, bf16=False):
    import torch
    from rank_kv_cache_amd import buffers
    B = cache.batch
    H, d = L.num_heads, L.head_dim
    out = torch.full((B, chunk, H, d), float("nan"), dtype=torch.float32, device="cuda")
    nws = sk.starkv_prefill_workspace_bytes(L, B, pos0, chunk)
    assert nws > 0
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    dl = None if chunk_lens is None else torch.tensor(np.asarray(chunk_lens, np.int32), device="cuda")
    dbk = bk if hasattr(bk, "data_ptr") else buffers.to_device(bk, bf16=bf16)
    dbv = bv if hasattr(bv, "data_ptr") else buffers.to_device(bv, bf16=bf16)
    sk.starkv_prefill_attn(L, cache, pos0, chunk, dl, buffers.to_device(np.ascontiguousarray(q, np.float32)),
                           dbk, dbv, out, ws, nws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_rows(got, pos0, chunk_lens, ref_row, rows, what):
    worst = 0.0
    for b, l in rows:
        if l >= chunk_lens[b]:
            assert np.all(got[b, l] == 0), (what, b, l)
            continue
        want = ref_row(b, l, pos0 + l + 1)
        e = rel_err(got[b, l], want)
        worst = max(worst, e)
        assert np.all(np.isfinite(got[b, l])) and e <= TOL, (what, b, l, e)
    say(f"[prefill] {what}: {len(rows)} rows, worst {worst:.3e}")
    return worst


def _latent_case(dtype, d, ranks, rv, B, pos0, chunk, seed, scale_q=1.0):
    H = len(ranks)
    T = pos0 + chunk
    w = synth.Workload(f"pf{seed}", batch=B, heads=H, head_dim=d, seq_len=T, dtype=dtype,
                       layer_seed=seed, cache_seed=seed + 1, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = np.random.default_rng(seed + 2).standard_normal((B, chunk, H, d)).astype(np.float32) * scale_q
    return ld, zk, zv, q


@pytest.mark.parametrize("dtype,d,chunk,pos0", [("f16", 128, 64, 0), ("f16", 128, 70, 37),
                                                ("bf16", 128, 33, 130), ("f16", 64, 100, 5),
                                                ("bf16", 64, 97, 64), ("bf16", 128, 64, 10),
                                                ("f16", 128, 64, 1000)])
def test_prefill_latent_every_row(dtype, d, chunk, pos0):
    """Every row of small chunks: the first tokens of a prompt (pos0 0), a chunk after a cached
    prefix, chunk lengths whose query grouping is 4 (64, 100), 2 (70) and 1 (33, 97), and a
    chunk after a 1000-token prefix (the value side then splits the sequence)."""
    ranks = [16, 48, 32, 64] if d == 128 else [16, 32, 48, 64]
    rv = 160
    B = 2
    ld, zk, zv, q = _latent_case(dtype, d, ranks, rv, B, pos0, chunk, 500 + chunk + pos0)
    L = latent_layer(len(ranks), d, ranks, rv, dtype)
    dev = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
    bf16 = dtype == "bf16"
    got = _prefill(L, dev.cache, pos0, chunk, q, dev.bk, dev.bv, bf16=bf16)
    rows = [(b, l) for b in range(B) for l in range(chunk)]
    _check_rows(got, pos0, [chunk] * B,
                lambda b, l, n: oracle.decode_latent(zk[b:b + 1, :n], zv[b:b + 1, :n], ld.bk, ld.bv,
                                                     q[b:b + 1, l], ranks, bf16=bf16)[0],
                rows, f"{dtype} d={d} chunk={chunk} pos0={pos0}")


@pytest.mark.parametrize("dtype,ranks,rv,chunk,pos0", [
    ("f16", [24, 40, 12, 100], 100, 45, 19),
    ("f16", [16, 48, 32, 64], 160, 1, 0),
    ("bf16", [16, 48, 32, 64], 96, 1, 200),
])
def test_prefill_edge_shapes(dtype, ranks, rv, chunk, pos0):
    """Key ranks off the 16-channel step and a value rank of 100 (stored rounded up to 112, the
    value chunks then end in zero rows); a one-query chunk at position 0 (the first token attends
    to itself alone) and after a 200-token prefix."""
    d, B = 128, 2
    ld, zk, zv, q = _latent_case(dtype, d, ranks, rv, B, pos0, chunk, 700 + chunk + pos0)
    L = latent_layer(len(ranks), d, ranks, rv, dtype)
    dev = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
    bf16 = dtype == "bf16"
    got = _prefill(L, dev.cache, pos0, chunk, q, dev.bk, dev.bv, bf16=bf16)
    rows = [(b, l) for b in range(B) for l in range(chunk)]
    _check_rows(got, pos0, [chunk] * B,
                lambda b, l, n: oracle.decode_latent(zk[b:b + 1, :n], zv[b:b + 1, :n], ld.bk, ld.bv,
                                                     q[b:b + 1, l], ranks, bf16=bf16)[0],
                rows, f"{dtype} ranks={ranks} rv={rv} chunk={chunk} pos0={pos0}")


def test_prefill_ragged_chunks():
    """Per-sequence chunk lengths (0, 1, 31, 64 of a 64-query call): rows past a sequence's chunk
    are empty and give zeros."""
    ranks, rv, d, B, pos0, chunk = [32, 16, 64], 96, 128, 4, 50, 64
    ld, zk, zv, q = _latent_case("f16", d, ranks, rv, B, pos0, chunk, 610)
    L = latent_layer(len(ranks), d, ranks, rv, "f16")
    dev = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
    lens = [0, 1, 31, 64]
    got = _prefill(L, dev.cache, pos0, chunk, q, dev.bk, dev.bv, chunk_lens=lens)
    rows = [(b, l) for b in range(B) for l in range(chunk)]
    _check_rows(got, pos0, lens,
                lambda b, l, n: oracle.decode_latent(zk[b:b + 1, :n], zv[b:b + 1, :n], ld.bk, ld.bv,
                                                     q[b:b + 1, l], ranks)[0],
                rows, "ragged chunks")


def test_prefill_peaked_attention():
    """Queries eight times larger: sharp attention, where the error of the query-key product
    shows up directly in the probabilities."""
    ranks, rv, d, B, pos0, chunk = [64, 48, 16, 32], 128, 128, 1, 90, 40
    ld, zk, zv, q = _latent_case("f16", d, ranks, rv, B, pos0, chunk, 620, scale_q=8.0)
    L = latent_layer(len(ranks), d, ranks, rv, "f16")
    dev = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
    got = _prefill(L, dev.cache, pos0, chunk, q, dev.bk, dev.bv)
    rows = [(0, l) for l in range(chunk)]
    _check_rows(got, pos0, [chunk],
                lambda b, l, n: oracle.decode_latent(zk[b:b + 1, :n], zv[b:b + 1, :n], ld.bk, ld.bv,
                                                     q[b:b + 1, l], ranks)[0],
                rows, "peaked (q x 8)")


@pytest.mark.parametrize("pos0,chunk,d", [(0, 128, 128), (100, 92, 128), (64, 64, 128), (64, 64, 64)])
def test_prefill_q43(pos0, chunk, d):
    """Mixed 4/3-bit cache holding exactly the prefix plus the chunk (so its partial last group is
    in the tail): every row against the oracle's quantise / dequantise of the same rows; head dims
    128 and 64."""
    from test_gpu_q43 import _append, q43_layer
    from rank_kv_cache_amd import buffers
    ranks, rv, B = ([16, 64, 32, 48] if d == 128 else [16, 32, 48, 64]), 96, 2
    T = pos0 + chunk
    cap = ((T + 63) // 64) * 64 + 64
    ld, zk, zv, q = _latent_case("f16", d, ranks, rv, B, pos0, chunk, 630 + pos0 + d)
    L = q43_layer(len(ranks), d, ranks, rv)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    _append(L, cache, zk, zv, [T])
    got = _prefill(L, cache, pos0, chunk, q, ld.bk, ld.bv)
    bits_k, bits_v = oracle.channel_bits(ranks, FRAC), oracle.channel_bits([rv], FRAC)
    deq = []
    for b in range(B):
        ck, mk, tk = oracle.q43_pack(zk[b:b + 1], bits_k, cap)
        cv, mv, tv = oracle.q43_pack(zv[b:b + 1], bits_v, cap)
        deq.append((oracle.q43_unpack(ck, mk, tk, bits_k, T, cap), oracle.q43_unpack(cv, mv, tv, bits_v, T, cap)))
    rows = [(b, l) for b in range(B) for l in range(chunk)]
    _check_rows(got, pos0, [chunk] * B,
                lambda b, l, n: oracle.decode_latent(deq[b][0][:, :n], deq[b][1][:, :n], ld.bk, ld.bv,
                                                     q[b:b + 1, l], ranks)[0],
                rows, f"q43 d={d} pos0={pos0} chunk={chunk}")


def test_prefill_longchat_chunk_2048_sampled():
    """A 2048-query chunk on the LongChat-shaped layer (32 heads, key ranks U{16..64}, r_v 1024,
    binary16), sampled rows including the first and the last, in the library's default
    configuration."""
    w = synth.WORKLOADS["longchat_b16_t4096_f16"]
    chunk, pos0 = 2048, 0
    ld = synth.draw_layer(w)
    zk, zv = synth.draw_latent_cache(w, ld, batches=[0], seq_len=chunk)
    ranks, rv = ld.key_ranks, ld.value_rank
    H, d = w.heads, w.head_dim
    q = np.random.default_rng(640).standard_normal((1, chunk, H, d)).astype(np.float32)
    L = latent_layer(H, d, ranks, rv, "f16")
    dev = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
    got = _prefill(L, dev.cache, pos0, chunk, q, dev.bk, dev.bv)
    rng = np.random.default_rng(641)
    rows = [(0, 0), (0, 1), (0, 31), (0, 32), (0, 1023), (0, chunk - 1)] + \
           [(0, int(l)) for l in rng.integers(0, chunk, 6)]
    _check_rows(got, pos0, [chunk],
                lambda b, l, n: oracle.decode_latent(zk[:, :n], zv[:, :n], ld.bk, ld.bv, q[:, l], ranks)[0],
                rows, "longchat chunk 2048")


def test_prefill_q43_ragged():
    """Mixed 4/3-bit cache filled per sequence to pos0 + chunk_len(b) (groups complete at different
    tokens in different sequences, partial groups in the tails): every row against the oracle's
    quantise / dequantise of that sequence's own rows; rows past a sequence's chunk are zero."""
    from test_gpu_q43 import q43_layer
    from test_gpu_ragged import _ragged_fill
    from rank_kv_cache_amd import buffers
    ranks, rv, d, B, pos0, chunk = [16, 64, 32, 48], 96, 128, 4, 100, 92
    lens = [0, 45, 92, 7]
    fills = [pos0 + n for n in lens]
    cap = 256
    ld, zk, zv, q = _latent_case("f16", d, ranks, rv, B, pos0, chunk, 650)
    L = q43_layer(len(ranks), d, ranks, rv)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    _ragged_fill(L, cache, zk, zv, fills)
    got = _prefill(L, cache, pos0, chunk, q, ld.bk, ld.bv, chunk_lens=lens)
    bits_k, bits_v = oracle.channel_bits(ranks, FRAC), oracle.channel_bits([rv], FRAC)
    deq = []
    for b, n in enumerate(fills):
        ck, mk, tk = oracle.q43_pack(zk[b:b + 1, :n], bits_k, cap)
        cv, mv, tv = oracle.q43_pack(zv[b:b + 1, :n], bits_v, cap)
        deq.append((oracle.q43_unpack(ck, mk, tk, bits_k, n, cap), oracle.q43_unpack(cv, mv, tv, bits_v, n, cap)))
    rows = [(b, l) for b in range(B) for l in range(chunk)]
    _check_rows(got, pos0, lens,
                lambda b, l, n: oracle.decode_latent(deq[b][0][:, :n], deq[b][1][:, :n], ld.bk, ld.bv,
                                                     q[b:b + 1, l], ranks)[0],
                rows, "q43 ragged fills")


@pytest.mark.parametrize("dtype", ["f16", "q43"])
def test_prefill_paged(dtype):
    """A paged cache (shuffled block table, poisoned spare pages) gives the same outputs as the
    contiguous cache bit for bit, and matches the oracle; binary16 with ragged chunks, mixed
    4/3-bit with full ones."""
    from test_gpu_paged import paged_cache, _append_chunks
    from test_gpu_q43 import q43_layer
    from rank_kv_cache_amd import buffers
    ranks, rv, d, B, pos0, chunk = [32, 16, 48], 80, 128, 3, 70, 64
    T = pos0 + chunk
    cap = 192
    lens = [20, 64, 50] if dtype == "f16" else None
    ld, zk, zv, q = _latent_case("f16", d, ranks, rv, B, pos0, chunk, 660 + (dtype == "q43"))
    L = q43_layer(len(ranks), d, ranks, rv) if dtype == "q43" else latent_layer(len(ranks), d, ranks, rv, "f16")
    flat = buffers.alloc_cache(L, B, cap, fill=0xFF)
    paged, keep = paged_cache(L, B, cap, 661)
    for c in (flat, paged):
        _append_chunks(L, c, zk, zv, [pos0, chunk])
    a = _prefill(L, flat, pos0, chunk, q, ld.bk, ld.bv, chunk_lens=lens)
    b_ = _prefill(L, paged, pos0, chunk, q, ld.bk, ld.bv, chunk_lens=lens)
    assert np.array_equal(a.view(np.uint32), b_.view(np.uint32))
    lens_ = lens or [chunk] * B
    if dtype == "q43":
        bits_k, bits_v = oracle.channel_bits(ranks, FRAC), oracle.channel_bits([rv], FRAC)
        ck, mk, tk = oracle.q43_pack(zk, bits_k, cap)
        cv, mv, tv = oracle.q43_pack(zv, bits_v, cap)
        rk_, rv_ = oracle.q43_unpack(ck, mk, tk, bits_k, T, cap), oracle.q43_unpack(cv, mv, tv, bits_v, T, cap)
    else:
        rk_, rv_ = zk, zv
    rows = [(b, l) for b in range(B) for l in range(chunk)]
    _check_rows(a, pos0, lens_,
                lambda b, l, n: oracle.decode_latent(rk_[b:b + 1, :n], rv_[b:b + 1, :n], ld.bk, ld.bv,
                                                     q[b:b + 1, l], ranks)[0],
                rows, f"paged {dtype}")
