"""GPU parity for ragged batches (serving): decode where every sequence has its own length, and
the one-token-per-sequence append at per-sequence positions (idle slots skipped). Each sequence
is checked against the oracle on its own prefix; a sequence of length 0 must give zeros. Ragged
caches are read back per sequence through single-sequence views of the batch buffers."""
import numpy as np
import pytest

import oracle
import rank_kv_cache_amd as sk
from rank_kv_cache_amd import synth

from gpu_support import DeviceLayer, dense_layer, latent_layer, rel_err, say

pytestmark = pytest.mark.gpu
TOL = 2e-3
FRAC = 0.25


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.lib()


def _ragged_decode(L, cache, lens, q, bk, bv, num_splits=0, bf16=False):
    import torch
    from rank_kv_cache_amd import buffers
    B = cache.batch
    T = int(max(lens))
    d_lens = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    nws = sk.starkv_decode_workspace_bytes(L, B, T, num_splits)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    sk.starkv_decode_attn_ragged(L, cache, T, d_lens, buffers.to_device(np.ascontiguousarray(q, np.float32)),
                                 None if bk is None else buffers.to_device(bk, bf16=bf16),
                                 None if bv is None else buffers.to_device(bv, bf16=bf16),
                                 out, num_splits, ws, nws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _seq_view(L, cache, b):
    """A batch-1 view of sequence b of a cache (the buffers are sequence-major)."""
    B = cache.batch
    sizes = sk.starkv_cache_bytes(L, B, cache.capacity)
    pad = 32 if L.cache_dtype == sk.Q43 else 0
    bufs = [cache.zk, cache.zv, cache.zk_meta, cache.zv_meta, cache.zk_tail, cache.zv_tail]
    ptrs = []
    for i, (t, n) in enumerate(zip(bufs, sizes)):
        if t is None or n == 0:
            ptrs.append(None)
            continue
        per = (n - (pad if i < 2 else 0)) // B
        assert per % 16 == 0
        ptrs.append(t.data_ptr() + b * per)
    return sk.Cache(1, cache.capacity, *ptrs)


def _check_rows(lens, got_fn, ref_fn, what):
    for b, n in enumerate(lens):
        got, ref = got_fn(b), ref_fn(b)
        if n == 0:
            assert np.all(got == 0), (what, b)
            continue
        e = rel_err(got, ref)
        say(f"[ragged] {what} b={b} len={n}: {e:.3e}")
        assert np.all(np.isfinite(got)) and e <= TOL, (what, b, n, e)


@pytest.mark.parametrize("dtype,ranks,rv", [("f16", [16, 32, 48, 64], 160), ("bf16", [5, 17, 30, 64], 100),
                                             ("f32", [16, 16, 32, 48], 64)])
def test_ragged_decode_latent(dtype, ranks, rv):
    H, d, B, T = 4, 128, 7, 200
    lens = [1, 63, 64, 65, 130, 200, 0]
    w = synth.Workload("rg", batch=B, heads=H, head_dim=d, seq_len=T, dtype=dtype, layer_seed=161,
                       cache_seed=162, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(163, 0, B, H, d)
    L = latent_layer(H, d, ranks, rv, dtype)
    dl = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
    bf16 = dtype == "bf16"
    for S in (0, 3):
        got = _ragged_decode(L, dl.cache, lens, q, ld.bk, ld.bv, S, bf16)
        _check_rows(lens, lambda b: got[b],
                    lambda b: oracle.decode_latent(zk[b:b + 1, :max(lens[b], 1)], zv[b:b + 1, :max(lens[b], 1)],
                                                   ld.bk, ld.bv, q[b:b + 1], ranks, bf16=bf16)[0],
                    f"{dtype} splits={S}")


def test_ragged_decode_dense():
    H, d, B, T = 8, 64, 5, 150
    lens = [150, 1, 0, 64, 97]
    k, v = synth.draw_dense_cache(171, 0, B, T, H * d, "f16")
    q = synth.draw_queries(172, 0, B, H, d)
    L = dense_layer(H, d, "f16")
    dl = DeviceLayer(L, k, v)
    for S in (0, 2):
        got = _ragged_decode(L, dl.cache, lens, q, None, None, S)
        _check_rows(lens, lambda b: got[b],
                    lambda b: oracle.decode_dense(k[b:b + 1, :max(lens[b], 1)], v[b:b + 1, :max(lens[b], 1)],
                                                  q[b:b + 1])[0], f"dense splits={S}")


def _ragged_fill(L, cache, zk, zv, lens, bf16=False):
    """Append token t of every sequence still shorter than its target length, one step per t."""
    import torch
    from rank_kv_cache_amd import buffers
    dzk, dzv = buffers.to_device(zk, bf16=bf16), buffers.to_device(zv, bf16=bf16)
    for t in range(int(max(lens))):
        pos = torch.tensor([t if t < n else -1 for n in lens], dtype=torch.int32, device="cuda")
        sk.starkv_append_latents_ragged(L, cache, pos, dzk[:, t].contiguous(), dzv[:, t].contiguous())
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,ranks,rv", [("f16", [16, 48], 64), ("f16", [7, 33], 40), ("bf16", [16, 48], 64)])
def test_ragged_append_fp(dtype, ranks, rv):
    import torch
    from rank_kv_cache_amd import buffers
    H, d, B = 2, 128, 4
    lens = [70, 1, 0, 129]
    T = max(lens)
    w = synth.Workload("ra", batch=B, heads=H, head_dim=d, seq_len=T, dtype=dtype, layer_seed=181,
                       cache_seed=182, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(183, 0, B, H, d)
    L = latent_layer(H, d, ranks, rv, dtype)
    bf16 = dtype == "bf16"
    cache = buffers.alloc_cache(L, B, 192, fill=0xFF)
    _ragged_fill(L, cache, zk, zv, lens, bf16)
    tdt = buffers.elem_torch_dtype(L.cache_dtype)
    for b, n in enumerate(lens):
        if n == 0:
            continue
        view = _seq_view(L, cache, b)
        ok = torch.empty((1, n, sum(ranks)), dtype=tdt, device="cuda")
        ov = torch.empty((1, n, rv), dtype=tdt, device="cuda")
        sk.starkv_dequant(L, view, n, 0, n, ok, ov)
        torch.cuda.synchronize()
        assert np.array_equal(buffers.to_host(ok).view(np.uint16), zk[b:b + 1, :n].view(np.uint16)), b
        assert np.array_equal(buffers.to_host(ov).view(np.uint16), zv[b:b + 1, :n].view(np.uint16)), b
    got = _ragged_decode(L, cache, lens, q, ld.bk, ld.bv, 0, bf16)
    _check_rows(lens, lambda b: got[b],
                lambda b: oracle.decode_latent(zk[b:b + 1, :max(lens[b], 1)], zv[b:b + 1, :max(lens[b], 1)],
                                               ld.bk, ld.bv, q[b:b + 1], ranks, bf16=bf16)[0],
                f"ragged append {dtype} ranks={ranks}")


def test_ragged_append_q43():
    """Mixed 4/3-bit cache filled by per-sequence appends: groups complete at different steps in
    different sequences. Each sequence's read-back must equal the oracle's quantise ->
    dequantise of its own rows bit for bit, and ragged decode must match the oracle on them."""
    import torch
    from rank_kv_cache_amd import buffers
    H, d, B, cap = 3, 128, 4, 192
    ranks, rv = [16, 64, 32], 96
    lens = [130, 64, 1, 100]
    T = max(lens)
    w = synth.Workload("rq", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=191,
                       cache_seed=192, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(193, 0, B, H, d)
    L = sk.Layer(num_heads=H, head_dim=d, key_ranks=tuple(ranks), value_rank=rv,
                 cache_dtype=sk.Q43, q_top_fraction=FRAC)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    _ragged_fill(L, cache, zk, zv, lens)
    bits_k, bits_v = oracle.channel_bits(ranks, FRAC), oracle.channel_bits([rv], FRAC)
    deq = {}
    for b, n in enumerate(lens):
        ck, mk, tk = oracle.q43_pack(zk[b:b + 1, :n], bits_k, cap)
        cv, mv, tv = oracle.q43_pack(zv[b:b + 1, :n], bits_v, cap)
        deq[b] = (oracle.q43_unpack(ck, mk, tk, bits_k, n, cap), oracle.q43_unpack(cv, mv, tv, bits_v, n, cap))
        view = _seq_view(L, cache, b)
        ok = torch.empty((1, n, sum(ranks)), dtype=torch.float16, device="cuda")
        ov = torch.empty((1, n, rv), dtype=torch.float16, device="cuda")
        sk.starkv_dequant(L, view, n, 0, n, ok, ov)
        torch.cuda.synchronize()
        assert np.array_equal(ok.cpu().numpy().view(np.uint16), deq[b][0].view(np.uint16)), b
        assert np.array_equal(ov.cpu().numpy().view(np.uint16), deq[b][1].view(np.uint16)), b
    got = _ragged_decode(L, cache, lens, q, ld.bk, ld.bv, 0)
    _check_rows(lens, lambda b: got[b],
                lambda b: oracle.decode_latent(deq[b][0], deq[b][1], ld.bk, ld.bv, q[b:b + 1], ranks)[0],
                "ragged q43")


def test_ragged_append_dense():
    import torch
    from rank_kv_cache_amd import buffers
    H, d, B = 4, 64, 3
    lens = [10, 0, 65]
    k, v = synth.draw_dense_cache(201, 0, B, max(lens), H * d, "f16")
    q = synth.draw_queries(202, 0, B, H, d)
    L = dense_layer(H, d, "f16")
    cache = buffers.alloc_cache(L, B, 128, fill=0xFF)
    _ragged_fill(L, cache, k, v, lens)
    got = _ragged_decode(L, cache, lens, q, None, None, 0)
    _check_rows(lens, lambda b: got[b],
                lambda b: oracle.decode_dense(k[b:b + 1, :max(lens[b], 1)], v[b:b + 1, :max(lens[b], 1)],
                                              q[b:b + 1])[0], "ragged dense append")
