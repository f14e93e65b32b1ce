"""GPU parity of latent-cache decode attention against the fp64 oracle (through the C ABI).

Tolerance (from the decode contract): max |gpu - oracle| <= 2e-3 * RMS(oracle) for fp32 / fp16 /
bf16 latents. Every case prints its name, shape and measured error before asserting.
"""
import numpy as np
import pytest

import oracle
from rank_kv_cache_amd import synth

from gpu_support import DeviceLayer, latent_layer, rel_err, say, workload_arrays

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_kv_cache_amd as sk
    sk.lib()


def _oracle(ld, zk, zv, q, dtype, **kw):
    return oracle.decode_latent(zk, zv, ld.bk, ld.bv, q, ld.key_ranks, bf16=(dtype == "bf16"), **kw)


def test_tiny_f32_full():
    w = synth.WORKLOADS["tiny_b1_h4_d64_t256_f32"]
    ld, zk, zv, q = workload_arrays(w)
    say(f"[tiny] B={w.batch} H={w.heads} d={w.head_dim} T={w.seq_len} f32")
    dl = DeviceLayer(latent_layer(w.heads, w.head_dim, ld.key_ranks, ld.value_rank, "f32"),
                     zk, zv, ld.bk, ld.bv)
    got = dl.decode(q)
    ref = _oracle(ld, zk, zv, q, "f32")
    e = rel_err(got, ref)
    say(f"[tiny] rel err {e:.3e}")
    assert e <= TOL
    assert e <= 1e-4          # fp32 latents: much tighter than the contract


def test_longchat_t4096_full():
    w = synth.WORKLOADS["longchat_b16_t4096_f16"]
    ld, zk, zv, q = workload_arrays(w)
    say(f"[longchat4k] ranks={ld.key_ranks.tolist()} r_v={ld.value_rank}")
    dl = DeviceLayer(latent_layer(w.heads, w.head_dim, ld.key_ranks, ld.value_rank, "f16"),
                     zk, zv, ld.bk, ld.bv)
    got = dl.decode(q)
    ref = _oracle(ld, zk, zv, q, "f16")
    e = rel_err(got, ref)
    say(f"[longchat4k] rel err {e:.3e}")
    assert e <= TOL
    for S in (1, 2, 7):
        g2 = dl.decode(q, num_splits=S)
        e2 = rel_err(g2, ref)
        say(f"[longchat4k] splits={S} rel err {e2:.3e}")
        assert e2 <= TOL
    runs = dl.decode(q, repeat=3)
    assert all(np.array_equal(runs[0], r) for r in runs[1:]), "decode is not bitwise deterministic"


def test_longchat_t32768_sampled():
    """Full-size long-context workload in the benchmark's launch configuration; the oracle
    evaluates sampled (b, h) pairs one by one."""
    w = synth.WORKLOADS["longchat_b16_t32768_f16"]
    ld, zk, zv, q = workload_arrays(w)
    say(f"[longchat32k] generated {zk.nbytes / 1e9:.2f}+{zv.nbytes / 1e9:.2f} GB")
    dl = DeviceLayer(latent_layer(w.heads, w.head_dim, ld.key_ranks, ld.value_rank, "f16"),
                     zk, zv, ld.bk, ld.bv)
    got = dl.decode(q)
    rng = np.random.default_rng(123)
    pairs = [(0, 0), (w.batch - 1, w.heads - 1)] + [(int(b), int(h)) for b, h in
                                                      zip(rng.integers(0, w.batch, 10), rng.integers(0, w.heads, 10))]
    ref = _oracle(ld, zk, zv, q, "f16", pairs=pairs)
    sub = np.stack([got[b, h] for b, h in pairs])
    e = rel_err(sub, ref)
    say(f"[longchat32k] sampled {len(pairs)} pairs rel err {e:.3e}")
    assert e <= TOL
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("dtype,d", [("f16", 128), ("bf16", 128), ("f32", 128), ("f16", 64),
                                     ("bf16", 64), ("f32", 64)])
def test_dtypes_and_head_dims(dtype, d):
    rng = np.random.default_rng({"f16": 1, "bf16": 2, "f32": 3}[dtype] * 1000 + d)
    H, B, T = 12, 3, 700
    ranks = rng.choice(np.arange(16, d + 1, 16), size=H)
    rv = 272           # ragged last value column tile (272 = 8.5 * 32)
    w = synth.Workload("t", batch=B, heads=H, head_dim=d, seq_len=T, dtype=dtype, layer_seed=11,
                       cache_seed=12, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(12, 0, B, H, d)
    say(f"[dtype] {dtype} d={d} ranks={ranks.tolist()} rv={rv} T={T}")
    dl = DeviceLayer(latent_layer(H, d, ranks, rv, dtype), zk, zv, ld.bk, ld.bv, capacity=768)
    got = dl.decode(q)
    ref = _oracle(ld, zk, zv, q, dtype)
    e = rel_err(got, ref)
    say(f"[dtype] {dtype} d={d} rel err {e:.3e}")
    assert e <= TOL


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 129, 320])
def test_edge_lengths_poisoned_cache(T):
    """Ragged tails: every byte past seq_len is NaN; the kernels must never read it into a sum."""
    H, B, d, rv = 6, 2, 128, 96
    ranks = [16, 64, 32, 48, 128, 16]
    w = synth.Workload("e", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=21,
                       cache_seed=22 + T, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(22 + T, 0, B, H, d)
    dl = DeviceLayer(latent_layer(H, d, ranks, rv, "f16"), zk, zv, ld.bk, ld.bv, capacity=384)
    for S in (0, 1, 3):
        got = dl.decode(q, num_splits=S)
        ref = _oracle(ld, zk, zv, q, "f16")
        e = rel_err(got, ref)
        say(f"[edge] T={T} splits={S} rel err {e:.3e}")
        assert np.all(np.isfinite(got)) and e <= TOL
    # attending to a prefix of what is cached
    if T > 1:
        got = dl.decode(q, seq_len=T - 1)
        ref = _oracle(ld, zk, zv, q, "f16", seq_len=T - 1)
        assert rel_err(got, ref) <= TOL


def test_peaked_attention_and_custom_scale():
    """Scaled-up queries make attention peaked; a non-default base and scale exercise the RoPE
    table and the softmax scale."""
    H, B, d, T, rv = 8, 2, 128, 1000, 512
    rng = np.random.default_rng(5)
    ranks = rng.choice([16, 32, 48, 64], size=H)
    w = synth.Workload("p", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=31,
                       cache_seed=32, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(32, 0, B, H, d) * 8.0
    dl = DeviceLayer(latent_layer(H, d, ranks, rv, "f16"), zk, zv, ld.bk, ld.bv)
    e = rel_err(dl.decode(q), _oracle(ld, zk, zv, q, "f16"))
    say(f"[peaked] rel err {e:.3e}")
    assert e <= TOL
    dl2 = DeviceLayer(latent_layer(H, d, ranks, rv, "f16", rope_base=500000.0, sm_scale=0.05),
                      zk, zv, ld.bk, ld.bv)
    e2 = rel_err(dl2.decode(q), _oracle(ld, zk, zv, q, "f16", rope_base=500000.0, scale=0.05))
    say(f"[base/scale] rel err {e2:.3e}")
    assert e2 <= TOL


# Rank mixes: all heads at most 64 (the twelve-wave score kernel holds a unit in registers), a few
# heads above 64 among rank-16 heads, and mostly large ranks (second column tile loaded inside the
# unit); each at a length with a ragged last block, with and without split-K.
@pytest.mark.parametrize("name,ranks", [
    ("small", [16, 32, 48, 64, 32, 16]),
    ("mixed", [16, 96, 16, 16, 128, 16, 16, 64]),
    ("large", [64, 80, 96, 64, 48, 128]),
])
def test_rank_mixes(name, ranks):
    H, B, d, rv = len(ranks), 2, 128, 160
    for T in (1000, 4161):
        w = synth.Workload("k", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16",
                           layer_seed=41, cache_seed=42 + T, value_rank=rv, power=0.5)
        ld = synth.draw_layer(w, key_ranks=ranks)
        zk, zv = synth.draw_latent_cache(w, ld)
        q = synth.draw_queries(43 + T, 0, B, H, d)
        dl = DeviceLayer(latent_layer(H, d, ranks, rv, "f16"), zk, zv, ld.bk, ld.bv)
        for S in (0, 3):
            got = dl.decode(q, num_splits=S)
            e = rel_err(got, _oracle(ld, zk, zv, q, "f16"))
            say(f"[ranks] {name} mean rank {np.mean(ranks):.1f} T={T} splits={S} rel err {e:.3e}")
            assert np.all(np.isfinite(got)) and e <= TOL


def test_append_chunks_and_readback():
    """Cache built by many appends (prefill, then one token at a time) is byte-identical to the
    input rows, and attends identically."""
    H, B, d, T, rv = 4, 3, 128, 200, 128
    ranks = [32, 16, 64, 48]
    w = synth.Workload("a", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=41,
                       cache_seed=42, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(42, 0, B, H, d)
    L = latent_layer(H, d, ranks, rv, "f16")
    bulk = DeviceLayer(L, zk, zv, ld.bk, ld.bv, capacity=256)
    chunks = [61, 3, 64, 70] + [1] * 2
    inc = DeviceLayer(L, zk, zv, ld.bk, ld.bv, capacity=256, chunks=chunks)
    rk, rv_ = inc.readback(0, T)
    assert np.array_equal(rk.view(np.uint16), zk.view(np.uint16))
    assert np.array_equal(rv_.view(np.uint16), zv.view(np.uint16))
    rk2, rv2 = inc.readback(37, 171)
    assert np.array_equal(rk2.view(np.uint16), zk[:, 37:171].view(np.uint16))
    assert np.array_equal(rv2.view(np.uint16), zv[:, 37:171].view(np.uint16))
    assert np.array_equal(bulk.decode(q), inc.decode(q))


def test_all_negative_scores():
    """Keys that point against the back-rotated query at every position: z_n solves
    B^T z = -u_n R_n^T q in the least-squares sense (u_n in [0.3, 3]), so every score
    (R_n^T q) . (B^T z_n) is minus a squared norm and each 32-token tile's maximum is negative
    (the kernel takes the tile maxima over order-preserving integer keys of the float scores,
    whose negative half has its magnitude bits flipped)."""
    H, B, d, T, rv = 2, 1, 128, 300, 64
    ranks = np.array([32, 48])
    w = synth.Workload("n", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=51,
                       cache_seed=52, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(53, 0, B, H, d)
    rng = np.random.default_rng(54)
    zk = zk.astype(np.float64)
    off = 0
    smax = -np.inf
    for h, r in enumerate(ranks):
        bh = np.asarray(ld.bk[off:off + r], dtype=np.float64)          # (r, d)
        for n in range(T):
            qn = oracle.rope(np.asarray(q[0, h], dtype=np.float64), -n)  # R_n^T q
            zk[0, n, off:off + r] = -rng.uniform(0.3, 3.0) * np.linalg.lstsq(bh.T, qn, rcond=None)[0]
        z16 = zk[0, :, off:off + r].astype(np.float16).astype(np.float64)
        for n in range(T):
            smax = max(smax, float(oracle.rope(np.asarray(q[0, h], dtype=np.float64), -n) @ (bh.T @ z16[n])))
        off += r
    zk = zk.astype(np.float16)
    say(f"[negative] largest score {smax:.3f}")
    assert smax < 0.0
    dl = DeviceLayer(latent_layer(H, d, ranks, rv, "f16"), zk, zv, ld.bk, ld.bv)
    e = rel_err(dl.decode(q), _oracle(ld, zk, zv, q, "f16"))
    say(f"[negative] rel err {e:.3e}")
    assert e <= TOL
