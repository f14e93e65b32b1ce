"""GPU parity of the fused append front-end (Alg. 2 steps 1-3): hidden states projected to key
and value latents on the matrix cores and stored straight into the cache, against the oracle's
fp64 products rounded once to the storage type.

Where the fp32 accumulation of the kernel and the exact product round to different neighbours
(only possible next to a rounding midpoint), both results are valid; the random cases therefore
check that every stored value is a correct rounding up to a tiny accumulation slack, and that such
cases are rare. Exact-arithmetic cases (quarter-integer inputs, small-integer weights) must match
the oracle bit for bit, including the mixed 4/3-bit cache's codes, scales and zero points."""
import numpy as np
import pytest

import oracle
import rank_kv_cache_amd as sk
from rank_kv_cache_amd import synth

from gpu_support import DeviceLayer, dense_layer, latent_layer, rel_err, say

pytestmark = pytest.mark.gpu
FRAC = 0.25
MANT = {"f16": 10, "bf16": 7, "f32": 23}
EMIN = {"f16": -14, "bf16": -126, "f32": -126}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.lib()


def _f64(a, dtype):
    return oracle.to_f64(a, dtype == "bf16")


def _ulp(v, dtype):
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** EMIN[dtype])))
    return 2.0 ** (np.maximum(e, EMIN[dtype]) - MANT[dtype])


def _check_rounding(got, exact, dtype, what):
    """got (storage) is a nearest rounding of exact, up to an fp32-accumulation slack."""
    g = _f64(got, dtype)
    slack = 1e-5 * float(np.max(np.abs(exact)))
    err = np.abs(g - exact)
    assert np.all(err <= 0.5 * _ulp(exact, dtype) + slack), what
    if dtype != "f32":               # fp32 storage keeps the accumulation's own last bits
        ref = _f64(oracle.round_to_storage(exact, dtype), dtype)
        frac = float(np.mean(g != ref))
        say(f"[append_tokens] {what}: {frac:.2e} of values rounded to the other neighbour")
        assert frac <= 0.02, what


def _append_tokens(L, cache, pos, x, a_k, a_v, bf16=False):
    import torch
    from rank_kv_cache_amd import buffers
    B, n, D = x.shape
    nws = sk.starkv_append_tokens_workspace_bytes(L, B, n, D)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    sk.starkv_append_tokens(L, cache, pos, n, buffers.to_device(np.ascontiguousarray(x, np.float32)),
                            D, buffers.to_device(a_k, bf16=bf16), buffers.to_device(a_v, bf16=bf16),
                            ws, nws)
    torch.cuda.synchronize()


def _weights(rng, rows, cols, dtype):
    return synth._store((rng.standard_normal((rows, cols)) / np.sqrt(cols)).astype(np.float32), dtype)


def _exact_inputs(rng, B, n, D, Ck, Cv, dtype):
    x = (rng.integers(-4, 5, (B, n, D)) * 0.25).astype(np.float32)
    a_k = synth._store(rng.integers(-3, 4, (Ck, D)).astype(np.float32), dtype)
    a_v = synth._store(rng.integers(-3, 4, (Cv, D)).astype(np.float32), dtype)
    return x, a_k, a_v


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_append_tokens_latent(dtype):
    """Appends of 30 tokens (across a 64-token block boundary) and then one token after 100
    tokens stored by starkv_append_latents; the earlier tokens must be untouched."""
    H, d, B, T0, D = 4, 128, 3, 100, 512
    ranks, rv = [16, 32, 48, 64], 160
    w = synth.Workload("at", batch=B, heads=H, head_dim=d, seq_len=T0, dtype=dtype, layer_seed=111,
                       cache_seed=112, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk0, zv0 = synth.draw_latent_cache(w, ld)
    L = latent_layer(H, d, ranks, rv, dtype)
    dl = DeviceLayer(L, zk0, zv0, ld.bk, ld.bv, capacity=192)
    rng = np.random.default_rng(113)
    a_k, a_v = _weights(rng, sum(ranks), D, dtype), _weights(rng, rv, D, dtype)
    x1 = rng.standard_normal((B, 30, D)).astype(np.float32)
    x2 = rng.standard_normal((B, 1, D)).astype(np.float32)
    bf16 = dtype == "bf16"
    _append_tokens(L, dl.cache, T0, x1, a_k, a_v, bf16)
    _append_tokens(L, dl.cache, T0 + 30, x2, a_k, a_v, bf16)
    T = T0 + 31
    rk, rvv = dl.readback(0, T, seq_len=T)
    assert np.array_equal(rk[:, :T0], zk0) and np.array_equal(rvv[:, :T0], zv0)
    x = np.concatenate([x1, x2], axis=1).astype(np.float64)
    _check_rounding(rk[:, T0:], x @ _f64(a_k, dtype).T, dtype, f"{dtype} keys")
    _check_rounding(rvv[:, T0:], x @ _f64(a_v, dtype).T, dtype, f"{dtype} values")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_append_tokens_exact_arithmetic(dtype):
    H, d, B, D = 2, 64, 5, 256
    ranks, rv = [16, 48], 80
    L = latent_layer(H, d, ranks, rv, dtype)
    rng = np.random.default_rng(114)
    x, a_k, a_v = _exact_inputs(rng, B, 70, D, sum(ranks), rv, dtype)
    zk_e, zv_e = oracle.project_tokens(x, a_k, a_v, dtype)
    dl = DeviceLayer(L, zk_e[:, :0], zv_e[:, :0], capacity=128)
    _append_tokens(L, dl.cache, 0, x, a_k, a_v, dtype == "bf16")
    rk, rvv = dl.readback(0, 70, seq_len=70)
    assert np.array_equal(rk.view(np.uint16), zk_e.view(np.uint16))
    assert np.array_equal(rvv.view(np.uint16), zv_e.view(np.uint16))


def test_append_tokens_dense():
    H, d, B, T0, D = 4, 64, 2, 10, 320
    k0, v0 = synth.draw_dense_cache(115, 0, B, T0, H * d, "f16")
    L = dense_layer(H, d, "f16")
    dl = DeviceLayer(L, k0, v0, capacity=64)
    rng = np.random.default_rng(116)
    w_k, w_v = _weights(rng, H * d, D, "f16"), _weights(rng, H * d, D, "f16")
    x = rng.standard_normal((B, 7, D)).astype(np.float32)
    _append_tokens(L, dl.cache, T0, x, w_k, w_v)
    rk, rvv = dl.readback(0, T0 + 7, seq_len=T0 + 7)
    assert np.array_equal(rk[:, :T0], k0) and np.array_equal(rvv[:, :T0], v0)
    x64 = x.astype(np.float64)
    _check_rounding(rk[:, T0:], x64 @ w_k.astype(np.float64).T, "f16", "dense keys")
    _check_rounding(rvv[:, T0:], x64 @ w_v.astype(np.float64).T, "f16", "dense values")


def test_append_tokens_q43_exact():
    """Mixed 4/3-bit cache: 40 tokens by starkv_append_latents, then token appends of 150 (which
    completes groups 0 and 1 and leaves 62 rows in the tail), 1 and 1 (completing group 2). The
    whole cache read back must equal the oracle's quantise -> dequantise of its own latents."""
    import torch
    from test_gpu_q43 import _append, _readback, q43_layer
    from rank_kv_cache_amd import buffers
    H, d, B, D = 3, 128, 2, 192
    ranks, rv = [16, 64, 32], 96
    cap = 256
    rng = np.random.default_rng(117)
    x, a_k, a_v = _exact_inputs(rng, B, 152, D, sum(ranks), rv, "f16")
    zk_new, zv_new = oracle.project_tokens(x, a_k, a_v, "f16")
    w = synth.Workload("aq", batch=B, heads=H, head_dim=d, seq_len=40, dtype="f16", layer_seed=118,
                       cache_seed=119, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk0, zv0 = synth.draw_latent_cache(w, ld)
    L = q43_layer(H, d, ranks, rv)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    _append(L, cache, zk0, zv0, [40])
    _append_tokens(L, cache, 40, x[:, :150], a_k, a_v)
    _append_tokens(L, cache, 190, x[:, 150:151], a_k, a_v)
    _append_tokens(L, cache, 191, x[:, 151:152], a_k, a_v)
    T = 192
    zk = np.concatenate([zk0, zk_new], axis=1)
    zv = np.concatenate([zv0, zv_new], axis=1)
    bits_k = oracle.channel_bits(ranks, FRAC)
    bits_v = oracle.channel_bits([rv], FRAC)
    for t_end in (T,):
        ck, mk, tk = oracle.q43_pack(zk[:, :t_end], bits_k, cap)
        cv, mv, tv = oracle.q43_pack(zv[:, :t_end], bits_v, cap)
        want_k = oracle.q43_unpack(ck, mk, tk, bits_k, t_end, cap)
        want_v = oracle.q43_unpack(cv, mv, tv, bits_v, t_end, cap)
        rk, rvv = _readback(L, cache, t_end, 0, t_end, sum(ranks), rv)
        assert np.array_equal(rk.view(np.uint16), want_k.view(np.uint16))
        assert np.array_equal(rvv.view(np.uint16), want_v.view(np.uint16))
    torch.cuda.synchronize()


def test_decode_step_chain():
    """One whole decode step of a latent layer through the library: append the new token from its
    hidden state, attend over the cache, project the heads' outputs; against the oracle's chain
    (its own latents for the new token, fp64 attention, fp64 projection)."""
    import torch
    from rank_kv_cache_amd import buffers
    H, d, B, T, D, hidden = 8, 128, 4, 300, 1024, 1024
    w = synth.Workload("chain", batch=B, heads=H, head_dim=d, seq_len=T - 1, dtype="f16",
                       layer_seed=120, cache_seed=121, value_rank=512,
                       key_rank_choices=(16, 32, 48, 64), power=0.5)
    ld = synth.draw_layer(w)
    ranks = [int(r) for r in ld.key_ranks]
    zk0, zv0 = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(122, 0, B, H, d)
    rng = np.random.default_rng(123)
    a_k, a_v = _weights(rng, sum(ranks), D, "f16"), _weights(rng, 512, D, "f16")
    wo_t = _weights(rng, hidden, H * d, "f16")
    x = rng.standard_normal((B, 1, D)).astype(np.float32)
    L = latent_layer(H, d, ranks, 512, "f16")
    dl = DeviceLayer(L, zk0, zv0, ld.bk, ld.bv, capacity=320)
    _append_tokens(L, dl.cache, T - 1, x, a_k, a_v)
    o = dl.decode(q, seq_len=T)
    y = torch.empty((B, hidden), dtype=torch.float32, device="cuda")
    nws = sk.starkv_output_projection_workspace_bytes(L, B, hidden)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    sk.starkv_output_projection(L, B, buffers.to_device(o), buffers.to_device(wo_t), hidden, y,
                                ws, nws)
    torch.cuda.synchronize()
    zk1, zv1 = oracle.project_tokens(x, a_k, a_v, "f16")
    zk = np.concatenate([zk0, zk1], axis=1)
    zv = np.concatenate([zv0, zv1], axis=1)
    ref = oracle.output_projection(oracle.decode_latent(zk, zv, ld.bk, ld.bv, q, ranks), wo_t)
    e = rel_err(y.cpu().numpy(), ref)
    say(f"[decode step chain] rel err {e:.3e}")
    assert e <= 2e-3
