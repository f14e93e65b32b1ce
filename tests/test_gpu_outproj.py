"""GPU parity of the layer's output projection (Alg. 2 step 8): y = concat_h(o_h) . W_o after
decode attention, for latent layers in each storage type and for an exempt (dense) layer, against
the oracle's attention followed by its fp64 matrix product. Sizes span several 32-output tiles
with a ragged last tile, several 64-wide K tiles and splits, and a batch that is not a multiple of
the kernel's 32-row tile; an exact-arithmetic case must match bit for bit."""
import numpy as np
import pytest

import oracle
import rank_kv_cache_amd as sk
from rank_kv_cache_amd import synth

from gpu_support import DeviceLayer, dense_layer, latent_layer, rel_err, say

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.lib()


def _project(layer, o, wo_t, hidden, bf16=False):
    import torch
    from rank_kv_cache_amd import buffers
    B = o.shape[0]
    y = torch.full((B, hidden), float("nan"), dtype=torch.float32, device="cuda")
    nws = sk.starkv_output_projection_workspace_bytes(layer, B, hidden)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    sk.starkv_output_projection(layer, B, buffers.to_device(np.ascontiguousarray(o, np.float32)),
                                buffers.to_device(wo_t, bf16=bf16), hidden, y, ws, nws)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _weights(rng, rows, cols, dtype):
    return synth._store((rng.standard_normal((rows, cols)) / np.sqrt(cols)).astype(np.float32), dtype)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_latent_layer_output_projection(dtype):
    H, d, B, T, hidden = 4, 128, 5, 200, 300
    ranks, rv = [16, 32, 48, 64], 160
    w = synth.Workload("op", batch=B, heads=H, head_dim=d, seq_len=T, dtype=dtype, layer_seed=101,
                       cache_seed=102, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(103, 0, B, H, d)
    wo_t = _weights(np.random.default_rng(104), hidden, H * d, dtype)
    bf16 = dtype == "bf16"
    L = latent_layer(H, d, ranks, rv, dtype)
    o = DeviceLayer(L, zk, zv, ld.bk, ld.bv).decode(q)
    y = _project(L, o, wo_t, hidden, bf16=bf16)
    ref = oracle.output_projection(
        oracle.decode_latent(zk, zv, ld.bk, ld.bv, q, ranks, bf16=bf16), wo_t, bf16=bf16)
    e = rel_err(y, ref)
    say(f"[outproj] latent {dtype} rel err {e:.3e}")
    assert np.all(np.isfinite(y)) and e <= TOL


def test_dense_layer_output_projection():
    H, d, B, T, hidden = 8, 64, 3, 130, 70
    k, v = synth.draw_dense_cache(105, 0, B, T, H * d, "f16")
    q = synth.draw_queries(106, 0, B, H, d)
    wo_t = _weights(np.random.default_rng(107), hidden, H * d, "f16")
    L = dense_layer(H, d, "f16")
    o = DeviceLayer(L, k, v).decode(q)
    y = _project(L, o, wo_t, hidden)
    ref = oracle.output_projection(oracle.decode_dense(k, v, q), wo_t)
    e = rel_err(y, ref)
    say(f"[outproj] dense rel err {e:.3e}")
    assert np.all(np.isfinite(y)) and e <= TOL


@pytest.mark.parametrize("dtype,B", [("f16", 33), ("bf16", 16), ("f32", 7)])
def test_projection_alone_matches_matrix_product(dtype, B):
    """The projection by itself on given fp32 rows at the LongChat shape (H*d = 4096 inputs,
    4096 outputs): the 16-bit split of the rows keeps the result at fp32 accuracy."""
    H, d, hidden = 32, 128, 4096
    L = latent_layer(H, d, [16] * H, 64, dtype)
    rng = np.random.default_rng(108)
    o = rng.standard_normal((B, H, d)).astype(np.float32)
    wo_t = _weights(rng, hidden, H * d, dtype)
    y = _project(L, o, wo_t, hidden, bf16=dtype == "bf16")
    ref = oracle.output_projection(o, wo_t, bf16=dtype == "bf16")
    e = rel_err(y, ref)
    say(f"[outproj] alone {dtype} B={B} rel err {e:.3e}")
    # Bound, as a fraction of RMS(y) with y_n = sum over K = 4096 inputs:
    # * the 16-bit split drops r = o - hi - lo, |r| of order u^2 |o| (u = 2^-11 for binary16,
    #   2^-8 for bfloat16); with o - hi spread over half an ulp of o and r over half an ulp of
    #   o - hi, rms(r) is about u^2 / 3 of |o|, so the dropped sum has relative rms about 2^-16 / 3
    #   = 5e-6 (bfloat16), 2^-22 / 3 = 8e-8 (binary16), and about 4.5 rms over the 65-135 k outputs
    #   of a call: 2.3e-5 and 4e-7;
    # * fp32 accumulation of exact products in K-slices of about 512 terms: rounding rms about
    #   2^-24 / sqrt(3) * sqrt(512 / 2) = 5.5e-7, 2.5e-6 at 4.5 rms.
    # Measured: 7.9e-7 (binary16), 1.0e-6 (fp32), 1.0e-5 (bfloat16).
    assert e <= (5e-5 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_projection_exact_arithmetic(dtype):
    """Quarter-integer rows times small-integer weights: every product and partial sum is exact in
    fp32, so the result must equal the oracle's bit for bit whatever the split and order."""
    H, d, B, hidden = 8, 64, 37, 200
    L = latent_layer(H, d, [16] * H, 64, dtype)
    rng = np.random.default_rng(109)
    o = (rng.integers(-8, 9, (B, H, d)) * 0.25).astype(np.float32)
    wo_t = synth._store(rng.integers(-3, 4, (hidden, H * d)).astype(np.float32), dtype)
    y = _project(L, o, wo_t, hidden, bf16=dtype == "bf16")
    ref = oracle.output_projection(o, wo_t, bf16=dtype == "bf16")
    assert np.array_equal(y.astype(np.float64), ref)


@pytest.mark.parametrize("dtype,splits", [("f16", 0), ("bf16", 3)])
def test_decode_attn_project_one_call(dtype, splits):
    """Decode attention and the output projection in one call: bit for bit the two-call path
    (the same kernels with the heads' outputs kept in the workspace), and the oracle's attention
    followed by its fp64 product within the decode bar."""
    import torch
    from rank_kv_cache_amd import buffers
    H, d, B, T, hidden = 6, 128, 7, 333, 260
    ranks, rv = [16, 64, 32, 48, 16, 80], 224
    w = synth.Workload("op1", batch=B, heads=H, head_dim=d, seq_len=T, dtype=dtype, layer_seed=111,
                       cache_seed=112, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(113, 0, B, H, d)
    bf16 = dtype == "bf16"
    wo_t = _weights(np.random.default_rng(114), hidden, H * d, dtype)
    L = latent_layer(H, d, ranks, rv, dtype)
    dl = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
    dq = buffers.to_device(np.ascontiguousarray(q, np.float32))
    dwo = buffers.to_device(wo_t, bf16=bf16)
    nws = sk.starkv_decode_attn_project_workspace_bytes(L, B, T, splits, hidden)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    y1 = torch.full((B, hidden), float("nan"), dtype=torch.float32, device="cuda")
    sk.starkv_decode_attn_project(L, dl.cache, T, dq, dl.bk, dl.bv, dwo, hidden, y1, splits, ws, nws)
    torch.cuda.synchronize()
    # two calls
    o = dl.decode(q, num_splits=splits)
    y2 = _project(L, o, wo_t, hidden, bf16=bf16)
    got = y1.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), y2.view(np.uint32))
    ref = oracle.output_projection(
        oracle.decode_latent(zk, zv, ld.bk, ld.bv, q, ranks, bf16=bf16), wo_t, bf16=bf16)
    e = rel_err(got, ref)
    say(f"[outproj] one call {dtype} splits={splits}: bit-equal to two calls, rel err {e:.3e}")
    assert np.all(np.isfinite(got)) and e <= TOL
