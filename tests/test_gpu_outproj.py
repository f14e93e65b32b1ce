"""GPU parity of the layer's output projection (Alg. 2 step 8): y = concat_h(o_h) . W_o after
decode attention, for latent layers in each storage type and for an exempt (dense) layer, against
the oracle's attention followed by its fp64 matrix product. Sizes span several 64-column tiles with
a ragged last tile and a batch that is not a multiple of the kernel's sequence chunk."""
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


def _project(layer, o, wo_np, hidden, bf16=False):
    import torch
    from rank_kv_cache_amd import buffers
    B = o.shape[0]
    y = torch.full((B, hidden), float("nan"), dtype=torch.float32, device="cuda")
    sk.starkv_output_projection(layer, B, buffers.to_device(np.ascontiguousarray(o, np.float32)),
                                buffers.to_device(wo_np, bf16=bf16), hidden, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_latent_layer_output_projection(dtype):
    H, d, B, T, hidden = 4, 128, 5, 200, 300
    ranks, rv = [16, 32, 48, 64], 160
    w = synth.Workload("op", batch=B, heads=H, head_dim=d, seq_len=T, dtype=dtype, layer_seed=101,
                       cache_seed=102, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(103, 0, B, H, d)
    rng = np.random.default_rng(104)
    wo32 = (rng.standard_normal((H * d, hidden)) / np.sqrt(H * d)).astype(np.float32)
    wo = synth._store(wo32, dtype)
    bf16 = dtype == "bf16"
    L = latent_layer(H, d, ranks, rv, dtype)
    dl = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
    o = dl.decode(q)
    y = _project(L, o, wo, hidden, bf16=bf16)
    ref = oracle.output_projection(
        oracle.decode_latent(zk, zv, ld.bk, ld.bv, q, ranks, bf16=bf16), wo, bf16=bf16)
    e = rel_err(y, ref)
    say(f"[outproj] latent {dtype} rel err {e:.3e}")
    assert np.all(np.isfinite(y)) and e <= TOL


def test_dense_layer_output_projection():
    H, d, B, T, hidden = 8, 64, 3, 130, 70
    k, v = synth.draw_dense_cache(105, 0, B, T, H * d, "f16")
    q = synth.draw_queries(106, 0, B, H, d)
    rng = np.random.default_rng(107)
    wo = (rng.standard_normal((H * d, hidden)) / np.sqrt(H * d)).astype(np.float16)
    L = dense_layer(H, d, "f16")
    dl = DeviceLayer(L, k, v)
    o = dl.decode(q)
    y = _project(L, o, wo, hidden)
    ref = oracle.output_projection(oracle.decode_dense(k, v, q), wo)
    e = rel_err(y, ref)
    say(f"[outproj] dense rel err {e:.3e}")
    assert np.all(np.isfinite(y)) and e <= TOL


def test_projection_alone_matches_matrix_product():
    """The projection by itself on given fp32 rows: only fp32 summation order differs from fp64."""
    H, d, B, hidden = 32, 128, 33, 4096
    L = latent_layer(H, d, [16] * H, 64, "f16")
    rng = np.random.default_rng(108)
    o = rng.standard_normal((B, H, d)).astype(np.float32)
    wo = (rng.standard_normal((H * d, hidden)) / np.sqrt(H * d)).astype(np.float16)
    y = _project(L, o, wo, hidden)
    ref = oracle.output_projection(o, wo)
    e = rel_err(y, ref)
    say(f"[outproj] alone rel err {e:.3e}")
    assert e <= 1e-5
