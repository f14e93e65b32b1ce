"""GPU parity of exempt-layer (dense K/V) decode attention against the fp64 oracle."""
import numpy as np
import pytest

import oracle
from rank_kv_cache_amd import synth

from gpu_support import DeviceLayer, dense_layer, rel_err, say

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype,d,T", [("f16", 128, 1000), ("f16", 128, 1), ("bf16", 128, 333),
                                       ("f32", 64, 129), ("f16", 64, 64)])
def test_dense_parity(dtype, d, T):
    B, H = 3, 32 if d == 128 else 8
    k, v = synth.draw_dense_cache(51, 0, B, T, H * d, dtype=dtype)
    q = synth.draw_queries(51, 0, B, H, d)
    say(f"[dense] {dtype} d={d} T={T} H={H}")
    dl = DeviceLayer(dense_layer(H, d, dtype), k, v, capacity=((T + 63) // 64) * 64 + 64)
    ref = oracle.decode_dense(k, v, q, bf16=(dtype == "bf16"))
    for S in (0, 1, 5):
        got = dl.decode(q, num_splits=S)
        e = rel_err(got, ref)
        say(f"[dense] {dtype} d={d} T={T} splits={S} rel err {e:.3e}")
        assert np.all(np.isfinite(got)) and e <= TOL
    rk, rvv = dl.readback(0, T)
    assert np.array_equal(rk.view(np.uint8), k.view(np.uint8))
    assert np.array_equal(rvv.view(np.uint8), v.view(np.uint8))
