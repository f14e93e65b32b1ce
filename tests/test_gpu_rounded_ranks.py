"""GPU parity for latent ranks that are not multiples of 16 (the kernels' 16-channel tile): the
cache stores each rank rounded up with zero channels, while rows, factors and read-back keep the
true ranks. Caches are poisoned with NaN bytes first, so a padding channel that were left
unwritten would turn every score into NaN."""
import numpy as np
import pytest

import oracle
import rank_kv_cache_amd as sk
from rank_kv_cache_amd import synth

from gpu_support import DeviceLayer, latent_layer, rel_err, say

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.lib()


def _draw(dtype, H, d, ranks, rv, T, seed):
    w = synth.Workload("rr", batch=3, heads=H, head_dim=d, seq_len=T, dtype=dtype, layer_seed=seed,
                       cache_seed=seed + 1, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(seed + 2, 0, 3, H, d)
    return ld, zk, zv, q


@pytest.mark.parametrize("dtype,d,ranks,rv", [
    ("f16", 128, [5, 17, 30, 64, 1, 128], 100),
    ("bf16", 128, [33, 7, 96, 50], 272),
    ("f32", 64, [3, 64, 33, 50], 20),
])
def test_rounded_ranks_append_readback_decode(dtype, d, ranks, rv):
    H, T = len(ranks), 200
    ld, zk, zv, q = _draw(dtype, H, d, ranks, rv, T, 131)
    L = latent_layer(H, d, ranks, rv, dtype)
    dl = DeviceLayer(L, zk, zv, ld.bk, ld.bv, capacity=256, chunks=[130, 1, 69])
    rk, rvv = dl.readback(0, T)
    assert np.array_equal(rk.view(np.uint8), zk.view(np.uint8))
    assert np.array_equal(rvv.view(np.uint8), zv.view(np.uint8))
    bf16 = dtype == "bf16"
    for Tq in (T, 64, 1):
        ref = oracle.decode_latent(zk[:, :Tq], zv[:, :Tq], ld.bk, ld.bv, q, ranks, bf16=bf16)
        for S in (0, 3):
            got = dl.decode(q, seq_len=Tq, num_splits=S)
            e = rel_err(got, ref)
            say(f"[rounded ranks] {dtype} d={d} ranks={ranks} rv={rv} T={Tq} splits={S}: {e:.3e}")
            assert np.all(np.isfinite(got)) and e <= TOL


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_rounded_ranks_append_tokens_exact(dtype):
    """Hidden-state appends into a layer with rounded ranks: quarter-integer inputs and small
    integer weights make every product exact, so the stored latents must equal the oracle's bit
    for bit; decode then runs on them."""
    import torch
    from rank_kv_cache_amd import buffers
    H, d, D, B, n = 3, 128, 128, 2, 70
    ranks, rv = [9, 40, 23], 50
    L = latent_layer(H, d, ranks, rv, dtype)
    rng = np.random.default_rng(141)
    x = (rng.integers(-4, 5, (B, n, D)) * 0.25).astype(np.float32)
    a_k = synth._store(rng.integers(-3, 4, (sum(ranks), D)).astype(np.float32), dtype)
    a_v = synth._store(rng.integers(-3, 4, (rv, D)).astype(np.float32), dtype)
    zk_e, zv_e = oracle.project_tokens(x, a_k, a_v, dtype)
    w = synth.Workload("rt", batch=B, heads=H, head_dim=d, seq_len=1, dtype=dtype, layer_seed=142,
                       cache_seed=143, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    dl = DeviceLayer(L, zk_e[:, :0], zv_e[:, :0], ld.bk, ld.bv, capacity=128)
    bf16 = dtype == "bf16"
    nws = sk.starkv_append_tokens_workspace_bytes(L, B, n, D)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    sk.starkv_append_tokens(L, dl.cache, 0, n, buffers.to_device(x), D,
                            buffers.to_device(a_k, bf16=bf16), buffers.to_device(a_v, bf16=bf16),
                            ws, nws)
    torch.cuda.synchronize()
    rk, rvv = dl.readback(0, n, seq_len=n)
    assert np.array_equal(rk.view(np.uint16), zk_e.view(np.uint16))
    assert np.array_equal(rvv.view(np.uint16), zv_e.view(np.uint16))
    q = synth.draw_queries(144, 0, B, H, d) * 0.05
    got = dl.decode(q, seq_len=n)
    ref = oracle.decode_latent(zk_e, zv_e, ld.bk, ld.bv, q, ranks, bf16=bf16)
    e = rel_err(got, ref)
    say(f"[rounded ranks] append_tokens {dtype} decode: {e:.3e}")
    assert np.all(np.isfinite(got)) and e <= TOL


def test_rounded_ranks_rotation():
    """The device rotation on latent rows of a binary16 layer with odd ranks uses the true widths
    (each head's latent rotated in blocks of the largest power of two dividing its rank)."""
    import torch
    from rank_kv_cache_amd import buffers
    H, d = 4, 128
    ranks = [24, 40, 12, 100]
    L = latent_layer(H, d, ranks, 48, "f16")
    rng = np.random.default_rng(151)
    x = rng.standard_normal((37, sum(ranks))).astype(np.float16)
    out = torch.empty((37, sum(ranks)), dtype=torch.float16, device="cuda")
    sk.starkv_hadamard_rotate(L, 0, 0, 37, buffers.to_device(x), out)
    torch.cuda.synchronize()
    want = oracle.rotate_rows(x, oracle.latent_segments(ranks, 0.0))
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want.view(np.uint16))
