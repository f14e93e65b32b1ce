"""The decode entry point that allocates nothing (its workspace is a fixed per-GPU array inside the
library) against the one that takes a caller workspace: the same kernels with the same splits, so
the outputs must agree bit for bit; two calls in a row, the second with a smaller input (fewer
sequences, a shorter length, another layer), then a request larger than the array, refused."""
import numpy as np
import pytest

import oracle
import rank_kv_cache_amd as sk
from rank_kv_cache_amd import synth

from gpu_support import DeviceLayer, latent_layer, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.lib()


def _both(L, dl, T, q, splits):
    import torch
    from rank_kv_cache_amd import buffers
    B = dl.cache.batch
    dq = buffers.to_device(np.ascontiguousarray(q, np.float32))
    ref = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    nws = sk.starkv_decode_workspace_bytes(L, B, T, splits)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    sk.starkv_decode_attn(L, dl.cache, T, dq, dl.bk, dl.bv, ref, splits, ws, nws)
    got = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    sk.starkv_decode_attn_noalloc(L, dl.cache, T, dq, dl.bk, dl.bv, got, splits)
    torch.cuda.synchronize()
    return got.cpu().numpy(), ref.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_twice():
    assert sk.starkv_decode_attn_noalloc_max_bytes() == 64 << 20
    cases = [
        # (heads, ranks, r_v, batch, T, splits): the second call is smaller in every size
        (8, [16, 32, 48, 64, 16, 32, 48, 64], 512, 6, 3000, 0),
        (4, [16, 64, 32, 48], 256, 3, 700, 3),
    ]
    for i, (H, ranks, rv, B, T, S) in enumerate(cases):
        d = 128
        w = synth.Workload(f"na{i}", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16",
                           layer_seed=300 + i, cache_seed=310 + i, value_rank=rv, power=0.5)
        ld = synth.draw_layer(w, key_ranks=ranks)
        zk, zv = synth.draw_latent_cache(w, ld)
        q = synth.draw_queries(320 + i, 0, B, H, d)
        L = latent_layer(H, d, ranks, rv, "f16")
        dl = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
        got, ref = _both(L, dl, T, q, S)
        assert np.all(np.isfinite(got))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"call {i}"
        # and both agree with the oracle on sampled pairs, to the decode bar
        pairs = [(0, 0), (B - 1, H - 1), (B // 2, H // 2)]
        want = oracle.decode_latent(zk, zv, ld.bk, ld.bv, q, ranks, pairs=pairs)
        e = rel_err(np.stack([got[b, h] for b, h in pairs]), want)
        say(f"[noalloc] call {i}: B={B} H={H} T={T} splits={S}: bit-equal, oracle rel err {e:.3e}")
        assert e <= 2e-3


def test_noalloc_refuses_oversized_request():
    """A workspace beyond the array is refused before anything is enqueued (no device pointer
    below is dereferenced)."""
    L = latent_layer(32, 128, [64] * 32, 2048, "f16")
    cache = sk.Cache(batch=64, capacity=1 << 16, zk=0x10000, zv=0x10000)
    assert sk.starkv_decode_workspace_bytes(L, 64, 1 << 16, 0) > 64 << 20
    st = sk.starkv_decode_attn_noalloc(L, cache, 1 << 16, 0x10000, 0x10000, 0x10000, 0x10000, 0,
                                       check=False)
    assert st == 7                                       # STARKV_ERR_WORKSPACE
