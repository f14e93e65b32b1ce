"""GPU parity for nq queries per cached sequence sharing one key rebuild and one latent stream
(starkv_decode_attn_multi): every query row against the oracle on its own prefix; nq = 1 through
this entry point equals starkv_decode_attn bit for bit."""
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


def _multi(L, cache, nq, max_len, lens, q, bk, bv, S=0, bf16=False):
    import torch
    from rank_kv_cache_amd import buffers
    rows = q.shape[0]
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    nws = sk.starkv_decode_multi_workspace_bytes(L, cache.batch, nq, max_len, S)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    dl = None if lens is None else torch.tensor(np.asarray(lens, np.int32), device="cuda")
    sk.starkv_decode_attn_multi(L, cache, nq, max_len, dl, buffers.to_device(np.ascontiguousarray(q, np.float32)),
                                buffers.to_device(bk, bf16=bf16), buffers.to_device(bv, bf16=bf16),
                                out, S, ws, nws)
    torch.cuda.synchronize()
    assert rows == cache.batch * nq
    return out.cpu().numpy()


def _case(dtype, ranks, rv, T, seed):
    H, d, B = len(ranks), 128, 3
    w = synth.Workload("mu", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16" if dtype == "q43" else dtype,
                       layer_seed=seed, cache_seed=seed + 1, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    return H, d, B, ld, zk, zv


@pytest.mark.parametrize("dtype,nq,ranks,rv", [
    ("f16", 2, [16, 32, 48, 64], 160), ("f16", 4, [16, 32, 48, 64], 160),
    ("bf16", 4, [33, 7, 64, 50], 100), ("f16", 2, [96, 16, 80, 32], 272)])
def test_multi_causal(dtype, nq, ranks, rv):
    T = 200
    H, d, B, ld, zk, zv = _case(dtype, ranks, rv, T, 271)
    L = latent_layer(H, d, ranks, rv, dtype)
    dl = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
    q = np.random.default_rng(272).standard_normal((B * nq, H, d)).astype(np.float32)
    lens = [T - nq + 1 + i for _ in range(B) for i in range(nq)]
    lens[1] = 0                                            # an empty row
    lens[-1] = 64                                          # a row much shorter than its neighbours
    bf16 = dtype == "bf16"
    for S in (0, 3):
        got = _multi(L, dl.cache, nq, T, lens, q, ld.bk, ld.bv, S, bf16)
        worst = 0.0
        for r, n in enumerate(lens):
            b = r // nq
            if n == 0:
                assert np.all(got[r] == 0), r
                continue
            ref = oracle.decode_latent(zk[b:b + 1, :n], zv[b:b + 1, :n], ld.bk, ld.bv, q[r:r + 1],
                                       ranks, bf16=bf16)[0]
            e = rel_err(got[r], ref)
            worst = max(worst, e)
            assert np.all(np.isfinite(got[r])) and e <= TOL, (r, n, e)
        say(f"[multi] {dtype} nq={nq} ranks={ranks} splits={S}: worst {worst:.3e}")


def test_multi_q43():
    from test_gpu_q43 import _append, q43_layer
    from rank_kv_cache_amd import buffers
    T, cap, nq = 150, 192, 4
    ranks, rv = [16, 64, 32], 96
    H, d, B, ld, zk, zv = _case("q43", ranks, rv, T, 281)
    L = q43_layer(H, d, ranks, rv)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    _append(L, cache, zk, zv, [T])
    bits_k, bits_v = oracle.channel_bits(ranks, FRAC), oracle.channel_bits([rv], FRAC)
    q = np.random.default_rng(282).standard_normal((B * nq, H, d)).astype(np.float32)
    lens = [T, 128, 64, T] * B                              # whole groups or everything appended
    got = _multi(L, cache, nq, T, lens, q, ld.bk, ld.bv)
    for r, n in enumerate(lens):
        b = r // nq
        dk = oracle.q43_unpack(*oracle.q43_pack(zk[b:b + 1, :n], bits_k, cap), bits_k, n, cap)
        dv = oracle.q43_unpack(*oracle.q43_pack(zv[b:b + 1, :n], bits_v, cap), bits_v, n, cap)
        ref = oracle.decode_latent(dk, dv, ld.bk, ld.bv, q[r:r + 1], ranks)[0]
        assert rel_err(got[r], ref) <= TOL, r
    say("[multi] q43 nq=4 ok")


def test_multi_single_query_is_decode():
    import torch
    from rank_kv_cache_amd import buffers
    T = 130
    ranks, rv = [16, 32, 48, 64], 160
    H, d, B, ld, zk, zv = _case("f16", ranks, rv, T, 291)
    L = latent_layer(H, d, ranks, rv, "f16")
    dl = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
    q = synth.draw_queries(292, 0, B, H, d)
    a = dl.decode(q)
    b = _multi(L, dl.cache, 1, T, None, q, ld.bk, ld.bv)
    assert np.array_equal(a, b)
