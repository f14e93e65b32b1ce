"""GPU checks of paged caches: every 64-token block of a sequence lives in a page of a shared pool
named by a block table (pages shuffled, spare NaN-poisoned pages in the pool). Appends (bulk,
small, token projection, ragged), read-back and decode on the paged cache must give exactly the
contiguous cache's results (the kernels' arithmetic does not depend on where a block lives), and
decode must match the oracle."""
import numpy as np
import pytest

import oracle
import rank_kv_cache_amd as sk
from rank_kv_cache_amd import synth

from gpu_support import DeviceLayer, dense_layer, latent_layer, rel_err, say

pytestmark = pytest.mark.gpu
FRAC = 0.25


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.lib()


def paged_cache(L, B, cap, seed, spare=5):
    """A pool of B * cap/64 + spare pages (poisoned), a shuffled block table with two spare
    columns (pointing at page 0, never read), per-sequence tails."""
    import torch
    from rank_kv_cache_amd import buffers
    nb = cap // 64
    P = B * nb + spare
    pool = buffers.alloc_cache(L, P, 64, fill=0xFF)
    tails = buffers.alloc_cache(L, B, cap, fill=0xFF)
    perm = np.random.default_rng(seed).permutation(P)[:B * nb].astype(np.int32)
    stride = nb + 2
    table = np.zeros((B, stride), np.int32)
    table[:, :nb] = perm.reshape(B, nb)
    t = torch.tensor(table, device="cuda")
    return sk.Cache(B, cap, pool.zk, pool.zv, pool.zk_meta, pool.zv_meta, tails.zk_tail,
                    tails.zv_tail, block_table=t, table_stride=stride), (pool, tails, t)


def _append_chunks(L, cache, zk, zv, chunks, bf16=False):
    import torch
    from rank_kv_cache_amd import buffers
    dzk, dzv = buffers.to_device(zk, bf16=bf16), buffers.to_device(zv, bf16=bf16)
    pos = 0
    for n in chunks:
        sk.starkv_append_latents(L, cache, pos, n, dzk[:, pos:pos + n].contiguous(),
                                 dzv[:, pos:pos + n].contiguous())
        pos += n
    torch.cuda.synchronize()


def _readback(L, cache, T, Ck, Cv):
    import torch
    from rank_kv_cache_amd import buffers
    tdt = buffers.elem_torch_dtype(L.cache_dtype)
    ok = torch.empty((cache.batch, T, Ck), dtype=tdt, device="cuda")
    ov = torch.empty((cache.batch, T, Cv), dtype=tdt, device="cuda")
    sk.starkv_dequant(L, cache, T, 0, T, ok, ov)
    torch.cuda.synchronize()
    return buffers.to_host(ok), buffers.to_host(ov)


def _decode(L, cache, T, q, bk, bv, S=0, bf16=False):
    import torch
    from rank_kv_cache_amd import buffers
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    nws = sk.starkv_decode_workspace_bytes(L, cache.batch, T, S)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    sk.starkv_decode_attn(L, cache, T, buffers.to_device(np.ascontiguousarray(q, np.float32)),
                          None if bk is None else buffers.to_device(bk, bf16=bf16),
                          None if bv is None else buffers.to_device(bv, bf16=bf16), out, S, ws, nws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("dtype,ranks,rv", [("f16", [16, 32, 48, 64], 160), ("bf16", [5, 17, 30, 64], 100),
                                             ("q43", [16, 64, 32, 48], 96)])
def test_paged_latent(dtype, ranks, rv):
    from rank_kv_cache_amd import buffers
    H, d, B, T, cap = 4, 128, 3, 200, 256
    sdt = "f16" if dtype == "q43" else dtype
    w = synth.Workload("pg", batch=B, heads=H, head_dim=d, seq_len=T, dtype=sdt, layer_seed=241,
                       cache_seed=242, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(243, 0, B, H, d)
    if dtype == "q43":
        L = sk.Layer(num_heads=H, head_dim=d, key_ranks=tuple(ranks), value_rank=rv,
                     cache_dtype=sk.Q43, q_top_fraction=FRAC)
    else:
        L = latent_layer(H, d, ranks, rv, dtype)
    bf16 = dtype == "bf16"
    flat = buffers.alloc_cache(L, B, cap, fill=0xFF)
    paged, _keep = paged_cache(L, B, cap, 244)
    chunks = [130, 1, 69]
    _append_chunks(L, flat, zk, zv, chunks, bf16)
    _append_chunks(L, paged, zk, zv, chunks, bf16)
    fk, fv = _readback(L, flat, T, sum(ranks), rv)
    pk, pv = _readback(L, paged, T, sum(ranks), rv)
    assert np.array_equal(fk.view(np.uint8), pk.view(np.uint8))
    assert np.array_equal(fv.view(np.uint8), pv.view(np.uint8))
    for S in (0, 3):
        a = _decode(L, flat, T, q, ld.bk, ld.bv, S, bf16)
        b = _decode(L, paged, T, q, ld.bk, ld.bv, S, bf16)
        assert np.array_equal(a, b), S
    rk, rvv = zk, zv
    if dtype == "q43":                   # the oracle's own quantise -> dequantise of the rows
        bits_k, bits_v = oracle.channel_bits(ranks, FRAC), oracle.channel_bits([rv], FRAC)
        rk = oracle.q43_unpack(*oracle.q43_pack(zk, bits_k, cap), bits_k, T, cap)
        rvv = oracle.q43_unpack(*oracle.q43_pack(zv, bits_v, cap), bits_v, T, cap)
        assert np.array_equal(pk.view(np.uint16), rk.view(np.uint16))
        assert np.array_equal(pv.view(np.uint16), rvv.view(np.uint16))
    ref = oracle.decode_latent(rk, rvv, ld.bk, ld.bv, q, ranks, bf16=bf16)
    e = rel_err(b, ref)
    say(f"[paged] {dtype} ranks={ranks}: paged == contiguous, oracle rel err {e:.3e}")
    assert e <= 2e-3


def test_paged_dense_and_ragged():
    import torch
    from rank_kv_cache_amd import buffers
    H, d, B, T, cap = 4, 64, 3, 150, 192
    k, v = synth.draw_dense_cache(251, 0, B, T, H * d, "f16")
    q = synth.draw_queries(252, 0, B, H, d)
    L = dense_layer(H, d, "f16")
    flat = buffers.alloc_cache(L, B, cap, fill=0xFF)
    paged, _keep = paged_cache(L, B, cap, 253)
    _append_chunks(L, flat, k, v, [100, 50])
    _append_chunks(L, paged, k, v, [100, 50])
    fk, fv = _readback(L, flat, T, H * d, H * d)
    pk, pv = _readback(L, paged, T, H * d, H * d)
    assert np.array_equal(fk.view(np.uint16), pk.view(np.uint16))
    assert np.array_equal(fv.view(np.uint16), pv.view(np.uint16))
    # ragged one-token appends and ragged decode on both
    lens = [151, 150, 152]
    k2, v2 = synth.draw_dense_cache(254, 0, B, 2, H * d, "f16")
    dk2, dv2 = buffers.to_device(k2), buffers.to_device(v2)
    for step in range(2):
        pos = torch.tensor([T + step if T + step < n else -1 for n in lens], dtype=torch.int32, device="cuda")
        for c in (flat, paged):
            sk.starkv_append_latents_ragged(L, c, pos, dk2[:, step].contiguous(), dv2[:, step].contiguous())
    torch.cuda.synchronize()
    dl = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    outs = []
    for c in (flat, paged):
        out = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
        nws = sk.starkv_decode_workspace_bytes(L, B, max(lens), 0)
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        sk.starkv_decode_attn_ragged(L, c, max(lens), dl, buffers.to_device(q), None, None, out, 0, ws, nws)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    kk = np.concatenate([k, k2], axis=1)
    vv = np.concatenate([v, v2], axis=1)
    for b, n in enumerate(lens):
        ref = oracle.decode_dense(kk[b:b + 1, :n], vv[b:b + 1, :n], q[b:b + 1])[0]
        assert rel_err(outs[1][b], ref) <= 2e-3, b
    say("[paged] dense + ragged: paged == contiguous")


def test_paged_append_tokens():
    """Hidden-state appends (latent block layout and dense rows) into paged caches."""
    import torch
    from rank_kv_cache_amd import buffers
    H, d, B, D, n, cap = 2, 128, 2, 128, 70, 128
    rng = np.random.default_rng(261)
    x = rng.standard_normal((B, n, D)).astype(np.float32)
    for L, Ck, Cv in ((latent_layer(H, d, [16, 48], 64, "f16"), 64, 64), (dense_layer(H, d, "f16"), H * d, H * d)):
        a_k = (rng.standard_normal((Ck, D)) / np.sqrt(D)).astype(np.float16)
        a_v = (rng.standard_normal((Cv, D)) / np.sqrt(D)).astype(np.float16)
        flat = buffers.alloc_cache(L, B, cap, fill=0xFF)
        paged, _keep = paged_cache(L, B, cap, 262)
        nws = sk.starkv_append_tokens_workspace_bytes(L, B, n, D)
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        for c in (flat, paged):
            sk.starkv_append_tokens(L, c, 0, n, buffers.to_device(x), D, buffers.to_device(a_k),
                                    buffers.to_device(a_v), ws, nws)
        torch.cuda.synchronize()
        fk, fv = _readback(L, flat, n, Ck, Cv)
        pk, pv = _readback(L, paged, n, Ck, Cv)
        assert np.array_equal(fk.view(np.uint16), pk.view(np.uint16))
        assert np.array_equal(fv.view(np.uint16), pv.view(np.uint16))
    say("[paged] token appends: paged == contiguous")
