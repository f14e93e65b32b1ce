"""GPU parity for several queries per cached sequence (speculative-decoding verification, chunks of
causal prefill queries): query row i reads sequence query_seq[i] and attends to its first
query_len[i] tokens. Each row is checked against the oracle on that sequence's prefix."""
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


def _queries(L, cache, qseq, qlen, q, bk, bv, num_splits=0, bf16=False):
    import torch
    from rank_kv_cache_amd import buffers
    n = len(qseq)
    mx = int(max(qlen))
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    nws = sk.starkv_decode_workspace_bytes(L, n, mx, num_splits)
    ws = torch.full((nws,), 0xFF, dtype=torch.uint8, device="cuda")
    sk.starkv_decode_attn_queries(
        L, cache, n, torch.tensor(np.asarray(qseq, np.int32), device="cuda"),
        torch.tensor(np.asarray(qlen, np.int32), device="cuda"), mx,
        buffers.to_device(np.ascontiguousarray(q, np.float32)),
        None if bk is None else buffers.to_device(bk, bf16=bf16),
        None if bv is None else buffers.to_device(bv, bf16=bf16), out, num_splits, ws, nws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check(qseq, qlen, got, ref_fn, what):
    worst = 0.0
    for i, (b, n) in enumerate(zip(qseq, qlen)):
        if n == 0:
            assert np.all(got[i] == 0), (what, i)
            continue
        e = rel_err(got[i], ref_fn(i, b, n))
        worst = max(worst, e)
        assert np.all(np.isfinite(got[i])) and e <= TOL, (what, i, b, n, e)
    say(f"[queries] {what}: {len(qseq)} rows, worst {worst:.3e}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_speculative_verification_latent(dtype):
    """Five causal queries at the last five positions of each of three sequences, interleaved,
    plus a parallel-sampling pair (same sequence and length) and an empty row."""
    H, d, B, T = 4, 128, 3, 150
    ranks, rv = [16, 32, 48, 64], 160
    w = synth.Workload("mq", batch=B, heads=H, head_dim=d, seq_len=T, dtype=dtype, layer_seed=211,
                       cache_seed=212, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    L = latent_layer(H, d, ranks, rv, dtype)
    dl = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
    qseq, qlen = [], []
    for p in range(145, 150):
        for b in range(B):
            qseq.append(b)
            qlen.append(p + 1)
    qseq += [1, 1, 0]
    qlen += [77, 77, 0]
    q = np.random.default_rng(213).standard_normal((len(qseq), H, d)).astype(np.float32)
    bf16 = dtype == "bf16"
    for S in (0, 2):
        got = _queries(L, dl.cache, qseq, qlen, q, ld.bk, ld.bv, S, bf16)
        _check(qseq, qlen, got,
               lambda i, b, n: oracle.decode_latent(zk[b:b + 1, :n], zv[b:b + 1, :n], ld.bk, ld.bv,
                                                    q[i:i + 1], ranks, bf16=bf16)[0],
               f"{dtype} splits={S}")


def test_queries_dense():
    H, d, B, T = 8, 128, 2, 100
    k, v = synth.draw_dense_cache(221, 0, B, T, H * d, "f16")
    L = dense_layer(H, d, "f16")
    dl = DeviceLayer(L, k, v)
    qseq = [0, 1, 0, 1, 1]
    qlen = [100, 99, 1, 64, 65]
    q = np.random.default_rng(222).standard_normal((len(qseq), H, d)).astype(np.float32)
    got = _queries(L, dl.cache, qseq, qlen, q, None, None)
    _check(qseq, qlen, got,
           lambda i, b, n: oracle.decode_dense(k[b:b + 1, :n], v[b:b + 1, :n], q[i:i + 1])[0], "dense")


def test_queries_q43():
    from test_gpu_q43 import _append, q43_layer
    from rank_kv_cache_amd import buffers
    H, d, B, T, cap = 3, 128, 2, 150, 192
    ranks, rv = [16, 64, 32], 96
    w = synth.Workload("mqq", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=231,
                       cache_seed=232, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    L = q43_layer(H, d, ranks, rv)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    _append(L, cache, zk, zv, [T])
    bits_k, bits_v = oracle.channel_bits(ranks, FRAC), oracle.channel_bits([rv], FRAC)
    qseq = [0, 1, 1, 0, 1]
    qlen = [150, 128, 64, 64, 150]          # whole groups, or everything appended
    q = np.random.default_rng(233).standard_normal((len(qseq), H, d)).astype(np.float32)
    got = _queries(L, cache, qseq, qlen, q, ld.bk, ld.bv)

    def ref(i, b, n):
        ck, mk, tk = oracle.q43_pack(zk[b:b + 1, :n], bits_k, cap)
        cv, mv, tv = oracle.q43_pack(zv[b:b + 1, :n], bits_v, cap)
        dk = oracle.q43_unpack(ck, mk, tk, bits_k, n, cap)
        dv = oracle.q43_unpack(cv, mv, tv, bits_v, n, cap)
        return oracle.decode_latent(dk, dv, ld.bk, ld.bv, q[i:i + 1], ranks)[0]

    _check(qseq, qlen, got, ref, "q43")


def test_queries_q43_causal_across_group():
    """Speculative verification on a mixed 4/3-bit cache with causal lengths that cross a 64-token
    group boundary: rows shorter than their sequence's fill end inside a group that is already
    quantised (the longest row of the sequence reaches the fill, whose partial last group is in
    the tail). The oracle quantises the sequence up to its fill and truncates to each row."""
    from test_gpu_q43 import _append, q43_layer
    from rank_kv_cache_amd import buffers
    H, d, B, T, cap = 3, 128, 2, 150, 192
    ranks, rv = [16, 64, 32], 96
    w = synth.Workload("mqx", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=241,
                       cache_seed=242, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    L = q43_layer(H, d, ranks, rv)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    _append(L, cache, zk, zv, [T])
    bits_k, bits_v = oracle.channel_bits(ranks, FRAC), oracle.channel_bits([rv], FRAC)
    qseq, qlen = [], []
    for n in (150, 131, 129, 128, 127, 126, 100, 65, 63):
        for b in range(B):
            qseq.append(b)
            qlen.append(n)
    order = np.random.default_rng(243).permutation(len(qseq))
    qseq, qlen = [qseq[i] for i in order], [qlen[i] for i in order]
    q = np.random.default_rng(244).standard_normal((len(qseq), H, d)).astype(np.float32)
    full = {}
    for b in range(B):
        ck, mk, tk = oracle.q43_pack(zk[b:b + 1], bits_k, cap)
        cv, mv, tv = oracle.q43_pack(zv[b:b + 1], bits_v, cap)
        full[b] = (oracle.q43_unpack(ck, mk, tk, bits_k, T, cap),
                   oracle.q43_unpack(cv, mv, tv, bits_v, T, cap))
    for S in (0, 2):
        got = _queries(L, cache, qseq, qlen, q, ld.bk, ld.bv, S)
        _check(qseq, qlen, got,
               lambda i, b, n: oracle.decode_latent(full[b][0][:, :n], full[b][1][:, :n], ld.bk,
                                                    ld.bv, q[i:i + 1], ranks)[0],
               f"q43 across group, splits={S}")
