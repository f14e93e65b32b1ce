"""Grouped query attention (several query heads per latent KV head, as in the LLaMA-3 models the
pages evaluate; the ledger of the reading notes counts KV heads) through the multi-query entry
point. The layer describes the H_kv KV heads; the G = H_q / H_kv query heads that share KV head
h (query heads h*G .. h*G + G - 1) become G query rows of their sequence, row b*G + g holding
query head h*G + g in head slot h, so one key rebuild, one rotation and one latent stream serve
all of them, and the output step applies KV head h's B_v slice to each. Checked against the
oracle's attention of every query head over its own KV head."""
import numpy as np
import pytest

import oracle
import rank_kv_cache_amd as sk
from rank_kv_cache_amd import synth

from gpu_support import DeviceLayer, latent_layer, rel_err, say
from test_gpu_multi import _multi

pytestmark = pytest.mark.gpu
TOL = 2e-3
FRAC = 0.25


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.lib()


def gqa_rows(q, G):
    """[B][H_kv * G][d] query heads -> [B * G][H_kv][d] rows (row b*G + g, slot h = head h*G + g)."""
    B, Hq, d = q.shape
    return np.ascontiguousarray(q.reshape(B, Hq // G, G, d).transpose(0, 2, 1, 3).reshape(B * G, Hq // G, d))


def gqa_heads(o, B, G):
    """The inverse of gqa_rows on the outputs."""
    _, Hkv, d = o.shape
    return o.reshape(B, G, Hkv, d).transpose(0, 2, 1, 3).reshape(B, Hkv * G, d)


@pytest.mark.parametrize("dtype,G", [("f16", 4), ("bf16", 2), ("q43", 4)])
def test_gqa_decode(dtype, G):
    from rank_kv_cache_amd import buffers
    Hkv, d, B, T = 4, 128, 3, 300
    ranks, rv = [16, 48, 32, 64], 128
    w = synth.Workload("gqa", batch=B, heads=Hkv, head_dim=d, seq_len=T,
                       dtype="f16" if dtype == "q43" else dtype, layer_seed=701, cache_seed=702,
                       value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = np.random.default_rng(703).standard_normal((B, Hkv * G, d)).astype(np.float32)
    bf16 = dtype == "bf16"
    if dtype == "q43":
        from test_gpu_q43 import _append, q43_layer
        cap = 320
        L = q43_layer(Hkv, d, ranks, rv)
        cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
        _append(L, cache, zk, zv, [T])
        bits_k, bits_v = oracle.channel_bits(ranks, FRAC), oracle.channel_bits([rv], FRAC)
        ck, mk, tk = oracle.q43_pack(zk, bits_k, cap)
        cv, mv, tv = oracle.q43_pack(zv, bits_v, cap)
        rk_, rv_ = oracle.q43_unpack(ck, mk, tk, bits_k, T, cap), oracle.q43_unpack(cv, mv, tv, bits_v, T, cap)
    else:
        L = latent_layer(Hkv, d, ranks, rv, dtype)
        dl = DeviceLayer(L, zk, zv, ld.bk, ld.bv)
        cache = dl.cache
        rk_, rv_ = zk, zv
    got = gqa_heads(_multi(L, cache, G, T, None, gqa_rows(q, G), ld.bk, ld.bv, bf16=bf16), B, G)
    worst = 0.0
    for g in range(G):
        # query heads h*G + g, one per KV head h
        ref = oracle.decode_latent(rk_, rv_, ld.bk, ld.bv, np.ascontiguousarray(q[:, g::G]), ranks, bf16=bf16)
        e = rel_err(got[:, g::G], ref)
        worst = max(worst, e)
        assert np.all(np.isfinite(got[:, g::G])) and e <= TOL, (g, e)
    say(f"[gqa] {dtype} H_q={Hkv * G} H_kv={Hkv}: worst {worst:.3e}")


def test_gqa_row_mapping_roundtrip():
    """gqa_rows / gqa_heads place query head h*G + g in row g, slot h, and back."""
    B, Hkv, G, d = 2, 3, 4, 5
    q = np.arange(B * Hkv * G * d, dtype=np.float32).reshape(B, Hkv * G, d)
    r = gqa_rows(q, G)
    for b in range(B):
        for g in range(G):
            for h in range(Hkv):
                assert np.array_equal(r[b * G + g, h], q[b, h * G + g])
    assert np.array_equal(gqa_heads(r, B, G), q)
