"""GPU checks of the mixed 4/3-bit latent cache against the oracle's quantiser.

Dequantisation must be bit-exact: rows read back with starkv_dequant equal the oracle's
quantise -> dequantise of the same binary16 rows, for complete groups (codes, scale, zero) and for
the unfinished group (the binary16 tail). The scale / zero bit patterns and the value latent's
packed bytes (same channel-major layout as the oracle) are compared byte for byte too; the key
latent's token-major packing is checked by re-packing the oracle's codes into that layout here.
"""
import numpy as np
import pytest

import oracle
import rank_kv_cache_amd as sk
from rank_kv_cache_amd import synth

from gpu_support import say

pytestmark = pytest.mark.gpu
FRAC = 0.25


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.lib()


def q43_layer(H, d, ranks, rv):
    return sk.Layer(num_heads=H, head_dim=d, key_ranks=tuple(int(r) for r in ranks), value_rank=rv,
                    cache_dtype=sk.Q43, q_top_fraction=FRAC)


def _append(layer, cache, zk, zv, chunks):
    from rank_kv_cache_amd import buffers
    dzk, dzv = buffers.to_device(zk), buffers.to_device(zv)
    pos = 0
    for n in chunks:
        sk.starkv_append_latents(layer, cache, pos, n, dzk[:, pos:pos + n].contiguous(),
                                 dzv[:, pos:pos + n].contiguous())
        pos += n
    return pos


def _readback(layer, cache, T, t0, t1, Ck, Cv):
    import torch
    from rank_kv_cache_amd import buffers
    B = cache.batch
    ok = torch.empty((B, t1 - t0, Ck), dtype=torch.float16, device="cuda")
    ov = torch.empty((B, t1 - t0, Cv), dtype=torch.float16, device="cuda")
    sk.starkv_dequant(layer, cache, T, t0, t1, ok, ov)
    torch.cuda.synchronize()
    return buffers.to_host(ok), buffers.to_host(ov)


def _key_rows_layout(codes_o, bits, cap_blocks):
    """Re-pack the oracle's per-channel codes (channel-major) into the library's token-major key
    layout: per 16-channel group, 64 rows of 48 + n bits (low three bits of each channel, then the
    fourth bits of the n leading 4-bit channels), groups in channel order."""
    C = bits.shape[0]
    off, offs = 0, []
    for c in range(C):
        offs.append(off)
        off += 8 * int(bits[c])
    q = [oracle.unpack_codes(codes_o[offs[c]:offs[c] + 8 * int(bits[c])], int(bits[c]))
         for c in range(C)]
    out = []
    for g16 in range(C // 16):
        ch = list(range(16 * g16, 16 * g16 + 16))
        n = sum(1 for c in ch if bits[c] == 4)
        assert all(bits[c] == 4 for c in ch[:n])
        acc = np.zeros(64 * (48 + n), np.uint8)
        for t in range(64):
            base = t * (48 + n)
            for e, c in enumerate(ch):
                for k in range(3):
                    acc[base + 3 * e + k] = (q[c][t] >> k) & 1
                if e < n:
                    acc[base + 48 + e] = (q[c][t] >> 3) & 1
        out.append(np.packbits(acc, bitorder="little"))
    return np.concatenate(out)


@pytest.mark.parametrize("chunks", [[64 * 3 + 21], [61, 3, 64, 70, 1, 1, 13]])
def test_q43_append_dequant_bit_exact(chunks):
    import torch
    from rank_kv_cache_amd import buffers
    H, d, B = 6, 128, 2
    ranks = [16, 48, 32, 64, 16, 80]
    rv = 272
    T = sum(chunks)
    cap = 64 * 5
    w = synth.Workload("q", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=61,
                       cache_seed=62, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    L = q43_layer(H, d, ranks, rv)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    assert _append(L, cache, zk, zv, chunks) == T
    bits_k = oracle.channel_bits(ranks, FRAC)
    bits_v = oracle.channel_bits([rv], FRAC)
    ck, mk, tk = oracle.q43_pack(zk, bits_k, cap)
    cv, mv, tv = oracle.q43_pack(zv, bits_v, cap)
    say(f"[q43] chunks={chunks} T={T} key block bytes {ck.shape[2]} value block bytes {cv.shape[2]}")
    rk, rvv = _readback(L, cache, T, 0, T, sum(ranks), rv)
    want_k = oracle.q43_unpack(ck, mk, tk, bits_k, T, cap)
    want_v = oracle.q43_unpack(cv, mv, tv, bits_v, T, cap)
    assert np.array_equal(rk.view(np.uint16), want_k.view(np.uint16))
    assert np.array_equal(rvv.view(np.uint16), want_v.view(np.uint16))
    # a sub-range that starts and ends inside groups
    rk2, rv2 = _readback(L, cache, T, 37, 171, sum(ranks), rv)
    assert np.array_equal(rk2.view(np.uint16), want_k[:, 37:171].view(np.uint16))
    assert np.array_equal(rv2.view(np.uint16), want_v[:, 37:171].view(np.uint16))
    # metadata and packed bytes of the complete groups
    full = T // 64
    sizes = sk.starkv_cache_bytes(L, B, cap)
    meta_k = cache.zk_meta.cpu().numpy().view(np.uint16).reshape(B, cap // 64, sum(ranks), 2)
    meta_v = cache.zv_meta.cpu().numpy().view(np.uint16).reshape(B, cap // 64, rv, 2)
    assert np.array_equal(meta_k[:, :full], mk[:, :full])
    assert np.array_equal(meta_v[:, :full], mv[:, :full])
    vbytes = cv.shape[2]
    gv = cache.zv.cpu().numpy()[:B * (cap // 64) * vbytes].reshape(B, cap // 64, vbytes)
    assert np.array_equal(gv[:, :full], cv[:, :full])
    kbytes = (sizes[0] - 32) // (B * (cap // 64))
    gk = cache.zk.cpu().numpy()[:B * (cap // 64) * kbytes].reshape(B, cap // 64, kbytes)
    for b in range(B):
        for g in range(full):
            assert np.array_equal(gk[b, g], _key_rows_layout(ck[b, g], bits_k, cap // 64)), (b, g)
