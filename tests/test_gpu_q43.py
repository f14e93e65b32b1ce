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
    # library meta layout: per block a row of scales then a row of zero points
    meta_k = cache.zk_meta.cpu().numpy().view(np.uint16).reshape(B, cap // 64, 2, sum(ranks)).transpose(0, 1, 3, 2)
    meta_v = cache.zv_meta.cpu().numpy().view(np.uint16).reshape(B, cap // 64, 2, rv).transpose(0, 1, 3, 2)
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


def _q43_reference(ld, zk16, zv16, q, ranks, rv, T, cap, pairs=None):
    """Oracle attention on the oracle's own quantise -> dequantise of the same binary16 rows."""
    bits_k = oracle.channel_bits(ranks, FRAC)
    bits_v = oracle.channel_bits([rv], FRAC)
    ck, mk, tk = oracle.q43_pack(zk16, bits_k, cap)
    cv, mv, tv = oracle.q43_pack(zv16, bits_v, cap)
    dk = oracle.q43_unpack(ck, mk, tk, bits_k, T, cap)
    dv = oracle.q43_unpack(cv, mv, tv, bits_v, T, cap)
    return oracle.decode_latent(dk, dv, ld.bk, ld.bv, q, ranks, pairs=pairs)


def _gpu_decode(L, cache, T, q, bk, bv, num_splits=0):
    import torch
    from rank_kv_cache_amd import buffers
    B = cache.batch
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    ws, nws = buffers.alloc_workspace(L, B, T, num_splits)
    ws.fill_(0xFF)
    sk.starkv_decode_attn(L, cache, T, buffers.to_device(np.ascontiguousarray(q, np.float32)),
                          buffers.to_device(bk), buffers.to_device(bv), out, num_splits, ws, nws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_q43_decode_parity_rotated():
    """Blockwise-Hadamard-rotated latents and factors (rotation by the oracle, as offline
    preparation), mixed 4/3-bit cache built by chunked appends, decode at several lengths
    including a partial last group."""
    from rank_kv_cache_amd import buffers
    from gpu_support import rel_err
    H, d, B = 6, 128, 2
    ranks = [16, 48, 32, 64, 16, 80]
    rv = 272
    T, cap = 64 * 3 + 21, 64 * 5
    w = synth.Workload("qd", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=71,
                       cache_seed=72, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(72, 0, B, H, d)
    seg_k = oracle.latent_segments(ranks, FRAC)
    seg_v = oracle.latent_segments([rv], FRAC)
    zk_r, zv_r = oracle.rotate_rows(zk, seg_k), oracle.rotate_rows(zv, seg_v)
    ld.bk = oracle.rotate_factor(ld.bk, seg_k)
    ld.bv = oracle.rotate_factor(ld.bv, seg_v)
    L = q43_layer(H, d, ranks, rv)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    _append(L, cache, zk_r, zv_r, [61, 3, 64, 70, 1, 1, 13])
    for Tq in (T, 192, 64):
        ref = _q43_reference(ld, zk_r[:, :Tq], zv_r[:, :Tq], q, ranks, rv, Tq, cap)
        for S in (0, 1, 3):
            got = _gpu_decode(L, cache, Tq, q, ld.bk, ld.bv, S)
            e = rel_err(got, ref)
            say(f"[q43 decode] T={Tq} splits={S} rel err {e:.3e}")
            # same dequantised values on both sides: only fp32 vs fp64 arithmetic differs
            assert np.all(np.isfinite(got)) and e <= 2e-3


def _device_rotate(L, which, kind, n, x16):
    import torch
    from rank_kv_cache_amd import buffers
    src = buffers.to_device(x16)
    dst = torch.empty(src.shape, dtype=torch.float16, device="cuda")
    sk.starkv_hadamard_rotate(L, which, kind, n, src, dst)
    del src
    return dst


def test_q43_decode_full_size_sampled():
    """The quantised LongChat-shaped workload at full size (B=16, T=16384) in the library's
    default launch configuration, on blockwise-Hadamard-rotated latents and factors as the
    quantised configuration specifies (Zhou notes, section 6.1 and Fig. 5: rotate, then quantise).
    The GPU side rotates every row with the device rotation; the oracle rotates the sampled
    sequences itself, and the two rotations must agree bit for bit on them. The oracle then
    evaluates sampled (sequence, head) pairs on its own quantisation and dequantisation of its
    own rotated rows."""
    import torch
    from rank_kv_cache_amd import buffers
    from gpu_support import rel_err
    w = synth.WORKLOADS["longchat_b16_t16384_q43"]
    ld = synth.draw_layer(w)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(w.cache_seed, 0, w.batch, w.heads, w.head_dim)
    ranks, rv = ld.key_ranks, ld.value_rank
    B, T, H, d = w.batch, w.seq_len, w.heads, w.head_dim
    L = q43_layer(H, d, ranks, rv)
    seg_k = oracle.latent_segments(ranks, FRAC)
    seg_v = oracle.latent_segments([rv], FRAC)
    dzk = _device_rotate(L, 0, 0, B * T, zk)
    dzv = _device_rotate(L, 1, 0, B * T, zv)
    dbk = _device_rotate(L, 0, 1, d, ld.bk)
    dbv = _device_rotate(L, 1, 1, H * d, ld.bv)
    cache = buffers.alloc_cache(L, B, T)
    sk.starkv_append_latents(L, cache, 0, T, dzk, dzv)
    out = torch.full((B, H, d), float("nan"), dtype=torch.float32, device="cuda")
    ws, nws = buffers.alloc_workspace(L, B, T, 0)
    sk.starkv_decode_attn(L, cache, T, buffers.to_device(q), dbk, dbv, out, 0, ws, nws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    sel_b = [0, B - 1]
    zk_r = oracle.rotate_rows(zk[sel_b], seg_k)
    zv_r = oracle.rotate_rows(zv[sel_b], seg_v)
    bk_r = oracle.rotate_factor(ld.bk, seg_k)
    bv_r = oracle.rotate_factor(ld.bv, seg_v)
    for dev, host in ((dzk, zk_r), (dzv, zv_r)):
        assert np.array_equal(buffers.to_host(dev[sel_b]).view(np.uint16), host.view(np.uint16))
    assert np.array_equal(buffers.to_host(dbk).view(np.uint16), bk_r.view(np.uint16))
    assert np.array_equal(buffers.to_host(dbv).view(np.uint16), bv_r.view(np.uint16))
    del dzk, dzv
    rng = np.random.default_rng(7)
    pairs = [(0, 0), (1, H - 1)] + [(int(rng.integers(0, 2)), int(h)) for h in rng.integers(0, H, 6)]
    ld.bk, ld.bv = bk_r, bv_r
    ref = _q43_reference(ld, zk_r, zv_r, q[sel_b], ranks, rv, T, T, pairs=pairs)
    sub = np.stack([got[sel_b[b], h] for b, h in pairs])
    e = rel_err(sub, ref)
    say(f"[q43 full, rotated] sampled {len(pairs)} pairs rel err {e:.3e}")
    assert np.all(np.isfinite(got)) and e <= 2e-3


@pytest.mark.parametrize("which,kind", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_hadamard_rotate_bit_exact(which, kind):
    """Device blockwise Hadamard rotation of binary16 latent rows (kind 0) and factor rows (kind 1)
    equals the oracle's rotation bit for bit: exact signed sums, one fp64 product with 1/sqrt(b),
    one rounding to binary16. Ranks include widths whose block size is below 64 (hi parts of 4, 12
    channels; r_v = 272 splits into 68 + 204)."""
    import torch
    from rank_kv_cache_amd import buffers
    H, d = 6, 128
    ranks = [16, 48, 32, 64, 16, 80]
    rv = 272
    L = q43_layer(H, d, ranks, rv)
    rng = np.random.default_rng(90 + 2 * which + kind)
    C = sum(ranks) if which == 0 else rv
    segs = oracle.latent_segments(ranks if which == 0 else [rv], FRAC)
    if kind == 0:
        n = 37
        x = (rng.standard_normal((n, C)) * 3.0).astype(np.float16)
        x[0, :8] = np.array([65504, -65504, 6e-8, -6e-8, 0, -0.0, 1e-5, 2.0], np.float16)
        want = oracle.rotate_rows(x, segs)
    else:
        n = d if which == 0 else H * d
        x = (rng.standard_normal((C, n)) / np.sqrt(16)).astype(np.float16)
        want = oracle.rotate_factor(x, segs)
    src = buffers.to_device(x)
    dst = torch.full(x.shape, float("nan"), dtype=torch.float16, device="cuda")
    sk.starkv_hadamard_rotate(L, which, kind, n, src, dst)
    torch.cuda.synchronize()
    got = buffers.to_host(dst)
    bad = np.argwhere(got.view(np.uint16) != want.view(np.uint16))
    say(f"[hadamard] which={which} kind={kind} mismatches {len(bad)}")
    assert len(bad) == 0, bad[:5]


@pytest.mark.parametrize("T", [1, 37, 64, 65, 130])
def test_q43_decode_short_lengths(T):
    """Quantised caches holding only a tail (T < 64), exactly one group, and one group plus a
    short tail, built by 1-token appends at the end; decode over all appended tokens."""
    from rank_kv_cache_amd import buffers
    from gpu_support import rel_err
    H, d, B = 6, 128, 2
    ranks = [16, 48, 32, 64, 16, 80]
    rv = 272
    cap = 192
    w = synth.Workload("qs", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=81,
                       cache_seed=82 + T, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(83, T, B, H, d)
    L = q43_layer(H, d, ranks, rv)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    chunks = [T] if T < 3 else [T - 2, 1, 1]
    _append(L, cache, zk, zv, chunks)
    ref = _q43_reference(ld, zk, zv, q, ranks, rv, T, cap)
    for S in (0, 2):
        got = _gpu_decode(L, cache, T, q, ld.bk, ld.bv, S)
        e = rel_err(got, ref)
        say(f"[q43 short] T={T} splits={S} rel err {e:.3e}")
        assert np.all(np.isfinite(got)) and e <= 2e-3


@pytest.mark.parametrize("ranks", [[64, 80, 96, 64, 48, 128], [16, 96, 16, 16, 112, 16]])
def test_q43_decode_rank_mixes(ranks):
    """Mostly large key ranks, and a few large heads among rank-16 ones, against the oracle on the
    same dequantised values."""
    from rank_kv_cache_amd import buffers
    from gpu_support import rel_err
    H, d, B, T, rv = len(ranks), 128, 2, 700, 208
    cap = 768
    w = synth.Workload("qk", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=91,
                       cache_seed=92, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(93, 0, B, H, d)
    L = q43_layer(H, d, ranks, rv)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    _append(L, cache, zk, zv, [T])
    ref = _q43_reference(ld, zk, zv, q, ranks, rv, T, cap)
    for S in (0, 2):
        got = _gpu_decode(L, cache, T, q, ld.bk, ld.bv, S)
        e = rel_err(got, ref)
        say(f"[q43 ranks] mean rank {np.mean(ranks):.1f} splits={S} rel err {e:.3e}")
        assert np.all(np.isfinite(got)) and e <= 2e-3


@pytest.mark.parametrize("frac,d,ranks", [(0.2, 128, [16, 48, 80, 32]), (0.2, 128, [16, 32, 64, 48, 32]),
                                           (1.0, 128, [16, 48, 80, 32]), (0.0, 128, [16, 48, 80, 32]),
                                           (0.25, 64, [16, 32, 48, 64])])
def test_q43_fractions_and_head_dim(frac, d, ranks):
    """Quantisation variants the pages measure: the paper's 20 % at 4 bits (3.2 bits per value),
    uniform 4-bit (fraction 1), uniform 3-bit (fraction 0), and head_dim 64. Read-back must be
    bit-exact and decode within tolerance of the oracle's dequantisation, with the fraction passed
    as the binary32 value the library receives. The second 20 % case keeps every rank at or below
    64 (the score kernel's staged path) with odd counts of 4-bit channels, so head code runs start
    8 bytes past a 16-byte boundary."""
    from rank_kv_cache_amd import buffers
    from gpu_support import rel_err
    H, B = len(ranks), 2
    if ranks == [16, 32, 64, 48, 32]:
        # byte offset of each head's code run in a block: 16-channel groups of 48 + n bits per token
        bits = oracle.channel_bits(ranks, float(np.float32(frac)))
        starts, off, c = [], 0, 0
        for r in ranks:
            starts.append(off)
            for g in range(r // 16):
                off += 8 * (48 + int((bits[c + 16 * g:c + 16 * g + 16] == 4).sum()))
            c += r
        assert any(x % 16 == 8 for x in starts), starts
    rv = 208
    T, cap = 150, 192
    f32 = float(np.float32(frac))
    w = synth.Workload("qf", batch=B, heads=H, head_dim=d, seq_len=T, dtype="f16", layer_seed=91,
                       cache_seed=92, value_rank=rv, power=0.5)
    ld = synth.draw_layer(w, key_ranks=ranks)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(93, 0, B, H, d)
    L = sk.Layer(num_heads=H, head_dim=d, key_ranks=tuple(ranks), value_rank=rv, cache_dtype=sk.Q43,
                 q_top_fraction=frac)
    cache = buffers.alloc_cache(L, B, cap, fill=0xFF)
    _append(L, cache, zk, zv, [100, 1, 49])
    bits_k = oracle.channel_bits(ranks, f32)
    bits_v = oracle.channel_bits([rv], f32)
    ck, mk, tk = oracle.q43_pack(zk, bits_k, cap)
    cv, mv, tv = oracle.q43_pack(zv, bits_v, cap)
    dk = oracle.q43_unpack(ck, mk, tk, bits_k, T, cap)
    dv = oracle.q43_unpack(cv, mv, tv, bits_v, T, cap)
    rk, rvv = _readback(L, cache, T, 0, T, sum(ranks), rv)
    assert np.array_equal(rk.view(np.uint16), dk.view(np.uint16))
    assert np.array_equal(rvv.view(np.uint16), dv.view(np.uint16))
    ref = oracle.decode_latent(dk, dv, ld.bk, ld.bv, q, ranks)
    got = _gpu_decode(L, cache, T, q, ld.bk, ld.bv)
    e = rel_err(got, ref)
    say(f"[q43 frac] frac={frac} d={d} 4-bit channels k={int((bits_k == 4).sum())} v={int((bits_v == 4).sum())} rel err {e:.3e}")
    assert np.all(np.isfinite(got)) and e <= 2e-3
