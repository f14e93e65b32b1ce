"""The C ABI on the CPU: the library loads, exports every function include/starkv.h declares, and
rejects invalid arguments with the documented status before anything is enqueued (so none of
these calls reaches the GPU; device pointers below are never dereferenced)."""
import os
import re
import subprocess

import pytest

import rank_kv_cache_amd as sk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "starkv.h")
FAKE = 0x10000          # 16-byte aligned, never dereferenced: validation rejects first
MISAL = 0x10008


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(starkv_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_header_symbols():
    L = sk.lib()
    decl = declared_functions()
    assert set(decl) == set(sk.EXPORTED_SYMBOLS)
    for name in decl:
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", sk.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (starkv_[a-z_]+)$", out, flags=re.M))
    assert set(decl) <= exported
    assert sk.starkv_version() == 100
    for code in range(10):
        assert sk.starkv_status_string(code)


def _latent(**kw):
    base = dict(num_heads=4, head_dim=128, key_ranks=(16, 32, 48, 64), value_rank=256,
                cache_dtype=sk.F16)
    base.update(kw)
    return sk.Layer(**base)


def _cache(**kw):
    base = dict(batch=2, capacity=256, zk=FAKE, zv=FAKE)
    base.update(kw)
    return sk.Cache(**base)


def st_decode(layer, cache, seq_len=100, q=FAKE, bk=FAKE, bv=FAKE, out=FAKE, ns=0, ws=FAKE,
              nws=1 << 40):
    return sk.starkv_decode_attn(layer, cache, seq_len, q, bk, bv, out, ns, ws, nws, check=False)


def test_decode_validation():
    E = {n: i for i, n in enumerate(["OK", "NULL", "SHAPE", "RANK", "DTYPE", "MISAL", "CAP", "WS",
                                     "UNSUP", "DEV"])}
    L, Cc = _latent(), _cache()
    assert st_decode(None, Cc) == E["NULL"]
    assert st_decode(L, None) == E["NULL"]
    assert st_decode(_latent(num_heads=0), Cc) == E["SHAPE"]
    assert st_decode(_latent(head_dim=63), Cc) == E["SHAPE"]
    assert st_decode(_latent(rope_base=1.0), Cc) == E["SHAPE"]
    assert st_decode(_latent(rope_base=float("nan")), Cc) == E["SHAPE"]
    assert st_decode(_latent(cache_dtype=7), Cc) == E["DTYPE"]
    assert st_decode(_latent(factor_dtype=sk.F32), Cc) == E["DTYPE"]
    assert st_decode(_latent(cache_dtype=sk.Q43, factor_dtype=sk.BF16), Cc) == E["DTYPE"]
    # fp caches take any rank in [1, head_dim]; the mixed 4/3-bit layout needs multiples of 16
    assert st_decode(_latent(cache_dtype=sk.Q43, key_ranks=(16, 32, 40, 64)), Cc) == E["RANK"]
    assert st_decode(_latent(key_ranks=(16, 32, 48, 144)), Cc) == E["RANK"]
    assert st_decode(_latent(key_ranks=(0, 32, 48, 64)), Cc) == E["RANK"]
    assert st_decode(_latent(cache_dtype=sk.Q43, value_rank=100), Cc) == E["RANK"]
    assert st_decode(_latent(value_rank=0), Cc) == E["RANK"]
    assert st_decode(_latent(value_rank=4096), Cc) == E["RANK"]
    assert st_decode(_latent(value_rank=2064), Cc) == E["RANK"]
    assert st_decode(_latent(num_heads=40, key_ranks=(16,) * 40), Cc) == E["UNSUP"]
    assert st_decode(_latent(head_dim=96), Cc) == E["UNSUP"]
    assert st_decode(L, _cache(capacity=100)) == E["CAP"]
    assert st_decode(L, _cache(capacity=0)) == E["CAP"]
    assert st_decode(L, _cache(batch=-1)) == E["SHAPE"]
    assert st_decode(L, _cache(zk=None)) == E["NULL"]
    assert st_decode(L, _cache(zv=MISAL)) == E["MISAL"]
    assert st_decode(L, Cc, seq_len=0) == E["SHAPE"]
    assert st_decode(L, Cc, seq_len=257) == E["CAP"]
    assert st_decode(L, Cc, q=None) == E["NULL"]
    assert st_decode(L, Cc, bk=None) == E["NULL"]
    assert st_decode(L, Cc, out=MISAL) == E["MISAL"]
    assert st_decode(L, Cc, ns=-1) == E["SHAPE"]
    assert st_decode(L, Cc, ws=None) == E["WS"]
    need = sk.starkv_decode_workspace_bytes(L, 2, 100, 0)
    assert need > 0
    assert st_decode(L, Cc, nws=need - 1) == E["WS"]
    assert st_decode(L, Cc, ws=MISAL) == E["MISAL"]
    q43 = _latent(cache_dtype=sk.Q43)
    assert st_decode(q43, Cc) == E["NULL"]                 # meta / tail buffers missing
    assert st_decode(_latent(cache_dtype=sk.Q43, q_group=32), Cc) == E["UNSUP"]
    # empty batch: nothing to do, OK without touching anything
    assert st_decode(L, _cache(batch=0, zk=None, zv=None), q=None, out=None, ws=None) == E["OK"]
    dense = sk.Layer(num_heads=4, head_dim=128, dense=True, cache_dtype=sk.F16)
    assert st_decode(dense, Cc, bk=None, bv=None, ws=None) == E["WS"]
    assert st_decode(sk.Layer(num_heads=4, head_dim=128, dense=True, cache_dtype=sk.Q43), Cc) == E["DTYPE"]


def test_append_and_dequant_validation():
    L, Cc = _latent(), _cache()
    ap = lambda *a, **k: sk.starkv_append_latents(*a, check=False, **k)
    assert ap(L, Cc, -1, 4, FAKE, FAKE) == 2
    assert ap(L, Cc, 0, -4, FAKE, FAKE) == 2
    assert ap(L, Cc, 250, 7, FAKE, FAKE) == 6
    assert ap(L, Cc, 0, 4, None, FAKE) == 1
    assert ap(L, Cc, 0, 4, FAKE, MISAL) == 5
    assert ap(L, Cc, 10, 0, None, None) == 0               # nothing to append
    assert ap(L, _cache(batch=0, zk=None, zv=None), 0, 4, None, None) == 0
    dq = lambda *a: sk.starkv_dequant(*a, check=False)
    assert dq(L, Cc, 100, -1, 5, FAKE, FAKE) == 2
    assert dq(L, Cc, 100, 6, 5, FAKE, FAKE) == 2
    assert dq(L, Cc, 100, 0, 101, FAKE, FAKE) == 6
    assert dq(L, Cc, 300, 0, 10, FAKE, FAKE) == 6
    assert dq(L, Cc, 100, 0, 10, MISAL, None) == 5
    assert dq(L, Cc, 100, 7, 7, FAKE, FAKE) == 0           # empty range


def test_cache_bytes():
    L = _latent()
    s = sk.starkv_cache_bytes(L, 3, 128)
    assert s[0] == 3 * 128 * 160 * 2 and s[1] == 3 * 128 * 256 * 2 and s[2:] == [0, 0, 0, 0]
    Lf = _latent(cache_dtype=sk.F32, factor_dtype=sk.F32)
    assert sk.starkv_cache_bytes(Lf, 1, 64)[0] == 64 * 160 * 4
    D = sk.Layer(num_heads=32, head_dim=128, dense=True, cache_dtype=sk.F16)
    s = sk.starkv_cache_bytes(D, 2, 64)
    assert s[0] == s[1] == 2 * 64 * 4096 * 2
    with pytest.raises(sk.StarkvError):
        sk.starkv_cache_bytes(L, 1, 100)


def test_workspace_sizes_and_planner():
    L = _latent()
    # default: splits = ceil(256 / B) capped by the tile count
    w16 = sk.starkv_decode_workspace_bytes(L, 16, 32768, 0)
    w1 = sk.starkv_decode_workspace_bytes(L, 16, 32768, 1)
    assert w16 > w1 > 0
    assert sk.starkv_decode_workspace_bytes(L, 16, 0, 0) == 0
    assert sk.starkv_decode_workspace_bytes(None, 16, 10, 0) == 0


def test_hadamard_validation():
    """Argument checks of the rotation happen on the host before anything is enqueued."""
    L16 = sk.Layer(num_heads=2, head_dim=64, key_ranks=(16, 32), value_rank=64, cache_dtype=sk.F16)
    L32 = sk.Layer(num_heads=2, head_dim=64, key_ranks=(16, 32), value_rank=64, cache_dtype=sk.F32)
    dense = sk.Layer(num_heads=2, head_dim=64, dense=True, cache_dtype=sk.F16)
    rot = lambda *a: sk.starkv_hadamard_rotate(*a, check=False)
    assert rot(L16, 2, 0, 4, FAKE, FAKE) == 2                # which
    assert rot(L16, 0, 2, 4, FAKE, FAKE) == 2                # kind
    assert rot(L16, 0, 0, -1, FAKE, FAKE) == 2
    assert rot(L16, 0, 1, 63, FAKE, FAKE) == 2               # factor rows need head_dim columns
    assert rot(L16, 1, 1, 64, FAKE, FAKE) == 2               # value factor: H * d columns
    assert rot(L32, 0, 0, 4, FAKE, FAKE) == 4                # binary16 only
    assert rot(dense, 0, 0, 4, FAKE, FAKE) == 8
    assert rot(L16, 0, 0, 4, None, FAKE) == 1
    assert rot(L16, 0, 0, 0, None, None) == 0                # nothing to rotate


def test_output_projection_validation():
    L = _latent()
    op = lambda *a, ws=FAKE, nws=1 << 40: sk.starkv_output_projection(*a, ws, nws, check=False)
    assert op(L, -1, FAKE, FAKE, 8, FAKE) == 2
    assert op(L, 2, FAKE, FAKE, 0, FAKE) == 2
    assert op(L, 2, None, FAKE, 8, FAKE) == 1
    assert op(L, 2, FAKE, FAKE, 8, FAKE, ws=None) == 1
    assert op(L, 2, FAKE, FAKE, 8, 0x10002) == 5               # y needs 4-byte alignment
    assert op(L, 2, FAKE + 4, FAKE, 8, FAKE) == 5              # o needs 16
    assert op(L, 2, FAKE, FAKE, 8, FAKE, nws=16) == 7
    assert op(L, 0, None, None, 8, None, ws=None) == 0         # nothing to project


def test_linear_workspace_sizes():
    """Split planning is host arithmetic: about two 4-wave workgroups per CU, each wave at least
    one 64-wide K tile; the workspace holds one fp32 [rows][outputs] slice per split."""
    L = sk.Layer(num_heads=32, head_dim=128, key_ranks=(16, 32, 48, 64) * 8, value_rank=1024,
                 cache_dtype=sk.F16)
    # 4096 outputs in 32 tiles of 128 -> 16 splits of K = 4096 (one 64-wide tile per wave)
    assert sk.starkv_output_projection_workspace_bytes(L, 16, 4096) == 16 * 16 * 4096 * 4
    # R_k + r_v = 1280 + 1024 outputs (18 tiles) -> 29 wanted, capped at 16 by the K tiles
    assert sk.starkv_append_tokens_workspace_bytes(L, 16, 1, 4096) == 16 * 16 * 2304 * 4
    assert sk.starkv_output_projection_workspace_bytes(L, 0, 4096) == 0
    assert sk.starkv_append_tokens_workspace_bytes(L, 16, 1, 32) == 0
    # many rows: launches of at most 1024 rows; fewer splits as the row tiles grow
    big = sk.starkv_append_tokens_workspace_bytes(L, 16, 4096, 4096)
    assert 1024 * 2304 * 4 <= big <= 2 * 1024 * 2304 * 4


def test_append_tokens_validation():
    L, Cc = _latent(), _cache()
    at = lambda pos=0, n=1, x=FAKE, D=64, ak=FAKE, av=FAKE, ws=FAKE, nws=1 << 40, L=L, Cc=Cc: \
        sk.starkv_append_tokens(L, Cc, pos, n, x, D, ak, av, ws, nws, check=False)
    assert at(pos=-1) == 2 and at(n=-1) == 2 and at(D=0) == 2
    assert at(D=96) == 8                                       # model_dim not a multiple of 64
    assert at(pos=250, n=7) == 6                               # past the capacity (256)
    assert at(n=0, x=None) == 0
    assert at(x=None) == 1 and at(ak=None) == 1 and at(av=None) == 1 and at(ws=None) == 1
    assert at(x=FAKE + 8) == 5 and at(ak=FAKE + 2) == 5
    assert at(nws=0) == 7
    assert at(L=_latent(cache_dtype=sk.BF16, factor_dtype=sk.F16)) == 4
    assert at(Cc=_cache(batch=0), x=None) == 0


def test_rounded_rank_sizes():
    """Ranks that are not multiples of 16 are stored rounded up to the 16-channel tile (the extra
    channels hold zeros): cache and workspace sizes follow the stored widths, while the token
    append's projection works on the true ones."""
    L = _latent(key_ranks=(5, 17, 30, 64), value_rank=100)
    s = sk.starkv_cache_bytes(L, 3, 128)
    assert s[0] == 3 * 128 * (16 + 32 + 32 + 64) * 2 and s[1] == 3 * 128 * 112 * 2
    assert s[2:] == [0, 0, 0, 0]
    L16 = _latent(key_ranks=(16, 32, 32, 64), value_rank=112)
    assert sk.starkv_decode_workspace_bytes(L, 2, 1000) == sk.starkv_decode_workspace_bytes(L16, 2, 1000)
    # append projection outputs: 5 + 17 + 30 + 64 = 116 key + 100 value channels in one tile
    assert sk.starkv_append_tokens_workspace_bytes(L, 2, 1, 64) % 256 == 0
    assert sk.starkv_append_tokens_workspace_bytes(L, 2, 1, 64) >= 2 * 216 * 4
    fp32 = _latent(key_ranks=(1, 2, 3, 4), value_rank=1, cache_dtype=sk.F32)
    assert sk.starkv_cache_bytes(fp32, 1, 64)[0] == 64 * 64 * 4


def test_ragged_validation():
    L, Cc = _latent(), _cache()
    rd = lambda lens=FAKE, Cc=Cc: sk.starkv_decode_attn_ragged(L, Cc, 100, lens, FAKE, FAKE, FAKE,
                                                               FAKE, 0, FAKE, 1 << 40, check=False)
    assert rd(lens=None) == 1
    assert rd(lens=FAKE + 2) == 5
    assert rd(Cc=_cache(batch=0), lens=None) == 0
    assert sk.starkv_decode_attn_ragged(L, Cc, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40,
                                        check=False) == 2
    assert sk.starkv_decode_attn_ragged(L, Cc, 300, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40,
                                        check=False) == 6
    ra = lambda pos=FAKE, zk=FAKE, zv=FAKE, Cc=Cc: sk.starkv_append_latents_ragged(L, Cc, pos, zk,
                                                                                    zv, check=False)
    assert ra(pos=None) == 1 and ra(zk=None) == 1 and ra(zv=None) == 1
    assert ra(pos=FAKE + 2) == 5 and ra(zk=FAKE + 8) == 5
    assert ra(Cc=_cache(batch=0), pos=None) == 0


def test_queries_validation():
    L, Cc = _latent(), _cache()
    dq = lambda n=3, qs=FAKE, ql=FAKE, Cc=Cc, mx=100: sk.starkv_decode_attn_queries(
        L, Cc, n, qs, ql, mx, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40, check=False)
    assert dq(n=-1) == 2
    assert dq(qs=None) == 1 and dq(ql=None) == 1
    assert dq(qs=FAKE + 2) == 5 and dq(ql=FAKE + 1) == 5
    assert dq(n=0, qs=None, ql=None) == 0
    assert dq(Cc=_cache(batch=0)) == 2                      # queries but no cache sequence
    assert dq(mx=0) == 2 and dq(mx=300) == 6


def test_paged_cache_validation():
    L = _latent()
    paged = lambda stride=4, table=FAKE: _cache(block_table=table, table_stride=stride)
    # capacity 256 tokens = 4 blocks per sequence: the table needs at least 4 columns
    assert st_decode(L, paged(stride=3)) == 6
    assert st_decode(L, paged(table=FAKE + 2)) == 5
    import ctypes
    assert ctypes.sizeof(sk._Cache) == 72                    # matches the C struct


def test_multi_validation():
    L, Cc = _latent(), _cache()
    mu = lambda nq=2, lens=None, L=L, Cc=Cc: sk.starkv_decode_attn_multi(
        L, Cc, nq, 100, lens, FAKE, FAKE, FAKE, FAKE, 0, FAKE, 1 << 40, check=False)
    assert mu(nq=0) == 2 and mu(nq=3) == 8 and mu(nq=8) == 8
    assert mu(L=_latent(cache_dtype=sk.F32)) == 8           # fp32 shares keys only with nq = 1
    assert mu(L=sk.Layer(num_heads=4, head_dim=128, dense=True, cache_dtype=sk.F16)) == 8
    assert mu(lens=FAKE + 2) == 5
    assert mu(Cc=_cache(batch=0)) == 0
    assert sk.starkv_decode_multi_workspace_bytes(L, 2, 3, 100) == 0
    a = sk.starkv_decode_multi_workspace_bytes(L, 2, 4, 1000)
    assert a > sk.starkv_decode_workspace_bytes(L, 2, 1000) and a % 256 == 0


def test_decode_length_limits():
    """At most 256 splits of at most 256 / nq blocks of 64 tokens (the value kernel's per-split
    table holds 2 * 256 / nq tile factors per query row and head): longer requests are
    UNSUPPORTED and their workspace size is 0, before anything is enqueued."""
    L = _latent()
    big = _cache(capacity=1 << 23)
    full = 256 * 256 * 64                                    # 4,194,304 tokens
    mu = lambda nq, mx: sk.starkv_decode_attn_multi(L, big, nq, mx, None, FAKE, FAKE, FAKE, FAKE, 0,
                                                    FAKE, 1 << 50, check=False)
    for nq in (1, 2, 4):
        lim = full // nq
        assert sk.starkv_decode_multi_workspace_bytes(L, 2, nq, lim) > 0
        assert sk.starkv_decode_multi_workspace_bytes(L, 2, nq, lim + 1) == 0
        assert mu(nq, lim + 1) == 8
    assert st_decode(L, big, seq_len=full + 1, nws=1 << 50) == 8
    assert sk.starkv_decode_workspace_bytes(L, 2, full) > 0
    assert sk.starkv_decode_workspace_bytes(L, 2, full + 1) == 0
    dense = sk.Layer(num_heads=4, head_dim=128, dense=True, cache_dtype=sk.F16)
    assert st_decode(dense, big, seq_len=full + 1, nws=1 << 50) == 8


def test_noalloc_validation():
    """The no-allocation decode refuses requests whose workspace exceeds its fixed array, and
    invalid ones with the shared validation's status, before any device work (and before it
    looks up the array's device address)."""
    L = _latent(num_heads=32, key_ranks=(64,) * 32, value_rank=2048)
    big = _cache(batch=64, capacity=1 << 16)
    assert sk.starkv_decode_attn_noalloc_max_bytes() == 64 << 20
    assert sk.starkv_decode_workspace_bytes(L, 64, 1 << 16, 0) > 64 << 20
    na = lambda L=L, Cc=big, T=1 << 16: sk.starkv_decode_attn_noalloc(L, Cc, T, FAKE, FAKE, FAKE,
                                                                      FAKE, 0, check=False)
    assert na() == 7
    assert na(Cc=_cache(batch=64, capacity=1 << 23), T=(1 << 22) + 64) == 8   # beyond the planner
    assert na(L=None) == 1 and na(Cc=None) == 1 and na(T=0) == 2
    assert na(Cc=_cache(batch=0), T=100) == 0                                    # nothing to do


def test_prefill_validation():
    L, Cc = _latent(), _cache()
    pf = lambda L=L, Cc=Cc, pos0=10, chunk=20, lens=None, q=FAKE, ws=FAKE, nws=1 << 40: \
        sk.starkv_prefill_attn(L, Cc, pos0, chunk, lens, q, FAKE, FAKE, FAKE, ws, nws, check=False)
    assert sk.starkv_prefill_workspace_bytes(L, 2, 10, 20) > 0
    assert pf(pos0=-1) == 2 and pf(chunk=0) == 2
    assert pf(pos0=200, chunk=100) == 6                      # beyond the capacity of 256
    assert pf(L=sk.Layer(num_heads=4, head_dim=128, dense=True, cache_dtype=sk.F16)) == 8
    assert pf(L=_latent(cache_dtype=sk.F32, factor_dtype=sk.F32)) == 8
    assert pf(q=None) == 1 and pf(q=MISAL) == 5 and pf(lens=FAKE + 2) == 5
    assert pf(ws=None) == 7 and pf(nws=16) == 7
    assert pf(Cc=_cache(batch=0)) == 0
    assert sk.starkv_prefill_workspace_bytes(L, 2, -1, 20) == 0
    assert sk.starkv_prefill_workspace_bytes(L, 2, 0, 0) == 0
    # the length limit (4,194,304 tokens of fill) and the query-count limit (batch * chunk <= 2^30)
    big = _cache(capacity=1 << 23)
    assert pf(Cc=big, pos0=(1 << 22) - 10, chunk=20) == 8
    assert sk.starkv_prefill_workspace_bytes(L, 2, (1 << 22) - 10, 20) == 0
    assert pf(Cc=_cache(batch=1 << 11, capacity=1 << 20), pos0=0, chunk=(1 << 19) + 64) == 8
    # 16-bit key latents are read in place: only the mixed 4/3-bit layer stages key rows
    q43 = _latent(cache_dtype=sk.Q43)
    Rk, T = 16 + 32 + 48 + 64, 32
    assert sk.starkv_prefill_workspace_bytes(q43, 2, 0, T) >= \
        sk.starkv_prefill_workspace_bytes(L, 2, 0, T) + 2 * T * Rk * 2


def test_decode_project_validation():
    L, Cc = _latent(), _cache()
    dp = lambda Cc=Cc, hidden=300, wo=FAKE, y=FAKE, T=100, ws=FAKE, nws=1 << 40: \
        sk.starkv_decode_attn_project(L, Cc, T, FAKE, FAKE, FAKE, wo, hidden, y, 0, ws, nws, check=False)
    assert sk.starkv_decode_attn_project_workspace_bytes(L, 2, 100, 0, 300) > \
        sk.starkv_decode_workspace_bytes(L, 2, 100, 0)
    assert dp(hidden=0) == 2 and dp(wo=None) == 1 and dp(y=None) == 1
    assert dp(wo=MISAL) == 5 and dp(y=FAKE + 2) == 5
    assert dp(T=300) == 6 and dp(T=0) == 2                   # the decode's own validation
    assert dp(ws=None) == 7 and dp(nws=64) == 7
    assert dp(Cc=_cache(batch=0)) == 0
