"""Python face of the fp64 CPU oracle (``oracle/starkv_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` use it. The HIP library never imports it and it never imports the HIP library; the
two meet only through arrays drawn by ``rank_kv_cache_amd.synth``.

The arithmetic lives in C (plain loops, fp64). This module marshals numpy arrays and holds the
layer-level bookkeeping the oracle needs (key offsets, rotation segments, per-channel bit widths),
each restated from the pages' description (citations in the C file and next to each helper).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "starkv_oracle.c")
# STARKV_ORACLE_LIB names another build of the same source (the sanitizer build of the tests)
_LIB = os.environ.get("STARKV_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

F64, F32, F16, BF16 = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, fp64, OpenMP over independent (b, h) pairs)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fno-fast-math",
                               "-ffp-contract=off", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def build_sanitized(out: str) -> str:
    """The same source with AddressSanitizer and UndefinedBehaviorSanitizer (gcc), for the
    sanitizer test; load it through STARKV_ORACLE_LIB with the sanitizer runtimes preloaded."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fno-fast-math",
                           "-ffp-contract=off", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                           "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, out)
    return out


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = C.CDLL(_LIB)
        vp, dp, ip = C.c_void_p, C.POINTER(C.c_double), C.POINTER(C.c_int)
        L.orc_f16_to_f64.restype = C.c_double
        L.orc_f16_to_f64.argtypes = [C.c_uint16]
        L.orc_f64_to_f16.restype = C.c_uint16
        L.orc_f64_to_f16.argtypes = [C.c_double]
        L.orc_bf16_to_f64.restype = C.c_double
        L.orc_bf16_to_f64.argtypes = [C.c_uint16]
        L.orc_f64_to_bf16.restype = C.c_uint16
        L.orc_f64_to_bf16.argtypes = [C.c_double]
        L.orc_round_array.restype = None
        L.orc_round_array.argtypes = [C.c_long, dp, C.c_int, vp]
        L.orc_rope_theta.restype = C.c_double
        L.orc_rope_theta.argtypes = [C.c_int, C.c_int, C.c_double]
        L.orc_rope.restype = None
        L.orc_rope.argtypes = [dp, C.c_int, C.c_double, C.c_double, dp]
        L.orc_decode_latent.restype = C.c_int
        L.orc_decode_latent.argtypes = [C.c_int, C.c_int, C.c_int, C.c_long, ip, C.c_int, C.c_int,
                                        vp, vp, dp, dp, dp, C.c_double, C.c_double, C.c_int, ip,
                                        C.c_int, dp]
        L.orc_decode_dense.restype = C.c_int
        L.orc_decode_dense.argtypes = [C.c_int, C.c_int, C.c_int, C.c_long, C.c_int, vp, vp, dp,
                                       C.c_double, C.c_double, C.c_int, ip, dp]
        L.orc_hadamard.restype = C.c_int
        L.orc_hadamard.argtypes = [C.c_int, dp]
        L.orc_hadamard_block.restype = C.c_int
        L.orc_hadamard_block.argtypes = [C.c_int]
        L.orc_n_hi.restype = C.c_int
        L.orc_n_hi.argtypes = [C.c_int, C.c_double]
        L.orc_rotate_rows_f64.restype = C.c_int
        L.orc_rotate_rows_f64.argtypes = [C.c_long, C.c_int, C.c_int, ip, dp, dp]
        L.orc_rotate_factor_f64.restype = C.c_int
        L.orc_rotate_factor_f64.argtypes = [C.c_int, C.c_int, C.c_int, ip, dp, dp]
        L.orc_rotate_rows_f16.restype = C.c_int
        L.orc_rotate_rows_f16.argtypes = [C.c_long, C.c_int, C.c_int, ip, vp, vp]
        L.orc_rotate_factor_f16.restype = C.c_int
        L.orc_rotate_factor_f16.argtypes = [C.c_int, C.c_int, C.c_int, ip, vp, vp]
        L.orc_quantize_group.restype = None
        L.orc_quantize_group.argtypes = [vp, C.c_long, C.c_int, vp, vp, vp]
        L.orc_unpack_code.restype = C.c_int
        L.orc_unpack_code.argtypes = [vp, C.c_int, C.c_int]
        L.orc_dequant_value.restype = C.c_uint16
        L.orc_dequant_value.argtypes = [C.c_int, C.c_uint16, C.c_uint16]
        L.orc_q43_block_bytes.restype = C.c_long
        L.orc_q43_block_bytes.argtypes = [C.c_int, vp]
        L.orc_q43_pack.restype = C.c_int
        L.orc_q43_pack.argtypes = [C.c_int, C.c_long, C.c_long, C.c_int, vp, vp, vp, vp, vp]
        L.orc_q43_unpack.restype = C.c_int
        L.orc_q43_unpack.argtypes = [C.c_int, C.c_long, C.c_long, C.c_int, vp, vp, vp, vp,
                                     C.c_long, C.c_long, vp]
        L.orc_threads.restype = C.c_int
        L.orc_threads.argtypes = []
        L.orc_set_threads.restype = None
        L.orc_set_threads.argtypes = [C.c_int]
        _lib = L
    return _lib


def _dp(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_double))


def _ip(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int))


def _vp(a: np.ndarray):
    return C.c_void_p(a.ctypes.data)


def _latent_dtype(a: np.ndarray, bf16: bool) -> int:
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16
    if a.dtype == np.uint16 and bf16:
        return BF16
    raise TypeError(f"unsupported latent dtype {a.dtype} (bf16={bf16})")


def to_f64(a: np.ndarray, bf16: bool = False) -> np.ndarray:
    """Exact widening of fp32 / fp16 / bf16-bit arrays to fp64."""
    if a.dtype == np.uint16 and bf16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def threads() -> int:
    return int(lib().orc_threads())


def set_threads(n: int) -> None:
    """OpenMP threads of later oracle calls (timing only: results do not depend on it)."""
    lib().orc_set_threads(int(n))


# ----------------------------------------------------------------------------------------------
# scalar formats
# ----------------------------------------------------------------------------------------------

def f16_to_f64(bits: int) -> float:
    return float(lib().orc_f16_to_f64(int(bits)))


def f64_to_f16(x: float) -> int:
    return int(lib().orc_f64_to_f16(float(x)))


def f64_to_bf16(x: float) -> int:
    return int(lib().orc_f64_to_bf16(float(x)))


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values once, nearest-even, to a storage type: "f32" (float32 array), "f16"
    (float16 array) or "bf16" (uint16 bit patterns)."""
    x64 = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    code = {"f32": F32, "f16": F16, "bf16": BF16}[dtype]
    out = np.empty(x64.shape, {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}[dtype])
    lib().orc_round_array(x64.size, _dp(x64), code, _vp(out))
    return out.view(np.float16) if dtype == "f16" else out


# ----------------------------------------------------------------------------------------------
# RoPE and attention
# ----------------------------------------------------------------------------------------------

def rope_theta(i: int, d: int, base: float = 10000.0) -> float:
    return float(lib().orc_rope_theta(i, d, base))


def rope(x: np.ndarray, pos: float, base: float = 10000.0) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty_like(x)
    lib().orc_rope(_dp(x), x.shape[0], float(pos), float(base), _dp(out))
    return out


def _pairs_arr(pairs, B, H):
    if pairs is None:
        return None, B * H
    p = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    assert np.all((p[:, 0] >= 0) & (p[:, 0] < B) & (p[:, 1] >= 0) & (p[:, 1] < H))
    return p, p.shape[0]


def decode_latent(zk, zv, bk, bv, q, key_ranks, *, rope_base=10000.0, scale=None, pairs=None,
                  form="latent", bf16=False, seq_len=None) -> np.ndarray:
    """fp64 decode attention over latent caches.

    zk [B, T, R_k], zv [B, T, r_v] (fp64 / fp32 / fp16, or bf16 bits with ``bf16=True``);
    bk [R_k, d], bv [r_v, H*d]; q [B, H, d] (post-RoPE); key_ranks [H].
    Returns [B, H, d], or [len(pairs), d] when ``pairs`` lists (b, h) pairs.
    ``seq_len`` (default T) attends to the first seq_len cached tokens.
    """
    zk = np.ascontiguousarray(zk)
    zv = np.ascontiguousarray(zv)
    B, T, Rk = zk.shape
    if seq_len is not None and seq_len != T:
        zk = np.ascontiguousarray(zk[:, :seq_len])
        zv = np.ascontiguousarray(zv[:, :seq_len])
        T = seq_len
    rv = zv.shape[2]
    kr = np.ascontiguousarray(np.asarray(key_ranks, dtype=np.int32))
    H = kr.shape[0]
    assert int(kr.sum()) == Rk
    bk64 = np.ascontiguousarray(to_f64(bk, bf16))
    bv64 = np.ascontiguousarray(to_f64(bv, bf16))
    d = bk64.shape[1]
    assert bv64.shape == (rv, H * d)
    q64 = np.ascontiguousarray(np.asarray(q, dtype=np.float64))
    assert q64.shape == (B, H, d)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    p, n = _pairs_arr(pairs, B, H)
    out = np.empty((n, d), np.float64)
    dt = _latent_dtype(zk, bf16)
    assert _latent_dtype(zv, bf16) == dt
    rc = lib().orc_decode_latent(B, H, d, T, _ip(kr), rv, dt, _vp(zk), _vp(zv), _dp(bk64),
                                 _dp(bv64), _dp(q64), float(rope_base), float(scale), n,
                                 None if p is None else _ip(p), 0 if form == "latent" else 1,
                                 _dp(out))
    if rc != 0:
        raise RuntimeError("orc_decode_latent failed")
    return out.reshape(B, H, d) if pairs is None else out


def decode_dense(k, v, q, *, rope_base=10000.0, scale=None, pairs=None, bf16=False,
                 seq_len=None) -> np.ndarray:
    """fp64 decode attention for a dense (exempt) layer: k, v [B, T, H*d] pre-RoPE, q [B, H, d]."""
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    B, T, W = k.shape
    if seq_len is not None and seq_len != T:
        k = np.ascontiguousarray(k[:, :seq_len])
        v = np.ascontiguousarray(v[:, :seq_len])
        T = seq_len
    q64 = np.ascontiguousarray(np.asarray(q, dtype=np.float64))
    H, d = q64.shape[1], q64.shape[2]
    assert W == H * d
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    p, n = _pairs_arr(pairs, B, H)
    out = np.empty((n, d), np.float64)
    dt = _latent_dtype(k, bf16)
    rc = lib().orc_decode_dense(B, H, d, T, dt, _vp(k), _vp(v), _dp(q64), float(rope_base),
                                float(scale), n, None if p is None else _ip(p), _dp(out))
    if rc != 0:
        raise RuntimeError("orc_decode_dense failed")
    return out.reshape(B, H, d) if pairs is None else out


# ----------------------------------------------------------------------------------------------
# Blockwise Hadamard rotation and mixed-precision bookkeeping
# ----------------------------------------------------------------------------------------------

def output_projection(out: np.ndarray, wo_t: np.ndarray, bf16: bool = False) -> np.ndarray:
    """Notes, Algorithm 2 step 8: y[b] = concat_h(out[b][h]) . W_o in fp64 (a plain matrix
    product). out [B, H, d]; wo_t = W_o transposed, [hidden, H*d] (fp64 / fp32 / fp16, or bf16
    bits with bf16=True)."""
    o = np.asarray(out, dtype=np.float64)
    B = o.shape[0]
    return o.reshape(B, -1) @ to_f64(np.asarray(wo_t), bf16).T


def project_tokens(x: np.ndarray, a_k_t: np.ndarray, a_v_t: np.ndarray, dtype: str):
    """Notes, Algorithm 2 steps 1-2: the new tokens' key and value latents x . A_k and x . A_v in
    fp64 (plain matrix products; any rotation is already inside the weights), each rounded once
    to the storage type ("f32", "f16", "bf16"; binary16 for a mixed 4/3-bit cache).
    x [B, n, D]; a_k_t = A_k transposed [C_k, D], a_v_t [C_v, D] (fp64 / fp32 / fp16, or bf16
    bits when dtype is "bf16"). Returns (zk [B, n, C_k], zv [B, n, C_v]) in the storage type."""
    bf16 = dtype == "bf16"
    x64 = np.asarray(x, dtype=np.float64)
    zk = x64 @ to_f64(np.asarray(a_k_t), bf16).T
    zv = x64 @ to_f64(np.asarray(a_v_t), bf16).T
    return round_to_storage(zk, dtype), round_to_storage(zv, dtype)


def hadamard(n: int) -> np.ndarray:
    out = np.empty((n, n), np.float64)
    if lib().orc_hadamard(n, _dp(out)) != 0:
        raise ValueError("n must be a power of two")
    return out


def hadamard_block(width: int) -> int:
    return int(lib().orc_hadamard_block(width))


def n_hi(r: int, frac: float) -> int:
    return int(lib().orc_n_hi(r, frac))


def latent_segments(ranks, frac: float):
    """Rotation segments (start, width) of a concatenation of latents of the given widths: each
    latent contributes its first n_hi channels and its remaining channels (empty ones dropped)."""
    segs, off = [], 0
    for r in ranks:
        nh = n_hi(int(r), frac)
        if nh > 0:
            segs.append((off, nh))
        if r - nh > 0:
            segs.append((off + nh, int(r) - nh))
        off += int(r)
    return np.asarray(segs, dtype=np.int32).reshape(-1, 2)


def channel_bits(ranks, frac: float, bits_hi: int = 4, bits_lo: int = 3) -> np.ndarray:
    out = []
    for r in ranks:
        nh = n_hi(int(r), frac)
        out += [bits_hi] * nh + [bits_lo] * (int(r) - nh)
    return np.asarray(out, dtype=np.uint8)


def rotate_rows(x: np.ndarray, segs: np.ndarray) -> np.ndarray:
    """x [..., C] -> x . blockdiag(H) over the segments. fp64 in/out, or fp16 in/out (rounded)."""
    shape = x.shape
    Cw = shape[-1]
    segs = np.ascontiguousarray(segs, dtype=np.int32)
    if x.dtype == np.float16:
        xs = np.ascontiguousarray(x).view(np.uint16).reshape(-1, Cw)
        out = np.empty_like(xs)
        lib().orc_rotate_rows_f16(xs.shape[0], Cw, segs.shape[0], _ip(segs), _vp(xs), _vp(out))
        return out.view(np.float16).reshape(shape)
    xs = np.ascontiguousarray(x, dtype=np.float64).reshape(-1, Cw)
    out = np.empty_like(xs)
    lib().orc_rotate_rows_f64(xs.shape[0], Cw, segs.shape[0], _ip(segs), _dp(xs), _dp(out))
    return out.reshape(shape)


def rotate_factor(bmat: np.ndarray, segs: np.ndarray) -> np.ndarray:
    """bmat [C, ncols] -> blockdiag(H)^T . bmat over the row segments (fp64, or fp16 rounded)."""
    Cr, ncols = bmat.shape
    segs = np.ascontiguousarray(segs, dtype=np.int32)
    if bmat.dtype == np.float16:
        bs = np.ascontiguousarray(bmat).view(np.uint16)
        out = np.empty_like(bs)
        lib().orc_rotate_factor_f16(Cr, ncols, segs.shape[0], _ip(segs), _vp(bs), _vp(out))
        return out.view(np.float16)
    bs = np.ascontiguousarray(bmat, dtype=np.float64)
    out = np.empty_like(bs)
    lib().orc_rotate_factor_f64(Cr, ncols, segs.shape[0], _ip(segs), _dp(bs), _dp(out))
    return out


def quantize_group(x16: np.ndarray, bits: int):
    """64 fp16 values -> (packed code bytes, scale bits, zero bits)."""
    xs = np.ascontiguousarray(np.asarray(x16, dtype=np.float16)).view(np.uint16)
    assert xs.shape == (64,)
    codes = np.zeros(8 * bits, np.uint8)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint16)
    lib().orc_quantize_group(_vp(xs), 1, bits, _vp(codes), _vp(s), _vp(z))
    return codes, int(s[0]), int(z[0])


def unpack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    return np.array([lib().orc_unpack_code(_vp(c), bits, t) for t in range(64)], np.int32)


def dequant_value(code: int, s16: int, z16: int) -> int:
    return int(lib().orc_dequant_value(int(code), int(s16), int(z16)))


def q43_block_bytes(bits: np.ndarray) -> int:
    b = np.ascontiguousarray(bits, dtype=np.uint8)
    return int(lib().orc_q43_block_bytes(b.shape[0], _vp(b)))


def q43_pack(x16: np.ndarray, bits: np.ndarray, capacity: int):
    """x16 [B, T, C] fp16 -> (codes [B, cap/64, block_bytes] u8, meta [B, cap/64, C, 2] u16,
    tail [B, 64, C] u16)."""
    x = np.ascontiguousarray(x16, dtype=np.float16).view(np.uint16)
    B, T, Cw = x.shape
    b = np.ascontiguousarray(bits, dtype=np.uint8)
    assert b.shape == (Cw,)
    bb = q43_block_bytes(b)
    nblk = capacity // 64
    codes = np.zeros((B, nblk, bb), np.uint8)
    meta = np.zeros((B, nblk, Cw, 2), np.uint16)
    tail = np.zeros((B, 64, Cw), np.uint16)
    rc = lib().orc_q43_pack(B, T, capacity, Cw, _vp(b), _vp(x), _vp(codes), _vp(meta), _vp(tail))
    if rc != 0:
        raise ValueError("bad q43_pack arguments")
    return codes, meta, tail


def q43_unpack(codes, meta, tail, bits, seq_len: int, capacity: int, t0: int = 0,
               t1: int | None = None) -> np.ndarray:
    """Dequantise tokens [t0, t1) -> fp16 [B, t1-t0, C]."""
    t1 = seq_len if t1 is None else t1
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    meta = np.ascontiguousarray(meta, dtype=np.uint16)
    tail = np.ascontiguousarray(tail, dtype=np.uint16)
    b = np.ascontiguousarray(bits, dtype=np.uint8)
    B, Cw = codes.shape[0], b.shape[0]
    out = np.zeros((B, t1 - t0, Cw), np.uint16)
    rc = lib().orc_q43_unpack(B, seq_len, capacity, Cw, _vp(b), _vp(codes), _vp(meta),
                              _vp(tail), t0, t1, _vp(out))
    if rc != 0:
        raise ValueError("bad q43_unpack arguments")
    return out.view(np.float16)
