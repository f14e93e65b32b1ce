"""Python binding of libstarkv.so, the MI355X (gfx950) latent-KV decode-attention library.

Argument marshalling only: every computation runs in the library's HIP kernels. Function names
match the C ABI in include/starkv.h. Device buffers are passed as torch tensors (their data
pointers) or raw integer addresses; PyTorch is used for device memory and streams only.

Loading fails loudly when the library has not been built (``python -m rank_kv_cache_amd.build``);
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "F32", "F16", "BF16", "Q43", "StarkvError", "Layer", "Cache", "lib", "library_path",
    "starkv_version", "starkv_status_string", "starkv_cache_bytes", "starkv_append_latents",
    "starkv_decode_workspace_bytes", "starkv_decode_attn", "starkv_dequant",
    "starkv_hadamard_rotate", "starkv_decode_attn_timed", "starkv_output_projection",
    "starkv_output_projection_workspace_bytes", "starkv_append_tokens",
    "starkv_append_tokens_workspace_bytes", "starkv_decode_attn_ragged",
    "starkv_append_latents_ragged", "starkv_decode_attn_queries", "starkv_decode_attn_multi",
    "starkv_decode_multi_workspace_bytes",
    "EXPORTED_SYMBOLS",
]

F32, F16, BF16, Q43 = 0, 1, 2, 3
_STATUS = ["OK", "ERR_NULL", "ERR_SHAPE", "ERR_RANK_ALIGN", "ERR_DTYPE", "ERR_MISALIGNED",
           "ERR_CAPACITY", "ERR_WORKSPACE", "ERR_UNSUPPORTED", "ERR_DEVICE"]

EXPORTED_SYMBOLS = ["starkv_cache_bytes", "starkv_append_latents", "starkv_decode_workspace_bytes",
                    "starkv_decode_attn", "starkv_decode_attn_timed", "starkv_dequant", "starkv_hadamard_rotate",
                    "starkv_output_projection", "starkv_output_projection_workspace_bytes",
                    "starkv_append_tokens", "starkv_append_tokens_workspace_bytes",
                    "starkv_decode_attn_ragged", "starkv_append_latents_ragged",
                    "starkv_decode_attn_queries", "starkv_decode_attn_multi",
                    "starkv_decode_multi_workspace_bytes",
                    "starkv_decode_attn_noalloc", "starkv_decode_attn_noalloc_max_bytes",
                    "starkv_prefill_attn", "starkv_prefill_workspace_bytes",
                    "starkv_decode_attn_project", "starkv_decode_attn_project_workspace_bytes",
                    "starkv_status_string", "starkv_version"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# STARKV_LIBRARY names another build of the library (the host-sanitizer build of the tests); there
# is no fallback: a missing library raises
_LIB_PATH = os.environ.get("STARKV_LIBRARY") or os.path.join(_HERE, "libstarkv.so")
_lib = None


class StarkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = _STATUS[status] if 0 <= status < len(_STATUS) else str(status)
        msg = lib().starkv_status_string(status).decode() if _lib is not None else name
        super().__init__(f"{where}: STARKV_{name} ({msg})")


class _Layer(C.Structure):
    _fields_ = [("num_heads", C.c_int32), ("head_dim", C.c_int32),
                ("key_ranks", C.POINTER(C.c_int32)), ("value_rank", C.c_int32),
                ("dense", C.c_int32), ("cache_dtype", C.c_int32), ("factor_dtype", C.c_int32),
                ("rope_base", C.c_double), ("sm_scale", C.c_float), ("q_top_fraction", C.c_float),
                ("q_bits_hi", C.c_int32), ("q_bits_lo", C.c_int32), ("q_group", C.c_int32)]


class _Cache(C.Structure):
    _fields_ = [("batch", C.c_int32), ("capacity", C.c_int32),
                ("zk", C.c_void_p), ("zv", C.c_void_p), ("zk_meta", C.c_void_p),
                ("zv_meta", C.c_void_p), ("zk_tail", C.c_void_p), ("zv_tail", C.c_void_p),
                ("block_table", C.c_void_p), ("table_stride", C.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m rank_kv_cache_amd.build`")
        L = C.CDLL(_LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        LP, CP = C.POINTER(_Layer), C.POINTER(_Cache)
        L.starkv_version.restype = i32
        L.starkv_version.argtypes = []
        L.starkv_status_string.restype = C.c_char_p
        L.starkv_status_string.argtypes = [C.c_int]
        L.starkv_cache_bytes.restype = C.c_int
        L.starkv_cache_bytes.argtypes = [LP, i32, i32, C.POINTER(sz)]
        L.starkv_append_latents.restype = C.c_int
        L.starkv_append_latents.argtypes = [LP, CP, i64, i64, vp, vp, vp]
        L.starkv_decode_workspace_bytes.restype = sz
        L.starkv_decode_workspace_bytes.argtypes = [LP, i32, i64, i32]
        L.starkv_decode_attn.restype = C.c_int
        L.starkv_decode_attn.argtypes = [LP, CP, i64, vp, vp, vp, vp, i32, vp, sz, vp]
        L.starkv_decode_attn_project_workspace_bytes.restype = sz
        L.starkv_decode_attn_project_workspace_bytes.argtypes = [LP, i32, i64, i32, i32]
        L.starkv_decode_attn_project.restype = C.c_int
        L.starkv_decode_attn_project.argtypes = [LP, CP, i64, vp, vp, vp, vp, i32, vp, i32, vp, sz, vp]
        L.starkv_prefill_workspace_bytes.restype = sz
        L.starkv_prefill_workspace_bytes.argtypes = [LP, i32, i64, i32]
        L.starkv_prefill_attn.restype = C.c_int
        L.starkv_prefill_attn.argtypes = [LP, CP, i64, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.starkv_decode_attn_noalloc.restype = C.c_int
        L.starkv_decode_attn_noalloc.argtypes = [LP, CP, i64, vp, vp, vp, vp, i32, vp]
        L.starkv_decode_attn_noalloc_max_bytes.restype = sz
        L.starkv_decode_attn_noalloc_max_bytes.argtypes = []
        L.starkv_decode_attn_ragged.restype = C.c_int
        L.starkv_decode_attn_ragged.argtypes = [LP, CP, i64, vp, vp, vp, vp, vp, i32, vp, sz, vp]
        L.starkv_decode_attn_queries.restype = C.c_int
        L.starkv_decode_attn_queries.argtypes = [LP, CP, i32, vp, vp, i64, vp, vp, vp, vp, i32, vp,
                                                 sz, vp]
        L.starkv_decode_multi_workspace_bytes.restype = sz
        L.starkv_decode_multi_workspace_bytes.argtypes = [LP, i32, i32, i64, i32]
        L.starkv_decode_attn_multi.restype = C.c_int
        L.starkv_decode_attn_multi.argtypes = [LP, CP, i32, i64, vp, vp, vp, vp, vp, i32, vp, sz, vp]
        L.starkv_append_latents_ragged.restype = C.c_int
        L.starkv_append_latents_ragged.argtypes = [LP, CP, vp, vp, vp, vp]
        L.starkv_decode_attn_timed.restype = C.c_int
        L.starkv_decode_attn_timed.argtypes = [LP, CP, i64, vp, vp, vp, vp, i32, vp, sz, vp, vp, vp, vp]
        L.starkv_dequant.restype = C.c_int
        L.starkv_dequant.argtypes = [LP, CP, i64, i64, i64, vp, vp, vp]
        L.starkv_hadamard_rotate.restype = C.c_int
        L.starkv_hadamard_rotate.argtypes = [LP, i32, i32, i64, vp, vp, vp]
        L.starkv_output_projection.restype = C.c_int
        L.starkv_output_projection.argtypes = [LP, i32, vp, vp, i32, vp, vp, sz, vp]
        L.starkv_output_projection_workspace_bytes.restype = sz
        L.starkv_output_projection_workspace_bytes.argtypes = [LP, i32, i32]
        L.starkv_append_tokens.restype = C.c_int
        L.starkv_append_tokens.argtypes = [LP, CP, i64, i64, vp, i32, vp, vp, vp, sz, vp]
        L.starkv_append_tokens_workspace_bytes.restype = sz
        L.starkv_append_tokens_workspace_bytes.argtypes = [LP, i32, i64, i32]
        _lib = L
    return _lib


def _ptr(x):
    """Device address of a torch tensor, an int address, or None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


@dataclass
class Layer:
    """Host descriptor of one attention layer (mirrors ``starkv_layer``)."""
    num_heads: int
    head_dim: int
    key_ranks: tuple = ()
    value_rank: int = 0
    dense: bool = False
    cache_dtype: int = F16
    factor_dtype: int = -1            # -1: the matching type (F16 for Q43 caches)
    rope_base: float = 10000.0
    sm_scale: float = 0.0
    q_top_fraction: float = 0.25
    q_bits_hi: int = 4
    q_bits_lo: int = 3
    q_group: int = 64
    _c: object = field(default=None, repr=False, compare=False)
    _ranks: object = field(default=None, repr=False, compare=False)

    def c(self):
        ranks = np.ascontiguousarray(np.asarray(self.key_ranks, dtype=np.int32))
        self._ranks = ranks
        fdt = self.factor_dtype
        if fdt < 0:
            fdt = F16 if self.cache_dtype == Q43 else self.cache_dtype
        self._c = _Layer(self.num_heads, self.head_dim,
                         ranks.ctypes.data_as(C.POINTER(C.c_int32)) if ranks.size else None,
                         self.value_rank, int(bool(self.dense)), self.cache_dtype, fdt,
                         self.rope_base, self.sm_scale, self.q_top_fraction, self.q_bits_hi,
                         self.q_bits_lo, self.q_group)
        return self._c


@dataclass
class Cache:
    """Device buffers of one layer's cache (mirrors ``starkv_cache``); tensors or addresses."""
    batch: int
    capacity: int
    zk: object = None
    zv: object = None
    zk_meta: object = None
    zv_meta: object = None
    zk_tail: object = None
    zv_tail: object = None
    block_table: object = None        # paged cache: [batch][table_stride] int32 page indices
    table_stride: int = 0

    def c(self):
        return _Cache(self.batch, self.capacity, _ptr(self.zk), _ptr(self.zv), _ptr(self.zk_meta),
                      _ptr(self.zv_meta), _ptr(self.zk_tail), _ptr(self.zv_tail),
                      _ptr(self.block_table), self.table_stride)


def _layer_ptr(layer):
    if layer is None:
        return None
    return C.byref(layer.c())


def _cache_ptr(cache):
    if cache is None:
        return None
    return C.byref(cache.c())


def _check(status: int, where: str):
    if status != 0:
        raise StarkvError(status, where)


def starkv_version() -> int:
    return int(lib().starkv_version())


def starkv_status_string(status: int) -> str:
    return lib().starkv_status_string(int(status)).decode()


def starkv_cache_bytes(layer: Layer, batch: int, capacity: int):
    out = (C.c_size_t * 6)()
    _check(lib().starkv_cache_bytes(_layer_ptr(layer), batch, capacity, out), "starkv_cache_bytes")
    return [int(v) for v in out]


def starkv_append_latents(layer, cache, pos, n_new, zk_new, zv_new, stream=None, check=True):
    st = lib().starkv_append_latents(_layer_ptr(layer), _cache_ptr(cache), pos, n_new, _ptr(zk_new),
                                     _ptr(zv_new), _stream(stream))
    if check:
        _check(st, "starkv_append_latents")
    return st


def starkv_decode_workspace_bytes(layer, batch, seq_len, num_splits=0) -> int:
    return int(lib().starkv_decode_workspace_bytes(_layer_ptr(layer), batch, seq_len, num_splits))


def starkv_decode_attn(layer, cache, seq_len, q, bk, bv, out, num_splits=0, workspace=None,
                       workspace_bytes=0, stream=None, check=True):
    st = lib().starkv_decode_attn(_layer_ptr(layer), _cache_ptr(cache), seq_len, _ptr(q), _ptr(bk),
                                  _ptr(bv), _ptr(out), num_splits, _ptr(workspace),
                                  int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "starkv_decode_attn")
    return st


def starkv_decode_attn_project_workspace_bytes(layer, batch, seq_len, num_splits, hidden) -> int:
    return int(lib().starkv_decode_attn_project_workspace_bytes(_layer_ptr(layer), batch, seq_len,
                                                                num_splits, hidden))


def starkv_decode_attn_project(layer, cache, seq_len, q, bk, bv, wo, hidden, y, num_splits=0,
                               workspace=None, workspace_bytes=0, stream=None, check=True):
    st = lib().starkv_decode_attn_project(_layer_ptr(layer), _cache_ptr(cache), seq_len, _ptr(q),
                                          _ptr(bk), _ptr(bv), _ptr(wo), hidden, _ptr(y), num_splits,
                                          _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "starkv_decode_attn_project")
    return st


def starkv_prefill_workspace_bytes(layer, batch, pos0, chunk) -> int:
    return int(lib().starkv_prefill_workspace_bytes(_layer_ptr(layer), batch, pos0, chunk))


def starkv_prefill_attn(layer, cache, pos0, chunk, chunk_lens, q, bk, bv, out, workspace=None,
                        workspace_bytes=0, stream=None, check=True):
    st = lib().starkv_prefill_attn(_layer_ptr(layer), _cache_ptr(cache), pos0, chunk,
                                   _ptr(chunk_lens), _ptr(q), _ptr(bk), _ptr(bv), _ptr(out),
                                   _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "starkv_prefill_attn")
    return st


def starkv_decode_attn_noalloc_max_bytes() -> int:
    return int(lib().starkv_decode_attn_noalloc_max_bytes())


def starkv_decode_attn_noalloc(layer, cache, seq_len, q, bk, bv, out, num_splits=0, stream=None,
                               check=True):
    st = lib().starkv_decode_attn_noalloc(_layer_ptr(layer), _cache_ptr(cache), seq_len, _ptr(q),
                                          _ptr(bk), _ptr(bv), _ptr(out), num_splits,
                                          _stream(stream))
    if check:
        _check(st, "starkv_decode_attn_noalloc")
    return st


def starkv_decode_attn_ragged(layer, cache, max_seq_len, seq_lens, q, bk, bv, out, num_splits=0,
                              workspace=None, workspace_bytes=0, stream=None, check=True):
    st = lib().starkv_decode_attn_ragged(_layer_ptr(layer), _cache_ptr(cache), max_seq_len,
                                         _ptr(seq_lens), _ptr(q), _ptr(bk), _ptr(bv), _ptr(out),
                                         num_splits, _ptr(workspace), int(workspace_bytes),
                                         _stream(stream))
    if check:
        _check(st, "starkv_decode_attn_ragged")
    return st


def starkv_decode_attn_queries(layer, cache, num_queries, query_seq, query_len, max_len, q, bk,
                               bv, out, num_splits=0, workspace=None, workspace_bytes=0,
                               stream=None, check=True):
    st = lib().starkv_decode_attn_queries(_layer_ptr(layer), _cache_ptr(cache), num_queries,
                                          _ptr(query_seq), _ptr(query_len), max_len, _ptr(q),
                                          _ptr(bk), _ptr(bv), _ptr(out), num_splits,
                                          _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "starkv_decode_attn_queries")
    return st


def starkv_decode_multi_workspace_bytes(layer, batch, nq, max_len, num_splits=0) -> int:
    return int(lib().starkv_decode_multi_workspace_bytes(_layer_ptr(layer), batch, nq, max_len,
                                                         num_splits))


def starkv_decode_attn_multi(layer, cache, nq, max_len, q_lens, q, bk, bv, out, num_splits=0,
                             workspace=None, workspace_bytes=0, stream=None, check=True):
    st = lib().starkv_decode_attn_multi(_layer_ptr(layer), _cache_ptr(cache), nq, max_len,
                                        _ptr(q_lens), _ptr(q), _ptr(bk), _ptr(bv), _ptr(out),
                                        num_splits, _ptr(workspace), int(workspace_bytes),
                                        _stream(stream))
    if check:
        _check(st, "starkv_decode_attn_multi")
    return st


def starkv_append_latents_ragged(layer, cache, positions, zk_new, zv_new, stream=None, check=True):
    st = lib().starkv_append_latents_ragged(_layer_ptr(layer), _cache_ptr(cache), _ptr(positions),
                                            _ptr(zk_new), _ptr(zv_new), _stream(stream))
    if check:
        _check(st, "starkv_append_latents_ragged")
    return st


def starkv_decode_attn_timed(layer, cache, seq_len, q, bk, bv, out, num_splits=0, workspace=None,
                             workspace_bytes=0, stream=None, event_begin=None, event_mid=None,
                             event_end=None, check=True):
    st = lib().starkv_decode_attn_timed(_layer_ptr(layer), _cache_ptr(cache), seq_len, _ptr(q),
                                        _ptr(bk), _ptr(bv), _ptr(out), num_splits, _ptr(workspace),
                                        int(workspace_bytes), _stream(stream), event_begin,
                                        event_mid, event_end)
    if check:
        _check(st, "starkv_decode_attn_timed")
    return st


def starkv_dequant(layer, cache, seq_len, t0, t1, zk_out, zv_out, stream=None, check=True):
    st = lib().starkv_dequant(_layer_ptr(layer), _cache_ptr(cache), seq_len, t0, t1, _ptr(zk_out),
                              _ptr(zv_out), _stream(stream))
    if check:
        _check(st, "starkv_dequant")
    return st


def starkv_hadamard_rotate(layer, which, kind, n, src, dst, stream=None, check=True):
    st = lib().starkv_hadamard_rotate(_layer_ptr(layer), which, kind, n, _ptr(src), _ptr(dst),
                                      _stream(stream))
    if check:
        _check(st, "starkv_hadamard_rotate")
    return st


def starkv_output_projection_workspace_bytes(layer, batch, hidden) -> int:
    return int(lib().starkv_output_projection_workspace_bytes(_layer_ptr(layer), batch, hidden))


def starkv_output_projection(layer, batch, o, wo, hidden, y, workspace=None, workspace_bytes=0,
                             stream=None, check=True):
    st = lib().starkv_output_projection(_layer_ptr(layer), batch, _ptr(o), _ptr(wo), hidden,
                                        _ptr(y), _ptr(workspace), int(workspace_bytes),
                                        _stream(stream))
    if check:
        _check(st, "starkv_output_projection")
    return st


def starkv_append_tokens_workspace_bytes(layer, batch, n_new, model_dim) -> int:
    return int(lib().starkv_append_tokens_workspace_bytes(_layer_ptr(layer), batch, n_new,
                                                          model_dim))


def starkv_append_tokens(layer, cache, pos, n_new, x, model_dim, a_k, a_v, workspace=None,
                         workspace_bytes=0, stream=None, check=True):
    st = lib().starkv_append_tokens(_layer_ptr(layer), _cache_ptr(cache), pos, n_new, _ptr(x),
                                    model_dim, _ptr(a_k), _ptr(a_v), _ptr(workspace),
                                    int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "starkv_append_tokens")
    return st
