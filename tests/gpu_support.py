"""Shared helpers of the GPU parity tests: build a cache through the C ABI from synthetic arrays,
run decode attention, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import rank_kv_cache_amd as sk
from rank_kv_cache_amd import synth

DT_CODE = {"f32": sk.F32, "f16": sk.F16, "bf16": sk.BF16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / RMS(ref)."""
    rms = float(np.sqrt(np.mean(np.asarray(ref, np.float64) ** 2)))
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref))) / rms


def latent_layer(H, d, ranks, rv, dtype: str, rope_base=10000.0, sm_scale=0.0):
    return sk.Layer(num_heads=H, head_dim=d, key_ranks=tuple(int(r) for r in ranks), value_rank=rv,
                    dense=False, cache_dtype=DT_CODE[dtype], rope_base=rope_base, sm_scale=sm_scale)


def dense_layer(H, d, dtype: str):
    return sk.Layer(num_heads=H, head_dim=d, dense=True, cache_dtype=DT_CODE[dtype])


class DeviceLayer:
    """A layer's cache + factors on the device, built by bulk (or chunked) appends."""

    def __init__(self, layer: sk.Layer, zk, zv, bk=None, bv=None, capacity=None, chunks=None,
                 poison=True):
        import torch
        from rank_kv_cache_amd import buffers
        self.layer = layer
        bf16 = layer.cache_dtype == sk.BF16
        B, T = zk.shape[0], zk.shape[1]
        cap = capacity if capacity is not None else ((T + 63) // 64) * 64
        self.cache = buffers.alloc_cache(layer, B, cap, fill=0xFF if poison else None)
        self.T = T
        dzk = buffers.to_device(zk, bf16=bf16)
        dzv = buffers.to_device(zv, bf16=bf16)
        pos = 0
        for n in (chunks or [T]):
            sk.starkv_append_latents(layer, self.cache, pos, n, dzk[:, pos:pos + n].contiguous(),
                                     dzv[:, pos:pos + n].contiguous())
            pos += n
        assert pos == T
        self.bk = None if bk is None else buffers.to_device(bk, bf16=bf16)
        self.bv = None if bv is None else buffers.to_device(bv, bf16=bf16)
        torch.cuda.synchronize()
        del dzk, dzv

    def decode(self, q: np.ndarray, seq_len=None, num_splits=0, repeat=1):
        import torch
        from rank_kv_cache_amd import buffers
        B = self.cache.batch
        seq_len = self.T if seq_len is None else seq_len
        dq = buffers.to_device(np.ascontiguousarray(q, np.float32))
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        ws, nws = buffers.alloc_workspace(self.layer, B, seq_len, num_splits)
        ws.fill_(0xFF)
        outs = []
        for _ in range(repeat):
            sk.starkv_decode_attn(self.layer, self.cache, seq_len, dq, self.bk, self.bv, out,
                                  num_splits, ws, nws)
            torch.cuda.synchronize()
            outs.append(out.cpu().numpy().copy())
        return outs[0] if repeat == 1 else outs

    def readback(self, t0, t1, seq_len=None):
        import torch
        from rank_kv_cache_amd import buffers
        L = self.layer
        B = self.cache.batch
        seq_len = self.T if seq_len is None else seq_len
        tdt = buffers.elem_torch_dtype(L.cache_dtype)
        wk = L.num_heads * L.head_dim if L.dense else int(sum(L.key_ranks))
        wv = L.num_heads * L.head_dim if L.dense else L.value_rank
        zk = torch.empty((B, t1 - t0, wk), dtype=tdt, device="cuda")
        zv = torch.empty((B, t1 - t0, wv), dtype=tdt, device="cuda")
        sk.starkv_dequant(L, self.cache, seq_len, t0, t1, zk, zv)
        torch.cuda.synchronize()
        return buffers.to_host(zk), buffers.to_host(zv)


def workload_arrays(w: synth.Workload, batches=None, seq_len=None):
    ld = synth.draw_layer(w)
    zk, zv = synth.draw_latent_cache(w, ld, batches=batches, seq_len=seq_len)
    q = synth.draw_queries(w.cache_seed, 0, w.batch, w.heads, w.head_dim)
    if batches is not None:
        q = q[list(batches)]
    return ld, zk, zv, q
