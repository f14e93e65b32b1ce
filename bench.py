"""Benchmark of single-token decode attention over a low-rank latent KV cache on one MI355X.

A step is one decode step for the whole batch. For a single-layer workload: append the new token's
key and value latents at the last position (starkv_append_latents), then attend from the latent
cache over all T cached tokens (starkv_decode_attn: score kernel, value kernel, log-sum-exp merge,
per-head B_v projection). For the 32-layer model step the same is done for every layer in order,
the three exempt layers attending over full-width fp16 K/V. Inputs are synthetic (seeded) and
already resident in HBM when timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--scrub-mib N]

Prints one JSON line. ``value`` is decode tokens per second (one new token per sequence per step,
B / step time). ``roofline`` prices the dominant kernel (the one with the largest total time; all
appear under ``kernels``) on HBM: its algorithmic bytes (latent bytes it must read: key latents
for the score kernel, value latent for the value kernel, codes plus scales / zero points for a
mixed 4/3-bit cache, K and V for an exempt layer) over its duration from HIP events recorded
around its launch on the launch stream, against MI355X's 8 TB/s, and against a device-copy
ceiling measured in the same run. Beside it: the kernel's algorithmic vector and matrix work over
the same duration against the published fp32 vector and fp16 matrix peaks, and the counter
figures (HBM traffic, MfmaUtil, VALUBusy) of the rocprofv3 summary taken on the same kernel
sources (null when the sources have changed since). With ``--extras``, ``projections`` times,
apart from the step, the two dense products around a latent layer's attention (the fused token
down-projection + append and the output projection) with HIP events, and ``queries`` times four
queries per sequence (speculative-decoding verification) through the per-row multi-query entry
point and through the one that shares each key and latent stream between a sequence's queries.
``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of (sequence, head) pairs of the
same workload, scaled to the whole workload, on all host threads and on one.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                     # MI355X HBM3E, AMD datasheet
# MI355X published peaks: fp32 vector 157.3 TFLOP/s (counts the packed fp32 forms, which this
# build does not emit: 256 CUs x 4 SIMDs x 16 lanes x 2 flop x 2.4 GHz = 78.6 without them);
# dense fp16 / bf16 matrix 2.5 PFLOP/s
VALU_PEAK_TFLOPS = 157.3
VALU_PEAK_NONPACKED_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
MFMA_F16_PEAK_TFLOPS = 2500.0
DEFAULT_WORKLOAD = "longchat_b16_t32768_f16"
MODEL_WORKLOAD = "model32_b32_t8192_f16"
METRIC = "decode attn tokens/sec and achieved latent-KV HBM GB/s (% of peak), B=16 T=32K"

# Hardware-counter figures per launch from rocprofv3 runs of this bench's command for the workload
# (the summaries, with their commands, are the files named here): HBM bytes read + written
# (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, the factors a plain copy of known size gives), MfmaUtil
# and VALUBusy (percent, rocprofv3's derived counters). Each workload's figures carry the digest of
# the kernel sources they were measured on; when the sources differ they are reported as null.
KERNEL_SOURCES = ("latent_decode.hip", "dense_decode.hip", "common.hpp")
MEASURED = {
    "longchat_b16_t32768_f16": {
        "digest": "70039981d02b5189",
        "source": "profiles/latent_decode_counters_longchat_b16_t32768_f16.md",
        "kernels": {
            "latent_scores": {"traffic": 1438133496, "mfma_util_pct": 25.6, "valu_busy_pct": 65.8},
            "latent_values": {"traffic": 1142625440, "mfma_util_pct": 7.7, "valu_busy_pct": 6.6},
        },
    },
    "longchat_b16_t16384_f16": {
        "digest": "70039981d02b5189",
        "source": "profiles/latent_decode_counters_longchat_b16_t16384.md",
        "kernels": {
            "latent_scores": {"traffic": 719437768, "mfma_util_pct": 24.1, "valu_busy_pct": 63.6},
            "latent_values": {"traffic": 585869984, "mfma_util_pct": 6.8, "valu_busy_pct": 7.0},
        },
    },
    "model32_b32_t8192_f16": {
        "digest": "70039981d02b5189",
        "source": "profiles/model32_counters_b32_t8192_f16.md",
        "kernels": {      # latent kernels: means over the 29 latent layers' launches
            "latent_scores": {"traffic": 963049756, "mfma_util_pct": 22.3, "valu_busy_pct": 49.6},
            "latent_values": {"traffic": 635022727, "mfma_util_pct": 5.8, "valu_busy_pct": 7.3},
            "dense_attention": {"traffic": 4311075335, "mfma_util_pct": 0.0, "valu_busy_pct": 26.1},
        },
    },
    "longchat_b16_t16384_q43": {
        "digest": "70039981d02b5189",
        "source": "profiles/latent_decode_counters_longchat_b16_t16384.md",
        "kernels": {
            "latent_scores": {"traffic": 240687280, "mfma_util_pct": 16.0, "valu_busy_pct": 69.8},
            "latent_values": {"traffic": 179143104, "mfma_util_pct": 9.8, "valu_busy_pct": 44.7},
        },
    },
}


def kernel_source_digest() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "rank_kv_cache_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEventCreate / hipEventElapsedTime through the HIP runtime torch already loaded."""

    def __init__(self):
        import torch
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.hip = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def record(self, e, stream):
        rc = self.hip.hipEventRecord(e, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(e.value)
        return out

    def elapsed_ms(self, e0, e1) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


class LayerRun:
    """One layer's device state for the benchmark: cache prefilled with T-1 tokens, the new
    token's rows, factors, query, output, and the algorithmic bytes of its streaming kernels."""

    def __init__(self, layer, cache, new_k, new_v, bk, bv, q, out, T, dense, key_bytes,
                 value_bytes):
        self.layer, self.cache, self.new_k, self.new_v = layer, cache, new_k, new_v
        self.bk, self.bv, self.q, self.out, self.T = bk, bv, q, out, T
        self.dense, self.key_bytes, self.value_bytes = dense, key_bytes, value_bytes


class OracleSample:
    """Accumulates oracle wall time on sampled (sequence, head) pairs, scaled per layer."""

    def __init__(self):
        import oracle
        self.threads = oracle.threads()
        self.full_s = 0.0
        self.spent = 0.0
        self.pairs = 0
        self.total_pairs = 0
        # the same oracle on one host thread, on a smaller sample (a quarter of the budget)
        self.one_thread_s = 0.0
        self.one_thread_spent = 0.0
        self.one_thread_pairs = 0

    def time_pairs(self, fn, B, H, budget_s, seed, extra_per_seq=None):
        """fn(pairs) runs the oracle on a list of (b, h); extra_per_seq(b) times per-sequence
        preparation (dequantisation) that the oracle repeats for each sequence it touches."""
        import oracle
        thr = oracle.threads()
        rng = np.random.default_rng(seed)
        order = rng.permutation(B * H)
        done, spent, chunk = 0, 0.0, max(1, thr)
        while done < B * H and spent < budget_s:
            sel = order[done:done + chunk]
            pairs = [(int(i) // H, int(i) % H) for i in sel]
            t0 = time.perf_counter()
            fn(pairs)
            spent += time.perf_counter() - t0
            done += len(sel)
            per_pair = spent / done
            chunk = int(min(max(chunk, (budget_s - spent) / max(per_pair, 1e-9)), B * H - done))
            if chunk <= 0:
                break
        full = spent * (B * H) / done
        if extra_per_seq is not None:
            t0 = time.perf_counter()
            extra_per_seq(0)
            e = time.perf_counter() - t0
            spent += e
            full += e * B
        self.full_s += full
        self.spent += spent
        self.pairs += done
        self.total_pairs += B * H
        # one thread: pairs one at a time until a quarter of the budget is spent
        oracle.set_threads(1)
        try:
            spent1, done1 = 0.0, 0
            while done1 < B * H and spent1 < budget_s / 4:
                i = int(order[done1])
                t0 = time.perf_counter()
                fn([(i // H, i % H)])
                spent1 += time.perf_counter() - t0
                done1 += 1
            full1 = spent1 * (B * H) / done1
            if extra_per_seq is not None:
                t0 = time.perf_counter()
                extra_per_seq(0)
                e1 = time.perf_counter() - t0
                spent1 += e1
                full1 += e1 * B
        finally:
            oracle.set_threads(thr)
        self.one_thread_s += full1
        self.one_thread_spent += spent1
        self.one_thread_pairs += done1
        return full


def measure_copy_ceiling(hip, stream, mib=1024, reps=5):
    """Device-copy ceiling of this GPU: one elementwise copy kernel reading and writing `mib` MiB,
    timed with HIP events on the launch stream; returns (bytes read + written) / median time."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    ev = hip.create(2 * reps)
    dst.copy_(src)
    for i in range(reps):
        hip.record(ev[2 * i], stream.cuda_stream)
        dst.copy_(src)
        hip.record(ev[2 * i + 1], stream.cuda_stream)
    torch.cuda.synchronize()
    ms = [hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(reps)]
    hip.destroy(ev)
    del src, dst
    return 2 * n * 4 / (statistics.median(ms) * 1e-3) / 1e9


def cache_capacity(T):
    return ((T + 63) // 64) * 64


def latent_kernel_bytes(sk, layer, B, T, Rk, rv, esz, quantized):
    """Algorithmic bytes one launch of the score / value kernel must read."""
    if not quantized:
        return B * T * Rk * esz, B * T * rv * esz
    cap = cache_capacity(T)
    sizes = sk.starkv_cache_bytes(layer, B, cap)
    pad = 32                                          # readers' window padding after the blocks
    nb_cap = cap // 64
    kbb = (sizes[0] - pad) // (B * nb_cap)
    vbb = (sizes[1] - pad) // (B * nb_cap)
    full, tail = T // 64, T % 64
    kb = B * (full * (kbb + 4 * Rk) + tail * Rk * 2)
    vb = B * (full * (vbb + 4 * rv) + tail * rv * 2)
    return kb, vb


def build_latent_run(sk, buffers, layer, zk, zv, bk_h, bv_h, q_h, T, bf16, quantized):
    import torch
    B = zk.shape[0]
    cap = cache_capacity(T)
    cache = buffers.alloc_cache(layer, B, cap)
    dzk = buffers.to_device(zk, bf16=bf16)
    dzv = buffers.to_device(zv, bf16=bf16)
    dbk = buffers.to_device(bk_h, bf16=bf16)
    dbv = buffers.to_device(bv_h, bf16=bf16)
    H, d = q_h.shape[1], q_h.shape[2]
    if quantized:
        # the quantised layer stores blockwise-Hadamard-rotated latents (Zhou notes, section 6.1:
        # rotate, then quantise); the rotation is absorbed into the factors. It is offline
        # preparation, done here on the device before the cache is built, outside the timed steps.
        def rot(x, which, kind, n):
            y = torch.empty_like(x)
            sk.starkv_hadamard_rotate(layer, which, kind, n, x, y)
            return y
        dzk, dzv = rot(dzk, 0, 0, B * T), rot(dzv, 1, 0, B * T)
        dbk, dbv = rot(dbk, 0, 1, d), rot(dbv, 1, 1, H * d)
    sk.starkv_append_latents(layer, cache, 0, T - 1, dzk[:, :T - 1].contiguous(),
                             dzv[:, :T - 1].contiguous())
    new_k = dzk[:, T - 1:].contiguous()
    new_v = dzv[:, T - 1:].contiguous()
    del dzk, dzv
    out = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    esz = zk.dtype.itemsize
    kb, vb = latent_kernel_bytes(sk, layer, B, T, zk.shape[2], zv.shape[2], esz, quantized)
    return LayerRun(layer, cache, new_k, new_v, dbk, dbv, buffers.to_device(q_h), out, T, False,
                    kb, vb)


def build_dense_run(sk, buffers, layer, k, v, q_h, T):
    import torch
    B = k.shape[0]
    cache = buffers.alloc_cache(layer, B, cache_capacity(T))
    dk = buffers.to_device(k)
    dv = buffers.to_device(v)
    sk.starkv_append_latents(layer, cache, 0, T - 1, dk[:, :T - 1].contiguous(),
                             dv[:, :T - 1].contiguous())
    new_k = dk[:, T - 1:].contiguous()
    new_v = dv[:, T - 1:].contiguous()
    del dk, dv
    H, d = q_h.shape[1], q_h.shape[2]
    out = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    kvb = B * T * k.shape[2] * k.dtype.itemsize
    return LayerRun(layer, cache, new_k, new_v, None, None, buffers.to_device(q_h), out, T, True,
                    kvb, kvb)


def setup_single(a, sk, buffers, synth, sample):
    w = synth.WORKLOADS[a.workload]
    B, H, d, T = w.batch, w.heads, w.head_dim, w.seq_len
    t_gen = time.perf_counter()
    ld = synth.draw_layer(w)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(w.cache_seed, 0, B, H, d)
    Rk, rv = int(ld.key_ranks.sum()), ld.value_rank
    log(f"[bench] {w.name}: B={B} H={H} d={d} T={T} R_k={Rk} r_v={rv} {w.dtype}"
        f"{' mixed 4/3-bit cache' if w.quantized else ''}; generated "
        f"{(zk.nbytes + zv.nbytes) / 1e9:.2f} GB in {time.perf_counter() - t_gen:.1f} s")
    if w.quantized:
        # the generator's rows are rotated on the device before they enter the cache (see
        # build_latent_run)
        layer = sk.Layer(num_heads=H, head_dim=d, key_ranks=tuple(int(r) for r in ld.key_ranks),
                         value_rank=rv, cache_dtype=sk.Q43, rope_base=w.rope_base,
                         q_top_fraction=w.q_top_fraction)
    else:
        dt_code = {"f32": sk.F32, "f16": sk.F16, "bf16": sk.BF16}[w.dtype]
        layer = sk.Layer(num_heads=H, head_dim=d, key_ranks=tuple(int(r) for r in ld.key_ranks),
                         value_rank=rv, cache_dtype=dt_code, rope_base=w.rope_base)
    bf16 = w.dtype == "bf16"
    run = build_latent_run(sk, buffers, layer, zk, zv, ld.bk, ld.bv, q, T, bf16, w.quantized)
    if sample is not None:
        sample_latent_layer(sample, w, ld, zk, zv, q, a.cpu_budget, w.quantized, seed=2024)
    desc = {"workload": w.name, "batch": B, "heads": H, "head_dim": d, "seq_len": T,
            "key_rank_sum": Rk, "value_rank": rv,
            "latent_dtype": ("q43" if w.q_top_fraction < 1 else "q4") if w.quantized else w.dtype,
            "layers": 1}
    if w.quantized:
        desc["q_top_fraction"] = w.q_top_fraction
    return [run], desc, "f16" if w.quantized else w.dtype, B


def sample_latent_layer(sample, w, ld, zk, zv, q, budget, quantized, seed):
    import oracle
    oracle.lib()
    if not quantized:
        sample.time_pairs(lambda pairs: oracle.decode_latent(zk, zv, ld.bk, ld.bv, q, ld.key_ranks,
                                                             pairs=pairs),
                          w.batch, w.heads, budget, seed)
        return
    # the oracle's mixed 4/3-bit path: the cache is quantised once when it is built (not timed);
    # a step dequantises every sequence (timed once, scaled by B) and attends on the result. The
    # oracle's work does not depend on the values, so it runs on the generator's rows without the
    # offline rotation (which is not part of a step on either side).
    T = zk.shape[1]
    cap = cache_capacity(T)
    bits_k = oracle.channel_bits(ld.key_ranks, w.q_top_fraction)
    bits_v = oracle.channel_bits([ld.value_rank], w.q_top_fraction)
    pk = oracle.q43_pack(zk, bits_k, cap)
    pv = oracle.q43_pack(zv, bits_v, cap)
    dk = oracle.q43_unpack(*pk, bits_k, T, cap)
    dv = oracle.q43_unpack(*pv, bits_v, T, cap)

    def unpack_one(b):
        oracle.q43_unpack(*(x[b:b + 1] for x in pk), bits_k, T, cap)
        oracle.q43_unpack(*(x[b:b + 1] for x in pv), bits_v, T, cap)

    sample.time_pairs(lambda pairs: oracle.decode_latent(dk, dv, ld.bk, ld.bv, q, ld.key_ranks,
                                                         pairs=pairs),
                      w.batch, w.heads, budget, seed, extra_per_seq=unpack_one)


def setup_model(a, sk, buffers, synth, sample):
    import oracle
    spec = synth.MODEL_STEP
    layers = synth.model_layers()
    B, H, d, T = spec["batch"], spec["heads"], spec["head_dim"], spec["seq_len"]
    runs = []
    latent_bytes = dense_bytes = 0
    t_gen = time.perf_counter()
    per_layer_budget = a.cpu_budget / len(layers)
    for ml in layers:
        w = ml.workload
        q = synth.draw_queries(spec["seed"], ml.index, B, H, d)
        if ml.dense:
            k, v = synth.draw_dense_cache(spec["seed"], ml.index, B, T, H * d, spec["dtype"])
            layer = sk.Layer(num_heads=H, head_dim=d, dense=True, cache_dtype=sk.F16)
            runs.append(build_dense_run(sk, buffers, layer, k, v, q, T))
            dense_bytes += 2 * k.nbytes
            if sample is not None:
                sample.time_pairs(lambda pairs: oracle.decode_dense(k, v, q, pairs=pairs), B, H,
                                  per_layer_budget, 100 + ml.index)
            del k, v
        else:
            ld = synth.draw_model_layer(ml)
            zk, zv = synth.draw_latent_cache(w, ld, layer=ml.index)
            layer = sk.Layer(num_heads=H, head_dim=d, key_ranks=tuple(int(r) for r in ld.key_ranks),
                             value_rank=ld.value_rank, cache_dtype=sk.F16)
            runs.append(build_latent_run(sk, buffers, layer, zk, zv, ld.bk, ld.bv, q, T, False,
                                         False))
            latent_bytes += zk.nbytes + zv.nbytes
            if sample is not None:
                sample.time_pairs(lambda pairs: oracle.decode_latent(zk, zv, ld.bk, ld.bv, q,
                                                                     ld.key_ranks, pairs=pairs),
                                  B, H, per_layer_budget, 100 + ml.index)
            del zk, zv
        log(f"[bench] layer {ml.index:2d} {'dense' if ml.dense else 'latent'} ready "
            f"({time.perf_counter() - t_gen:.1f} s)")
    desc = {"workload": spec["name"], "batch": B, "heads": H, "head_dim": d, "seq_len": T,
            "layers": len(layers), "dense_layers": list(spec["dense_layers"]),
            "latent_dtype": spec["dtype"], "latent_gb": round(latent_bytes / 1e9, 2),
            "dense_gb": round(dense_bytes / 1e9, 2)}
    return runs, desc, spec["dtype"], B


def measure_projections(sk, buffers, run, B, stream, hip, steps, model_dim=4096, hidden=4096):
    """The two dense products around one latent layer's attention, timed apart from the step with
    HIP events on the launch stream: the fused append front-end (the new token's hidden state
    projected to its key and value latents and stored in the cache at the step's position) and the
    output projection of the heads' outputs (LLaMA-7B widths: hidden 4096). Weights are random in
    the layer's factor type (binary16), inputs resident in HBM. Before each timed call a 512 MiB
    buffer is rewritten so that the weights come from HBM, as in a decode step where the KV cache
    stream evicts them from the last-level cache. Algorithmic bytes: the weights, the fp32 rows
    read and the outputs written, each once."""
    import torch
    L = run.layer
    H, d = L.num_heads, L.head_dim
    Rk, rv = int(sum(L.key_ranks)), L.value_rank
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    a_k = (torch.randn((Rk, model_dim), device="cuda", generator=g) / model_dim ** 0.5).half()
    a_v = (torch.randn((rv, model_dim), device="cuda", generator=g) / model_dim ** 0.5).half()
    wo_t = (torch.randn((hidden, H * d), device="cuda", generator=g) / (H * d) ** 0.5).half()
    x = torch.randn((B, 1, model_dim), device="cuda", generator=g)
    y = torch.empty((B, hidden), dtype=torch.float32, device="cuda")
    nws = max(sk.starkv_append_tokens_workspace_bytes(L, B, 1, model_dim),
              sk.starkv_output_projection_workspace_bytes(L, B, hidden))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    flush = torch.zeros(512 << 20, dtype=torch.uint8, device="cuda")
    sp = stream.cuda_stream
    calls = {
        "append_tokens": (lambda: sk.starkv_append_tokens(L, run.cache, run.T - 1, 1, x, model_dim,
                                                          a_k, a_v, ws, nws, stream=stream),
                          (Rk + rv) * model_dim * 2 + B * model_dim * 4 + B * (Rk + rv) * 2,
                          f"B={B}: x [{B}][{model_dim}] fp32 -> {Rk} key + {rv} value latent "
                          f"channels, binary16 weights"),
        "output_projection": (lambda: sk.starkv_output_projection(L, B, run.out, wo_t, hidden, y,
                                                                  ws, nws, stream=stream),
                              hidden * H * d * 2 + B * H * d * 4 + B * hidden * 4,
                              f"B={B}: o [{B}][{H * d}] fp32 -> y [{B}][{hidden}], binary16 W_o"),
    }
    res = {}
    for name, (fn, nbytes, shape) in calls.items():
        for _ in range(3):
            fn()
        ev = hip.create(2 * steps)
        torch.cuda.synchronize()
        for i in range(steps):
            flush.bitwise_not_()
            hip.record(ev[2 * i], sp)
            fn()
            hip.record(ev[2 * i + 1], sp)
        torch.cuda.synchronize()
        us = statistics.fmean(hip.elapsed_ms(ev[2 * i], ev[2 * i + 1]) for i in range(steps)) * 1e3
        hip.destroy(ev)
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"avg_us": us, "alg_bytes": nbytes, "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                     "shape": shape}
        log(f"[bench] {name}: {us:.2f} us, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of HBM)")
    del flush
    return res


def measure_prefill(sk, buffers, synth, stream, hip, steps, batch=4, chunk=2048):
    """Prompt prefill through starkv_prefill_attn on the LongChat-shaped layer: `batch` sequences
    of `chunk` queries each at positions 0 .. chunk-1 over their own latents (binary16), timed with
    HIP events on the launch stream. Algorithmic work: the cheaper of the two exact orders of the
    plain definition of latent attention (causal) -- each cached key's rebuild 2*d*R_k and its
    values per head 2*r_v*H*d once, then per (query, key, head) 2*d flop for the score and 2*d for
    the value sum. (The latent order, values summed in latent space and B_v applied per query,
    costs 2*r_v per (query, key, head) instead, 3.3x more at this shape; it is not counted.)"""
    import torch
    w = synth.WORKLOADS["longchat_b16_t4096_f16"]
    ld = synth.draw_layer(w)
    zk, zv = synth.draw_latent_cache(w, ld, batches=list(range(batch)), seq_len=chunk)
    H, d, rv = w.heads, w.head_dim, ld.value_rank
    Rk = int(ld.key_ranks.sum())
    L = sk.Layer(num_heads=H, head_dim=d, key_ranks=tuple(int(r) for r in ld.key_ranks),
                 value_rank=rv, cache_dtype=sk.F16)
    cache = buffers.alloc_cache(L, batch, cache_capacity(chunk))
    sk.starkv_append_latents(L, cache, 0, chunk, buffers.to_device(zk), buffers.to_device(zv))
    del zk, zv
    bk, bv = buffers.to_device(ld.bk), buffers.to_device(ld.bv)
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    q = torch.randn((batch, chunk, H, d), device="cuda", generator=g)
    out = torch.empty_like(q)
    nws = sk.starkv_prefill_workspace_bytes(L, batch, 0, chunk)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    sp = stream.cuda_stream

    def call():
        sk.starkv_prefill_attn(L, cache, 0, chunk, None, q, bk, bv, out, ws, nws, stream=stream)

    for _ in range(2):
        call()
    ev = hip.create(2)
    torch.cuda.synchronize()
    hip.record(ev[0], sp)
    for _ in range(steps):
        call()
    hip.record(ev[1], sp)
    torch.cuda.synchronize()
    us = hip.elapsed_ms(ev[0], ev[1]) * 1e3 / steps
    hip.destroy(ev)
    if not bool(torch.isfinite(out).all()):
        raise SystemExit("non-finite prefill output")
    pairs = batch * chunk * (chunk + 1) // 2                  # causal (query, key) pairs
    flop = pairs * H * 4 * d + batch * chunk * (2 * d * Rk + 2 * rv * H * d)
    tf = flop / (us * 1e-6) / 1e12
    res = {"batch": batch, "chunk": chunk, "pos0": 0, "avg_us": us, "query_tokens_per_s": batch * chunk / (us * 1e-6),
           "alg_flop": flop, "roofline": {"bound": "mfma", "achieved": tf, "peak": MFMA_F16_PEAK_TFLOPS,
                                          "unit": "TFLOP/s", "frac": tf / MFMA_F16_PEAK_TFLOPS}}
    log(f"[bench] prefill: {batch} x {chunk} queries in {us:.1f} us ({tf:.1f} TFLOP/s algorithmic)")
    del ws, cache
    return res


def measure_decode_project(sk, buffers, run, B, stream, hip, steps, hidden=4096):
    """Decode attention followed by the output projection (LongChat-7B width, binary16 W_o): two
    calls (starkv_decode_attn, starkv_output_projection) against the one call that keeps the heads'
    outputs in its workspace (starkv_decode_attn_project), HIP events on the launch stream."""
    import torch
    L, T = run.layer, run.T
    H, d = L.num_heads, L.head_dim
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    wo = (torch.randn((hidden, H * d), device="cuda", generator=g) / (H * d) ** 0.5).to(torch.float16)
    y = torch.empty((B, hidden), dtype=torch.float32, device="cuda")
    o = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    nws_d = sk.starkv_decode_workspace_bytes(L, B, T, 0)
    nws_p = sk.starkv_output_projection_workspace_bytes(L, B, hidden)
    nws_1 = sk.starkv_decode_attn_project_workspace_bytes(L, B, T, 0, hidden)
    ws_d = torch.empty(nws_d, dtype=torch.uint8, device="cuda")
    ws_p = torch.empty(nws_p, dtype=torch.uint8, device="cuda")
    ws_1 = torch.empty(nws_1, dtype=torch.uint8, device="cuda")
    sp = stream.cuda_stream

    def two():
        sk.starkv_decode_attn(L, run.cache, T, run.q, run.bk, run.bv, o, 0, ws_d, nws_d, stream=stream)
        sk.starkv_output_projection(L, B, o, wo, hidden, y, ws_p, nws_p, stream=stream)

    def one():
        sk.starkv_decode_attn_project(L, run.cache, T, run.q, run.bk, run.bv, wo, hidden, y, 0, ws_1,
                                      nws_1, stream=stream)

    def timed(fn):
        for _ in range(2):
            fn()
        ev = hip.create(2)
        torch.cuda.synchronize()
        hip.record(ev[0], sp)
        for _ in range(steps):
            fn()
        hip.record(ev[1], sp)
        torch.cuda.synchronize()
        us = hip.elapsed_ms(ev[0], ev[1]) * 1e3 / steps
        hip.destroy(ev)
        return us

    res = {"hidden": hidden, "two_calls_avg_us": timed(two), "one_call_avg_us": timed(one)}
    log(f"[bench] decode + output projection: {res['two_calls_avg_us']:.1f} us in two calls, "
        f"{res['one_call_avg_us']:.1f} us in one")
    return res


def measure_queries(sk, run, B, stream, hip, steps, per_seq=4):
    """Several queries per sequence through starkv_decode_attn_queries, timed with HIP events on
    the launch stream: per_seq causal queries at the last per_seq positions of every sequence
    (speculative-decoding verification; for a mixed 4/3-bit cache, whose partial group fixes the
    length, per_seq samples at the full length). Each query row streams its sequence's latents;
    rows of one sequence that run close together find them in the caches."""
    import torch
    L, T = run.layer, run.T
    q43 = L.cache_dtype == sk.Q43
    seqs = [b for b in range(B) for _ in range(per_seq)]
    lens = [T if q43 else T - per_seq + 1 + i for _ in range(B) for i in range(per_seq)]
    n = len(seqs)
    H, d = L.num_heads, L.head_dim
    qs = torch.tensor(np.asarray(seqs, np.int32), device="cuda")
    ql = torch.tensor(np.asarray(lens, np.int32), device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    q = torch.randn((n, H, d), device="cuda", generator=g)
    out = torch.empty((n, H, d), dtype=torch.float32, device="cuda")
    nws = sk.starkv_decode_workspace_bytes(L, n, T, 0)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
    sp = stream.cuda_stream

    nws_m = sk.starkv_decode_multi_workspace_bytes(L, B, per_seq, T, 0)
    ws_m = torch.empty(nws_m, dtype=torch.uint8, device="cuda")
    out_m = torch.empty_like(out)

    def per_row():        # each row streams its sequence's latents on its own
        sk.starkv_decode_attn_queries(L, run.cache, n, qs, ql, T, q, run.bk, run.bv, out, 0, ws,
                                      nws, stream=stream)

    def shared():         # one key rebuild and one latent stream for a sequence's rows
        sk.starkv_decode_attn_multi(L, run.cache, per_seq, T, ql, q, run.bk, run.bv, out_m, 0,
                                    ws_m, nws_m, stream=stream)

    def timed(fn):
        for _ in range(2):
            fn()
        ev = hip.create(2)
        torch.cuda.synchronize()
        hip.record(ev[0], sp)
        for _ in range(steps):
            fn()
        hip.record(ev[1], sp)
        torch.cuda.synchronize()
        us = hip.elapsed_ms(ev[0], ev[1]) * 1e3 / steps
        hip.destroy(ev)
        return us

    us = timed(per_row)
    us_m = timed(shared)
    if not (bool(torch.isfinite(out).all()) and bool(torch.isfinite(out_m).all())):
        raise SystemExit("non-finite multi-query output")
    res = {"queries_per_sequence": per_seq, "query_rows": n, "causal": not q43,
           "avg_us": us, "us_per_query_row": us / n, "shared_avg_us": us_m,
           "shared_us_per_query_row": us_m / n}
    log(f"[bench] queries: {n} rows ({per_seq} per sequence) in {us:.1f} us per row, "
        f"{us_m:.1f} us shared")
    del ws, ws_m
    return res


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="a single-layer workload name, or " + MODEL_WORKLOAD)
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's split planner")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill of 4 x 2048 queries (for kernel profiles) and print "
                         "its JSON object")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="skip the device-copy ceiling measurement after the steps")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="oracle wall seconds")
    ap.add_argument("--extras", action="store_true",
                    help="after the steps, also time the token down-projection, the output "
                         "projection and several queries per sequence (outside the step; they call "
                         "the decode kernels with other shapes, so a kernel trace of such a run "
                         "mixes those calls with the step's)")
    ap.add_argument("--scrub-mib", type=int, default=0,
                    help="before every warm-up and timed step, rewrite a buffer of this many MiB so "
                         "that no cache line of the previous step survives in the last-level cache "
                         "(256 MB); the step time is then taken from HIP events recorded after the "
                         "rewrite, around the step alone")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="before the steps, stream this many MiB through one elementwise copy "
                         "kernel (reads and writes that many bytes once): the reference for "
                         "scaling HBM byte counters")
    a = ap.parse_args(argv)

    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported (the decode path "
              f"has no multi-GPU mode)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        return 2
    import rank_kv_cache_amd as sk
    from rank_kv_cache_amd import buffers, synth
    sk.lib()                                              # fails loudly if the library is missing

    if a.prefill_only:
        stream = torch.cuda.current_stream()
        res = measure_prefill(sk, buffers, synth, stream, HipEvents(), a.steps)
        print(json.dumps({"prefill": res}), flush=True)
        return 0

    sample = None if a.no_cpu_baseline else OracleSample()
    if a.workload == MODEL_WORKLOAD:
        runs, desc, dtype, B = setup_model(a, sk, buffers, synth, sample)
    elif a.workload in synth.WORKLOADS:
        runs, desc, dtype, B = setup_single(a, sk, buffers, synth, sample)
    else:
        raise SystemExit(f"unknown workload {a.workload!r}; choose from "
                         f"{sorted(synth.WORKLOADS) + [MODEL_WORKLOAD]}")
    ws_bytes = max(sk.starkv_decode_workspace_bytes(r.layer, B, r.T, a.splits) for r in runs)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()

    if a.copy_probe_mib > 0:
        n = a.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {a.copy_probe_mib} MiB read + {a.copy_probe_mib} MiB written")
        del src, dst

    stream = torch.cuda.current_stream()
    hip = HipEvents()
    nl = len(runs)
    ev = hip.create(3 * nl * a.steps)
    scrub = torch.zeros(a.scrub_mib << 20, dtype=torch.uint8, device="cuda") if a.scrub_mib > 0 else None
    sev = hip.create(2 * a.steps) if scrub is not None else []

    def step(i=None):
        if scrub is not None:
            scrub.bitwise_not_()
            if i is not None:
                hip.record(sev[2 * i], stream.cuda_stream)
        for li, r in enumerate(runs):
            sk.starkv_append_latents(r.layer, r.cache, r.T - 1, 1, r.new_k, r.new_v, stream=stream)
            if i is None:
                sk.starkv_decode_attn(r.layer, r.cache, r.T, r.q, r.bk, r.bv, r.out, a.splits, ws,
                                      ws_bytes, stream=stream)
            else:
                e = 3 * (i * nl + li)
                sk.starkv_decode_attn_timed(r.layer, r.cache, r.T, r.q, r.bk, r.bv, r.out,
                                            a.splits, ws, ws_bytes, stream=stream,
                                            event_begin=ev[e], event_mid=ev[e + 1],
                                            event_end=ev[e + 2])
        if scrub is not None and i is not None:
            hip.record(sev[2 * i + 1], stream.cuda_stream)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {a.warmup} steps done")
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    log(f"[bench] timed {a.steps} steps in {elapsed * 1e3:.2f} ms")

    # per-step kernel time by kind, summed over layers
    k_ms = {"latent_scores": [0.0] * a.steps, "latent_values": [0.0] * a.steps,
            "dense_attention": [0.0] * a.steps}
    k_bytes = {"latent_scores": 0, "latent_values": 0, "dense_attention": 0}
    k_launches = {"latent_scores": 0, "latent_values": 0, "dense_attention": 0}
    for li, r in enumerate(runs):
        if r.dense:
            k_bytes["dense_attention"] += 2 * r.key_bytes
            k_launches["dense_attention"] += 1
        else:
            k_bytes["latent_scores"] += r.key_bytes
            k_bytes["latent_values"] += r.value_bytes
            k_launches["latent_scores"] += 1
            k_launches["latent_values"] += 1
        for i in range(a.steps):
            e = 3 * (i * nl + li)
            if r.dense:
                k_ms["dense_attention"][i] += hip.elapsed_ms(ev[e], ev[e + 1])
            else:
                k_ms["latent_scores"][i] += hip.elapsed_ms(ev[e], ev[e + 1])
                k_ms["latent_values"][i] += hip.elapsed_ms(ev[e + 1], ev[e + 2])
    hip.destroy(ev)
    step_ms = [hip.elapsed_ms(sev[2 * i], sev[2 * i + 1]) for i in range(a.steps)] if sev else None
    hip.destroy(sev)
    del scrub

    for r in runs:
        res = r.out.cpu().numpy()
        if not np.all(np.isfinite(res)):
            raise SystemExit("non-finite attention output")
    copy_gbs = None if a.no_copy_ceiling else measure_copy_ceiling(hip, stream)

    projections = queries = prefill = decode_project = None
    if a.extras:
        lat = [r for r in runs if not r.dense]
        projections = measure_projections(sk, buffers, lat[0], B, stream, hip, a.steps)
        if len(runs) == 1:
            queries = measure_queries(sk, lat[0], B, stream, hip, min(a.steps, 10))
            if lat[0].layer.cache_dtype != sk.Q43:
                decode_project = measure_decode_project(sk, buffers, lat[0], B, stream, hip,
                                                        min(a.steps, 10))
        prefill = measure_prefill(sk, buffers, synth, stream, hip, min(a.steps, 5))

    # with a scrub between steps the wall clock would include it: the steps' own HIP events instead
    ms_per_step = statistics.fmean(step_ms) if step_ms else elapsed * 1e3 / a.steps
    kernels = {}
    for k in k_ms:
        if k_launches[k] == 0:
            continue
        avg = statistics.fmean(k_ms[k])
        kernels[k] = {"alg_bytes_per_step": k_bytes[k], "launches_per_step": k_launches[k],
                      "avg_us_per_step": avg * 1e3,
                      "avg_us_per_launch": avg * 1e3 / k_launches[k],
                      "median_us_per_step": statistics.median(k_ms[k]) * 1e3,
                      "gbs": k_bytes[k] / (avg * 1e-3) / 1e9}
    dom = max(kernels, key=lambda k: kernels[k]["avg_us_per_step"])
    total_bytes = sum(k_bytes.values())
    stream_ms = sum(statistics.fmean(k_ms[k]) for k in kernels)
    step_gbs = total_bytes / (ms_per_step * 1e-3) / 1e9
    desc.update({"splits": a.splits or "planner",
                 "kv_gb_per_step": round(total_bytes / 1e9, 3),
                 "kv_gbs_per_step": round(step_gbs, 1),
                 "kv_hbm_frac_per_step": round(step_gbs / HBM_PEAK_GBS, 4),
                 "kv_gbs_stream_kernels": round(total_bytes / (stream_ms * 1e-3) / 1e9, 1),
                 "cached_tokens_per_s": B * runs[0].T / (ms_per_step * 1e-3)})
    if a.scrub_mib > 0:
        desc["scrub_mib_between_steps"] = a.scrub_mib
    dk = kernels[dom]
    roofline = {"bound": "hbm", "achieved": dk["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": dk["gbs"] / HBM_PEAK_GBS, "traffic": None, "kernel": dom,
                "kernel_avg_us": dk["avg_us_per_launch"],
                "alg_bytes_per_launch": dk["alg_bytes_per_step"] // dk["launches_per_step"]}
    if copy_gbs:
        roofline["copy_ceiling_gbs"] = copy_gbs
        roofline["frac_of_copy_ceiling"] = dk["gbs"] / copy_gbs
    # algorithmic work per (cached token, sequence) of a latent layer: score kernel 2*d*R_k MFMA
    # flop (key rebuild) and 6*H*d + 5*H vector flop (RoPE and the dot with the query: 3 flop per
    # element, softmax: ~5 per head); value kernel 2*H*r_v MFMA flop (probabilities times latents)
    lat = [r for r in runs if not r.dense]
    if dom in ("latent_scores", "latent_values") and lat:
        t_s = dk["avg_us_per_step"] * 1e-6
        if dom == "latent_scores":
            mf = sum(B * r.T * 2 * r.layer.head_dim * sum(r.layer.key_ranks) for r in lat)
            vf = sum(B * r.T * r.layer.num_heads * (6 * r.layer.head_dim + 5) for r in lat)
            roofline["valu"] = {"achieved": vf / t_s / 1e12, "peak": VALU_PEAK_TFLOPS,
                                "unit": "TFLOP/s", "frac": vf / t_s / 1e12 / VALU_PEAK_TFLOPS,
                                "frac_of_nonpacked_peak": vf / t_s / 1e12 / VALU_PEAK_NONPACKED_TFLOPS,
                                "flop_per_step": vf}
        else:
            mf = sum(B * r.T * 2 * r.layer.num_heads * r.layer.value_rank for r in lat)
        roofline["mfma"] = {"achieved": mf / t_s / 1e12, "peak": MFMA_F16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": mf / t_s / 1e12 / MFMA_F16_PEAK_TFLOPS,
                            "flop_per_step": mf}
    meas = MEASURED.get(desc["workload"])
    digest = kernel_source_digest()
    if meas is not None and meas["digest"] == digest and dom in meas["kernels"]:
        roofline["traffic"] = meas["kernels"][dom]["traffic"]
        roofline["counters"] = {"source": meas["source"], "digest": digest,
                                "kernels": meas["kernels"]}
    else:
        roofline["counters"] = {"source": None, "note": "no counter run on these kernel sources "
                                                        f"(digest {digest})"}
    rec = {
        "metric": METRIC,
        "value": B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": desc,
        "roofline": roofline,
        "kernels": kernels,
    }
    if projections is not None:
        rec["projections"] = projections
    if decode_project is not None:
        rec["decode_project"] = decode_project
    if prefill is not None:
        rec["prefill"] = prefill
    if queries is not None:
        queries["vs_single_query_step"] = queries["avg_us"] / (ms_per_step * 1e3)
        queries["shared_vs_single_query_step"] = queries["shared_avg_us"] / (ms_per_step * 1e3)
        rec["queries"] = queries
    if sample is not None and sample.pairs:
        import oracle
        thr = sample.threads
        rec["cpu_baseline"] = {
            "value": B / sample.full_s, "unit": "tokens/s", "cores": thr, "kind": "oracle",
            "sample": f"{sample.pairs} of {sample.total_pairs} (sequence, head, layer) pairs of the "
                      f"same workload, full T, fp64, {sample.spent:.1f} s wall on {thr} threads; "
                      f"scaled per layer to all pairs ({sample.full_s:.1f} s per step)"}
        if sample.one_thread_s:
            rec["cpu_baseline"]["value_1thread"] = B / sample.one_thread_s
            rec["cpu_baseline"]["sample_1thread"] = (
                f"{sample.one_thread_pairs} pairs on 1 thread, {sample.one_thread_spent:.1f} s wall; "
                f"scaled the same way ({sample.one_thread_s:.1f} s per step)")
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
