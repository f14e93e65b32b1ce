"""Benchmark of single-token decode attention over a low-rank latent KV cache on one MI355X.

A step is one decode step of one attention layer for the whole batch: append the new token's key
and value latents at the last position (starkv_append_latents), then attend from the latent
cache over all T cached tokens (starkv_decode_attn: split kernel, log-sum-exp merge, per-head B_v
projection). Inputs are synthetic (seeded), already resident in HBM when timing starts.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints one JSON line. ``value`` is decode tokens per second (one new token per sequence per step,
B / step time). ``roofline`` prices the dominant kernel against MI355X's 8 TB/s HBM. The two
streaming kernels are the score kernel (reads the key latents, B * T * R_k elements) and the value
kernel (reads the value latent, B * T * r_v elements); each one's algorithmic bytes are divided by
its average duration from HIP events recorded around its launch on the launch stream, and the
slower one is reported (both appear under ``kernels``). ``cpu_baseline`` times the fp64 CPU oracle on a bounded
sample of (sequence, head) pairs of the same workload, scaled to the whole workload.
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
DEFAULT_WORKLOAD = "longchat_b16_t32768_f16"
METRIC = "decode attn tokens/sec and achieved latent-KV HBM GB/s (% of peak), B=16 T=32K"


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


def cpu_baseline(ld, zk, zv, q, B, H, budget_s: float):
    """Time the fp64 oracle on (b, h) pairs until about ``budget_s`` seconds of wall time have
    been spent; scale to all B*H pairs and report decode tokens/s of the whole workload."""
    import oracle
    oracle.lib()
    thr = oracle.threads()
    rng = np.random.default_rng(2024)
    order = rng.permutation(B * H)
    done, spent = 0, 0.0
    chunk = max(1, thr)
    while done < B * H and spent < budget_s:
        sel = order[done:done + chunk]
        pairs = [(int(i) // H, int(i) % H) for i in sel]
        t0 = time.perf_counter()
        oracle.decode_latent(zk, zv, ld.bk, ld.bv, q, ld.key_ranks, pairs=pairs)
        spent += time.perf_counter() - t0
        done += len(sel)
        per_pair = spent / done
        chunk = int(min(max(chunk, (budget_s - spent) / max(per_pair, 1e-9)), B * H - done))
        chunk = max(chunk, 0)
        if chunk == 0:
            break
    full_s = spent * (B * H) / done
    return {"value": B / full_s, "unit": "tokens/s", "cores": thr, "kind": "oracle",
            "sample": f"{done} of {B * H} (sequence, head) pairs of the same workload, full T, fp64 "
                      f"latent form, {spent:.1f} s wall on {thr} threads; scaled to all pairs "
                      f"({full_s:.1f} s per step)"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--splits", type=int, default=0, help="0 = the library's split planner")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="oracle wall seconds")
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

    w = synth.WORKLOADS[a.workload]
    if w.quantized:
        raise SystemExit("quantized workloads are not benchmarked by this script yet")
    B, H, d, T = w.batch, w.heads, w.head_dim, w.seq_len
    t_gen = time.perf_counter()
    ld = synth.draw_layer(w)
    zk, zv = synth.draw_latent_cache(w, ld)
    q = synth.draw_queries(w.cache_seed, 0, B, H, d)
    Rk, rv = int(ld.key_ranks.sum()), ld.value_rank
    esz = zk.dtype.itemsize
    log(f"[bench] {w.name}: B={B} H={H} d={d} T={T} R_k={Rk} r_v={rv} {w.dtype}; "
        f"generated {(zk.nbytes + zv.nbytes) / 1e9:.2f} GB in {time.perf_counter() - t_gen:.1f} s")

    dt_code = {"f32": sk.F32, "f16": sk.F16, "bf16": sk.BF16}[w.dtype]
    layer = sk.Layer(num_heads=H, head_dim=d, key_ranks=tuple(int(r) for r in ld.key_ranks),
                     value_rank=rv, cache_dtype=dt_code, rope_base=w.rope_base)
    bf16 = w.dtype == "bf16"
    cap = ((T + 63) // 64) * 64
    cache = buffers.alloc_cache(layer, B, cap)
    # prefill T-1 tokens; the step appends token T-1 and attends over T
    dzk = buffers.to_device(zk, bf16=bf16)
    dzv = buffers.to_device(zv, bf16=bf16)
    sk.starkv_append_latents(layer, cache, 0, T - 1, dzk[:, :T - 1].contiguous(),
                             dzv[:, :T - 1].contiguous())
    new_k = dzk[:, T - 1:].contiguous()
    new_v = dzv[:, T - 1:].contiguous()
    del dzk, dzv
    bk = buffers.to_device(ld.bk, bf16=bf16)
    bv = buffers.to_device(ld.bv, bf16=bf16)
    dq = buffers.to_device(q)
    out = torch.empty((B, H, d), dtype=torch.float32, device="cuda")
    ws, nws = buffers.alloc_workspace(layer, B, T, a.splits)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    hip = HipEvents()
    ev = hip.create(3 * a.steps)

    def step(i=None):
        sk.starkv_append_latents(layer, cache, T - 1, 1, new_k, new_v, stream=stream)
        if i is None:
            sk.starkv_decode_attn(layer, cache, T, dq, bk, bv, out, a.splits, ws, nws,
                                  stream=stream)
        else:
            sk.starkv_decode_attn_timed(layer, cache, T, dq, bk, bv, out, a.splits, ws, nws,
                                        stream=stream, event_begin=ev[3 * i],
                                        event_mid=ev[3 * i + 1], event_end=ev[3 * i + 2])

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {a.warmup} steps done")
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    score_ms = [hip.elapsed_ms(ev[3 * i], ev[3 * i + 1]) for i in range(a.steps)]
    value_ms = [hip.elapsed_ms(ev[3 * i + 1], ev[3 * i + 2]) for i in range(a.steps)]
    hip.destroy(ev)
    log(f"[bench] timed {a.steps} steps in {elapsed * 1e3:.2f} ms")

    res = out.cpu().numpy()
    if not np.all(np.isfinite(res)):
        raise SystemExit("non-finite attention output")

    ms_per_step = elapsed * 1e3 / a.steps
    score_avg, value_avg = statistics.fmean(score_ms), statistics.fmean(value_ms)
    key_bytes = B * T * Rk * esz                          # per launch of the score kernel
    val_bytes = B * T * rv * esz                          # per launch of the value kernel
    latent_bytes = key_bytes + val_bytes
    kernels = {
        "latent_scores": {"alg_bytes_per_launch": key_bytes, "avg_us": score_avg * 1e3,
                          "median_us": statistics.median(score_ms) * 1e3,
                          "gbs": key_bytes / (score_avg * 1e-3) / 1e9},
        "latent_values": {"alg_bytes_per_launch": val_bytes, "avg_us": value_avg * 1e3,
                          "median_us": statistics.median(value_ms) * 1e3,
                          "gbs": val_bytes / (value_avg * 1e-3) / 1e9},
    }
    dom = max(kernels, key=lambda k: kernels[k]["avg_us"])
    stream_gbs = latent_bytes / ((score_avg + value_avg) * 1e-3) / 1e9
    step_gbs = latent_bytes / (ms_per_step * 1e-3) / 1e9
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
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "head_dim": d, "seq_len": T,
                   "key_rank_sum": Rk, "value_rank": rv, "latent_dtype": w.dtype,
                   "splits": a.splits or "planner",
                   "latent_gbs_per_step": round(step_gbs, 1),
                   "latent_hbm_frac_per_step": round(step_gbs / HBM_PEAK_GBS, 4),
                   "latent_gbs_stream_kernels": round(stream_gbs, 1),
                   "cached_tokens_per_s": B * T / (ms_per_step * 1e-3)},
        "roofline": {"bound": "hbm", "kernel": dom,
                     "achieved": kernels[dom]["gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": kernels[dom]["gbs"] / HBM_PEAK_GBS, "traffic": None,
                     "kernel_avg_us": kernels[dom]["avg_us"],
                     "alg_bytes_per_launch": kernels[dom]["alg_bytes_per_launch"]},
        "kernels": kernels,
    }
    if not a.no_cpu_baseline:
        log(f"[bench] timing the oracle for ~{a.cpu_budget:.0f} s")
        rec["cpu_baseline"] = cpu_baseline(ld, zk, zv, q, B, H, a.cpu_budget)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
