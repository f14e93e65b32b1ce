"""GPU parity of the 32-layer decode step (batch 32, T 8192, layers 0, 1 and 31 exempt / dense).

Every layer's cache is built on the device from the seeded generator (prefill of T-1 tokens), then
one step runs as the benchmark runs it: for each layer in order, append the last token and decode
with the library's default launch configuration, all layers sharing one workspace. Each layer's
output is checked on sampled (sequence, head) pairs against the oracle, which regenerates only the
sampled sequences (each sequence has its own generator stream, so a subset equals the slice of the
full draw).
"""
import numpy as np
import pytest

import oracle
import rank_kv_cache_amd as sk
from rank_kv_cache_amd import synth

from gpu_support import rel_err, say

pytestmark = pytest.mark.gpu
TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sk.lib()


def test_model_step_sampled():
    import torch
    from rank_kv_cache_amd import buffers
    spec = synth.MODEL_STEP
    B, H, d, T = spec["batch"], spec["heads"], spec["head_dim"], spec["seq_len"]
    cap = ((T + 63) // 64) * 64
    layers = synth.model_layers()
    rng = np.random.default_rng(44)
    state = []
    for ml in layers:
        q = synth.draw_queries(spec["seed"], ml.index, B, H, d)
        if ml.dense:
            k, v = synth.draw_dense_cache(spec["seed"], ml.index, B, T, H * d, spec["dtype"])
            layer = sk.Layer(num_heads=H, head_dim=d, dense=True, cache_dtype=sk.F16)
            bk = bv = None
        else:
            ld = synth.draw_model_layer(ml)
            k, v = synth.draw_latent_cache(ml.workload, ld, layer=ml.index)
            layer = sk.Layer(num_heads=H, head_dim=d, key_ranks=tuple(int(r) for r in ld.key_ranks),
                             value_rank=ld.value_rank, cache_dtype=sk.F16)
            bk, bv = buffers.to_device(ld.bk), buffers.to_device(ld.bv)
        cache = buffers.alloc_cache(layer, B, cap)
        dk, dv = buffers.to_device(k), buffers.to_device(v)
        sk.starkv_append_latents(layer, cache, 0, T - 1, dk[:, :T - 1].contiguous(),
                                 dv[:, :T - 1].contiguous())
        new_k, new_v = dk[:, T - 1:].contiguous(), dv[:, T - 1:].contiguous()
        del dk, dv, k, v
        b_s = sorted(int(b) for b in rng.choice(B, size=2, replace=False))
        pairs = [(0, int(rng.integers(0, H))), (1, int(rng.integers(0, H)))]
        state.append((ml, layer, cache, new_k, new_v, bk, bv, q, b_s, pairs))
    torch.cuda.synchronize()
    say(f"[model] {len(layers)} layers built")

    ws_bytes = max(sk.starkv_decode_workspace_bytes(s[1], B, T) for s in state)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    outs = []
    for ml, layer, cache, new_k, new_v, bk, bv, q, _, _ in state:
        out = torch.full((B, H, d), float("nan"), dtype=torch.float32, device="cuda")
        sk.starkv_append_latents(layer, cache, T - 1, 1, new_k, new_v)
        sk.starkv_decode_attn(layer, cache, T, buffers.to_device(q), bk, bv, out, 0, ws, ws_bytes)
        outs.append(out)
    torch.cuda.synchronize()

    worst = 0.0
    for (ml, layer, cache, _, _, _, _, q, b_s, pairs), out in zip(state, outs):
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got)), ml.index
        sel = [(b_s[i], h) for i, h in pairs]
        if ml.dense:
            k, v = synth.draw_dense_cache(spec["seed"], ml.index, B, T, H * d, spec["dtype"],
                                          batches=b_s)
            ref = oracle.decode_dense(k, v, q[b_s], pairs=pairs)
        else:
            ld = synth.draw_model_layer(ml)
            zk, zv = synth.draw_latent_cache(ml.workload, ld, layer=ml.index, batches=b_s)
            ref = oracle.decode_latent(zk, zv, ld.bk, ld.bv, q[b_s], ld.key_ranks, pairs=pairs)
        e = rel_err(np.stack([got[b, h] for b, h in sel]), ref)
        worst = max(worst, e)
        assert e <= TOL, (ml.index, sel, e)
    say(f"[model] worst sampled rel err over {len(state)} layers {worst:.3e}")
