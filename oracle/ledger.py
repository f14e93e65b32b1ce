"""Cache-size and reconstruction-cost arithmetic of the STAR-KV pages (test infrastructure).

Everything here is the plain definition of a quantity the pages compute; tests pin each function
to the numbers the pages print (tests/golden/ledger_values.json).

* KV payload of a uniform cache: 2 (K and V) x B x T x layers x heads x head_dim x bits / 8 bytes
  (Zhou, STAR-KV reading notes, section 2.1).
* Latent cache: per layer, B x T x (sum_h r_k[h] + r_v) x mean_bits / 8 bytes; exempt layers at
  full width and 16 bits; factors and workspace are not payload (same notes, section 6.2).
* Mixed precision: mean bits = f * bits_hi + (1 - f) * bits_lo; ratio against an fp16 cache at
  retained-rank fraction rho = 16 / (rho * mean_bits) (same notes, section 6.1).
* Whole model with exempt layers: L / (n_exempt + (L - n_exempt) / layer_ratio) (section 6.2).
* Explicit per-token reconstruction multiplies (section 5.1): head-wise keys T*H*(rho*d)*d versus
  joint T*(rho*H*d)*(H*d), i.e. H times more for the joint form at equal retained fraction.
"""
from __future__ import annotations


def uniform_kv_bytes(batch, seq_len, layers, kv_heads, head_dim, bits):
    return 2 * batch * seq_len * layers * kv_heads * head_dim * bits / 8


def mean_bits(top_fraction, bits_hi, bits_lo):
    return top_fraction * bits_hi + (1.0 - top_fraction) * bits_lo


def ratio_vs_fp16(retained_fraction, bits):
    return 16.0 / (retained_fraction * bits)


def whole_model_ratio(n_layers, n_exempt, layer_ratio):
    return n_layers / (n_exempt + (n_layers - n_exempt) / layer_ratio)


def latent_layer_bytes(batch, seq_len, key_ranks, value_rank, bits):
    return batch * seq_len * (sum(int(r) for r in key_ranks) + value_rank) * bits / 8


def dense_layer_bytes(batch, seq_len, heads, head_dim, bits=16):
    return uniform_kv_bytes(batch, seq_len, 1, heads, head_dim, bits)


def model_payload_bytes(batch, seq_len, layers):
    """layers: iterable of dicts {dense, heads, head_dim, key_ranks, value_rank, bits}."""
    tot = 0.0
    for ly in layers:
        if ly["dense"]:
            tot += dense_layer_bytes(batch, seq_len, ly["heads"], ly["head_dim"], ly.get("bits", 16))
        else:
            tot += latent_layer_bytes(batch, seq_len, ly["key_ranks"], ly["value_rank"], ly["bits"])
    return tot


def explicit_reconstruction_mults(seq_len, heads, head_dim, retained_fraction, kind):
    if kind == "headwise":
        return seq_len * heads * (retained_fraction * head_dim) * head_dim
    if kind == "joint":
        return seq_len * (retained_fraction * heads * head_dim) * (heads * head_dim)
    raise ValueError(kind)
