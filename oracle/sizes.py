"""Cache-size formulas (technical review of arXiv 2606.08382).

* eq. 1 (section 2.1): dense payload M_KV = 2 B T L h_kv d_h b / 8 bytes,
  with h_kv the number of KV heads (not query heads) under GQA;
* eq. 14 (section 6.1): mean bits b_bar = f_hi * b_hi + (1 - f_hi) * b_lo and
  the payload compression 16 / (rho * b_bar) against an fp16 cache;
* eq. 15 (section 6.2): latent payload B T b_bar / 8 * sum over layers of
  (sum_h r^K_{l,h} + R^V_l), plus metadata and padding;
* eq. 16 (section 6.2): retained fraction with protected fp16 layers.
"""

from __future__ import annotations

from fractions import Fraction


def dense_kv_bytes(batch, tokens, layers, kv_heads, head_dim, bits):
    """Eq. 1."""
    return Fraction(2 * batch * tokens * layers * kv_heads * head_dim * bits, 8)


def mean_bits(frac_hi, bits_hi, bits_lo):
    """Eq. 14, left: weighted mean bits per stored latent coordinate."""
    f = Fraction(frac_hi)
    return f * bits_hi + (1 - f) * bits_lo


def payload_compression(rho, bbar, dense_bits=16):
    """Eq. 14, right: dense fp16 payload over latent payload."""
    return Fraction(dense_bits) / (Fraction(rho) * Fraction(bbar))


def latent_payload_bytes(batch, tokens, bbar, key_ranks, value_ranks):
    """Eq. 15 payload term: key_ranks[l] is the list of per-head key ranks of
    layer l and value_ranks[l] the joint value rank of layer l."""
    total = sum(sum(kr) + vr for kr, vr in zip(key_ranks, value_ranks))
    return Fraction(batch * tokens) * Fraction(bbar) / 8 * total


def protected_fraction(layers, protected, compressed_fraction):
    """Eq. 16: protected layers stay at full size, others shrink."""
    return (Fraction(protected, layers)
            + Fraction(layers - protected, layers) * Fraction(compressed_fraction))


def metadata_bytes(batch, tokens, key_groups_per_token, value_groups_per_token,
                   bytes_per_group=4):
    """Per-token quantization metadata (fp16 scale + fp16 zero per group)."""
    return batch * tokens * (key_groups_per_token + value_groups_per_token) \
        * bytes_per_group
