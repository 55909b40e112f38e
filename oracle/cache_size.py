"""Per-token KV-cache sizes, MLA versus standard multi-head attention.

Test infrastructure only (see the package docstring).

* MLA caches, per token and layer, the latent c_t (d_c values) and the
  decoupled RoPE key (d_h^R values), shared by all heads: (d_c + d_hR) * l
  elements per token over l layers ("Multi-head Latent Attention (MLA) și
  arhitectura DeepSeekMoE", opening paragraph; "02 — Multi-Latent Attention
  (MLA)", table in "Coste de memoria").
* Standard MHA caches k_t and v_t for every head: 2 * n_h * d_h * l elements
  per token ("02 — Multi-Latent Attention (MLA)", introduction and "Multi-head
  attention estándar"; "DeepSeek MLA" card, "MHA와 비교").
"""


def mla_elems_per_token(d_c, d_rope, n_layers=1):
    return (d_c + d_rope) * n_layers


def mha_elems_per_token(n_heads, d_head, n_layers=1):
    return 2 * n_heads * d_head * n_layers


def cache_bytes(elems_per_token, n_tokens, bytes_per_elem):
    return elems_per_token * n_tokens * bytes_per_elem


def gqa_groups_equivalent(d_c, d_rope, d_head):
    """Number of K/V head groups whose cache equals MLA's:
    2 * groups * d_head = d_c + d_rope."""
    return (d_c + d_rope) / (2.0 * d_head)
