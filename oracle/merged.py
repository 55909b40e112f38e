"""Precomputed absorbed weights, in fp64 — test infrastructure only (see the
package docstring).

The up-projections can be folded into the query and output projections ahead
of time, so that decode never forms per-head keys or values and runs on the
cached latent at O(d_c T) cost ("02 — Multi-Latent Attention (MLA)", "Coste
de cómputo": attention rearranged, with some matrix products precomputed, to
work from c_tau directly; "Atención latente de múltiples cabezas",
"Información técnica": the up-projection weights are absorbed into the query
and output projections; "Multi-head Latent Attention (MLA) și arhitectura
DeepSeekMoE", opening paragraph: the inverse projections can be absorbed
into the query and output projections). The rotary part of the query cannot
be folded this way and stays a separate input ("Atención latente de
múltiples cabezas", "Información técnica": the decoupled key path exists
because the rotation cannot be absorbed).

Readings where the pages are silent (the plainest one the rest supports):

* W_Q [H, d_nope, d_x]: head i's no-RoPE query is q_nope,i = W_Q,i x, with x
  in R^{d_x} the token's query input (its hidden state, or a query latent
  where the model compresses queries).
* W_O [d_out, H d_v]: the layer output is y = W_O [o_1; ..; o_H] with the
  heads' outputs concatenated in head order; W_O,i = W_O[:, i d_v : (i+1) d_v].
* Merged weights: A_i = W_UK,i^T W_Q,i  [d_c, d_x] (stacked [H, d_c, d_x]),
  and Bm = [W_O,1 W_UV,1 | .. | W_O,H W_UV,H]  [d_out, H d_c].
* An empty sequence gives y = 0 (each o_i is 0).
"""

import numpy as np

from .mla import _positions, decode_absorbed_heads
from .rope import rope


def merge_query_weight(w_q, w_uk):
    """A_i = W_UK,i^T W_Q,i for every head: [H, d_c, d_x] from W_Q
    [H, d_nope, d_x] and W_UK [H, d_nope, d_c]. Then A_i x = W_UK,i^T q_nope,i."""
    return np.stack([w_uk[i].T @ w_q[i] for i in range(w_q.shape[0])])


def merge_output_weight(w_o, w_uv):
    """Bm = [W_O,i W_UV,i]_i: [d_out, H d_c] from W_O [d_out, H d_v] and
    W_UV [H, d_v, d_c]. Then Bm [o^_1; ..; o^_H] = W_O [W_UV,1 o^_1; ..]."""
    H, d_v, _ = w_uv.shape
    return np.concatenate([w_o[:, i * d_v:(i + 1) * d_v] @ w_uv[i] for i in range(H)], axis=1)


def decode_merged(C, R, seq_start, seq_len, x, q_rope, a, bm, softmax_scale, rope_base, q_pos=None,
                  seqs=None):
    """Decode from merged weights. For each sequence b (L = seq_len[b] rows
    from seq_start[b]) and head i:

        q~_i = A_i x_b                                        (d_c)
        s    = softmax_scale * (C_b q~_i + R_b RoPE(q_rope[b,i], P_b))
        p    = softmax(s) over the L tokens
        o^_i = C_b^T p                                        (d_c)
    and y_b = Bm [o^_1; ..; o^_H]                             (d_out)

    C, R: decoded cache (fp64); x [B, d_x]; q_rope [B, H, d_hR] unrotated;
    a [H, d_c, d_x]; bm [d_out, H d_c]. ``seqs`` limits the work to those
    sequences (the other rows of y stay 0). Returns y [B, d_out]."""
    B = x.shape[0]
    H, d_c, _ = a.shape
    P = _positions(seq_len, q_pos)
    y = np.zeros((B, bm.shape[0]), dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_len[b])
        if L == 0:
            continue
        r0 = int(seq_start[b])
        Cb, Rb = C[r0:r0 + L], R[r0:r0 + L]
        q_lat = a @ x[b]                                    # [H, d_c]
        q_r = rope(q_rope[b], P[b], rope_base)              # [H, d_hR]
        s = softmax_scale * (Cb @ q_lat.T + Rb @ q_r.T)     # [L, H]
        e = np.exp(s - s.max(axis=0, keepdims=True))
        p = e / e.sum(axis=0, keepdims=True)
        o_hat = p.T @ Cb                                    # [H, d_c]
        y[b] = bm @ o_hat.reshape(H * d_c)
    return y


def decode_factored(C, R, seq_start, seq_len, x, q_rope, w_q, w_uk, w_uv, w_o, softmax_scale, rope_base,
                    q_pos=None, seqs=None):
    """The same output through the unmerged weights (a self-check form, pinned
    equal to :func:`decode_merged`; it needs no [H, d_c, d_x] or
    [d_out, H d_c] product, so it serves full-size samples):
    q_nope,i = W_Q,i x_b, o = absorbed decode, y_b = W_O [o_1; ..; o_H]."""
    B = x.shape[0]
    P = _positions(seq_len, q_pos)
    y = np.zeros((B, w_o.shape[0]), dtype=np.float64)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_len[b])
        r0 = int(seq_start[b])
        q_nope = np.einsum("hnx,x->hn", w_q, x[b])
        o = decode_absorbed_heads(C[r0:r0 + L], R[r0:r0 + L], q_nope, q_rope[b], w_uk, w_uv, softmax_scale,
                                  rope_base, P[b])
        y[b] = w_o @ o.reshape(-1)
    return y
