"""MLA append and decode in fp64: the definition the GPU path must reproduce.

Test infrastructure only (see the package docstring).

Notation (H heads; per head i):

    c_t   in R^{d_c}      latent of token t           c_t = W_DKV h_t
    k^R_t in R^{d_hR}     decoupled RoPE key, one per token, shared by heads
    W_UK,i : d_c -> d_nope,  W_UV,i : d_c -> d_v      up-projections per head

Sources:

* c_t = W_DKV h_t; k_t = W_UK c_t and v_t = W_UV c_t are rebuilt from the
  cached latent, which is all that is stored: "02 — Multi-Latent Attention
  (MLA)", section "La compresión de MLA".
* The key has a rotary part k^R (cached as it is, small) and a non-rotary
  part recovered from the latent: same page, "Truco de codificación
  posicional"; the cache holds (d_c + d_hR) values per token and layer:
  "Multi-head Latent Attention (MLA) și arhitectura DeepSeekMoE", opening
  paragraph.
* The score is a content term plus a positional term: "DeepSeek MLA" card,
  section on the problem RoPE causes.
* Per-head softmax attention with q, K, V reshaped to heads: "02 —
  Multi-Latent Attention (MLA)", "Multi-head attention estándar".
* Absorbed form: the up-projections fold into the query and output sides so
  attention runs directly on c_tau at O(d_c T) cost, and the result is not an
  approximation: "02 — Multi-Latent Attention (MLA)", "Coste de cómputo" and
  "Lo que MLA no es"; "Atención latente de múltiples cabezas", "Información
  técnica".

Readings where the pages are silent (the plainest one the rest supports):

* The query token's own latent is appended first; the query sits at position
  P_b = L_b - 1 and attends to positions 0 .. L_b - 1 inclusive (``q_pos``
  overrides P_b).
* k^R is stored already rotated (at its own position); q_rope arrives
  unrotated and is rotated at P_b.
* The softmax scale multiplies the whole (d_nope + d_hR)-wide score.
* Weight layouts: W_DKV [d_c, d_model], W_KR [d_hR, d_model],
  W_UK [H, d_nope, d_c], W_UV [H, d_v, d_c]; output o [B, H, d_v] with no
  output projection.
* An empty sequence (L_b = 0) gives o = 0.
"""

import numpy as np

from . import codecs
from .rope import rope

# ------------------------------------------------------------------ storage


def elem_bytes(dtype):
    return {"f32": 4, "bf16": 2, "fp8": 1}[dtype]


def decode_rows(rows, latent_dtype, rope_dtype, d_c, d_rope, scale=None):
    """Raw cache rows (uint8 [n_rows, row_stride]) -> (C, R) in exact fp64.

    A row is [c_kv (d_c elements) | k_rope (d_rope elements)], packed from
    byte 0; fp8 latents are multiplied by their row's fp32 scale."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    n = rows.shape[0]
    lb = d_c * elem_bytes(latent_dtype)
    rb = d_rope * elem_bytes(rope_dtype)
    lat = rows[:, :lb]
    rp = rows[:, lb:lb + rb]
    if latent_dtype == "f32":
        C = codecs.f32_decode(lat.copy().view(np.float32)).reshape(n, d_c)
    elif latent_dtype == "bf16":
        C = codecs.bf16_decode(lat.copy().view(np.uint16)).reshape(n, d_c)
    elif latent_dtype == "fp8":
        C = codecs.e4m3_decode(lat.copy()).reshape(n, d_c)
        C = C * np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]
    else:
        raise ValueError(latent_dtype)
    if rope_dtype == "f32":
        R = codecs.f32_decode(rp.copy().view(np.float32)).reshape(n, d_rope)
    elif rope_dtype == "bf16":
        R = codecs.bf16_decode(rp.copy().view(np.uint16)).reshape(n, d_rope)
    else:
        raise ValueError(rope_dtype)
    return C, R


def round_to_storage(x, dtype):
    """fp64 -> the nearest value of a storage dtype (still fp64)."""
    if dtype == "f32":
        return codecs.f32_encode(x).astype(np.float64)
    if dtype == "bf16":
        return codecs.bf16_round(x)
    raise ValueError(dtype)


# ------------------------------------------------------------------ append


def append(h, w_dkv, w_kr, seq_start, seq_len, rope_base, latent_dtype, rope_dtype):
    """Down-project new tokens into the latent cache.

    h: [B, n_new, d_model] fp64 (already decoded from its storage dtype).
    For sequence b and new token j the position is p = seq_len[b] + j and the
    row written is seq_start[b] + p. Per token:

        c   = W_DKV h               (fp64)
        k_r = RoPE(W_KR h, p)       (fp64)

    then both are rounded to their storage dtypes. An fp8 latent is stored as
    codes of c / s with s = amax(|c|) / 448 (fp32); the value it stands for is
    code * s.

    Returns a dict with ``rows`` [B, n_new] (int64 row indices), ``c``
    [B, n_new, d_c] and ``k_rope`` [B, n_new, d_rope] (the stored values,
    fp64), ``codes`` (fp8 only, uint8) and ``scale`` (fp8 only, fp32), and
    ``seq_len`` (seq_len + n_new).
    """
    h = np.asarray(h, dtype=np.float64)
    B, n_new, _ = h.shape
    seq_start = np.asarray(seq_start, dtype=np.int64)
    seq_len = np.asarray(seq_len, dtype=np.int64)
    pos = seq_len[:, None] + np.arange(n_new, dtype=np.int64)[None, :]
    c = h @ np.asarray(w_dkv, dtype=np.float64).T
    kr = rope(h @ np.asarray(w_kr, dtype=np.float64).T, pos, rope_base)
    out = {"rows": seq_start[:, None] + pos, "seq_len": seq_len + n_new}
    if latent_dtype == "fp8":
        scale = np.empty((B, n_new), dtype=np.float32)
        codes = np.empty(c.shape, dtype=np.uint8)
        for b in range(B):
            for j in range(n_new):
                s = codecs.e4m3_token_scale(c[b, j])
                scale[b, j] = s
                codes[b, j] = codecs.e4m3_encode(c[b, j] / np.float64(s))
        out["scale"] = scale
        out["codes"] = codes
        out["c"] = codecs.e4m3_decode(codes) * scale.astype(np.float64)[..., None]
    else:
        out["c"] = round_to_storage(c, latent_dtype)
    out["k_rope"] = round_to_storage(kr, rope_dtype)
    return out


# ------------------------------------------------------------------ decode


def _query(q_nope_bi, q_rope_bi, pos, rope_base):
    return np.concatenate([q_nope_bi, rope(q_rope_bi, pos, rope_base)])


def _positions(seq_len, q_pos):
    seq_len = np.asarray(seq_len, dtype=np.int64)
    if q_pos is None:
        return seq_len - 1
    return np.asarray(q_pos, dtype=np.int64)


def _pairs(B, H, pairs):
    if pairs is None:
        return [(b, i) for b in range(B) for i in range(H)]
    return [(int(b), int(i)) for b, i in pairs]


def decode(C, R, seq_start, seq_len, q_nope, q_rope, w_uk, w_uv, softmax_scale,
           rope_base, q_pos=None, pairs=None, chunk=2048):
    """Non-absorbed MLA decode: rebuild per-head K and V from the latent and run
    standard softmax attention. This is the definition.

    C [n_rows, d_c], R [n_rows, d_hR]: decoded cache (fp64).
    q_nope [B, H, d_nope], q_rope [B, H, d_hR] (q_rope unrotated).
    For each (b, i), with L = seq_len[b] and rows seq_start[b] .. + L - 1:

        K = [C_b W_UK,i^T | R_b]          (L x (d_nope + d_hR))
        V = C_b W_UV,i^T                  (L x d_v)
        q = [q_nope[b,i] ; RoPE(q_rope[b,i], P_b)]
        s = softmax_scale * K q
        p = exp(s - max s) / sum(exp(s - max s))
        o[b,i] = V^T p

    Tokens are processed in chunks of ``chunk`` rows only to bound memory;
    the scores are all formed before the softmax (two passes, exact).

    Returns o [B, H, d_v] if ``pairs`` is None, else [len(pairs), d_v].
    """
    B, H, _ = q_nope.shape
    d_v = w_uv.shape[1]
    P = _positions(seq_len, q_pos)
    todo = _pairs(B, H, pairs)
    out = np.zeros((len(todo), d_v), dtype=np.float64)
    for n, (b, i) in enumerate(todo):
        L = int(seq_len[b])
        if L == 0:
            continue
        r0 = int(seq_start[b])
        q = _query(q_nope[b, i], q_rope[b, i], P[b], rope_base)
        s = np.empty(L, dtype=np.float64)
        for t0 in range(0, L, chunk):
            t1 = min(L, t0 + chunk)
            Cc = C[r0 + t0:r0 + t1]
            K = np.concatenate([Cc @ w_uk[i].T, R[r0 + t0:r0 + t1]], axis=1)
            s[t0:t1] = softmax_scale * (K @ q)
        e = np.exp(s - s.max())
        p = e / e.sum()
        o = np.zeros(d_v, dtype=np.float64)
        for t0 in range(0, L, chunk):
            t1 = min(L, t0 + chunk)
            V = C[r0 + t0:r0 + t1] @ w_uv[i].T
            o += V.T @ p[t0:t1]
        out[n] = o
    if pairs is None:
        return out.reshape(B, H, d_v)
    return out


def decode_absorbed(C, R, seq_start, seq_len, q_nope, q_rope, w_uk, w_uv,
                    softmax_scale, rope_base, q_pos=None, pairs=None):
    """Absorbed MLA decode (self-check of the rearrangement, not used for parity):

        q~   = W_UK,i^T q_nope[b,i]                 (d_c)
        s    = softmax_scale * (C_b q~ + R_b RoPE(q_rope[b,i], P_b))
        p    = softmax(s)
        o^   = C_b^T p                              (d_c, latent space)
        o    = W_UV,i o^

    Equal to :func:`decode` in exact arithmetic (associativity of the matrix
    products)."""
    B, H, _ = q_nope.shape
    d_v = w_uv.shape[1]
    P = _positions(seq_len, q_pos)
    todo = _pairs(B, H, pairs)
    out = np.zeros((len(todo), d_v), dtype=np.float64)
    for n, (b, i) in enumerate(todo):
        L = int(seq_len[b])
        if L == 0:
            continue
        r0 = int(seq_start[b])
        Cb, Rb = C[r0:r0 + L], R[r0:r0 + L]
        q_lat = w_uk[i].T @ q_nope[b, i]
        q_r = rope(q_rope[b, i], P[b], rope_base)
        s = softmax_scale * (Cb @ q_lat + Rb @ q_r)
        e = np.exp(s - s.max())
        p = e / e.sum()
        out[n] = w_uv[i] @ (Cb.T @ p)
    if pairs is None:
        return out.reshape(B, H, d_v)
    return out


def decode_absorbed_heads(Cb, Rb, q_nope_b, q_rope_b, w_uk, w_uv, softmax_scale, rope_base, pos):
    """The absorbed form of :func:`decode_absorbed` for every head of one
    sequence at once, with the per-head vectors stacked into matrices (a
    self-check form, pinned equal to the per-head forms; it lets whole
    outputs be compared at full size):

        Q~ [H, d_c]  with row i = W_UK,i^T q_nope[i]
        Qr [H, d_hR] with row i = RoPE(q_rope[i], pos)
        S  = softmax_scale * (C_b Q~^T + R_b Qr^T)      [L, H]
        P  = column-wise softmax of S                   (each head over the L tokens)
        O^ = P^T C_b                                    [H, d_c]
        o[i] = W_UV,i O^[i]                             [H, d_v]

    Cb [L, d_c] and Rb [L, d_hR] are the sequence's own cached rows (fp64);
    q_nope_b [H, d_nope], q_rope_b [H, d_hR] (unrotated); pos the query
    position. L = 0 gives zeros."""
    H = q_nope_b.shape[0]
    d_v = w_uv.shape[1]
    if Cb.shape[0] == 0:
        return np.zeros((H, d_v), dtype=np.float64)
    q_lat = np.einsum("hnc,hn->hc", w_uk, q_nope_b)
    q_r = rope(q_rope_b, pos, rope_base)
    s = softmax_scale * (Cb @ q_lat.T + Rb @ q_r.T)
    e = np.exp(s - s.max(axis=0, keepdims=True))
    p = e / e.sum(axis=0, keepdims=True)
    o_hat = p.T @ Cb
    return np.einsum("hvc,hc->hv", w_uv, o_hat)


# ------------------------------------------------------ several query tokens


def decode_multi(C, R, seq_start, seq_len, q_nope, q_rope, w_uk, w_uv, softmax_scale,
                 rope_base, q_pos=None, triples=None, absorbed=False):
    """Decode of Q new query tokens per sequence (the use the pages name next
    to MLA: multi-token prediction and speculative decoding, "Multi-head Latent
    Attention (MLA) și arhitectura DeepSeekMoE", "Concepte cheie și
    caracteristici"; "02 — Multi-Latent Attention (MLA)", "Lo que esta fase NO
    cubre"). The pages give no formula for it; the plainest reading, causal
    attention among the new tokens, is taken:

    * the Q new tokens are the last Q cached rows of the sequence (appended
      before the decode, as for one token);
    * query j (j = 0 .. Q-1) sits at position P_b - (Q - 1 - j), with P_b =
      q_pos[b] or seq_len[b] - 1, and sees rows 0 .. seq_len[b] - 1 - (Q - 1 - j):
      itself and what precedes it, never a later new token;
    * so query j is exactly one single-token decode over the cache truncated
      to the rows it sees, which is how it is computed here.

    q_nope [B, Q, H, d_nope], q_rope [B, Q, H, d_hR]. A query that sees no row
    (seq_len[b] < Q - j) gives 0. Returns o [B, Q, H, d_v], or [len(triples),
    d_v] for a list of (b, j, i) triples."""
    B, Q, H, _ = q_nope.shape
    d_v = w_uv.shape[1]
    fn = decode_absorbed if absorbed else decode
    L = np.asarray(seq_len, dtype=np.int64)
    P = _positions(seq_len, q_pos)
    if triples is None:
        out = np.zeros((B, Q, H, d_v), dtype=np.float64)
        for j in range(Q):
            back = Q - 1 - j
            out[:, j] = fn(C, R, seq_start, np.maximum(L - back, 0), q_nope[:, j], q_rope[:, j], w_uk, w_uv,
                           softmax_scale, rope_base, q_pos=P - back)
        return out
    out = np.zeros((len(triples), d_v), dtype=np.float64)
    for n, (b, j, i) in enumerate(triples):
        back = Q - 1 - int(j)
        out[n] = fn(C, R, seq_start, np.maximum(L - back, 0), q_nope[:, j], q_rope[:, j], w_uk, w_uv,
                    softmax_scale, rope_base, q_pos=P - back, pairs=[(int(b), int(i))])[0]
    return out


# ------------------------------------------------------------------ split merge


def partial_attention(s, V):
    """Softmax attention over one subset of tokens, kept mergeable:
    returns (o_s, lse_s) with o_s = sum_t softmax(s)_t V_t over the subset and
    lse_s = log sum_t exp(s_t). An empty subset gives (0, -inf)."""
    s = np.asarray(s, dtype=np.float64)
    if s.size == 0:
        return np.zeros(V.shape[1:], dtype=np.float64), -np.inf
    m = s.max()
    e = np.exp(s - m)
    return (e / e.sum()) @ V, m + np.log(e.sum())


def lse_merge(parts):
    """Merge split partials [(o_s, lse_s), ...] into the unsplit result:

        M = max_s lse_s,  w_s = exp(lse_s - M),  o = sum_s w_s o_s / sum_s w_s

    Splits with lse_s = -inf weigh 0; if every split is empty the result is 0.
    (Split-K over the sequence is not on the pages; this is the log-sum-exp
    identity that makes it exact.)"""
    lses = np.array([l for _, l in parts], dtype=np.float64)
    if not np.isfinite(lses).any():
        return np.zeros_like(np.asarray(parts[0][0], dtype=np.float64))
    M = lses[np.isfinite(lses)].max()
    w = np.where(np.isfinite(lses), np.exp(lses - M), 0.0)
    num = sum(wi * np.asarray(o, dtype=np.float64) for wi, (o, _) in zip(w, parts))
    return num / w.sum()
