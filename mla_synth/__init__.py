"""Seeded synthetic inputs for MLA decode, shared by the GPU tests, the oracle
tests and the benchmark.

This module only draws random numbers, lays them out and casts them to their
storage dtypes with PyTorch's CPU casts (``torch.bfloat16``,
``torch.float8_e4m3fn``); it holds none of the attention arithmetic. Neither
the oracle nor the HIP path is imported here.

Workloads (DeepSeek-V3-shaped: latent width 512 and RoPE key width 64 are the
``kv_lora_rank`` / ``qk_rope_head_dim`` values quoted in "Multi-head Latent
Attention (MLA) și arhitectura DeepSeekMoE", "Concepte cheie"; the other sizes
are the workloads' own):

  tiny_f32     B=1, H=4, d_model=64, d_c=32, d_hR=8, d_nope=16, d_v=16,
               64 tokens appended from h (positions 0..63), q = W_Q h_63, fp32.
  v3_b1_4k     B=1, H=128, d_c=512, d_hR=64, d_nope=128, d_v=128, L=4096, bf16.
  v3_b32_ragged  B=32, L ~ U{4096..8192}, bf16 (ragged contiguous cache).
  v3_b32_8k    B=32, L=8192 for every sequence (the literal "ctx=8K").
  v3_b4_128k   B=4, L=131072, 1 % of rows (1311 per sequence) scaled x8.
  v3_b128_fp8  B=128, L_old = floor(exp(U[ln 1024, ln 32768])), fp8 e4m3
               latent with one fp32 scale per token, bf16 k_rope, plus one
               appended token per sequence from h [128, 7168] (bf16).

Draw order, fixed: lengths -> latents -> k_rope -> spike rows -> h -> q_nope
-> q_rope -> W_DKV -> W_KR -> W_UK -> W_UV -> W_Q. Activations are N(0, 1);
weights are N(0, 1/fan_in) with fan_in = d_c for W_UK and W_UV and d_model
for W_DKV, W_KR and W_Q. Seeds: workload k of the list above uses seed k
unless told otherwise.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
F8_MAX = 448.0

WORKLOADS = {
    "tiny_f32": dict(H=4, d_c=32, d_rope=8, d_nope=16, d_v=16, d_model=64, B=1,
                     lens=("const", 0), n_new=64, latent_dtype="f32", rope_dtype="f32",
                     act_dtype="f32", query_from_h=True, seed=0),
    "v3_b1_4k": dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128, B=1,
                     lens=("const", 4096), latent_dtype="bf16", rope_dtype="bf16",
                     act_dtype="bf16", seed=1),
    "v3_b32_ragged": dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128, B=32,
                          lens=("uniform", 4096, 8192), latent_dtype="bf16",
                          rope_dtype="bf16", act_dtype="bf16", seed=2),
    "v3_b4_128k": dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128, B=4,
                       lens=("const", 131072), latent_dtype="bf16", rope_dtype="bf16",
                       act_dtype="bf16", spike_frac=0.01, spike_mult=8.0, seed=3),
    "v3_b128_fp8": dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128, d_model=7168,
                        B=128, lens=("loguniform", 1024, 32768), n_new=1,
                        latent_dtype="fp8", rope_dtype="bf16", act_dtype="bf16", seed=4),
    "v3_b32_8k": dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128, B=32,
                      lens=("const", 8192), latent_dtype="bf16", rope_dtype="bf16",
                      act_dtype="bf16", seed=2),
}


@dataclass
class Case:
    """One decode problem in storage form (NumPy, host memory).

    rows: uint8 [n_rows, row_stride]; a row is [c_kv | k_rope] from byte 0.
    scale: float32 [n_rows] (fp8 latent only) or None.
    lens: cached rows per sequence before any append (int32 [B]).
    seq_start / seq_cap: first row and capacity of each sequence (int32 [B]).
    Activations and weights are float32 (act_dtype "f32") or uint16 bf16 bits.
    """
    name: str
    H: int
    d_c: int
    d_rope: int
    d_nope: int
    d_v: int
    d_model: int
    B: int
    latent_dtype: str
    rope_dtype: str
    act_dtype: str
    softmax_scale: float
    rope_base: float
    row_stride: int
    lens: np.ndarray
    seq_start: np.ndarray
    seq_cap: np.ndarray
    rows: np.ndarray
    scale: object
    q_nope: np.ndarray
    q_rope: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    n_new: int = 0
    h: object = None
    w_dkv: object = None
    w_kr: object = None
    extra: dict = field(default_factory=dict)

    @property
    def n_rows(self):
        return self.rows.shape[0]

    @property
    def row_bytes(self):
        """Algorithmic bytes read per cached token (scale included)."""
        rb = self.d_c * ELEM_BYTES[self.latent_dtype] + self.d_rope * ELEM_BYTES[self.rope_dtype]
        return rb + (4 if self.latent_dtype == "fp8" else 0)


def _normal(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def to_storage(x, dtype):
    """float32 array -> storage array: float32 itself, or uint16 bf16 bits
    (PyTorch's round-to-nearest-even cast)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def fp8_rows(x):
    """float32 latents [n, d] -> (uint8 e4m3fn codes, float32 per-row scale)
    with the row's largest magnitude mapped to 448 (scale 1 for a zero row);
    the cast is PyTorch's float8_e4m3fn cast."""
    amax = np.abs(x).max(axis=1)
    s = np.where(amax > 0, amax / np.float32(F8_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(x / s[:, None], -F8_MAX, F8_MAX)
    codes = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, s


def draw_lens(rng, spec, B):
    kind = spec[0]
    if kind == "const":
        return np.full(B, spec[1], dtype=np.int32)
    if kind == "uniform":
        return rng.integers(spec[1], spec[2], size=B, endpoint=True).astype(np.int32)
    if kind == "loguniform":
        u = rng.uniform(math.log(spec[1]), math.log(spec[2]), size=B)
        return np.clip(np.floor(np.exp(u)), spec[1], spec[2]).astype(np.int32)
    if kind == "list":
        return np.asarray(spec[1], dtype=np.int32)
    raise ValueError(kind)


def make_case(name="custom", *, H, d_c, d_rope, d_nope, d_v, B, lens,
              latent_dtype, rope_dtype, act_dtype, seed, d_model=None, n_new=0,
              spike_frac=0.0, spike_mult=8.0, query_from_h=False, extra_cap=0,
              softmax_scale=None, rope_base=10000.0, row_pad=0, gap_rows=0,
              cache_std=1.0):
    """Build one seeded case. ``lens`` is a spec tuple (see :func:`draw_lens`).

    ``extra_cap`` adds spare capacity per sequence beyond ``n_new``; ``gap_rows``
    puts unused rows between sequences; ``row_pad`` adds bytes to each row
    (row_stride stays a multiple of 16)."""
    rng = np.random.default_rng(seed)
    lens_a = draw_lens(rng, lens, B)
    cap = lens_a + n_new + extra_cap
    seq_start = np.zeros(B, dtype=np.int32)
    acc = 0
    for b in range(B):
        seq_start[b] = acc
        acc += int(cap[b]) + gap_rows
    n_rows = max(acc, 1)
    lat_b = d_c * ELEM_BYTES[latent_dtype]
    rope_b = d_rope * ELEM_BYTES[rope_dtype]
    row_stride = -(-(lat_b + rope_b + row_pad) // 16) * 16
    rows = np.zeros((n_rows, row_stride), dtype=np.uint8)
    scale = np.ones(n_rows, dtype=np.float32) if latent_dtype == "fp8" else None

    # latents and k_rope for the cached rows, sequence by sequence
    total = int(lens_a.sum())
    lat = _normal(rng, (total, d_c), cache_std)
    kr = _normal(rng, (total, d_rope), cache_std)
    if spike_frac > 0:
        off = 0
        for b in range(B):
            L = int(lens_a[b])
            k = int(round(spike_frac * L))
            idx = rng.choice(L, size=k, replace=False) + off
            lat[idx] *= np.float32(spike_mult)
            kr[idx] *= np.float32(spike_mult)
            off += L
    row_idx = np.concatenate([np.arange(int(seq_start[b]), int(seq_start[b]) + int(lens_a[b]))
                              for b in range(B)]) if total else np.zeros(0, dtype=np.int64)
    if total:
        if latent_dtype == "fp8":
            codes, s = fp8_rows(lat)
            rows[row_idx, :lat_b] = codes
            scale[row_idx] = s
        else:
            rows[row_idx, :lat_b] = to_storage(lat, latent_dtype).view(np.uint8).reshape(total, lat_b)
        rows[row_idx, lat_b:lat_b + rope_b] = to_storage(kr, rope_dtype).view(np.uint8).reshape(total, rope_b)
    del lat, kr

    h = None
    if n_new:
        if d_model is None:
            raise ValueError("appending needs d_model")
        h = _normal(rng, (B, n_new, d_model))
    q_nope = _normal(rng, (B, H, d_nope))
    q_rope = _normal(rng, (B, H, d_rope))
    w_dkv = w_kr = None
    if n_new:
        w_dkv = _normal(rng, (d_c, d_model), 1.0 / math.sqrt(d_model))
        w_kr = _normal(rng, (d_rope, d_model), 1.0 / math.sqrt(d_model))
    w_uk = _normal(rng, (H, d_nope, d_c), 1.0 / math.sqrt(d_c))
    w_uv = _normal(rng, (H, d_v, d_c), 1.0 / math.sqrt(d_c))
    extra = {}
    if query_from_h:
        # The query projection sits outside the decode path: q = W_Q h of the
        # last appended token, formed here in fp64 and handed to both sides
        # rounded to fp32. W_Q is [H * (d_nope + d_rope), d_model].
        w_q = _normal(rng, (H * (d_nope + d_rope), d_model), 1.0 / math.sqrt(d_model))
        q = (w_q.astype(np.float64) @ h[:, -1, :].astype(np.float64).T).T.reshape(B, H, d_nope + d_rope)
        q_nope = q[..., :d_nope].astype(np.float32)
        q_rope = q[..., d_nope:].astype(np.float32)
        extra["w_q"] = w_q
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d_nope + d_rope)
    st = lambda x: None if x is None else to_storage(x, act_dtype)
    return Case(name=name, H=H, d_c=d_c, d_rope=d_rope, d_nope=d_nope, d_v=d_v,
                d_model=d_model or 0, B=B, latent_dtype=latent_dtype, rope_dtype=rope_dtype,
                act_dtype=act_dtype, softmax_scale=float(softmax_scale), rope_base=float(rope_base),
                row_stride=row_stride, lens=lens_a, seq_start=seq_start,
                seq_cap=cap.astype(np.int32), rows=rows, scale=scale,
                q_nope=st(q_nope), q_rope=st(q_rope), w_uk=st(w_uk), w_uv=st(w_uv),
                n_new=n_new, h=st(h), w_dkv=st(w_dkv), w_kr=st(w_kr), extra=extra)


def multi_queries(case, q_len, seed):
    """Queries of q_len new tokens per sequence for a several-token decode:
    q_nope [B, q_len, H, d_nope] and q_rope [B, q_len, H, d_rope], N(0, 1), in
    the case's activation dtype. The last token's queries are the case's own,
    the earlier ones come from ``seed``."""
    rng = np.random.default_rng(seed)
    B, H = case.B, case.H
    shape_n, shape_r = (B, q_len, H, case.d_nope), (B, q_len, H, case.d_rope)
    q_nope = np.empty(shape_n, dtype=case.q_nope.dtype)
    q_rope = np.empty(shape_r, dtype=case.q_rope.dtype)
    q_nope[:, :q_len - 1] = to_storage(_normal(rng, (B, q_len - 1, H, case.d_nope)), case.act_dtype)
    q_rope[:, :q_len - 1] = to_storage(_normal(rng, (B, q_len - 1, H, case.d_rope)), case.act_dtype)
    q_nope[:, q_len - 1] = case.q_nope
    q_rope[:, q_len - 1] = case.q_rope
    return q_nope, q_rope


def merged_inputs(case, d_x, d_out, seed):
    """Inputs of a decode from precomputed absorbed weights, drawn from their
    own generator (``seed``) so the case's own draws are unchanged, in this
    order: x [B, d_x] N(0, 1) (each sequence's query input), W_Q
    [H, d_nope, d_x] N(0, 1/d_x), W_O [d_out, H d_v] N(0, 1/(H d_v)); all in
    the case's activation dtype. The rotary query is the case's q_rope."""
    rng = np.random.default_rng(seed)
    x = _normal(rng, (case.B, d_x))
    w_q = _normal(rng, (case.H, case.d_nope, d_x), 1.0 / math.sqrt(d_x))
    w_o = _normal(rng, (d_out, case.H * case.d_v), 1.0 / math.sqrt(case.H * case.d_v))
    return to_storage(x, case.act_dtype), to_storage(w_q, case.act_dtype), to_storage(w_o, case.act_dtype)


def workload(name, seed=None, **overrides):
    """Build one of the named workloads (see the module docstring)."""
    kw = dict(WORKLOADS[name])
    if seed is not None:
        kw["seed"] = seed
    kw.update(overrides)
    return make_case(name, **kw)
