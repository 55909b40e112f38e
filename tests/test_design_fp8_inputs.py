"""fp8-input matrix-core products for the fp8 cache, emulated in fp64 on the
oracle's own inputs (CPU only; no part of the library is involved), against
the fp8-cache tolerance max|err| / rms(ref) <= 6e-2:

* one e4m3 value per element misses it: q~ quantised with one scale per
  head, or P times the token scale with one scale per head or per 32-token
  tile (e4m3 keeps 4 significant bits);
* hi + lo pairs meet it with a wide margin: q~ = s (hi + s_lo lo) per head
  and P times the token scale the same way per 32-token tile, each part an
  e4m3 value with its own scale (about 8 significant bits): 3.2e-3 with both
  paired. The matrix cores then run two fp8 products where one fp16 product
  ran; at twice the fp16 rate that is the same matrix-core time."""
import numpy as np

import mla_synth
from oracle import codecs
from oracle import mla as omla
from oracle.rope import rope
from tests.helpers import TOL_FP8_REL, act_to_f64, oracle_cache

LOG2E = 1.4426950408889634


def _q8(v, mode):
    """v through e4m3 with one scale for all of v ("e4m3"), or as a hi + lo
    pair with a scale each ("hilo"); "exact" leaves it."""
    if mode == "exact":
        return v
    s = np.abs(v).max() / 448.0
    if s == 0:
        return v
    hi = codecs.e4m3_round(v / s)
    if mode == "e4m3":
        return s * hi
    r = v / s - hi
    ls = np.abs(r).max() / 448.0
    return s * hi if ls == 0 else s * hi + s * ls * codecs.e4m3_round(r / ls)


def _p8(pp, mode, tile=32):
    out = np.empty_like(pp)
    for t0 in range(0, len(pp), tile):
        out[t0:t0 + tile] = _q8(pp[t0:t0 + tile], mode)
    return out


def _emulate_modes(lens, seed, q_mode, p_mode):
    """Scores from q~ in q_mode; P times the token scale in p_mode per 32-token tile."""
    case = mla_synth.make_case("fp8_inputs", H=128, d_c=512, d_rope=64, d_nope=128, d_v=128, B=len(lens),
                               lens=("list", lens), latent_dtype="fp8", rope_dtype="bf16", act_dtype="bf16",
                               seed=seed)
    C, R = oracle_cache(case)
    qn, qr = act_to_f64(case.q_nope, "bf16"), act_to_f64(case.q_rope, "bf16")
    wuk, wuv = act_to_f64(case.w_uk, "bf16"), act_to_f64(case.w_uv, "bf16")
    ref = omla.decode_absorbed(C, R, case.seq_start, case.lens, qn, qr, wuk, wuv, case.softmax_scale, case.rope_base)
    out = np.zeros_like(ref)
    for b, L in enumerate(int(x) for x in case.lens):
        s0 = int(case.seq_start[b])
        sc = case.scale[s0:s0 + L].astype(np.float64)
        codes = C[s0:s0 + L] / sc[:, None]
        for h in range(case.H):
            qt = wuk[h].T @ qn[b, h] * case.softmax_scale * LOG2E
            q_r = rope(qr[b, h], L - 1, case.rope_base) * case.softmax_scale * LOG2E
            s = sc * (codes @ _q8(qt, q_mode)) + R[s0:s0 + L] @ q_r
            p = np.exp2(s - s.max())
            out[b, h] = wuv[h] @ (_p8(p * sc, p_mode) @ codes / p.sum())
    return float(np.abs(out - ref).max() / np.sqrt(np.mean(ref ** 2)))


def _emulate(lens, seed, quant_q, quant_p):
    case = mla_synth.make_case("fp8_inputs", H=128, d_c=512, d_rope=64, d_nope=128, d_v=128, B=len(lens),
                               lens=("list", lens), latent_dtype="fp8", rope_dtype="bf16", act_dtype="bf16",
                               seed=seed)
    C, R = oracle_cache(case)
    qn, qr = act_to_f64(case.q_nope, "bf16"), act_to_f64(case.q_rope, "bf16")
    wuk, wuv = act_to_f64(case.w_uk, "bf16"), act_to_f64(case.w_uv, "bf16")
    ref = omla.decode_absorbed(C, R, case.seq_start, case.lens, qn, qr, wuk, wuv, case.softmax_scale, case.rope_base)
    out = np.zeros_like(ref)
    for b, L in enumerate(int(x) for x in case.lens):
        s0 = int(case.seq_start[b])
        sc = case.scale[s0:s0 + L].astype(np.float64)
        codes = C[s0:s0 + L] / sc[:, None]  # the stored e4m3 values
        for h in range(case.H):
            qt = wuk[h].T @ qn[b, h] * case.softmax_scale * LOG2E
            q_r = rope(qr[b, h], L - 1, case.rope_base) * case.softmax_scale * LOG2E
            if quant_q:
                qs = np.abs(qt).max() / 448.0
                s = sc * qs * (codes @ codecs.e4m3_round(qt / qs)) + R[s0:s0 + L] @ q_r
            else:
                s = sc * (codes @ qt) + R[s0:s0 + L] @ q_r
            p = np.exp2(s - s.max())
            pp = p * sc
            if quant_p:
                ps = pp.max() / 448.0
                pp = ps * codecs.e4m3_round(pp / ps)
            out[b, h] = wuv[h] @ (pp @ codes / p.sum())
    return float(np.abs(out - ref).max() / np.sqrt(np.mean(ref ** 2)))


def test_emulation_is_exact_without_quantisation():
    assert _emulate([1, 7, 31, 100], 5, False, False) < 1e-12


def test_fp8_query_or_probabilities_miss_the_fp8_tolerance():
    assert _emulate([1, 7, 31, 100], 5, True, False) > TOL_FP8_REL
    assert _emulate([1, 7, 31, 100], 5, False, True) > TOL_FP8_REL


def test_single_e4m3_per_tile_probabilities_miss_the_tolerance():
    assert _emulate_modes([1, 7, 31, 100], 5, "exact", "e4m3") > TOL_FP8_REL


def test_hi_lo_pairs_meet_the_tolerance():
    assert _emulate_modes([1, 7, 31, 100], 5, "hilo", "exact") < 1e-2
    assert _emulate_modes([1, 7, 31, 100], 5, "exact", "hilo") < 1e-2
    assert _emulate_modes([1, 7, 31, 100, 700], 6, "hilo", "hilo") < 1e-2
