"""Why the fp8 cache keeps fp16 matrix-core products: an fp64 emulation of
fp8-input products (q~ quantised per head to e4m3; P times the token scale
quantised per head to e4m3; scales folded into the fp32 results) misses the
fp8-cache tolerance (max|err| / rms(ref) <= 6e-2) on the oracle's own inputs.
CPU only; no part of the library is involved."""
import numpy as np

import mla_synth
from oracle import codecs
from oracle import mla as omla
from oracle.rope import rope
from tests.helpers import TOL_FP8_REL, act_to_f64, oracle_cache

LOG2E = 1.4426950408889634


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
