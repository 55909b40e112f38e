"""CPU check of the matrix-core path's numeric domain (a design record, not
a kernel test).

* Range: the cached bf16 values widened to fp16 the way the kernel converts
  them (round toward zero, saturating at 65504), everything else exact,
  decoded by the oracle's absorbed form. Inside the stated range (row scales
  2^-14 .. 2^13) the widening alone costs well under the bf16 tolerance;
  uniformly at 2^-20 (fp16 subnormals) or at 2^15 (saturation) it exceeds
  the tolerance by itself, which is why those caches belong on the fp32
  kernels.
* Accuracy: every fp16 carrier the kernel uses (widened cache, absorbed
  query and rotated rope query pre-multiplied by softmax_scale * log2 e and
  rounded to nearest, probabilities rounded to nearest before the value
  product, fp32 sums). The query's rounding (relative 2^-11) moves each
  score by an amount that grows with the score's size, so the output's
  error grows with the largest score: it stays within the bf16 tolerance
  plus 2^-13 times the largest |score| in log2 units."""
import numpy as np
import pytest

from oracle import mla as omla
from oracle.rope import rope
from tests.helpers import TOL_BF16_REL, act_to_f64, make, oracle_full, rel_rms_err

V3 = dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128)


def f16_toward_zero(x):
    f = x.astype(np.float16).astype(np.float64)  # round to nearest (may overflow to inf)
    away = np.abs(f) > np.abs(x)
    toward = np.nextafter(f.astype(np.float16), np.float16(0)).astype(np.float64)
    return np.clip(np.where(away, toward, f), -65504.0, 65504.0)


def widening_error(scale_exp):
    case = make(B=4, lens=("list", [1, 33, 200, 700]), latent_dtype="bf16", rope_dtype="bf16", act_dtype="bf16",
                seed=190, cache_std=2.0 ** scale_exp, **V3)
    ref = oracle_full(case)
    C, R = omla.decode_rows(case.rows, "bf16", "bf16", case.d_c, case.d_rope)
    with np.errstate(over="ignore"):
        C16, R16 = f16_toward_zero(C), f16_toward_zero(R)
    qn, qr = act_to_f64(case.q_nope, "bf16"), act_to_f64(case.q_rope, "bf16")
    wuk, wuv = act_to_f64(case.w_uk, "bf16"), act_to_f64(case.w_uv, "bf16")
    out = np.zeros_like(ref)
    for b in range(case.B):
        s0, L = int(case.seq_start[b]), int(case.lens[b])
        out[b] = omla.decode_absorbed_heads(C16[s0:s0 + L], R16[s0:s0 + L], qn[b], qr[b], wuk, wuv,
                                            case.softmax_scale, case.rope_base, L - 1)
    return float(np.max(np.abs(out - ref)) / np.sqrt(np.mean(ref ** 2)))


@pytest.mark.parametrize("scale_exp", [-14, 0, 13])
def test_widening_inside_the_domain_costs_little(scale_exp):
    assert widening_error(scale_exp) < 5e-3


@pytest.mark.parametrize("scale_exp", [-20, 15])
def test_widening_outside_the_domain_exceeds_the_tolerance(scale_exp):
    assert widening_error(scale_exp) > 2e-2


LOG2E = 1.4426950408889634
LENS = [1, 31, 32, 33, 100, 700, 0, 64, 200]


def f16_nearest(x):
    return x.astype(np.float16).astype(np.float64)


def carriers_error(scale_exp, seed):
    """Decode with every fp16 carrier of the matrix-core path; returns the
    error against the oracle (max |err| / rms) and the largest |score| in
    log2 units (exact)."""
    case = make(B=len(LENS), lens=("list", LENS), latent_dtype="bf16", rope_dtype="bf16", act_dtype="bf16",
                seed=seed, cache_std=2.0 ** scale_exp, **V3)
    ref = oracle_full(case)
    C, R = omla.decode_rows(case.rows, "bf16", "bf16", case.d_c, case.d_rope)
    qn, qr = act_to_f64(case.q_nope, "bf16"), act_to_f64(case.q_rope, "bf16")
    wuk, wuv = act_to_f64(case.w_uk, "bf16"), act_to_f64(case.w_uv, "bf16")
    k = case.softmax_scale * LOG2E
    out = np.zeros_like(ref)
    smax = 0.0
    for b in range(case.B):
        s0, L = int(case.seq_start[b]), int(case.lens[b])
        if L == 0:
            continue
        Cb, Rb = f16_toward_zero(C[s0:s0 + L]), f16_toward_zero(R[s0:s0 + L])
        q_lat = np.einsum("hnc,hn->hc", wuk, qn[b]) * k
        q_r = rope(qr[b], L - 1, case.rope_base) * k
        smax = max(smax, float(np.max(np.abs(C[s0:s0 + L] @ q_lat.T + R[s0:s0 + L] @ q_r.T))))
        s = Cb @ f16_nearest(q_lat).T + Rb @ f16_nearest(q_r).T
        e = np.exp2(s - s.max(axis=0, keepdims=True))
        out[b] = np.einsum("hvc,hc->hv", wuv, (f16_nearest(e).T @ Cb) / e.sum(axis=0)[:, None])
    return rel_rms_err(out, ref), smax


@pytest.mark.parametrize("scale_exp", [-14, 0, 3, 5, 8])
def test_query_rounding_error_grows_with_the_largest_score(scale_exp):
    err, smax = carriers_error(scale_exp, 140 + scale_exp)
    assert err <= TOL_BF16_REL + 2.0 ** -13 * smax
    if smax <= 64:
        assert err <= TOL_BF16_REL
    if scale_exp == 8:  # scores near 1800: the bound's second term is needed
        assert err > TOL_BF16_REL
