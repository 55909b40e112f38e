"""GPU tests of the matrix-core path's numeric domain (fp16 carriers for the
cached values and the absorbed query; see mla_decode in include/mla.h):

* caches whose scores stay below 64 in log2 units decode within the bf16
  tolerance of the oracle, from rows at 2^-14 in scale up, also with
  planted rows far smaller (2^-20, negligible beside the others) or far
  larger (2^13, dominating the softmax) than the rest;
* larger scores (caches at 2^5 and 2^8: scores near 230 and 1800) decode
  within the bf16 tolerance plus 2^-13 times the largest |score|, the
  query's fp16 rounding;
* a cache uniformly at 2^-20, or reaching 2^15, is outside the domain: the
  fp32 kernels (MLA_FORCE_GENERIC=1) decode it within 1e-4 plus the score
  term of fp32's rounding (2^-26 times the largest |score|);
* the library's own producers report values beyond fp16's range
  (MLA_ERR_RANGE): mla_append for the rows it writes (stored as they are),
  the decode for an absorbed query."""
import numpy as np
import pytest

from oracle import mla as omla
from oracle.rope import rope
from tests.helpers import DeviceRun, TOL_BF16_REL, TOL_FP8_REL, act_to_f64, make, oracle_full, rel_rms_err, to_np

pytestmark = pytest.mark.gpu

V3 = dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128)
LENS = [1, 31, 32, 33, 100, 700, 0, 64, 200]
MLA_ERR_RANGE = 7


def case_at(scale_exp, seed, **kw):
    return make(B=len(LENS), lens=("list", LENS), latent_dtype="bf16", rope_dtype="bf16", act_dtype="bf16",
                seed=seed, cache_std=2.0 ** scale_exp, **V3, **kw)


def max_log2_score(case):
    """Largest |softmax_scale * log2 e * q.k| over every head and token."""
    C, R = omla.decode_rows(case.rows, case.latent_dtype, case.rope_dtype, case.d_c, case.d_rope)
    qn, qr = act_to_f64(case.q_nope, case.act_dtype), act_to_f64(case.q_rope, case.act_dtype)
    wuk = act_to_f64(case.w_uk, case.act_dtype)
    out = 0.0
    for b in range(case.B):
        s0, L = int(case.seq_start[b]), int(case.lens[b])
        if L == 0:
            continue
        q_lat = np.einsum("hnc,hn->hc", wuk, qn[b])
        q_r = rope(qr[b], L - 1, case.rope_base)
        s = C[s0:s0 + L] @ q_lat.T + R[s0:s0 + L] @ q_r.T
        out = max(out, float(np.max(np.abs(s))) * case.softmax_scale * 1.4426950408889634)
    return out


@pytest.mark.parametrize("scale_exp", [-14, -8, 0, 3])
def test_cache_scales_inside_the_domain(gpu, scale_exp):
    case = case_at(scale_exp, 140 + scale_exp)
    assert max_log2_score(case) <= 64
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(n_workers=20))
    assert run.status() == 0
    assert rel_rms_err(o, oracle_full(case)) <= TOL_BF16_REL


@pytest.mark.parametrize("scale_exp", [5, 8])
def test_large_scores_error_bounded_by_the_query_rounding(gpu, scale_exp):
    case = case_at(scale_exp, 140 + scale_exp)
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(n_workers=20))
    assert run.status() == 0
    assert rel_rms_err(o, oracle_full(case)) <= TOL_BF16_REL + 2.0 ** -13 * max_log2_score(case)


@pytest.mark.parametrize("spike_exp", [-20, 13])
def test_planted_rows_far_from_the_rest(gpu, spike_exp):
    case = make(B=len(LENS), lens=("list", LENS), latent_dtype="bf16", rope_dtype="bf16", act_dtype="bf16",
                seed=160 + spike_exp, spike_frac=0.05, spike_mult=2.0 ** spike_exp, **V3)
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(n_workers=20))
    assert run.status() == 0
    assert rel_rms_err(o, oracle_full(case)) <= TOL_BF16_REL


@pytest.mark.parametrize("scale_exp", [-20, 15])
def test_outside_the_domain_the_fp32_kernels_decode(gpu, scale_exp, monkeypatch):
    case = case_at(scale_exp, 170 + scale_exp)
    monkeypatch.setenv("MLA_FORCE_GENERIC", "1")
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(n_workers=20))
    assert run.status() == 0
    # fp32 carriers: the fp16 bound's score term scaled by 2^-13 (24 significand bits, not 11)
    assert rel_rms_err(o, oracle_full(case)) <= 1e-4 + 2.0 ** -26 * max_log2_score(case)


def scale_bf16(bits, exp):
    """bf16 bit patterns times 2^exp (exponent field shifted; zeros stay)."""
    bits = bits.astype(np.int32)
    nz = (bits & 0x7F80) != 0
    return np.where(nz, bits + (exp << 7), bits).astype(np.uint16)


@pytest.mark.parametrize("latent", ["bf16", "fp8"])
def test_append_reports_rows_beyond_fp16(gpu, latent):
    """h times 2^17: every appended latent row is near 2^17 in scale, past
    fp16's 65504; the rows are stored (they are valid bf16 / fp8 data) and
    the status word says MLA_ERR_RANGE."""
    lens = [5, 40]
    case = make(B=2, lens=("list", lens), latent_dtype=latent, rope_dtype="bf16", act_dtype="bf16", seed=180,
                n_new=1, d_model=1024, extra_cap=4, **V3)
    case.h = scale_bf16(case.h, 17)
    run = DeviceRun(gpu, case)
    before = run.t["rows"].cpu().numpy().copy()
    run.append()
    assert run.status() == MLA_ERR_RANGE
    assert run.t["seq_len"].cpu().tolist() == [6, 41]
    after = run.t["rows"].cpu().numpy()
    changed = np.flatnonzero(np.any(after != before, axis=1)).tolist()
    assert changed == [int(case.seq_start[b]) + lens[b] for b in range(2)]


def test_append_in_range_reports_nothing(gpu):
    lens = [5, 40]
    case = make(B=2, lens=("list", lens), latent_dtype="fp8", rope_dtype="bf16", act_dtype="bf16", seed=181,
                n_new=1, d_model=1024, extra_cap=4, **V3)
    run = DeviceRun(gpu, case)
    o = to_np(run.append_decode())
    assert run.status() == 0
    assert rel_rms_err(o, oracle_full(case)) <= TOL_FP8_REL


def test_decode_reports_query_beyond_fp16(gpu):
    """q_nope times 2^20: the absorbed query passes 65504 after the softmax
    scale, so the decode reports MLA_ERR_RANGE."""
    case = case_at(0, 182)
    case.q_nope = scale_bf16(case.q_nope, 20)
    run = DeviceRun(gpu, case)
    run.decode(n_workers=20)
    assert run.status() == MLA_ERR_RANGE
