"""GPU parity at the workloads' full sizes, through the C ABI, in the launch
configuration the benchmark times (default plan over all CUs, bf16 output).

Every output (all sequences, all heads) is compared with the oracle's
all-heads absorbed form (pinned equal to the definition by the CPU tests),
run one sequence at a time on the host; the bound is max|err| / rms with the
rms over the whole reference output. A few (sequence, head) outputs are also
compared with the non-absorbed definition itself."""
import numpy as np
import pytest

import mla_synth
from tests.helpers import (DeviceRun, TOL_BF16_REL, TOL_FP8_REL, oracle_append, oracle_cache, oracle_decode,
                           oracle_full, rel_rms_err, to_np)

pytestmark = pytest.mark.gpu


def full_check(case, o, tol, def_pairs=()):
    """Whole-output check, plus the definition on def_pairs."""
    ref = oracle_full(case)
    err = rel_rms_err(o, ref)
    assert err <= tol, f"all outputs: max|err|/rms {err:.3e} > {tol}"
    if def_pairs:
        seqs = sorted({b for b, _ in def_pairs})
        C, R = oracle_cache(case, seqs=seqs)
        ref_def = oracle_decode(case, pairs=list(def_pairs), absorbed=False, C=C, R=R)
        got = np.stack([o[b, i] for b, i in def_pairs])
        rms = float(np.sqrt(np.mean(ref ** 2)))
        err_def = float(np.max(np.abs(got - ref_def))) / rms
        assert err_def <= tol, f"outputs vs the definition: {err_def:.3e}"
    return err


def test_workload_v3_b1_4k(gpu):
    """One sequence of 4096 tokens, H=128."""
    case = mla_synth.workload("v3_b1_4k")
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(o_dtype="bf16"))
    assert run.status() == 0
    full_check(case, o, TOL_BF16_REL, def_pairs=[(0, 0), (0, 77)])


def test_workload_v3_b32_ragged_bench_config(gpu):
    """The benchmark's workload and launch configuration."""
    case = mla_synth.workload("v3_b32_ragged")
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(o_dtype="bf16"))
    assert run.status() == 0
    full_check(case, o, TOL_BF16_REL, def_pairs=[(0, 5), (17, 64), (31, 127)])


def test_workload_v3_b32_8k(gpu):
    case = mla_synth.workload("v3_b32_8k")
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(o_dtype="bf16"))
    assert run.status() == 0
    full_check(case, o, TOL_BF16_REL, def_pairs=[(3, 9)])


def test_workload_v3_b4_128k(gpu):
    """Four sequences of 131072 tokens with 1 % of rows scaled x8 (peaked
    softmax rows), split over many work items per sequence."""
    case = mla_synth.workload("v3_b4_128k")
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(o_dtype="bf16"))
    assert run.status() == 0
    full_check(case, o, TOL_BF16_REL, def_pairs=[(2, 100)])


def test_workload_v3_b128_fp8_append_decode(gpu):
    """128 sequences, fp8 e4m3 latents with per-token scales, one token
    appended per sequence from h [128, 7168] before attention (one call).
    The appended rows land at seq_start + L_old exactly, with codes within
    one fp8 step and scales within 1e-5 of the oracle's own append; every
    output is compared end to end."""
    case = mla_synth.workload("v3_b128_fp8")
    run = DeviceRun(gpu, case)
    o = to_np(run.append_decode(o_dtype="bf16"))
    assert run.status() == 0
    assert np.array_equal(run.t["seq_len"].cpu().numpy(), case.lens + 1)
    ap = oracle_append(case)
    rows = ap["rows"].reshape(-1)
    assert np.array_equal(rows, case.seq_start.astype(np.int64) + case.lens)
    from oracle import mla as omla
    got_rows = run.t["rows"][rows].cpu().numpy()
    scale = run.t["scale"][rows].cpu().numpy()
    s_ref = ap["scale"].reshape(-1)
    assert np.allclose(scale, s_ref, rtol=1e-5, atol=0)
    C, R = omla.decode_rows(got_rows, "fp8", "bf16", case.d_c, case.d_rope, scale)
    refC = ap["c"].reshape(len(rows), -1)
    step = np.maximum(np.abs(refC) * 2.0 ** -3, s_ref[:, None].astype(np.float64) * 2.0 ** -9)
    assert np.all(np.abs(C - refC) <= step * 1.0001)
    refR = ap["k_rope"].reshape(len(rows), -1)
    assert np.all(np.abs(R - refR) <= np.abs(refR) * 2.0 ** -7 + 1e-6)
    full_check(case, o, TOL_FP8_REL)
