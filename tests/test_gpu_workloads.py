"""GPU parity at the workloads' full sizes, through the C ABI, in the launch
configuration the benchmark times (default plan over all CUs, bf16 output).

The oracle cannot afford every output at these sizes, so each test compares
sampled (sequence, head) outputs, computed one by one: mostly with the
oracle's absorbed form (pinned equal to the definition by the CPU tests),
plus a few with the non-absorbed definition itself. The error bound is
max|err| / rms over the sampled reference outputs. Only the sampled
sequences' rows are decoded to fp64, to bound host memory."""
import numpy as np
import pytest

import mla_synth
from tests.helpers import (DeviceRun, TOL_BF16_REL, TOL_FP8_REL, oracle_append, oracle_cache, oracle_decode,
                           rel_rms_err, to_np)

pytestmark = pytest.mark.gpu


def sample_pairs(case, n, seed, nonempty=True):
    rng = np.random.default_rng(seed)
    bs = [b for b in range(case.B) if case.lens[b] + case.n_new > 0] if nonempty else list(range(case.B))
    return [(int(rng.choice(bs)), int(rng.integers(case.H))) for _ in range(n)]


def sampled_check(case, o, pairs, tol, n_def=0):
    seqs = sorted({b for b, _ in pairs})
    C, R = oracle_cache(case, seqs=seqs)
    ref = oracle_decode(case, pairs=pairs, absorbed=True, C=C.copy(), R=R.copy())
    got = np.stack([o[b, i] for b, i in pairs])
    err = rel_rms_err(got, ref)
    assert err <= tol, f"sampled outputs: max|err|/rms {err:.3e} > {tol}"
    if n_def:
        dp = pairs[:n_def]
        ref_def = oracle_decode(case, pairs=dp, absorbed=False, C=C, R=R)
        got_def = np.stack([o[b, i] for b, i in dp])
        # rms of the larger sample: a handful of outputs is too few to estimate it
        rms = float(np.sqrt(np.mean(ref ** 2)))
        err_def = float(np.max(np.abs(got_def - ref_def))) / rms
        assert err_def <= tol, f"sampled outputs vs definition: {err_def:.3e}"
    return err


def test_workload_v3_b1_4k(gpu):
    """One sequence of 4096 tokens, H=128: every output against the absorbed
    oracle, two against the definition."""
    case = mla_synth.workload("v3_b1_4k")
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(o_dtype="bf16"))
    assert run.status() == 0
    ref = oracle_decode(case, absorbed=True)
    assert rel_rms_err(o, ref) <= TOL_BF16_REL
    ref_def = oracle_decode(case, pairs=[(0, 0), (0, 77)])
    assert rel_rms_err(np.stack([o[0, 0], o[0, 77]]), ref_def) <= TOL_BF16_REL


def test_workload_v3_b32_ragged_bench_config(gpu):
    """The benchmark's workload and launch configuration."""
    case = mla_synth.workload("v3_b32_ragged")
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(o_dtype="bf16"))
    assert run.status() == 0
    sampled_check(case, o, sample_pairs(case, 24, seed=1), TOL_BF16_REL, n_def=3)


def test_workload_v3_b32_8k(gpu):
    case = mla_synth.workload("v3_b32_8k")
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(o_dtype="bf16"))
    assert run.status() == 0
    sampled_check(case, o, sample_pairs(case, 12, seed=2), TOL_BF16_REL)


def test_workload_v3_b4_128k(gpu):
    """Four sequences of 131072 tokens with 1 % of rows scaled x8 (peaked
    softmax rows), split over many work items per sequence."""
    case = mla_synth.workload("v3_b4_128k")
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(o_dtype="bf16"))
    assert run.status() == 0
    sampled_check(case, o, sample_pairs(case, 16, seed=3), TOL_BF16_REL)


def test_workload_v3_b128_fp8_append_decode(gpu):
    """128 sequences, fp8 e4m3 latents with per-token scales, one token
    appended per sequence from h [128, 7168] before attention (one call).
    The appended rows land at seq_start + L_old exactly, with codes within
    one fp8 step and scales within 1e-5 of the oracle's own append; the
    sampled outputs are compared end to end."""
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
    sampled_check(case, o, sample_pairs(case, 24, seed=4), TOL_FP8_REL)
