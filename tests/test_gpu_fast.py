"""GPU parity of the matrix-core path (DeepSeek-V3 shape: H=128, d_c=512,
d_hR=64, d_nope=128, d_v=128, bf16 q/weights) against the oracle, through the
C ABI. Ragged and edge-case lengths, bf16 and fp8 latents, fast path versus
the generic kernels, split invariance, determinism, explicit positions."""
import os

import numpy as np
import pytest
import torch

from tests.helpers import (GpuRun, TOL_BF16_REL, TOL_FP8_REL, make, oracle_decode, rel_rms_err,
                           to_np)

pytestmark = pytest.mark.gpu

V3 = dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128)
EDGE_LENS = [1, 31, 32, 33, 100, 700, 0, 64]


def v3_case(lens, latent="bf16", seed=50, **kw):
    return make(B=len(lens), lens=("list", lens), latent_dtype=latent, rope_dtype="bf16",
                act_dtype="bf16", seed=seed, **V3, **kw)


def check(case, o, tol, n_def=6, seed=0):
    """All outputs against the oracle's absorbed form (pinned equal to the
    definition), plus sampled (b, head) pairs against the non-absorbed
    definition itself."""
    ref = oracle_decode(case, absorbed=True)
    err = rel_rms_err(o, ref)
    assert err <= tol, f"all outputs: max|err|/rms {err:.3e} > {tol}"
    rng = np.random.default_rng(seed)
    nz = [b for b in range(case.B) if case.lens[b] + case.n_new > 0]
    pairs = [(int(rng.choice(nz)), int(rng.integers(case.H))) for _ in range(n_def)]
    ref_def = oracle_decode(case, pairs=pairs)
    got = np.stack([o[b, i] for b, i in pairs])
    err_def = rel_rms_err(got, ref_def)
    assert err_def <= tol, f"sampled pairs vs definition: {err_def:.3e}"
    return err


@pytest.mark.parametrize("latent", ["bf16", "fp8"])
def test_fast_decode_edge_lengths(gpu, latent):
    case = v3_case(EDGE_LENS, latent, gap_rows=2)
    run = GpuRun(gpu, case)
    o = to_np(run.decode(n_workers=16))
    assert run.status() == 0
    check(case, o, TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL)
    assert np.all(o[EDGE_LENS.index(0)] == 0)


@pytest.mark.parametrize("latent", ["bf16", "fp8"])
def test_fast_matches_generic_path(gpu, latent, monkeypatch):
    case = v3_case([77, 300, 1025], latent, seed=51)
    run = GpuRun(gpu, case)
    fast = to_np(run.decode(n_workers=8))
    monkeypatch.setenv("MLA_FORCE_GENERIC", "1")
    gen = to_np(run.decode(n_workers=8))
    monkeypatch.delenv("MLA_FORCE_GENERIC")
    # the generic path keeps q~ and P in fp32 (it agrees with the oracle to
    # ~1e-5); the fast one rounds q~ to fp16 and P to bf16, so the two differ
    # by the fast path's own rounding error
    tol = TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL
    ref = oracle_decode(case, absorbed=True)
    assert rel_rms_err(gen, ref) <= 1e-4
    assert rel_rms_err(fast, ref) <= tol
    assert rel_rms_err(fast, gen) <= tol


def test_fast_split_invariance_and_determinism(gpu):
    case = v3_case([2000, 513], seed=52)
    run = GpuRun(gpu, case)
    p1 = run.plan(n_workers=1)
    p64 = run.plan(n_workers=64)
    o1 = to_np(run.decode(plan=p1))
    o64 = to_np(run.decode(plan=p64))
    o64b = to_np(run.decode(plan=p64))
    assert np.array_equal(o64, o64b), "not bitwise reproducible"
    # different splits round P (bf16) relative to different running maxima
    check(case, o64, TOL_BF16_REL)
    check(case, o1, TOL_BF16_REL)
    assert rel_rms_err(o64, o1) <= TOL_BF16_REL


def test_fast_explicit_positions_and_bf16_output(gpu):
    case = v3_case([90, 257], seed=53)
    run = GpuRun(gpu, case)
    q_pos = np.array([5000, 3], dtype=np.int32)
    o = to_np(run.decode(q_pos=torch.from_numpy(q_pos).cuda(), o_dtype="bf16"))
    ref = oracle_decode(case, absorbed=True, q_pos=q_pos)
    assert rel_rms_err(o, ref) <= TOL_BF16_REL


def test_fast_plan_mismatch(gpu):
    case = v3_case([64, 40], seed=54)
    run = GpuRun(gpu, case)
    plan = run.plan(lens=[64, 41])
    o = to_np(run.decode(plan=plan))
    assert run.status() == 6
    assert np.all(o[1] == 0)
    ref = oracle_decode(case, absorbed=True)
    assert rel_rms_err(o[0], ref[0]) <= TOL_BF16_REL


def test_fast_spiky_rows(gpu):
    """A few rows scaled x8 give peaked softmax rows (the long-context
    workload's structure at a small size)."""
    case = v3_case([3000, 1500], seed=55, spike_frac=0.01, spike_mult=8.0)
    run = GpuRun(gpu, case)
    o = to_np(run.decode())
    check(case, o, TOL_BF16_REL)
