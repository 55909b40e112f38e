"""GPU test of mla_decode_noalloc, the decode for callers that cannot
allocate: through the C ABI it gives mla_decode's output bit for bit (same
kernels; its workspace is the library's own per-GPU array), on two calls in
a row where the second is smaller, and that output meets the oracle's
tolerance; the device status word is cleared per call and reported; a plan
too large for the array is refused before any launch."""
import pytest
import torch

from tests.helpers import (DT, DeviceRun, TOL_BF16_REL, TOL_F32_ABS, TOL_FP8_REL, make, max_abs_err, oracle_full,
                           rel_rms_err, to_np)

pytestmark = pytest.mark.gpu

V3 = dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128)


def noalloc(gpu, run, plan, o_dtype="f32", q_pos=None):
    c = run.case
    o = torch.empty((c.B, c.H, c.d_v), dtype=torch.float32 if o_dtype == "f32" else torch.bfloat16,
                    device=run.t["rows"].device)
    st = torch.full((1,), -1, dtype=torch.int32, device=o.device)
    gpu.mla_decode_noalloc(run.d, run.cache, plan, run.t["q_nope"], run.t["q_rope"], q_pos, run.t["w_uk"],
                           run.t["w_uv"], DT[c.act_dtype], o, DT[o_dtype], dev_status=st)
    return o, st


@pytest.mark.parametrize("latent", ["bf16", "fp8"])
def test_noalloc_matches_decode_two_calls_second_smaller(gpu, latent):
    tol = TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL
    big = make(B=12, lens=("list", [3000, 1, 64, 700, 0, 4096, 33, 2500, 128, 31, 900, 5000]), latent_dtype=latent,
               rope_dtype="bf16", act_dtype="bf16", seed=120, **V3)
    small = make(B=3, lens=("list", [40, 1, 300]), latent_dtype=latent, rope_dtype="bf16", act_dtype="bf16",
                 seed=121, **V3)
    outs = []
    for case in (big, small):
        run = DeviceRun(gpu, case)
        plan = run.plan()
        # fp32 output: the batch mixes one-token sequences (|o| ~ 1) with
        # long ones (|o| ~ 0.03), so rounding to bf16 alone would cost about
        # 2 % of the whole-output rms; the bound measures the arithmetic
        ref = run.decode(plan=plan)
        assert run.status() == 0
        got, st = noalloc(gpu, run, plan)
        torch.cuda.synchronize()
        assert st.item() == 0
        assert torch.equal(got, ref)
        assert rel_rms_err(to_np(got), oracle_full(case)) <= tol
        outs.append(got)
    assert outs[0].shape[0] == 12 and outs[1].shape[0] == 3
    # bf16 output: the same bits as mla_decode's
    run = DeviceRun(gpu, small)
    plan = run.plan()
    ref = run.decode(plan=plan, o_dtype="bf16")
    got, st = noalloc(gpu, run, plan, o_dtype="bf16")
    torch.cuda.synchronize()
    assert st.item() == 0 and torch.equal(got, ref)


def test_noalloc_generic_path_fp32(gpu):
    case = make(B=3, lens=("list", [5, 64, 130]), latent_dtype="f32", rope_dtype="f32", act_dtype="f32", seed=122,
                H=4, d_c=32, d_rope=8, d_nope=16, d_v=16)
    run = DeviceRun(gpu, case)
    plan = run.plan(n_workers=7)
    ref = run.decode(plan=plan)
    got, st = noalloc(gpu, run, plan)
    torch.cuda.synchronize()
    assert st.item() == 0
    assert torch.equal(got, ref)
    assert max_abs_err(to_np(got), oracle_full(case)) <= TOL_F32_ABS


def test_noalloc_status_cleared_per_call_and_oversize_refused(gpu):
    case = make(B=2, lens=("list", [100, 50]), latent_dtype="bf16", rope_dtype="bf16", act_dtype="bf16", seed=123,
                **V3)
    run = DeviceRun(gpu, case)
    wrong = run.plan(lens=[100, 51])  # a plan for other lengths: MLA_ERR_PLAN
    _, st = noalloc(gpu, run, wrong)
    torch.cuda.synchronize()
    assert st.item() == 6
    good = run.plan()
    got, st = noalloc(gpu, run, good)
    torch.cuda.synchronize()
    assert st.item() == 0
    assert rel_rms_err(to_np(got), oracle_full(case)) <= TOL_BF16_REL
    # 600 work items of 128 heads: 600 x 128 KB of partials pass the array
    big = run.plan(lens=[100000, 100000], n_workers=600)
    with pytest.raises(gpu.MLAError) as e:
        noalloc(gpu, run, big)
    assert e.value.status == 5  # MLA_ERR_WORKSPACE
