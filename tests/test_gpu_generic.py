"""GPU parity of the generic (fp32 VALU) path and of the boundary's host and
device error handling, against the oracle. Calls go through the C ABI."""
import numpy as np
import pytest
import torch

import mla_synth
from tests.helpers import (DeviceRun, TOL_BF16_REL, TOL_F32_ABS, TOL_FP8_REL, max_abs_err, make,
                           oracle_append, oracle_decode, rel_rms_err, to_np)

pytestmark = pytest.mark.gpu


def test_tiny_f32_append_then_decode(gpu):
    """The tiny fp32 workload: 64 tokens appended from h (positions 0..63),
    then one decode step with q = W_Q h_63."""
    case = mla_synth.workload("tiny_f32")
    run = DeviceRun(gpu, case)
    run.append()
    assert run.status() == 0
    assert run.t["seq_len"].cpu().tolist() == [64]
    ap = oracle_append(case)
    rows = run.t["rows"].cpu().numpy()
    got = rows[:64, :case.d_c * 4].copy().view(np.float32).astype(np.float64)
    ref = ap["c"][0]
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
    got_r = rows[:64, case.d_c * 4:case.d_c * 4 + case.d_rope * 4].copy().view(np.float32)
    assert np.max(np.abs(got_r - ap["k_rope"][0])) <= 1e-5 * np.max(np.abs(ap["k_rope"][0]))
    o = to_np(run.decode())
    ref_o = oracle_decode(case)
    assert max_abs_err(o, ref_o) <= TOL_F32_ABS


@pytest.mark.parametrize("latent", ["f32", "bf16", "fp8"])
def test_append_indexing_canary(gpu, latent):
    """Rows land exactly at seq_start + seq_len + j; every other byte of the
    cache is left as it was; seq_len rises by n_new."""
    rope = "f32" if latent == "f32" else "bf16"
    case = make(H=2, d_c=32, d_rope=8, d_nope=16, d_v=16, d_model=48, B=3,
                lens=("list", [3, 0, 5]), n_new=4, extra_cap=2, gap_rows=3,
                latent_dtype=latent, rope_dtype=rope, act_dtype="f32", seed=40)
    run = DeviceRun(gpu, case)
    canary = torch.full_like(run.t["rows"], 0xA5)
    # keep the pre-existing valid rows, canary everywhere else
    valid = np.zeros(case.n_rows, dtype=bool)
    for b in range(case.B):
        valid[case.seq_start[b]:case.seq_start[b] + case.lens[b]] = True
    vmask = torch.from_numpy(valid).to(canary.device)
    run.t["rows"].copy_(torch.where(vmask[:, None], run.t["rows"], canary))
    before = run.t["rows"].cpu().numpy().copy()
    if run.t["scale"] is not None:
        run.t["scale"].fill_(-7.0)
    run.append()
    assert run.status() == 0
    after = run.t["rows"].cpu().numpy()
    written = np.zeros(case.n_rows, dtype=bool)
    for b in range(case.B):
        r0 = case.seq_start[b] + case.lens[b]
        written[r0:r0 + case.n_new] = True
    assert np.array_equal(after[~written], before[~written])
    assert run.t["seq_len"].cpu().tolist() == [7, 4, 9]
    ap = oracle_append(case)
    rows = ap["rows"].reshape(-1)
    assert np.array_equal(np.sort(rows), np.nonzero(written)[0])
    from oracle import mla as omla
    scale = run.t["scale"].cpu().numpy() if run.t["scale"] is not None else None
    C, R = omla.decode_rows(after[rows], latent, rope, case.d_c, case.d_rope,
                            None if scale is None else scale[rows])
    refC = ap["c"].reshape(len(rows), -1)
    refR = ap["k_rope"].reshape(len(rows), -1)
    if latent == "fp8":
        s_ref = ap["scale"].reshape(-1)
        assert np.allclose(scale[rows], s_ref, rtol=1e-5, atol=0)
        # one fp8 step: 2^-3 relative for normals, plus the subnormal step
        step = np.maximum(np.abs(refC) * 2.0 ** -3, s_ref[:, None].astype(np.float64) * 2.0 ** -9)
        assert np.all(np.abs(C - refC) <= step * 1.0001)
    elif latent == "bf16":
        assert np.all(np.abs(C - refC) <= np.abs(refC) * 2.0 ** -7 + 1e-30)
    else:
        assert np.max(np.abs(C - refC)) <= 1e-5 * np.max(np.abs(refC))
    tol_r = 2.0 ** -7 if rope == "bf16" else 1e-5
    assert np.all(np.abs(R - refR) <= np.abs(refR) * tol_r + 1e-6)
    if scale is not None:
        untouched = np.ones(case.n_rows, dtype=bool)
        untouched[rows] = False
        assert np.all(scale[untouched] == -7.0)


def test_append_past_capacity_is_refused(gpu):
    case = make(H=2, d_c=32, d_rope=8, d_nope=16, d_v=16, d_model=32, B=2,
                lens=("list", [5, 2]), n_new=3, latent_dtype="bf16", rope_dtype="bf16",
                act_dtype="f32", seed=41)
    run = DeviceRun(gpu, case)
    # shrink sequence 0's capacity so the append does not fit
    cap = case.seq_cap.copy()
    cap[0] = 6
    run.t["seq_cap"].copy_(torch.from_numpy(cap).to(run.t["seq_cap"].device))
    before = run.t["rows"].cpu().numpy().copy()
    run.append()
    assert run.status() == 3  # MLA_ERR_CAPACITY
    after = run.t["rows"].cpu().numpy()
    s0 = case.seq_start[0]
    assert np.array_equal(after[s0:s0 + cap[0]], before[s0:s0 + cap[0]])
    assert run.t["seq_len"].cpu().tolist() == [5, 5]  # sequence 1 appended, 0 untouched


@pytest.mark.parametrize("latent", ["f32", "bf16", "fp8"])
def test_generic_decode_ragged(gpu, latent):
    rope = "f32" if latent == "f32" else "bf16"
    act = "f32" if latent == "f32" else "bf16"
    case = make(H=4, d_c=48, d_rope=8, d_nope=16, d_v=24, B=6,
                lens=("list", [1, 31, 32, 33, 300, 0]), gap_rows=1,
                latent_dtype=latent, rope_dtype=rope, act_dtype=act, seed=42)
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(n_workers=16))
    assert run.status() == 0
    ref = oracle_decode(case)
    if latent == "f32":
        assert max_abs_err(o, ref) <= TOL_F32_ABS
    else:
        tol = TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL
        assert rel_rms_err(o, ref) <= tol
    assert np.all(o[5] == 0)  # empty sequence


def test_split_invariance_and_determinism(gpu):
    case = make(H=4, d_c=32, d_rope=8, d_nope=16, d_v=16, B=3, lens=("list", [700, 65, 1]),
                latent_dtype="f32", rope_dtype="f32", act_dtype="f32", seed=43)
    run = DeviceRun(gpu, case)
    p1 = run.plan(n_workers=1)
    p64 = run.plan(n_workers=64)
    assert p1.n_items == 3 and p64.n_items > 3
    o1 = to_np(run.decode(plan=p1))
    o64 = to_np(run.decode(plan=p64))
    o64b = to_np(run.decode(plan=p64))
    assert np.array_equal(o64, o64b)
    assert rel_rms_err(o64, o1) <= 1e-5
    assert max_abs_err(o64, oracle_decode(case)) <= TOL_F32_ABS


def test_explicit_query_positions(gpu):
    case = make(H=2, d_c=32, d_rope=8, d_nope=16, d_v=16, B=2, lens=("list", [40, 9]),
                latent_dtype="f32", rope_dtype="f32", act_dtype="f32", seed=44)
    run = DeviceRun(gpu, case)
    q_pos = np.array([1000, 3], dtype=np.int32)
    o = to_np(run.decode(q_pos=torch.from_numpy(q_pos).cuda()))
    assert max_abs_err(o, oracle_decode(case, q_pos=q_pos)) <= TOL_F32_ABS


def test_plan_mismatch_is_reported_and_zeroed(gpu):
    case = make(H=2, d_c=32, d_rope=8, d_nope=16, d_v=16, B=2, lens=("list", [40, 9]),
                latent_dtype="f32", rope_dtype="f32", act_dtype="f32", seed=45)
    run = DeviceRun(gpu, case)
    plan = run.plan(lens=[40, 10])  # the device says 9
    o = to_np(run.decode(plan=plan))
    assert run.status() == 6  # MLA_ERR_PLAN
    assert np.all(o[1] == 0)
    assert max_abs_err(o[0], oracle_decode(case)[0]) <= TOL_F32_ABS


def test_host_validation_before_any_launch(gpu):
    case = make(H=2, d_c=32, d_rope=8, d_nope=16, d_v=16, B=1, lens=("list", [4]),
                latent_dtype="f32", rope_dtype="f32", act_dtype="f32", seed=46)
    run = DeviceRun(gpu, case)
    plan = run.plan()
    ws = run.workspace(plan)
    o = torch.empty((1, 2, 16), device="cuda")
    small = ws[:256]
    with pytest.raises(gpu.MLAError) as e:
        gpu.mla_decode(run.d, run.cache, plan, run.t["q_nope"], run.t["q_rope"], None,
                       run.t["w_uk"], run.t["w_uv"], 0, o, 0, small)
    assert e.value.status == 5  # MLA_ERR_WORKSPACE
    with pytest.raises(gpu.MLAError) as e:
        gpu.mla_decode(run.d, run.cache, plan, run.t["q_nope"], run.t["q_rope"], None,
                       run.t["w_uk"], run.t["w_uv"], 7, o, 0, ws)
    assert e.value.status == 1


@pytest.mark.parametrize("n_bytes", [16, 4096 + 48, (1 << 20) + 16 * 7])
def test_calib_read_folds_every_word(gpu, n_bytes):
    """The stream-read ceiling kernel reads every word exactly once: its XOR
    of the buffer equals the host's (sizes below, at and past the grid's
    unrolled stride), and a second call restores the sink."""
    import compressed_kv_cache_absorbed_amd as m
    rng = np.random.default_rng(n_bytes)
    host = rng.integers(0, 2**32, size=n_bytes // 4, dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32).copy()).to("cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    m.mla_calib_read(src, n_bytes, sink)
    torch.cuda.synchronize()
    want = int(np.bitwise_xor.reduce(host))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == want
    m.mla_calib_read(src, n_bytes, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu()[0]) == 0
