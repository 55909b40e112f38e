"""GPU parity of the matrix-core path (DeepSeek-V3 shape: H=128, d_c=512,
d_hR=64, d_nope=128, d_v=128, bf16 q/weights) against the oracle, through the
C ABI. Ragged and edge-case lengths, bf16 and fp8 latents, fast path versus
the generic kernels, split invariance, determinism, explicit positions."""
import os

import numpy as np
import pytest
import torch

from tests.helpers import (DeviceRun, TOL_BF16_REL, TOL_FP8_REL, make, oracle_append, oracle_decode,
                           rel_rms_err, to_np)

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
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(n_workers=16))
    assert run.status() == 0
    check(case, o, TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL)
    assert np.all(o[EDGE_LENS.index(0)] == 0)


@pytest.mark.parametrize("latent", ["bf16", "fp8"])
def test_fast_matches_generic_path(gpu, latent, monkeypatch):
    case = v3_case([77, 300, 1025], latent, seed=51)
    run = DeviceRun(gpu, case)
    fast = to_np(run.decode(n_workers=8))
    monkeypatch.setenv("MLA_FORCE_GENERIC", "1")
    gen = to_np(run.decode(n_workers=8))
    monkeypatch.delenv("MLA_FORCE_GENERIC")
    # the generic path keeps q~ and P in fp32 (it agrees with the oracle to
    # ~1e-5); the fast one rounds q~, P and the cached values to fp16, so the
    # two differ by the fast path's own rounding error
    tol = TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL
    ref = oracle_decode(case, absorbed=True)
    assert rel_rms_err(gen, ref) <= 1e-4
    assert rel_rms_err(fast, ref) <= tol
    assert rel_rms_err(fast, gen) <= tol


@pytest.mark.parametrize("latent", ["bf16", "fp8"])
def test_ranges_of_many_items(gpu, latent):
    """Three workgroups over nine sequences: each walks several items one
    after the other, ranges begin and end inside sequences, and an empty and
    a one-token sequence sit between them. All outputs against the oracle."""
    lens = [33, 1, 700, 64, 5, 2000, 31, 0, 129]
    case = v3_case(lens, latent, seed=58)
    run = DeviceRun(gpu, case)
    plan = run.plan(n_workers=3)
    ranges = plan.ranges()
    assert len(ranges) == 3 and max(k1 - k0 for k0, k1 in ranges) >= 3
    items = plan.items()
    assert any(items[k0][0] == items[k0 - 1][0] for k0, _ in ranges[1:])  # a sequence split between ranges
    o = to_np(run.decode(plan=plan))
    assert run.status() == 0
    check(case, o, TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL)
    assert np.all(o[lens.index(0)] == 0)


@pytest.mark.parametrize("workers", [16, 5])
def test_fp8_matrix_cores_and_widening_kernel(gpu, monkeypatch, workers):
    """An fp8 cache runs on the fp8 matrix cores by default (e4m3 codes
    straight from the tile, q~ and P as hi + lo e4m3 pairs); MLA_FP8_WIDEN=1
    selects the kernel that widens the codes to fp16 first. Both against the
    oracle over the edge lengths (with ranges of several items at 5
    workers), and against each other, within the bf16 tolerance: the fp8
    products' own error is far inside the fp8 one (the emulation of exactly
    this arithmetic gives 3.2e-3), and the widened codes are exact in fp16."""
    case = v3_case(EDGE_LENS, "fp8", seed=57, gap_rows=2)
    run = DeviceRun(gpu, case)
    o8 = to_np(run.decode(n_workers=workers))
    monkeypatch.setenv("MLA_FP8_WIDEN", "1")
    o16 = to_np(run.decode(n_workers=workers))
    monkeypatch.delenv("MLA_FP8_WIDEN")
    assert run.status() == 0
    ref = oracle_decode(case, absorbed=True)
    e8, e16, e816 = rel_rms_err(o8, ref), rel_rms_err(o16, ref), rel_rms_err(o8, o16)
    print(f"fp8 matrix cores {e8:.2e}, widening kernel {e16:.2e}, between them {e816:.2e}")
    assert max(e8, e16, e816) <= TOL_BF16_REL
    assert np.all(o8[EDGE_LENS.index(0)] == 0) and np.all(o16[EDGE_LENS.index(0)] == 0)


@pytest.mark.parametrize("latent", ["bf16", "fp8"])
def test_fast_256_heads(gpu, latent):
    """Two 128-head blocks per work item (split-K grid of two rows of
    workgroups), and a head count the combine kernel maps across XCDs in
    two rounds."""
    lens = [45, 300, 0, 97, 1024]
    case = make(B=len(lens), lens=("list", lens), latent_dtype=latent, rope_dtype="bf16", act_dtype="bf16",
                seed=70, H=256, d_c=512, d_rope=64, d_nope=128, d_v=128)
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(n_workers=12))
    assert run.status() == 0
    check(case, o, TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL)
    assert np.all(o[2] == 0)


@pytest.mark.parametrize("B,max_len,splits", [(1, 400, 4), (1, 6000, 300), (3, 400, 4), (8, 400, 4),
                                               (12, 400, 4), (20, 400, 4), (20, 1200, 24)])
def test_fast_combine_group_sizes(gpu, B, max_len, splits):
    """The combine kernel groups 1, 2, 4, 8 or 16 sequences per workgroup
    (by batch size); every grouping, with a partial last group, and more
    splits per sequence than one batch of row loads holds (B = 1 with 182
    splits, 128 a batch; B = 20 with up to 18, 12 a batch)."""
    rng = np.random.default_rng(1000 + B + max_len)
    lens = [int(x) for x in rng.integers(max_len // 2 if max_len > 1000 else 1, max_len, size=B)]
    case = v3_case(lens, seed=60 + B)
    run = DeviceRun(gpu, case)
    o = to_np(run.decode(n_workers=splits * B + 3))
    assert run.status() == 0
    check(case, o, TOL_BF16_REL)


def test_fast_split_invariance_and_determinism(gpu):
    case = v3_case([2000, 513], seed=52)
    run = DeviceRun(gpu, case)
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
    run = DeviceRun(gpu, case)
    q_pos = np.array([5000, 3], dtype=np.int32)
    o = to_np(run.decode(q_pos=torch.from_numpy(q_pos).cuda(), o_dtype="bf16"))
    ref = oracle_decode(case, absorbed=True, q_pos=q_pos)
    assert rel_rms_err(o, ref) <= TOL_BF16_REL


def test_fast_plan_mismatch(gpu):
    case = v3_case([64, 40], seed=54)
    run = DeviceRun(gpu, case)
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
    run = DeviceRun(gpu, case)
    o = to_np(run.decode())
    check(case, o, TOL_BF16_REL)


@pytest.mark.parametrize("latent", ["f32", "bf16", "fp8"])
def test_fast_append_rows_and_canary(gpu, latent, monkeypatch):
    """The matrix-core append (bf16 h and weights, d_model a multiple of
    512): rows land exactly at seq_start + seq_len + j (one sequence at a
    position near 70000), every other byte stays as it was, values and fp8
    scales match the oracle's own append within one storage step, and the
    result equals the generic append's up to that rounding."""
    rope = "f32" if latent == "f32" else "bf16"
    case = make(B=5, lens=("list", [3, 0, 70001, 40, 31]), n_new=3, d_model=1024, extra_cap=1, gap_rows=2,
                latent_dtype=latent, rope_dtype=rope, act_dtype="bf16", seed=56, **V3)
    run = DeviceRun(gpu, case)
    valid = np.zeros(case.n_rows, dtype=bool)
    for b in range(case.B):
        valid[case.seq_start[b]:case.seq_start[b] + case.lens[b]] = True
    vmask = torch.from_numpy(valid).to(run.t["rows"].device)
    run.t["rows"].copy_(torch.where(vmask[:, None], run.t["rows"], torch.full_like(run.t["rows"], 0xA5)))
    before = run.t["rows"].cpu().numpy().copy()
    if run.t["scale"] is not None:
        run.t["scale"].fill_(-7.0)
    run.append()
    assert run.status() == 0
    after = run.t["rows"].cpu().numpy()
    assert np.array_equal(run.t["seq_len"].cpu().numpy(), case.lens + 3)
    ap = oracle_append(case)
    rows = ap["rows"].reshape(-1)
    written = np.zeros(case.n_rows, dtype=bool)
    written[rows] = True
    for b in range(case.B):
        r0 = case.seq_start[b] + case.lens[b]
        assert np.all(written[r0:r0 + 3])
    assert np.array_equal(after[~written], before[~written])
    from oracle import mla as omla
    scale = run.t["scale"].cpu().numpy() if run.t["scale"] is not None else None
    C, R = omla.decode_rows(after[rows], latent, rope, case.d_c, case.d_rope, None if scale is None else scale[rows])
    refC = ap["c"].reshape(len(rows), -1)
    refR = ap["k_rope"].reshape(len(rows), -1)
    if latent == "fp8":
        s_ref = ap["scale"].reshape(-1)
        assert np.allclose(scale[rows], s_ref, rtol=1e-5, atol=0)
        step = np.maximum(np.abs(refC) * 2.0 ** -3, s_ref[:, None].astype(np.float64) * 2.0 ** -9)
        assert np.all(np.abs(C - refC) <= step * 1.0001)
        untouched = np.ones(case.n_rows, dtype=bool)
        untouched[rows] = False
        assert np.all(scale[untouched] == -7.0)
    elif latent == "bf16":
        assert np.all(np.abs(C - refC) <= np.abs(refC) * 2.0 ** -7 + 1e-30)
    else:
        assert np.max(np.abs(C - refC)) <= 1e-5 * np.max(np.abs(refC))
    tol_r = 2.0 ** -7 if rope == "bf16" else 1e-5
    assert np.all(np.abs(R - refR) <= np.abs(refR) * tol_r + 1e-6)
    # the generic append of the same tokens agrees within the same rounding
    run2 = DeviceRun(gpu, case)
    monkeypatch.setenv("MLA_FORCE_GENERIC", "1")
    run2.append()
    monkeypatch.delenv("MLA_FORCE_GENERIC")
    assert run2.status() == 0
    C2, R2 = omla.decode_rows(run2.t["rows"].cpu().numpy()[rows], latent, rope, case.d_c, case.d_rope,
                              None if scale is None else run2.t["scale"].cpu().numpy()[rows])
    assert np.max(np.abs(C2 - C)) <= np.max(np.abs(refC)) * (2.0 ** -3 if latent == "fp8" else 2.0 ** -7)


def test_plan_copy_reuse_and_invalidation(gpu):
    """A workspace keeps the device copy of the last plan it ran, so a second
    decode with the same plan skips the upload. An append through the same
    workspace overwrites that copy and must force the next decode to upload
    the plan again: decode cache A, append into cache B with the shared
    workspace, decode A again with the same plan -> identical outputs."""
    case_a = v3_case([300, 77, 1025], seed=57)
    case_b = make(B=2, lens=("list", [5, 9]), n_new=2, d_model=512, latent_dtype="bf16", rope_dtype="bf16",
                  act_dtype="bf16", seed=58, **V3)
    run_a = DeviceRun(gpu, case_a)
    run_b = DeviceRun(gpu, case_b)
    plan_a = run_a.plan(n_workers=8)
    o1 = to_np(run_a.decode(plan=plan_a))
    o2 = to_np(run_a.decode(plan=plan_a))
    assert np.array_equal(o1, o2)
    need = max(run_a.ws.numel(), gpu.mla_append_workspace_bytes(run_b.d, case_b.B, case_b.n_new))
    if run_a.ws.numel() < need:
        run_a.ws = torch.empty(need, dtype=torch.uint8, device=run_a.ws.device)
        gpu.mla_workspace_init(run_a.ws)
        o1 = to_np(run_a.decode(plan=plan_a))
    run_b.ws = run_a.ws
    run_b.append()
    assert run_b.status() == 0
    o3 = to_np(run_a.decode(plan=plan_a))
    assert np.array_equal(o1, o3)
    check(case_a, o3, TOL_BF16_REL)


def test_streams_and_separate_workspaces(gpu):
    """Calls run on the stream they are given; two decodes with their own
    workspaces on two streams at once give the default-stream result."""
    case = v3_case([300, 1500, 64, 999], seed=57)
    run = DeviceRun(gpu, case)
    plan = run.plan(n_workers=12)
    ref = run.decode(plan=plan).clone()
    assert run.status() == 0
    m, t, c = gpu, run.t, case
    need = m.mla_decode_workspace_bytes(run.d, plan)
    outs, wss, streams = [], [], [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        m.mla_workspace_init(ws)
        wss.append(ws)
        outs.append(torch.empty((c.B, c.H, c.d_v), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    for rep in range(3):
        for s, ws, o in zip(streams, wss, outs):
            with torch.cuda.stream(s):
                m.mla_decode(run.d, run.cache, plan, t["q_nope"], t["q_rope"], None, t["w_uk"], t["w_uv"],
                             1, o, 0, ws, stream=s.cuda_stream)
        torch.cuda.synchronize()
        for ws, o in zip(wss, outs):
            assert m.mla_device_error(ws, reset=True) == 0
            assert torch.equal(o, ref)


@pytest.mark.parametrize("latent", ["bf16", "fp8"])
def test_fast_many_groups_per_workgroup(gpu, latent):
    """70 sequences: the combine deals a head's 5 groups of 16 sequences (the
    last of 6) to its 2 workgroups, 3 and 2 groups each, which keep their
    W_UV rows across them; each absorb workgroup runs its weight quarter over
    3 blocks of 32 sequences (the last of 6) one after the other."""
    rng = np.random.default_rng(1070)
    lens = [int(x) for x in rng.integers(1, 600, size=70)]
    case = v3_case(lens, latent, seed=61)
    run = DeviceRun(gpu, case)
    o = to_np(run.decode())
    assert run.status() == 0
    check(case, o, TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL)


@pytest.mark.parametrize("seed", [0, 1, 2, 3, 4])
def test_fast_random_shapes(gpu, seed):
    """Seeded random batches: 1-12 sequences of 0-3000 tokens, a random worker
    count for the plan, bf16 or fp8 latents, fp32 or bf16 output."""
    rng = np.random.default_rng(500 + seed)
    B = int(rng.integers(1, 13))
    lens = [int(x) for x in rng.integers(0, 3000, size=B)]
    lens[int(rng.integers(B))] = max(lens) + 1  # at least one non-empty sequence
    latent = "fp8" if rng.random() < 0.4 else "bf16"
    case = v3_case(lens, latent, seed=600 + seed)
    run = DeviceRun(gpu, case)
    workers = int(rng.integers(1, 400))
    o_dtype = "bf16" if rng.random() < 0.3 else "f32"
    o = run.decode(n_workers=workers, o_dtype=o_dtype)
    assert run.status() == 0
    tol = TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL
    if o_dtype == "bf16":
        o32 = run.decode(n_workers=workers)
        assert torch.equal(o, o32.to(torch.bfloat16))
        o = o32
    check(case, to_np(o), tol, seed=seed)


def test_tensor_level_calls_match_the_abi(gpu):
    """decode() / append_decode() read the dtypes off the tensors and allocate
    the output and workspace; the results are the entry points' bit for bit."""
    bf = lambda t: t.view(torch.bfloat16)  # noqa: E731  (bf16 bit patterns on the device)
    case = v3_case([77, 300, 1025], "bf16", seed=58)
    run = DeviceRun(gpu, case)
    plan = run.plan()
    ref = run.decode(plan=plan)
    got = gpu.decode(run.d, run.cache, plan, bf(run.t["q_nope"]), bf(run.t["q_rope"]), bf(run.t["w_uk"]),
                     bf(run.t["w_uv"]))
    out16 = gpu.decode(run.d, run.cache, plan, bf(run.t["q_nope"]), bf(run.t["q_rope"]), bf(run.t["w_uk"]),
                       bf(run.t["w_uv"]), out=torch.empty((case.B, case.H, case.d_v), dtype=torch.bfloat16,
                                                          device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(out16, ref.to(torch.bfloat16))

    case = v3_case([40, 700], "fp8", seed=59, n_new=1, d_model=7168)
    a, b = DeviceRun(gpu, case), DeviceRun(gpu, case)
    ref = a.append_decode()
    plan = b.plan()
    got = gpu.append_decode(b.d, b.cache, plan, bf(b.t["h"]), bf(b.t["w_dkv"]), bf(b.t["w_kr"]),
                            bf(b.t["q_nope"]), bf(b.t["q_rope"]), bf(b.t["w_uk"]), bf(b.t["w_uv"]),
                            ws=b.workspace(plan))  # a workspace of our own, to read its status word
    torch.cuda.synchronize()
    assert a.status() == 0 and b.status() == 0
    assert torch.equal(got, ref)
    with pytest.raises(ValueError):
        gpu.decode(b.d, b.cache, plan, b.t["q_nope"], b.t["q_rope"], b.t["w_uk"], b.t["w_uv"])  # int16 bits


@pytest.mark.parametrize("generic", [False, True])
def test_default_softmax_scale_is_the_library_default(gpu, generic, monkeypatch):
    """softmax_scale 0 in mla_dims (what dims() passes when none is given)
    decodes bit for bit like an explicit (d_nope + d_rope)^-1/2, computed in
    double and rounded once to float, on both paths."""
    case = v3_case([77, 300, 1025], seed=57)
    run = DeviceRun(gpu, case)
    if generic:
        monkeypatch.setenv("MLA_FORCE_GENERIC", "1")
    explicit = float(np.float32(1.0 / np.sqrt(np.float64(case.d_nope + case.d_rope))))
    run.d = gpu.dims(case.H, case.d_c, case.d_rope, case.d_nope, case.d_v, case.d_model, explicit, case.rope_base)
    o1 = run.decode(n_workers=8)
    run.d = gpu.dims(case.H, case.d_c, case.d_rope, case.d_nope, case.d_v, case.d_model, None, case.rope_base)
    assert run.d.softmax_scale == 0.0
    o2 = run.decode(n_workers=8)
    assert run.status() == 0
    assert torch.equal(o1, o2)
