"""GPU tests of the paged latent cache (block table, blocks of a multiple of
32 rows): decode, several-token decode and append on a shuffled paged copy
of a case give bit-for-bit the results of the contiguous cache (the kernels
see the same rows, only their addresses move), on the matrix-core and the
generic path, and every paged output is also compared with the oracle at
the workloads' tolerances (rms over the whole output); a block id outside
the cache is reported, not followed, and an append into such a block, or
past the cache's rows, leaves the sequence untouched."""
import numpy as np
import pytest
import torch

import mla_synth
from tests.helpers import (DeviceRun, TOL_BF16_REL, TOL_F32_ABS, TOL_FP8_REL, make, max_abs_err, oracle_decode,
                           oracle_decode_multi, oracle_full, paged_layout, rel_rms_err, to_np)


def tol(latent):
    return TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL

pytestmark = pytest.mark.gpu

V3 = dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128)
LENS = [1, 31, 32, 33, 100, 700, 0, 64, 200]


def v3_case(latent, seed, lens=LENS, **kw):
    return make(B=len(lens), lens=("list", lens), latent_dtype=latent, rope_dtype="bf16", act_dtype="bf16",
                seed=seed, **V3, **kw)


@pytest.mark.parametrize("latent,bt", [("bf16", 64), ("fp8", 32), ("bf16", 128)])
def test_paged_decode_matches_contiguous(gpu, latent, bt):
    case = v3_case(latent, 100)
    flat = DeviceRun(gpu, case)
    paged = DeviceRun(gpu, case, paged=paged_layout(case, bt, seed=bt) + (bt,))
    plan = flat.plan(n_workers=20)
    a = flat.decode(plan=plan)
    b = paged.decode(plan=plan)
    assert flat.status() == 0 and paged.status() == 0
    assert torch.equal(a, b)
    assert rel_rms_err(to_np(b), oracle_full(case)) <= tol(latent)


@pytest.mark.parametrize("latent", ["bf16", "fp8"])
def test_paged_multi_token_decode_matches_contiguous(gpu, latent):
    case = v3_case(latent, 101)
    qn, qr = mla_synth.multi_queries(case, 3, seed=4)
    flat = DeviceRun(gpu, case)
    paged = DeviceRun(gpu, case, paged=paged_layout(case, 64, seed=5) + (64,))
    plan = flat.plan(n_workers=16)
    a = flat.decode_multi(3, qn, qr, plan=plan)
    b = paged.decode_multi(3, qn, qr, plan=plan)
    assert flat.status() == 0 and paged.status() == 0
    assert torch.equal(a, b)
    ref = oracle_decode_multi(case, qn, qr, absorbed=True)
    assert rel_rms_err(to_np(b), ref) <= tol(latent)


def test_paged_generic_path_fp32(gpu):
    case = make(B=3, lens=("list", [5, 64, 130]), latent_dtype="f32", rope_dtype="f32", act_dtype="f32", seed=102,
                H=4, d_c=32, d_rope=8, d_nope=16, d_v=16)
    flat = DeviceRun(gpu, case)
    paged = DeviceRun(gpu, case, paged=paged_layout(case, 32, seed=6) + (32,))
    plan = flat.plan(n_workers=5)
    a, b = flat.decode(plan=plan), paged.decode(plan=plan)
    assert flat.status() == 0 and paged.status() == 0
    assert torch.equal(a, b)
    assert max_abs_err(to_np(b), oracle_decode(case)) <= TOL_F32_ABS


@pytest.mark.parametrize("latent", ["bf16", "fp8"])
def test_paged_append_then_decode_matches_contiguous(gpu, latent):
    lens = [3, 40, 63, 64, 500]
    case = make(B=len(lens), lens=("list", lens), latent_dtype=latent, rope_dtype="bf16", act_dtype="bf16",
                seed=103, n_new=1, d_model=1024, extra_cap=30, **V3)
    flat = DeviceRun(gpu, case)
    bt = 32
    layout = paged_layout(case, bt, seed=7)
    paged = DeviceRun(gpu, case, paged=layout + (bt,))
    plan = flat.plan()
    a = flat.append_decode(plan=plan)
    b = paged.append_decode(plan=plan)
    assert flat.status() == 0 and paged.status() == 0
    assert torch.equal(a, b)
    assert rel_rms_err(to_np(b), oracle_full(case)) <= tol(latent)
    # the appended rows sit where the block table maps them, byte for byte
    rows_f = flat.t["rows"].cpu().numpy()
    rows_p = paged.t["rows"].cpu().numpy()
    table = layout[2]
    for bi, L in enumerate(lens):
        t = L  # the new token's position
        src = int(case.seq_start[bi]) + t
        dst = int(table[bi, t // bt]) * bt + t % bt
        np.testing.assert_array_equal(rows_p[dst], rows_f[src])
        if latent == "fp8":
            assert flat.t["scale"][src].item() == paged.t["scale"][dst].item()
    assert np.all(flat.t["seq_len"].cpu().numpy() == np.array(lens) + 1)
    assert np.all(paged.t["seq_len"].cpu().numpy() == np.array(lens) + 1)


def test_paged_bad_block_id_is_reported(gpu):
    case = v3_case("bf16", 104, lens=[100, 300])
    rows, scale, table, = paged_layout(case, 64, seed=8)
    table[1, 2] = 1 << 20  # outside the cache
    paged = DeviceRun(gpu, case, paged=(rows, scale, table, 64))
    paged.decode(n_workers=4)
    assert paged.status() == 6  # MLA_ERR_PLAN


def test_paged_append_into_a_bad_block_leaves_the_sequence_untouched(gpu):
    """The new token of sequence 1 falls in a block whose id is outside the
    cache: that sequence's rows and length stay as they were (MLA_ERR_PLAN),
    the other sequences append."""
    lens = [3, 64, 40]
    case = make(B=len(lens), lens=("list", lens), latent_dtype="bf16", rope_dtype="bf16", act_dtype="bf16",
                seed=105, n_new=1, d_model=1024, extra_cap=30, **V3)
    rows, scale, table = paged_layout(case, 32, seed=9)
    table[1, 64 // 32] = 1 << 20  # the block of sequence 1's token 64
    run = DeviceRun(gpu, case, paged=(rows, scale, table, 32))
    before = run.t["rows"].cpu().numpy().copy()
    run.append()
    assert run.status() == 6  # MLA_ERR_PLAN
    assert run.t["seq_len"].cpu().tolist() == [4, 64, 41]
    after = run.t["rows"].cpu().numpy()
    changed = np.flatnonzero(np.any(after != before, axis=1))
    expect = sorted(int(table[b, L // 32]) * 32 + L % 32 for b, L in ((0, 3), (2, 40)))
    assert changed.tolist() == expect


@pytest.mark.parametrize("path", ["fast", "generic"])
def test_append_past_the_cache_rows_leaves_the_sequence_untouched(gpu, path, monkeypatch):
    """A contiguous sequence whose capacity still has room but whose next row
    lies past the cache's last row (n_rows) is refused: length and rows
    unchanged (MLA_ERR_CAPACITY); the others append. Both append paths."""
    lens = [5, 9]
    case = make(B=2, lens=("list", lens), latent_dtype="bf16", rope_dtype="bf16", act_dtype="bf16", seed=106,
                n_new=1, d_model=1024, extra_cap=8, **V3)
    if path == "generic":
        monkeypatch.setenv("MLA_FORCE_GENERIC", "1")
    run = DeviceRun(gpu, case)
    # the cache as the caller describes it ends right after sequence 1's 9th row
    last = int(case.seq_start[1]) + lens[1]
    run.cache.n_rows = last
    before = run.t["rows"].cpu().numpy().copy()
    run.append()
    assert run.status() == 3  # MLA_ERR_CAPACITY
    assert run.t["seq_len"].cpu().tolist() == [6, 9]
    after = run.t["rows"].cpu().numpy()
    changed = np.flatnonzero(np.any(after != before, axis=1)).tolist()
    assert changed == [int(case.seq_start[0]) + lens[0]]
