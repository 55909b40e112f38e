"""GPU parity of the several-token decode (mla_decode_multi: q_len new query
tokens per sequence, causal among them) against the oracle, through the C
ABI: ragged and edge lengths (shorter than q_len included), bf16 and fp8
latents, q_len 1 equal to mla_decode bit for bit, explicit positions, a
longer ragged batch on sampled outputs."""
import numpy as np
import pytest
import torch

import mla_synth
from tests.helpers import (DeviceRun, TOL_BF16_REL, TOL_FP8_REL, make, oracle_decode_multi, rel_rms_err, to_np)

pytestmark = pytest.mark.gpu

V3 = dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128)


def v3_case(lens, latent="bf16", seed=80):
    return make(B=len(lens), lens=("list", lens), latent_dtype=latent, rope_dtype="bf16", act_dtype="bf16",
                seed=seed, **V3)


@pytest.mark.parametrize("latent,q_len", [("bf16", 2), ("bf16", 4), ("fp8", 3), ("bf16", 16)])
def test_multi_edge_lengths(gpu, latent, q_len):
    lens = [1, 2, 3, 31, 33, 100, 700, 0, 64, 15]
    case = v3_case(lens, latent)
    qn, qr = mla_synth.multi_queries(case, q_len, seed=90 + q_len)
    run = DeviceRun(gpu, case)
    o = to_np(run.decode_multi(q_len, qn, qr, n_workers=24))
    assert run.status() == 0
    ref = oracle_decode_multi(case, qn, qr)
    tol = TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL
    err = rel_rms_err(o, ref)
    assert err <= tol, f"max|err|/rms {err:.3e}"
    # queries that see no row (a sequence shorter than the tokens after them) give exactly 0
    for b, L in enumerate(lens):
        for j in range(q_len):
            if L - (q_len - 1 - j) <= 0:
                assert np.all(o[b, j] == 0), (b, j)
    # sampled outputs against the non-absorbed definition itself
    rng = np.random.default_rng(q_len)
    tri = [(int(rng.integers(len(lens))), int(rng.integers(q_len)), int(rng.integers(128))) for _ in range(8)]
    tri = [t for t in tri if lens[t[0]] - (q_len - 1 - t[1]) > 0]
    got = np.stack([o[b, j, i] for b, j, i in tri])
    assert rel_rms_err(got, oracle_decode_multi(case, qn, qr, triples=tri, absorbed=False)) <= tol


def test_multi_one_token_is_decode(gpu):
    case = v3_case([5, 300, 77, 1025], seed=81)
    qn, qr = mla_synth.multi_queries(case, 1, seed=1)
    run = DeviceRun(gpu, case)
    plan = run.plan(n_workers=9)
    single = to_np(run.decode(plan=plan))
    multi = to_np(run.decode_multi(1, qn, qr, plan=plan))
    assert run.status() == 0
    np.testing.assert_array_equal(multi[:, 0], single)


def test_multi_explicit_positions_bf16_output(gpu):
    lens = [40, 300, 9]
    case = v3_case(lens, seed=82)
    q_len = 4
    qn, qr = mla_synth.multi_queries(case, q_len, seed=3)
    run = DeviceRun(gpu, case)
    pos = torch.from_numpy(np.array([1000, 7, 3], dtype=np.int32)).cuda()
    plan = run.plan(n_workers=6)
    o32 = run.decode_multi(q_len, qn, qr, plan=plan, q_pos=pos)
    o16 = run.decode_multi(q_len, qn, qr, plan=plan, q_pos=pos, o_dtype="bf16")
    assert run.status() == 0
    ref = oracle_decode_multi(case, qn, qr, q_pos=pos.cpu().numpy())
    assert rel_rms_err(to_np(o32), ref) <= TOL_BF16_REL
    # the bf16 output is the fp32 result rounded once (round to nearest even)
    assert torch.equal(o16, o32.to(torch.bfloat16))


def test_multi_ragged_batch_sampled(gpu):
    """32 sequences of 4K-8K tokens, 4 new tokens each: sampled outputs."""
    case = mla_synth.workload("v3_b32_ragged")
    q_len = 4
    qn, qr = mla_synth.multi_queries(case, q_len, seed=5)
    run = DeviceRun(gpu, case)
    # the plan the benchmark uses: ranges cut for four head blocks each
    plan = run.m.mla_plan_create_multi(run.d, (case.lens + case.n_new).tolist(), q_len)
    o = to_np(run.decode_multi(q_len, qn, qr, plan=plan))
    assert run.status() == 0
    rng = np.random.default_rng(7)
    tri = [(int(rng.integers(32)), int(rng.integers(q_len)), int(rng.integers(128))) for _ in range(12)]
    seqs = sorted({b for b, _, _ in tri})
    from tests.helpers import oracle_cache
    C, R = oracle_cache(case, seqs=seqs)
    ref = oracle_decode_multi(case, qn, qr, triples=tri, C=C, R=R)
    got = np.stack([o[b, j, i] for b, j, i in tri])
    assert rel_rms_err(got, ref) <= TOL_BF16_REL


def test_multi_many_units_and_groups(gpu):
    """40 sequences, 2 new tokens each (256 query heads): each absorb
    workgroup runs its weight quarter over 2 tokens x 2 blocks of 32
    sequences (the second block of 8), and each combine workgroup of a head
    loops over its 3 groups of 16 sequences (the last of 8)."""
    rng = np.random.default_rng(1040)
    lens = [int(x) for x in rng.integers(0, 500, size=40)]
    lens[3] = 1
    case = v3_case(lens, "bf16", seed=84)
    qn, qr = mla_synth.multi_queries(case, 2, seed=97)
    run = DeviceRun(gpu, case)
    o = to_np(run.decode_multi(2, qn, qr))
    assert run.status() == 0
    assert rel_rms_err(o, oracle_decode_multi(case, qn, qr)) <= TOL_BF16_REL


@pytest.mark.parametrize("latent,q_len,workers", [("bf16", 4, 24), ("fp8", 3, 24), ("bf16", 2, 0), ("bf16", 16, 40)])
def test_multi_plan_for_tokens(gpu, latent, q_len, workers):
    """A plan from mla_plan_create_multi (ranges cut for the head blocks of
    q_len tokens: fewer, longer ranges) against the oracle, over the edge
    lengths."""
    lens = [1, 2, 3, 31, 33, 100, 700, 0, 64, 15]
    case = v3_case(lens, latent, seed=83)
    qn, qr = mla_synth.multi_queries(case, q_len, seed=95 + q_len)
    run = DeviceRun(gpu, case)
    plan = run.m.mla_plan_create_multi(run.d, lens, q_len, workers)
    blocks = (q_len * 128 + 127) // 128
    assert len(plan.ranges()) <= max(1, (workers or 256) // blocks)
    o = to_np(run.decode_multi(q_len, qn, qr, plan=plan))
    assert run.status() == 0
    tol = TOL_FP8_REL if latent == "fp8" else TOL_BF16_REL
    assert rel_rms_err(o, oracle_decode_multi(case, qn, qr)) <= tol
