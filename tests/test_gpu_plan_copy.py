"""GPU tests of the workspace's plan copy. The library keeps no record of
which workspace holds which plan: the first kernel of every decode checks
the copy against the plan's checksum and fetches it again from the plan's
pinned host block when they differ. So a workspace the caller overwrites
between calls, or shares between plans, still gives the right results."""
import numpy as np
import pytest
import torch

from tests.helpers import DeviceRun, TOL_BF16_REL, TOL_F32_ABS, make, max_abs_err, oracle_full, rel_rms_err, to_np

pytestmark = pytest.mark.gpu

V3 = dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128)
LENS = [1, 31, 32, 33, 100, 700, 0, 64, 200]


def v3_case(seed):
    return make(B=len(LENS), lens=("list", LENS), latent_dtype="bf16", rope_dtype="bf16", act_dtype="bf16",
                seed=seed, **V3)


@pytest.mark.parametrize("path", ["fast", "generic"])
def test_workspace_overwritten_between_decodes(gpu, path, monkeypatch):
    """Every byte of the workspace past the status word set to 0xFF between
    two decodes on one plan: the second decode refetches the plan and gives
    the first one's output bit for bit, with no device error."""
    if path == "generic":
        monkeypatch.setenv("MLA_FORCE_GENERIC", "1")
        case = make(B=3, lens=("list", [5, 64, 130]), latent_dtype="f32", rope_dtype="f32", act_dtype="f32",
                    seed=110, H=4, d_c=32, d_rope=8, d_nope=16, d_v=16)
    else:
        case = v3_case(110)
    run = DeviceRun(gpu, case)
    plan = run.plan(n_workers=20)
    a = run.decode(plan=plan)
    assert run.status() == 0
    run.ws[256:].fill_(0xFF)
    b = run.decode(plan=plan)
    assert run.status() == 0
    assert torch.equal(a, b)
    ref = oracle_full(case)
    if path == "generic":
        assert max_abs_err(to_np(b), ref) <= TOL_F32_ABS
    else:
        assert rel_rms_err(to_np(b), ref) <= TOL_BF16_REL


def test_plans_alternating_on_one_workspace(gpu):
    """Two plans of different item counts decode alternately on one
    workspace (each call finds the other plan's copy there): both give the
    oracle's output, the same each time."""
    case = v3_case(111)
    run = DeviceRun(gpu, case)
    p1, p2 = run.plan(n_workers=20), run.plan(n_workers=7)
    assert p1.n_items != p2.n_items
    ref = oracle_full(case)
    outs = []
    for plan in (p1, p2, p1, p2):
        o = run.decode(plan=plan)
        assert run.status() == 0
        outs.append(o.clone())
        assert rel_rms_err(to_np(o), ref) <= TOL_BF16_REL
    assert torch.equal(outs[0], outs[2]) and torch.equal(outs[1], outs[3])


def test_fresh_workspace_of_stale_bytes(gpu):
    """A workspace whose plan region holds another plan's valid copy (the
    bytes a freed workspace leaves behind): the decode notices and refetches."""
    case = v3_case(112)
    run = DeviceRun(gpu, case)
    p1, p2 = run.plan(n_workers=20), run.plan(n_workers=5)
    run.decode(plan=p1)
    assert run.status() == 0
    stale = run.ws.clone()  # holds p1's copy
    run.ws = stale
    o = run.decode(plan=p2)
    assert run.status() == 0
    assert rel_rms_err(to_np(o), oracle_full(case)) <= TOL_BF16_REL
    assert np.isfinite(to_np(o)).all()
