"""GPU parity of the decode from precomputed absorbed weights (C ABI through
the binding) against oracle.merged:

* the one-time merges (W_UK,i^T W_Q,i and W_O,i W_UV,i) element by element,
  read through the documented storage (row-major, or fragment-tiled when the
  shape allows): fp32 within 1e-5 of the largest value; bf16 within one
  bf16 ulp of the exact product (fp32 sums rounded once);
* mla_decode_merged end to end (the GPU's own merged weights, the oracle's
  fp64 ones): fp32 kernels within 1e-4 (max |err| / rms), the matrix-core
  path within the bf16 tolerance 2e-2, over ragged lengths with an empty
  sequence, several tiles and tails, bf16 and fp32 outputs;
* the same bf16 inputs through the fp32 kernels (MLA_FORCE_GENERIC=1);
* the full-size workload (batch 32, lengths U[4096, 8192], query latent
  1536 wide, d_out 7168), every output of three sampled sequences against
  the oracle's unmerged form (pinned equal to the merged one);
* a query past fp16's range reports MLA_ERR_RANGE."""
import numpy as np
import pytest
import torch

import mla_synth
from mla_synth.device import _t
from oracle import merged as om
from tests.helpers import (DT, DeviceRun, TOL_BF16_REL, act_to_f64, make, oracle_cache, rel_rms_err, to_np)

pytestmark = pytest.mark.gpu

V3 = dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128)
LENS = [1, 31, 32, 33, 100, 700, 0, 64, 200]
MLA_ERR_RANGE = 7


class Merged:
    """A case plus x, W_Q, W_O on the device, merged there."""

    def __init__(self, m, case, d_x, d_out, seed):
        self.m, self.case, self.d_x, self.d_out = m, case, d_x, d_out
        self.run = DeviceRun(m, case)
        self.x, self.w_q, self.w_o = mla_synth.merged_inputs(case, d_x, d_out, seed)
        dev = self.run.t["rows"].device
        self.tx, self.tq, self.to = _t(self.x, dev), _t(self.w_q, dev), _t(self.w_o, dev)
        wdt = torch.float32 if case.act_dtype == "f32" else torch.bfloat16
        self.a = torch.empty((case.H, case.d_c, d_x), dtype=wdt, device=dev)
        self.bm = torch.empty((d_out, case.H * case.d_c), dtype=wdt, device=dev)
        d, wt = self.run.d, DT[case.act_dtype]
        m.mla_merge_query_weight(d, d_x, self.tq, self.run.t["w_uk"], wt, self.a)
        m.mla_merge_output_weight(d, d_out, self.to, self.run.t["w_uv"], wt, self.bm)

    def decode(self, y_dtype="f32", q_pos=None):
        c, m, r = self.case, self.m, self.run
        plan = r.plan()
        need = m.mla_decode_merged_workspace_bytes(r.d, plan, self.d_out)
        ws = torch.empty(need, dtype=torch.uint8, device=self.tx.device)
        m.mla_workspace_init(ws)
        r.ws = ws
        y = torch.empty((c.B, self.d_out), dtype=torch.float32 if y_dtype == "f32" else torch.bfloat16,
                        device=self.tx.device)
        m.mla_decode_merged(r.d, r.cache, plan, self.d_x, self.tx, r.t["q_rope"], q_pos, self.a, self.d_out,
                            self.bm, DT[c.act_dtype], y, DT[y_dtype], ws)
        return y

    def f64(self, name):
        return act_to_f64(getattr(self, name), self.case.act_dtype)

    def oracle_weights(self):
        c = self.case
        a = om.merge_query_weight(self.f64("w_q"), act_to_f64(c.w_uk, c.act_dtype))
        bm = om.merge_output_weight(self.f64("w_o"), act_to_f64(c.w_uv, c.act_dtype))
        return a, bm

    def oracle(self):
        c = self.case
        C, R = oracle_cache(c)
        a, bm = self.oracle_weights()
        return om.decode_merged(C, R, c.seq_start, c.lens, self.f64("x"), act_to_f64(c.q_rope, c.act_dtype), a, bm,
                                c.softmax_scale, c.rope_base)


def untile(w, R, K):
    """A merged weight as the header documents its storage: fragment-tiled
    when R % 32 == 0 and K % 64 == 0 (element (r, k) at ((r / 32) (K / 64) +
    k / 64) 2048 + ((k % 32) / 8) 512 + (r % 32 + 32 ((k % 64) / 32)) 8 +
    k % 8), else row-major; returned as [R, K]."""
    flat = np.asarray(w).reshape(-1)
    if R % 32 or K % 64:
        return flat.reshape(R, K)
    # [tile row, tile k, f (k % 32 / 8), h (k % 64 / 32), r % 32, k % 8]
    t = flat.reshape(R // 32, K // 64, 4, 2, 32, 8)
    return t.transpose(0, 4, 1, 3, 2, 5).reshape(R, K)


def test_untile_reads_the_documented_offsets():
    R, K = 64, 128
    rng = np.random.default_rng(0)
    dense = rng.standard_normal((R, K))
    flat = np.empty(R * K)
    for r in range(R):
        for k in range(K):
            off = ((r // 32) * (K // 64) + k // 64) * 2048 + ((k % 32) // 8) * 512 + (r % 32 + 32 * ((k % 64) // 32)) * 8 + k % 8
            flat[off] = dense[r, k]
    assert np.array_equal(untile(flat, R, K), dense)


def tiny_f32(seed):
    return make(B=4, H=4, d_c=32, d_rope=8, d_nope=16, d_v=16, lens=("list", [5, 0, 70, 33]), latent_dtype="f32",
                rope_dtype="f32", act_dtype="f32", seed=seed)


def v3_case(seed, latent="bf16"):
    return make(B=len(LENS), lens=("list", LENS), latent_dtype=latent, rope_dtype="bf16", act_dtype="bf16",
                seed=seed, **V3)


def test_merges_f32_match_oracle(gpu):
    """Shapes that keep the row-major storage (d_x = 24, d_out = 20)."""
    mg = Merged(gpu, tiny_f32(200), d_x=24, d_out=20, seed=201)
    a, bm = mg.oracle_weights()
    c = mg.case
    assert np.max(np.abs(untile(to_np(mg.a), c.H * c.d_c, 24) - a.reshape(c.H * c.d_c, 24))) <= 1e-5 * np.max(np.abs(a))
    assert np.max(np.abs(untile(to_np(mg.bm), 20, c.H * c.d_c) - bm)) <= 1e-5 * np.max(np.abs(bm))


@pytest.mark.parametrize("d_x,d_out", [(512, 256), (1024, 384)])
def test_merges_bf16_within_one_ulp(gpu, d_x, d_out):
    """The fragment-tiled storage (both weights' shapes allow it)."""
    mg = Merged(gpu, v3_case(202), d_x=d_x, d_out=d_out, seed=203)
    c = mg.case
    shapes = ((c.H * c.d_c, d_x), (d_out, c.H * c.d_c))
    for got, exact, (R, K) in zip((mg.a, mg.bm), mg.oracle_weights(), shapes):
        g = untile(to_np(got), R, K)
        exact = exact.reshape(R, K)
        ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
        assert np.all(np.abs(g - exact) <= ulp + 1e-6 * np.max(np.abs(exact)))


@pytest.mark.parametrize("seed", [210, 211])
def test_decode_merged_fp32_kernels(gpu, seed):
    mg = Merged(gpu, tiny_f32(seed), d_x=24, d_out=20, seed=seed + 50)
    y = to_np(mg.decode())
    assert mg.run.status() == 0
    ref = mg.oracle()
    assert rel_rms_err(y, ref) <= 1e-4
    assert np.all(y[1] == 0)  # the empty sequence


@pytest.mark.parametrize("y_dtype", ["f32", "bf16"])
def test_decode_merged_matrix_cores(gpu, y_dtype):
    """The merged weights are stored in bf16 (the emulation with bf16 A and Bm
    and exact arithmetic otherwise gives 1.4e-2 on this case); a bf16 y adds
    its own rounding, up to half an ulp (2^-8 relative) of the largest
    output, 7.5 times the rms here."""
    mg = Merged(gpu, v3_case(220), d_x=512, d_out=256, seed=221)
    y = to_np(mg.decode(y_dtype))
    assert mg.run.status() == 0
    ref = mg.oracle()
    tol = TOL_BF16_REL
    if y_dtype == "bf16":
        tol += 2.0 ** -8 * np.max(np.abs(ref)) / np.sqrt(np.mean(ref ** 2))
    assert rel_rms_err(y, ref) <= tol
    assert np.all(y[6] == 0)


def test_decode_merged_fp8_cache(gpu):
    mg = Merged(gpu, v3_case(222, latent="fp8"), d_x=512, d_out=384, seed=223)
    y = to_np(mg.decode())
    assert mg.run.status() == 0
    assert rel_rms_err(y, mg.oracle()) <= 6e-2


def test_decode_merged_bf16_on_the_fp32_kernels(gpu, monkeypatch):
    monkeypatch.setenv("MLA_FORCE_GENERIC", "1")
    mg = Merged(gpu, v3_case(224), d_x=512, d_out=256, seed=225)
    y = to_np(mg.decode())
    assert mg.run.status() == 0
    assert rel_rms_err(y, mg.oracle()) <= TOL_BF16_REL


def test_decode_merged_full_size_sampled(gpu):
    case = mla_synth.workload("v3_b32_ragged")
    mg = Merged(gpu, case, d_x=1536, d_out=7168, seed=230)
    y = to_np(mg.decode())
    assert mg.run.status() == 0
    seqs = [0, 13, 31]
    C, R = oracle_cache(case, seqs=seqs)
    c = case
    ref = om.decode_factored(C, R, c.seq_start, c.lens, mg.f64("x"), act_to_f64(c.q_rope, c.act_dtype),
                             mg.f64("w_q"), act_to_f64(c.w_uk, c.act_dtype), act_to_f64(c.w_uv, c.act_dtype),
                             mg.f64("w_o"), c.softmax_scale, c.rope_base, seqs=seqs)
    assert rel_rms_err(y[seqs], ref[seqs]) <= TOL_BF16_REL


def test_decode_merged_reports_query_beyond_fp16(gpu):
    mg = Merged(gpu, v3_case(240), d_x=512, d_out=128, seed=241)
    mg.tx.view(torch.bfloat16).mul_(2.0 ** 20)
    mg.decode()
    assert mg.run.status() == MLA_ERR_RANGE
