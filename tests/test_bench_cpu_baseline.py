"""The CPU-baseline leg of bench.py on the host: the oracle's non-absorbed
decode timed on a bounded sample of (sequence, head) pairs and scaled to the
step, the absorbed form beside it, and the sampled parity figure. A stand-in
for the GPU result supplies the oracle's own outputs, so the parity figure
must come out at rounding level (the leg compares with whatever outputs it
is handed)."""
import numpy as np
import pytest

import bench
import mla_synth
from oracle import mla as omla
from tests.helpers import act_to_f64, oracle_cache


class _Host:
    def __init__(self, a):
        self.a = a

    def float(self):
        return self

    def cpu(self):
        return self

    def numpy(self):
        return self.a


def test_cpu_baseline_fields_and_sampled_parity():
    case = mla_synth.workload("v3_b1_4k")
    C, R = oracle_cache(case)
    o = omla.decode(C, R, case.seq_start, case.lens, act_to_f64(case.q_nope, "bf16"),
                    act_to_f64(case.q_rope, "bf16"), act_to_f64(case.w_uk, "bf16"), act_to_f64(case.w_uv, "bf16"),
                    case.softmax_scale, case.rope_base, pairs=[(0, i) for i in range(case.H)])
    res = {"case": case, "o": _Host(np.asarray(o).reshape(case.B, case.H, case.d_v)),
           "cache_bytes": int(case.lens.sum()) * case.row_bytes}
    r = bench.cpu_baseline(res, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "GB/s"
    assert r["value"] > 0 and r["step_seconds"] > 0 and r["tokens_per_s"] > 0
    assert r["absorbed_value"] > 0 and r["absorbed_step_seconds"] > 0
    assert r["tokens_per_s"] == pytest.approx(case.B / r["step_seconds"], rel=1e-2)
    assert r["parity_max_err_over_rms"] < 1e-9
