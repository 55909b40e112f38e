"""A plain C caller (tests/c/decode_files.c, built by __graft_entry__.build())
runs the whole decode through libmla's C ABI with no Python or torch in the
process; its output is checked against the oracle."""
import os
import subprocess

import numpy as np
import pytest

from tests.helpers import TOL_BF16_REL, make, oracle_decode, rel_rms_err

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "decode_files")


def _write(d, name, arr):
    np.ascontiguousarray(arr).tofile(os.path.join(d, name))


@pytest.mark.parametrize("lens", [[1, 700, 1500], [0, 33, 4096, 64]])
def test_c_program_decode_matches_oracle(gpu, tmp_path, lens):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built; run __graft_entry__.build()")
    case = make(B=len(lens), lens=("list", lens), latent_dtype="bf16", rope_dtype="bf16", act_dtype="bf16",
                seed=70 + len(lens), H=128, d_c=512, d_rope=64, d_nope=128, d_v=128)
    d = str(tmp_path)
    n_rows = case.rows.shape[0]
    meta = np.array([case.B, case.H, n_rows, case.row_stride], dtype=np.int32).tobytes()
    meta += np.array([case.softmax_scale], dtype=np.float32).tobytes()
    with open(os.path.join(d, "meta.bin"), "wb") as f:
        f.write(meta)
    _write(d, "lens.bin", case.lens.astype(np.int32))
    _write(d, "start.bin", case.seq_start.astype(np.int32))
    _write(d, "cap.bin", case.seq_cap.astype(np.int32))
    _write(d, "rows.bin", case.rows.astype(np.uint8))
    for k in ("q_nope", "q_rope", "w_uk", "w_uv"):
        a = getattr(case, k)
        assert a.dtype == np.uint16, (k, a.dtype)  # bf16 bit patterns
        _write(d, f"{k}.bin", a)
    print(f"C caller: lens {lens}", flush=True)
    r = subprocess.run([EXE, d], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"exit {r.returncode}: {r.stdout}{r.stderr}"
    assert "decode_files ok" in r.stdout
    o = np.fromfile(os.path.join(d, "o.bin"), dtype=np.float32).reshape(case.B, case.H, case.d_v)
    ref = oracle_decode(case, absorbed=True)
    err = rel_rms_err(o.astype(np.float64), ref)
    assert err <= TOL_BF16_REL, f"max|err|/rms {err:.3e}"
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(o[b] == 0)
