"""Host-side checks of libmla that need no GPU: the library loads, exports every
entry point include/mla.h declares, the split planner's invariants hold, and
invalid arguments are refused before any HIP call."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import compressed_kv_cache_absorbed_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    txt = open(os.path.join(ROOT, "include", "mla.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = m.load()
    names = header_functions()
    assert names, "no declarations found"
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", m.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (mla_[a-z0-9_]+)", out))
    assert set(names) <= exported
    assert sorted(m.EXPORTED) == sorted(names)


def test_version_and_status_strings():
    assert m.mla_abi_version() == 1
    for k, v in m.STATUS.items():
        assert m.mla_status_str(k) == v


def d128():
    return m.dims(128, 512, 64, 128, 128)


@pytest.mark.parametrize("lens,workers", [
    ([4096] * 32, 256), (list(range(4096, 8193, 128)), 256), ([131072] * 4, 256),
    ([1, 0, 33, 5000, 31, 32], 8), ([0, 0], 4), ([7], 1), ([1000] * 300, 256),
    # total past 2^31 tokens: the planner's sums are 64-bit
    ([2**30] * 3, 256), ([2**31 - 1, 5, 2**31 - 33], 1024),
])
def test_plan_covers_every_token_once(lens, workers):
    p = m.mla_plan_create(d128(), lens, workers)
    items = p.items()
    cover = {b: [] for b in range(len(lens))}
    for b, t0, t1 in items:
        assert 0 <= t0 < t1 <= lens[b]
        cover[b].append((t0, t1))
    for b, L in enumerate(lens):
        segs = sorted(cover[b])
        pos = 0
        for t0, t1 in segs:
            assert t0 == pos
            pos = t1
        assert pos == L
        # items of one sequence are contiguous in the list (the combine needs it)
        idx = [k for k, it in enumerate(items) if it[0] == b]
        assert idx == list(range(idx[0], idx[0] + len(idx))) if idx else True
        # boundaries on tile multiples
        for t0, t1 in segs:
            assert t0 % 32 == 0
    nonempty = sum(1 for L in lens if L)
    if nonempty <= workers:
        assert len(items) <= max(workers, nonempty)


def test_plan_balances_equal_sequences():
    p = m.mla_plan_create(d128(), [8192] * 32, 256)
    sizes = [t1 - t0 for _, t0, t1 in p.items()]
    assert len(sizes) == 256 and max(sizes) == min(sizes) == 1024


def test_plan_ragged_makespan_near_ideal():
    rng = np.random.default_rng(2)
    lens = rng.integers(4096, 8192, 32, endpoint=True).tolist()
    p = m.mla_plan_create(d128(), lens, 256)
    sizes = [t1 - t0 for _, t0, t1 in p.items()]
    assert len(sizes) <= 256
    ideal = sum(lens) / 256
    assert max(sizes) <= 1.25 * ideal + 32


def test_plan_rejects_bad_input():
    h = ctypes.c_void_p()
    lib = m.load()
    d = d128()
    bad = (ctypes.c_int32 * 2)(5, -1)
    assert lib.mla_plan_create(ctypes.byref(d), bad, 2, 4, ctypes.byref(h)) == 1
    good = (ctypes.c_int32 * 2)(5, 1)
    assert lib.mla_plan_create(ctypes.byref(d), good, 0, 4, ctypes.byref(h)) == 1
    assert lib.mla_plan_create(None, good, 2, 4, ctypes.byref(h)) == 1
    assert lib.mla_plan_create(ctypes.byref(d), good, 2, -3, ctypes.byref(h)) == 1


def _cache_struct(**over):
    c = m.MlaCache(1, 1, 4096, 1152, None, 100, 2, 8192, 8192, 8192)
    for k, v in over.items():
        setattr(c, k, v)
    return c


def test_validation_rejects_before_launch():
    """All of these fail validation, so no HIP call is made (no GPU here)."""
    lib = m.load()
    d = d128()
    plan = m.mla_plan_create(d, [10, 20], 4)
    P = 4096  # a fake, 16-aligned "device" address: never dereferenced
    ws_need = m.mla_decode_workspace_bytes(d, plan)
    assert ws_need > 0

    def dec(c, qw=1, od=0, ws_bytes=ws_need, ptrs=(P,) * 7, dd=d):
        qn, qr, wuk, wuv, o, ws, _ = ptrs
        return lib.mla_decode(ctypes.byref(dd), ctypes.byref(c), plan.handle, qn, qr, None, wuk, wuv,
                              qw, o, od, ws, ws_bytes, None)

    assert dec(_cache_struct(), ws_bytes=ws_need - 1) == 5
    assert dec(_cache_struct(row_stride=1000)) == 1           # not a multiple of 16
    assert dec(_cache_struct(row_stride=1024)) == 1           # row narrower than c_kv + k_rope
    assert dec(_cache_struct(rows=4100)) == 1                 # misaligned
    assert dec(_cache_struct(latent_dtype=2)) == 1            # fp8 without scale
    assert dec(_cache_struct(scale=P)) == 1                   # scale without fp8
    assert dec(_cache_struct(rope_dtype=2)) == 1              # fp8 k_rope not supported
    assert dec(_cache_struct(batch=3)) == 1                   # plan is for 2 sequences
    assert dec(_cache_struct(), qw=2) == 1
    assert dec(_cache_struct(), od=2) == 1
    assert dec(_cache_struct(), ptrs=(P, 0, P, P, P, P, P)) == 1
    odd = m.dims(128, 512, 63, 128, 128)
    assert dec(_cache_struct(), dd=odd) == 1                  # odd RoPE width
    # append
    c = _cache_struct()
    da = m.dims(128, 512, 64, 128, 128, d_model=7168)
    wsa = m.mla_append_workspace_bytes(da, 2, 1)
    assert lib.mla_append(ctypes.byref(da), ctypes.byref(c), P, -1, P, P, 1, P, wsa, None) == 1
    assert lib.mla_append(ctypes.byref(da), ctypes.byref(c), P, 1, P, P, 2, P, wsa, None) == 1
    assert lib.mla_append(ctypes.byref(da), ctypes.byref(c), None, 1, P, P, 1, P, wsa, None) == 1
    assert lib.mla_append(ctypes.byref(da), ctypes.byref(c), P, 1, P, P, 1, P, 16, None) == 5
    # several query tokens: 1 <= q_len <= 16, the matrix-core path only, a
    # workspace sized for q_len
    ws4 = m.mla_decode_multi_workspace_bytes(d, plan, 4)
    assert ws4 > ws_need and m.mla_decode_multi_workspace_bytes(d, plan, 1) == ws_need
    assert m.mla_decode_multi_workspace_bytes(d, plan, 0) == 0
    assert m.mla_decode_multi_workspace_bytes(d, plan, 17) == 0

    def decm(c, q_len, ws_bytes, dd=d, qw=1):
        return lib.mla_decode_multi(ctypes.byref(dd), ctypes.byref(c), plan.handle, q_len, P, P, None, P, P, qw, P,
                                    0, P, ws_bytes, None)

    assert decm(_cache_struct(), 0, ws4) == 1
    assert decm(_cache_struct(), 17, 1 << 40) == 1
    assert decm(_cache_struct(), 4, ws4 - 1) == 5
    assert decm(_cache_struct(), 4, ws4, qw=0) == 2                # fp32 weights: generic path, one token only
    small = m.dims(4, 32, 8, 16, 16)
    plan_s = m.mla_plan_create(small, [10, 20], 4)
    c_s = _cache_struct(row_stride=256)
    assert lib.mla_decode_multi(ctypes.byref(small), ctypes.byref(c_s), plan_s.handle, 2, P, P, None, P, P, 0, P, 0,
                                P, 1 << 30, None) == 2
    # paged caches: blocks of a multiple of 32 rows, a table of at least one
    # block per sequence; seq_start may then be NULL (and is required otherwise)
    assert dec(_cache_struct(seq_start=None)) == 1
    assert dec(_cache_struct(seq_start=None, block_table=P, block_tokens=48, max_blocks=4)) == 1
    assert dec(_cache_struct(seq_start=None, block_table=P, block_tokens=64, max_blocks=0)) == 1
    assert dec(_cache_struct(seq_start=None, block_table=P, block_tokens=0, max_blocks=4)) == 1
    # calibration copy and workspace init validate too
    assert lib.mla_calib_copy(P, P, 17, None) == 1
    assert lib.mla_calib_read(P, 17, P, None) == 1
    assert lib.mla_calib_read(None, 16, P, None) == 1
    assert lib.mla_calib_read(P, 16, None, None) == 1
    assert lib.mla_calib_read(P, 16, P + 2, None) == 1
    assert lib.mla_workspace_init(None, 256, None) == 1


def test_workspace_sizes_grow_with_plan():
    d = d128()
    small = m.mla_decode_workspace_bytes(d, m.mla_plan_create(d, [100], 4))
    big = m.mla_decode_workspace_bytes(d, m.mla_plan_create(d, [100000] * 8, 256))
    assert 0 < small < big
    assert big >= 256 * 128 * 512 * 4  # fp32 partial per item and head


def test_one_size_workspace_covers_decode_and_one_token_append():
    d = d128()  # no d_model: decode only
    plan = m.mla_plan_create(d, [100, 5000, 0], 16)
    assert m.mla_workspace_bytes(d, plan) == m.mla_decode_workspace_bytes(d, plan)
    dm = m.dims(128, 512, 64, 128, 128, d_model=7168)
    for lens in ([100, 5000, 0], [1] * 300):
        plan = m.mla_plan_create(dm, lens, 16)
        one = m.mla_workspace_bytes(dm, plan)
        assert one == max(m.mla_decode_workspace_bytes(dm, plan), m.mla_append_workspace_bytes(dm, len(lens), 1))
    lib = m.load()
    assert lib.mla_workspace_bytes(None, plan.handle) == 0
    assert lib.mla_workspace_bytes(ctypes.byref(dm), None) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libmla.so every entry point raises: there is no CPU fallback."""
    monkeypatch.setattr(m, "_LIB", None)
    monkeypatch.setattr(m, "lib_path", lambda: str(tmp_path / "libmla.so"))
    with pytest.raises(RuntimeError, match="not built"):
        m.load()
    with pytest.raises(RuntimeError, match="not built"):
        m.mla_abi_version()
    with pytest.raises(RuntimeError, match="not built"):
        m.mla_plan_create(d128(), [10, 20], 4)


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU; asking for more exits with a message and
    touches no device."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
