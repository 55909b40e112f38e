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
    check_plan(m.mla_plan_create(d128(), lens, workers), lens, workers)


def check_plan(p, lens, workers):
    """Every token of every sequence in exactly one item, a sequence's items
    contiguous and in order on tile boundaries, the ranges cutting the item
    list in order into at most `workers` non-empty runs."""
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
    # the ranges cut the item list in order into at most `workers` non-empty runs
    ranges = p.ranges()
    assert len(ranges) <= workers
    assert [k for r in ranges for k in range(*r)] == list(range(len(items)))
    assert all(k1 > k0 for k0, k1 in ranges)
    assert (len(ranges) == 0) == (sum(lens) == 0)


def test_plan_invariants_on_seeded_random_batches():
    """Both planners on 400 seeded random batches (uniform, log-uniform, tiny
    and edge lengths; 1-2000 workers; 1-16 query tokens for the multi plan),
    against the same invariants; the multi plan's ranges are also bounded by
    the workers per head block and its items equal the one-token plan's at
    that worker count."""
    rng = np.random.default_rng(7)
    for it in range(400):
        B = int(rng.integers(1, 300))
        kind = it % 4
        if kind == 0:
            lens = rng.integers(0, 70000, size=B)
        elif kind == 1:
            lens = np.exp(rng.uniform(0, 12, size=B)).astype(np.int64)
        elif kind == 2:
            lens = rng.integers(0, 40, size=B)
        else:
            lens = rng.choice([0, 1, 31, 32, 33, 4096, 131072], size=B)
        lens = [int(x) for x in lens]
        workers = int(rng.integers(1, 2000))
        if it % 2 == 0:
            check_plan(m.mla_plan_create(d128(), lens, workers), lens, workers)
        else:
            q_len = int(rng.integers(1, 17))
            p = m.mla_plan_create_multi(d128(), lens, q_len, workers)
            per_block = max(1, workers // q_len)
            check_plan(p, lens, per_block)
            assert p.items() == m.mla_plan_create(d128(), lens, per_block).items()


ITEM_COST = 6  # the planner's fixed cost of an item, in tiles


def range_costs(p):
    """Tiles plus ITEM_COST per item, the planner's cost, of every range."""
    items = p.items()
    return [sum((items[k][2] - items[k][1] + 31) // 32 + ITEM_COST for k in range(k0, k1)) for k0, k1 in p.ranges()]


def test_plan_balances_equal_sequences():
    p = m.mla_plan_create(d128(), [8192] * 32, 256)
    sizes = [t1 - t0 for _, t0, t1 in p.items()]
    assert len(sizes) == 256 and max(sizes) == min(sizes) == 1024
    assert p.ranges() == [(k, k + 1) for k in range(256)]


@pytest.mark.parametrize("lens,workers", [
    (np.random.default_rng(2).integers(4096, 8192, 32, endpoint=True).tolist(), 256),
    (np.exp(np.random.default_rng(3).uniform(np.log(1024), np.log(32768), 128)).astype(int).tolist(), 256),
    ([100000, 10, 10, 5000] + [64] * 40, 256), ([33] * 1000, 256), ([65536], 100),
])
def test_plan_ranges_balanced(lens, workers):
    """Each range costs at most the average cost, counting one more item per
    sequence and per range (the splits), plus one piece of slack."""
    p = m.mla_plan_create(d128(), lens, workers)
    tiles = sum((L + 31) // 32 for L in lens)
    nonempty = sum(1 for L in lens if L)
    costs = range_costs(p)
    assert max(costs) <= (tiles + ITEM_COST * (nonempty + workers)) / workers + ITEM_COST + 2
    # the longest range's tiles within 6 % + 3 tiles of the balanced share
    items = p.items()
    rt = [sum((items[k][2] - items[k][1] + 31) // 32 for k in range(*r)) for r in p.ranges()]
    assert max(rt) <= 1.06 * tiles / workers + 3 or len(lens) > workers


def test_plan_lognormal_lengths_beat_per_sequence_chunks():
    """Log-uniform lengths 1K..32K over 128 sequences: no range holds more
    than 2 % over the balanced share of tiles (one common chunk size per
    sequence would leave the longest chunk about a third over it)."""
    lens = np.exp(np.random.default_rng(4).uniform(np.log(1024), np.log(32768), 128)).astype(int).tolist()
    p = m.mla_plan_create(d128(), lens, 256)
    items = p.items()
    rt = [sum((items[k][2] - items[k][1] + 31) // 32 for k in range(*r)) for r in p.ranges()]
    share = sum((L + 31) // 32 for L in lens) / 256
    assert max(rt) <= 1.02 * share + 2


@pytest.mark.parametrize("q_len,workers", [(1, 256), (2, 256), (4, 256), (16, 256), (3, 7), (4, 2)])
def test_plan_multi_ranges_per_head_blocks(q_len, workers):
    """mla_plan_create_multi cuts at most n_workers / ceil(q_len H / 128)
    ranges (at least one), covering every token once, balanced like a
    one-token plan of that many workers; q_len 1 is mla_plan_create."""
    lens = np.random.default_rng(q_len).integers(1, 9000, 40).tolist()
    p = m.mla_plan_create_multi(d128(), lens, q_len, workers)
    blocks = q_len  # H = 128: one head block per token
    W = max(1, workers // blocks)
    assert len(p.ranges()) <= W
    assert sorted((b, t0, t1) for b, t0, t1 in p.items()) == sorted(m.mla_plan_create(d128(), lens, W).items())
    if q_len == 1:
        assert p.items() == m.mla_plan_create(d128(), lens, workers).items()


def test_plan_multi_rejects_bad_q_len():
    h = ctypes.c_void_p()
    lib = m.load()
    d = d128()
    good = (ctypes.c_int32 * 2)(10, 20)
    for q in (0, 17, -1):
        assert lib.mla_plan_create_multi(ctypes.byref(d), good, 2, q, 4, ctypes.byref(h)) == 1


def test_plan_inspection_rejects_bad_index():
    p = m.mla_plan_create(d128(), [100, 5000], 8)
    lib = m.load()
    k0, k1 = ctypes.c_int32(), ctypes.c_int32()
    n = lib.mla_plan_num_ranges(p.handle)
    assert 1 <= n <= 8
    assert lib.mla_plan_range(p.handle, n - 1, ctypes.byref(k0), ctypes.byref(k1)) == 0 and k1.value == p.n_items
    for j in (-1, n):
        assert lib.mla_plan_range(p.handle, j, ctypes.byref(k0), ctypes.byref(k1)) == 1
    assert lib.mla_plan_range(p.handle, 0, None, ctypes.byref(k1)) == 1
    assert lib.mla_plan_num_ranges(None) == -1


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


def test_merged_weight_calls_validate_before_launch():
    """The precomputed-weights entry points refuse bad arguments with no HIP call."""
    lib = m.load()
    d = d128()
    plan = m.mla_plan_create(d, [10, 20], 4)
    P = 4096
    # merges: sizes >= 1, F32 or BF16, 16-byte aligned non-NULL pointers
    for fn in (lib.mla_merge_query_weight, lib.mla_merge_output_weight):
        assert fn(ctypes.byref(d), 0, P, P, 1, P, None) == 1
        assert fn(ctypes.byref(d), 256, P, P, 2, P, None) == 1
        assert fn(ctypes.byref(d), 256, None, P, 1, P, None) == 1
        assert fn(ctypes.byref(d), 256, P, P + 2, 1, P, None) == 1
        assert fn(ctypes.byref(m.dims(128, 512, 63, 128, 128)), 256, P, P, 1, P, None) == 1
    need = m.mla_decode_merged_workspace_bytes(d, plan, 7168)
    assert need > m.mla_decode_workspace_bytes(d, plan)
    # o^ (4 bytes per latent value) and 16 splits of fp32 outputs
    assert need >= m.mla_decode_workspace_bytes(d, plan) + 4 * 2 * 128 * 512 + 4 * 16 * 2 * 7168
    assert m.mla_decode_merged_workspace_bytes(d, plan, 0) == 0

    def dm(c, d_x=1536, d_out=7168, wt=1, yt=0, ws_bytes=need, x=P, bm=P):
        return lib.mla_decode_merged(ctypes.byref(d), ctypes.byref(c), plan.handle, d_x, x, P, None, P, d_out, bm,
                                     wt, P, yt, P, ws_bytes, None)

    assert dm(_cache_struct(), ws_bytes=need - 1) == 5
    assert dm(_cache_struct(), d_x=0) == 1
    assert dm(_cache_struct(), d_out=0) == 1
    assert dm(_cache_struct(), wt=2) == 1
    assert dm(_cache_struct(), yt=2) == 1
    assert dm(_cache_struct(), x=None) == 1
    assert dm(_cache_struct(), bm=P + 8) == 1
    assert dm(_cache_struct(batch=3)) == 1
    # the fp32 kernels stage x in 64 KB of LDS: d_x up to 16384
    assert dm(_cache_struct(), d_x=16385 * 2, wt=0, ws_bytes=1 << 40) == 2


def test_tensor_calls_check_dtypes_and_shapes():
    """The tensor-level calls refuse, before touching a device, activations
    and weights of mixed dtypes or of sizes that do not match the dims and
    the plan's batch (either would make a kernel read past a buffer), and a
    self-allocated workspace on an explicit stream (it would be freed while
    the stream may still use it)."""
    import torch
    d = d128()
    plan = m.mla_plan_create(d, [10, 20], 4)
    c = _cache_struct()
    bf = torch.bfloat16

    def z(*shape, dt=bf):
        return torch.zeros(shape, dtype=dt)

    ok = dict(q_nope=z(2, 128, 128), q_rope=z(2, 128, 64), w_uk=z(128, 128, 512), w_uv=z(128, 128, 512))
    bad = [
        dict(w_uk=z(128, 128, 512, dt=torch.float32)),  # f32 weights with bf16 queries
        dict(q_rope=z(2, 128, 64, dt=torch.float32)),
        dict(q_nope=z(3, 128, 128)),                    # batch differs from the plan
        dict(q_nope=z(2, 128, 128, dt=torch.float16)),  # not f32 or bf16
        dict(w_uv=z(128, 128, 256)),
    ]
    for over in bad:
        args = dict(ok, **over)
        with pytest.raises(ValueError):
            m.decode(d, c, plan, args["q_nope"], args["q_rope"], args["w_uk"], args["w_uv"])
    with pytest.raises(ValueError):
        m.decode(d, c, plan, **ok, out=z(2, 128, 64, dt=torch.float32))
    with pytest.raises(ValueError):
        m.decode(d, c, plan, **ok, stream=1234)
    da = m.dims(128, 512, 64, 128, 128, d_model=256)
    h, wd, wk = z(2, 1, 256), z(512, 256), z(64, 256)
    with pytest.raises(ValueError):
        m.append(da, c, h, wd, z(64, 256, dt=torch.float32))
    with pytest.raises(ValueError):
        m.append(da, c, z(2, 1, 128), wd, wk)
    with pytest.raises(ValueError):
        m.append(da, c, z(3, 1, 256), wd, wk)
    with pytest.raises(ValueError):
        m.append(da, c, h, wd, wk, stream=1234)
    with pytest.raises(ValueError):
        m.append_decode(da, c, plan, h, wd, wk, ok["q_nope"].float(), ok["q_rope"].float(), ok["w_uk"].float(),
                        ok["w_uv"].float())


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
