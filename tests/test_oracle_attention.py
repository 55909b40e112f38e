"""Pins for oracle.mla (append, non-absorbed decode, absorbed decode, split merge)
against brute force, PyTorch's scaled_dot_product_attention, closed-form
special cases and invariants."""
import math

import numpy as np
import pytest
import torch

import mla_synth
from oracle import codecs, mla
from oracle.rope import rope


def rel_rms(a, b):
    return np.max(np.abs(a - b)) / max(np.sqrt(np.mean(b ** 2)), 1e-300)


def random_problem(seed, H=3, d_c=6, d_rope=4, d_nope=5, d_v=7, lens=(1, 4, 9), gap=2):
    rng = np.random.default_rng(seed)
    B = len(lens)
    starts, acc = [], gap
    for L in lens:
        starts.append(acc)
        acc += L + gap
    C = rng.standard_normal((acc, d_c))
    R = rng.standard_normal((acc, d_rope))
    return dict(
        C=C, R=R, seq_start=np.array(starts), seq_len=np.array(lens),
        q_nope=rng.standard_normal((B, H, d_nope)), q_rope=rng.standard_normal((B, H, d_rope)),
        w_uk=rng.standard_normal((H, d_nope, d_c)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c),
        softmax_scale=1.0 / math.sqrt(d_nope + d_rope), rope_base=10000.0)


def brute_force(p, q_pos=None):
    """Scalar loops over tokens and dimensions, written independently of the
    matrix form."""
    C, R = p["C"], p["R"]
    B, H, d_nope = p["q_nope"].shape
    d_rope = p["q_rope"].shape[2]
    d_c = C.shape[1]
    d_v = p["w_uv"].shape[1]
    out = np.zeros((B, H, d_v))
    for b in range(B):
        L = int(p["seq_len"][b])
        start = int(p["seq_start"][b])
        pos = L - 1 if q_pos is None else int(q_pos[b])
        for i in range(H):
            qr = p["q_rope"][b, i]
            qrot = []
            for j in range(d_rope // 2):
                a = pos * p["rope_base"] ** (-2.0 * j / d_rope)
                qrot += [qr[2 * j] * math.cos(a) - qr[2 * j + 1] * math.sin(a),
                         qr[2 * j] * math.sin(a) + qr[2 * j + 1] * math.cos(a)]
            scores = []
            for t in range(L):
                row = start + t
                s = 0.0
                for n in range(d_nope):
                    k_n = sum(p["w_uk"][i, n, c] * C[row, c] for c in range(d_c))
                    s += p["q_nope"][b, i, n] * k_n
                for j in range(d_rope):
                    s += qrot[j] * R[row, j]
                scores.append(p["softmax_scale"] * s)
            if not scores:
                continue
            m = max(scores)
            e = [math.exp(x - m) for x in scores]
            z = sum(e)
            for v in range(d_v):
                acc = 0.0
                for t in range(L):
                    v_t = sum(p["w_uv"][i, v, c] * C[start + t, c] for c in range(d_c))
                    acc += e[t] / z * v_t
                out[b, i, v] = acc
    return out


def run(fn, p, **kw):
    return fn(p["C"], p["R"], p["seq_start"], p["seq_len"], p["q_nope"], p["q_rope"],
              p["w_uk"], p["w_uv"], p["softmax_scale"], p["rope_base"], **kw)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_vs_brute_force(seed):
    p = random_problem(seed)
    assert rel_rms(run(mla.decode, p), brute_force(p)) < 1e-12


def test_decode_vs_brute_force_explicit_positions():
    p = random_problem(5, lens=(3, 6))
    q_pos = np.array([100, 7])
    assert rel_rms(run(mla.decode, p, q_pos=q_pos), brute_force(p, q_pos)) < 1e-12


def test_decode_vs_torch_sdpa():
    p = random_problem(9, H=4, d_c=16, d_rope=8, d_nope=12, d_v=10, lens=(33, 1, 70))
    o = run(mla.decode, p)
    for b in range(3):
        L, s0 = int(p["seq_len"][b]), int(p["seq_start"][b])
        Cb = torch.from_numpy(p["C"][s0:s0 + L])
        Rb = torch.from_numpy(p["R"][s0:s0 + L])
        for i in range(4):
            K = torch.cat([Cb @ torch.from_numpy(p["w_uk"][i]).T, Rb], dim=1)
            V = Cb @ torch.from_numpy(p["w_uv"][i]).T
            qr = torch.from_numpy(rope(p["q_rope"][b, i], L - 1, 10000.0))
            q = torch.cat([torch.from_numpy(p["q_nope"][b, i]), qr])
            ref = torch.nn.functional.scaled_dot_product_attention(
                q.view(1, 1, 1, -1), K.view(1, 1, L, -1), V.view(1, 1, L, -1),
                scale=p["softmax_scale"]).view(-1).numpy()
            assert np.max(np.abs(o[b, i] - ref)) < 1e-12 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("seed", [0, 3])
def test_absorbed_equals_non_absorbed(seed):
    p = random_problem(seed, H=4, d_c=32, d_rope=8, d_nope=16, d_v=16, lens=(64, 5, 130))
    assert rel_rms(run(mla.decode_absorbed, p), run(mla.decode, p)) < 1e-12


def test_absorbed_equals_non_absorbed_deepseek_shape_sampled():
    p = random_problem(21, H=8, d_c=512, d_rope=64, d_nope=128, d_v=128, lens=(3000,))
    pairs = [(0, 0), (0, 5)]
    a = run(mla.decode_absorbed, p, pairs=pairs)
    n = run(mla.decode, p, pairs=pairs, chunk=1024)
    assert rel_rms(a, n) < 1e-12


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorbed_heads_form_equals_per_head_forms(seed):
    """The all-heads matrix form equals the per-(sequence, head) absorbed form
    and the non-absorbed definition, on ragged random problems (an empty
    sequence included) and explicit query positions."""
    rng = np.random.default_rng(300 + seed)
    B, H, d_c, d_r, d_n, d_v = 4, 5, 24, 8, 12, 10
    lens = np.array([17, 1, 0, 40])
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]) + 3
    n = int(starts[-1] + lens[-1] + 2)
    C, R = rng.standard_normal((n, d_c)), rng.standard_normal((n, d_r))
    qn, qr = rng.standard_normal((B, H, d_n)), rng.standard_normal((B, H, d_r))
    wuk, wuv = rng.standard_normal((H, d_n, d_c)) / 5, rng.standard_normal((H, d_v, d_c)) / 5
    pos = np.array([16, 7, 3, 100])
    for q_pos in (None, pos):
        ref = mla.decode(C, R, starts, lens, qn, qr, wuk, wuv, 0.3, 10000.0, q_pos=q_pos)
        ref_abs = mla.decode_absorbed(C, R, starts, lens, qn, qr, wuk, wuv, 0.3, 10000.0, q_pos=q_pos)
        for b in range(B):
            P = lens[b] - 1 if q_pos is None else q_pos[b]
            s0, L = int(starts[b]), int(lens[b])
            got = mla.decode_absorbed_heads(C[s0:s0 + L], R[s0:s0 + L], qn[b], qr[b], wuk, wuv, 0.3, 10000.0, P)
            scale = max(np.sqrt(np.mean(ref ** 2)), 1e-300)
            assert np.max(np.abs(got - ref[b])) <= 1e-12 * scale
            assert np.max(np.abs(got - ref_abs[b])) <= 1e-12 * scale


def test_single_token_gives_value_of_that_token():
    p = random_problem(4, lens=(1, 1))
    o = run(mla.decode, p)
    for b in range(2):
        c0 = p["C"][p["seq_start"][b]]
        for i in range(3):
            assert np.allclose(o[b, i], p["w_uv"][i] @ c0, rtol=1e-13, atol=1e-13)


def test_zero_query_gives_mean_value():
    p = random_problem(6, lens=(11,))
    p["q_nope"][:] = 0
    p["q_rope"][:] = 0
    o = run(mla.decode, p)
    s0 = p["seq_start"][0]
    mean_c = p["C"][s0:s0 + 11].mean(axis=0)
    for i in range(3):
        assert np.allclose(o[0, i], p["w_uv"][i] @ mean_c, rtol=1e-12, atol=1e-13)


def test_identical_rows_give_that_value_for_any_query():
    p = random_problem(8, lens=(13,))
    s0 = p["seq_start"][0]
    p["C"][s0:s0 + 13] = p["C"][s0]
    o = run(mla.decode, p)
    for i in range(3):
        assert np.allclose(o[0, i], p["w_uv"][i] @ p["C"][s0], rtol=1e-12, atol=1e-13)


def test_dominant_positional_score_selects_its_token():
    """Plant, in one token's RoPE key, a large multiple of the query's rotated
    fastest pair (theta_0 = 1): that token must win the softmax. Fails if the
    positional term is dropped, or the query is rotated at the wrong position
    or in the wrong direction."""
    # L - 1 = 11: a sign error turns pair 0 by 22 rad = pi + 0.009 rad
    p = random_problem(10, H=2, lens=(12,))
    L, s0, tau = 12, int(p["seq_start"][0]), 7
    # both heads get the same rope query so one planted key serves both
    p["q_rope"][0, 1] = p["q_rope"][0, 0]
    q_rot = rope(p["q_rope"][0, 0], L - 1, 10000.0)
    key = np.zeros_like(q_rot)
    key[:2] = q_rot[:2] / (q_rot[:2] @ q_rot[:2])
    p["R"][s0 + tau] = 60.0 * key / p["softmax_scale"]
    o = run(mla.decode, p)
    for i in range(2):
        assert np.allclose(o[0, i], p["w_uv"][i] @ p["C"][s0 + tau], rtol=1e-9, atol=1e-9)
    # a query three positions later turns pair 0 by 3 rad (cos 3 < -0.98): the
    # planted score becomes strongly negative and the token no longer dominates
    o2 = run(mla.decode, p, q_pos=np.array([L + 2]))
    assert not np.allclose(o2[0, 0], p["w_uv"][0] @ p["C"][s0 + tau], rtol=1e-2, atol=1e-2)
    # rotating the query the other way (a sign error) also breaks dominance
    p_wrong = dict(p)
    p_wrong["q_rope"] = p["q_rope"].copy()
    p_wrong["q_rope"][0, 0] = rope(rope(p["q_rope"][0, 0], -(L - 1), 10000.0), -(L - 1), 10000.0)
    o3 = run(mla.decode, p_wrong)
    assert not np.allclose(o3[0, 0], p["w_uv"][0] @ p["C"][s0 + tau], rtol=1e-2, atol=1e-2)


def test_permuting_cached_rows_leaves_output_unchanged():
    p = random_problem(12, lens=(17,))
    o = run(mla.decode, p)
    s0 = int(p["seq_start"][0])
    perm = np.random.default_rng(0).permutation(17) + s0
    p["C"][s0:s0 + 17] = p["C"][perm]
    p["R"][s0:s0 + 17] = p["R"][perm]
    assert rel_rms(run(mla.decode, p), o) < 1e-12


def test_empty_sequence_gives_zero():
    p = random_problem(13, lens=(0, 5))
    o = run(mla.decode, p)
    assert np.all(o[0] == 0)
    assert rel_rms(o[1], brute_force(p)[1]) < 1e-12


def test_rows_outside_the_sequence_are_ignored():
    p = random_problem(14, lens=(6, 6), gap=3)
    o = run(mla.decode, p)
    # scribble over the gaps between sequences
    for b in range(2):
        s0, L = int(p["seq_start"][b]), int(p["seq_len"][b])
        p["C"][s0 + L:s0 + L + 3] = 1e6
        p["C"][max(0, s0 - 3):s0] = -1e6
    assert np.array_equal(run(mla.decode, p), o)


@pytest.mark.parametrize("seed", range(4))
def test_lse_merge_of_any_partition_equals_unsplit(seed):
    rng = np.random.default_rng(seed)
    L, dv = 97, 6
    s = rng.standard_normal(L) * 3
    V = rng.standard_normal((L, dv))
    full, lse_full = mla.partial_attention(s, V)
    e = np.exp(s - s.max())
    assert np.allclose(full, (e / e.sum()) @ V, rtol=1e-13)
    assert lse_full == pytest.approx(np.log(np.exp(s).sum()), rel=1e-13)
    cuts = np.sort(rng.choice(np.arange(0, L + 1), size=6, replace=True))
    bounds = [0] + list(cuts) + [L]
    parts = [mla.partial_attention(s[a:b], V[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
    assert np.allclose(mla.lse_merge(parts), full, rtol=1e-12, atol=1e-14)


def test_lse_merge_all_empty_is_zero():
    parts = [mla.partial_attention(np.zeros(0), np.zeros((0, 4)))] * 3
    assert np.array_equal(mla.lse_merge(parts), np.zeros(4))


# ------------------------------------------------------------------ append


def test_append_rows_positions_and_values():
    rng = np.random.default_rng(30)
    B, n_new, d_model, d_c, d_rope = 3, 4, 10, 6, 4
    h = rng.standard_normal((B, n_new, d_model))
    w_dkv = rng.standard_normal((d_c, d_model))
    w_kr = rng.standard_normal((d_rope, d_model))
    seq_start = np.array([0, 50, 20])
    seq_len = np.array([0, 7, 3])
    out = mla.append(h, w_dkv, w_kr, seq_start, seq_len, 10000.0, "f32", "f32")
    assert out["rows"].tolist() == [[0, 1, 2, 3], [57, 58, 59, 60], [23, 24, 25, 26]]
    assert out["seq_len"].tolist() == [4, 11, 7]
    for b in range(B):
        for j in range(n_new):
            p = seq_len[b] + j
            c = [sum(w_dkv[r, k] * h[b, j, k] for k in range(d_model)) for r in range(d_c)]
            assert np.allclose(out["c"][b, j], np.float32(c), rtol=0, atol=0)
            kr = w_kr @ h[b, j]
            kr_rot = []
            for jj in range(d_rope // 2):
                a = p * 10000.0 ** (-2.0 * jj / d_rope)
                kr_rot += [kr[2 * jj] * math.cos(a) - kr[2 * jj + 1] * math.sin(a),
                           kr[2 * jj] * math.sin(a) + kr[2 * jj + 1] * math.cos(a)]
            assert np.allclose(out["k_rope"][b, j], np.float32(kr_rot), rtol=1e-6, atol=1e-7)


def test_append_bf16_and_fp8_storage_rounding():
    rng = np.random.default_rng(31)
    h = rng.standard_normal((2, 1, 64))
    w_dkv = rng.standard_normal((32, 64)) / 8
    w_kr = rng.standard_normal((8, 64)) / 8
    o16 = mla.append(h, w_dkv, w_kr, [0, 10], [2, 5], 10000.0, "bf16", "bf16")
    exact = h[:, 0] @ w_dkv.T
    assert np.array_equal(o16["c"][:, 0], codecs.bf16_round(exact))
    o8 = mla.append(h, w_dkv, w_kr, [0, 10], [2, 5], 10000.0, "fp8", "bf16")
    for b in range(2):
        s = o8["scale"][b, 0]
        assert s == np.float32(np.abs(exact[b]).max() / 448.0)
        assert np.abs(o8["codes"][b, 0].view(np.int8)).max() <= 0x7E
        assert np.allclose(o8["c"][b, 0], exact[b], rtol=2.0 ** -4, atol=float(s) * 2.0 ** -10)
    assert np.array_equal(o8["k_rope"], o16["k_rope"])


def test_decode_rows_layout():
    """A row is [c_kv | k_rope] from byte 0: check by building bytes by hand."""
    d_c, d_r = 4, 2
    c = np.array([[1.0, -2.0, 0.5, 3.0], [0.25, 0.0, -1.0, 8.0]])
    r = np.array([[10.0, -10.0], [0.125, 2.0]])
    rows = np.zeros((2, 16), dtype=np.uint8)
    rows[:, :8] = codecs.bf16_encode(c).view(np.uint8).reshape(2, 8)
    rows[:, 8:12] = codecs.bf16_encode(r).view(np.uint8).reshape(2, 4)
    C, R = mla.decode_rows(rows, "bf16", "bf16", d_c, d_r)
    assert np.array_equal(C, c) and np.array_equal(R, r)
    rows8 = np.zeros((2, 16), dtype=np.uint8)
    rows8[:, :4] = codecs.e4m3_encode(c)
    rows8[:, 4:8] = codecs.bf16_encode(r).view(np.uint8).reshape(2, 4)
    C8, R8 = mla.decode_rows(rows8, "fp8", "bf16", d_c, d_r, scale=np.array([2.0, 0.5], np.float32))
    assert np.array_equal(C8, c * np.array([[2.0], [0.5]])) and np.array_equal(R8, r)


def test_synth_tiny_workload_end_to_end_consistent():
    """The tiny fp32 workload through the oracle: append 64 tokens from h, then
    decode at position 63; absorbed and non-absorbed forms agree."""
    case = mla_synth.workload("tiny_f32")
    h = case.h.astype(np.float64)
    ap = mla.append(h, case.w_dkv.astype(np.float64), case.w_kr.astype(np.float64),
                    case.seq_start, case.lens, case.rope_base, "f32", "f32")
    assert ap["rows"].tolist() == [list(range(64))]
    C = ap["c"].reshape(64, -1)
    R = ap["k_rope"].reshape(64, -1)
    args = (C, R, case.seq_start, ap["seq_len"], case.q_nope.astype(np.float64),
            case.q_rope.astype(np.float64), case.w_uk.astype(np.float64),
            case.w_uv.astype(np.float64), case.softmax_scale, case.rope_base)
    o = mla.decode(*args)
    assert o.shape == (1, 4, 16)
    assert rel_rms(mla.decode_absorbed(*args), o) < 1e-12
    assert case.softmax_scale == 1.0 / math.sqrt(24)
