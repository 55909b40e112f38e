"""Pins for oracle.mla.decode_multi (several new query tokens per sequence,
causal among them) against a masked matrix form written independently of the
per-query truncation, special cases and invariants."""
import math

import numpy as np

from oracle import mla


def problem(seed, Q, H=3, d_c=6, d_rope=4, d_nope=5, d_v=7, lens=(1, 3, 4, 9), gap=2):
    rng = np.random.default_rng(seed)
    B = len(lens)
    starts, acc = [], gap
    for L in lens:
        starts.append(acc)
        acc += L + gap
    return dict(
        C=rng.standard_normal((acc, d_c)), R=rng.standard_normal((acc, d_rope)),
        seq_start=np.array(starts), seq_len=np.array(lens),
        q_nope=rng.standard_normal((B, Q, H, d_nope)), q_rope=rng.standard_normal((B, Q, H, d_rope)),
        w_uk=rng.standard_normal((H, d_nope, d_c)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c),
        softmax_scale=1.0 / math.sqrt(d_nope + d_rope), rope_base=10000.0)


def run(p, **kw):
    return mla.decode_multi(p["C"], p["R"], p["seq_start"], p["seq_len"], p["q_nope"], p["q_rope"], p["w_uk"],
                            p["w_uv"], p["softmax_scale"], p["rope_base"], **kw)


def masked_form(p, q_pos=None):
    """All Q queries of a sequence at once: a [Q x L] score matrix, the causal
    mask (query j sees token t iff t <= L - Q + j), one softmax per row. K and
    V are rebuilt per head; RoPE by its definition on pairs (2k, 2k+1)."""
    B, Q, H, d_nope = p["q_nope"].shape
    d_rope = p["q_rope"].shape[3]
    d_v = p["w_uv"].shape[1]
    out = np.zeros((B, Q, H, d_v))
    for b in range(B):
        L, r0 = int(p["seq_len"][b]), int(p["seq_start"][b])
        last = L - 1 if q_pos is None else int(q_pos[b])
        Cb, Rb = p["C"][r0:r0 + L], p["R"][r0:r0 + L]
        for i in range(H):
            K = np.concatenate([Cb @ p["w_uk"][i].T, Rb], axis=1)
            V = Cb @ p["w_uv"][i].T
            qs = np.zeros((Q, d_nope + d_rope))
            for j in range(Q):
                pos = last - (Q - 1 - j)
                x = p["q_rope"][b, j, i]
                ang = pos * p["rope_base"] ** (-2.0 * np.arange(d_rope // 2) / d_rope)
                rot = np.empty(d_rope)
                rot[0::2] = x[0::2] * np.cos(ang) - x[1::2] * np.sin(ang)
                rot[1::2] = x[0::2] * np.sin(ang) + x[1::2] * np.cos(ang)
                qs[j] = np.concatenate([p["q_nope"][b, j, i], rot])
            S = p["softmax_scale"] * qs @ K.T                                # [Q, L]
            allowed = np.arange(L)[None, :] <= (L - Q + np.arange(Q))[:, None]
            for j in range(Q):
                if not allowed[j].any():
                    continue
                s = np.where(allowed[j], S[j], -np.inf)
                e = np.exp(s - s[allowed[j]].max())
                out[b, j, i] = V.T @ (e / e.sum())
    return out


def test_matches_masked_matrix_form():
    for Q in (1, 2, 3, 5):
        p = problem(10 + Q, Q)
        np.testing.assert_allclose(run(p), masked_form(p), rtol=0, atol=1e-12)


def test_explicit_positions():
    p = problem(20, 3)
    q_pos = np.array([7, 2, 100, 12])
    np.testing.assert_allclose(run(p, q_pos=q_pos), masked_form(p, q_pos=q_pos), rtol=0, atol=1e-12)


def test_one_query_is_the_single_token_decode():
    p = problem(21, 1)
    single = mla.decode(p["C"], p["R"], p["seq_start"], p["seq_len"], p["q_nope"][:, 0], p["q_rope"][:, 0],
                        p["w_uk"], p["w_uv"], p["softmax_scale"], p["rope_base"])
    np.testing.assert_array_equal(run(p)[:, 0], single)


def test_last_query_sees_the_whole_cache():
    p = problem(22, 4, lens=(6, 9))
    single = mla.decode(p["C"], p["R"], p["seq_start"], p["seq_len"], p["q_nope"][:, 3], p["q_rope"][:, 3],
                        p["w_uk"], p["w_uv"], p["softmax_scale"], p["rope_base"])
    np.testing.assert_allclose(run(p)[:, 3], single, rtol=0, atol=1e-13)


def test_causal_later_rows_do_not_matter():
    """Query j of a sequence of length L ignores rows L - Q + j + 1 .. L - 1."""
    p = problem(23, 4, lens=(9,))
    base = run(p)
    r0, L = int(p["seq_start"][0]), 9
    p["C"][r0 + L - 1] += 100.0  # the last new token: only the last query sees it
    p["R"][r0 + L - 1] -= 50.0
    moved = run(p)
    np.testing.assert_array_equal(moved[0, :3], base[0, :3])
    assert np.max(np.abs(moved[0, 3] - base[0, 3])) > 1e-3


def test_queries_that_see_nothing_give_zero():
    p = problem(24, 4, lens=(2, 0))
    o = run(p)
    assert np.all(o[0, :2] == 0) and np.all(o[1] == 0)
    assert np.all(np.abs(o[0, 2:]) > 0)


def test_absorbed_equals_definition():
    p = problem(25, 3)
    np.testing.assert_allclose(run(p, absorbed=True), run(p), rtol=0, atol=1e-12)


def test_triples_match_full_output():
    p = problem(26, 3)
    full = run(p)
    tri = [(0, 0, 1), (3, 2, 0), (2, 1, 2)]
    np.testing.assert_allclose(run(p, triples=tri), np.stack([full[b, j, i] for b, j, i in tri]), rtol=0, atol=0)
