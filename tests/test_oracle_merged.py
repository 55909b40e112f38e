"""Pins of oracle.merged (precomputed absorbed weights) against things other
than itself:

* the merged decode equals the definition (non-absorbed per-head attention,
  oracle.mla.decode, pinned on its own) followed by the output projection,
  with the no-RoPE query formed as W_Q x: folding the weights changes
  nothing in exact arithmetic ("02 — Multi-Latent Attention (MLA)", "Lo que
  MLA no es");
* the merged weights, element by element, from explicit loops on tiny sizes;
* with W_Q and W_O identities (d_x = d_nope, d_out = d_v, one head) the
  merged decode is the plain decode;
* planted mistakes (another head's W_O block, another head's W_Q, the RoPE
  term dropped) fail the first pin."""
import numpy as np
import pytest

import mla_synth
from oracle import merged as om
from oracle import mla as omla
from tests.helpers import act_to_f64, make, oracle_cache


def tiny(seed=5, B=3, H=4, lens=(7, 0, 12)):
    return make(B=B, H=H, d_c=32, d_rope=8, d_nope=16, d_v=16, lens=("list", list(lens)), latent_dtype="f32",
                rope_dtype="f32", act_dtype="f32", seed=seed)


def parts(case, d_x=24, d_out=20, seed=11):
    x, w_q, w_o = (np.asarray(v, np.float64) for v in mla_synth.merged_inputs(case, d_x, d_out, seed))
    C, R = oracle_cache(case)
    w_uk, w_uv = act_to_f64(case.w_uk, "f32"), act_to_f64(case.w_uv, "f32")
    q_rope = act_to_f64(case.q_rope, "f32")
    return x, w_q, w_o, C, R, w_uk, w_uv, q_rope


def definition_then_w_o(case, x, w_q, w_o, C, R, w_uk, w_uv, q_rope):
    q_nope = np.einsum("hnx,bx->bhn", w_q, x)
    o = omla.decode(C, R, case.seq_start, case.lens, q_nope, q_rope, w_uk, w_uv, case.softmax_scale,
                    case.rope_base)
    return np.stack([w_o @ o[b].reshape(-1) for b in range(case.B)])


@pytest.mark.parametrize("seed", [5, 6])
def test_merged_decode_equals_definition_then_output_projection(seed):
    case = tiny(seed)
    x, w_q, w_o, C, R, w_uk, w_uv, q_rope = parts(case, seed=seed + 100)
    a = om.merge_query_weight(w_q, w_uk)
    bm = om.merge_output_weight(w_o, w_uv)
    y = om.decode_merged(C, R, case.seq_start, case.lens, x, q_rope, a, bm, case.softmax_scale, case.rope_base)
    ref = definition_then_w_o(case, x, w_q, w_o, C, R, w_uk, w_uv, q_rope)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    assert np.all(y[1] == 0)  # the empty sequence


def test_merged_weights_by_explicit_loops():
    rng = np.random.default_rng(3)
    H, d_nope, d_c, d_x, d_v, d_out = 2, 3, 4, 5, 3, 4
    w_q = rng.standard_normal((H, d_nope, d_x))
    w_uk = rng.standard_normal((H, d_nope, d_c))
    w_uv = rng.standard_normal((H, d_v, d_c))
    w_o = rng.standard_normal((d_out, H * d_v))
    a = om.merge_query_weight(w_q, w_uk)
    bm = om.merge_output_weight(w_o, w_uv)
    assert a.shape == (H, d_c, d_x) and bm.shape == (d_out, H * d_c)
    for i in range(H):
        for c in range(d_c):
            for xx in range(d_x):
                want = sum(w_uk[i, n, c] * w_q[i, n, xx] for n in range(d_nope))
                assert abs(a[i, c, xx] - want) <= 1e-12
    for o in range(d_out):
        for i in range(H):
            for c in range(d_c):
                want = sum(w_o[o, i * d_v + v] * w_uv[i, v, c] for v in range(d_v))
                assert abs(bm[o, i * d_c + c] - want) <= 1e-12


def test_identity_projections_reduce_to_plain_decode():
    case = tiny(7, B=2, H=1, lens=(9, 30))
    C, R = oracle_cache(case)
    w_uk, w_uv = act_to_f64(case.w_uk, "f32"), act_to_f64(case.w_uv, "f32")
    q_nope, q_rope = act_to_f64(case.q_nope, "f32"), act_to_f64(case.q_rope, "f32")
    w_q = np.eye(case.d_nope)[None]
    w_o = np.eye(case.d_v)
    y = om.decode_merged(C, R, case.seq_start, case.lens, q_nope[:, 0, :], q_rope, om.merge_query_weight(w_q, w_uk),
                         om.merge_output_weight(w_o, w_uv), case.softmax_scale, case.rope_base)
    o = omla.decode(C, R, case.seq_start, case.lens, q_nope, q_rope, w_uk, w_uv, case.softmax_scale, case.rope_base)
    assert np.max(np.abs(y - o[:, 0, :])) <= 1e-12 * np.max(np.abs(o))


def test_factored_form_equals_merged():
    case = tiny(8)
    x, w_q, w_o, C, R, w_uk, w_uv, q_rope = parts(case, seed=108)
    y = om.decode_merged(C, R, case.seq_start, case.lens, x, q_rope, om.merge_query_weight(w_q, w_uk),
                         om.merge_output_weight(w_o, w_uv), case.softmax_scale, case.rope_base)
    f = om.decode_factored(C, R, case.seq_start, case.lens, x, q_rope, w_q, w_uk, w_uv, w_o, case.softmax_scale,
                           case.rope_base)
    assert np.max(np.abs(y - f)) <= 1e-12 * np.max(np.abs(f))
    sub = om.decode_merged(C, R, case.seq_start, case.lens, x, q_rope, om.merge_query_weight(w_q, w_uk),
                           om.merge_output_weight(w_o, w_uv), case.softmax_scale, case.rope_base, seqs=[2])
    assert np.all(sub[:2] == 0) and np.array_equal(sub[2], y[2])


# ------------------------------------------------------- planted mistakes

ORIG_MQ, ORIG_MO, ORIG_ROPE = om.merge_query_weight, om.merge_output_weight, om.rope


def _mo_next_head_block(w_o, w_uv):
    H, d_v, _ = w_uv.shape
    return np.concatenate([w_o[:, ((i + 1) % H) * d_v:((i + 1) % H + 1) * d_v] @ w_uv[i] for i in range(H)], axis=1)


def _mq_next_head(w_q, w_uk):
    H = w_q.shape[0]
    return np.stack([w_uk[i].T @ w_q[(i + 1) % H] for i in range(H)])


def _rope_zero(x, pos, base):
    return np.zeros_like(np.asarray(x, dtype=np.float64))


@pytest.mark.parametrize("target,bad", [("merge_output_weight", _mo_next_head_block),
                                        ("merge_query_weight", _mq_next_head), ("rope", _rope_zero)])
def test_planted_mistakes_fail_the_definition_pin(monkeypatch, target, bad):
    monkeypatch.setattr(om, target, bad)
    with pytest.raises(AssertionError):
        test_merged_decode_equals_definition_then_output_projection(5)
