"""Plant plausible mistakes in the oracle (CPU only, via monkeypatch) and check
that the pins catch each one: a pin that passes with a broken oracle pins
nothing."""
import numpy as np
import pytest

import oracle.mla as omla
import oracle.rope as orope
from oracle import codecs
from tests import test_oracle_attention as ta
from tests import test_oracle_codecs as tc
from tests import test_oracle_rope as tr


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


ORIG_ROPE = orope.rope


def _rope_wrong_sign(x, pos, base):
    return ORIG_ROPE(x, -np.asarray(pos), base)


def _rope_halves_pairing(x, pos, base):
    """Pairs (j, j + d/2) instead of interleaved (2j, 2j+1)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = orope.rope_angles(pos, d, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


@pytest.mark.parametrize("bad", [_rope_wrong_sign, _rope_halves_pairing])
def test_rope_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(tr, "rope", bad)
    caught = _fails(tr.test_two_dims_rotate_by_p_radians_counterclockwise) or \
        _fails(tr.test_pair_frequencies)
    assert caught


def test_rope_mistake_in_decode_is_caught(monkeypatch):
    monkeypatch.setattr(omla, "rope", _rope_wrong_sign)
    assert _fails(ta.test_decode_vs_brute_force, 0) or _fails(ta.test_dominant_positional_score_selects_its_token)


def test_dropped_positional_term_is_caught(monkeypatch):
    monkeypatch.setattr(omla, "_query", lambda qn, qr, pos, base: np.concatenate([qn, 0 * qr]))
    assert _fails(ta.test_decode_vs_brute_force, 1)
    assert _fails(ta.test_dominant_positional_score_selects_its_token)


def test_query_position_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(omla, "_positions", lambda seq_len, q_pos: np.asarray(seq_len) if q_pos is None else np.asarray(q_pos))
    assert _fails(ta.test_decode_vs_brute_force, 2)


def test_missing_softmax_scale_is_caught(monkeypatch):
    orig = omla.decode

    def no_scale(*a, **k):
        a = list(a)
        a[8] = 1.0
        return orig(*a, **k)
    monkeypatch.setattr(omla, "decode", no_scale)
    assert _fails(ta.test_decode_vs_brute_force, 0)
    assert _fails(ta.test_decode_vs_torch_sdpa)


def test_transposed_value_projection_is_caught(monkeypatch):
    """Using W_UV's transpose only type-checks when d_v == d_c; the pins run
    square shapes too through the absorbed / brute-force checks."""
    orig = omla.decode

    def bad(C, R, seq_start, seq_len, q_nope, q_rope, w_uk, w_uv, *a, **k):
        return orig(C, R, seq_start, seq_len, q_nope, q_rope, w_uk, np.swapaxes(w_uv, 1, 2), *a, **k)
    monkeypatch.setattr(omla, "decode", bad)
    p = ta.random_problem(3, d_c=6, d_v=6)
    assert ta.rel_rms(ta.run(omla.decode, p), ta.brute_force(p)) > 1e-6


def test_append_ignoring_seq_len_is_caught(monkeypatch):
    orig = omla.append

    def bad(h, w_dkv, w_kr, seq_start, seq_len, *a):
        out = orig(h, w_dkv, w_kr, seq_start, np.zeros_like(np.asarray(seq_len)), *a)
        return out
    monkeypatch.setattr(omla, "append", bad)
    assert _fails(ta.test_append_rows_positions_and_values)


def test_fp8_wrong_bias_is_caught(monkeypatch):
    def bad_value(code):
        code = int(code) & 0xFF
        sign = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 0xF, code & 7
        if e == 0xF and m == 7:
            return float("nan")
        if e == 0:
            return sign * m / 8.0 * 2.0 ** (1 - 8)
        return sign * (1 + m / 8.0) * 2.0 ** (e - 8)
    monkeypatch.setattr(codecs, "E4M3_TABLE", np.array([bad_value(c) for c in range(256)]))
    assert _fails(tc.test_e4m3_table_matches_torch_and_definition)


def test_bf16_truncation_is_caught(monkeypatch):
    monkeypatch.setattr(codecs, "bf16_round",
                        lambda x: (np.asarray(x, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64))
    assert _fails(tc.test_bf16_encode_matches_torch_random)


def test_lse_merge_without_max_shift_weights_is_caught(monkeypatch):
    def bad(parts):
        return sum(np.asarray(o) for o, _ in parts) / len(parts)
    monkeypatch.setattr(omla, "lse_merge", bad)
    assert _fails(ta.test_lse_merge_of_any_partition_equals_unsplit, 1)


def _multi_window_off_by_one(C, R, seq_start, seq_len, q_nope, q_rope, w_uk, w_uv, softmax_scale, rope_base,
                             q_pos=None, triples=None, absorbed=False):
    """Query j sees one row too many (the next new token)."""
    B, Q = q_nope.shape[:2]
    L = np.asarray(seq_len, dtype=np.int64)
    P = L - 1 if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    out = np.zeros((B, Q, q_nope.shape[2], w_uv.shape[1]))
    for j in range(Q):
        back = max(Q - 2 - j, 0)
        out[:, j] = omla.decode(C, R, seq_start, np.maximum(L - back, 0), q_nope[:, j], q_rope[:, j], w_uk, w_uv,
                                softmax_scale, rope_base, q_pos=P - (Q - 1 - j))
    return out


def _multi_position_not_shifted(C, R, seq_start, seq_len, q_nope, q_rope, w_uk, w_uv, softmax_scale, rope_base,
                                q_pos=None, triples=None, absorbed=False):
    """Every query rotated at the last position instead of its own."""
    B, Q = q_nope.shape[:2]
    L = np.asarray(seq_len, dtype=np.int64)
    out = np.zeros((B, Q, q_nope.shape[2], w_uv.shape[1]))
    for j in range(Q):
        back = Q - 1 - j
        out[:, j] = omla.decode(C, R, seq_start, np.maximum(L - back, 0), q_nope[:, j], q_rope[:, j], w_uk, w_uv,
                                softmax_scale, rope_base, q_pos=L - 1)
    return out


@pytest.mark.parametrize("bad", [_multi_window_off_by_one, _multi_position_not_shifted])
def test_multi_query_mistakes_are_caught(monkeypatch, bad):
    from tests import test_oracle_multi as tm
    monkeypatch.setattr(omla, "decode_multi", bad)
    assert _fails(tm.test_matches_masked_matrix_form)
