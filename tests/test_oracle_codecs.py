"""Pins for oracle.codecs: bf16 and OCP fp8 e4m3fn against PyTorch's CPU casts
(a library routine independent of the oracle) and against the formats'
defining values."""
import numpy as np
import pytest
import torch

from oracle import codecs


def _torch_bf16_bits(x):
    # torch rounds fp32 -> bf16 once; inputs here are fp32-representable
    x32 = np.asarray(x, dtype=np.float32)
    assert np.array_equal(x32.astype(np.float64), np.asarray(x, dtype=np.float64))
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_encode_matches_torch_random():
    rng = np.random.default_rng(123)
    x = np.concatenate([rng.standard_normal(500_000) * 10.0 ** rng.integers(-30, 30, 500_000),
                        rng.standard_normal(500_000)]).astype(np.float32).astype(np.float64)
    assert np.array_equal(codecs.bf16_encode(x), _torch_bf16_bits(x))


def test_bf16_rounds_the_exact_value_once():
    # 1 + 2^-8 + 2^-30 lies just above the tie between 1 and 1 + 2^-7: the
    # nearest bf16 is 1 + 2^-7. (Rounding through fp32 first would land on the
    # tie and then go to the even 1.0.)
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert codecs.bf16_round(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert codecs.bf16_round(np.array([-x]))[0] == -(1.0 + 2.0 ** -7)


def test_bf16_encode_ties_and_edges():
    one = 1.0
    ulp = 2.0 ** -7
    x = np.array([0.0, -0.0, one, one + ulp / 2, one + 3 * ulp / 2, -(one + ulp / 2),
                  2.0 ** -126, 2.0 ** -133, 3 * 2.0 ** -134, 2.0 ** -149, 3.3895313892515355e38,
                  65504.0, 0.1, -0.1, 1 / 3]).astype(np.float32).astype(np.float64)
    assert np.array_equal(codecs.bf16_encode(x), _torch_bf16_bits(x))
    # ties to even, by hand: 1 + ulp/2 -> 1 (even), 1 + 3ulp/2 -> 1 + 2ulp
    assert codecs.bf16_round(np.array([one + ulp / 2]))[0] == one
    assert codecs.bf16_round(np.array([one + 3 * ulp / 2]))[0] == one + 2 * ulp


def test_bf16_decode_roundtrip_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = codecs.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(v[fin], ref[fin])
    assert np.array_equal(np.isnan(v), np.isnan(ref))
    # every finite non-zero pattern re-encodes to itself (zero: both signs)
    nz = fin & (v != 0)
    assert np.array_equal(codecs.bf16_encode(v[nz]), bits[nz])


def test_e4m3_table_matches_torch_and_definition():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    tab = codecs.E4M3_TABLE
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(tab[fin], ref[fin])
    # defining values of the format
    assert np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    assert tab[0x7E] == 448.0 and tab[0x38] == 1.0 and tab[0x01] == 2.0 ** -9
    assert tab[0x08] == 2.0 ** -6 and tab[0x07] == 7 * 2.0 ** -9 and tab[0xB8] == -1.0
    assert np.isnan(tab).sum() == 2  # no infinities, two NaN codes


def test_e4m3_encode_in_range_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-448, 448, 100_000),
                        rng.standard_normal(100_000) * 2.0 ** rng.integers(-12, 8, 100_000)])
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = codecs.e4m3_encode(x)
    # torch keeps -0 for tiny negatives, as does the oracle
    assert np.array_equal(got, ref)


def test_e4m3_saturation_and_ties():
    # beyond the largest finite value the oracle saturates (the format has no inf)
    x = np.array([449.0, 463.9, 464.0, 1000.0, -1e9])
    assert list(codecs.e4m3_round(x)) == [448.0, 448.0, 448.0, 448.0, -448.0]
    # ties to even: between 1.0 (mantissa 0) and 1.125 (mantissa 1) -> 1.0;
    # between 1.125 and 1.25 (mantissa 2) -> 1.25
    assert codecs.e4m3_round(np.array([1.0625]))[0] == 1.0
    assert codecs.e4m3_round(np.array([1.1875]))[0] == 1.25
    # subnormal spacing 2^-9: 1.5 * 2^-9 is a tie between codes 1 and 2 -> 2
    assert codecs.e4m3_round(np.array([1.5 * 2.0 ** -9]))[0] == 2 * 2.0 ** -9
    assert codecs.e4m3_round(np.array([0.4 * 2.0 ** -9]))[0] == 0.0


def test_e4m3_token_scale_rule():
    rng = np.random.default_rng(3)
    c = rng.standard_normal(512)
    s = codecs.e4m3_token_scale(c)
    assert s == np.float32(np.abs(c).max() / 448.0)
    q = codecs.e4m3_decode(codecs.e4m3_encode(c / np.float64(s))) * np.float64(s)
    # the largest element round-trips to within one fp8 step of itself
    k = np.argmax(np.abs(c))
    assert abs(q[k] - c[k]) <= 2.0 ** -3 * abs(c[k])
    assert codecs.e4m3_token_scale(np.zeros(8)) == np.float32(1.0)


def test_e4m3_quantisation_error_bound():
    """Each element of a quantised row is within half a step of its value:
    |x - x^| <= 2^-4 |x| for normals, <= s 2^-10 in the subnormal range."""
    rng = np.random.default_rng(11)
    for _ in range(20):
        c = rng.standard_normal(512) * 10.0 ** rng.uniform(-3, 3)
        s = np.float64(codecs.e4m3_token_scale(c))
        y = c / s
        x_hat = codecs.e4m3_decode(codecs.e4m3_encode(y)) * s
        err = np.abs(x_hat - c)
        normal = np.abs(y) >= 2.0 ** -6
        assert np.all(err[normal] <= 2.0 ** -4 * np.abs(c[normal]) * (1 + 1e-12))
        assert np.all(err[~normal] <= s * 2.0 ** -10 * (1 + 1e-12))


@pytest.mark.parametrize("x", [0.0, 1.0, -2.5, 3.0e-39])
def test_f32_roundtrip(x):
    assert codecs.f32_decode(codecs.f32_encode(np.array([x])))[0] == np.float32(x)
