"""The seeded input recipe (mla_synth): length distributions, layout, the
long-context spike rows and reproducibility. CPU only; small cases, and the
lengths of the large workloads drawn the way the workloads draw them."""
import math

import numpy as np

import mla_synth

V3 = dict(H=128, d_c=512, d_rope=64, d_nope=128, d_v=128)


def _lens(name):
    spec = mla_synth.WORKLOADS[name]
    return mla_synth.draw_lens(np.random.default_rng(spec["seed"]), spec["lens"], spec["B"])


def test_ragged_lengths_are_uniform_integers_in_range():
    lens = _lens("v3_b32_ragged")
    assert lens.shape == (32,) and lens.dtype == np.int32
    assert lens.min() >= 4096 and lens.max() <= 8192
    assert int(lens.sum()) == 194934  # the bench workload's cache: 194934 rows x 1152 B
    big = mla_synth.draw_lens(np.random.default_rng(0), ("uniform", 4096, 8192), 200000)
    assert big.min() == 4096 and big.max() == 8192  # both ends inclusive
    assert abs(big.mean() - 6144) < 10


def test_fp8_lengths_are_log_uniform():
    lens = _lens("v3_b128_fp8")
    assert lens.shape == (128,) and lens.min() >= 1024 and lens.max() <= 32768
    big = mla_synth.draw_lens(np.random.default_rng(1), ("loguniform", 1024, 32768), 200000).astype(np.float64)
    # log-uniform: log2 of the length is uniform on [10, 15]
    l2 = np.log2(big)
    assert abs(l2.mean() - 12.5) < 0.01
    assert abs(np.mean(l2 < 11) - 0.2) < 0.01
    assert abs(big.mean() - (32768 - 1024) / math.log(32)) < 0.01 * big.mean()


def test_layout_rows_and_offsets():
    case = mla_synth.make_case("t", B=3, lens=("list", [5, 0, 9]), latent_dtype="bf16", rope_dtype="bf16",
                               act_dtype="bf16", seed=1, n_new=2, d_model=64, gap_rows=3, **V3)
    assert case.row_stride == 1152 and case.row_stride % 16 == 0
    assert list(case.seq_cap) == [7, 2, 11]
    assert list(case.seq_start) == [0, 10, 15]
    assert case.rows.shape == (29, 1152)  # every sequence is followed by its gap rows
    # rows past each sequence's length (capacity and gaps) are left zero
    for b, (s, L) in enumerate(zip(case.seq_start, case.lens)):
        assert not case.rows[s + L:s + case.seq_cap[b]].any()
    fp8 = mla_synth.make_case("t", B=1, lens=("list", [4]), latent_dtype="fp8", rope_dtype="bf16",
                              act_dtype="bf16", seed=1, **V3)
    assert fp8.row_stride == 640 and fp8.scale is not None and fp8.scale.shape == (4,)


def test_spike_rows_are_exactly_scaled():
    kw = dict(B=2, lens=("list", [1000, 3000]), latent_dtype="bf16", rope_dtype="bf16", act_dtype="bf16",
              seed=9, **V3)
    plain = mla_synth.make_case("p", **kw)
    spiky = mla_synth.make_case("s", spike_frac=0.01, spike_mult=8.0, **kw)
    a = plain.rows.view(np.uint16)
    b = spiky.rows.view(np.uint16)
    # bf16 bits to float: multiplying by 8 is exact, so spike rows are exactly 8x
    fa = (a.astype(np.uint32) << 16).view(np.float32)
    fb = (b.astype(np.uint32) << 16).view(np.float32)
    for s, L in zip(plain.seq_start, plain.lens):
        ra, rb = fa[s:s + L], fb[s:s + L]
        scaled = np.all(rb == 8 * ra, axis=1) & np.any(ra != 0, axis=1)
        same = np.all(rb == ra, axis=1)
        assert np.all(scaled | same)
        assert int(scaled.sum()) == round(0.01 * L)  # distinct rows, whole row (c_kv and k_rope)


def test_same_seed_same_case():
    kw = dict(B=2, lens=("uniform", 10, 40), latent_dtype="fp8", rope_dtype="bf16", act_dtype="bf16", seed=5, **V3)
    x, y = mla_synth.make_case("a", **kw), mla_synth.make_case("b", **kw)
    for k in ("rows", "scale", "lens", "q_nope", "q_rope", "w_uk", "w_uv"):
        assert np.array_equal(getattr(x, k), getattr(y, k)), k
    z = mla_synth.make_case("c", **dict(kw, seed=6))
    assert not np.array_equal(x.q_nope, z.q_nope)
