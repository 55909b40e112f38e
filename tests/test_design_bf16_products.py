"""Why the bf16 cache is widened to fp16 before the matrix-core products,
emulated in fp64 on the oracle's own inputs (CPU only; no part of the
library is involved), against the bf16 tolerance max|err| / rms(ref) <= 2e-2.

The score products need both operands in one type. Reading the cached bf16
tile as it is would put the absorbed query q~ = [W_UK^T q_nope ; RoPE(q_rope)]
(scaled) in bf16 too: 8 significant bits instead of fp16's 11. That misses
the tolerance once the latents carry outliers (1 % of the rows scaled by 8,
as in the long-context workload) or a larger spread (std 8), because a score
error grows with |q~| |c_t| and the softmax turns it into a relative error
of the weights. fp16 q~ against the exact bf16 values (the widened tile)
meets it with a wide margin in the same cases. The softmax weights alone in
bf16 would still meet it; it is the query that needs fp16."""
import numpy as np

import mla_synth
from oracle import codecs
from oracle import mla as omla
from oracle.rope import rope
from tests.helpers import TOL_BF16_REL, act_to_f64, oracle_cache

LOG2E = 1.4426950408889634


def _f16(x):
    """Nearest fp16 value (10 fraction bits, gradual underflow below 2^-14)."""
    return codecs._round_to_grid(x, 10, -14)


def _emulate(lens, seed, round_q, round_p, **kw):
    """Scores from q~ rounded by round_q against the exact cached values, the
    weights 2^(s - max) rounded by round_p, the latent-space output rounded
    to fp16 (the split partials), then W_UV in fp64."""
    case = mla_synth.make_case("bf16_products", H=128, d_c=512, d_rope=64, d_nope=128, d_v=128, B=len(lens),
                               lens=("list", lens), latent_dtype="bf16", rope_dtype="bf16", act_dtype="bf16",
                               seed=seed, **kw)
    C, R = oracle_cache(case)
    qn, qr = act_to_f64(case.q_nope, "bf16"), act_to_f64(case.q_rope, "bf16")
    wuk, wuv = act_to_f64(case.w_uk, "bf16"), act_to_f64(case.w_uv, "bf16")
    ref = omla.decode_absorbed(C, R, case.seq_start, case.lens, qn, qr, wuk, wuv, case.softmax_scale, case.rope_base)
    out = np.zeros_like(ref)
    for b, L in enumerate(int(x) for x in case.lens):
        s0 = int(case.seq_start[b])
        K, KR = C[s0:s0 + L], R[s0:s0 + L]
        for h in range(case.H):
            qt = wuk[h].T @ qn[b, h] * case.softmax_scale * LOG2E
            q_r = rope(qr[b, h], L - 1, case.rope_base) * case.softmax_scale * LOG2E
            s = K @ round_q(qt) + KR @ round_q(q_r)
            p = np.exp2(s - s.max())
            out[b, h] = wuv[h] @ _f16((round_p(p) @ K) / p.sum())
    return float(np.abs(out - ref).max() / np.sqrt(np.mean(ref ** 2)))


def _exact(x):
    return x


def test_emulation_matches_the_oracle_up_to_the_fp16_partials():
    assert _emulate([1, 7, 31], 5, _exact, lambda p: p) < 1e-3  # only the fp16 partials remain


def test_bf16_query_misses_the_tolerance_with_outlier_rows():
    kw = dict(spike_frac=0.01, spike_mult=8.0)
    assert _emulate([4096], 3, codecs.bf16_round, _f16, **kw) > TOL_BF16_REL
    assert _emulate([4096], 3, _f16, _f16, **kw) < TOL_BF16_REL / 2
    assert _emulate([4096], 3, _f16, codecs.bf16_round, **kw) < TOL_BF16_REL / 2


def test_bf16_query_misses_the_tolerance_with_wider_latents():
    assert _emulate([2048, 3000], 7, codecs.bf16_round, _f16, cache_std=8.0) > TOL_BF16_REL
    assert _emulate([2048, 3000], 7, _f16, _f16, cache_std=8.0) < TOL_BF16_REL / 2
