"""Rotary position embedding for the decoupled RoPE key and query.

Test infrastructure only (see the package docstring).

"02 — Multi-Latent Attention (MLA)", section "Truco de codificación
posicional": the key is split into a rotary part of small width d_h^R (about
64), cached as it is, and a non-rotary part recovered from the latent; the
rotation itself is only referenced there, not defined. The "DeepSeek MLA" card
(section on the RoPE problem) says RoPE is applied to Q and K by position.

Reading taken (the pages leave the pairing and frequencies open): the original
rotary scheme with interleaved pairs. For x in R^d (d even) at absolute
position p (starting at 0) and j = 0 .. d/2 - 1:

    theta_j = base ** (-2 j / d)
    (x[2j], x[2j+1]) <- (x[2j] cos(p theta_j) - x[2j+1] sin(p theta_j),
                         x[2j] sin(p theta_j) + x[2j+1] cos(p theta_j))

Everything is fp64.
"""

import numpy as np


def rope_angles(pos, d, base):
    """Angles p * theta_j, shape pos.shape + (d/2,), in fp64."""
    if d % 2:
        raise ValueError("RoPE width must be even")
    j = np.arange(d // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * j / d)
    return np.asarray(pos, dtype=np.float64)[..., None] * theta


def rope(x, pos, base):
    """Rotate the last axis of ``x`` (width d) at position(s) ``pos``.

    ``pos`` broadcasts against ``x.shape[:-1]``."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = rope_angles(pos, d, base)
    cos, sin = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = x0 * cos - x1 * sin
    out[..., 1::2] = x0 * sin + x1 * cos
    return out
