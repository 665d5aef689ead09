"""Rotary position embedding (oracle, float64).  TEST INFRASTRUCTURE ONLY.

Follows tiny_agent ``generate.py``, function ``_rope_pos``: a head vector x of
size D is cut into halves x1 = x[:D/2], x2 = x[D/2:]; coordinate pair
(x1[d], x2[d]) is rotated by the angle pos * theta_d, giving
(x1 cos - x2 sin, x1 sin + x2 cos).  Each token uses its own absolute
position (Lab 07 section 2 says the rotation must use the same absolute
positions as the mask; pycraft-1 ``kv_cache.py`` header says a key is rotated
once at its true position and never again).

Reading (the pages never print the frequencies): theta_d = base ** (-2 d / D),
d = 0 .. D/2 - 1, the usual Llama choice.  ``base == 0`` means "already
rotated": the identity.

Pins: identity at position 0, norm preservation, relativity
<R(q,m),R(k,n)> = <R(q,m-n),k> and a unit-vector value check; and, for the
frequency schedule and the half-split pairing, a comparison with the
``transformers`` Llama rotary embedding within the error bound of its float32
tables (the colibri PR, "Tests done", checks against that model), including
exact-angle cases at positions up to 32767.  A wrong exponent, the
interleaved pairing or a flipped sign fails those bounds.
"""

import numpy as np


def inv_freq(head_dim: int, base: float) -> np.ndarray:
    """theta_d = base ** (-2 d / D) for d < D/2 (float64)."""
    d = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * d / head_dim)


def angles(pos, head_dim: int, base: float) -> np.ndarray:
    """(len(pos), D/2) angles pos * theta_d, float64."""
    pos = np.asarray(pos, dtype=np.float64).reshape(-1)
    return pos[:, None] * inv_freq(head_dim, base)[None, :]


def rotate(x, pos, base: float) -> np.ndarray:
    """Rotate x (T, H, D) at per-token absolute positions pos (T,).

    Returns a new float64 array; ``base == 0`` returns x unchanged (as float64).
    """
    x = np.asarray(x, dtype=np.float64)
    if base == 0:
        return x.copy()
    T, H, D = x.shape
    ang = angles(pos, D, base)                     # (T, D/2)
    cos = np.cos(ang)[:, None, :]                  # (T, 1, D/2)
    sin = np.sin(ang)[:, None, :]
    x1 = x[..., : D // 2]
    x2 = x[..., D // 2:]
    return np.concatenate((x1 * cos - x2 * sin, x1 * sin + x2 * cos), axis=-1)
