"""Softmax attention over an explicit key selection (oracle, float64).
TEST INFRASTRUCTURE ONLY.

``softmax_attend`` is the one place the oracle turns scores into an output.
It follows tiny_agent ``generate.py`` ``_append_chunk`` (scores times
1/sqrt(D), masked entries excluded, softmax, probability-weighted sum of V) and
its grouped-query rule: query head h reads KV head h // (Hq / Hkv) (the query
is viewed per KV head, pycraft-1 ``kv_cache.py`` header: storage is
pre-expansion and re-expanded on read).  Differences from that page, on
purpose: everything is float64 and masked keys are removed instead of being
filled with a large negative number (identical in exact arithmetic).

Scores are formed as an elementwise product summed over D for each key on its
own, and the weighted sum runs over keys in the order given, so two callers
that pass the same keys in the same order get bit-identical results no matter
how many other keys they looked at.  The ring-versus-window check relies on
this.

Pins: closed forms (zero query -> mean of visible V; a single visible key ->
that V; identical keys -> mean V) and a cross-check against
``torch.nn.functional.scaled_dot_product_attention`` in float64 with
repeat-expanded K/V and an explicit boolean mask (tests).

``full_forward`` is one sequence run without any cache: positions 0..T-1, a
T x T causal mask written from its definition (key j visible to query i iff
j <= i), the sliding clamp, and optionally tinyllm's left-padding rule.
"""

import math

import numpy as np

from . import mask as _mask
from . import rope as _rope


def softmax_attend(q, K, V, scale=None) -> np.ndarray:
    """Attention of one query token over an explicit list of keys.

    q: (Hq, D) rotated query; K, V: (n, Hkv, D) rotated keys / values of the
    visible keys, n >= 1, in the order to sum.  Returns (Hq, D) float64.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, D = q.shape
    n, Hkv, _ = K.shape
    if n == 0:
        raise ValueError("a query must see at least one key")
    if Hq % Hkv:
        raise ValueError("n_q_head must be a multiple of n_kv_head")
    rep = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((Hq, D), dtype=np.float64)
    for g in range(Hkv):
        Kg = np.ascontiguousarray(K[:, g, :])                     # (n, D)
        Vg = V[:, g, :]
        qg = q[g * rep:(g + 1) * rep]                             # (rep, D)
        # s[j, r] = sum_d K[j, d] q[r, d]: each key's sum over D on its own
        s = (Kg[:, None, :] * qg[None, :, :]).sum(axis=2) * scale  # (n, rep)
        for r in range(rep):
            p = np.exp(s[:, r] - s[:, r].max())
            p = p / p.sum()
            out[g * rep + r] = (p[:, None] * Vg).sum(axis=0)
    return out


def attend_rows(qrot, Krot, V, blocked) -> np.ndarray:
    """qrot (n, Hq, D); Krot, V (T, Hkv, D); blocked (n, T) bool -> (n, Hq, D)."""
    n = qrot.shape[0]
    out = np.empty((n,) + qrot.shape[1:], dtype=np.float64)
    for i in range(n):
        sel = np.flatnonzero(~blocked[i])
        out[i] = softmax_attend(qrot[i], Krot[sel], V[sel])
    return out


def full_forward(q, k, v, window: int = 0, base: float = 10000.0, first=None):
    """One sequence, no cache: q (T, Hq, D), raw k, v (T, Hkv, D) -> (T, Hq, D).

    Positions are 0..T-1.  ``first``: index of the first real token of a
    left-padded sequence (keys before it hidden, the diagonal kept).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T = q.shape[0]
    pos = np.arange(T)
    qrot = _rope.rotate(q, pos, base)
    krot = _rope.rotate(k, pos, base)
    i = pos[:, None]
    j = pos[None, :]
    if first is None:
        blocked = j > i
    else:
        blocked = _mask.padded_blocked(0, T, int(first))
    blocked = blocked | _mask.window_blocked(i, j, window)
    return attend_rows(qrot, krot, v, blocked)
