"""Attention masks (oracle).  TEST INFRASTRUCTURE ONLY.

Polarity: the functions here return True where attention is NOT allowed
("blocked"), the convention of Lab 07 section 2.

* ``offset_mask(t_new, pos)``: Lab 07 section 2, "The offset mask".  With pos
  tokens cached, new query i sits at absolute position pos + i and may see key
  j exactly when j <= pos + i; the mask has shape (t_new, pos + t_new).
  Pinned by the page's worked example (t_new = 2, pos = 3, fixture in
  tests/golden) and by a brute-force check of the pycraft-1 self-test shapes.
* ``window_blocked(qpos, kpos, W)``: the sliding clamp of the colibri PR
  "inkling: ring-buffer KV cache for sliding-window layers", section "What
  this does": a sliding layer scans keys from qpos - W + 1 to qpos, i.e. W keys
  including the query's own.  Equivalently (tiny_agent ``_append_chunk``,
  local mask) a key is visible when qpos - kpos < W.  W == 0 means a global
  layer (no clamp).  Pinned by the ring-versus-window equality check.
* ``padded_blocked(start, T, first)``: tinyllm ``kv_cache.py``,
  ``padded_causal_mask``: causal, keys before ``first`` hidden, the diagonal
  always kept so that no query row is empty.  Pinned by left-padding
  invariance.
* ``left_pad_blocked(qpos, kpos, first)``: the padding term of the same mask
  on its own (keys before ``first`` hidden except a query's own key), for
  combining with the offset mask and the sliding clamp.
"""

import numpy as np


def offset_mask(t_new: int, pos: int) -> np.ndarray:
    """(t_new, pos + t_new) bool, True where key j > pos + i (not allowed)."""
    i = np.arange(t_new)[:, None]
    j = np.arange(pos + t_new)[None, :]
    return j > pos + i


def window_blocked(qpos, kpos, window: int) -> np.ndarray:
    """True where key kpos lies outside the W-key window ending at qpos.

    Broadcasts qpos against kpos.  window == 0: nothing is blocked.
    """
    qpos = np.asarray(qpos)
    kpos = np.asarray(kpos)
    if window <= 0:
        return np.zeros(np.broadcast(qpos, kpos).shape, dtype=bool)
    return (qpos - kpos) >= window


def padded_blocked(start: int, T: int, first: int) -> np.ndarray:
    """(T, start + T) bool for one row whose first real key is ``first``.

    Blocked: j > start + i (causal), or j < first unless j == start + i.
    """
    i = np.arange(T)[:, None]
    j = np.arange(start + T)[None, :]
    qpos = start + i
    causal_blocked = j > qpos
    pad_blocked = (j < first) & (j != qpos)
    return causal_blocked | pad_blocked


def left_pad_blocked(qpos, kpos, first: int) -> np.ndarray:
    """True where key kpos is left padding (kpos < first) and not the
    query's own key.  Broadcasts qpos against kpos."""
    qpos = np.asarray(qpos)
    kpos = np.asarray(kpos)
    return (kpos < first) & (kpos != qpos)

