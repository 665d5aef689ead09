"""The incremental definition of cached GQA attention with append (oracle).
TEST INFRASTRUCTURE ONLY.

``OracleCache`` holds no cache in the GPU sense: per layer and row it keeps
the list of raw (pre-RoPE) keys and values of every real token appended so
far, plus ``lens`` (tokens per row).  One step is

1. capacity check before anything changes: if any row would pass
   ``max_len``, raise ``CacheFull`` and leave the state untouched (tiny_agent
   ``append``; pycraft-1 ``KVCache.update``; Lab 07 Tips);
2. per layer, in order: append the raw k, v of the valid tokens (token i of
   row b is valid iff i < n_new[b], tiny_agent ``_append_chunk``), then attend:
   query i of row b sits at pos = lens[b] + i, every cached key j is rotated
   again at position j, the query at pos, and the query sees key j iff the
   offset mask allows it (j <= pos, Lab 07 section 2) and, on a sliding layer,
   pos - j < W (colibri PR, "What this does");
3. after every layer has run, ``lens += n_new`` once (pycraft-1
   ``KVCache.update`` docstring and ``advance``; Lab 07 "Given"; tinyllm
   ``end_step``).

Hybrid layer groups (tiny_agent ``generate.py`` module docstring and
``_append_chunk``): a layer may have a joint partner ``joint[l] = j`` (an
earlier layer, the group's global store); its queries then attend, with ONE
softmax, to layer j's keys under layer j's rules (all positions up to the
query: a global store) together with its own keys under its own rules (the
last W positions: the per-layer ring).  Layer j must have been appended in
the same step first; its own outputs are not part of the group's result.

Left padding (tinyllm ``kv_cache.py``: ``padded_causal_mask`` and
``SlotKVCache``): a row may start with ``first[b]`` pad tokens; keys before
``first[b]`` are hidden from every query of the row except the pad's own
query, which sees only itself.  ``set_first`` sets it, ``reset`` clears it,
``admit`` copies whole rows (history, length, first) from another cache, as
the slot cache admits a finished batched prefill.

Padded queries (i >= n_new[b]) and idle rows (n_new[b] == 0) produce exact
zeros: the pages leave these outputs unspecified (tiny_agent says garbage);
zero is this implementation's reading.  Parity status: pinned by the
chunked-equals-single, incremental-equals-full, ring-equals-window, offset
mask, closed-form and library cross-checks in tests/test_oracle_*.py.

``slot_indices`` is the integer addressing model the GPU must reproduce bit
for bit (tiny_agent ``_append_chunk``: padding goes to the scratch index;
sliding rings keep the last W real tokens of a chunk at pos % W and send the
rest to scratch; colibri PR "How it works": a layer is a ring iff
0 < W < max_len).  Pinned by the exhaustive index simulation.

``RingModel`` is an explicit W-slot ring store with a scratch slot, written
stage-then-commit and read by a clamped scan, as the colibri PR describes.  It
exists only to check the oracle against a second, independent formulation
(the ring-equals-window check); the GPU path is compared with
``OracleCache``.
"""

import math

import numpy as np

from . import attention as _attn
from . import mask as _mask
from . import rope as _rope


class CacheFull(ValueError):
    """A step would write past max_len; nothing was changed."""


def is_ring(window: int, max_len: int, use_ring: bool = True) -> bool:
    """colibri PR, kv_ring_rows: a sliding layer is a ring iff 0 < W < max_len."""
    return bool(use_ring) and 0 < window < max_len


def ring_rows(window: int, max_len: int, use_ring: bool = True) -> int:
    """Rows of a layer's cache, excluding the scratch row."""
    return window if is_ring(window, max_len, use_ring) else max_len


def slot_indices(lens, n_new, C: int, window: int, max_len: int,
                 use_ring: bool = True) -> np.ndarray:
    """(B, C) int64 cache row written by token i of row b.

    Full layout: pos if valid else max_len (scratch).
    Ring layout: pos % W if valid and pos >= lens + n_new - W (the last W
    real tokens of the chunk), else W (scratch).
    """
    lens = np.asarray(lens, dtype=np.int64)
    n_new = np.asarray(n_new, dtype=np.int64)
    i = np.arange(C, dtype=np.int64)[None, :]
    pos = lens[:, None] + i
    valid = i < n_new[:, None]
    if is_ring(window, max_len, use_ring):
        new_lens = lens + n_new
        keep = valid & (pos >= new_lens[:, None] - window)
        return np.where(keep, pos % window, window)
    return np.where(valid, pos, max_len)


class OracleCache:
    """No-cache reference for a stack of attention layers over B rows."""

    def __init__(self, batch: int, n_q_head: int, n_kv_head, head_dim: int,
                 max_len: int, window, rope_base: float = 10000.0, joint=None):
        n_kv_head = [int(h) for h in n_kv_head]
        window = [int(w) for w in window]
        if len(n_kv_head) != len(window):
            raise ValueError("n_kv_head and window need one entry per layer")
        joint = [-1] * len(window) if joint is None else [int(j) for j in joint]
        if len(joint) != len(window):
            raise ValueError("joint needs one entry per layer")
        for l, j in enumerate(joint):
            if j >= 0 and (j >= l or n_kv_head[j] != n_kv_head[l] or joint[j] >= 0):
                raise ValueError("a joint partner is an earlier layer with the same KV heads "
                                 "and no partner of its own")
        self.joint = joint
        self.batch = int(batch)
        self.n_layer = len(n_kv_head)
        self.n_q_head = int(n_q_head)
        self.n_kv_head = n_kv_head
        self.head_dim = int(head_dim)
        self.max_len = int(max_len)
        self.window = window
        self.rope_base = float(rope_base)
        self.lens = np.zeros(self.batch, dtype=np.int64)
        self.first = np.zeros(self.batch, dtype=np.int64)
        D = self.head_dim
        self.hist_k = [[np.zeros((0, h, D)) for _ in range(self.batch)] for h in n_kv_head]
        self.hist_v = [[np.zeros((0, h, D)) for _ in range(self.batch)] for h in n_kv_head]

    # -- pieces kept as methods so that tests can plant known mistakes ------
    def _query_positions(self, b: int, n: int) -> np.ndarray:
        return self.lens[b] + np.arange(n)

    def _blocked(self, layer: int, b: int, n: int) -> np.ndarray:
        """(n, lens[b] + n) True where query i of row b may not see key j."""
        pos = int(self.lens[b])
        blocked = _mask.offset_mask(n, pos)
        qpos = self._query_positions(b, n)[:, None]
        kpos = np.arange(pos + n)[None, :]
        blocked = blocked | _mask.window_blocked(qpos, kpos, self.window[layer])
        return blocked | _mask.left_pad_blocked(qpos, kpos, int(self.first[b]))

    # -- the step ------------------------------------------------------------
    def check_capacity(self, n_new) -> np.ndarray:
        n_new = np.asarray(n_new, dtype=np.int64).reshape(-1)
        if n_new.shape[0] != self.batch:
            raise ValueError("n_new needs one entry per row")
        if (n_new < 0).any():
            raise ValueError("n_new must be >= 0")
        if (self.lens + n_new > self.max_len).any():
            raise CacheFull("KV cache full")
        return n_new

    def layer_step(self, layer: int, n_new, q, k, v, compute: bool = True) -> np.ndarray:
        """Append layer ``layer``'s new tokens, then attend.  Does not advance.

        q: (B, C, Hq, D); k, v: (B, C, Hkv, D) raw (pre-RoPE) values.
        Returns (B, C, Hq, D) float64 with zeros at padded / idle positions.
        ``compute=False`` only appends (history for steps nobody checks) and
        returns None.
        """
        n_new = np.asarray(n_new, dtype=np.int64)
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        B, C, Hq, D = q.shape
        out = np.zeros((B, C, Hq, D), dtype=np.float64)
        for b in range(B):
            n = int(n_new[b])
            if n == 0:
                continue
            self.hist_k[layer][b] = np.concatenate((self.hist_k[layer][b], k[b, :n]), axis=0)
            self.hist_v[layer][b] = np.concatenate((self.hist_v[layer][b], v[b, :n]), axis=0)
            if not compute:
                continue
            qrot = _rope.rotate(q[b, :n], self._query_positions(b, n), self.rope_base)
            krot, vals, blocked = self._keys(layer, b, n)
            out[b, :n] = _attn.attend_rows(qrot, krot, vals, blocked)
        return out if compute else None

    def _keys(self, layer: int, b: int, n: int):
        """Rotated keys, values and the (n, keys) blocked mask the current
        step's n queries of row b attend to: the joint partner's keys (if
        any) followed by the layer's own, each under its own layer's rules."""
        T = int(self.lens[b]) + n
        parts = [self.joint[layer]] if self.joint[layer] >= 0 else []
        parts.append(layer)
        ks, vs, bl = [], [], []
        for l in parts:
            if self.hist_k[l][b].shape[0] != T:
                raise ValueError("append the joint partner's tokens of this step first")
            ks.append(_rope.rotate(self.hist_k[l][b], np.arange(T), self.rope_base))
            vs.append(self.hist_v[l][b])
            bl.append(self._blocked(l, b, n))
        return np.concatenate(ks), np.concatenate(vs), np.concatenate(bl, axis=1)

    def query_rows(self, layer: int, b: int, n: int, q_b, idx) -> np.ndarray:
        """Outputs of the queries ``idx`` (a subset of 0..n-1) of row b, whose
        n new tokens were appended to layer ``layer`` in the current step
        (``layer_step``, lens not yet advanced).  q_b: (n, Hq, D) raw queries
        of the row.  The same definition as ``layer_step`` restricted to these
        queries, for checking a few outputs of workloads too large to attend
        in full.  Returns (len(idx), Hq, D) float64."""
        idx = np.asarray(idx, dtype=np.int64)
        q_b = np.asarray(q_b, dtype=np.float64)
        T = int(self.lens[b]) + int(n)
        if self.hist_k[layer][b].shape[0] != T:
            raise ValueError("append this step's tokens (layer_step) before querying")
        qrot = _rope.rotate(q_b[idx], self._query_positions(b, n)[idx], self.rope_base)
        krot, vals, blocked = self._keys(layer, b, n)
        return _attn.attend_rows(qrot, krot, vals, blocked[idx])

    def advance(self, n_new) -> None:
        self.lens = self.lens + np.asarray(n_new, dtype=np.int64)

    def step(self, n_new, layers, compute: bool = True) -> list:
        """One step over every layer: ``layers[l] = (q, k, v)``.  Returns outputs."""
        n_new = self.check_capacity(n_new)
        if len(layers) != self.n_layer:
            raise ValueError("one (q, k, v) per layer")
        outs = [self.layer_step(l, n_new, *layers[l], compute=compute)
                for l in range(self.n_layer)]
        self.advance(n_new)
        return outs

    def reset(self, rows) -> None:
        """Empty these rows: their lengths drop to 0, their history is gone and
        they have no left padding."""
        for b in np.asarray(rows, dtype=np.int64).reshape(-1):
            self.lens[b] = 0
            self.first[b] = 0
            for l in range(self.n_layer):
                self.hist_k[l][b] = self.hist_k[l][b][:0]
                self.hist_v[l][b] = self.hist_v[l][b][:0]

    def set_first(self, rows, first) -> None:
        """Rows ``rows`` start with ``first`` pad positions (0 = none)."""
        rows = np.asarray(rows, dtype=np.int64).reshape(-1)
        first = np.asarray(first, dtype=np.int64).reshape(-1)
        if rows.shape != first.shape or (first < 0).any():
            raise ValueError("one first >= 0 per row")
        self.first[rows] = first

    def admit(self, rows, src: "OracleCache", src_rows) -> None:
        """Row rows[j] becomes a copy of src's row src_rows[j]: history of every
        layer, length and left padding."""
        rows = np.asarray(rows, dtype=np.int64).reshape(-1)
        src_rows = np.asarray(src_rows, dtype=np.int64).reshape(-1)
        if rows.shape != src_rows.shape:
            raise ValueError("one source row per row")
        if (src.n_kv_head != self.n_kv_head or src.window != self.window
                or src.head_dim != self.head_dim or src.joint != self.joint):
            raise ValueError("caches of different layer shapes")
        if (src.lens[src_rows] > self.max_len).any():
            raise CacheFull("admitted row longer than max_len")
        for b, sb in zip(rows, src_rows):
            self.lens[b] = src.lens[sb]
            self.first[b] = src.first[sb]
            for l in range(self.n_layer):
                self.hist_k[l][b] = src.hist_k[l][sb].copy()
                self.hist_v[l][b] = src.hist_v[l][sb].copy()

    def history(self, layer: int, b: int):
        """Raw (k, v) of row b, layer ``layer``: each (lens[b], Hkv, D)."""
        return self.hist_k[layer][b], self.hist_v[layer][b]


class RingModel:
    """Explicit ring-buffer store for ONE sliding layer (self-check only).

    Holds W + 1 slots per row (slot W is scratch) of rotated K and of V plus
    a tag per slot (the position it holds, -1 when empty).  A step stages the
    chunk, scores every valid query by scanning positions qpos - W + 1 ..
    qpos (history rows from the ring at t % W, the chunk's own rows from the
    staged chunk), and only then commits the last W real tokens at pos % W
    (colibri PR, "How it works").  ``append_first=True`` commits before
    scoring: a known mistake, used to show the ring check has teeth.
    """

    def __init__(self, batch: int, n_q_head: int, n_kv_head: int, head_dim: int,
                 window: int, rope_base: float = 10000.0, append_first: bool = False):
        if window <= 0:
            raise ValueError("a ring needs window > 0")
        self.batch, self.W, self.D = batch, window, head_dim
        self.n_q_head, self.n_kv_head = n_q_head, n_kv_head
        self.rope_base = rope_base
        self.append_first = append_first
        self.K = np.zeros((batch, window + 1, n_kv_head, head_dim))
        self.V = np.zeros((batch, window + 1, n_kv_head, head_dim))
        self.tag = np.full((batch, window + 1), -1, dtype=np.int64)
        self.lens = np.zeros(batch, dtype=np.int64)
        self.reads = []   # (row, position read, slot or -1 for the chunk)

    def _commit(self, b, pos_row, krot, vrow, keep):
        W = self.W
        for i in range(len(pos_row)):
            s = pos_row[i] % W if keep[i] else W
            self.K[b, s] = krot[i]
            self.V[b, s] = vrow[i]
            self.tag[b, s] = pos_row[i] if keep[i] else -1

    def step(self, n_new, q, k, v) -> np.ndarray:
        n_new = np.asarray(n_new, dtype=np.int64)
        B, C, Hq, D = q.shape
        W = self.W
        out = np.zeros((B, C, Hq, D), dtype=np.float64)
        for b in range(B):
            n = int(n_new[b])
            if n == 0:
                continue
            L = int(self.lens[b])
            pos = L + np.arange(n)
            krot = _rope.rotate(k[b, :n], pos, self.rope_base)
            qrot = _rope.rotate(q[b, :n], pos, self.rope_base)
            vrow = np.asarray(v[b, :n], dtype=np.float64)
            keep = pos >= L + n - W
            if self.append_first:
                self._commit(b, pos, krot, vrow, keep)
            for i in range(n):
                qpos = L + i
                t0 = max(0, qpos - W + 1)
                ks, vs = [], []
                for t in range(t0, qpos + 1):
                    if t >= L and not self.append_first:
                        ks.append(krot[t - L])
                        vs.append(vrow[t - L])
                        self.reads.append((b, t, -1))
                    else:
                        s = t % W
                        ks.append(self.K[b, s])
                        vs.append(self.V[b, s])
                        self.reads.append((b, t, s))
                out[b, i] = _attn.softmax_attend(qrot[i], np.stack(ks), np.stack(vs),
                                                 1.0 / math.sqrt(D))
            if not self.append_first:
                self._commit(b, pos, krot, vrow, keep)
            self.lens[b] = L + n
        return out

    def reset(self, rows) -> None:
        """Lengths drop to 0; slot contents and tags are left as they are."""
        for b in np.asarray(rows, dtype=np.int64).reshape(-1):
            self.lens[b] = 0
