"""KV-cache byte counts (oracle).  TEST INFRASTRUCTURE ONLY.

Lab 07 section 1 gives the size per cached token as
2 * n_layer * n_kv_head * head_dim * bytes (K and V, GQA-shrunk), and
pycraft-1 ``KVCache.memory_bytes`` multiplies that by batch and max_len.
With sliding-window rings (colibri PR "How it works", kv_ring_rows) a ring
layer holds W rows instead of max_len.  Per-layer KV-head counts allow the
inkling shapes of that PR's memory table (16 KV heads on sliding layers, 8 on
global ones).

Pins: the Lab 07 answer (98,304 bytes for its Config at batch 3, float32) and
every figure of the colibri PR's memory table and per-token growth line
(fixtures in tests/golden).
"""

from .cache import is_ring, ring_rows


def kv_nbytes(batch: int, n_kv_head, head_dim: int, max_len: int, window,
              dtype_bytes: int, use_ring: bool = True) -> int:
    """Sum over layers of 2 * B * Hkv_l * rows_l * D * bytes (no scratch rows)."""
    n_kv_head = list(n_kv_head)
    window = list(window)
    if len(n_kv_head) != len(window):
        raise ValueError("one n_kv_head and one window per layer")
    total = 0
    for hkv, w in zip(n_kv_head, window):
        rows = ring_rows(int(w), int(max_len), use_ring)
        total += 2 * int(batch) * int(hkv) * rows * int(head_dim) * int(dtype_bytes)
    return total


def kv_bytes_per_token(n_kv_head, head_dim: int, dtype_bytes: int, window=None,
                       max_len: int = 0, use_ring: bool = True) -> int:
    """Growth of the cache per extra token of context (batch 1).

    Every layer whose cache is full-length grows by 2 * Hkv * D * bytes per
    token (Lab 07 section 1); a ring layer (0 < W < max_len) has a fixed
    size and does not grow.
    """
    n_kv_head = list(n_kv_head)
    if window is None:
        window = [0] * len(n_kv_head)
    total = 0
    for hkv, w in zip(n_kv_head, window):
        grows = not (max_len > 0 and is_ring(int(w), int(max_len), use_ring))
        if grows:
            total += 2 * int(hkv) * int(head_dim) * int(dtype_bytes)
    return total
