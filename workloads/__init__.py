"""Seeded synthetic workloads shared by the tests, the smoke check and the bench.

This module holds shapes, schedules and random draws only: no RoPE, no mask,
no attention arithmetic.  Both the oracle side and the GPU side take their
inputs from here, so they see identical values.

Values: q, k, v ~ N(0, 1) drawn in float32 on the CPU with a seeded
``torch.Generator`` and rounded (round-to-nearest-even) to the workload dtype.
Every draw has its own seed derived from a key tuple (workload, layer, step,
tensor[, row]), so any step or any single row can be regenerated on its own.

The five workloads are the cached-attention cases of the kv_cached_gqa_append
study (sizes as given there; readings of open points are in the design
notes):

  small_fp32   1 layer, B1, Hq8/Hkv2, D64, fp32, max_len 64, full cache;
               chunks 5,5,5,2 (a 17-token prompt) then 24 one-token steps
  ring_bf16    8 layers (0-6 sliding W=8 rings, 7 global), B4, Hq8/Hkv2, D64,
               bf16, max_len 64; 12-token prompts + 24 decode steps, then a
               reset and one 36-token chunk (S > W)
  decode_b64   32 full layers, max_len 8192, B64, Hq32/Hkv8, D128, bf16;
               initial lens ~ U[1, 8128]; one token per row per step with 6
               rows idle per step; 64 steps
  mixed_b32    32 layers, max_len 32768, B32, Hq32/Hkv8, D128, bf16, C=64;
               half the rows n_new=1, the rest n_new ~ U{0..64}; initial lens
               ~ U[0, 30000]
  long_5to1    66 layers (55 sliding W=512 rings, 11 global), B8, Hq64/Hkv8,
               D128, bf16, max_len 32768; 510 prefill chunks of 64 then 128
               decode steps
"""

from dataclasses import dataclass, field
import hashlib

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    n_layer: int
    batch: int
    n_q_head: int
    n_kv_head: tuple
    head_dim: int
    max_len: int
    window: tuple
    dtype: str                 # "f32" or "bf16"
    max_chunk: int
    rope_base: float = 10000.0
    use_ring: bool = True
    n_pages: int = 0           # > 0: paged full layers with a pool of this many 16-row pages
    joint: tuple = ()          # per layer: joint softmax partner layer, -1 none (empty: none)
    notes: str = field(default="", compare=False)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def dtype_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


def interleaved_layout(n_layer: int, ratio: int, window: int) -> tuple:
    """Window per layer for an r:1 sliding:global stack: layer l is global
    (window 0) iff (l + 1) % (r + 1) == 0, otherwise sliding with ``window``."""
    return tuple(0 if (l + 1) % (ratio + 1) == 0 else window for l in range(n_layer))


SMALL_FP32 = Workload("small_fp32", 1, 1, 8, (2,), 64, 64, (0,), "f32", 8)
RING_BF16 = Workload("ring_bf16", 8, 4, 8, (2,) * 8, 64, 64,
                     (8,) * 7 + (0,), "bf16", 36)
DECODE_B64 = Workload("decode_b64", 32, 64, 32, (8,) * 32, 128, 8192, (0,) * 32, "bf16", 64)
MIXED_B32 = Workload("mixed_b32", 32, 32, 32, (8,) * 32, 128, 32768, (0,) * 32, "bf16", 64)
LONG_5TO1 = Workload("long_5to1", 66, 8, 64, (8,) * 66, 128, 32768,
                     interleaved_layout(66, 5, 512), "bf16", 64)

ALL = {w.name: w for w in (SMALL_FP32, RING_BF16, DECODE_B64, MIXED_B32, LONG_5TO1)}


# -- seeds and draws -----------------------------------------------------------
def seed_of(*key) -> int:
    """Stable 63-bit seed from a key tuple (independent of PYTHONHASHSEED)."""
    h = hashlib.sha256(repr(key).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def normal(shape, dtype, *key) -> torch.Tensor:
    """N(0,1) float32 draw on the CPU for ``key``, rounded to ``dtype``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_of(*key))
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(dtype)


def step_qkv(wl: Workload, layer: int, step: int, C: int, tag: str = ""):
    """q (B, C, Hq, D), k, v (B, C, Hkv_l, D) CPU tensors for one layer-step."""
    B, D = wl.batch, wl.head_dim
    hq, hkv = wl.n_q_head, wl.n_kv_head[layer]
    dt = wl.torch_dtype
    q = normal((B, C, hq, D), dt, wl.name, tag, layer, step, "q")
    k = normal((B, C, hkv, D), dt, wl.name, tag, layer, step, "k")
    v = normal((B, C, hkv, D), dt, wl.name, tag, layer, step, "v")
    return q, k, v


def row_qkv(wl: Workload, layer: int, step: int, row: int, C: int, tag: str = ""):
    """Per-row draw: q (C, Hq, D), k, v (C, Hkv_l, D) for one row of one step."""
    D = wl.head_dim
    hq, hkv = wl.n_q_head, wl.n_kv_head[layer]
    dt = wl.torch_dtype
    q = normal((C, hq, D), dt, wl.name, tag, "row", layer, step, row, "q")
    k = normal((C, hkv, D), dt, wl.name, tag, "row", layer, step, row, "k")
    v = normal((C, hkv, D), dt, wl.name, tag, "row", layer, step, row, "v")
    return q, k, v


def device_normal(shape, dtype, device, *key) -> torch.Tensor:
    """N(0,1) draw for ``key`` made on ``device`` by a seeded torch generator
    there (float32, rounded to ``dtype``): for histories too large to draw on
    the CPU.  The values differ from ``normal``'s for the same key; a checker
    copies the rows it needs back to the host."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_of("device", *key))
    return torch.randn(*shape, generator=g, dtype=torch.float32, device=device).to(dtype)


def device_step_qkv(wl: Workload, layer: int, step: int, C: int, device, tag: str = ""):
    """q (B, C, Hq, D), k, v (B, C, Hkv_l, D) drawn on ``device``."""
    B, D = wl.batch, wl.head_dim
    hq, hkv = wl.n_q_head, wl.n_kv_head[layer]
    dt = wl.torch_dtype
    q = device_normal((B, C, hq, D), dt, device, wl.name, tag, layer, step, "q")
    k = device_normal((B, C, hkv, D), dt, device, wl.name, tag, layer, step, "k")
    v = device_normal((B, C, hkv, D), dt, device, wl.name, tag, layer, step, "v")
    return q, k, v


def rng(*key) -> np.random.Generator:
    return np.random.default_rng(seed_of(*key))


# -- schedules: lists of (n_new per row, C) per step ----------------------------
def schedule_small_fp32():
    """17-token prompt in chunks 5,5,5,2, then 24 single-token steps."""
    steps = [(np.array([n]), n) for n in (5, 5, 5, 2)]
    steps += [(np.array([1]), 1) for _ in range(24)]
    return steps


def schedule_ring_bf16(batch: int = 4):
    """Phase 1: 12-token prompts then 24 decode steps (the W=8 ring wraps
    four times and more).  Phase 2 (after a reset of every row): one
    36-token chunk, longer than the window."""
    phase1 = [(np.full(batch, 12), 12)] + [(np.full(batch, 1), 1) for _ in range(24)]
    phase2 = [(np.full(batch, 36), 36)]
    return phase1, phase2


def initial_lens_decode_b64(batch: int = 64, lo: int = 1, hi: int = 8128):
    """Starting lengths ~ U[1, 8128]: 64 more steps then end at or below 8192."""
    return rng("decode_b64", "lens").integers(lo, hi + 1, size=batch)


def n_new_decode_b64(step: int, batch: int = 64, idle: int = 6):
    """One token per row, except ``idle`` rows (redrawn each step) with none."""
    n = np.ones(batch, dtype=np.int64)
    r = rng("decode_b64", "idle", step)
    n[r.choice(batch, size=idle, replace=False)] = 0
    return n


def initial_lens_mixed_b32(batch: int = 32, hi: int = 30000):
    return rng("mixed_b32", "lens").integers(0, hi + 1, size=batch)


def n_new_mixed_b32(step: int, batch: int = 32, C: int = 64):
    """A seeded random half of the rows decode one token; the others take
    n_new ~ U{0..C} (right-padded to C)."""
    r = rng("mixed_b32", "n_new", step)
    n = r.integers(0, C + 1, size=batch)
    n[r.choice(batch, size=batch // 2, replace=False)] = 1
    return n


def schedule_long_5to1(chunks: int = 510, chunk: int = 64, decodes: int = 128, batch: int = 8):
    """510 prefill chunks of 64 tokens (32,640 tokens), then 128 decode steps
    (ending at exactly 32,768 = max_len)."""
    return ([(np.full(batch, chunk), chunk)] * chunks
            + [(np.full(batch, 1), 1)] * decodes)


def fill_plan(target_lens, chunk: int = 64):
    """Steps that bring every row from 0 to target_lens in chunks of at most
    ``chunk`` tokens: a list of (n_new per row, C)."""
    target = np.asarray(target_lens, dtype=np.int64)
    done = np.zeros_like(target)
    plan = []
    while (done < target).any():
        n = np.minimum(chunk, target - done)
        C = int(n.max())
        plan.append((n, C))
        done += n
    return plan
