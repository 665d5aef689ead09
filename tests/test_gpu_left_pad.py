"""Left-padded rows and slot admit / release on the GPU against the oracle.

A row's first `first` positions are padding (tinyllm "kv_cache.py",
padded_causal_mask): keys there are hidden from the row's real queries and a
pad query sees only itself.  Rows of one cache are admitted into another
(SlotKVCache.admit) by copying their stored rows, length and padding.
"""

import numpy as np
import pytest
import torch

import kv_cached_gqa_append_amd as K
import workloads as wl
from gpu_harness import Pair, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _prefill(pair, lens, chunk):
    for n, C in wl.fill_plan(lens, chunk):
        pair.step(n, C)


@pytest.mark.parametrize("use_ring,fused", [(True, False), (True, True), (False, True)])
def test_left_padded_prefill_then_decode(use_ring, fused):
    # global layer + W = 16 sliding layer (a ring, or a full layout with the
    # window as a mask); pads of 5, 0, 40 and 70 positions (two whole chunks
    # of pads in row 3); rows 0 and 2 decode with pads still inside the window
    say(f"case: left padding, D128 rep4, ring={use_ring}, fused decode={fused}")
    work = wl.Workload("leftpad", 2, 4, 32, (8, 8), 128, 256, (0, 16), "bf16", 64,
                       use_ring=use_ring)
    pair = Pair(work, poison=True, tag=f"lp{int(use_ring)}{int(fused)}")
    pair.set_first([0, 1, 2, 3], [5, 0, 40, 70])
    _prefill(pair, [12, 30, 45, 90], 32)
    for s in range(12):
        pair.step(wl.n_new_decode_b64(s, batch=4, idle=1), 1, fused=fused)
    for l in range(work.n_layer):
        pair.check_cache_rows(l)
    say(f"  worst abs {pair.worst:.2e} rel {pair.worst_rel:.2e}")


def test_left_padded_float32_generic_path():
    say("case: left padding, fp32 (generic attention), ring W=6 + global")
    work = wl.Workload("leftpad32", 2, 3, 8, (2, 2), 64, 64, (6, 0), "f32", 16)
    pair = Pair(work, poison=True, tag="lp32")
    pair.set_first([0, 1, 2], [3, 9, 0])
    _prefill(pair, [7, 14, 5], 16)
    _prefill(pair, [2, 0, 9], 4)
    for s in range(8):
        pair.step(wl.n_new_decode_b64(s, batch=3, idle=1), 1)


def test_admit_and_release_slots():
    # A left-padded batched prefill in one cache; its rows admitted into a
    # cache with more rows and a longer max_len; decode there; release a slot
    # and admit another row into it.
    say("case: admit rows of a prefill cache into slots, decode, release, re-admit")
    kw = dict(n_q_head=32, n_kv_head=(8, 8), head_dim=128, window=(0, 24), dtype="bf16",
              max_chunk=64)
    pre = wl.Workload("admit_src", 2, 3, max_len=160, **kw)
    slots = wl.Workload("admit_dst", 2, 5, max_len=256, **kw)
    src = Pair(pre, poison=True, tag="asrc")
    dst = Pair(slots, poison=True, tag="adst")
    src.set_first([0, 1, 2], [11, 0, 3])
    src.step([50, 50, 50], 50)                     # prompts 39, 50, 47 after padding
    src.step([0, 30, 1], 30)
    dst.admit([4, 0, 2], src, [0, 1, 2])
    assert dst.cache.lens() == [80, 0, 51, 0, 50]
    torch.cuda.synchronize()
    for l in range(2):                             # the copied rows, bit for bit
        rows = src.cache.layer_layout(l).rows
        for d, r in ((4, 0), (0, 1), (2, 2)):
            n = min(int(src.ref.lens[r]), rows)
            for view in (lambda c: c.k_view(l), lambda c: c.v_view(l)):
                a = view(src.cache)[r, :, :n].contiguous().view(torch.int16)
                b = view(dst.cache)[d, :, :n].contiguous().view(torch.int16)
                assert torch.equal(a, b), f"layer {l}: row {r} -> slot {d} differs"
    for s in range(6):
        dst.step(np.array([1, 0, 1, 0, 1]), 1, fused=(s % 2 == 0))
    dst.reset([0])
    dst.admit([0], src, [2])
    dst.step(np.array([1, 3, 1, 0, 2]), 3)
    for s in range(4):
        dst.step(np.array([1, 1, 1, 0, 1]), 1)
    for l in range(2):
        dst.check_cache_rows(l)
    say(f"  worst abs {dst.worst:.2e} rel {dst.worst_rel:.2e}")
    # guards
    other = Pair(wl.Workload("admit_bad", 2, 2, 32, (8, 8), 128, 256, (0, 32), "bf16", 64))
    with pytest.raises(ValueError):
        other.cache.admit([0], src.cache, [0])     # different window
    tiny = Pair(wl.Workload("admit_tiny", 2, 2, 32, (8, 8), 128, 60, (0, 24), "bf16", 64))
    with pytest.raises(K.CacheFullError):
        tiny.cache.admit([0], src.cache, [1])      # 80 rows > max_len 60
    with pytest.raises(ValueError):
        dst.cache.admit([1, 1], src.cache, [0, 1])  # a slot twice
    torch.cuda.synchronize()


def test_left_pad_static_graph_matches_eager():
    # the device planner reads the rows' left padding as the host planner does
    say("case: left padding in a captured static step, bits equal to eager")
    work = wl.Workload("lp_static", 2, 4, 32, (8, 8), 128, 512, (0, 40), "bf16", 64,
                       use_ring=False)
    a = Pair(work, poison=True, tag="lps")
    b = Pair(work, poison=True, tag="lps")
    for p in (a, b):
        p.set_first([0, 1, 2, 3], [100, 0, 7, 250])
        for n, C in wl.fill_plan([130, 60, 300, 260], 64):
            p.step(n, C, check=False)
    g = K.StaticDecodeGraph(b.cache, fused=True)
    for s in range(5):
        n = wl.n_new_decode_b64(s, batch=4, idle=1)
        for l in range(work.n_layer):
            q, k, v = wl.step_qkv(work, l, a.step_no, 1, "lps")
            g.q[l].copy_(q)
            g.k[l].copy_(k)
            g.v[l].copy_(v)
        g.n_new.copy_(torch.as_tensor(n, dtype=torch.int32))
        g.replay()
        outs = a.step(n, 1, fused=True)
        torch.cuda.synchronize()
        for l in range(work.n_layer):
            assert torch.equal(g.out[l], outs[l]), f"replay {s} layer {l}"
    b.cache.sync_lens()
    assert b.cache.lens() == a.cache.lens()
