"""Paged KV ("Lab 07 - KV cache and sampling", Stretch: fixed 16-token blocks
and a per-sequence block table) on the GPU.

A paged cache must give the same bits as the contiguous one (the kernels do
the same arithmetic on the same rows; only where a row's blocks live
differs), meet the oracle bar, refuse a step the page pool cannot hold with
nothing changed, and return a released row's pages for reuse.
"""

import numpy as np
import pytest
import torch

import kv_cached_gqa_append_amd as K
import workloads as wl
from gpu_harness import Pair, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _both(work, n_pages, tag):
    a = Pair(work, poison=True, tag=tag)
    b = Pair(work.replace(n_pages=n_pages), poison=True, tag=tag)
    return a, b


def _same_step(a, b, n, C, fused=False):
    oa = a.step(n, C, fused=fused)
    ob = b.step(n, C, fused=fused)
    for l, (x, y) in enumerate(zip(oa, ob)):
        assert torch.equal(x, y), f"step {a.step_no - 1} layer {l}: paged output differs"


@pytest.mark.parametrize("use_ring,fused", [(True, False), (True, True), (False, True)])
def test_paged_equals_contiguous(use_ring, fused):
    # global layer + W = 40 sliding layer (a ring, or with use_ring=False a
    # paged full layout masked by the window); rows grow in turns so their
    # pages interleave in the pool; chunk, mixed and one-token steps
    say(f"case: paged vs contiguous, D128 rep4, ring={use_ring}, fused decode={fused}")
    work = wl.Workload("paged", 2, 5, 32, (8, 8), 128, 400, (0, 40), "bf16", 64,
                       use_ring=use_ring)
    a, b = _both(work, 5 * 400 // 16 + 3, f"pg{int(use_ring)}{int(fused)}")
    for n in ([37, 0, 64, 5, 16], [0, 64, 1, 17, 16], [64, 3, 0, 64, 1], [9, 64, 33, 2, 47]):
        _same_step(a, b, n, 64)
    for s in range(10):
        _same_step(a, b, wl.n_new_decode_b64(s, batch=5, idle=1), 1, fused=fused)
    _same_step(a, b, [1, 64, 2, 1, 0], 64)
    st = b.cache.page_stats()
    assert st["used"] == sum(a.cache.lens())
    assert st["allocated"] == sum(-(-L // 16) for L in a.cache.lens()) * 16
    say(f"  pages {st}; worst abs {b.worst:.2e} rel {b.worst_rel:.2e}")


def test_paged_float32_generic_path():
    say("case: paged fp32 (generic attention), ring W=6 + global")
    work = wl.Workload("paged32", 2, 3, 8, (2, 2), 64, 64, (6, 0), "f32", 16)
    a, b = _both(work, 14, "pg32")
    for n, C in wl.fill_plan([21, 14, 33], 16):
        _same_step(a, b, n, C)
    for s in range(6):
        _same_step(a, b, wl.n_new_decode_b64(s, batch=3, idle=1), 1)


def test_paged_pool_full_then_release():
    # 12 pages of 16 rows for 3 rows of up to 128 positions
    say("case: paged pool runs out (nothing taken), release returns pages")
    work = wl.Workload("paged_small", 2, 3, 32, (8, 8), 128, 128, (0, 0), "bf16", 64,
                       n_pages=12)
    p = Pair(work, poison=True, tag="pgs")
    p.step([64, 40, 50], 64)                       # 4 + 3 + 4 = 11 pages
    assert p.cache.page_stats() == {"used": 154, "allocated": 176, "reserved": 192}
    q, k, v = (t.to(DEV) for t in wl.step_qkv(work, 0, 99, 20))
    with pytest.raises(K.CacheFullError):
        p.cache.append(0, k, v, [20, 0, 0])        # needs 2 more pages, 1 free
    assert p.cache.page_stats()["allocated"] == 176 and p.cache.lens() == [64, 40, 50]
    p.step([0, 8, 14], 14)                          # 40 -> 48, 50 -> 64: no new page
    p.step([16, 0, 0], 16)                          # the last free page
    assert p.cache.page_stats()["allocated"] == 192
    p.reset([1])                                    # 3 pages back
    assert p.cache.page_stats()["allocated"] == 144
    p.step([0, 24, 0], 24)                          # 2 of them
    for s in range(5):                              # row 0 takes the last one
        p.step([1, 1, 0], 1, fused=(s % 2 == 0))
    assert p.cache.page_stats() == {"used": 85 + 29 + 64, "allocated": 192, "reserved": 192}
    say(f"  worst abs {p.worst:.2e} rel {p.worst_rel:.2e}")


def test_paged_admit_both_ways():
    say("case: admit contiguous -> paged and paged -> contiguous, then decode")
    kw = dict(n_q_head=32, n_kv_head=(8, 8), head_dim=128, window=(0, 24), dtype="bf16",
              max_chunk=64)
    flat = Pair(wl.Workload("adm_flat", 2, 3, max_len=160, **kw), poison=True, tag="af")
    paged = Pair(wl.Workload("adm_paged", 2, 4, max_len=256, n_pages=40, **kw), poison=True,
                 tag="ap")
    flat.set_first([1], [5])
    flat.step([50, 37, 64], 64)
    flat.step([13, 0, 2], 13)
    paged.admit([3, 1, 0], flat, [0, 1, 2])
    for s in range(5):
        paged.step(np.array([1, 1, 0, 1]), 1, fused=(s % 2 == 1))
    back = Pair(wl.Workload("adm_back", 2, 2, max_len=256, **kw), poison=True, tag="ab")
    back.admit([1, 0], paged, [0, 3])
    for s in range(4):
        back.step(np.array([1, 1]), 1)
    say(f"  worst abs {max(paged.worst, back.worst):.2e}")


def test_paged_static_graph():
    say("case: paged static step in a graph: reserved pages, bits equal eager, full flag")
    work = wl.Workload("paged_static", 2, 4, 32, (8, 8), 128, 512, (0, 0), "bf16", 64,
                       n_pages=4 * 512 // 16)
    a = Pair(work, poison=True, tag="pgg")
    b = Pair(work, poison=True, tag="pgg")
    for p in (a, b):
        for n, C in wl.fill_plan([100, 31, 254, 7], 64):
            p.step(n, C, check=False)
    b.cache.reserve([0, 1, 2, 3], [108, 40, 256, 15])   # row 2: room for 2 more tokens
    g = K.StaticDecodeGraph(b.cache, fused=True)
    for s in range(6):
        n = np.array([1, 1, 1 if s < 2 else 0, 1])
        for l in range(work.n_layer):
            q, k, v = wl.step_qkv(work, l, a.step_no, 1, "pgg")
            g.q[l].copy_(q)
            g.k[l].copy_(k)
            g.v[l].copy_(v)
        g.n_new.copy_(torch.as_tensor(n, dtype=torch.int32))
        g.replay()
        outs = a.step(n, 1, fused=True)
        torch.cuda.synchronize()
        for l in range(work.n_layer):
            assert torch.equal(g.out[l], outs[l]), f"replay {s} layer {l}"
    assert b.cache.static_status() == 0
    g.n_new.copy_(torch.tensor([0, 0, 1, 0], dtype=torch.int32))   # row 2 has no page left
    g.replay()
    torch.cuda.synchronize()
    assert b.cache.static_status() == K.KVC_STATIC_FULL
    b.cache.sync_lens()
    assert b.cache.lens() == a.cache.lens()
