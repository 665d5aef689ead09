"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every case prints its name before it touches the GPU.  Inputs are the seeded
draws of ``workloads``; bars are stated in ``gpu_harness``.
"""

import numpy as np
import pytest
import torch

import kv_cached_gqa_append_amd as K
import workloads as wl
from gpu_harness import Pair, say

pytestmark = pytest.mark.gpu


def _fill(pair, target_lens, chunk=64):
    for n, C in wl.fill_plan(target_lens, chunk):
        pair.step(n, C, check=False)


def test_small_fp32_chunks_then_decode():
    # 17-token prompt in chunks 5,5,5,2, then 24 one-token steps; fp32 bar 1e-5.
    say("case: small_fp32 schedule")
    pair = Pair(wl.SMALL_FP32)
    for n, C in wl.schedule_small_fp32():
        pair.step(n, C)
    pair.check_cache_rows(0)
    say(f"  worst abs {pair.worst:.2e}")


def test_small_fp32_ring_layer_generic_path():
    say("case: fp32 ring layer (W=6) with chunks wider than the window")
    work = wl.Workload("fp32_ring", 2, 3, 8, (2, 4), 32, 40, (6, 0), "f32", 16)
    pair = Pair(work, poison=True)
    for n, C in [([9, 3, 0], 9), ([1, 1, 1], 1), ([16, 2, 5], 16), ([1, 0, 1], 1), ([3, 7, 1], 7)]:
        pair.step(n, C)
    pair.check_cache_rows(0)
    pair.check_cache_rows(1)


def test_ring_bf16_wraps_then_reset_and_long_chunk():
    # 8 layers (7 rings of W=8, one global), 12-token prompts + 24 decode
    # steps (the ring wraps 4+ times), then a reset and one 36-token chunk.
    say("case: ring_bf16 phase 1 (poisoned buffer)")
    work = wl.RING_BF16
    pair = Pair(work, poison=True)
    phase1, phase2 = wl.schedule_ring_bf16(work.batch)
    for n, C in phase1:
        pair.step(n, C)
    for l in range(work.n_layer):
        pair.check_cache_rows(l)
    say("case: ring_bf16 reset + 36-token chunk over a NaN-filled cache")
    pair.reset(list(range(work.batch)))
    for l in range(work.n_layer):
        pair.cache.k_view(l).fill_(float("nan"))
        pair.cache.v_raw(l).fill_(float("nan"))
    for n, C in phase2:
        pair.step(n, C)
    for l in range(work.n_layer):
        pair.check_cache_rows(l)
    say(f"  worst abs {pair.worst:.2e} rel {pair.worst_rel:.2e}")


def test_ring_and_full_layouts_agree():
    say("case: ring layout vs full layout with window mask")
    work = wl.RING_BF16
    phase1, _ = wl.schedule_ring_bf16(work.batch)
    a = Pair(work, tag="g7")
    b = Pair(work.replace(use_ring=False), tag="g7")
    for n, C in phase1[:10]:
        oa = a.step(n, C)
        ob = b.step(n, C)
        for x, y in zip(oa, ob):
            assert float((x.float() - y.float()).abs().max()) <= 2e-2


def test_mixed_batch_decode_and_chunks_with_splits():
    # Rows at very different lengths; decode rows (n=1), chunk rows (n>=2),
    # idle rows and right padding in the same call; a global layer and a
    # W=200 ring layer; lengths long enough for several key splits.
    say("case: mixed decode/chunk batch, D128 rep4")
    work = wl.Workload("mixed_small", 2, 5, 32, (8, 8), 128, 1700, (0, 200), "bf16", 64)
    pair = Pair(work, poison=True)
    _fill(pair, [0, 300, 1100, 1400, 37])
    for n in ([64, 1, 17, 1, 0], [1, 64, 1, 2, 64], [0, 5, 64, 1, 1], [33, 1, 1, 64, 2]):
        pair.step(n, 64)
    say(f"  worst abs {pair.worst:.2e} rel {pair.worst_rel:.2e}")


def test_rep8_ring_and_global_prefill_then_decode():
    say("case: rep 8 (Hq64/Hkv8), W=64 ring + global, 64-token chunks then decode")
    work = wl.Workload("rep8_small", 2, 2, 64, (8, 8), 128, 512, (64, 0), "bf16", 64)
    pair = Pair(work, poison=True)
    for s in range(5):
        pair.step([64, 64 if s < 4 else 30], 64, check=(s >= 3))
    for _ in range(6):
        pair.step([1, 1], 1)
    pair.check_cache_rows(0)
    pair.check_cache_rows(1)


# ring_small "1" (default): with fewer 8-wave workgroups than CUs, a ring
# layer's chunk rows all go to the 4-wave launch; "0": rows by size as on a
# global layer (8-wave workgroups for more than 128 query rows)
@pytest.mark.parametrize("ring_small", ["1", "0"])
@pytest.mark.parametrize("D,rep", [(64, 2), (128, 4), (128, 8)])
def test_ring_full_chunks_write_outputs_directly(D, rep, ring_small, monkeypatch):
    # When every row of a step is a full chunk, a ring layer's chunk kernel
    # writes the final outputs itself (one split per row, no merge launch):
    # checked against the oracle and for the same bits as the merge launch
    # (KVC_CHUNK_DIRECT=0), over steps that wrap the W=48 ring, with padded
    # and idle rows in between (those steps take the merge launch).
    say(f"case: ring full chunks, direct outputs, D={D} rep={rep} ring_small={ring_small}")
    monkeypatch.setenv("KVC_CHUNK_RING_SMALL", ring_small)
    work = wl.Workload(f"ring_direct_{D}_{rep}", 2, 3, 2 * rep, (2, 2), D, 400, (48, 0),
                       "bf16", 40)
    monkeypatch.setenv("KVC_CHUNK_DIRECT", "0")
    ref = Pair(work, poison=True, tag="rd")
    monkeypatch.setenv("KVC_CHUNK_DIRECT", "1")
    pair = Pair(work, poison=True, tag="rd")
    for n in ([40, 40, 40], [40, 40, 40], [40, 17, 0], [40, 40, 40], [40, 40, 40], [1, 1, 1],
              [40, 40, 40]):
        C = max(n)
        got = pair.step(n, C)
        want = ref.step(n, C, check=False)
        for l in range(work.n_layer):
            assert torch.equal(got[l], want[l]), f"n {n} layer {l}: differs from the merge launch"
    pair.check_cache_rows(0)
    say(f"  worst abs {pair.worst:.2e} rel {pair.worst_rel:.2e}")


def test_decode_many_splits():
    say("case: decode with lengths up to ~3000 (many splits), D128 rep4")
    work = wl.Workload("decode_splits", 1, 6, 32, (8,), 128, 3200, (0,), "bf16", 64)
    pair = Pair(work, poison=True)
    _fill(pair, [2900, 17, 1024, 1025, 256, 3100])
    for s in range(3):
        pair.step(wl.n_new_decode_b64(s, batch=6, idle=1), 1)


@pytest.mark.parametrize("D,rep", [(64, 1), (64, 2), (64, 8), (128, 1), (128, 2), (128, 16)])
def test_head_shapes(D, rep):
    say(f"case: head shapes D={D} rep={rep}")
    hkv = 2
    work = wl.Workload(f"shape_{D}_{rep}", 1, 3, hkv * rep, (hkv,), D, 400, (0,), "bf16", 40)
    pair = Pair(work, poison=True)
    _fill(pair, [300, 40, 5], chunk=40)
    pair.step([40, 1, 3], 40)
    pair.step([1, 1, 1], 1)


def test_guards_and_step_order():
    say("case: guards (full, dtype, batch, step order)")
    work = wl.Workload("guards", 2, 2, 8, (2, 2), 64, 20, (0, 4), "bf16", 16)
    pair = Pair(work)
    pair.step([8, 3], 8)
    c = pair.cache
    dev = pair.device
    q, k, v = (t.to(dev) for t in wl.step_qkv(work, 0, 99, 8))
    # capacity: row 0 at 8 + 13 > 20
    with pytest.raises(K.CacheFullError):
        c.append(0, torch.zeros(2, 13, 2, 64, dtype=torch.bfloat16, device=dev),
                 torch.zeros(2, 13, 2, 64, dtype=torch.bfloat16, device=dev), [13, 0])
    assert c.lens() == [8, 3]
    with pytest.raises(TypeError):
        c.append(0, k.float(), v.float(), [1, 1])
    with pytest.raises(ValueError):
        c.append(0, k[:1], v[:1], [1])
    with pytest.raises(K.StepOrderError):
        c.attend(0, q)                                    # attend before append
    c.append(0, k, v, [2, 2])
    with pytest.raises(ValueError):
        c.attend(0, q[:, :4].contiguous())                 # fewer tokens than the step's C
    with pytest.raises(K.StepOrderError):
        c.append(0, k, v, [2, 2])                          # same layer twice
    with pytest.raises(K.StepOrderError):
        c.append(1, k, v, [2, 1])                          # different n_new in a step
    with pytest.raises(K.StepOrderError):
        c.advance()                                        # layer 0 not attended
    with pytest.raises(K.StepOrderError):
        c.reset([0])                                       # reset inside a step
    c.attend(0, q)
    c.append(1, k, v, [2, 2])
    with pytest.raises(K.StepOrderError):
        c.advance()                                        # layer 1 not attended
    c.attend(1, q)
    c.advance()
    assert c.lens() == [10, 5]
    torch.cuda.synchronize()


# -- the one-token step through kvc_append_attend ---------------------------------
def _same_cache(a, b, layer):
    # Raw bits of the cache rows proper (rows never written hold the NaN
    # poison in both).  The scratch row is left out: the padded tokens of a
    # chunk all land there in one append, in no fixed order.
    rows = a.cache.layer_layout(layer).rows
    ka = a.cache.k_view(layer)[:, :, :rows].view(torch.int16)
    kb = b.cache.k_view(layer)[:, :, :rows].view(torch.int16)
    va = a.cache.v_view(layer)[:, :, :rows].view(torch.int16)
    vb = b.cache.v_view(layer)[:, :, :rows].view(torch.int16)
    assert torch.equal(ka, kb), f"layer {layer}: K differs"
    assert torch.equal(va, vb), f"layer {layer}: V differs"


def _fused_vs_two_calls(work, prompts, decode_steps, tag):
    """Drive two caches with the same inputs, one through append_attend and
    one through append + attend; both meet the oracle bar, and the one-token
    steps agree bit for bit (same stores, same arithmetic in the same order)."""
    a = Pair(work, poison=True, tag=tag)
    b = Pair(work, poison=True, tag=tag)
    for n, C in prompts:
        a.step(n, C, fused=True)
        b.step(n, C)
    for n in decode_steps:
        oa = a.step(n, 1, fused=True)
        ob = b.step(n, 1)
        for l, (x, y) in enumerate(zip(oa, ob)):
            assert torch.equal(x, y), f"layer {l}: fused output differs from append + attend"
    for l in range(work.n_layer):
        _same_cache(a, b, l)
        a.check_cache_rows(l)
    say(f"  worst abs {a.worst:.2e} rel {a.worst_rel:.2e}")


# merge "1": the appending decode merges its splits (KVC_FUSED_MERGE=1); "0"
# (default): it appends and attends, and the merge kernel combines the splits
# wg "1" (default): the ring layers' one-token steps take the workgroup form;
# "0": the split plan (and the merge kernel, or with merge "1" the in-launch
# merge), as a longer window would
@pytest.mark.parametrize("merge,wg", [("0", "1"), ("0", "0"), ("1", "0")])
def test_fused_decode_rings_and_idle_rows(merge, wg, monkeypatch):
    monkeypatch.setenv("KVC_FUSED_MERGE", merge)
    monkeypatch.setenv("KVC_DECODE_WG", wg)
    say(f"case: fused one-token steps, ring_bf16 (rings W=8 + global), idle rows, "
        f"merge={merge} wg={wg}")
    work = wl.RING_BF16
    prompts = [(np.array([12, 3, 9, 0]), 12)]
    steps = [np.array([1, 1, 1, 1]), np.array([1, 0, 1, 1]), np.array([0, 1, 1, 0])]
    steps += [wl.n_new_decode_b64(s, batch=4, idle=1) for s in range(20)]
    _fused_vs_two_calls(work, prompts, steps, "fused_ring")


# One-token steps of ring layers with REP 8 and 16 take the workgroup form on
# the matrix cores: rings of 48 and 200 slots (a partial last 32-key tile),
# rows short of the window, filling it and wrapped past it, idle rows; both
# entry points against the oracle, and bit for bit against each other.
@pytest.mark.parametrize("D,rep", [(64, 8), (64, 16), (128, 8), (128, 16)])
def test_ring_decode_matrix_core_form(D, rep):
    say(f"case: ring one-token steps, workgroup form on the matrix cores, D={D} rep={rep}, "
        f"W=48/200, idle rows")
    hkv = 2
    work = wl.Workload(f"wgm_{D}_{rep}", 2, 5, hkv * rep, (hkv, hkv), D, 600, (48, 200),
                       "bf16", 64)
    prompts = wl.fill_plan([5, 47, 130, 260, 0], 64)
    steps = [np.array([1, 1, 1, 1, 1])]
    steps += [wl.n_new_decode_b64(s, batch=5, idle=1) for s in range(12)]
    _fused_vs_two_calls(work, prompts, steps, f"wgm{D}_{rep}")


# Chunk steps of ring layers through kvc_append_attend: when every row holds
# 2 .. 64 tokens the chunk kernel reads them from the caller's K and V,
# scores them before the history and commits the kept ones to the ring
# itself (no staging, no append launch).  Rings of 8, 48 and 200 slots beside
# a global layer; rows longer than the window, wrapping, lengths off the
# 8-row grid, padded tokens; steps with a one-token row take append + attend.
# Outputs against the oracle, slots and cache rows bit for bit against the
# two calls; the fused cache's staging is never written.
# ring_small "1" (default) sends every row of these small batches to the
# 128-row query tiles, in the key-halves form (kh "1", default) or in 4-wave
# workgroups (kh "0"); ring_small "0" sorts rows by size into both launches.
@pytest.mark.parametrize("D,rep,ring_small,kh", [(64, 4, "1", "1"), (128, 8, "1", "1"),
                                                 (128, 8, "1", "0"), (128, 8, "0", "1"),
                                                 (128, 1, "1", "1")])
def test_fused_ring_chunk_steps(D, rep, ring_small, kh, monkeypatch):
    monkeypatch.setenv("KVC_CHUNK_RING_SMALL", ring_small)
    monkeypatch.setenv("KVC_CHUNK_KEY_HALVES", kh)
    say(f"case: ring chunk steps through kvc_append_attend, D={D} rep={rep} "
        f"ring_small={ring_small} key_halves={kh}, W=8/48/200 + global")
    hkv = 2
    work = wl.Workload(f"rchunk_{D}_{rep}", 4, 4, hkv * rep, (hkv,) * 4, D, 700,
                       (8, 48, 200, 0), "bf16", 64)
    prompts = [(np.array([64, 2, 37, 13]), 64), (np.array([5, 64, 2, 30]), 64),
               (np.array([12, 9, 33, 2]), 40), (np.array([3, 7, 64, 5]), 64),
               (np.array([1, 6, 2, 4]), 6), (np.array([64, 64, 64, 64]), 64),
               (np.array([17, 2, 50, 64]), 64)]
    a = Pair(work, poison=True, tag="rchunk")
    b = Pair(work, poison=True, tag="rchunk")
    for s, (n, C) in enumerate(prompts):
        a.step(n, C, fused=True)
        b.step(n, C)
        if s == 3:  # (every step so far had rows of 2 .. 64 tokens only)
            for l in range(3):
                for view in (a.cache.k_view(l, staging=True), a.cache.v_view(l, staging=True)):
                    assert bool(torch.isnan(view.float()).all()), \
                        f"layer {l}: a fused chunk step wrote staging"
    for n in [np.array([1, 1, 1, 1]), np.array([1, 0, 1, 1])]:
        oa = a.step(n, 1, fused=True)
        ob = b.step(n, 1)
        for l, (x, y) in enumerate(zip(oa, ob)):
            assert torch.equal(x, y), f"layer {l}: fused output differs from append + attend"
    for l in range(work.n_layer):
        _same_cache(a, b, l)
        a.check_cache_rows(l)
    say(f"  worst abs {a.worst:.2e} rel {a.worst_rel:.2e}")


@pytest.mark.parametrize("merge", ["0", "1"])
def test_fused_decode_many_splits(merge, monkeypatch):
    monkeypatch.setenv("KVC_FUSED_MERGE", merge)
    say(f"case: fused one-token steps with many key splits, D128 rep4, W=700 window mask, "
        f"merge={merge}")
    work = wl.Workload("fused_splits", 2, 6, 32, (8, 8), 128, 3200, (0, 700), "bf16", 64,
                       use_ring=False)
    a = Pair(work, poison=True, tag="fs")
    b = Pair(work, poison=True, tag="fs")
    for n, C in wl.fill_plan([2900, 17, 1024, 1025, 256, 3100], 64):
        a.step(n, C, check=False)
        b.step(n, C, check=False)
    for s in range(4):
        n = wl.n_new_decode_b64(s, batch=6, idle=1)
        oa = a.step(n, 1, fused=True)
        ob = b.step(n, 1)
        for l, (x, y) in enumerate(zip(oa, ob)):
            assert torch.equal(x, y), f"step {s} layer {l}: fused output differs"
    for l in range(work.n_layer):
        _same_cache(a, b, l)
    say(f"  worst abs {a.worst:.2e} rel {a.worst_rel:.2e}")


@pytest.mark.parametrize("merge", ["0", "1"])
@pytest.mark.parametrize("D,rep", [(64, 1), (64, 16), (128, 2), (128, 8), (128, 16)])
def test_fused_head_shapes(D, rep, merge, monkeypatch):
    monkeypatch.setenv("KVC_FUSED_MERGE", merge)
    say(f"case: fused head shapes D={D} rep={rep} merge={merge}")
    hkv = 2
    work = wl.Workload(f"fshape_{D}_{rep}", 1, 3, hkv * rep, (hkv,), D, 400, (0,), "bf16", 40)
    _fused_vs_two_calls(work, wl.fill_plan([300, 40, 5], 40),
                        [np.array([1, 1, 1]), np.array([1, 0, 1])], f"fs{D}_{rep}")


# The appending decode stores the new row's V after its tile loads and the
# appending wave's own tile takes the values in registers: the new row at
# every position of its 16-row block (both halves of the lanes' key ranges),
# on a full layer and on a W = 48 ring (the workgroup form), bit for bit
# against append + attend.
@pytest.mark.parametrize("D,rep", [(64, 1), (64, 4), (128, 2), (128, 4)])
def test_fused_new_row_every_block_position(D, rep):
    say(f"case: fused one-token steps, new row at every block position, D={D} rep={rep}")
    hkv = 2
    work = wl.Workload(f"fpos_{D}_{rep}", 2, 4, hkv * rep, (hkv, hkv), D, 400, (0, 48), "bf16",
                       40)
    prompts = wl.fill_plan([33, 100, 7, 250], 40)
    steps = [np.array([1, 1, 1, 1])] * 17 + [np.array([1, 0, 1, 1])]
    _fused_vs_two_calls(work, prompts, steps, f"fpos{D}_{rep}")


def test_fused_guards():
    say("case: fused entry point keeps the step protocol")
    work = wl.Workload("fguards", 2, 2, 8, (2, 2), 64, 20, (0, 4), "bf16", 16)
    pair = Pair(work)
    pair.step([8, 3], 8)
    c, dev = pair.cache, pair.device
    q, k, v = (t.to(dev) for t in wl.step_qkv(work, 0, 99, 1))
    c.append_attend(0, q, k, v, [1, 1])
    with pytest.raises(K.StepOrderError):
        c.append_attend(0, q, k, v, [1, 1])                # same layer twice
    with pytest.raises(K.StepOrderError):
        c.append_attend(1, q, k, v, [1, 0])                # different n_new in a step
    with pytest.raises(K.StepOrderError):
        c.attend(0, q)                                     # already attended
    c.append_attend(1, q, k, v, [1, 1])
    c.advance()
    assert c.lens() == [9, 4]
    big = torch.zeros(2, 1, 2, 64, dtype=torch.bfloat16, device=dev)
    for _ in range(11):
        c.append_attend(0, q, big, big, [1, 0])
        c.append_attend(1, q, big, big, [1, 0])
        c.advance()
    with pytest.raises(K.CacheFullError):
        c.append_attend(0, q, big, big, [1, 0])            # row 0 at 20 = max_len
    assert c.lens() == [20, 4]
    torch.cuda.synchronize()
