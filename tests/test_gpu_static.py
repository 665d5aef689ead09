"""Static one-token steps (kvc_static_begin) captured in a HIP graph.

A replay reads its token counts from device memory and plans its decode
splits on the device, so it must give the same bits as the eager step that
the host plans (which meets the oracle bar: every eager step here is checked
against the oracle, or at full size against the sampled oracle).  Every
replay is checked, with eager work and synchronisations between replays.
"""

import numpy as np
import pytest
import torch

import kv_cached_gqa_append_amd as K
import oracle
import workloads as wl
from gpu_harness import Pair, SampledOracle, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _same_cache(a_cache, b_cache, layer):
    # raw bits of the cache rows proper; the scratch row takes the padded
    # tokens of idle rows in no fixed order and is left out
    rows = a_cache.layer_layout(layer).rows
    for view in (lambda c: c.k_view(layer), lambda c: c.v_view(layer)):
        x = view(a_cache)[:, :, :rows].contiguous().view(torch.int16)
        y = view(b_cache)[:, :, :rows].contiguous().view(torch.int16)
        assert torch.equal(x, y), f"layer {layer}: cache rows differ"


def _load(g, work, step, tag):
    """The step's seeded inputs (the ones Pair.step draws) into the graph."""
    for l in range(work.n_layer):
        q, k, v = wl.step_qkv(work, l, step, 1, tag)
        g.q[l].copy_(q)
        g.k[l].copy_(k)
        g.v[l].copy_(v)


def _graph_vs_eager(work, fill_lens, counts, tag, fused, chunk=64):
    a = Pair(work, poison=True, tag=tag)       # eager, checked against the oracle
    b = Pair(work, poison=True, tag=tag)       # replays of a captured step
    for n, C in wl.fill_plan(fill_lens, chunk):
        a.step(n, C, check=False)
        b.step(n, C, check=False)
    g = K.StaticDecodeGraph(b.cache, fused=fused, slots=True)
    for s, n in enumerate(counts):
        n = np.asarray(n, dtype=np.int64)
        lens_before = a.ref.lens.copy()
        _load(g, work, a.step_no, tag)
        g.n_new.copy_(torch.as_tensor(n, dtype=torch.int32))
        g.replay()
        outs = a.step(n, 1, fused=fused)
        torch.cuda.synchronize()
        for l in range(work.n_layer):
            assert torch.equal(g.out[l], outs[l]), f"replay {s} layer {l}: output differs"
            want = oracle.slot_indices(lens_before, n, 1, work.window[l], work.max_len,
                                       work.use_ring)
            assert np.array_equal(g.slot[l].cpu().numpy(), want), f"replay {s} layer {l}: slots"
        assert b.cache.device_lens().tolist() == [int(x) for x in a.ref.lens]
    with pytest.raises(K.StepOrderError):
        b.cache.lens()                          # host mirror stale after replays
    b.cache.sync_lens()
    assert b.cache.lens() == a.cache.lens()
    for l in range(work.n_layer):
        _same_cache(a.cache, b.cache, l)
        a.check_cache_rows(l)
    assert b.cache.static_status() == 0
    say(f"  {len(counts)} replays bit-exact; eager worst abs {a.worst:.2e} rel {a.worst_rel:.2e}")


@pytest.mark.parametrize("fused", [True, False])
def test_static_graph_many_splits_and_idle_rows(fused):
    say(f"case: static graph, D128 rep4, global + W=700 window mask, many splits, fused={fused}")
    work = wl.Workload("static_splits", 2, 6, 32, (8, 8), 128, 3200, (0, 700), "bf16", 64,
                       use_ring=False)
    counts = [wl.n_new_decode_b64(s, batch=6, idle=1) for s in range(5)]
    counts.append(np.ones(6, dtype=np.int64))
    counts.append(np.zeros(6, dtype=np.int64))
    _graph_vs_eager(work, [2900, 17, 1024, 1025, 256, 3100], counts, f"st{int(fused)}", fused)


@pytest.mark.parametrize("fused", [True, False])
def test_static_graph_rings(fused):
    say(f"case: static graph, ring_bf16 (W=8 rings + global) wrapping, fused={fused}")
    work = wl.RING_BF16
    counts = [np.array([1, 1, 1, 1]), np.array([1, 0, 1, 1])]
    counts += [wl.n_new_decode_b64(s, batch=4, idle=1) for s in range(14)]
    _graph_vs_eager(work, [12, 3, 9, 0], counts, f"sr{int(fused)}", fused, chunk=12)


def test_static_graph_float32_generic_path():
    say("case: static graph, small_fp32 (generic attention path)")
    work = wl.SMALL_FP32
    counts = [np.array([1])] * 6 + [np.array([0]), np.array([1])]
    _graph_vs_eager(work, [17], counts, "sf", fused=True, chunk=5)


def test_static_rejects_whole_step_and_keeps_protocol():
    say("case: static steps reject bad counts / full rows, sticky flags, protocol")
    work = wl.Workload("static_guard", 2, 3, 8, (2, 2), 64, 12, (0, 4), "bf16", 16)
    pair = Pair(work, poison=True, tag="sg")
    for n, C in wl.fill_plan([10, 3, 11], 16):
        pair.step(n, C, check=False)
    c = pair.cache
    g = K.StaticDecodeGraph(c, fused=True, slots=True)
    q, k, v = (t.to(DEV) for t in wl.step_qkv(work, 0, 77, 1))
    with pytest.raises(K.StepOrderError):
        c.append(0, k, v, [1, 1, 1])           # mirror stale after the capture
    with pytest.raises(K.StepOrderError):
        c.lens()
    c.sync_lens()
    assert c.lens() == [10, 3, 11]

    def replay(n):
        _load(g, work, 500, "sg")
        g.n_new.copy_(torch.as_tensor(n, dtype=torch.int32))
        g.replay()
        torch.cuda.synchronize()

    replay([1, 1, 1])
    assert c.device_lens().tolist() == [11, 4, 12]
    assert c.static_status() == 0
    before = [(c.k_view(l).clone(), c.v_view(l).clone()) for l in range(2)]
    for n, flag in (([0, 1, 1], K.KVC_STATIC_FULL), ([2, 0, 0], K.KVC_STATIC_BAD_COUNT),
                    ([-1, 0, 0], K.KVC_STATIC_BAD_COUNT)):
        say(f"  rejected replay n_new {n}")
        for l in range(2):
            g.out[l].fill_(1.0)
            g.slot[l].fill_(-7)
        replay(n)
        assert c.device_lens().tolist() == [11, 4, 12]
        for l in range(2):
            assert (g.out[l] == 0).all(), "rejected step: outputs not zero"
            rows = c.layer_layout(l).rows
            for x, y in zip(before[l], (c.k_view(l), c.v_view(l))):
                assert torch.equal(x[:, :, :rows].view(torch.int16),
                                   y[:, :, :rows].view(torch.int16)), "rejected step wrote"
            ring = oracle.cache.is_ring(work.window[l], work.max_len, work.use_ring)
            scratch = work.window[l] if ring else work.max_len
            assert (g.slot[l].cpu() == scratch).all()
        assert c.static_status() == flag
        assert c.static_status() == 0           # read clears
    replay([1, 1, 0])
    assert c.device_lens().tolist() == [12, 5, 12]
    assert c.static_status() == 0

    # an eager (uncaptured) static step keeps the protocol
    c.sync_lens()
    n_dev = torch.tensor([0, 1, 0], dtype=torch.int32, device=DEV)
    c.static_begin(n_dev)
    with pytest.raises(K.StepOrderError):
        c.static_begin(n_dev)                   # already in a step
    with pytest.raises(ValueError):
        c.append(0, k, v, [0, 1, 0])            # host counts inside a static step
    k2 = torch.zeros(3, 2, 2, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        c.append(0, k2, k2, None)               # C != 1
    c.append_attend(0, q, k, v, None)
    with pytest.raises(K.StepOrderError):
        c.advance()                             # layer 1 not done
    c.append(1, k, v, None)
    c.attend(1, q)
    c.advance()
    c.sync_lens()
    assert c.lens() == [12, 6, 12]
    with pytest.raises(ValueError):
        c.static_begin(torch.zeros(4, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()


def test_static_graph_decode_b64_full_size():
    # The headline shape (B64, Hq32/Hkv8, D128, max_len 8192, lengths
    # ~ U[1, 8128], 6 idle rows per step) on two layers: the device planner
    # against the host planner at the bench's launch configuration.
    say("case: static graph at decode_b64 full size (2 layers) vs eager, sampled oracle")
    work = wl.DECODE_B64.replace(n_layer=2, n_kv_head=(8, 8), window=(0, 0))
    steps = 4
    lens0 = np.minimum(wl.initial_lens_decode_b64(work.batch), work.max_len - steps)
    cfg = K.config_from_workload(work)
    eager, graphed = K.Cache(cfg, DEV), K.Cache(cfg, DEV)
    r = wl.rng("static_full", "rows")
    rows = sorted({int(np.argmax(lens0)), int(np.argmin(lens0))} |
                  set(int(x) for x in r.choice(work.batch, 3, replace=False)))
    so = SampledOracle(work, rows)
    for si, (n, C) in enumerate(wl.fill_plan(lens0, 64)):
        for l in range(work.n_layer):
            q, k, v = wl.device_step_qkv(work, l, si, C, DEV, "sfill")
            for c in (eager, graphed):
                c.append(l, k, v, n)
                c.attend(l, q)
            so.record(l, k, v, n)
        for c in (eager, graphed):
            c.advance()
    torch.cuda.synchronize()
    g = K.StaticDecodeGraph(graphed, fused=True, slots=False)
    for s in range(steps):
        n = wl.n_new_decode_b64(s, work.batch)
        say(f"  replay {s}: idle rows {np.flatnonzero(n == 0).tolist()}")
        qkv = [wl.device_step_qkv(work, l, 10_000 + s, 1, DEV, "sdec") for l in range(2)]
        for l, (q, k, v) in enumerate(qkv):
            g.q[l].copy_(q)
            g.k[l].copy_(k)
            g.v[l].copy_(v)
        g.n_new.copy_(torch.as_tensor(n, dtype=torch.int32))
        g.replay()
        outs = [eager.append_attend(l, q, k, v, n) for l, (q, k, v) in enumerate(qkv)]
        eager.advance()
        torch.cuda.synchronize()
        for l in range(2):
            assert torch.equal(g.out[l], outs[l]), f"replay {s} layer {l}: output differs"
        mx, rel = so.check_step(n, qkv, outs, lambda b, nb: [0], f"static decode_b64 step {s}")
        say(f"    sampled rows {rows}: worst abs {mx:.2e} rel {rel:.2e}")
        assert graphed.device_lens().tolist() == eager.device_lens().tolist()
    graphed.sync_lens()
    assert graphed.lens() == eager.lens()
    for l in range(2):
        _same_cache(eager, graphed, l)
    assert graphed.static_status() == 0
