"""GPU parity at the workloads' full sizes, on sampled rows.

Each test builds the full per-layer shape of a workload (rows, heads, head
dim, max_len, lengths), drives every row through the C ABI in the launch
configuration the bench times, and checks chosen queries of a few rows
against the oracle (the oracle finishes them in seconds; all rows at these
sizes it would not).  Properties that hold at any size are checked on every
row: slot indices and lengths bit-exact, padded and idle outputs exactly
zero, outputs finite, and (for one-token steps) kvc_append_attend equal bit
for bit to append + attend.  Histories are drawn on the GPU from
seeded generators (``workloads.device_step_qkv``); the sampled rows' tokens
are copied back for the oracle.
"""

import numpy as np
import pytest
import torch

import kv_cached_gqa_append_amd as K
import oracle
import workloads as wl
from gpu_harness import SampledOracle, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _slots_ok(so_dev, lens, n_new, C, work, layer, what):
    want = oracle.slot_indices(lens, n_new, C, work.window[layer], work.max_len, work.use_ring)
    got = so_dev.cpu().numpy()
    assert np.array_equal(got, want), f"{what}: slot indices differ"


def _fill(caches, work, target, tag, sampled, chunk=64):
    plan = wl.fill_plan(target, chunk)
    for si, (n, C) in enumerate(plan):
        for l in range(work.n_layer):
            q, k, v = wl.device_step_qkv(work, l, si, C, DEV, tag)
            for c in caches:
                c.append(l, k, v, n)
                c.attend(l, q)
            sampled.record(l, k, v, n)
        for c in caches:
            c.advance()
        if si % 64 == 0:
            say(f"  fill step {si + 1}/{len(plan)}")
    torch.cuda.synchronize()


def test_decode_b64_full_size():
    # 64 rows, Hq 32 / Hkv 8, D 128, max_len 8192, lengths ~ U[1, 8128] (the
    # bench's), 6 idle rows per step; two layers of that shape.
    say("case: decode_b64 full size (2 layers), fused vs append + attend, sampled oracle")
    steps = 4
    work = wl.DECODE_B64.replace(n_layer=2, n_kv_head=(8, 8), window=(0, 0))
    lens0 = np.minimum(wl.initial_lens_decode_b64(work.batch), work.max_len - steps)
    cfg = K.config_from_workload(work)
    fused, two = K.Cache(cfg, DEV), K.Cache(cfg, DEV)
    r = wl.rng("full_sizes", "decode_rows")
    rows = sorted({int(np.argmax(lens0)), int(np.argmin(lens0))} |
                  set(int(x) for x in r.choice(work.batch, 4, replace=False)))
    so = SampledOracle(work, rows)
    _fill([fused, two], work, lens0, "dfill", so)
    lens = lens0.astype(np.int64)
    worst = (0.0, 0.0)
    for s in range(steps):
        n = wl.n_new_decode_b64(s, work.batch)
        say(f"  decode step {s}: idle rows {np.flatnonzero(n == 0).tolist()}")
        qkv = [wl.device_step_qkv(work, l, 10_000 + s, 1, DEV, "ddec") for l in range(2)]
        outs_f, outs_t, slots = [], [], []
        for l, (q, k, v) in enumerate(qkv):
            sf = torch.full((work.batch, 1), -7, dtype=torch.int32, device=DEV)
            st = torch.full((work.batch, 1), -7, dtype=torch.int32, device=DEV)
            outs_f.append(fused.append_attend(l, q, k, v, n, slot_out=sf))
            two.append(l, k, v, n, slot_out=st)
            outs_t.append(two.attend(l, q))
            slots.append((sf, st))
        fused.advance()
        two.advance()
        torch.cuda.synchronize()
        for l in range(2):
            diff = float((outs_f[l].float() - outs_t[l].float()).abs().max())
            assert torch.equal(outs_f[l], outs_t[l]), \
                f"step {s} layer {l}: fused != two calls (max abs diff {diff:.3e})"
            assert torch.isfinite(outs_f[l].float()).all()
            _slots_ok(slots[l][0], lens, n, 1, work, l, f"step {s} layer {l} fused")
            _slots_ok(slots[l][1], lens, n, 1, work, l, f"step {s} layer {l} two calls")
        m = so.check_step(n, qkv, outs_f, lambda b, nb: [0], f"decode_b64 step {s}")
        worst = (max(worst[0], m[0]), max(worst[1], m[1]))
        lens = lens + n
        assert fused.lens() == lens.tolist() == two.lens()
        assert fused.device_lens().tolist() == lens.tolist()
    say(f"  worst abs {worst[0]:.2e} rel {worst[1]:.2e} on rows {rows}")


def test_mixed_b32_full_size():
    # 32 rows, Hq 32 / Hkv 8, D 128, max_len 32768, starting lengths
    # ~ U[0, 30000]; right-padded C = 64 steps where half the rows decode one
    # token and the rest take 0..64.
    say("case: mixed_b32 full size (1 layer), sampled oracle")
    work = wl.MIXED_B32.replace(n_layer=1, n_kv_head=(8,), window=(0,))
    lens0 = wl.initial_lens_mixed_b32(work.batch)
    cache = K.Cache(K.config_from_workload(work), DEV)
    n_steps = [wl.n_new_mixed_b32(s, work.batch) for s in range(2)]
    n0 = n_steps[0]
    r = wl.rng("full_sizes", "mixed_rows")
    pick = {int(np.argmax(lens0)), int(np.argmin(lens0)), int(np.argmax(n0)),
            int(np.flatnonzero(n0 == 1)[0])}
    if (n0 == 0).any():
        pick.add(int(np.flatnonzero(n0 == 0)[0]))
    pick |= set(int(x) for x in r.choice(work.batch, 1))
    rows = sorted(pick)
    so = SampledOracle(work, rows)
    _fill([cache], work, lens0, "mfill", so)
    lens = lens0.astype(np.int64)
    for s, n in enumerate(n_steps):
        say(f"  mixed step {s}: n_new {n.tolist()}")
        q, k, v = wl.device_step_qkv(work, 0, 20_000 + s, 64, DEV, "mstep")
        sl = torch.full((work.batch, 64), -7, dtype=torch.int32, device=DEV)
        cache.append(0, k, v, n, slot_out=sl)
        out = cache.attend(0, q)
        cache.advance()
        torch.cuda.synchronize()
        _slots_ok(sl, lens, n, 64, work, 0, f"mixed step {s}")
        o = out.float()
        assert torch.isfinite(o).all()
        pad = torch.arange(64, device=DEV)[None, :] >= torch.as_tensor(n, device=DEV)[:, None]
        assert (o[pad] == 0).all(), "padded / idle outputs not zero"
        mx, rel = so.check_step(n, [(q, k, v)], [out],
                                lambda b, nb: sorted({0, nb // 2, nb - 1}), f"mixed step {s}")
        say(f"    rows {rows}: worst abs {mx:.2e} rel {rel:.2e}")
        lens = lens + n
        assert cache.lens() == lens.tolist()


def test_long_5to1_full_size():
    # B 8, Hq 64 / Hkv 8, D 128, max_len 32768: a W = 512 ring layer and a
    # global layer (the 5:1 stack's two layer kinds), 510 prefill chunks of
    # 64 tokens then 128 one-token steps, ending exactly at max_len.
    say("case: long_5to1 full size (ring W=512 + global), sampled oracle")
    work = wl.LONG_5TO1.replace(n_layer=2, n_kv_head=(8, 8), window=(512, 0))
    sched = wl.schedule_long_5to1(batch=work.batch)
    cache = K.Cache(K.config_from_workload(work), DEV)
    rows = [0, 5]
    so = SampledOracle(work, rows)
    checks = {0, 8, 300, 509, 510, 577, len(sched) - 1}
    lens = np.zeros(work.batch, dtype=np.int64)
    for s, (n, C) in enumerate(sched):
        qkv = [wl.device_step_qkv(work, l, s, C, DEV, "long") for l in range(2)]
        outs, slots = [], []
        for l, (q, k, v) in enumerate(qkv):
            sl = torch.full((work.batch, C), -7, dtype=torch.int32, device=DEV)
            # (every step through kvc_append_attend, as the bench runs it:
            # the ring layer's chunk steps then take the unstaged form)
            outs.append(cache.append_attend(l, q, k, v, n, slot_out=sl))
            slots.append(sl)
        cache.advance()
        if s in checks:
            torch.cuda.synchronize()
            for l in range(2):
                _slots_ok(slots[l], lens, n, C, work, l, f"long step {s} layer {l}")
                assert torch.isfinite(outs[l].float()).all()
            qi = (lambda b, nb: [0, 31, 63]) if C > 1 else (lambda b, nb: [0])
            mx, rel = so.check_step(n, qkv, outs, qi, f"long step {s}")
            say(f"  step {s} (lens {int(lens[0])}): worst abs {mx:.2e} rel {rel:.2e}")
        else:
            for l in range(2):
                so.record(l, qkv[l][1], qkv[l][2], n)
        lens = lens + n
        if s % 100 == 0:
            say(f"  step {s + 1}/{len(sched)}")
    torch.cuda.synchronize()
    assert cache.lens() == [work.max_len] * work.batch
    z = torch.zeros(work.batch, 1, 8, work.head_dim, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(K.CacheFullError):
        cache.append(0, z, z, [1] + [0] * (work.batch - 1))


def test_decode_b64_paged_full_size():
    # The headline shape on a paged cache (pool = the contiguous cache's
    # rows) against the contiguous cache, bit for bit, with a sampled oracle
    # on a few rows; rows fill in turns, so their pages interleave.
    say("case: decode_b64 full size (2 layers), paged vs contiguous, sampled oracle")
    steps = 3
    work = wl.DECODE_B64.replace(n_layer=2, n_kv_head=(8, 8), window=(0, 0))
    paged_work = work.replace(n_pages=work.batch * work.max_len // 16)
    lens0 = np.minimum(wl.initial_lens_decode_b64(work.batch), work.max_len - steps)
    flat = K.Cache(K.config_from_workload(work), DEV)
    paged = K.Cache(K.config_from_workload(paged_work), DEV)
    r = wl.rng("full_sizes", "paged_rows")
    rows = sorted({int(np.argmax(lens0))} | set(int(x) for x in r.choice(work.batch, 3, replace=False)))
    so = SampledOracle(work, rows)
    _fill([flat, paged], work, lens0, "pfill", so)
    st = paged.page_stats()
    assert st["used"] == int(lens0.sum()) and st["allocated"] == int(sum(-(-int(L) // 16) for L in lens0)) * 16
    for s in range(steps):
        n = wl.n_new_decode_b64(s, work.batch)
        qkv = [wl.device_step_qkv(work, l, 30_000 + s, 1, DEV, "pdec") for l in range(2)]
        of, op = [], []
        for l, (q, k, v) in enumerate(qkv):
            flat.append(l, k, v, n)
            of.append(flat.attend(l, q))
            op.append(paged.append_attend(l, q, k, v, n) if s % 2 else
                      (paged.append(l, k, v, n), paged.attend(l, q))[1])
        flat.advance()
        paged.advance()
        torch.cuda.synchronize()
        for l in range(2):  # (odd steps: the paged cache through kvc_append_attend)
            assert torch.equal(of[l], op[l]), f"step {s} layer {l}: paged output differs"
        mx, rel = so.check_step(n, qkv, op, lambda b, nb: [0], f"paged decode_b64 step {s}")
        say(f"  step {s}: rows {rows} worst abs {mx:.2e} rel {rel:.2e}")
    assert paged.lens() == flat.lens()
