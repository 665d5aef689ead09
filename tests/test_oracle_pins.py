"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage it checks.  None of these tests calls the GPU
path; they run on any CPU in a few seconds.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from oracle import cache as ocache
from oracle import mask as omask
from oracle import rope as orope
from oracle import sizes as osizes
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(t):
    return t.double().numpy()


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------------------
# Offset mask: Lab 07 section 2 worked example; pycraft-1 self-test shapes.
# ---------------------------------------------------------------------------
def test_offset_mask_worked_example():
    rows = _golden_lines("offset_mask_t2_pos3.txt")
    expected = np.array([[c == "T" for c in r] for r in rows])
    got = oracle.offset_mask(2, 3)
    assert got.shape == (2, 5)
    assert np.array_equal(got, expected)


def test_offset_mask_pos0_is_upper_triangular():
    # Lab 07 section 2: with nothing cached it is the usual causal mask.
    for t in (1, 2, 5, 9):
        assert np.array_equal(oracle.offset_mask(t, 0), np.triu(np.ones((t, t), bool), k=1))


@pytest.mark.parametrize("q_len,offset", [(4, 7), (3, 1), (2, 2)])
def test_offset_mask_brute_force(q_len, offset):
    # pycraft-1 kv_cache.py self-test: mask[i][j] allowed iff j <= offset + i,
    # shape (q_len, offset + q_len).
    got = oracle.offset_mask(q_len, offset)
    assert got.shape == (q_len, offset + q_len)
    for i in range(q_len):
        for j in range(offset + q_len):
            assert bool(got[i, j]) == (not (j <= offset + i))


# ---------------------------------------------------------------------------
# Chunked prefill = one forward (Lab 07 section 3), incremental = full.
# ---------------------------------------------------------------------------
def _run_schedule(oc, work, schedule, tag=""):
    """Feed a schedule through an OracleCache; collect per-row outputs."""
    outs = [[[] for _ in range(oc.batch)] for _ in range(oc.n_layer)]
    for step, (n_new, C) in enumerate(schedule):
        layers = []
        for l in range(oc.n_layer):
            q, k, v = wl.step_qkv(work, l, step, C, tag)
            layers.append((_f64(q), _f64(k), _f64(v)))
        res = oc.step(n_new, layers)
        for l in range(oc.n_layer):
            for b in range(oc.batch):
                outs[l][b].append((layers[l], res[l][b, : n_new[b]], int(n_new[b])))
    return outs


def _collect_row(work, schedule, layer, b, tag=""):
    q_all, k_all, v_all = [], [], []
    for step, (n_new, C) in enumerate(schedule):
        q, k, v = wl.step_qkv(work, layer, step, C, tag)
        n = int(n_new[b])
        q_all.append(_f64(q)[b, :n]); k_all.append(_f64(k)[b, :n]); v_all.append(_f64(v)[b, :n])
    return np.concatenate(q_all), np.concatenate(k_all), np.concatenate(v_all)


def _oracle_for(work, batch=None):
    return oracle.OracleCache(batch or work.batch, work.n_q_head, work.n_kv_head,
                              work.head_dim, work.max_len, work.window, work.rope_base)


def _incremental_vs_full(work, schedule, tag="", tol=1e-12):
    oc = _oracle_for(work)
    outs = _run_schedule(oc, work, schedule, tag)
    worst = 0.0
    for l in range(work.n_layer):
        for b in range(work.batch):
            q, k, v = _collect_row(work, schedule, l, b, tag)
            full = oracle.full_forward(q, k, v, work.window[l], work.rope_base)
            inc = np.concatenate([o for (_, o, _) in outs[l][b]], axis=0)
            assert inc.shape == full.shape
            worst = max(worst, float(np.abs(inc - full).max()) if inc.size else 0.0)
    assert worst <= tol, worst
    return worst


def test_chunked_prefill_5_5_5_2_equals_single_forward():
    # Lab 07 section 3: a 17-token prompt as chunks 5,5,5,2 gives the same
    # result as one 17-token forward (the lab's bar is 1e-5; fp64 here).
    work = wl.SMALL_FP32
    sched = [(np.array([n]), n) for n in (5, 5, 5, 2)]
    _incremental_vs_full(work, sched)


def test_small_fp32_whole_schedule_equals_full():
    _incremental_vs_full(wl.SMALL_FP32, wl.schedule_small_fp32())


_TWO_LAYER = wl.Workload("pin_two_layer", 2, 2, 8, (2, 2), 16, 40, (0, 0), "f32", 8)


def test_prefill_then_decode_equals_full_two_layers():
    # Lab 07 "What to implement" row 3: prefill 8 then decode 12 one at a
    # time equals a full forward; two layers so that a mistimed advance shows.
    sched = [(np.array([8, 8]), 8)] + [(np.array([1, 1]), 1)] * 12
    _incremental_vs_full(_TWO_LAYER, sched)


def test_chunks_of_five_equal_full_two_layers():
    sched = [(np.array([5, 5]), 5)] * 4
    _incremental_vs_full(_TWO_LAYER, sched)


def test_ragged_rows_equal_full():
    # Per-row lengths differ: rows with n_new 0 are untouched (tiny_agent
    # append docstring), right-padded chunks (C larger than a row's n_new).
    work = wl.Workload("pin_ragged", 2, 3, 4, (2, 1), 8, 40, (0, 3), "f32", 8)
    sched = [(np.array([3, 0, 5]), 6), (np.array([1, 4, 0]), 4), (np.array([0, 1, 7]), 8),
             (np.array([2, 2, 2]), 3), (np.array([1, 0, 1]), 1)]
    _incremental_vs_full(work, sched)


def test_padded_and_idle_outputs_are_zero():
    work = wl.Workload("pin_pad", 1, 3, 4, (2,), 8, 20, (0,), "f32", 6)
    oc = _oracle_for(work)
    q, k, v = wl.step_qkv(work, 0, 0, 6)
    out = oc.step(np.array([2, 0, 6]), [(_f64(q), _f64(k), _f64(v))])[0]
    assert np.all(out[0, 2:] == 0) and np.all(out[1] == 0)
    assert np.all(np.abs(out[0, :2]).sum(-1) > 0) and np.all(np.abs(out[2]).sum(-1) > 0)


# ---------------------------------------------------------------------------
# Ring = full cache + window mask (colibri PR, TL;DR and "Tests done").
# ---------------------------------------------------------------------------
def _ring_vs_window(work, phases, ring_cls=oracle.RingModel, tag="", window_fn=None):
    """Run layer 0 (a sliding layer) through a RingModel and an OracleCache."""
    W = work.window[0]
    ring = ring_cls(work.batch, work.n_q_head, work.n_kv_head[0], work.head_dim, W,
                    work.rope_base)
    one = work.replace(n_layer=1, n_kv_head=work.n_kv_head[:1], window=(W,))
    oc = _oracle_for(one)
    step = 0
    diffs = []
    for pi, phase in enumerate(phases):
        if pi > 0:
            rows = np.arange(work.batch)
            ring.reset(rows)
            oc.reset(rows)
        for n_new, C in phase:
            q, k, v = wl.step_qkv(one, 0, step, C, tag)
            ref = oc.step(n_new, [(_f64(q), _f64(k), _f64(v))])[0]
            got = ring.step(n_new, _f64(q), _f64(k), _f64(v))
            diffs.append(np.array_equal(ref, got))
            step += 1
    return all(diffs)


def test_ring_equals_full_with_window_bit_identical():
    work = wl.RING_BF16
    phase1, phase2 = wl.schedule_ring_bf16(work.batch)
    assert _ring_vs_window(work, [phase1, phase2])


def test_ring_equals_window_random_chunks():
    # Chunks wider than W, idle rows and a dirty ring after reset.
    work = wl.Workload("pin_ring_rand", 1, 3, 4, (2,), 16, 200, (5,), "f32", 16)
    r = wl.rng("pin_ring_rand")
    phases = []
    for _ in range(3):
        ph = []
        for _ in range(10):
            n = r.integers(0, 13, size=3)
            ph.append((n, int(max(1, n.max()))))
        phases.append(ph)
    assert _ring_vs_window(work, phases)


# ---------------------------------------------------------------------------
# Exhaustive index simulation of the addressing model (colibri PR,
# "Tests done": prefill, decode, window >= max_t, reuse over a dirty ring).
# ---------------------------------------------------------------------------
def _simulate_addressing(W, max_len, rng):
    ring = ocache.is_ring(W, max_len)
    rows = ocache.ring_rows(W, max_len)
    scratch = rows
    tags = np.full(rows + 1, -1, dtype=np.int64)
    lens = 0
    for _ in range(12):
        if rng.random() < 0.15:
            lens = 0                               # reset: tags stay dirty
            continue
        room = max_len - lens
        n = int(rng.integers(0, room + 1)) if room > 0 else 0
        C = n + int(rng.integers(0, 3))
        if C == 0:
            continue
        slots = oracle.slot_indices([lens], [n], C, W, max_len)[0]
        # padded tokens always go to scratch
        assert np.all(slots[n:] == scratch)
        # reads of every valid query: history from the ring, the chunk from staging
        for i in range(n):
            p = lens + i
            lo = max(0, p - W + 1) if W > 0 else 0
            for t in range(lo, p + 1):
                if t < lens:
                    s = t % W if ring else t
                    assert s != scratch
                    assert tags[s] == t, (W, max_len, lens, n, p, t, s, tags)
        # commit
        new_lens = lens + n
        for i in range(n):
            p = lens + i
            if ring:
                kept = p >= new_lens - W
                assert slots[i] == (p % W if kept else scratch)
            else:
                assert slots[i] == p
            if slots[i] != scratch:
                tags[slots[i]] = p
        lens = new_lens
        if ring:
            # after a step the ring holds exactly positions [max(0, lens-W), lens)
            want = set(range(max(0, lens - W), lens))
            have = {int(tags[(t % W)]) for t in want}
            assert have == want
            if n == 1:
                # one-token step: the visible window occupies slots [0, min(p+1, W))
                p = lens - 1
                vis = {int(x) for x in tags[: min(p + 1, W)]}
                assert vis == set(range(max(0, p - W + 1), p + 1))


def test_exhaustive_index_simulation():
    rng = np.random.default_rng(830)
    for W in range(1, 10):
        for max_len in range(1, 25):
            for _ in range(6):
                _simulate_addressing(W, max_len, rng)


def test_window_at_least_max_len_is_full_layout():
    assert not ocache.is_ring(8, 8) and not ocache.is_ring(9, 8)
    s = oracle.slot_indices([3], [2], 4, 8, 8)
    assert list(s[0]) == [3, 4, 8, 8]
    # the window can never clip when W >= max_len: same output as global
    work = wl.Workload("pin_wmax", 1, 2, 4, (2,), 8, 12, (12,), "f32", 12)
    glob = work.replace(window=(0,))
    sched = [(np.array([5, 12]), 12), (np.array([1, 0]), 1)]
    a = _oracle_for(work); b = _oracle_for(glob)
    for step, (n, C) in enumerate(sched):
        q, k, v = wl.step_qkv(work, 0, step, C)
        x = a.step(n, [(_f64(q), _f64(k), _f64(v))])[0]
        y = b.step(n, [(_f64(q), _f64(k), _f64(v))])[0]
        assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# Left padding (tinyllm module docstring; padded_causal_mask) and shifts.
# ---------------------------------------------------------------------------
def test_left_padding_invariance():
    g = np.random.default_rng(7)
    T, P, Hq, Hkv, D = 9, 4, 4, 2, 8
    q = g.standard_normal((T, Hq, D)); k = g.standard_normal((T, Hkv, D)); v = g.standard_normal((T, Hkv, D))
    pad = lambda x: np.concatenate([g.standard_normal((P,) + x.shape[1:]) * 5, x])
    plain = oracle.full_forward(q, k, v)
    padded = oracle.full_forward(pad(q), pad(k), pad(v), first=P)
    assert np.abs(padded[P:] - plain).max() <= 1e-12


def test_position_shift_invariance():
    g = np.random.default_rng(8)
    T, Hq, Hkv, D, shift = 7, 4, 2, 16, 1234
    q = g.standard_normal((T, Hq, D)); k = g.standard_normal((T, Hkv, D)); v = g.standard_normal((T, Hkv, D))
    blocked = np.arange(T)[None, :] > np.arange(T)[:, None]
    outs = []
    for s in (0, shift):
        pos = np.arange(T) + s
        outs.append(oatt.attend_rows(orope.rotate(q, pos, 1e4), orope.rotate(k, pos, 1e4), v, blocked))
    assert np.abs(outs[0] - outs[1]).max() <= 1e-10


# ---------------------------------------------------------------------------
# Left-padded rows in the incremental oracle (tinyllm kv_cache.py:
# padded_causal_mask, and the slot cache's admit / release).
# ---------------------------------------------------------------------------
_PAD_WORK = wl.Workload("pin_leftpad", 2, 3, 8, (2, 4), 16, 64, (0, 6), "f32", 40)


def _leftpad_tokens(pads, reals, seed=11):
    """Per row: pads[b] pad tokens (large random values) then reals[b] real
    tokens, per layer; returns q, k, v lists [layer][row] of (P+R, H, D)."""
    g = np.random.default_rng(seed)
    w = _PAD_WORK
    out = []
    for l in range(w.n_layer):
        hk = w.n_kv_head[l]
        rows = []
        for P, R in zip(pads, reals):
            mk = lambda h, scale: g.standard_normal((P + R, h, w.head_dim)) * scale
            q, k, v = mk(w.n_q_head, 1.0), mk(hk, 1.0), mk(hk, 1.0)
            q[:P] *= 5; k[:P] *= 5; v[:P] *= 5
            rows.append((q, k, v))
        out.append(rows)
    return out


def _feed(oc, toks, starts, counts, C):
    """One step: row b takes tokens starts[b] .. starts[b]+counts[b]-1."""
    layers = []
    for l in range(oc.n_layer):
        hq, hk, D = oc.n_q_head, oc.n_kv_head[l], oc.head_dim
        q = np.zeros((oc.batch, C, hq, D)); k = np.zeros((oc.batch, C, hk, D)); v = np.zeros_like(k)
        for b in range(oc.batch):
            s, n = starts[b], counts[b]
            tq, tk, tv = toks[l][b]
            q[b, :n], k[b, :n], v[b, :n] = tq[s:s + n], tk[s:s + n], tv[s:s + n]
        layers.append((q, k, v))
    return oc.step(np.asarray(counts), layers)


def _leftpad_run(pads, reals, prefill_chunk, decodes):
    """Outputs per step of an unpadded and a left-padded run of the same real
    tokens: lists of (layer outputs, starts, counts) for each run."""
    w = _PAD_WORK
    n_tok = [R + decodes for R in reals]
    toks_pad = _leftpad_tokens(pads, n_tok)
    toks_plain = [[(q[P:], k[P:], v[P:]) for (q, k, v), P in zip(rows, pads)] for rows in toks_pad]
    runs = []
    for toks, lead, first in ((toks_plain, [0] * len(pads), False), (toks_pad, pads, True)):
        oc = _oracle_for(w)
        if first:
            oc.set_first(np.arange(w.batch), pads)
        steps = []
        done = [0] * w.batch
        prompt = [L + R for L, R in zip(lead, reals)]
        while any(d < p for d, p in zip(done, prompt)):
            cnt = [min(prefill_chunk, p - d) for d, p in zip(done, prompt)]
            steps.append((_feed(oc, toks, list(done), cnt, prefill_chunk), list(done), cnt))
            done = [d + c for d, c in zip(done, cnt)]
        for _ in range(decodes):
            cnt = [1] * w.batch
            steps.append((_feed(oc, toks, list(done), cnt, 1), list(done), cnt))
            done = [d + 1 for d in done]
        runs.append((steps, toks))
    return runs


def _token_outputs(steps, batch, n_layer):
    """[layer][row] -> outputs of every token, in position order."""
    res = [[[] for _ in range(batch)] for _ in range(n_layer)]
    for outs, starts, counts in steps:
        for l in range(n_layer):
            for b in range(batch):
                res[l][b].append(outs[l][b, :counts[b]])
    return [[np.concatenate(r) for r in rl] for rl in res]


@pytest.mark.parametrize("chunk", [40, 5])
def test_oracle_left_padded_rows_equal_unpadded(chunk):
    # tinyllm kv_cache.py module docstring: with left padding no per-row RoPE
    # positions are needed (RoPE depends on distances only and padding shifts
    # a row's real tokens alike); pad keys are masked.  So the real tokens'
    # outputs of a left-padded row equal those of the same row unpadded, on a
    # global and a sliding (W = 6) layer, for a prefill in one chunk or in
    # chunks of 5 and for decode steps after it.
    pads, reals, decodes = [4, 0, 9], [7, 11, 3], 8
    (plain, _), (padded, toks) = _leftpad_run(pads, reals, chunk, decodes)
    w = _PAD_WORK
    a = _token_outputs(plain, w.batch, w.n_layer)
    b = _token_outputs(padded, w.batch, w.n_layer)
    worst = 0.0
    for l in range(w.n_layer):
        for r in range(w.batch):
            P = pads[r]
            worst = max(worst, float(np.abs(b[l][r][P:] - a[l][r]).max()))
    assert worst <= 1e-12, worst


def test_oracle_pad_queries_see_only_themselves():
    # padded_causal_mask keeps the diagonal: a pad query's softmax has one
    # key, so its output is its own value (its KV head's), exactly.
    pads, reals = [4, 0, 9], [7, 11, 3]
    (_, _), (padded, toks) = _leftpad_run(pads, reals, 40, 0)
    w = _PAD_WORK
    b = _token_outputs(padded, w.batch, w.n_layer)
    for l in range(w.n_layer):
        rep = w.n_q_head // w.n_kv_head[l]
        for r in range(w.batch):
            P = pads[r]
            v = toks[l][r][2][:P]                              # (P, Hkv, D)
            assert np.array_equal(b[l][r][:P], np.repeat(v, rep, axis=1))


def test_oracle_admit_copies_rows():
    # SlotKVCache.admit: a finished (left-padded) prefill's rows become slots;
    # decoding the slots then equals decoding the prefill cache itself.
    w = _PAD_WORK
    pads, reals = [4, 0, 9], [7, 11, 3]
    toks = _leftpad_tokens(pads, [R + 4 for R in reals], seed=12)
    src = _oracle_for(w)
    src.set_first(np.arange(3), pads)
    prompt = [P + R for P, R in zip(pads, reals)]
    _feed(src, toks, [0, 0, 0], prompt, max(prompt))
    dst = _oracle_for(w)
    dst.admit([2, 0, 1], src, [0, 1, 2])
    assert list(dst.lens) == [prompt[1], prompt[2], prompt[0]]
    assert list(dst.first) == [pads[1], pads[2], pads[0]]
    perm = [1, 2, 0]
    toks_dst = [[rows[i] for i in perm] for rows in toks]
    for s in range(4):
        a = _feed(src, toks, [p + s for p in prompt], [1, 1, 1], 1)
        b = _feed(dst, toks_dst, [prompt[i] + s for i in perm], [1, 1, 1], 1)
        for l in range(w.n_layer):
            assert np.array_equal(a[l][perm], b[l])
    dst.reset([0])
    assert dst.lens[0] == 0 and dst.first[0] == 0


def test_mutation_left_pad_ignored(monkeypatch):
    monkeypatch.setattr(omask, "left_pad_blocked",
                        lambda qpos, kpos, first: np.zeros(np.broadcast(np.asarray(qpos), np.asarray(kpos)).shape, dtype=bool))
    assert _fails(lambda: test_oracle_left_padded_rows_equal_unpadded(40))


def test_mutation_left_pad_hides_diagonal(monkeypatch):
    monkeypatch.setattr(omask, "left_pad_blocked",
                        lambda qpos, kpos, first: np.asarray(kpos) < first + 0 * np.asarray(qpos))
    assert _fails(test_oracle_pad_queries_see_only_themselves)


# ---------------------------------------------------------------------------
# Hybrid layer groups (tiny_agent generate.py: a group-global K/V written by
# the group's full layer plus a per-layer ring, one softmax over both).
# ---------------------------------------------------------------------------
_GROUP = dict(n_kv_head=[2, 2, 2], window=[0, 5, 3], joint=[-1, 0, 0])


def _group_oracle(batch=2, max_len=40):
    return oracle.OracleCache(batch, 4, _GROUP["n_kv_head"], 16, max_len, _GROUP["window"],
                              joint=_GROUP["joint"])


def _group_inputs(g, B, C):
    return [(g.standard_normal((B, C, 4, 16)), g.standard_normal((B, C, 2, 16)),
             g.standard_normal((B, C, 2, 16))) for _ in range(3)]


def test_joint_layers_match_sdpa_over_both_stores():
    # torch's float64 scaled_dot_product_attention over the concatenated keys
    # of the group store (visible: j <= p) and the layer's ring (visible:
    # j <= p and p - j < W), heads expanded by repeat_interleave.
    g = np.random.default_rng(21)
    oc = _group_oracle(batch=1)
    steps = [(np.array([9]), 9), (np.array([4]), 4), (np.array([1]), 1)]
    hist = [[[], []] for _ in range(3)]
    for n, C in steps:
        layers = _group_inputs(g, 1, C)
        outs = oc.step(n, layers)
        for l in range(3):
            hist[l][0].append(layers[l][1][0, :n[0]])
            hist[l][1].append(layers[l][2][0, :n[0]])
        T = int(oc.lens[0])
        pos_q = np.arange(T - n[0], T)
        for l in (1, 2):
            parts_k, parts_v, masks = [], [], []
            for src, W in ((0, 0), (l, _GROUP["window"][l])):
                k = np.concatenate(hist[src][0]); v = np.concatenate(hist[src][1])
                parts_k.append(orope.rotate(k, np.arange(T), 1e4)); parts_v.append(v)
                j = np.arange(T)[None, :]
                ok = j <= pos_q[:, None]
                if W:
                    ok = ok & (pos_q[:, None] - j < W)
                masks.append(ok)
            K = torch.from_numpy(np.concatenate(parts_k)).permute(1, 0, 2).repeat_interleave(2, 0)
            V = torch.from_numpy(np.concatenate(parts_v)).permute(1, 0, 2).repeat_interleave(2, 0)
            Q = torch.from_numpy(orope.rotate(layers[l][0][0, :n[0]], pos_q, 1e4)).permute(1, 0, 2)
            M = torch.from_numpy(np.concatenate(masks, axis=1))
            ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=M)
            got = outs[l][0, :n[0]]
            assert np.abs(ref.permute(1, 0, 2).numpy() - got).max() <= 1e-12


def test_joint_with_identical_stores_equals_single():
    # duplicated keys (same K and V in the group store and in a ring that
    # sees every position) leave the softmax weights' ratios unchanged
    g = np.random.default_rng(22)
    dup = oracle.OracleCache(2, 4, [2, 2], 16, 40, [0, 40], joint=[-1, 0])
    single = oracle.OracleCache(2, 4, [2], 16, 40, [0])
    for n, C in ((np.array([7, 3]), 7), (np.array([1, 5]), 5), (np.array([1, 1]), 1)):
        q, k, v = _group_inputs(g, 2, C)[0]
        a = dup.step(n, [(q, k, v), (q, k, v)])[1]
        b = single.step(n, [(q, k, v)])[0]
        assert np.abs(a - b).max() <= 1e-12


def test_joint_layers_chunked_equals_single_chunk():
    g = np.random.default_rng(23)
    T = 17
    data = _group_inputs(g, 2, T)
    one, many = _group_oracle(), _group_oracle()
    full = one.step(np.array([T, T]), data)
    outs, done = [], 0
    for C in (5, 5, 5, 2):
        part = [tuple(x[:, done:done + C] for x in layer) for layer in data]
        outs.append(many.step(np.array([C, C]), part))
        done += C
    for l in (1, 2):
        got = np.concatenate([o[l] for o in outs], axis=1)
        assert np.abs(got - full[l]).max() <= 1e-12


def test_mutation_joint_ignored(monkeypatch):
    def own_only(self, layer, b, n):
        T = int(self.lens[b]) + n
        return (orope.rotate(self.hist_k[layer][b], np.arange(T), self.rope_base),
                self.hist_v[layer][b], self._blocked(layer, b, n))
    monkeypatch.setattr(ocache.OracleCache, "_keys", own_only)
    assert _fails(test_joint_layers_match_sdpa_over_both_stores)


# ---------------------------------------------------------------------------
# Sizes: Lab 07 answer 1; colibri PR "Expected memory savings".
# ---------------------------------------------------------------------------
def test_kv_bytes_lab07():
    (name, n_layer, batch, hkv, max_len, hd, nb, want), = _golden_lines("kv_bytes_lab07.txt")
    got = oracle.kv_nbytes(int(batch), [int(hkv)] * int(n_layer), int(hd), int(max_len),
                           [0] * int(n_layer), int(nb))
    assert got == int(want) == 98304


def _as_printed(x, printed: str) -> bool:
    """x rounds to the printed figure (within half a unit of its last digit)."""
    digits = len(printed.split(".")[1]) if "." in printed else 0
    return abs(x - float(printed)) <= 0.5 * 10.0 ** (-digits) + 1e-9


_INKLING_HKV = [16 if (l + 1) % 6 else 8 for l in range(66)]
_INKLING_W = [512 if (l + 1) % 6 else 0 for l in range(66)]


def test_inkling_memory_table():
    lines = _golden_lines("inkling_memory_table.txt")
    GiB, KiB, MiB = 2.0 ** 30, 2.0 ** 10, 2.0 ** 20
    assert sum(1 for l in range(66) if _INKLING_W[l]) == 55
    for ln in lines:
        if ln[0] == "table":
            ctx, full_gb, ring_gb, factor = int(ln[1]), float(ln[2]), float(ln[3]), float(ln[4])
            full = oracle.kv_nbytes(1, _INKLING_HKV, 128, ctx, _INKLING_W, 4, use_ring=False)
            ring = oracle.kv_nbytes(1, _INKLING_HKV, 128, ctx, _INKLING_W, 4, use_ring=True)
            assert _as_printed(full / GiB, ln[2])
            assert _as_printed(ring / GiB, ln[3])
            assert _as_printed(full / ring, ln[4])
        elif ln[0] == "per_token":
            full_kb = osizes.kv_bytes_per_token(_INKLING_HKV, 128, 4) / KiB
            ring_kb = osizes.kv_bytes_per_token(_INKLING_HKV, 128, 4, _INKLING_W, 32768) / KiB
            assert (full_kb, ring_kb) == (float(ln[1]), float(ln[2]))
        elif ln[0] == "sliding_total":
            hkv = [h for h, w in zip(_INKLING_HKV, _INKLING_W) if w]
            tot = oracle.kv_nbytes(1, hkv, 128, 32768, [512] * len(hkv), 4)
            assert tot / MiB == float(ln[1])


# ---------------------------------------------------------------------------
# Softmax / GQA: closed forms and a library routine.
# ---------------------------------------------------------------------------
def test_zero_query_gives_mean_of_visible_values():
    g = np.random.default_rng(1)
    K = g.standard_normal((6, 2, 8)); V = g.standard_normal((6, 2, 8))
    out = oracle.softmax_attend(np.zeros((4, 8)), K, V)
    assert np.abs(out[0] - V[:, 0].mean(0)).max() < 1e-14
    assert np.abs(out[3] - V[:, 1].mean(0)).max() < 1e-14


def test_single_visible_key_returns_its_value():
    g = np.random.default_rng(2)
    q, k, v = g.standard_normal((3, 4, 8)), g.standard_normal((3, 2, 8)), g.standard_normal((3, 2, 8))
    out = oracle.full_forward(q, k, v)          # position 0 sees only itself
    assert np.abs(out[0, :2] - v[0, 0]).max() < 1e-15
    out_w1 = oracle.full_forward(q, k, v, window=1)   # W = 1: only self, always
    for t in range(3):
        assert np.abs(out_w1[t, 2:] - v[t, 1]).max() < 1e-15


def test_identical_keys_give_mean_value():
    g = np.random.default_rng(3)
    K = np.repeat(g.standard_normal((1, 2, 8)), 5, axis=0)
    V = g.standard_normal((5, 2, 8))
    out = oracle.softmax_attend(g.standard_normal((4, 8)), K, V)
    assert np.abs(out[1] - V[:, 0].mean(0)).max() < 1e-14


def test_matches_torch_sdpa_float64():
    g = torch.Generator().manual_seed(4)
    B, T, Hq, Hkv, D, W = 1, 11, 8, 2, 16, 4
    q = torch.randn(T, Hq, D, generator=g, dtype=torch.float64)
    k = torch.randn(T, Hkv, D, generator=g, dtype=torch.float64)
    v = torch.randn(T, Hkv, D, generator=g, dtype=torch.float64)
    for window in (0, W):
        ours = oracle.full_forward(q.numpy(), k.numpy(), v.numpy(), window=window)
        pos = np.arange(T)
        qr = torch.from_numpy(orope.rotate(q.numpy(), pos, 1e4)).transpose(0, 1)[None]
        kr = torch.from_numpy(orope.rotate(k.numpy(), pos, 1e4)).transpose(0, 1)[None]
        vr = v.transpose(0, 1)[None]
        kr = kr.repeat_interleave(Hq // Hkv, dim=1)
        vr = vr.repeat_interleave(Hq // Hkv, dim=1)
        i = torch.arange(T)[:, None]; j = torch.arange(T)[None, :]
        allowed = j <= i
        if window:
            allowed &= (i - j) < window
        ref = torch.nn.functional.scaled_dot_product_attention(qr, kr, vr, attn_mask=allowed)
        ref = ref[0].transpose(0, 1).numpy()
        assert np.abs(ours - ref).max() <= 1e-12


# ---------------------------------------------------------------------------
# RoPE properties (tinyllm docstring: q.k depends only on the distance).
# ---------------------------------------------------------------------------
def test_rope_properties():
    g = np.random.default_rng(5)
    x = g.standard_normal((6, 3, 32))
    assert np.array_equal(orope.rotate(x, np.zeros(6), 1e4), x)
    r = orope.rotate(x, np.arange(6) * 1000 + 7, 1e4)
    assert np.abs(np.linalg.norm(r, axis=-1) - np.linalg.norm(x, axis=-1)).max() < 1e-12
    q = g.standard_normal((1, 1, 32)); k = g.standard_normal((1, 1, 32))
    for m, n in [(5, 2), (300, 17), (9000, 8999)]:
        lhs = (orope.rotate(q, [m], 1e4) * orope.rotate(k, [n], 1e4)).sum()
        rhs = (orope.rotate(q, [m - n], 1e4) * k).sum()
        assert abs(lhs - rhs) < 1e-9


def test_rope_half_split_unit_vector():
    # tiny_agent _rope_pos: pair (d, d + D/2); frequency theta_d = base^(-2d/D).
    D, p, base = 8, 3, 10000.0
    for d in range(D // 2):
        e = np.zeros((1, 1, D)); e[0, 0, d] = 1.0
        r = orope.rotate(e, [p], base)[0, 0]
        th = p * base ** (-2.0 * d / D)
        want = np.zeros(D); want[d] = math.cos(th); want[d + D // 2] = math.sin(th)
        assert np.abs(r - want).max() < 1e-15


# ---------------------------------------------------------------------------
# Mutations (Lab 07 "Common bugs"; pycraft-1 build_attn_mask; colibri PR
# "How it works"): each planted mistake must fail one of the checks above.
# ---------------------------------------------------------------------------
def _fails(fn):
    try:
        fn()
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def test_mutation_rope_restarts_each_chunk(monkeypatch):
    monkeypatch.setattr(ocache.OracleCache, "_query_positions", lambda self, b, n: np.arange(n))
    assert _fails(test_chunked_prefill_5_5_5_2_equals_single_forward)


def test_mutation_mask_built_square(monkeypatch):
    orig = omask.offset_mask
    monkeypatch.setattr(omask, "offset_mask", lambda t, pos: orig(t, 0))
    assert _fails(test_chunked_prefill_5_5_5_2_equals_single_forward)


def test_mutation_advance_inside_layer_loop(monkeypatch):
    def bad_step(self, n_new, layers):
        n_new = self.check_capacity(n_new)
        outs = []
        for l in range(self.n_layer):
            outs.append(self.layer_step(l, n_new, *layers[l]))
            self.advance(n_new)
        return outs
    monkeypatch.setattr(ocache.OracleCache, "step", bad_step)
    assert _fails(test_prefill_then_decode_equals_full_two_layers)


def test_mutation_ring_append_before_scoring():
    work = wl.RING_BF16
    phase1, phase2 = wl.schedule_ring_bf16(work.batch)
    bad = lambda *a, **k: oracle.RingModel(*a, append_first=True, **k)
    assert not _ring_vs_window(work, [phase1, phase2], ring_cls=bad)


def test_mutation_top_left_causal(monkeypatch):
    monkeypatch.setattr(omask, "offset_mask",
                        lambda t, pos: np.arange(pos + t)[None, :] > np.arange(t)[:, None])
    assert _fails(test_prefill_then_decode_equals_full_two_layers)


def test_mutation_window_off_by_one(monkeypatch):
    def loose(qpos, kpos, window):
        qpos = np.asarray(qpos); kpos = np.asarray(kpos)
        if window <= 0:
            return np.zeros(np.broadcast(qpos, kpos).shape, dtype=bool)
        return (qpos - kpos) > window
    monkeypatch.setattr(omask, "window_blocked", loose)
    assert _fails(test_ring_equals_full_with_window_bit_identical)


# ---------------------------------------------------------------------------
# Guards (tiny_agent append; pycraft-1 update; Lab 07 Tips).
# ---------------------------------------------------------------------------
def test_overflow_raises_and_leaves_state():
    work = wl.Workload("pin_full", 1, 2, 4, (2,), 8, 10, (0,), "f32", 8)
    oc = _oracle_for(work)
    q, k, v = wl.step_qkv(work, 0, 0, 8)
    oc.step(np.array([8, 3]), [(_f64(q), _f64(k), _f64(v))])
    before = (oc.lens.copy(), [h.copy() for h in oc.hist_k[0]])
    q, k, v = wl.step_qkv(work, 0, 1, 3)
    with pytest.raises(oracle.CacheFull):
        oc.step(np.array([3, 1]), [(_f64(q), _f64(k), _f64(v))])
    assert np.array_equal(oc.lens, before[0])
    assert all(np.array_equal(a, b) for a, b in zip(oc.hist_k[0], before[1]))
    # filling exactly to max_len is allowed
    z = lambda h: np.zeros((2, 7, h, 8))
    oc.step(np.array([2, 7]), [(z(4), z(2), z(2))])
    assert list(oc.lens) == [10, 10]


def test_reset_empties_rows():
    work = wl.Workload("pin_reset", 1, 2, 4, (2,), 8, 10, (0,), "f32", 8)
    oc = _oracle_for(work)
    q, k, v = wl.step_qkv(work, 0, 0, 4)
    oc.step(np.array([4, 4]), [(_f64(q), _f64(k), _f64(v))])
    oc.reset([1])
    assert list(oc.lens) == [4, 0] and oc.hist_k[0][1].shape[0] == 0


def test_query_rows_is_layer_step_restricted():
    # Sampled queries of a step (used to check outputs of large workloads)
    # equal the full step's outputs for those queries, bit for bit, on a
    # global and a sliding layer, after an uneven history built in one go.
    work = wl.Workload("pin_qrows", 2, 3, 8, (2, 4), 16, 60, (0, 5), "f32", 16)
    full, part = _oracle_for(work), _oracle_for(work)
    n0 = np.array([13, 0, 7])
    layers = [tuple(_f64(t) for t in wl.step_qkv(work, l, 0, 13)) for l in range(2)]
    full.step(n0, layers, compute=False)
    part.step(n0, layers, compute=False)
    n1 = np.array([9, 3, 1])
    layers = [tuple(_f64(t) for t in wl.step_qkv(work, l, 1, 9)) for l in range(2)]
    for l in range(2):
        exp = full.layer_step(l, n1, *layers[l])
        part.layer_step(l, n1, *layers[l], compute=False)
        for b in range(3):
            idx = np.arange(int(n1[b]))[::2]
            got = part.query_rows(l, b, int(n1[b]), layers[l][0][b], idx)
            assert np.array_equal(got, exp[b, idx])
