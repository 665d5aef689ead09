"""Decode throughput of cached GQA attention with append on one MI355X.

Workload (the headline case): continuous-batch decode over 32 full-cache
layers, B = 64 rows, Hq 32 / Hkv 8, head_dim 128, bf16, max_len 8192; initial
row lengths ~ U[1, 8128]; each step every row decodes one token except 6
idle rows (n_new = 0, redrawn per step).  The history is filled through the
real protocol in 64-token chunks before timing (untimed); q/k/v are
synthetic N(0, 1) tensors already resident in HBM.

One step = for each of the 32 layers one kvc_append_attend (an appending
decode kernel: RoPE + append of the new token + decode attention, then the
split merge), then one kvc_advance; the appending decode kernel is the
roofline kernel.  A second timed leg then runs the same steps through
kvc_append + kvc_attend (append, decode attention and split-merge kernels)
and reports it next to the headline (``--two-call`` makes it the headline,
``--no-other-leg`` skips it), and a
third replays a captured static step (kvc_static_begin, kvc_append_attend
per layer, kvc_advance) from a HIP graph, reported as ``graph``.  Warmup
steps run first; the timed steps are bracketed by torch.cuda.synchronize().
Kernel durations come from HIP events that each dispatch stamps at its own
start and end on the launch stream.

Further legs, each reported in its own object of the same JSON line:
``prefill`` (the chunk-attention kernel's MFMA rate on one global layer of
the long-context workload, prefilled in 510 chunks of 64), ``mixed`` (the
mixed workload: B32, max_len 32768, right-padded C = 64 steps mixing one-token
and chunk rows) and ``long_decode`` (one-token steps of the 66-layer 5:1
long-context stack at 32k, through both entry points).

Prints one JSON line.  ``--gpus N`` with N > 1 exits: this path runs on one
GPU.  ``--cpu-baseline-seconds 0`` skips the oracle timing.
"""

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import kv_cached_gqa_append_amd as K  # noqa: E402
import workloads as wl  # noqa: E402

PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "kv_cached_gqa_append_amd", "csrc", "kernels.hip")
COUNTER_SUMMARY = {False: os.path.join(ROOT, "profiles", "k_decode_decode_b64_hbm.md"),
                   True: os.path.join(ROOT, "profiles", "k_decode_fused_decode_b64_hbm.md")}
COPY_BYTES = 2 ** 30   # the --copy-probe device copy: 1 GiB read, 1 GiB written


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_kernel_bytes(lens, n_new, work):
    """Algorithmic bytes one decode launch (one layer) must move: the visible
    K and V rows of every decoding row read once per KV head, plus its
    queries read.  lens: lengths before the step."""
    s = work.dtype_bytes
    hkv, D, hq = work.n_kv_head[0], work.head_dim, work.n_q_head
    act = n_new == 1
    kv = int(((lens[act] + 1) * hkv * D * s * 2).sum())
    qb = int(act.sum()) * hq * D * s
    return kv + qb


def fused_kernel_bytes(lens, n_new, work):
    """Algorithmic bytes of one appending decode launch of kvc_append_attend
    (one layer): the decode bytes and every row's new (or padded) k and v
    read and written to its slot (the merge kernel writes the outputs)."""
    s = work.dtype_bytes
    hkv, D, B = work.n_kv_head[0], work.head_dim, work.batch
    return decode_kernel_bytes(lens, n_new, work) + B * hkv * D * s * 2 * 2


def step_bytes(lens, n_new, work):
    """Algorithmic bytes of one whole step (all layers): attention reads, the
    new rows (k, v read and written), queries read, outputs written."""
    s = work.dtype_bytes
    hkv, D, hq = work.n_kv_head[0], work.head_dim, work.n_q_head
    act = n_new == 1
    per_layer = decode_kernel_bytes(lens, n_new, work)
    per_layer += int(act.sum()) * (hkv * D * s * 2 * 2 + hq * D * s)
    return per_layer * work.n_layer


def kernels_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def workload_for(layers):
    work = wl.DECODE_B64
    if layers:
        work = work.replace(n_layer=layers, n_kv_head=work.n_kv_head[:layers],
                            window=work.window[:layers])
    return work


def plan_lens(work, steps, warmup, legs=1):
    """Initial lengths (clipped so every step of every timed leg fits) and the
    n_new schedule."""
    total = (steps + warmup) * legs
    lens0 = wl.initial_lens_decode_b64(work.batch)
    if lens0.max() + total > work.max_len:
        lens0 = np.minimum(lens0, work.max_len - total)
    return lens0, [wl.n_new_decode_b64(s, work.batch) for s in range(total)]


def timed_decode_bytes(work, steps, warmup, fused=False):
    """Algorithmic bytes of each timed decode launch, in launch order (runs
    of one timed leg, --no-other-leg)."""
    per_launch = fused_kernel_bytes if fused else decode_kernel_bytes
    lens0, sched = plan_lens(work, steps, warmup, 3)
    lens = lens0.copy()
    for s in range(warmup):
        lens = lens + sched[s]
    out = []
    for s in range(warmup, warmup + steps):
        out += [per_launch(lens, sched[s], work)] * work.n_layer
        lens = lens + sched[s]
    return out


def _kname(name):
    for k in ("k_decode", "k_combine", "k_append", "k_chunk", "k_advance", "k_commit",
              "k_set_rows", "k_generic", "k_static_begin"):
        if k in name:
            return k
    return name if len(name) <= 40 else name[:37] + "..."


def summarize_trace(trace_csv, steps, warmup, layers, fused=False):
    """Markdown table of the timed region of a rocprofv3 kernel trace of this
    bench: the dispatches from the first timed step's n_new upload on."""
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    names = [_kname(r["Kernel_Name"]) for r in rows]
    work = workload_for(layers)
    dec = [i for i, n in enumerate(names) if n == "k_decode"]
    # the timed steps' decode launches are the last steps * n_layer (the
    # prefill leg after them launches none); the region ends at the last
    # timed step's advance
    first = dec[-steps * work.n_layer]
    while names[first] != "k_set_rows":            # the step's n_new upload
        first -= 1
    last = dec[-1]
    while names[last] != "k_advance":              # the last timed step's advance
        last += 1
    sel = rows[first:last + 1]
    t0, t1 = int(sel[0]["Start_Timestamp"]), int(sel[-1]["End_Timestamp"])
    by = {}
    for r in sel:
        by.setdefault(_kname(r["Kernel_Name"]), []).append(
            (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    gaps = [(int(b["Start_Timestamp"]) - int(a["End_Timestamp"])) / 1e3
            for a, b in zip(sel[:-1], sel[1:])]
    nb = timed_decode_bytes(work, steps, warmup, fused)
    out = [f"timed region: {len(sel)} dispatches, {(t1 - t0) / 1e6:.3f} ms, "
           f"{(t1 - t0) / 1e3 / steps:.1f} us per step", "",
           "| kernel | dispatches | avg us | median us | min us | max us |",
           "|---|---|---|---|---|---|"]
    for k, v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
        v = np.asarray(v)
        out.append(f"| {k} | {len(v)} | {v.mean():.2f} | {np.median(v):.2f} | {v.min():.2f} | "
                   f"{v.max():.2f} |")
    g = np.asarray(gaps)
    out += ["", f"idle between dispatches: {g.sum() / 1e3:.3f} ms in total, {g.mean():.2f} us "
            f"average", ""]
    dv = np.asarray(by["k_decode"])
    out.append(f"k_decode: {np.mean(nb) / 1e9:.4f} GB algorithmic per launch / "
               f"{dv.mean():.2f} us = {np.mean(nb) / (dv.mean() * 1e3):.1f} GB/s")
    return "\n".join(out)


def summarize_counters(fetch_csv, write_csv, steps, warmup, layers, fused=False):
    """Markdown summary of FETCH_SIZE / WRITE_SIZE per timed decode dispatch,
    scaled by what the same counters read for the 1 GiB copy probe."""
    work = workload_for(layers)
    nb = timed_decode_bytes(work, steps, warmup, fused)
    vals = {}
    for tag, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Dispatch_Id"]))
        dec = [float(r["Counter_Value"]) * 1024 for r in rows if "k_decode" in r["Kernel_Name"]]
        copy = [float(r["Counter_Value"]) * 1024 for r in rows
                if "copyBuffer" in r["Kernel_Name"]]
        if not copy:
            raise SystemExit(f"{path}: no copy probe dispatch (run with --copy-probe)")
        factor = COPY_BYTES / copy[-1]
        vals[tag] = (np.asarray(dec[-len(nb):]) * factor, factor, copy[-1])
    fetch, ff, fc = vals["FETCH_SIZE"]
    write, wf, wc = vals["WRITE_SIZE"]
    traffic = fetch + write
    ratio = float(traffic.sum() / np.sum(nb))
    out = [f"copy probe (1 GiB read + 1 GiB written): FETCH_SIZE {fc / 1024:.1f} KiB -> factor "
           f"{ff:.3f}; WRITE_SIZE {wc / 1024:.1f} KiB -> factor {wf:.3f}", "",
           "| timed decode dispatch | FETCH bytes (scaled) | WRITE bytes (scaled) | traffic | "
           "algorithmic | traffic / algorithmic |", "|---|---|---|---|---|---|"]
    for i, (a, b, c) in enumerate(zip(fetch, write, nb)):
        out.append(f"| {i} | {a:.4e} | {b:.4e} | {a + b:.4e} | {c:.4e} | {(a + b) / c:.4f} |")
    out += ["", f"kernels_sha256_16: {kernels_sha()}",
            f"traffic_bytes_per_launch: {traffic.mean():.6e}",
            f"algorithmic_bytes_per_launch: {np.mean(nb):.6e}",
            f"traffic_ratio: {ratio:.4f}"]
    return "\n".join(out)


def summarize_mfma(csv_path, chunks, chunk=64):
    """Markdown summary of a rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
    GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 run of --prefill-only: MFMA
    busy fraction of the chunk-attention dispatches (busy cycles summed over
    the SIMDs / (active cycles x SIMDs)) and the bf16 MFMA flops they issued
    (MOPS x 512) against the algorithmic flops.  The trace reports
    GRBM_GUI_ACTIVE summed over the 8 XCDs' counters; active cycles are that
    sum / 8."""
    simds, xcds = 256 * 4, 8
    per = {}
    for r in csv.DictReader(open(csv_path)):
        if "k_chunk" not in r["Kernel_Name"]:
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), {})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    ids = sorted(per)
    busy = np.array([per[i]["SQ_VALU_MFMA_BUSY_CYCLES"] for i in ids])
    gui = np.array([per[i]["GRBM_GUI_ACTIVE"] for i in ids]) / xcds
    mops = np.array([per[i]["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for i in ids])
    util = busy / (gui * simds)
    work = wl.LONG_5TO1.replace(n_layer=1, n_kv_head=(8,), window=(0,))
    alg = prefill_flops(work, chunks * chunk)
    out = [f"k_chunk dispatches: {len(ids)}", "",
           "| dispatches | MFMA busy (mean) | MFMA busy (cycle-weighted) | bf16 MFMA flops issued | "
           "algorithmic flops | issued / algorithmic |", "|---|---|---|---|---|---|",
           f"| {len(ids)} | {util.mean():.4f} | {busy.sum() / (gui.sum() * simds):.4f} | "
           f"{mops.sum() * 512:.4e} | {alg:.4e} | {mops.sum() * 512 / alg:.3f} |", "",
           "| chunk index | active cycles | MFMA busy | issued TFLOP/s |", "|---|---|---|---|"]
    for i in list(range(0, len(ids), max(1, len(ids) // 10))) + [len(ids) - 1]:
        d = per[ids[i]]
        out.append(f"| {i} | {gui[i]:.0f} | {util[i]:.4f} | "
                   f"{mops[i] * 512 / (d['ns'] * 1e-9) / 1e12:.1f} |")
    return "\n".join(out)


def _union_us(iv):
    """Length of the union of (start, end) nanosecond intervals, in us."""
    tot, cs, ce = 0, None, None
    for a, b in sorted(iv):
        if ce is None or a > ce:
            if ce is not None:
                tot += ce - cs
            cs, ce = a, b
        else:
            ce = max(ce, b)
    if ce is not None:
        tot += ce - cs
    return tot / 1e3


def _csv_steps(path, order="Start_Timestamp", counter=None):
    """The dispatches of a rocprofv3 csv (kernel trace, or one counter of a
    --pmc run), cut into protocol steps: each step ends with its k_advance.
    A dispatch is (kind, start ns, end ns, counter value)."""
    rows = [r for r in csv.DictReader(open(path))
            if counter is None or r.get("Counter_Name") == counter]
    rows.sort(key=lambda r: int(r[order]))
    steps, cur = [], []
    for r in rows:
        cur.append((_kname(r["Kernel_Name"]), int(r["Start_Timestamp"]),
                    int(r["End_Timestamp"]), float(r.get("Counter_Value") or 0.0)))
        if cur[-1][0] == "k_advance":
            steps.append(cur)
            cur = []
    return steps, cur


def _split_layers(step, first="k_append"):
    """The dispatches of one step, per layer: each layer starts at its first
    kernel (k_append through kvc_append + kvc_attend, k_decode through
    kvc_append_attend); what precedes the first layer (the step's count
    upload) and the closing k_advance are left out.  first "chunk": chunk
    steps through kvc_append_attend, where a global layer starts at its
    k_append and a ring layer, which appends inside its one chunk launch, at
    a k_chunk once the open layer has had its own."""
    layers = []
    for d in step:
        if first == "chunk":
            start = d[0] == "k_append" or (
                d[0] == "k_chunk" and (not layers or any(x[0] in ("k_chunk", "k_combine")
                                                         for x in layers[-1])))
        else:
            start = d[0] == first
        if start:
            layers.append([])
        if layers and d[0] != "k_advance":
            layers[-1].append(d)
    return layers


def _kind_table(dispatches, n_steps):
    out = ["| kernel | dispatches | summed us | union of spans us | avg us | per step us |",
           "|---|---|---|---|---|---|"]
    by = {}
    for d in dispatches:
        by.setdefault(d[0], []).append(d)
    for k, v in sorted(by.items(), key=lambda kv: -sum(d[2] - d[1] for d in kv[1])):
        tot = sum(d[2] - d[1] for d in v) / 1e3
        out.append(f"| {k} | {len(v)} | {tot:.1f} | {_union_us([(d[1], d[2]) for d in v]):.1f} | "
                   f"{tot / len(v):.2f} | {tot / n_steps:.1f} |")
    return out


def _layer_table(steps, window, first="k_append", dec_bytes=None):
    """Per layer kind (global / sliding ring): mean span of a layer (first
    dispatch start to last dispatch end), mean time its kernels kept the GPU
    busy (union of spans) and the mean per kernel kind; with dec_bytes (the
    algorithmic bytes of one layer's decode launch, per kind), the decode
    kernel's rate."""
    per = {"global": {"span": [], "busy": [], "kinds": {}},
           "ring": {"span": [], "busy": [], "kinds": {}}}
    for st in steps:
        for l, lay in enumerate(_split_layers(st, first)):
            p = per["global" if window[l] == 0 else "ring"]
            p["span"].append((max(d[2] for d in lay) - min(d[1] for d in lay)) / 1e3)
            p["busy"].append(_union_us([(d[1], d[2]) for d in lay]))
            for d in lay:
                p["kinds"].setdefault(d[0], []).append((d[2] - d[1]) / 1e3)
    out = ["| layer kind | layers timed | span us (mean) | busy us (mean) | per-kind avg us |" +
           (" decode GB/s |" if dec_bytes else ""),
           "|---|---|---|---|---|" + ("---|" if dec_bytes else "")]
    for k, p in per.items():
        if not p["span"]:
            continue
        kinds = ", ".join(f"{n} {np.mean(v):.2f} x{len(v) / len(p['span']):.2g}"
                          for n, v in sorted(p["kinds"].items()))
        row = (f"| {k} | {len(p['span'])} | {np.mean(p['span']):.2f} | "
               f"{np.mean(p['busy']):.2f} | {kinds} |")
        if dec_bytes:
            dv = p["kinds"].get("k_decode")
            row += f" {dec_bytes[k] / (np.mean(dv) * 1e3):.0f} |" if dv else " |"
        out.append(row)
    return out


def _periods(steps):
    """Advance-end to advance-end periods of consecutive steps, in ms."""
    ends = [st[-1][2] for st in steps]
    return np.diff(np.asarray(ends, dtype=np.int64)) / 1e6


def summarize_legs(trace_csv, only, steps, mixed_layers):
    """Markdown summary of a rocprofv3 kernel trace of `bench.py --only mixed`
    or `--only long_decode`: the steps are cut at each k_advance and the legs
    located by their step counts (the history fill, then the legs' warmup,
    timed and per-layer steps in the order the leg runs them)."""
    all_steps, _ = _csv_steps(trace_csv)
    out = [f"{len(all_steps)} protocol steps in the trace", ""]
    if only == "mixed":
        timed = all_steps[-steps:]
        per = _periods(all_steps[-steps - 1:])
        disp = [d for st in timed for d in st]
        att = [d for d in disp if d[0] in ("k_decode", "k_chunk", "k_combine")]
        union_ms = _union_us([(d[1], d[2]) for d in att]) / 1e3
        work = wl.MIXED_B32.replace(n_layer=mixed_layers, n_kv_head=(8,) * mixed_layers,
                                    window=(0,) * mixed_layers)
        lens = wl.initial_lens_mixed_b32(work.batch).astype(np.int64)
        sched = [wl.n_new_mixed_b32(i, work.batch, work.max_chunk) for i in range(2 + steps)]
        for n in sched[:2]:
            lens = lens + n
        att_b = 0
        for n in sched[2:]:
            att_b += mixed_layer_work(work, lens, n)[0] * mixed_layers
            lens = lens + n
        gbs = att_b / (union_ms / 1e3) / 1e9
        out += [f"## Timed steps: the last {steps} ({mixed_layers} layers each)", "",
                f"step period (advance to advance): {per.mean():.3f} ms mean", "",
                f"attention kernels (decode, chunk, combine): union of spans "
                f"{union_ms:.3f} ms, summed "
                f"{sum(d[2] - d[1] for d in att) / 1e6:.3f} ms over {steps} steps", "",
                f"attention: {att_b / 1e9:.2f} GB algorithmic over the union = {gbs:.0f} GB/s, "
                f"{gbs / PEAK_HBM_GBS:.4f} of the HBM peak", ""]
        out += _kind_table(disp, steps)
        return "\n".join(out)
    work = wl.LONG_5TO1
    win, W, S, C4 = work.window, 4, steps, 4
    fill = len(wl.fill_plan(np.full(work.batch, 510 * 64), 64))
    legs = [("prefill: 510 chunk steps of 64 (kvc_append_attend)", 0, fill, "chunk")]
    o = fill + W
    legs.append(("decode, kvc_append + kvc_attend (timed steps)", o, o + S, "k_append"))
    o += S + C4 + W
    legs.append(("decode, kvc_append_attend (timed steps)", o, o + S, "k_decode"))
    o += S + C4 + W
    legs.append(("decode, replays of the captured static step (timed steps)", o, o + S,
                 "k_decode"))
    B, D, sz = work.batch, work.head_dim, work.dtype_bytes
    for title, a, b, first in legs:
        sel = all_steps[a:b]
        if len(sel) != b - a:
            out += [f"## {title}: trace holds {len(sel)} of its {b - a} steps", ""]
            continue
        per = _periods(all_steps[max(a - 1, 0):b])
        out += [f"## {title}", "", f"steps {a}..{b - 1} of the trace; step period (advance to "
                f"advance) {per.mean():.3f} ms mean, {np.median(per):.3f} ms median", ""]
        out += _kind_table([d for st in sel for d in st], len(sel))
        dec_bytes = None
        if a > 0:
            # one-token steps: a layer's decode reads every visible key (global:
            # all, ring: the W newest) of each row and KV head, its queries and
            # outputs; the appending kernel also reads and writes the new k, v
            L = 510 * 64 + (a - fill)
            qo = B * work.n_q_head * D * sz * 2 + (B * 8 * D * sz * 4 if first == "k_decode" else 0)
            dec_bytes = {"global": B * (L + 1) * 8 * D * sz * 2 + qo,
                         "ring": B * min(L + 1, max(work.window)) * 8 * D * sz * 2 + qo}
        out += [""] + _layer_table(sel, win, first, dec_bytes)
        out.append("")
    return "\n".join(out)


def summarize_mixed_counters(fetch_csv, write_csv, steps, layers):
    """Markdown summary of FETCH_SIZE / WRITE_SIZE (two rocprofv3 --pmc runs of
    `bench.py --only mixed --copy-probe`) over the timed steps, per kernel
    kind, scaled by what the counters read for the 1 GiB copy probe, against
    the algorithmic bytes of those steps."""
    work = wl.MIXED_B32.replace(n_layer=layers, n_kv_head=(8,) * layers, window=(0,) * layers)
    lens = wl.initial_lens_mixed_b32(work.batch).astype(np.int64)
    sched = [wl.n_new_mixed_b32(s, work.batch, work.max_chunk) for s in range(2 + steps)]
    for n in sched[:2]:
        lens = lens + n
    att = app = 0
    for n in sched[2:]:
        a, p, _, _ = mixed_layer_work(work, lens, n)
        att, app = att + a * layers, app + p * layers
        lens = lens + n
    res = {}
    for tag, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        st, tail = _csv_steps(path, "Dispatch_Id", tag)
        copy = [d[3] * 1024 for d in tail if "copyBuffer" in d[0]]
        if not copy:
            raise SystemExit(f"{path}: no copy probe dispatch after the last step (--copy-probe)")
        f = COPY_BYTES / copy[-1]
        by = {}
        for s in st[-steps:]:
            for d in s:
                by[d[0]] = by.get(d[0], 0.0) + d[3] * 1024 * f
        res[tag] = (by, f, copy[-1])
    fb, ff, fc = res["FETCH_SIZE"]
    wb, wf, wc = res["WRITE_SIZE"]
    kinds = sorted(set(fb) | set(wb), key=lambda k: -(fb.get(k, 0) + wb.get(k, 0)))
    out = [f"copy probe (1 GiB read + 1 GiB written): FETCH_SIZE {fc / 1024:.1f} KiB -> factor "
           f"{ff:.3f}; WRITE_SIZE {wc / 1024:.1f} KiB -> factor {wf:.3f}", "",
           f"timed steps: {steps}, {layers} layers each", "",
           "| kernel | FETCH bytes (scaled) | WRITE bytes (scaled) |", "|---|---|---|"]
    for k in kinds:
        out.append(f"| {k} | {fb.get(k, 0):.4e} | {wb.get(k, 0):.4e} |")
    attk = ("k_decode", "k_chunk", "k_combine")
    ta = sum(fb.get(k, 0) + wb.get(k, 0) for k in attk)
    tp = fb.get("k_append", 0) + wb.get("k_append", 0)
    out += ["", f"attention kernels (decode, chunk, combine): traffic {ta:.4e} B, algorithmic "
            f"{att:.4e} B, ratio {ta / att:.4f}",
            f"append kernel: traffic {tp:.4e} B, algorithmic {app:.4e} B, ratio "
            f"{tp / app if app else float('nan'):.4f}", "",
            f"kernels_sha256_16: {kernels_sha()}"]
    return "\n".join(out)


def counter_traffic(bytes_per_launch, fused):
    """HBM traffic per decode launch from the committed counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        text = open(COUNTER_SUMMARY[fused]).read()
    except OSError:
        return None
    kv = dict(l.split(": ", 1) for l in text.splitlines()
              if l.startswith(("kernels_sha256_16:", "traffic_ratio:",
                               "traffic_bytes_per_launch:")))
    if kv.get("kernels_sha256_16") != kernels_sha():
        return None
    ratio = float(kv["traffic_ratio"])
    return {"bytes": round(ratio * bytes_per_launch), "ratio": ratio,
            "measured_bytes_per_launch": float(kv["traffic_bytes_per_launch"])}


def copy_probe(dev):
    """A 1 GiB device-to-device copy: the reference the HBM counters are
    scaled by."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).random_()
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    log("[bench] copy probe: 1 GiB read + 1 GiB written")
    del src, dst


def fill_history(cache, work, target, dev):
    """Bring every row to target[b] tokens in chunk steps of at most 64
    tokens through kvc_append_attend and kvc_advance."""
    B, D = work.batch, work.head_dim
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed_of(work.name, "fill"))
    C = 64
    q = torch.randn(B, C, work.n_q_head, D, generator=g, device=dev).to(work.torch_dtype)
    k = torch.randn(B, C, work.n_kv_head[0], D, generator=g, device=dev).to(work.torch_dtype)
    v = torch.randn(B, C, work.n_kv_head[0], D, generator=g, device=dev).to(work.torch_dtype)
    out = torch.empty_like(q)
    plan = wl.fill_plan(target, C)
    t0 = time.perf_counter()
    for si, (n, Cs) in enumerate(plan):
        for l in range(work.n_layer):
            cache.append_attend(l, q[:, :Cs].contiguous(), k[:, :Cs].contiguous(),
                                v[:, :Cs].contiguous(), n, out=out[:, :Cs].contiguous())
        cache.advance()
        if si % 16 == 0:
            torch.cuda.synchronize()
            log(f"[bench] fill step {si + 1}/{len(plan)} ({time.perf_counter() - t0:.1f}s)")
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"[bench] history filled: {len(plan)} chunk steps in {dt:.1f}s")
    return dt


PEAK_BF16_TFLOPS = 2500.0


def prefill_flops(work, n_tokens):
    """Algorithmic FLOPs of attending a B-row prefill of n_tokens tokens on
    one global layer: query at position p sees p + 1 keys; 4 * D flops per
    (query head, key) for QK^T and PV."""
    return 4.0 * work.head_dim * work.n_q_head * work.batch * n_tokens * (n_tokens + 1) / 2


def prefill_leg(dev, chunks, chunk=64):
    """Chunked prefill of one global layer of the long-context workload (B 8,
    Hq 64 / Hkv 8, D 128, bf16) to chunks * 64 tokens through the protocol,
    timing every chunk-attention launch: the MFMA-bound part of that
    workload's prefill."""
    work = wl.LONG_5TO1.replace(n_layer=1, n_kv_head=(8,), window=(0,))
    cache = K.Cache(K.config_from_workload(work), dev)
    B, D = work.batch, work.head_dim
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed_of(work.name, "prefill"))
    q = torch.randn(B, chunk, work.n_q_head, D, generator=g, device=dev).to(work.torch_dtype)
    k = torch.randn(B, chunk, 8, D, generator=g, device=dev).to(work.torch_dtype)
    v = torch.randn(B, chunk, 8, D, generator=g, device=dev).to(work.torch_dtype)
    out = torch.empty_like(q)
    n = np.full(B, chunk)
    K.kvc_timing_begin(cache.handle, chunks * 4 + 16)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(chunks):
        cache.append(0, k, v, n)
        cache.attend(0, q, out)
        cache.advance()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kt = K.kvc_timing_end(cache.handle)
    ms, launches = kt["chunk"]
    flops = prefill_flops(work, chunks * chunk)
    tflops = flops / (ms / 1e3) / 1e12
    log(f"[bench] prefill: {chunks} chunks of {chunk} to {chunks * chunk} tokens, chunk kernel "
        f"{ms:.1f} ms ({tflops:.0f} TFLOP/s), wall {dt * 1e3:.1f} ms")
    cache.close()
    return {"workload": f"long_5to1 global layer: B{B}, Hq{work.n_q_head}/Hkv8, D{D}, bf16, "
                        f"{chunks} chunks of {chunk} to {chunks * chunk} tokens",
            "kernel": "k_chunk<128,8>", "bound": "mfma", "unit": "TFLOP/s",
            "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "flops": flops,
            "chunk_kernel_ms": round(ms, 3), "launches": launches,
            "wall_ms": round(dt * 1e3, 3),
            "tokens_per_s": round(B * chunks * chunk / dt, 1)}


def mixed_layer_work(work, lens, n):
    """Algorithmic work of one layer of a right-padded mixed step: query i of
    row b (i < n_b) sits at position lens_b + i and sees lens_b + i + 1 keys.
    Returns (attention bytes, append bytes, FLOPs of the chunk rows (n >= 2),
    FLOPs of every row).  Attention bytes: each active row's visible K and V
    read once per KV head, its valid queries read and outputs written.
    Append bytes: every new k and v row read and written."""
    s = work.dtype_bytes
    hkv, hq, D = work.n_kv_head[0], work.n_q_head, work.head_dim
    lens = np.asarray(lens, dtype=np.int64)
    n = np.asarray(n, dtype=np.int64)
    act = n > 0
    att = int(((lens[act] + n[act]) * hkv * D * s * 2).sum()) + int(n.sum()) * hq * D * s * 2
    app = int(n.sum()) * hkv * D * s * 2 * 2
    keys = n * lens + n * (n + 1) // 2          # summed over the row's queries
    fl_all = 4.0 * D * hq * float(keys.sum())
    fl_chunk = 4.0 * D * hq * float(keys[n >= 2].sum())
    return att, app, fl_chunk, fl_all


def mixed_leg(dev, steps, warmup, layers):
    """The mixed workload (B 32, Hq 32 / Hkv 8, D 128, bf16, max_len 32768,
    right-padded C = 64 steps where half the rows decode one token and the
    rest take n_new ~ U{0..64}; initial lengths ~ U[0, 30000]) over
    ``layers`` full layers.  Attention GB/s = algorithmic bytes over the
    time the decode, chunk and combine launches kept the GPU busy (the union
    of their spans: the two chunk launches overlap on two streams); the chunk
    kernel's MFMA utilisation = the chunk rows' FLOPs over the union of its
    launches' spans; tokens/s = new
    tokens over the wall time of whole steps (append + attend per layer,
    advance)."""
    base = wl.MIXED_B32
    work = base.replace(n_layer=layers, n_kv_head=base.n_kv_head[:1] * layers,
                        window=(0,) * layers)
    lens0 = wl.initial_lens_mixed_b32(work.batch)
    cfg = K.config_from_workload(work)
    log(f"[bench] mixed: {layers} layers, buffer {K.kvc_nbytes(cfg, K.KVC_NB_ALLOC) / 2**30:.2f} GiB")
    cache = K.Cache(cfg, dev)
    fill_history(cache, work, lens0, dev)
    B, D, C = work.batch, work.head_dim, work.max_chunk
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed_of(work.name, "mixed"))
    mk = lambda h: torch.randn(B, C, h, D, generator=g, device=dev).to(work.torch_dtype)
    qs = [mk(work.n_q_head) for _ in range(layers)]
    ks = [mk(8) for _ in range(layers)]
    vs = [mk(8) for _ in range(layers)]
    outs = [torch.empty_like(x) for x in qs]
    sched = [wl.n_new_mixed_b32(s, B, C) for s in range(warmup + steps)]

    def run_step(n):
        for l in range(layers):
            cache.append(l, ks[l], vs[l], n)
            cache.attend(l, qs[l], outs[l])
        cache.advance()

    for n in sched[:warmup]:
        run_step(n)
    torch.cuda.synchronize()
    lens = np.asarray(cache.lens(), dtype=np.int64)
    att = app = flc = fla = tokens = 0
    for n in sched[warmup:]:
        a, p, fc, fa = mixed_layer_work(work, lens, n)
        att, app, flc, fla = att + a * layers, app + p * layers, flc + fc * layers, fla + fa * layers
        tokens += int(n.sum())
        lens = lens + n
    K.kvc_timing_begin(cache.handle, steps * layers * 6 + 16)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for n in sched[warmup:]:
        run_step(n)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    spans = K.kvc_timing_spans(cache.handle, steps * layers * 6 + 16)
    kt = K.kvc_timing_end(cache.handle)
    assert cache.lens() == lens.tolist()
    cache.close()
    # The 8-wave and 4-wave chunk launches run side by side on two streams:
    # kernel time is the union of the launches' spans (overlaps counted
    # once), the time the attention kernels kept the GPU busy.
    att_ms = K.busy_ms(spans, {"decode", "chunk", "combine"})
    chunk_ms = K.busy_ms(spans, {"chunk"})
    att_sum_ms = sum(kt[k][0] for k in ("decode", "chunk", "combine"))
    gbs = att / (att_ms / 1e3) / 1e9
    tf = flc / (chunk_ms / 1e3) / 1e12 if chunk_ms > 0 else 0.0
    kinds = {k: {"ms_total": round(v[0], 3), "launches": v[1],
                 "us_avg": round(v[0] * 1e3 / v[1], 2) if v[1] else None}
             for k, v in kt.items() if v[1]}
    log(f"[bench] mixed: {steps} steps in {dt:.3f}s ({dt * 1e3 / steps:.2f} ms/step over {layers} "
        f"layers), {tokens / dt:.0f} new tok/s, attention kernels {gbs:.0f} GB/s, chunk kernel "
        f"{tf:.0f} TFLOP/s (union of launch spans)")
    log(f"[bench] mixed kernels: {json.dumps(kinds)}")
    return {"workload": (f"mixed_b32: {layers} full layers, B{B}, Hq{work.n_q_head}/Hkv8, D{D}, "
                         f"bf16, max_len {work.max_len}, C={C}, half the rows n_new=1 and the "
                         f"rest U{{0..{C}}}, initial lens U[0,30000]"),
            "steps": steps, "warmup": warmup, "ms_per_step": round(dt * 1e3 / steps, 4),
            "tokens_per_s": round(tokens / dt, 1),
            "attention": {"bound": "hbm", "unit": "GB/s", "achieved": round(gbs, 1),
                          "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
                          "bytes": att, "kernel_ms": round(att_ms, 3),
                          "kernel_ms_summed": round(att_sum_ms, 3),
                          "kernels": "k_decode<128,4> + k_chunk<128,4> + k_combine",
                          "kernel_ms_is": "union of the launches' own spans (the two chunk "
                                          "launches overlap on two streams; counted once)"},
            "chunk_mfma": {"kernel": "k_chunk<128,4>", "unit": "TFLOP/s",
                           "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS,
                           "frac": round(tf / PEAK_BF16_TFLOPS, 4), "flops": flc,
                           "kernel_ms": round(chunk_ms, 3)},
            "flops_all_rows": fla, "append_bytes": app, "kernels": kinds}


def long_decode_leg(dev, steps, warmup, class_steps=4):
    """Decode of the long-context 5:1 stack (66 layers: 55 sliding W = 512
    rings, 11 global; B 8, Hq 64 / Hkv 8, D 128, bf16, max_len 32768) after
    its 510-chunk prefill to 32,640 tokens, one token per row per step, timed
    through both entry points in turn (kvc_append + kvc_attend, then
    kvc_append_attend), then as replays of a captured static step.  Attention GB/s = algorithmic bytes (global layers
    read every key, ring layers min(p + 1, W) keys; queries read, outputs
    written; through kvc_append_attend also the new k, v rows read and
    written)
    over the summed attention kernel time; a few more steps, timed a layer at
    a time, split that into global and ring layers."""
    work = wl.LONG_5TO1
    cfg = K.config_from_workload(work)
    full = K.config_from_workload(work.replace(use_ring=False))
    nb_ring, nb_full = K.kvc_nbytes(cfg, K.KVC_NB_KV), K.kvc_nbytes(full, K.KVC_NB_KV)
    log(f"[bench] long decode: KV {nb_ring / 2**30:.2f} GiB with rings "
        f"({nb_full / 2**30:.2f} GiB as full caches)")
    cache = K.Cache(cfg, dev)
    B, D, L = work.batch, work.head_dim, work.n_layer
    prefill = 510 * 64
    fill_s = fill_history(cache, work, np.full(B, prefill), dev)
    log(f"[bench] long prefill: {B * prefill / fill_s:.0f} tok/s over the {L}-layer stack "
        f"(510 chunk steps of 64 tokens, {fill_s:.2f} s wall, with the progress syncs)")
    assert 2 * (warmup + steps + class_steps) + warmup + steps <= work.max_len - prefill
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed_of(work.name, "decode"))
    mk = lambda h: torch.randn(B, 1, h, D, generator=g, device=dev).to(work.torch_dtype)
    qs = [mk(work.n_q_head) for _ in range(L)]
    ks = [mk(8) for _ in range(L)]
    vs = [mk(8) for _ in range(L)]
    outs = [torch.empty_like(x) for x in qs]
    n = np.ones(B, dtype=np.int64)
    s = work.dtype_bytes
    glob = [l for l in range(L) if work.window[l] == 0]

    def one_entry(fused):
        att_kinds = ("fused", "combine") if fused else ("decode", "combine")

        def layer_bytes(l, lens):
            vis = lens + 1 if work.window[l] == 0 else np.minimum(lens + 1, work.window[l])
            b = int((vis * 8 * D * s * 2).sum()) + B * work.n_q_head * D * s * 2
            return b + (B * 8 * D * s * 2 * 2 if fused else 0)

        def run_layer(l):
            if fused:
                cache.append_attend(l, qs[l], ks[l], vs[l], n, out=outs[l])
            else:
                cache.append(l, ks[l], vs[l], n)
                cache.attend(l, qs[l], outs[l])

        for _ in range(warmup):
            for l in range(L):
                run_layer(l)
            cache.advance()
        torch.cuda.synchronize()
        lens = np.asarray(cache.lens(), dtype=np.int64)
        att = sum(layer_bytes(l, lens + i) for i in range(steps) for l in range(L))
        K.kvc_timing_begin(cache.handle, steps * L * 4 + 16)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            for l in range(L):
                run_layer(l)
            cache.advance()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        kt = K.kvc_timing_end(cache.handle)
        att_ms = sum(kt[k][0] for k in att_kinds)
        # per layer kind: each layer's launches timed on their own
        per = {"global": [0, 0.0, 0], "ring": [0, 0.0, 0]}
        lens = np.asarray(cache.lens(), dtype=np.int64)
        for _ in range(class_steps):
            for l in range(L):
                K.kvc_timing_begin(cache.handle, 8)
                run_layer(l)
                t = K.kvc_timing_end(cache.handle)
                p = per["global" if l in glob else "ring"]
                p[0] += layer_bytes(l, lens)
                p[1] += sum(t[k][0] for k in att_kinds)
                p[2] += 1
            cache.advance()
            lens = lens + n
        gbs = att / (att_ms / 1e3) / 1e9
        by_kind = {k: {"layers": len(glob) if k == "global" else L - len(glob),
                       "gbs": round(v[0] / (v[1] / 1e3) / 1e9, 1) if v[1] else None,
                       "frac": (round(v[0] / (v[1] / 1e3) / 1e9 / PEAK_HBM_GBS, 4)
                                if v[1] else None),
                       "us_per_layer": round(v[1] * 1e3 / v[2], 2) if v[2] else None}
                   for k, v in per.items()}
        entry = "kvc_append_attend" if fused else "kvc_append+kvc_attend"
        log(f"[bench] long decode, {entry}: {steps} steps in {dt:.3f}s "
            f"({dt * 1e3 / steps:.3f} ms/step), {B * steps / dt:.0f} tok/s, attention kernels "
            f"{gbs:.0f} GB/s; by layer kind {json.dumps(by_kind)}")
        kinds = {k: {"ms_total": round(v[0], 3), "launches": v[1],
                     "us_avg": round(v[0] * 1e3 / v[1], 2) if v[1] else None}
                 for k, v in kt.items() if v[1]}
        return {"entry": entry, "ms_per_step": round(dt * 1e3 / steps, 4),
                "tokens_per_s": round(B * steps / dt, 1),
                "attention": {"bound": "hbm", "unit": "GB/s", "achieved": round(gbs, 1),
                              "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
                              "bytes": att, "kernel_ms": round(att_ms, 3)},
                "by_layer_kind": by_kind, "kernels": kinds}

    legs = [one_entry(False), one_entry(True)]

    def graph_step_bytes(lens, nn):
        tot = 0
        for l in range(L):
            vis = lens + 1 if work.window[l] == 0 else np.minimum(lens + 1, work.window[l])
            tot += int((vis * 8 * D * s * 2).sum()) + B * (work.n_q_head * D * s * 2 + 8 * D * s * 4)
        return tot

    gl = graph_leg(cache, work, qs, ks, vs, [n] * (warmup + steps), warmup, steps,
                   graph_step_bytes)
    log(f"[bench] long decode, graph replays: {gl['ms_per_step']:.3f} ms/step, "
        f"{gl['tokens_per_s']:.0f} tok/s, whole-step {gl['value']:.0f} GB/s")
    legs.append(gl)
    cache.close()
    return {"workload": (f"long_5to1 decode after a {prefill}-token prefill: {L} layers "
                         f"({L - len(glob)} sliding W=512 rings, {len(glob)} global), B{B}, "
                         f"Hq{work.n_q_head}/Hkv8, D{D}, bf16, max_len {work.max_len}"),
            "steps": steps, "warmup": warmup, "class_steps": class_steps,
            "kv_nbytes": {"rings": nb_ring, "full": nb_full},
            "prefill": {"tokens_per_s": round(B * prefill / fill_s, 1), "wall_s": round(fill_s, 3),
                        "what": "510 chunk steps of 64 tokens through kvc_append_attend "
                                "over all 66 layers, B 8, to 32,640 tokens"},
            "entries": legs}

def paged_leg(dev, steps, warmup):
    """The headline decode workload on a paged cache (a pool of B * max_len / 16
    pages, the contiguous cache's bytes; rows fill in turns, so their pages
    interleave in the pool), one-token steps through kvc_append +
    kvc_attend: the decode kernel's rate with a block-table lookup per tile."""
    base = wl.DECODE_B64
    work = base.replace(n_pages=base.batch * base.max_len // 16)
    lens0, sched = plan_lens(work, steps, warmup, 3)
    cache = K.Cache(K.config_from_workload(work), dev)
    fill_history(cache, work, lens0, dev)
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed_of(work.name, "paged"))
    B, D, L = work.batch, work.head_dim, work.n_layer
    mk = lambda h: torch.randn(B, 1, h, D, generator=g, device=dev).to(work.torch_dtype)
    qs = [mk(work.n_q_head) for _ in range(L)]
    ks = [mk(8) for _ in range(L)]
    vs = [mk(8) for _ in range(L)]
    outs = [torch.empty_like(x) for x in qs]

    def run_step(n):
        for l in range(L):
            cache.append(l, ks[l], vs[l], n)
            cache.attend(l, qs[l], outs[l])
        cache.advance()

    for n in sched[:warmup]:
        run_step(n)
    torch.cuda.synchronize()
    lens = np.asarray(cache.lens(), dtype=np.int64)
    kbytes = sbytes = tokens = 0
    for n in sched[warmup:warmup + steps]:
        kbytes += decode_kernel_bytes(lens, n, work) * L
        sbytes += step_bytes(lens, n, work)
        tokens += int(n.sum())
        lens = lens + n
    K.kvc_timing_begin(cache.handle, steps * L * 4 + 16)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for n in sched[warmup:warmup + steps]:
        run_step(n)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kt = K.kvc_timing_end(cache.handle)
    stats = cache.page_stats()
    cache.close()
    dec_ms, dec_n = kt["decode"]
    gbs = kbytes / (dec_ms / 1e3) / 1e9
    log(f"[bench] paged decode_b64: {steps} steps, {dt * 1e3 / steps:.3f} ms/step, "
        f"{tokens / dt:.0f} tok/s, decode kernel {dec_ms * 1e3 / dec_n:.1f} us "
        f"({gbs:.0f} GB/s); pages {stats}")
    return {"workload": f"decode_b64 on a paged cache of {work.n_pages} 16-row pages",
            "entry": "kvc_append+kvc_attend", "steps": steps, "warmup": warmup,
            "ms_per_step": round(dt * 1e3 / steps, 4), "tokens_per_s": round(tokens / dt, 1),
            "value": round(sbytes / dt / 1e9, 1), "unit": "GB/s",
            "kernel": "k_decode<128,4,paged>", "kernel_achieved": round(gbs, 1),
            "kernel_frac": round(gbs / PEAK_HBM_GBS, 4),
            "avg_launch_us": round(dec_ms * 1e3 / dec_n, 2), "page_stats": stats}

def graph_leg(cache, work, qs, ks, vs, sched, warmup, steps, step_bytes_fn):
    """One-token steps replayed from a captured HIP graph (kvc_static_begin,
    kvc_append_attend per layer, kvc_advance; counts copied into the graph's
    device input before each replay).  Whole-step figures only: kernel
    timing events cannot be recorded inside a replay."""
    dev = cache.buffer.device
    cache.sync_lens()
    g = K.StaticDecodeGraph(cache, fused=True)
    for l in range(work.n_layer):
        g.q[l].copy_(qs[l])
        g.k[l].copy_(ks[l])
        g.v[l].copy_(vs[l])
    n_dev = torch.tensor(np.stack(sched[:warmup + steps]), dtype=torch.int32, device=dev)
    for s in range(warmup):
        g.n_new.copy_(n_dev[s])
        g.replay()
    torch.cuda.synchronize()
    lens = cache.device_lens().cpu().numpy().astype(np.int64)
    sbytes, tokens = 0, 0
    for n in sched[warmup:warmup + steps]:
        sbytes += step_bytes_fn(lens, n)
        tokens += int(n.sum())
        lens = lens + n
    t0 = time.perf_counter()
    for s in range(warmup, warmup + steps):
        g.n_new.copy_(n_dev[s])
        g.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    cache.sync_lens()
    assert cache.lens() == lens.tolist()
    assert cache.static_status() == 0
    del g
    return {"entry": "static step in a HIP graph (kvc_static_begin + kvc_append_attend)",
            "value": round(sbytes / dt / 1e9, 1), "unit": "GB/s",
            "ms_per_step": round(dt * 1e3 / steps, 4),
            "tokens_per_s": round(tokens / dt, 1), "steps": steps, "warmup": warmup}

def cpu_baseline(work, lens_all, seconds):
    """Time the oracle on a bounded sample of the same workload."""
    import oracle
    n_rows = 4
    rows = np.arange(n_rows)
    lens = np.asarray(lens_all)[rows]
    ref = oracle.OracleCache(n_rows, work.n_q_head, [work.n_kv_head[0]], work.head_dim,
                             work.max_len, [0], work.rope_base)
    Cmax = int(lens.max())
    g = np.random.default_rng(wl.seed_of(work.name, "cpu_baseline"))
    hk = work.n_kv_head[0]
    k = g.standard_normal((n_rows, Cmax, hk, work.head_dim))
    v = g.standard_normal((n_rows, Cmax, hk, work.head_dim))
    q = np.zeros((n_rows, Cmax, work.n_q_head, work.head_dim))
    ref.step(lens, [(q, k, v)], compute=False)
    del k, v, q
    done_tokens, done_bytes = 0, 0
    t0 = time.perf_counter()
    step = 0
    while time.perf_counter() - t0 < seconds:
        q1 = g.standard_normal((n_rows, 1, work.n_q_head, work.head_dim))
        k1 = g.standard_normal((n_rows, 1, hk, work.head_dim))
        v1 = g.standard_normal((n_rows, 1, hk, work.head_dim))
        n = np.ones(n_rows, dtype=np.int64)
        if (ref.lens + n > work.max_len).any():
            break
        lens_before = ref.lens.copy()
        ref.step(n, [(q1, k1, v1)])
        done_tokens += n_rows
        done_bytes += decode_kernel_bytes(lens_before, n, work)
        step += 1
    dt = time.perf_counter() - t0
    per_row_layer = dt / max(done_tokens, 1)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {
        "value": 1.0 / (per_row_layer * work.n_layer),
        "unit": "tokens/s",
        "cores": cores,
        "torch_threads": torch.get_num_threads(),
        "kind": "oracle",
        "gbs_equiv": done_bytes / dt / 1e9,
        "sample": (f"oracle (float64, no cache) on {n_rows} rows with the workload's first "
                   f"{n_rows} initial lengths {lens.tolist()}, one layer, {step} decode steps "
                   f"({dt:.1f}s); tokens/s scaled to {work.n_layer} layers"),
    }


def cpu_baseline_long(seconds):
    """Time the oracle on a bounded sample of the long-context decode: one row
    at the prefilled context (32,640 tokens), one global layer and one
    W = 512 sliding layer of the 5:1 stack (B 8, Hq 64 / Hkv 8, D 128),
    alternating one-token steps until about ``seconds`` have passed; the
    per-row step of the 66-layer stack is scaled from the two layer kinds
    (11 global, 55 sliding).  The oracle re-rotates every cached key every
    step, by its definition."""
    import oracle
    work = wl.LONG_5TO1
    hq, D = work.n_q_head, work.head_dim
    L = 510 * 64
    ref = oracle.OracleCache(1, hq, [8, 8], D, work.max_len, [0, 512], work.rope_base)
    g = np.random.default_rng(wl.seed_of(work.name, "cpu_baseline"))
    k = g.standard_normal((1, L, 8, D))
    v = g.standard_normal((1, L, 8, D))
    ref.step(np.array([L]), [(np.zeros((1, L, hq, D)), k, v)] * 2, compute=False)
    del k, v
    n = np.ones(1, dtype=np.int64)
    t_kind = [0.0, 0.0]
    steps = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds and steps < 64:
        for layer in (0, 1):
            q1 = g.standard_normal((1, 1, hq, D))
            k1 = g.standard_normal((1, 1, 8, D))
            v1 = g.standard_normal((1, 1, 8, D))
            t = time.perf_counter()
            ref.layer_step(layer, n, q1, k1, v1)
            t_kind[layer] += time.perf_counter() - t
        ref.advance(n)
        steps += 1
    dt = time.perf_counter() - t0
    glob = sum(1 for w_ in work.window if w_ == 0)
    per_row_step = (glob * t_kind[0] + (work.n_layer - glob) * t_kind[1]) / max(steps, 1)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {
        "value": 1.0 / per_row_step,
        "unit": "tokens/s",
        "cores": cores,
        "torch_threads": torch.get_num_threads(),
        "kind": "oracle",
        "ms_per_layer": {"global": round(t_kind[0] * 1e3 / max(steps, 1), 1),
                         "ring": round(t_kind[1] * 1e3 / max(steps, 1), 1)},
        "sample": (f"oracle (float64, no cache) on one row at {L} tokens, one global and one "
                   f"W=512 sliding layer, {steps} one-token steps ({dt:.1f}s); the per-row "
                   f"step of the {work.n_layer}-layer stack scaled from them "
                   f"({glob} global, {work.n_layer - glob} sliding)"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=56)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--prefill-chunks", type=int, default=510,
                    help="chunks of the prefill leg (0 skips it)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="run only the prefill leg (counter runs) and print its object")
    ap.add_argument("--mixed-steps", type=int, default=8,
                    help="timed steps of the mixed leg (0 skips it)")
    ap.add_argument("--mixed-layers", type=int, default=32,
                    help="layers of the mixed leg")
    ap.add_argument("--long-decode-steps", type=int, default=32,
                    help="timed steps of the long-context decode leg (0 skips it)")
    ap.add_argument("--paged-steps", type=int, default=24,
                    help="timed steps of the paged decode leg (0 skips it)")
    ap.add_argument("--only", choices=("mixed", "long_decode", "paged"),
                    help="run only that leg and print its object")
    ap.add_argument("--two-call", action="store_true",
                    help="headline leg through kvc_append + kvc_attend (two calls per layer) "
                         "instead of kvc_append_attend (the appending decode + merge)")
    ap.add_argument("--no-other-leg", action="store_true",
                    help="skip the second timed leg through the other entry point")
    ap.add_argument("--layers", type=int, default=0,
                    help="fewer layers (counter runs: per-launch work is unchanged)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy, the reference for HBM counters")
    ap.add_argument("--summarize-mfma", metavar="COUNTER_CSV",
                    help="print the MFMA summary of a rocprofv3 --pmc run of --prefill-only "
                         "(same --prefill-chunks) and exit")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print the timed-region summary of a rocprofv3 kernel trace of this "
                         "bench (same --steps / --warmup / --layers) and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic summary of two rocprofv3 --pmc runs of this "
                         "bench (FETCH_SIZE, WRITE_SIZE; same --steps / --warmup / --layers, "
                         "--copy-probe) and exit")
    ap.add_argument("--summarize-legs", metavar="KERNEL_TRACE_CSV",
                    help="print the step summary of a rocprofv3 kernel trace of --only mixed or "
                         "--only long_decode (same --only and step counts) and exit")
    ap.add_argument("--summarize-mixed-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the HBM traffic summary of two rocprofv3 --pmc runs of --only "
                         "mixed --copy-probe (same --mixed-steps / --mixed-layers) and exit")
    args = ap.parse_args()
    if args.summarize_legs:
        n = args.mixed_steps if args.only == "mixed" else args.long_decode_steps
        print(summarize_legs(args.summarize_legs, args.only, n, args.mixed_layers))
        return
    if args.summarize_mixed_counters:
        print(summarize_mixed_counters(*args.summarize_mixed_counters, args.mixed_steps,
                                       args.mixed_layers))
        return
    if args.summarize_mfma:
        print(summarize_mfma(args.summarize_mfma, args.prefill_chunks))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.steps, args.warmup, args.layers,
                              not args.two_call))
        return
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, args.steps, args.warmup, args.layers,
                                 not args.two_call))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this hot path runs on one GPU; multi-GPU runs are not part of it "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_leg(dev, args.prefill_chunks)}), flush=True)
        return
    if args.only == "mixed":
        obj = {"mixed": mixed_leg(dev, args.mixed_steps, 2, args.mixed_layers)}
        if args.copy_probe:
            copy_probe(dev)
        print(json.dumps(obj), flush=True)
        return
    if args.only == "paged":
        print(json.dumps({"paged": paged_leg(dev, args.paged_steps, args.warmup)}), flush=True)
        return
    if args.only == "long_decode":
        print(json.dumps({"long_decode": long_decode_leg(dev, args.long_decode_steps, 4)}),
              flush=True)
        return
    work = workload_for(args.layers)
    legs = 1 if args.no_other_leg else 2
    # lengths clipped for three legs either way, so runs with and without the
    # other legs time the same workload
    lens0, schedule = plan_lens(work, args.steps, args.warmup, 3)
    cfg = K.config_from_workload(work)
    log(f"[bench] buffer {K.kvc_nbytes(cfg, K.KVC_NB_ALLOC) / 2**30:.2f} GiB "
        f"(KV {K.kvc_nbytes(cfg, K.KVC_NB_KV) / 2**30:.2f} GiB)")
    cache = K.Cache(cfg, dev)
    fill_history(cache, work, lens0, dev)

    # decode inputs, resident in HBM
    g = torch.Generator(device=dev)
    g.manual_seed(wl.seed_of(work.name, "decode"))
    B, D = work.batch, work.head_dim
    qs = [torch.randn(B, 1, work.n_q_head, D, generator=g, device=dev).to(work.torch_dtype)
          for _ in range(work.n_layer)]
    ks = [torch.randn(B, 1, work.n_kv_head[0], D, generator=g, device=dev).to(work.torch_dtype)
          for _ in range(work.n_layer)]
    vs = [torch.randn(B, 1, work.n_kv_head[0], D, generator=g, device=dev).to(work.torch_dtype)
          for _ in range(work.n_layer)]
    outs = [torch.empty_like(x) for x in qs]

    def timed_leg(fused, sched):
        """W warmup steps, then K timed steps of the schedule through one entry
        point; whole-step and roofline-kernel figures."""
        def run_step(n):
            if fused:
                for l in range(work.n_layer):
                    cache.append_attend(l, qs[l], ks[l], vs[l], n, out=outs[l])
            else:
                for l in range(work.n_layer):
                    cache.append(l, ks[l], vs[l], n)
                    cache.attend(l, qs[l], outs[l])
            cache.advance()

        # The warmup steps time every kernel kind (the per-kind figures); the
        # timed steps stamp events on the roofline kernel's launches only,
        # since a dispatch that stamps events leaves a longer gap before the
        # next one and would slow the whole step it is part of.
        roof_kind = "fused" if fused else "decode"
        K.kvc_timing_begin(cache.handle, args.warmup * work.n_layer * 4 + 16)
        for n in sched[:args.warmup]:
            run_step(n)
        torch.cuda.synchronize()
        kw = K.kvc_timing_end(cache.handle)
        lens_cur = np.asarray(cache.lens(), dtype=np.int64)
        kbytes, sbytes, tokens = 0, 0, 0
        per_launch = fused_kernel_bytes if fused else decode_kernel_bytes
        for n in sched[args.warmup:]:
            kbytes += per_launch(lens_cur, n, work) * work.n_layer
            sbytes += step_bytes(lens_cur, n, work)
            tokens += int(n.sum())
            lens_cur = lens_cur + n
        K.kvc_timing_begin(cache.handle, args.steps * work.n_layer + 16, kinds=(roof_kind,))
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for n in sched[args.warmup:]:
            run_step(n)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        kt = K.kvc_timing_end(cache.handle)
        assert cache.lens() == lens_cur.tolist()
        dec_ms, dec_n = kt[roof_kind]
        r = {"fused": fused, "dt": dt, "ms_step": dt * 1e3 / args.steps, "tokens": tokens,
             "value": sbytes / dt / 1e9, "kbytes": kbytes, "dec_n": dec_n,
             "dec_us": dec_ms * 1e3 / dec_n if dec_n else None,
             "achieved": kbytes / (dec_ms / 1e3) / 1e9 if dec_ms > 0 else 0.0,
             "kinds": {k: {"ms_total": round(v[0], 3), "launches": v[1],
                           "us_avg": round(v[0] * 1e3 / v[1], 2) if v[1] else None,
                           "from": "warmup steps"}
                       for k, v in kw.items() if v[1]}}
        log(f"[bench] {'kvc_append_attend' if fused else 'kvc_append+kvc_attend'}: "
            f"{args.steps} steps in {dt:.3f}s: {r['ms_step']:.3f} ms/step, "
            f"{tokens / dt:.0f} tok/s, whole-step {r['value']:.0f} GB/s, decode kernel "
            f"{r['achieved']:.0f} GB/s")
        log(f"[bench] kernels: {json.dumps(r['kinds'])}")
        return r

    per_leg = args.steps + args.warmup
    head = timed_leg(not args.two_call, schedule[:per_leg])
    other = None
    if legs == 2:
        o = timed_leg(args.two_call, schedule[per_leg:2 * per_leg])
        other = {"entry": "kvc_append_attend" if o["fused"] else "kvc_append+kvc_attend",
                 "value": round(o["value"], 1), "unit": "GB/s",
                 "ms_per_step": round(o["ms_step"], 4),
                 "tokens_per_s": round(o["tokens"] / o["dt"], 1),
                 "kernel": "k_decode<128,4,fused>" if o["fused"] else "k_decode<128,4>",
                 "kernel_achieved": round(o["achieved"], 1),
                 "kernel_frac": round(o["achieved"] / PEAK_HBM_GBS, 4),
                 "avg_launch_us": round(o["dec_us"], 2) if o["dec_us"] else None,
                 "kernels": o["kinds"]}
    graph = None
    if legs == 2:
        graph = graph_leg(cache, work, qs, ks, vs, schedule[2 * per_leg:], args.warmup, args.steps,
                          lambda lens, n: step_bytes(lens, n, work))
        log(f"[bench] graph replays: {graph['ms_per_step']:.3f} ms/step, "
            f"{graph['tokens_per_s']:.0f} tok/s, whole-step {graph['value']:.0f} GB/s")
    fused = head["fused"]
    dt, ms_step, tokens, value = head["dt"], head["ms_step"], head["tokens"], head["value"]
    achieved, kbytes, dec_n, kinds = head["achieved"], head["kbytes"], head["dec_n"], head["kinds"]

    if args.copy_probe:
        copy_probe(dev)

    cache.close()
    del cache, qs, ks, vs, outs
    torch.cuda.empty_cache()
    prefill = None
    if args.prefill_chunks > 0:
        prefill = prefill_leg(dev, args.prefill_chunks)
        torch.cuda.empty_cache()
    paged = None
    if args.paged_steps > 0:
        paged = paged_leg(dev, args.paged_steps, args.warmup)
        torch.cuda.empty_cache()
    mixed = None
    if args.mixed_steps > 0:
        mixed = mixed_leg(dev, args.mixed_steps, 2, args.mixed_layers)
        torch.cuda.empty_cache()
    long_decode = None
    if args.long_decode_steps > 0:
        long_decode = long_decode_leg(dev, args.long_decode_steps, 4)
        torch.cuda.empty_cache()
        if args.cpu_baseline_seconds > 0:
            log("[bench] timing the CPU oracle on a bounded long-context sample ...")
            long_decode["cpu_baseline"] = cpu_baseline_long(args.cpu_baseline_seconds)
            log(f"[bench] long-context cpu baseline: {long_decode['cpu_baseline']['value']:.4f} "
                f"tok/s ({long_decode['cpu_baseline']['sample']})")

    cpu = None
    if args.cpu_baseline_seconds > 0:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(work, lens0, args.cpu_baseline_seconds)
        log(f"[bench] cpu baseline: {cpu['value']:.3f} tok/s ({cpu['sample']})")

    traffic = counter_traffic(kbytes / max(dec_n, 1), fused)
    line = {
        "metric": "decode cached-attn HBM GB/s (% of peak) + tokens/s, B=64 ctx<=8k bf16",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "tokens_per_s": round(tokens / dt, 1),
        "pct_of_peak_hbm": round(100.0 * value / PEAK_HBM_GBS, 2),
        "config": {"workload": "decode_b64", "n_layer": work.n_layer, "batch": B,
                   "n_q_head": work.n_q_head, "n_kv_head": work.n_kv_head[0], "head_dim": D,
                   "max_len": work.max_len, "lens_init": f"U[1,8128] clipped at {int(lens0.max())}",
                   "idle_rows_per_step": 6,
                   "new_tokens_per_row": 1,
                   "entry": "kvc_append_attend" if fused else "kvc_append+kvc_attend"},
        "roofline": {"bound": "hbm",
                     "kernel": "k_decode<128,4,fused>" if fused else "k_decode<128,4>",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic["bytes"] if traffic else None,
                     "traffic_ratio": traffic["ratio"] if traffic else None,
                     "avg_launch_us": round(head["dec_us"], 2) if head["dec_us"] else None,
                     "bytes_per_launch": int(kbytes / max(dec_n, 1))},
        "kernels": kinds,
        "other_entry_point": other,
        "graph": graph,
        "prefill": prefill,
        "paged": paged,
        "mixed": mixed,
        "long_decode": long_decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
