"""Kernel timing by kind: a timed sequence stamps events on the chosen kinds
only (the bench times the roofline kernel alone inside its timed steps)."""

import numpy as np
import pytest

import kv_cached_gqa_append_amd as K
import workloads as wl
from gpu_harness import Pair, say

pytestmark = pytest.mark.gpu


def test_timing_counts_only_the_chosen_kinds():
    say("case: kernel timing restricted to the decode kind, then every kind")
    work = wl.Workload("timing_kinds", 2, 4, 8, (2, 2), 128, 256, (0, 0), "bf16", 32)
    pair = Pair(work, poison=True, tag="tk")
    for n, C in wl.fill_plan([100, 37, 64, 5], 32):
        pair.step(n, C, check=False)
    h = pair.cache.handle
    n = np.array([1, 1, 0, 1])
    K.kvc_timing_begin(h, 64, kinds=("decode",))
    pair.step(n, 1)
    t = K.kvc_timing_end(h)
    assert t["decode"][1] == work.n_layer and t["decode"][0] > 0.0, t
    assert all(v[1] == 0 for k, v in t.items() if k != "decode"), t
    K.kvc_timing_begin(h, 64)
    pair.step(n, 1)
    spans = K.kvc_timing_spans(h, 64)
    t = K.kvc_timing_end(h)
    for kind in ("append", "decode", "combine"):
        assert t[kind][1] == work.n_layer, (kind, t)
    # spans: one per timed launch, in launch order on one stream, so they do
    # not overlap and their union equals the summed kernel time
    assert len(spans) == sum(v[1] for v in t.values())
    assert all(b >= a >= 0.0 for _, a, b in spans)
    assert all(spans[i][1] >= spans[i - 1][2] - 1e-3 for i in range(1, len(spans)))
    tot = sum(v[0] for v in t.values())
    assert abs(K.busy_ms(spans, set(K.KERNEL_KINDS)) - tot) <= 1e-3 * len(spans) + 1e-6 * tot
    with pytest.raises(ValueError):  # a bit past the last kind: KVC_E_ARG
        K._check(K.lib().kvc_timing_begin_kinds(h, 8, 1 << len(K.KERNEL_KINDS)),
                 "kvc_timing_begin_kinds")
    say(f"  worst abs {pair.worst:.2e} rel {pair.worst_rel:.2e}")
