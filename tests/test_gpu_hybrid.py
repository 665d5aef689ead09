"""Hybrid layer groups on the GPU against the oracle (tiny_agent
"generate.py": a group-global K/V written by the group's full layer, a ring
per layer, one softmax over both).

Layers 0 and 3 are the groups' global stores; layers 1, 2 (group 0) and 4
(group 1) are per-layer rings whose attention also covers their group's
global keys.  Every step of every layer is compared with the oracle.
"""

import numpy as np
import pytest
import torch

import kv_cached_gqa_append_amd as K
import workloads as wl
from gpu_harness import Pair, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _group_work(name, dtype="bf16", D=128, hq=32, hkv=8, use_ring=True, n_pages=0):
    return wl.Workload(name, 5, 4, hq, (hkv,) * 5, D, 300, (0, 16, 8, 0, 16), dtype, 64,
                       use_ring=use_ring, n_pages=n_pages, joint=(-1, 0, 0, -1, 3))


@pytest.mark.parametrize("use_ring,n_pages,fused", [(True, 0, False), (True, 0, True),
                                                     (False, 0, False), (True, 80, True)])
def test_hybrid_groups_match_oracle(use_ring, n_pages, fused):
    say(f"case: hybrid groups, D128 rep4, rings={use_ring}, pages={n_pages}, fused={fused}")
    work = _group_work("hybrid", use_ring=use_ring, n_pages=n_pages)
    pair = Pair(work, poison=True, tag=f"hy{int(use_ring)}{n_pages}{int(fused)}")
    for n in ([40, 0, 64, 7], [64, 30, 1, 64], [1, 64, 0, 9]):
        pair.step(n, 64)
    for s in range(8):
        pair.step(wl.n_new_decode_b64(s, batch=4, idle=1), 1, fused=fused)
    pair.step([2, 1, 33, 0], 33)
    say(f"  worst abs {pair.worst:.2e} rel {pair.worst_rel:.2e}")


def test_hybrid_groups_float32_generic_path():
    say("case: hybrid groups, fp32 (generic attention)")
    work = _group_work("hybrid32", dtype="f32", D=64, hq=8, hkv=2)
    pair = Pair(work, poison=True, tag="hy32")
    for n, C in wl.fill_plan([21, 40, 9, 33], 16):
        pair.step(n, C)
    for s in range(5):
        pair.step(wl.n_new_decode_b64(s, batch=4, idle=1), 1)


def test_hybrid_protocol_and_config_checks():
    say("case: hybrid groups keep the step protocol; invalid partners rejected")
    work = _group_work("hybrid_guard", D=64, hq=8, hkv=2)
    pair = Pair(work)
    c = pair.cache
    q, k, v = (t.to(DEV) for t in wl.step_qkv(work, 0, 0, 4))
    n = [4, 4, 0, 1]
    c.append(1, k, v, n)
    with pytest.raises(K.StepOrderError):
        c.attend(1, q)                                  # the group store not appended yet
    c.append(0, k, v, n)
    c.attend(1, q)
    for l in (2, 3, 4):
        c.append(l, k, v, n)
    c.attend(2, q)
    with pytest.raises(K.StepOrderError):
        c.advance()                                     # layer 4 not attended
    c.attend(4, q)
    c.advance()                                         # the group stores need no attend
    assert c.lens() == [4, 4, 0, 1]
    with pytest.raises(ValueError):
        c.static_begin(torch.zeros(4, dtype=torch.int32, device=DEV))
    for joint in ((-1, 2, 0, -1, 3), (-1, 1, 0, -1, 3), (-1, 0, 1, -1, 3), (-1, 0, 0, -1, 3)):
        bad = work.replace(joint=joint, n_kv_head=(2, 2, 2, 1, 2) if joint == (-1, 0, 0, -1, 3)
                           else work.n_kv_head, n_q_head=8)
        with pytest.raises(ValueError):
            K.Cache(K.config_from_workload(bad), DEV)  # later / ring / chained / other heads
    torch.cuda.synchronize()
