"""kvc_attend_noalloc: the attention entry point whose split partials live in
the library's fixed per-GPU scratch array instead of the handle's buffer.

It runs the same kernels and the same split plan as kvc_attend, so its
outputs must equal kvc_attend's bit for bit; both are also checked against
the CPU oracle at the bf16 bar.  Each case makes two calls in a row on one
GPU, the second with a smaller input (the array keeps the first call's
contents), and a step whose partials exceed the array is refused with
nothing enqueued.
"""

import numpy as np
import pytest
import torch

import kv_cached_gqa_append_amd as K
import oracle
import workloads as wl
from gpu_harness import check_outputs, f64, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _twins(work):
    cfg = K.config_from_workload(work)
    a = K.Cache(cfg, DEV)
    b = K.Cache(K.config_from_workload(work), DEV)
    ref = oracle.OracleCache(work.batch, work.n_q_head, work.n_kv_head, work.head_dim,
                             work.max_len, work.window, work.rope_base)
    return a, b, ref


def _step(work, a, b, ref, step, n_new, C, noalloc=True):
    layers = [wl.step_qkv(work, l, step, C, "noalloc") for l in range(work.n_layer)]
    outs_a, outs_b = [], []
    for l, (q, k, v) in enumerate(layers):
        q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
        a.append(l, k, v, n_new)
        outs_a.append(a.attend(l, q))
        b.append(l, k, v, n_new)
        if noalloc:
            out = torch.full_like(q, float("nan"))
            outs_b.append(b.attend_noalloc(l, q, out))
        else:
            outs_b.append(b.attend(l, q))
    a.advance()
    b.advance()
    exp = ref.step(np.asarray(n_new), [tuple(f64(t) for t in x) for x in layers])
    torch.cuda.synchronize()
    for l in range(work.n_layer):
        assert torch.equal(outs_a[l], outs_b[l]), f"layer {l} step {step}: outputs differ"
        check_outputs(f64(outs_b[l]), exp[l], n_new, work.dtype, f"noalloc layer {l} step {step}")
    assert a.lens() == b.lens() == [int(x) for x in ref.lens]


def test_noalloc_equals_attend_chunk_then_smaller_steps():
    say("case: kvc_attend_noalloc vs kvc_attend, chunk C=24 then decode then C=8 (global + ring)")
    work = wl.Workload("noalloc_mix", 2, 6, 16, (4, 4), 128, 256, (0, 32), "bf16", 24)
    a, b, ref = _twins(work)
    _step(work, a, b, ref, 0, [24, 17, 0, 5, 24, 1], 24)
    _step(work, a, b, ref, 1, [1, 1, 0, 1, 1, 1], 1)
    _step(work, a, b, ref, 2, [8, 3, 1, 0, 8, 2], 8)


def test_noalloc_equals_attend_decode_b64_shape():
    # the headline decode shape (B 64, Hq 32 / Hkv 8, D 128): its partials
    # take 65 MiB of the 128 MiB array
    say("case: kvc_attend_noalloc vs kvc_attend, B64 Hq32/Hkv8 D128 decode steps")
    work = wl.Workload("noalloc_b64", 1, 64, 32, (8,), 128, 1024, (0,), "bf16", 64)
    a, b, ref = _twins(work)
    g = np.random.default_rng(7)
    # history through kvc_attend (a 64-token chunk step's partials would not fit)
    _step(work, a, b, ref, 0, [int(x) for x in g.integers(1, 65, 64)], 64, noalloc=False)
    n = [1] * 64
    for i in (3, 17, 40):
        n[i] = 0
    _step(work, a, b, ref, 1, n, 1)
    _step(work, a, b, ref, 2, [1] * 32 + [0] * 32, 1)


def test_noalloc_refuses_a_step_past_its_scratch():
    # B 16, Hq 32, D 128, a 64-token chunk: its chunk partials alone take
    # 16*64*32*16*(8 + 512) bytes, more than the array holds
    say("case: kvc_attend_noalloc refuses a step whose partials exceed the scratch")
    work = wl.Workload("noalloc_big", 1, 16, 32, (8,), 128, 256, (0,), "bf16", 64)
    c = K.Cache(K.config_from_workload(work), DEV)
    q, k, v = (t.to(DEV) for t in wl.step_qkv(work, 0, 0, 64, "noalloc"))
    n = [64] * 16
    c.append(0, k, v, n)
    out = torch.zeros_like(q)
    with pytest.raises(K.ScratchTooSmallError):
        c.attend_noalloc(0, q, out)
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0          # nothing was enqueued
    ref_out = c.attend(0, q)                      # the layer is still unattended
    c.advance()
    ref = oracle.OracleCache(work.batch, work.n_q_head, work.n_kv_head, work.head_dim,
                             work.max_len, work.window, work.rope_base)
    exp = ref.step(np.asarray(n), [tuple(f64(t) for t in wl.step_qkv(work, 0, 0, 64, "noalloc"))])
    torch.cuda.synchronize()
    check_outputs(f64(ref_out), exp[0], n, "bf16", "attend after a refused noalloc call")
