"""The device-assembly check of hand-placed tile waits has teeth (CPU only).

Each case is a small hand-written function body in the compiler's output
format: a ring of two tiles loaded from inline assembly, one wait per tile.
"""

from kv_cached_gqa_append_amd import asm_check

GOOD = """\
_Zk:
\t;;#ASMSTART
\tbuffer_load_dwordx4 v[10:13], v1, s[0:3], s4 offen offset:0 ; tile load
\t;;#ASMEND
\t;;#ASMSTART
\tbuffer_load_dwordx4 v[14:17], v1, s[0:3], s5 offen offset:0 ; tile load
\t;;#ASMEND
.LBB0_1:
\t;;#ASMSTART
\tbuffer_load_dwordx4 v[18:21], v1, s[0:3], s6 offen offset:0 ; tile load
\t;;#ASMEND
\t;;#ASMSTART
\ts_waitcnt vmcnt(2) ; tile wait v[10:13]
\t;;#ASMEND
\tv_dot2c_f32_bf16_e32 v30, v10, v11
\t;;#ASMSTART
\tbuffer_load_dwordx4 v[10:13], v1, s[0:3], s7 offen offset:0 ; tile load
\t;;#ASMEND
\t;;#ASMSTART
\ts_waitcnt vmcnt(2) ; tile wait v[14:17]
\t;;#ASMEND
\tv_dot2c_f32_bf16_e32 v30, v14, v15
\t;;#ASMSTART
\tbuffer_load_dwordx4 v[14:17], v1, s[0:3], s7 offen offset:0 ; tile load
\t;;#ASMEND
\t;;#ASMSTART
\ts_waitcnt vmcnt(2) ; tile wait v[18:21]
\t;;#ASMEND
\tv_dot2c_f32_bf16_e32 v30, v18, v19
\ts_cbranch_scc1 .LBB0_1
\t;;#ASMSTART
\ts_waitcnt vmcnt(0) ; tile wait v[10:13]
\t;;#ASMEND
\t;;#ASMSTART
\ts_waitcnt vmcnt(0) ; tile wait v[14:17]
\t;;#ASMEND
\tglobal_store_dword v[2:3], v30, off
\ts_endpgm
.Lfunc_end0:
"""


def _problems(text):
    n, probs = asm_check.check_assembly(text)
    assert n == 1
    return probs


def test_good_ring_passes():
    assert _problems(GOOD) == []


def test_copy_of_pending_register_is_caught():
    bad = GOOD.replace("\tv_dot2c_f32_bf16_e32 v30, v10, v11\n",
                       "\tv_dot2c_f32_bf16_e32 v30, v10, v11\n\tv_mov_b32_e32 v40, v19\n", 1)
    assert any("touches in-flight" in p for p in _problems(bad))


def test_write_into_pending_register_is_caught():
    bad = GOOD.replace("\tv_dot2c_f32_bf16_e32 v30, v14, v15\n",
                       "\tv_dot2c_f32_bf16_e32 v30, v14, v15\n\tv_mov_b32_e32 v12, 0\n", 1)
    assert any("touches in-flight" in p for p in _problems(bad))


def test_weak_wait_is_caught():
    bad = GOOD.replace("s_waitcnt vmcnt(2) ; tile wait v[10:13]",
                       "s_waitcnt vmcnt(3) ; tile wait v[10:13]", 1)
    assert any("does not retire" in p for p in _problems(bad))


def test_interleaved_compiler_load_is_caught():
    bad = GOOD.replace("\tv_dot2c_f32_bf16_e32 v30, v14, v15\n",
                       "\tv_dot2c_f32_bf16_e32 v30, v14, v15\n\tglobal_load_dword v50, v[2:3], off\n", 1)
    assert any("vector memory" in p for p in _problems(bad))


def test_unbalanced_loop_is_caught():
    # one extra load in the body that no wait retires: the loop head is reached
    # with different loads in flight from the entry and from the back edge
    bad = GOOD.replace("\ts_cbranch_scc1 .LBB0_1\n", """\t;;#ASMSTART
\tbuffer_load_dwordx4 v[22:25], v1, s[0:3], s7 offen offset:0 ; tile load
\t;;#ASMEND
\ts_cbranch_scc1 .LBB0_1
""", 1)
    assert any("paths with different loads" in p or "settle" in p for p in _problems(bad))


def test_join_with_different_loads_in_flight_is_caught():
    # a forward branch skips one load: after the join only vmcnt(0) is safe
    bad = GOOD.replace("""\t;;#ASMSTART
\tbuffer_load_dwordx4 v[14:17], v1, s[0:3], s7 offen offset:0 ; tile load
\t;;#ASMEND
""", """\ts_cbranch_scc0 .LBB0_9
\t;;#ASMSTART
\tbuffer_load_dwordx4 v[14:17], v1, s[0:3], s7 offen offset:0 ; tile load
\t;;#ASMEND
.LBB0_9:
""", 1)
    assert any("paths with different loads" in p for p in _problems(bad))


def test_missing_final_wait_is_caught():
    bad = GOOD.replace("\t;;#ASMSTART\n\ts_waitcnt vmcnt(0) ; tile wait v[10:13]\n\t;;#ASMEND\n", "", 1)
    bad = bad.replace("\t;;#ASMSTART\n\ts_waitcnt vmcnt(0) ; tile wait v[14:17]\n\t;;#ASMEND\n", "", 1)
    bad = bad.replace("global_store_dword v[2:3], v30, off", "v_mov_b32_e32 v11, 0", 1)
    assert any("touches in-flight" in p for p in _problems(bad))
