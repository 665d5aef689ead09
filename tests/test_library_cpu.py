"""The C ABI library without a GPU: it loads, exports every declared
function, and its pure host logic (sizes, config validation, status texts)
matches the pages' numbers.  No kernel is launched here."""

import ctypes
import os
import re

import pytest

import kv_cached_gqa_append_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "kvc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(kvc_[a-z_]+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"kvc_create", "kvc_reset", "kvc_append", "kvc_attend", "kvc_nbytes",
            "kvc_advance", "kvc_destroy"} <= set(names)
    lib = ctypes.CDLL(K.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/kvc.h but not exported"


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_nbytes_lab07_answer():
    (_, n_layer, batch, hkv, max_len, hd, nb, want), = _golden("kv_bytes_lab07.txt")
    assert int(nb) == 4
    cfg = K.make_config(int(n_layer), int(batch), int(hkv), int(hd), int(max_len), 1, "f32",
                        int(hkv), 0)
    assert K.kvc_nbytes(cfg, K.KVC_NB_KV) == int(want) == 98304
    assert K.kvc_nbytes(cfg, K.KVC_NB_ALLOC) > int(want)


def _as_printed(x, printed):
    digits = len(printed.split(".")[1]) if "." in printed else 0
    return abs(x - float(printed)) <= 0.5 * 10.0 ** (-digits) + 1e-9


def test_nbytes_inkling_table():
    hkv = [16 if (l + 1) % 6 else 8 for l in range(66)]
    win = [512 if (l + 1) % 6 else 0 for l in range(66)]
    for ln in _golden("inkling_memory_table.txt"):
        if ln[0] != "table":
            continue
        ctx = int(ln[1])
        full = K.kvc_nbytes(K.make_config(66, 1, 16, 128, ctx, 1, "f32", hkv, win, use_ring=False))
        ring = K.kvc_nbytes(K.make_config(66, 1, 16, 128, ctx, 1, "f32", hkv, win, use_ring=True))
        assert _as_printed(full / 2 ** 30, ln[2])
        assert _as_printed(ring / 2 ** 30, ln[3])
        assert _as_printed(full / ring, ln[4])


def test_nbytes_matches_workload_formula():
    import workloads as wl
    import oracle
    for w in wl.ALL.values():
        got = K.kvc_nbytes(K.config_from_workload(w), K.KVC_NB_KV)
        want = oracle.kv_nbytes(w.batch, w.n_kv_head, w.head_dim, w.max_len, w.window,
                                w.dtype_bytes, w.use_ring)
        assert got == want
    # the headline decode workload: 64 GiB of KV
    assert K.kvc_nbytes(K.config_from_workload(wl.DECODE_B64)) == 64 * 2 ** 30


@pytest.mark.parametrize("bad", [
    dict(n_layer=0), dict(batch=0), dict(head_dim=12), dict(head_dim=512), dict(max_len=0),
    dict(max_chunk=0), dict(max_chunk=2048), dict(n_kv_head=3), dict(window=-1),
    dict(rope_base=-1.0), dict(dtype=7), dict(n_q_head=6, n_kv_head=4),
])
def test_invalid_configs_are_rejected(bad):
    args = dict(n_layer=2, batch=2, n_q_head=8, head_dim=64, max_len=64, max_chunk=8,
                dtype="bf16", n_kv_head=2, window=0)
    args.update(bad)
    dtype = args.pop("dtype")
    if isinstance(dtype, int):
        cfg = K.make_config(dtype=0, **args)
        cfg.dtype = dtype
    else:
        cfg = K.make_config(dtype=dtype, **args)
    assert K.kvc_nbytes(cfg, K.KVC_NB_KV) == 0
    assert K.kvc_nbytes(cfg, K.KVC_NB_ALLOC) == 0
    h = ctypes.c_void_p()
    rc = K.lib().kvc_create(ctypes.byref(cfg), ctypes.c_void_p(256), ctypes.c_size_t(1 << 40),
                            None, ctypes.byref(h))
    assert rc in (K.KVC_E_ARG, K.KVC_E_DTYPE) and not h.value


def test_create_rejects_small_or_missing_buffer_before_any_device_call():
    cfg = K.make_config(1, 1, 8, 64, 64, 8, "f32", 2, 0)
    need = K.kvc_nbytes(cfg, K.KVC_NB_ALLOC)
    h = ctypes.c_void_p()
    assert K.lib().kvc_create(ctypes.byref(cfg), None, need, None, ctypes.byref(h)) == K.KVC_E_ARG
    assert K.lib().kvc_create(ctypes.byref(cfg), ctypes.c_void_p(256), need - 1, None,
                              ctypes.byref(h)) == K.KVC_E_ARG
    assert K.lib().kvc_create(ctypes.byref(cfg), ctypes.c_void_p(100), need, None,
                              ctypes.byref(h)) == K.KVC_E_ARG


def test_status_texts():
    assert K.kvc_strerror(K.KVC_E_FULL) == "KV cache full"
    assert K.kvc_strerror(K.KVC_OK) == "ok"
    for c in (K.KVC_E_ARG, K.KVC_E_DTYPE, K.KVC_E_STATE, K.KVC_E_HIP, 99):
        assert K.kvc_strerror(c)


def test_null_handle_calls_fail_cleanly():
    L = K.lib()
    assert L.kvc_advance(None, None) == K.KVC_E_ARG
    assert L.kvc_attend(None, 0, None, None, None) == K.KVC_E_ARG
    assert L.kvc_lens(None, None) == K.KVC_E_ARG
    L.kvc_destroy(None)


def test_paged_sizes_and_validation():
    # Lab 07 Stretch (16-token blocks): a paged full layer's K and V are the
    # pool, 2 * Hkv * n_pages * 16 * D * bytes; ring layers keep W rows per
    # row; a negative pool is rejected.
    full = K.make_config(2, 4, 8, 64, 256, 16, "bf16", [2, 2], [0, 32])
    paged = K.make_config(2, 4, 8, 64, 256, 16, "bf16", [2, 2], [0, 32], n_pages=40)
    ring_bytes = 2 * 4 * 2 * 32 * 64 * 2
    assert K.kvc_nbytes(full, K.KVC_NB_KV) == 2 * 4 * 2 * 256 * 64 * 2 + ring_bytes
    assert K.kvc_nbytes(paged, K.KVC_NB_KV) == 2 * 2 * 40 * 16 * 64 * 2 + ring_bytes
    assert K.kvc_nbytes(paged, K.KVC_NB_ALLOC) > K.kvc_nbytes(paged, K.KVC_NB_KV)
    bad = K.make_config(2, 4, 8, 64, 256, 16, "bf16", [2, 2], [0, 32], n_pages=-1)
    assert K.kvc_nbytes(bad, K.KVC_NB_KV) == 0


def test_joint_partner_validation():
    # tiny_agent hybrid groups: a layer's joint partner is an earlier
    # full-layout layer with the same KV heads and no partner of its own
    def nb(joint, hkv=(2, 2, 2, 2)):
        cfg = K.make_config(4, 2, 8, 64, 128, 16, "bf16", list(hkv), [0, 16, 8, 0], joint=joint)
        return K.kvc_nbytes(cfg, K.KVC_NB_ALLOC)
    assert nb([-1, 0, 0, -1]) > 0 and nb([-1, 0, 0, 0]) > 0
    assert nb([-1, 1, 0, -1]) == 0           # itself
    assert nb([-1, 2, 0, -1]) == 0           # a later layer
    assert nb([-1, 0, 1, -1]) == 0           # a ring
    assert nb([-1, 0, 0, -1], hkv=(2, 1, 2, 2)) == 0   # other KV heads


def test_region_of_two_gib_is_rejected():
    # colibri PR "Tests done": cache offsets must not overflow.  The kernels
    # address one (row, KV head) region of K or V with 32-bit offsets, so a
    # config whose region reaches 2^31 bytes is refused, not wrapped.
    def nb(max_len, dtype="bf16", head_dim=128, window=0, n_pages=0):
        cfg = K.make_config(1, 2, 8, head_dim, max_len, 1, dtype, 2, window, n_pages=n_pages)
        return K.kvc_nbytes(cfg, K.KVC_NB_ALLOC)
    # bf16 D 128: rows_alloc = round_up(max_len + 1, 32) + 16 rows of 256 B
    assert nb(8_388_575) > 0
    assert nb(8_388_576) == 0
    assert nb(9_000_000) == 0
    # D 64 bf16 holds twice the rows; fp32 half as many
    assert nb(16_777_000, head_dim=64) > 0 and nb(16_777_200, head_dim=64) == 0
    assert nb(4_194_000, dtype="f32") > 0 and nb(4_194_400, dtype="f32") == 0
    # a ring layer's region is its window's: a long max_len is fine there
    assert nb(9_000_000, window=4096) > 0
    # paged layers address the same logical rows
    assert nb(9_000_000, n_pages=64) == 0
