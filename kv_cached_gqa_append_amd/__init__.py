"""Python binding of ``libkvc.so``: cached GQA attention with append on MI355X.

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch provides device memory (the cache buffer, q/k/v/out tensors) and the
HIP stream (``torch.cuda.current_stream()``).  The C functions keep their
names (``kvc_nbytes``, ``kvc_create``, ``kvc_reset``, ``kvc_append``,
``kvc_attend``, ``kvc_advance``, ``kvc_lens``, ...); ``Cache`` bundles them
with a torch-allocated buffer.

Errors: status codes become exceptions, following pycraft-1
``KVCache.update``: a full cache raises ``CacheFullError`` (a ValueError),
a dtype mismatch ``TypeError``, a batch/shape mismatch ``ValueError``; a
call out of step order raises ``StepOrderError``.

The library must be built first (``__graft_entry__.build()`` or
``python -m kv_cached_gqa_append_amd.build``); there is no fallback.
"""

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvc.so")

KVC_OK, KVC_E_ARG, KVC_E_FULL, KVC_E_DTYPE, KVC_E_STATE, KVC_E_HIP = 0, -1, -2, -3, -4, -5
KVC_E_SCRATCH = -6
KVC_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024
KVC_F32, KVC_BF16 = 0, 1
KVC_NB_KV, KVC_NB_ALLOC = 0, 1
KVC_STATIC_BAD_COUNT, KVC_STATIC_FULL = 1, 2
KERNEL_KINDS = ("append", "decode", "chunk", "combine", "commit", "generic", "fused")

_DTYPES = {torch.float32: KVC_F32, torch.bfloat16: KVC_BF16}
_TORCH_OF = {KVC_F32: torch.float32, KVC_BF16: torch.bfloat16}


class KvcError(RuntimeError):
    pass


class CacheFullError(ValueError):
    """Some row would pass max_len; nothing was written."""


class StepOrderError(KvcError):
    """A call broke the append -> attend -> advance protocol."""


class ScratchTooSmallError(KvcError):
    """kvc_attend_noalloc: the step's partials exceed the fixed scratch."""


class KvcConfig(ctypes.Structure):
    _fields_ = [
        ("n_layer", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("n_q_head", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
        ("max_chunk", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("n_kv_head", ctypes.POINTER(ctypes.c_int32)),
        ("window", ctypes.POINTER(ctypes.c_int32)),
        ("use_ring", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("n_pages", ctypes.c_int32),
        ("joint", ctypes.POINTER(ctypes.c_int32)),
    ]


class KvcBufferInfo(ctypes.Structure):
    _fields_ = [
        ("total_bytes", ctypes.c_int64),
        ("kv_bytes", ctypes.c_int64),
        ("lens_offset", ctypes.c_int64),
        ("n_new_offset", ctypes.c_int64),
        ("rope_offset", ctypes.c_int64),
    ]


class KvcLayerInfo(ctypes.Structure):
    _fields_ = [
        ("k_offset", ctypes.c_int64),
        ("v_offset", ctypes.c_int64),
        ("stage_k_offset", ctypes.c_int64),
        ("stage_v_offset", ctypes.c_int64),
        ("n_kv_head", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("is_ring", ctypes.c_int32),
        ("rows", ctypes.c_int32),
        ("rows_alloc", ctypes.c_int32),
        ("stage_rows_alloc", ctypes.c_int32),
    ]


_lib = None


def lib():
    """The loaded ``libkvc.so`` (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_void_p
        L.kvc_nbytes.argtypes = [P(KvcConfig), ctypes.c_int]
        L.kvc_nbytes.restype = ctypes.c_size_t
        L.kvc_create.argtypes = [P(KvcConfig), VP, ctypes.c_size_t, VP, P(VP)]
        L.kvc_create.restype = ctypes.c_int
        L.kvc_destroy.argtypes = [VP]
        L.kvc_destroy.restype = None
        L.kvc_reset.argtypes = [VP, VP, I32, VP]
        L.kvc_reset.restype = ctypes.c_int
        L.kvc_append.argtypes = [VP, I32, VP, VP, VP, I32, VP, VP]
        L.kvc_append.restype = ctypes.c_int
        L.kvc_attend.argtypes = [VP, I32, VP, VP, VP]
        L.kvc_attend.restype = ctypes.c_int
        L.kvc_attend_noalloc.argtypes = [VP, I32, VP, VP, VP]
        L.kvc_attend_noalloc.restype = ctypes.c_int
        L.kvc_append_attend.argtypes = [VP, I32, VP, VP, VP, VP, I32, VP, VP, VP]
        L.kvc_append_attend.restype = ctypes.c_int
        L.kvc_advance.argtypes = [VP, VP]
        L.kvc_advance.restype = ctypes.c_int
        L.kvc_lens.argtypes = [VP, P(I32)]
        L.kvc_lens.restype = ctypes.c_int
        L.kvc_set_first.argtypes = [VP, VP, VP, I32, VP]
        L.kvc_set_first.restype = ctypes.c_int
        L.kvc_admit.argtypes = [VP, VP, VP, VP, I32, VP]
        L.kvc_admit.restype = ctypes.c_int
        L.kvc_page_stats.argtypes = [VP, P(ctypes.c_int64), P(ctypes.c_int64), P(ctypes.c_int64)]
        L.kvc_page_stats.restype = ctypes.c_int
        L.kvc_reserve.argtypes = [VP, VP, VP, I32, VP]
        L.kvc_reserve.restype = ctypes.c_int
        L.kvc_static_begin.argtypes = [VP, VP, VP]
        L.kvc_static_begin.restype = ctypes.c_int
        L.kvc_static_status.argtypes = [VP, P(I32), VP]
        L.kvc_static_status.restype = ctypes.c_int
        L.kvc_sync_lens.argtypes = [VP, VP]
        L.kvc_sync_lens.restype = ctypes.c_int
        L.kvc_layer_layout.argtypes = [VP, I32, P(KvcLayerInfo)]
        L.kvc_layer_layout.restype = ctypes.c_int
        L.kvc_buffer_info.argtypes = [VP, P(KvcBufferInfo)]
        L.kvc_buffer_info.restype = ctypes.c_int
        L.kvc_timing_begin.argtypes = [VP, I32]
        L.kvc_timing_begin.restype = ctypes.c_int
        L.kvc_timing_begin_kinds.argtypes = [VP, I32, I32]
        L.kvc_timing_begin_kinds.restype = ctypes.c_int
        L.kvc_timing_end.argtypes = [VP, P(ctypes.c_double), P(I32)]
        L.kvc_timing_end.restype = ctypes.c_int
        L.kvc_timing_spans.argtypes = [VP, I32, P(I32), P(ctypes.c_double), P(ctypes.c_double)]
        L.kvc_timing_spans.restype = ctypes.c_int
        L.kvc_strerror.argtypes = [ctypes.c_int]
        L.kvc_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def kvc_strerror(code: int) -> str:
    return lib().kvc_strerror(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code == KVC_OK:
        return
    msg = f"{what}: {kvc_strerror(code)}"
    if code == KVC_E_FULL:
        raise CacheFullError(msg)
    if code == KVC_E_DTYPE:
        raise TypeError(msg)
    if code == KVC_E_ARG:
        raise ValueError(msg)
    if code == KVC_E_STATE:
        raise StepOrderError(msg)
    if code == KVC_E_SCRATCH:
        raise ScratchTooSmallError(msg)
    raise KvcError(msg)


def make_config(n_layer, batch, n_q_head, head_dim, max_len, max_chunk, dtype,
                n_kv_head, window, use_ring=True, rope_base=10000.0, n_pages=0,
                joint=None) -> KvcConfig:
    """A ``KvcConfig`` that keeps its per-layer arrays alive."""
    if isinstance(dtype, torch.dtype):
        dtype = _DTYPES[dtype]
    elif isinstance(dtype, str):
        dtype = {"f32": KVC_F32, "bf16": KVC_BF16}[dtype]
    if isinstance(n_kv_head, int):
        n_kv_head = [n_kv_head] * n_layer
    if isinstance(window, int):
        window = [window] * n_layer
    hk = (ctypes.c_int32 * len(n_kv_head))(*[int(x) for x in n_kv_head])
    wn = (ctypes.c_int32 * len(window))(*[int(x) for x in window])
    jt = None
    if joint is not None and len(joint) and any(int(j) >= 0 for j in joint):
        jt = (ctypes.c_int32 * len(joint))(*[int(j) for j in joint])
    cfg = KvcConfig(int(n_layer), int(batch), int(n_q_head), int(head_dim), int(max_len),
                    int(max_chunk), int(dtype), hk, wn, int(bool(use_ring)), float(rope_base),
                    int(n_pages), jt)
    cfg._keep = (hk, wn, jt)
    return cfg


def config_from_workload(w) -> KvcConfig:
    """Config for a ``workloads.Workload``."""
    return make_config(w.n_layer, w.batch, w.n_q_head, w.head_dim, w.max_len, w.max_chunk,
                       w.dtype, list(w.n_kv_head), list(w.window), w.use_ring, w.rope_base,
                       getattr(w, "n_pages", 0), getattr(w, "joint", None) or None)


def kvc_nbytes(cfg: KvcConfig, what: int = KVC_NB_KV) -> int:
    return int(lib().kvc_nbytes(ctypes.byref(cfg), int(what)))


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def kvc_create(cfg: KvcConfig, buf: torch.Tensor, stream=None):
    if not (buf.is_cuda and buf.dtype == torch.uint8 and buf.is_contiguous()):
        raise ValueError("buffer must be a contiguous uint8 tensor on the GPU")
    h = ctypes.c_void_p()
    _check(lib().kvc_create(ctypes.byref(cfg), ctypes.c_void_p(buf.data_ptr()),
                            ctypes.c_size_t(buf.numel()), _stream_handle(stream),
                            ctypes.byref(h)), "kvc_create")
    return h


def kvc_destroy(h) -> None:
    lib().kvc_destroy(h)


class _Rows:
    """Host int32 array for the C ABI; ``ptr`` is valid while this lives."""

    __slots__ = ("arr", "ptr", "n")

    def __init__(self, values):
        arr = np.ascontiguousarray(values, dtype=np.int32)
        if arr.ndim != 1:
            raise ValueError("row values must be one-dimensional")
        self.n = int(arr.size)
        # (an empty list still passes a valid pointer, with count 0)
        self.arr = arr if arr.size else np.zeros(1, dtype=np.int32)
        self.ptr = ctypes.c_void_p(self.arr.ctypes.data)


def _rows_array(values):
    """(pointer, count) of int32 row values (None: a static step's counts
    are on the device, passed as NULL).  The pointer's owner rides along as
    a third element so that it outlives the call."""
    if values is None:
        return None, 0, None
    r = _Rows(values)
    return r.ptr, r.n, r


def kvc_reset(h, rows, stream=None) -> None:
    arr, n, _keep = _rows_array(rows)
    _check(lib().kvc_reset(h, arr, n, _stream_handle(stream)), "kvc_reset")


def kvc_append(h, layer: int, k: torch.Tensor, v: torch.Tensor, n_new, C: int,
               slot_out=None, stream=None) -> None:
    arr, _, _keep = _rows_array(n_new)
    so = ctypes.c_void_p(slot_out.data_ptr()) if slot_out is not None else ctypes.c_void_p()
    _check(lib().kvc_append(h, int(layer), ctypes.c_void_p(k.data_ptr()),
                            ctypes.c_void_p(v.data_ptr()), arr, int(C), so,
                            _stream_handle(stream)), "kvc_append")


def kvc_attend(h, layer: int, q: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    _check(lib().kvc_attend(h, int(layer), ctypes.c_void_p(q.data_ptr()),
                            ctypes.c_void_p(out.data_ptr()), _stream_handle(stream)),
           "kvc_attend")


def kvc_attend_noalloc(h, layer: int, q: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    _check(lib().kvc_attend_noalloc(h, int(layer), ctypes.c_void_p(q.data_ptr()),
                                    ctypes.c_void_p(out.data_ptr()), _stream_handle(stream)),
           "kvc_attend_noalloc")


def kvc_append_attend(h, layer: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_new,
                      C: int, out: torch.Tensor, slot_out=None, stream=None) -> None:
    arr, _, _keep = _rows_array(n_new)
    so = ctypes.c_void_p(slot_out.data_ptr()) if slot_out is not None else ctypes.c_void_p()
    _check(lib().kvc_append_attend(h, int(layer), ctypes.c_void_p(q.data_ptr()),
                                   ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                                   arr, int(C), so, ctypes.c_void_p(out.data_ptr()),
                                   _stream_handle(stream)), "kvc_append_attend")


def kvc_advance(h, stream=None) -> None:
    _check(lib().kvc_advance(h, _stream_handle(stream)), "kvc_advance")


def kvc_set_first(h, rows, first, stream=None) -> None:
    r, n, _kr = _rows_array(rows)
    f, m, _kf = _rows_array(first)
    if n != m:
        raise ValueError("one first per row")
    _check(lib().kvc_set_first(h, r, f, n, _stream_handle(stream)), "kvc_set_first")


def kvc_admit(dst, dst_rows, src, src_rows, stream=None) -> None:
    d, n, _kd = _rows_array(dst_rows)
    r, m, _kr = _rows_array(src_rows)
    if n != m:
        raise ValueError("one source row per row")
    _check(lib().kvc_admit(dst, d, src, r, n, _stream_handle(stream)), "kvc_admit")


def kvc_page_stats(h):
    u, a, r = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().kvc_page_stats(h, ctypes.byref(u), ctypes.byref(a), ctypes.byref(r)),
           "kvc_page_stats")
    return {"used": int(u.value), "allocated": int(a.value), "reserved": int(r.value)}


def kvc_reserve(h, rows, tokens, stream=None) -> None:
    r, n, _kr = _rows_array(rows)
    t, m, _kt = _rows_array(tokens)
    if n != m:
        raise ValueError("one token count per row")
    _check(lib().kvc_reserve(h, r, t, n, _stream_handle(stream)), "kvc_reserve")


def kvc_static_begin(h, n_new_dev: torch.Tensor, stream=None) -> None:
    _check(lib().kvc_static_begin(h, ctypes.c_void_p(n_new_dev.data_ptr()),
                                  _stream_handle(stream)), "kvc_static_begin")


def kvc_static_status(h, stream=None) -> int:
    v = ctypes.c_int32(0)
    _check(lib().kvc_static_status(h, ctypes.byref(v), _stream_handle(stream)),
           "kvc_static_status")
    return int(v.value)


def kvc_sync_lens(h, stream=None) -> None:
    _check(lib().kvc_sync_lens(h, _stream_handle(stream)), "kvc_sync_lens")


def kvc_lens(h, batch: int):
    arr = (ctypes.c_int32 * batch)()
    _check(lib().kvc_lens(h, arr), "kvc_lens")
    return [int(x) for x in arr]


def kvc_layer_layout(h, layer: int) -> KvcLayerInfo:
    info = KvcLayerInfo()
    _check(lib().kvc_layer_layout(h, int(layer), ctypes.byref(info)), "kvc_layer_layout")
    return info


def kvc_buffer_info(h) -> KvcBufferInfo:
    info = KvcBufferInfo()
    _check(lib().kvc_buffer_info(h, ctypes.byref(info)), "kvc_buffer_info")
    return info


def kvc_timing_begin(h, max_launches: int, kinds=None) -> None:
    """Time every kernel kind, or only ``kinds`` (names from KERNEL_KINDS)."""
    if kinds is None:
        _check(lib().kvc_timing_begin(h, int(max_launches)), "kvc_timing_begin")
        return
    mask = 0
    for k in kinds:
        mask |= 1 << KERNEL_KINDS.index(k)
    _check(lib().kvc_timing_begin_kinds(h, int(max_launches), mask), "kvc_timing_begin_kinds")


def kvc_timing_spans(h, cap: int):
    """[(kind, start_ms, end_ms)] of the timed launches so far (timing on)."""
    kinds = (ctypes.c_int32 * cap)()
    t0 = (ctypes.c_double * cap)()
    t1 = (ctypes.c_double * cap)()
    n = lib().kvc_timing_spans(h, int(cap), kinds, t0, t1)
    if n < 0:
        _check(n, "kvc_timing_spans")
    return [(KERNEL_KINDS[kinds[i]], float(t0[i]), float(t1[i])) for i in range(n)]


def busy_ms(spans, kinds):
    """Length of the union of the spans of these kinds (overlaps once)."""
    iv = sorted((a, b) for k, a, b in spans if k in kinds)
    total, cur_a, cur_b = 0.0, None, None
    for a, b in iv:
        if cur_b is None or a > cur_b:
            if cur_b is not None:
                total += cur_b - cur_a
            cur_a, cur_b = a, b
        else:
            cur_b = max(cur_b, b)
    if cur_b is not None:
        total += cur_b - cur_a
    return total


def kvc_timing_end(h):
    """{kind: (total_ms, launches)} for every kernel kind."""
    ms = (ctypes.c_double * len(KERNEL_KINDS))()
    cnt = (ctypes.c_int32 * len(KERNEL_KINDS))()
    _check(lib().kvc_timing_end(h, ms, cnt), "kvc_timing_end")
    return {k: (float(ms[i]), int(cnt[i])) for i, k in enumerate(KERNEL_KINDS)}


class Cache:
    """A handle plus its torch-allocated device buffer.

    Shapes: k, v (B, C, Hkv_l, D); q, out (B, C, Hq, D); contiguous, on the
    buffer's device, in the config dtype.
    """

    def __init__(self, cfg: KvcConfig, device="cuda", stream=None, buffer=None):
        self.cfg = cfg
        self.batch = cfg.batch
        self.n_layer = cfg.n_layer
        self.n_q_head = cfg.n_q_head
        self.head_dim = cfg.head_dim
        self.max_len = cfg.max_len
        self.max_chunk = cfg.max_chunk
        self.dtype = _TORCH_OF[cfg.dtype]
        self.n_kv_head = [cfg.n_kv_head[i] for i in range(cfg.n_layer)]
        nbytes = kvc_nbytes(cfg, KVC_NB_ALLOC)
        if nbytes == 0:
            raise ValueError("invalid kvc config")
        if buffer is None:
            buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        elif buffer.numel() < nbytes:
            raise ValueError(f"buffer holds {buffer.numel()} bytes, {nbytes} needed")
        self.buffer = buffer
        self.handle = kvc_create(cfg, self.buffer, stream)

    def close(self):
        if getattr(self, "handle", None):
            kvc_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- checks that mirror pycraft-1's guards ------------------------------------
    def _check_tensor(self, t: torch.Tensor, heads: int, C: int, name: str):
        if t.dtype != self.dtype:
            raise TypeError(f"{name}: cache dtype {self.dtype} != {t.dtype}")
        if t.device != self.buffer.device:
            raise ValueError(f"{name} must be on {self.buffer.device}")
        if t.dim() != 4 or t.shape[0] != self.batch:
            raise ValueError(f"{name}: batch {t.shape[0] if t.dim() else '?'} does not match "
                             f"cache batch {self.batch}")
        if tuple(t.shape[1:]) != (C, heads, self.head_dim):
            raise ValueError(f"{name}: shape {tuple(t.shape)} != {(self.batch, C, heads, self.head_dim)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")

    def append(self, layer, k, v, n_new, slot_out=None, stream=None):
        """n_new: host counts [B], or None inside a static step."""
        if n_new is not None and len(n_new) != self.batch:
            raise ValueError(f"n_new has {len(n_new)} entries, cache batch is {self.batch}")
        C = int(k.shape[1])
        hk = self.n_kv_head[layer]
        self._check_tensor(k, hk, C, "k")
        self._check_tensor(v, hk, C, "v")
        if slot_out is not None and (slot_out.dtype != torch.int32 or slot_out.numel() != self.batch * C):
            raise ValueError("slot_out must be int32 (B, C)")
        kvc_append(self.handle, layer, k, v, n_new, C, slot_out, stream)
        self._step_C = C

    def attend(self, layer, q, out=None, stream=None):
        # The library strides q and out by the chunk width its step latched
        # at the first append; a narrower tensor would be read past its end.
        # (Outside a step the library refuses the call: StepOrderError.)
        C = getattr(self, "_step_C", None)
        if C is not None and int(q.shape[1]) != C:
            raise ValueError(f"q: {int(q.shape[1])} tokens per row, the step's appends "
                             f"latched C = {C}")
        C = int(q.shape[1])
        self._check_tensor(q, self.n_q_head, C, "q")
        if out is None:
            out = torch.empty_like(q)
        else:
            self._check_tensor(out, self.n_q_head, C, "out")
        kvc_attend(self.handle, layer, q, out, stream)
        return out

    def attend_noalloc(self, layer, q, out, stream=None):
        """attend() with the split partials in the library's fixed per-GPU
        scratch: the caller passes ``out``; nothing is allocated."""
        C = getattr(self, "_step_C", None)
        if C is not None and int(q.shape[1]) != C:
            raise ValueError(f"q: {int(q.shape[1])} tokens per row, the step's appends "
                             f"latched C = {C}")
        C = int(q.shape[1])
        self._check_tensor(q, self.n_q_head, C, "q")
        self._check_tensor(out, self.n_q_head, C, "out")
        kvc_attend_noalloc(self.handle, layer, q, out, stream)
        return out

    def append_attend(self, layer, q, k, v, n_new, out=None, slot_out=None, stream=None):
        """append() then attend() of one layer in one call (an appending
        decode kernel and the merge for a one-token bf16 step; the chunk
        kernel alone, appending after scoring, for a ring layer's chunk step
        of 2 .. 64 tokens per row).  n_new: host counts [B], or None inside a
        static step."""
        if n_new is not None and len(n_new) != self.batch:
            raise ValueError(f"n_new has {len(n_new)} entries, cache batch is {self.batch}")
        C = int(k.shape[1])
        hk = self.n_kv_head[layer]
        self._check_tensor(k, hk, C, "k")
        self._check_tensor(v, hk, C, "v")
        self._check_tensor(q, self.n_q_head, C, "q")
        if out is None:
            out = torch.empty_like(q)
        else:
            self._check_tensor(out, self.n_q_head, C, "out")
        if slot_out is not None and (slot_out.dtype != torch.int32 or slot_out.numel() != self.batch * C):
            raise ValueError("slot_out must be int32 (B, C)")
        kvc_append_attend(self.handle, layer, q, k, v, n_new, C, out, slot_out, stream)
        self._step_C = C
        return out

    def advance(self, stream=None):
        kvc_advance(self.handle, stream)
        self._step_C = None

    def static_begin(self, n_new_dev: torch.Tensor, stream=None):
        """Begin a static one-token step whose counts (int32 [B], 0 or 1) are
        read from ``n_new_dev`` when the step runs."""
        if (n_new_dev.dtype != torch.int32 or n_new_dev.numel() != self.batch
                or not n_new_dev.is_contiguous() or n_new_dev.device != self.buffer.device):
            raise ValueError(f"n_new_dev must be a contiguous int32 tensor of {self.batch} "
                             f"entries on {self.buffer.device}")
        kvc_static_begin(self.handle, n_new_dev, stream)
        self._step_C = 1

    def static_status(self, stream=None) -> int:
        """Read and clear the sticky flags of static steps (KVC_STATIC_*)."""
        return kvc_static_status(self.handle, stream)

    def sync_lens(self, stream=None):
        """Refresh the host mirror of the row lengths from the device."""
        kvc_sync_lens(self.handle, stream)

    def reset(self, rows, stream=None):
        """Empty rows (release slots): length and left padding 0."""
        kvc_reset(self.handle, rows, stream)

    def page_stats(self):
        """Token counts: used (row lengths), allocated (pages held), reserved (pool)."""
        return kvc_page_stats(self.handle)

    def reserve(self, rows, tokens, stream=None):
        """Paged cache: pages for at least ``tokens`` positions of each row."""
        kvc_reserve(self.handle, rows, tokens, stream)

    def set_first(self, rows, first, stream=None):
        """Rows start with ``first`` left-pad positions (hidden keys)."""
        kvc_set_first(self.handle, rows, first, stream)

    def admit(self, rows, src: "Cache", src_rows, stream=None):
        """Rows ``rows`` become copies of ``src``'s rows ``src_rows``."""
        kvc_admit(self.handle, rows, src.handle, src_rows, stream)

    def lens(self):
        return kvc_lens(self.handle, self.batch)

    def device_lens(self):
        """The device copy of the row lengths (int32 [B]), read back."""
        info = kvc_buffer_info(self.handle)
        return self.buffer[info.lens_offset: info.lens_offset + 4 * self.batch].view(torch.int32).clone()

    def layer_layout(self, layer):
        return kvc_layer_layout(self.handle, layer)

    # -- inspection (tests): views of one layer's K and V -------------------------
    def _elem(self):
        return torch.empty((), dtype=self.dtype).element_size()

    def k_view(self, layer, staging=False):
        """(B, Hkv, rows_alloc, D) view of the stored (rotated) keys."""
        info = self.layer_layout(layer)
        off = info.stage_k_offset if staging else info.k_offset
        rows = info.stage_rows_alloc if staging else info.rows_alloc
        n = self.batch * info.n_kv_head * rows * self.head_dim
        s = self._elem()
        return self.buffer[off: off + n * s].view(self.dtype).view(
            self.batch, info.n_kv_head, rows, self.head_dim)

    def v_view(self, layer, staging=False):
        """(B, Hkv, rows_alloc, D) copy of the stored values (un-blocked)."""
        info = self.layer_layout(layer)
        off = info.stage_v_offset if staging else info.v_offset
        rows = info.stage_rows_alloc if staging else info.rows_alloc
        n = self.batch * info.n_kv_head * rows * self.head_dim
        s = self._elem()
        raw = self.buffer[off: off + n * s].view(self.dtype).view(
            self.batch, info.n_kv_head, rows // 16, self.head_dim, 16)
        return raw.permute(0, 1, 2, 4, 3).reshape(self.batch, info.n_kv_head, rows, self.head_dim)

    def v_raw(self, layer):
        """The blocked storage itself, (B, Hkv, rows_alloc/16, D, 16), as a view."""
        info = self.layer_layout(layer)
        n = self.batch * info.n_kv_head * info.rows_alloc * self.head_dim
        s = self._elem()
        return self.buffer[info.v_offset: info.v_offset + n * s].view(self.dtype).view(
            self.batch, info.n_kv_head, info.rows_alloc // 16, self.head_dim, 16)


class StaticDecodeGraph:
    """A one-token step over every layer of ``cache``, captured once in a HIP
    graph (through ``torch.cuda.CUDAGraph``) and replayed.

    The step reads its inputs from tensors this object owns: ``n_new`` (int32
    [B], 0 or 1 per row), ``q[l]`` (B, 1, Hq, D), ``k[l]`` and ``v[l]``
    (B, 1, Hkv_l, D); it writes ``out[l]`` and, with ``slots``, ``slot[l]``
    (int32 (B, 1)).  Fill the inputs, call ``replay()``; each replay is one
    kvc_static_begin, every layer's kvc_append_attend (``fused``) or
    kvc_append + kvc_attend, and kvc_advance.  The host mirror of the row
    lengths is stale after a replay: call ``cache.sync_lens()`` before eager
    steps.
    """

    def __init__(self, cache: "Cache", fused=True, slots=False):
        dev = cache.buffer.device
        B, Hq, D = cache.batch, cache.n_q_head, cache.head_dim
        self.cache = cache
        self.n_new = torch.zeros(B, dtype=torch.int32, device=dev)
        self.q = [torch.zeros(B, 1, Hq, D, dtype=cache.dtype, device=dev)
                  for _ in range(cache.n_layer)]
        self.k = [torch.zeros(B, 1, h, D, dtype=cache.dtype, device=dev) for h in cache.n_kv_head]
        self.v = [torch.zeros(B, 1, h, D, dtype=cache.dtype, device=dev) for h in cache.n_kv_head]
        self.out = [torch.zeros_like(x) for x in self.q]
        self.slot = ([torch.zeros(B, 1, dtype=torch.int32, device=dev)
                      for _ in range(cache.n_layer)] if slots else [None] * cache.n_layer)
        torch.cuda.synchronize(dev)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            cache.static_begin(self.n_new)
            for l in range(cache.n_layer):
                if fused:
                    cache.append_attend(l, self.q[l], self.k[l], self.v[l], None, out=self.out[l],
                                        slot_out=self.slot[l])
                else:
                    cache.append(l, self.k[l], self.v[l], None, slot_out=self.slot[l])
                    cache.attend(l, self.q[l], self.out[l])
            cache.advance()

    def replay(self):
        self.graph.replay()

