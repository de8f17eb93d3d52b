"""Thin ctypes binding of the C ABI in include/sf_kv.h.

Same names as the C entry points; argument marshalling only (torch tensors ->
device pointers, the current HIP stream -> void*).  Every step of the decode
path runs in the HIP library; there is no fallback: if libsf_kv.so is not
built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsf_kv.so")

SF_OK, SF_ERR_INVALID_ARG, SF_ERR_UNSUPPORTED, SF_ERR_HIP, SF_ERR_OOM, SF_ERR_TIMEOUT, SF_ERR_STATE = \
    0, -1, -2, -3, -4, -5, -6
SF_TIER_DEVICE, SF_TIER_HOST_PINNED = 0, 1
SF_K, SF_V = 0, 1
SF_DECODE_HIST_CLEAN = 1
SF_DECODE_SKIP_MISSES = 2
SF_DECODE_MULTI_PASS = 4
SF_DECODE_DROP_UNSELECTED = 8
SF_DECODE_ROWS16 = 16
SF_DECODE_SCORE_SOFTMAX = 32
SF_QUANT_FP16_SCALES = 1

c_i32, c_i64, c_vp, c_size = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t

EXPORTS = ("sf_status_string", "sf_last_error_string", "sf_kv_quantize", "sf_kv_quantize_ex", "sf_store_create",
           "sf_store_destroy", "sf_refine_store", "sf_store_clear_cache", "sf_store_check",
           "sf_decode_workspace_size", "sf_decode_step", "sf_decode_step_noalloc",
           "sf_decode_noalloc_max_bytes", "sf_decode_check", "sf_stream_read", "sf_decode_form",
           "sf_w_quantize", "sf_w_gemv_workspace_words", "sf_w_gemv")


class sf_geom(ctypes.Structure):
    _fields_ = [("head_dim", c_i32), ("n_q_heads", c_i32), ("n_kv_heads", c_i32),
                ("base_bits", c_i32), ("refine_bits", c_i32)]


class sf_wgeom(ctypes.Structure):
    _fields_ = [("m", c_i32), ("k", c_i32), ("base_bits", c_i32), ("refine_bits", c_i32), ("top_k", c_i32),
                ("chunk", c_i32)]


class sf_step_stats(ctypes.Structure):
    _fields_ = [("selected", c_i64), ("hits", c_i64), ("misses", c_i64), ("h2d_bytes", c_i64)]

    def as_dict(self):
        return {k: int(getattr(self, k)) for k, _ in self._fields_}


class sf_decode_args(ctypes.Structure):
    _fields_ = [("batch", c_i32), ("seq_off_host", ctypes.POINTER(c_i64)), ("seq_off_dev", c_vp),
                ("q", c_vp), ("k_codes", c_vp), ("k_scales", c_vp), ("v_codes", c_vp),
                ("v_scales", c_vp), ("cap", c_i64), ("store", c_vp), ("top_t", c_i32), ("out", c_vp),
                ("sel_out", c_vp), ("scores_out", c_vp), ("stats", ctypes.POINTER(sf_step_stats)),
                ("workspace", c_vp), ("workspace_bytes", c_size), ("flags", c_i32),
                ("start_events", c_vp * 5), ("events", c_vp * 5), ("rows16", c_vp)]


class SfError(RuntimeError):
    def __init__(self, status: int, what: str):
        lib = _LIB
        text = lib.sf_status_string(status).decode() if lib else str(status)
        detail = lib.sf_last_error_string().decode() if lib else ""
        super().__init__(f"{what}: {text}" + (f" ({detail})" if detail else ""))
        self.status = status


_LIB: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libsf_kv.so (after torch, so both share one HIP runtime)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    import torch  # noqa: F401  -- binds the library to torch's HIP runtime
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                           "(run `python -m selective_kv_cache_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.sf_status_string.restype = ctypes.c_char_p
    lib.sf_status_string.argtypes = [c_i32]
    lib.sf_last_error_string.restype = ctypes.c_char_p
    lib.sf_last_error_string.argtypes = []
    G = ctypes.POINTER(sf_geom)
    lib.sf_kv_quantize.argtypes = [G, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp]
    lib.sf_kv_quantize_ex.argtypes = [G, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_i32, c_vp]
    lib.sf_store_create.argtypes = [G, c_i64, c_i32, c_i32, c_i32, ctypes.POINTER(c_vp)]
    lib.sf_store_destroy.argtypes = [c_vp]
    lib.sf_refine_store.argtypes = [c_vp, c_i32, c_vp, c_i64, c_i64, c_vp]
    lib.sf_store_clear_cache.argtypes = [c_vp, c_vp]
    lib.sf_store_check.argtypes = [c_vp, c_vp]
    lib.sf_decode_workspace_size.argtypes = [G, c_i32, c_i64, c_i64, c_i32, ctypes.POINTER(c_size)]
    lib.sf_decode_step.argtypes = [G, ctypes.POINTER(sf_decode_args), c_vp]
    lib.sf_decode_step_noalloc.argtypes = [G, ctypes.POINTER(sf_decode_args), c_vp]
    lib.sf_decode_noalloc_max_bytes.argtypes = []
    lib.sf_decode_check.argtypes = [c_vp, c_vp]
    lib.sf_stream_read.argtypes = [c_vp, c_size, ctypes.c_uint32, c_vp, c_i32, c_vp]
    lib.sf_decode_form.argtypes = [G, ctypes.POINTER(sf_decode_args), ctypes.POINTER(c_i32)]
    WG = ctypes.POINTER(sf_wgeom)
    lib.sf_w_quantize.argtypes = [WG, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]
    lib.sf_w_gemv_workspace_words.argtypes = [WG, ctypes.POINTER(c_i32)]
    lib.sf_w_gemv.argtypes = [WG, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]
    for name in EXPORTS:
        if name not in ("sf_status_string", "sf_last_error_string", "sf_decode_noalloc_max_bytes"):
            getattr(lib, name).restype = c_i32
    lib.sf_decode_noalloc_max_bytes.restype = c_size
    _LIB = lib
    return lib


class TimingEvent:
    """A HIP event created without the system-scope fence (hipEventDisableSystemFence),
    for the ``events`` of sf_decode_step: it times the kernel it is attached to,
    not the cache write-back a fenced event adds after it."""

    _hip: Optional[ctypes.CDLL] = None
    _FLAGS = 0x20000000      # hipEventDisableSystemFence

    @classmethod
    def _runtime(cls) -> ctypes.CDLL:
        if cls._hip is None:
            load()                                     # torch first: one HIP runtime in the process
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(c_vp), ctypes.c_uint]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), c_vp, c_vp]
            hip.hipEventDestroy.argtypes = [c_vp]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        h = c_vp()
        rc = self._runtime().hipEventCreateWithFlags(ctypes.byref(h), self._FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.handle = h.value

    def elapsed_ms(self, end: "TimingEvent") -> float:
        ms = ctypes.c_float()
        rc = self._runtime().hipEventElapsedTime(ctypes.byref(ms), self.handle, end.handle)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self) -> None:
        if self.handle:
            self._runtime().hipEventDestroy(self.handle)
            self.handle = None


def _check(status: int, what: str) -> None:
    if status != SF_OK:
        raise SfError(status, what)


def _ptr(t) -> int:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_P_I64 = ctypes.POINTER(c_i64)


def _i64_ptr(a: np.ndarray):
    """Pointer to a contiguous int64 array's data (ndarray.ctypes.data_as
    costs tens of microseconds a call; a cast of the address does not)."""
    return ctypes.cast(a.ctypes.data, _P_I64)


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def geom(head_dim: int, n_q_heads: int, n_kv_heads: int, base_bits: int, refine_bits: int) -> sf_geom:
    return sf_geom(head_dim, n_q_heads, n_kv_heads, base_bits, refine_bits)


def sf_kv_quantize(g: sf_geom, x, n_tok: int, tok_begin: int, cap: int, codes, scales, refine_rows=None,
                   stream=None, flags: int = 0) -> None:
    """sf_kv_quantize, or sf_kv_quantize_ex when ``flags`` is nonzero."""
    lib = load()
    if flags:
        _check(lib.sf_kv_quantize_ex(ctypes.byref(g), _ptr(x), n_tok, tok_begin, cap, _ptr(codes), _ptr(scales),
                                     _ptr(refine_rows), flags, _stream(stream)), "sf_kv_quantize_ex")
        return
    _check(lib.sf_kv_quantize(ctypes.byref(g), _ptr(x), n_tok, tok_begin, cap, _ptr(codes), _ptr(scales),
                              _ptr(refine_rows), _stream(stream)), "sf_kv_quantize")


def sf_store_create(g: sf_geom, cap_tokens: int, max_seqs: int, tier: int, cache_slots: int) -> int:
    lib = load()
    h = c_vp()
    _check(lib.sf_store_create(ctypes.byref(g), cap_tokens, max_seqs, tier, cache_slots, ctypes.byref(h)),
           "sf_store_create")
    return h.value


def sf_store_destroy(store: int) -> None:
    _check(load().sf_store_destroy(store), "sf_store_destroy")


def sf_refine_store(store: int, which: int, refine_rows, tok_begin: int, n_tok: int, stream=None) -> None:
    _check(load().sf_refine_store(store, which, _ptr(refine_rows), tok_begin, n_tok, _stream(stream)),
           "sf_refine_store")


def sf_store_clear_cache(store: int, stream=None) -> None:
    _check(load().sf_store_clear_cache(store, _stream(stream)), "sf_store_clear_cache")


def sf_store_check(store: int, stream=None) -> int:
    """Debug check of the store; returns the status (SF_OK or SF_ERR_STATE)."""
    return int(load().sf_store_check(store, _stream(stream)))


def sf_decode_workspace_size(g: sf_geom, batch: int, total_tokens: int, max_seq_tokens: int,
                             top_t: int) -> int:
    n = c_size()
    _check(load().sf_decode_workspace_size(ctypes.byref(g), batch, total_tokens, max_seq_tokens, top_t,
                                           ctypes.byref(n)), "sf_decode_workspace_size")
    return int(n.value)


def sf_decode_form(g: sf_geom, seq_off_host: Sequence[int], top_t: int, store: Optional[int], flags: int = 0) -> int:
    """Kernels per step of sf_decode_step for these arguments: 1 or 5."""
    off = np.ascontiguousarray(np.asarray(seq_off_host, dtype=np.int64))
    a = sf_decode_args()
    a.batch = len(off) - 1
    a.seq_off_host = _i64_ptr(off)
    a.store, a.top_t, a.flags = store, top_t, flags
    k = c_i32()
    _check(load().sf_decode_form(ctypes.byref(g), ctypes.byref(a), ctypes.byref(k)), "sf_decode_form")
    return int(k.value)


def sf_decode_check(workspace=None, stream=None) -> int:
    """Status of the steps run on ``workspace`` (None: the no-alloc scratch)."""
    return int(load().sf_decode_check(_ptr(workspace), _stream(stream)))


def sf_stream_read(buf, nbytes: int, never: int, sink, blocks: int, stream=None) -> None:
    _check(load().sf_stream_read(_ptr(buf), nbytes, never, _ptr(sink), blocks, _stream(stream)), "sf_stream_read")


def sf_decode_noalloc_max_bytes() -> int:
    return int(load().sf_decode_noalloc_max_bytes())


def sf_decode_step(g: sf_geom, *, seq_off_host: Sequence[int], seq_off_dev, q, k_codes, k_scales, v_codes,
                   v_scales, cap: int, store: Optional[int], top_t: int, out, workspace, sel_out=None,
                   scores_out=None, want_stats: bool = False, events=None, stream=None, flags: int = 0,
                   noalloc: bool = False, rows16=None):
    """One decode step; returns the step statistics as a dict when asked.
    ``noalloc``: sf_decode_step_noalloc (the library's scratch; ``workspace``
    may then be None).  ``rows16``: the [2][Hkv][cap][D] fp16 rows for
    SF_DECODE_ROWS16."""
    off = np.ascontiguousarray(np.asarray(seq_off_host, dtype=np.int64))
    a = sf_decode_args()
    a.batch = len(off) - 1
    a.seq_off_host = _i64_ptr(off)
    a.seq_off_dev = _ptr(seq_off_dev)
    a.q, a.k_codes, a.k_scales = _ptr(q), _ptr(k_codes), _ptr(k_scales)
    a.v_codes, a.v_scales = _ptr(v_codes), _ptr(v_scales)
    a.cap, a.store, a.top_t = cap, store, top_t
    a.out, a.sel_out, a.scores_out = _ptr(out), _ptr(sel_out), _ptr(scores_out)
    st = sf_step_stats()
    a.stats = ctypes.pointer(st) if want_stats else None
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a.flags = flags
    a.rows16 = _ptr(rows16)
    if events is not None:
        # (start, stop) pairs of score, scan, resolve, attention, combine; a
        # stop alone, or None, allowed
        h = lambda e: None if e is None else (e.handle if hasattr(e, "handle") else
                                              e.cuda_event if hasattr(e, "cuda_event") else e)
        for i, e in enumerate(events):
            if isinstance(e, tuple):
                a.start_events[i], a.events[i] = h(e[0]), h(e[1])
            else:
                a.events[i] = h(e)
    fn = load().sf_decode_step_noalloc if noalloc else load().sf_decode_step
    _check(fn(ctypes.byref(g), ctypes.byref(a), _stream(stream)),
           "sf_decode_step_noalloc" if noalloc else "sf_decode_step")
    return st.as_dict() if want_stats else None


def wgeom(m: int, k: int, base_bits: int, refine_bits: int, top_k: int, chunk: int = 1024) -> sf_wgeom:
    return sf_wgeom(m, k, base_bits, refine_bits, top_k, chunk)


def sf_w_quantize(g: sf_wgeom, w, codes, scales, refine_cols, scratch, stream=None) -> None:
    _check(load().sf_w_quantize(ctypes.byref(g), _ptr(w), _ptr(codes), _ptr(scales), _ptr(refine_cols),
                                _ptr(scratch), _stream(stream)), "sf_w_quantize")


def sf_w_gemv_workspace_words(g: sf_wgeom) -> int:
    n = c_i32()
    _check(load().sf_w_gemv_workspace_words(ctypes.byref(g), ctypes.byref(n)), "sf_w_gemv_workspace_words")
    return n.value


def sf_w_gemv(g: sf_wgeom, codes, scales, refine_cols, x, y, sel, workspace, stream=None) -> None:
    _check(load().sf_w_gemv(ctypes.byref(g), _ptr(codes), _ptr(scales), _ptr(refine_cols), _ptr(x), _ptr(y),
                            _ptr(sel), _ptr(workspace), _stream(stream)), "sf_w_gemv")
