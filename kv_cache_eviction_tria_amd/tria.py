"""ctypes binding of libtria.so: the same entry points as include/tria.h.

Argument marshalling only: every step of the pass runs in the HIP kernels of
libtria.so.  PyTorch supplies device memory (tensors are passed by data
pointer) and the stream (torch's current stream unless one is given).  If the
library is not built this module raises on first use; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libtria.so")

TRIA_OK = 0
TRIA_E_INVAL = -1
TRIA_E_UNSUPPORTED = -2
TRIA_E_HIP = -3
TRIA_E_NOMEM = -4
TRIA_E_DEVICE = -5
TRIA_KV_F16 = 0
TRIA_KV_Q8_0 = 1
TRIA_MAX_SEQ = 64
TRIA_MAX_ROWS = 262144
TRIA_BLOCK = 16

_lock = threading.Lock()
_lib = None


class TriaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, tria_strerror(code), code))


class ModelDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("n_q_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("k_type", ctypes.c_int32), ("v_type", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("n_offsets", ctypes.c_int32),
                ("offsets", ctypes.POINTER(ctypes.c_int64))]


class Cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("pos", ctypes.c_void_p),
                ("cap", ctypes.c_int64)]


class PagedCache(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("pos_pool", ctypes.c_void_p), ("n_blocks", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("max_blocks", ctypes.c_int32)]


class Policy(ctypes.Structure):
    """tria_policy: when the decode loop runs an eviction pass."""
    _fields_ = [("trigger", ctypes.c_int32), ("protect_prefill", ctypes.c_int32),
                ("budget", ctypes.c_int64), ("divide_length", ctypes.c_int64),
                ("interval", ctypes.c_int64), ("sink", ctypes.c_int64),
                ("window", ctypes.c_int64)]


class DecodeState(ctypes.Structure):
    """tria_decode_state: rows in the cache, prompt rows, steps since the last pass."""
    _fields_ = [("n_rows", ctypes.c_int64), ("n_prompt", ctypes.c_int64),
                ("steps", ctypes.c_int64), ("passes", ctypes.c_int64)]


def lib():
    """Load libtria.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError("libtria.so is not built (%s); run "
                                  "kv_cache_eviction_tria_amd.build.build()" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
            L.tria_load_stats.restype = ctypes.c_int
            L.tria_load_stats.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(ModelDesc), vp, vp,
                                          vp, vp]
            L.tria_free.restype = None
            L.tria_free.argtypes = [vp]
            L.tria_strerror.restype = ctypes.c_char_p
            L.tria_strerror.argtypes = [ctypes.c_int]
            L.tria_last_hip_error.restype = ctypes.c_int
            L.tria_last_hip_error.argtypes = [vp]
            L.tria_row_bytes.restype = i64
            L.tria_row_bytes.argtypes = [i32, i32]
            L.tria_kept_count.restype = i64
            L.tria_kept_count.argtypes = [i64, i64, i64, i64]
            L.tria_score.restype = ctypes.c_int
            L.tria_score.argtypes = [vp, ctypes.POINTER(Cache), i64, vp, vp]
            L.tria_select.restype = i64
            L.tria_select.argtypes = [vp, vp, i64, i64, i64, i64, vp, vp, vp]
            L.tria_compact.restype = ctypes.c_int
            L.tria_compact.argtypes = [vp, ctypes.POINTER(Cache), i64, vp, i64, vp]
            L.tria_evict.restype = i64
            L.tria_evict.argtypes = [vp, ctypes.POINTER(Cache), i64, i64, i64, i64, vp]
            L.tria_evict_noalloc.restype = i64
            L.tria_evict_noalloc.argtypes = [vp, ctypes.POINTER(Cache), i64, i64, i64, i64, vp]
            L.tria_evict_paged_batch.restype = ctypes.c_int
            L.tria_evict_paged_batch.argtypes = [vp, ctypes.POINTER(PagedCache), i32, vp, vp, i64,
                                                 i64, vp, vp]
            L.tria_set_keep_mode.restype = ctypes.c_int
            L.tria_set_keep_mode.argtypes = [vp, i32]
            L.tria_set_compaction_workgroups.restype = ctypes.c_int
            L.tria_set_compaction_workgroups.argtypes = [vp, i32]
            L.tria_set_compaction.restype = ctypes.c_int
            L.tria_set_compaction.argtypes = [vp, i32]
            L.tria_decode_attention.restype = ctypes.c_int
            L.tria_decode_attention.argtypes = [vp, ctypes.POINTER(Cache), i64, vp,
                                                ctypes.c_float, vp, vp]
            L.tria_decode_attention_paged_batch.restype = ctypes.c_int
            L.tria_decode_attention_paged_batch.argtypes = [vp, ctypes.POINTER(PagedCache), i32,
                                                            vp, vp, ctypes.c_float, vp, vp]
            L.tria_policy_due.restype = ctypes.c_int
            L.tria_policy_due.argtypes = [ctypes.POINTER(Policy), ctypes.POINTER(DecodeState),
                                          ctypes.POINTER(i64), ctypes.POINTER(i64),
                                          ctypes.POINTER(i64)]
            L.tria_policy_peak_rows.restype = i64
            L.tria_policy_peak_rows.argtypes = [ctypes.POINTER(Policy), i64]
            L.tria_decode_step.restype = i64
            L.tria_decode_step.argtypes = [vp, ctypes.POINTER(Cache), ctypes.POINTER(Policy),
                                           ctypes.POINTER(DecodeState), vp]
            L.tria_calib_create.restype = ctypes.c_int
            L.tria_calib_create.argtypes = [ctypes.POINTER(vp), i32, i32, i32]
            L.tria_calib_add.restype = ctypes.c_int
            L.tria_calib_add.argtypes = [vp, i32, vp, i32, i64, i64, vp]
            L.tria_calib_add_layers.restype = ctypes.c_int
            L.tria_calib_add_layers.argtypes = [vp, i32, i32, vp, i32, i64, i64, i64, vp]
            L.tria_calib_tokens.restype = i64
            L.tria_calib_tokens.argtypes = [vp, i32]
            L.tria_calib_finish.restype = ctypes.c_int
            L.tria_calib_finish.argtypes = [vp, vp, vp, vp, vp, vp]
            L.tria_calib_free.restype = None
            L.tria_calib_free.argtypes = [vp]
            L.tria_device_status.restype = ctypes.c_int
            L.tria_device_status.argtypes = [vp]
            L.tria_timing_enable.restype = ctypes.c_int
            L.tria_timing_enable.argtypes = [vp, i32]
            L.tria_timing_read.restype = ctypes.c_int
            L.tria_timing_read.argtypes = [vp, vp, vp]
            _lib = L
    return _lib


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t, name, dtype=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must have dtype %s" % (name, dtype))
    return ctypes.c_void_p(t.data_ptr())


def _check(code, where):
    if code < 0:
        raise TriaError(int(code), where)
    return code


def tria_strerror(code: int) -> str:
    return lib().tria_strerror(int(code)).decode()


def tria_row_bytes(kv_type: int, head_dim: int) -> int:
    return int(lib().tria_row_bytes(kv_type, head_dim))


def tria_kept_count(n_tokens: int, budget: int, sink: int, window: int) -> int:
    return int(_check(lib().tria_kept_count(n_tokens, budget, sink, window), "tria_kept_count"))


class TriaCtx:
    """Owns a tria_ctx handle (device statistics and scratch)."""

    def __init__(self, handle, desc):
        self.handle = handle
        self.n_layers = desc.n_layers
        self.n_kv_heads = desc.n_kv_heads
        self.n_q_heads = desc.n_q_heads
        self.head_dim = desc.head_dim
        self.k_type = desc.k_type
        self.v_type = desc.v_type

    @property
    def G(self):
        return self.n_q_heads // self.n_kv_heads

    def close(self):
        if self.handle:
            lib().tria_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tria_load_stats(n_layers, n_kv_heads, n_q_heads, head_dim, k_type, v_type, rope_theta,
                    offsets, q_re, q_im, norm_w, stream=None) -> TriaCtx:
    """q_re, q_im, norm_w: host float32 arrays [L][Hq][hd/2] (numpy or CPU tensors)."""
    import numpy as np
    arrs = [np.ascontiguousarray(np.asarray(a, dtype=np.float32)) for a in (q_re, q_im, norm_w)]
    offs = (ctypes.c_int64 * len(offsets))(*[int(x) for x in offsets])
    d = ModelDesc(n_layers, n_kv_heads, n_q_heads, head_dim, k_type, v_type, float(rope_theta),
                  len(offsets), offs)
    h = ctypes.c_void_p()
    rc = lib().tria_load_stats(ctypes.byref(h), ctypes.byref(d),
                               *[a.ctypes.data_as(ctypes.c_void_p) for a in arrs],
                               _stream(stream) if torch.cuda.is_available() else None)
    _check(rc, "tria_load_stats")
    return TriaCtx(h, d)


def _cache(k, v, pos):
    return Cache(_ptr(k, "k", torch.uint8), _ptr(v, "v", torch.uint8),
                 _ptr(pos, "pos", torch.int32), pos.shape[-1])


def tria_score(ctx: TriaCtx, k, v, pos, n_tokens: int, raw_scores, stream=None) -> None:
    """k, v: uint8 [L,Hkv,cap,row_bytes]; pos: int32 [L,Hkv,cap];
    raw_scores: float32 [L,Hkv,n_tokens,G] (written)."""
    c = _cache(k, v, pos)
    _check(lib().tria_score(ctx.handle, ctypes.byref(c), n_tokens,
                            _ptr(raw_scores, "raw_scores", torch.float32), _stream(stream)),
           "tria_score")


def tria_select(ctx: TriaCtx, raw_scores, n_tokens: int, budget: int, sink: int, window: int,
                keep_idx, agg_out=None, stream=None) -> int:
    """keep_idx: int32 [L,Hkv,kept] (written); agg_out: float32 [L,Hkv,n_tokens] or None."""
    return int(_check(lib().tria_select(ctx.handle, _ptr(raw_scores, "raw_scores", torch.float32),
                                        n_tokens, budget, sink, window,
                                        _ptr(keep_idx, "keep_idx", torch.int32),
                                        _ptr(agg_out, "agg_out", torch.float32),
                                        _stream(stream)), "tria_select"))


def tria_compact(ctx: TriaCtx, k, v, pos, n_tokens: int, keep_idx, kept: int, stream=None) -> None:
    c = _cache(k, v, pos)
    _check(lib().tria_compact(ctx.handle, ctypes.byref(c), n_tokens,
                              _ptr(keep_idx, "keep_idx", torch.int32), kept, _stream(stream)),
           "tria_compact")


def tria_evict(ctx: TriaCtx, k, v, pos, n_tokens: int, budget: int, sink: int, window: int,
               stream=None) -> int:
    c = _cache(k, v, pos)
    return int(_check(lib().tria_evict(ctx.handle, ctypes.byref(c), n_tokens, budget, sink,
                                       window, _stream(stream)), "tria_evict"))


def tria_evict_noalloc(ctx: TriaCtx, k, v, pos, n_tokens: int, budget: int, sink: int,
                       window: int, stream=None) -> int:
    """tria_evict with the library's fixed per-GPU scratch (no allocation in the call)."""
    c = _cache(k, v, pos)
    return int(_check(lib().tria_evict_noalloc(ctx.handle, ctypes.byref(c), n_tokens, budget,
                                               sink, window, _stream(stream)),
                      "tria_evict_noalloc"))


TRIA_NOALLOC_SCRATCH_BYTES = 67108864  # 64 MiB


def tria_evict_paged_batch(ctx: TriaCtx, k_pool, v_pool, pos_pool, block_table, n_tokens,
                           budget, sink: int, window: int, stream=None):
    """k_pool, v_pool: uint8 [L,n_blocks,Hkv,16,row_bytes]; pos_pool: int32
    [L,n_blocks,Hkv,16]; block_table: int32 [n_seq,max_blocks] (device);
    n_tokens, budget: host sequences of length n_seq.  Returns kept counts."""
    n_seq = len(n_tokens)
    nt = (ctypes.c_int64 * n_seq)(*[int(x) for x in n_tokens])
    bd = (ctypes.c_int64 * n_seq)(*[int(x) for x in budget])
    kept = (ctypes.c_int64 * n_seq)()
    pc = PagedCache(_ptr(k_pool, "k_pool", torch.uint8), _ptr(v_pool, "v_pool", torch.uint8),
                    _ptr(pos_pool, "pos_pool", torch.int32), pos_pool.shape[1],
                    _ptr(block_table, "block_table", torch.int32), block_table.shape[1])
    _check(lib().tria_evict_paged_batch(ctx.handle, ctypes.byref(pc), n_seq, nt, bd, sink,
                                        window, kept, _stream(stream)), "tria_evict_paged_batch")
    return [int(x) for x in kept]


def tria_decode_attention(ctx: TriaCtx, k, v, pos, n_tokens: int, q, scale=None, out=None,
                          stream=None):
    """q: device fp32 [L, Hq, hd]; returns out (device fp32 [L, Hq, hd]).  scale
    defaults to 1/sqrt(hd)."""
    if scale is None:
        scale = 1.0 / float(ctx.head_dim) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    cache = _cache(k, v, pos)
    _check(lib().tria_decode_attention(ctx.handle, ctypes.byref(cache), int(n_tokens),
                                       _ptr(q, "q", torch.float32), float(scale),
                                       _ptr(out, "out", torch.float32), _stream(stream)),
           "tria_decode_attention")
    return out


def tria_decode_attention_paged_batch(ctx: TriaCtx, k_pool, v_pool, pos_pool, block_table,
                                      n_tokens, q, scale=None, out=None, stream=None):
    """q: device fp32 [n_seq, L, Hq, hd]; returns out of the same shape."""
    if scale is None:
        scale = 1.0 / float(ctx.head_dim) ** 0.5
    if out is None:
        out = torch.empty_like(q)
    n_seq = len(n_tokens)
    nt = (ctypes.c_int64 * n_seq)(*[int(x) for x in n_tokens])
    pc = PagedCache(_ptr(k_pool, "k_pool", torch.uint8), _ptr(v_pool, "v_pool", torch.uint8),
                    _ptr(pos_pool, "pos_pool", torch.int32), pos_pool.shape[1],
                    _ptr(block_table, "block_table", torch.int32), block_table.shape[1])
    _check(lib().tria_decode_attention_paged_batch(ctx.handle, ctypes.byref(pc), n_seq, nt,
                                                   _ptr(q, "q", torch.float32), float(scale),
                                                   _ptr(out, "out", torch.float32),
                                                   _stream(stream)),
           "tria_decode_attention_paged_batch")
    return out


TRIA_KEEP_PER_UNIT = 0
TRIA_KEEP_PER_KV_HEAD = 1
TRIA_KEEP_GLOBAL = 2


def tria_set_keep_mode(ctx: TriaCtx, mode: int) -> None:
    """Who shares a keep set: TRIA_KEEP_PER_UNIT (default), TRIA_KEEP_PER_KV_HEAD
    (one per KV head across layers) or TRIA_KEEP_GLOBAL (one for the cache)."""
    _check(lib().tria_set_keep_mode(ctx.handle, int(mode)), "tria_set_keep_mode")


TRIA_COMPACT_ORDERED = 0
TRIA_COMPACT_HOLE_FILL = 1

TRIA_TRIGGER_THRESHOLD = 0
TRIA_TRIGGER_INTERVAL = 1


def tria_policy_due(policy: Policy, state: DecodeState):
    """(budget, sink, window) of the pass due now, or None."""
    b, s_, w = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = _check(lib().tria_policy_due(ctypes.byref(policy), ctypes.byref(state), ctypes.byref(b),
                                      ctypes.byref(s_), ctypes.byref(w)), "tria_policy_due")
    return (b.value, s_.value, w.value) if rc == 1 else None


def tria_policy_peak_rows(policy: Policy, n_prompt: int) -> int:
    return int(_check(lib().tria_policy_peak_rows(ctypes.byref(policy), int(n_prompt)),
                      "tria_policy_peak_rows"))


def tria_decode_step(ctx: TriaCtx, k, v, pos, policy: Policy, state: DecodeState,
                     stream=None) -> int:
    """One decode step after the caller appended its row; returns the rows now held."""
    cache = _cache(k, v, pos)
    return int(_check(lib().tria_decode_step(ctx.handle, ctypes.byref(cache),
                                             ctypes.byref(policy), ctypes.byref(state),
                                             _stream(stream)), "tria_decode_step"))


TRIA_Q_F32 = 0
TRIA_Q_F16 = 1
TRIA_Q_BF16 = 2
_Q_TYPES = {torch.float32: TRIA_Q_F32, torch.float16: TRIA_Q_F16, torch.bfloat16: TRIA_Q_BF16}


class TriaCalib:
    """Owns a tria_calib handle: GPU accumulators of calibration statistics."""

    def __init__(self, n_layers: int, n_q_heads: int, head_dim: int):
        h = ctypes.c_void_p()
        _check(lib().tria_calib_create(ctypes.byref(h), int(n_layers), int(n_q_heads),
                                       int(head_dim)), "tria_calib_create")
        self.handle = h
        self.n_layers, self.n_q_heads, self.head_dim = n_layers, n_q_heads, head_dim

    def add(self, layer: int, q, stream=None) -> None:
        """q: device [n_tokens, n_q_heads * head_dim (or more)], fp32/fp16/bf16, rows
        contiguous in their first n_q_heads * head_dim values."""
        if not isinstance(q, torch.Tensor) or not q.is_cuda or q.dim() != 2:
            raise TypeError("q must be a 2-D CUDA tensor")
        if q.dtype not in _Q_TYPES or q.stride(1) != 1:
            raise TypeError("q must be fp32/fp16/bf16 with unit stride along a row")
        _check(lib().tria_calib_add(self.handle, int(layer), ctypes.c_void_p(q.data_ptr()),
                                    _Q_TYPES[q.dtype], q.shape[0], q.stride(0), _stream(stream)),
               "tria_calib_add")

    def add_layers(self, layer0: int, q, stream=None) -> None:
        """q: device [n_layers, n_tokens, n_q_heads * head_dim (or more)], fp32/fp16/bf16,
        layers layer0 .. layer0 + n_layers - 1 in one launch."""
        if not isinstance(q, torch.Tensor) or not q.is_cuda or q.dim() != 3:
            raise TypeError("q must be a 3-D CUDA tensor")
        if q.dtype not in _Q_TYPES or q.stride(2) != 1:
            raise TypeError("q must be fp32/fp16/bf16 with unit stride along a row")
        _check(lib().tria_calib_add_layers(self.handle, int(layer0), q.shape[0],
                                           ctypes.c_void_p(q.data_ptr()), _Q_TYPES[q.dtype],
                                           q.shape[1], q.stride(1), q.stride(0),
                                           _stream(stream)), "tria_calib_add_layers")

    def tokens(self, layer: int) -> int:
        return int(_check(lib().tria_calib_tokens(self.handle, int(layer)), "tria_calib_tokens"))

    def finish(self, stream=None):
        """Returns device fp32 tensors (q_re, q_im, q_abs, norm_w), each [L, Hq, hd/2]."""
        shape = (self.n_layers, self.n_q_heads, self.head_dim // 2)
        out = [torch.empty(shape, dtype=torch.float32, device="cuda") for _ in range(4)]
        _check(lib().tria_calib_finish(self.handle, *[ctypes.c_void_p(t.data_ptr()) for t in out],
                                       _stream(stream)), "tria_calib_finish")
        return tuple(out)

    def close(self):
        if self.handle:
            lib().tria_calib_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tria_set_compaction(ctx: TriaCtx, mode: int) -> None:
    """TRIA_COMPACT_ORDERED (default gather) or TRIA_COMPACT_HOLE_FILL (variant)."""
    _check(lib().tria_set_compaction(ctx.handle, int(mode)), "tria_set_compaction")


def tria_set_compaction_workgroups(ctx: TriaCtx, max_workgroups: int) -> None:
    """0: as many compaction workgroups as fit (default); 1: one, every task in order."""
    _check(lib().tria_set_compaction_workgroups(ctx.handle, int(max_workgroups)),
           "tria_set_compaction_workgroups")


def tria_device_status(ctx: TriaCtx) -> None:
    """Synchronise the device; raise if a compaction gave up a bounded wait."""
    _check(lib().tria_device_status(ctx.handle), "tria_device_status")


def tria_timing_enable(ctx: TriaCtx, enable: bool) -> None:
    _check(lib().tria_timing_enable(ctx.handle, 1 if enable else 0), "tria_timing_enable")


STAGES = ("score", "select", "compact")


def tria_timing_read(ctx: TriaCtx):
    """Summed kernel ms and launch counts per stage since the last read:
    ({stage: ms}, {stage: launches}, untimed_launches)."""
    ms = (ctypes.c_double * 3)()
    n = (ctypes.c_int64 * 3)()
    rc = lib().tria_timing_read(ctx.handle, ms, n)
    _check(rc, "tria_timing_read")
    return ({s: float(ms[i]) for i, s in enumerate(STAGES)},
            {s: int(n[i]) for i, s in enumerate(STAGES)}, int(rc))


def tria_free(ctx: TriaCtx) -> None:
    ctx.close()
