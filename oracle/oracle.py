"""ctypes front end of ``tria_oracle.c`` (fp64 CPU reference).

TEST INFRASTRUCTURE ONLY.  This module shares no code with the HIP library
and never imports the product package.  Each wrapper below only marshals
numpy arrays; the arithmetic lives in ``tria_oracle.c``, whose comments cite
the passages of the source pages each step follows:

* "TriAttention Native C++ Worklog" -- direct scoring of the stored rotated
  key with the query-side phase term and the additive |K_rot| term
  (section "Phase 9: final root cause ..."), absolute position for the phase
  (section "2026-04-18: later-compaction absolute-position bug isolated and
  fixed"), kept rows equal to the budget (compaction schedule logs).
* llama.cpp docs "TriAttention KV-Cache Eviction (--triattention)" --
  protect / sort / evict / compact (section 5, "Phase B") and per-head
  z-normalisation followed by a max over the GQA group (section 5, "Phase C").
* Shared keep sets (one per KV head across layers, or one for the whole
  cache): the worklog's per-head keep sets gathered in every layer and the
  llama.cpp page's global z-normalisation shader; the cross-unit reduction is
  read as the GQA group's max taken over the larger group.
* Decode attention over a (compacted) cache: softmax of scaled q.k over the
  unit's rows, weights times V, per query head of the GQA group -- the step
  the eviction pass exists to make cheaper.
* Calibration statistics: per query head and frequency pair, the mean
  pre-RoPE query pair, the mean pair magnitude and the norm weight
  q_abs - |q_mean| (llama.cpp page section 2, the generator's accumulation).
* Hole-filling compaction (a variant of the order-preserving gather): the
  page asks for the kept rows packed in place without gaps; the variant keeps
  the sinks first and the newest rows last, in order, and fills the holes
  below them from above.

Every function here is pinned by ``tests/test_oracle_pins.py`` against closed
forms, brute force and hand-worked fixtures.  One reading is not pinned by
anything on the pages: agreement with the upstream implementation's exact
conventions (normalisation population, offset set) -- parity unpinned there.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

KV_F16 = 0
KV_Q8_0 = 1

# compaction rule (tria_oracle.c, orc_evict_ex)
COMPACT_ORDERED = 0   # order-preserving gather (the pages' rule)
COMPACT_HOLEFILL = 1  # holes below the trailing run filled from above it

# keep-set sharing (tria_oracle.c, orc_evict_mode)
KEEP_UNIT = 0      # each (layer, KV head) unit selects on its own
KEEP_KV_HEAD = 1   # one keep set per KV head, shared by all layers
KEEP_GLOBAL = 2    # one keep set for the whole cache

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tria_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB = os.path.join(_BUILD, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP over units)."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
            vp = ctypes.c_void_p
            lib.orc_half_to_double.restype = dbl
            lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
            lib.orc_row_bytes.restype = i64
            lib.orc_row_bytes.argtypes = [i32, i32]
            lib.orc_decode_row.restype = i32
            lib.orc_decode_row.argtypes = [i32, vp, i32, vp]
            lib.orc_omega.restype = dbl
            lib.orc_omega.argtypes = [dbl, i32, i32]
            lib.orc_offset_mean.restype = None
            lib.orc_offset_mean.argtypes = [dbl, i32, i64, vp, i32, vp, vp]
            lib.orc_raw_scores_unit.restype = i32
            lib.orc_raw_scores_unit.argtypes = [i32, vp, i64, i64, i32, i32, vp, vp, vp, dbl,
                                                i64, vp, i32, vp]
            lib.orc_aggregate_unit.restype = None
            lib.orc_aggregate_unit.argtypes = [vp, i64, i32, vp, vp, vp]
            lib.orc_kept_count.restype = i64
            lib.orc_kept_count.argtypes = [i64, i64, i64, i64]
            lib.orc_select_unit.restype = i64
            lib.orc_select_unit.argtypes = [vp, i64, i64, i64, i64, vp]
            lib.orc_compact_rows.restype = i32
            lib.orc_compact_rows.argtypes = [vp, i64, vp, i64]
            lib.orc_evict.restype = i64
            lib.orc_evict.argtypes = [i32, i32, i32, i32, i32, i32, dbl, vp, i32, vp, vp, vp,
                                      i64, i64, i64, i64, i64, vp, vp, vp, vp, vp, vp, i32]
            lib.orc_evict_mode.restype = i64
            lib.orc_evict_mode.argtypes = [i32] + lib.orc_evict.argtypes
            lib.orc_evict_ex.restype = i64
            lib.orc_evict_ex.argtypes = [i32, i32] + lib.orc_evict.argtypes
            lib.orc_compact_holefill.restype = i64
            lib.orc_compact_holefill.argtypes = [vp, i64, vp, i64, i64]
            lib.orc_decode_attention_unit.restype = i32
            lib.orc_decode_attention_unit.argtypes = [i32, i32, vp, vp, i64, i32, i32, vp, dbl,
                                                      vp]
            lib.orc_calib_stats.restype = None
            lib.orc_calib_stats.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp]
            lib.orc_num_threads.restype = i32
            lib.orc_num_threads.argtypes = []
            lib.orc_last_stage_seconds.restype = None
            lib.orc_last_stage_seconds.argtypes = [vp]
            _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return _load().orc_num_threads()


def last_stage_seconds():
    """Wall-clock seconds of the last evict() call's stages: (raw scores and per-unit
    z-normalised maxima, group scores and selection, compaction)."""
    out = np.zeros(3, np.float64)
    _load().orc_last_stage_seconds(_p(out))
    return tuple(float(x) for x in out)


def half_to_double(bits: int) -> float:
    return _load().orc_half_to_double(int(bits) & 0xFFFF)


def row_bytes(kv_type: int, hd: int) -> int:
    return int(_load().orc_row_bytes(kv_type, hd))


def decode_rows(kv_type: int, rows: np.ndarray, hd: int) -> np.ndarray:
    """rows: uint8 [n, row_bytes] -> float64 [n, hd]."""
    rows = _c(rows, np.uint8).reshape(-1, row_bytes(kv_type, hd))
    out = np.empty((rows.shape[0], hd), np.float64)
    lib = _load()
    for i in range(rows.shape[0]):
        lib.orc_decode_row(kv_type, _p(rows[i]), hd, _p(out[i]))
    return out


def omega(theta: float, hd: int) -> np.ndarray:
    lib = _load()
    return np.array([lib.orc_omega(theta, hd, f) for f in range(hd // 2)])


def offset_mean(theta: float, hd: int, p: int, offsets) -> np.ndarray:
    """A_f for f < hd/2, complex128."""
    offs = _c(offsets, np.int64)
    re = np.empty(hd // 2, np.float64)
    im = np.empty(hd // 2, np.float64)
    _load().orc_offset_mean(theta, hd, int(p), _p(offs), len(offs), _p(re), _p(im))
    return re + 1j * im


def raw_scores_unit(kv_type: int, k_rows: np.ndarray, hd: int, q_re, q_im, w, theta: float,
                    p: int, offsets) -> np.ndarray:
    """k_rows: uint8 [n, row_bytes]; q_re/q_im/w: [G, F].  Returns [n, G] fp64."""
    rb = row_bytes(kv_type, hd)
    k_rows = _c(k_rows, np.uint8).reshape(-1, rb)
    q_re, q_im, w = (_c(x, np.float32).reshape(-1, hd // 2) for x in (q_re, q_im, w))
    G = q_re.shape[0]
    offs = _c(offsets, np.int64)
    n = k_rows.shape[0]
    out = np.empty((n, G), np.float64)
    rc = _load().orc_raw_scores_unit(kv_type, _p(k_rows), rb, n, hd, G, _p(q_re), _p(q_im),
                                     _p(w), float(theta), int(p), _p(offs), len(offs), _p(out))
    if rc != 0:
        raise MemoryError("oracle raw score failed")
    return out


def aggregate_unit(raw: np.ndarray):
    """raw: [n, G] -> (agg [n], mu [G], sigma [G])."""
    raw = _c(raw, np.float64)
    n, G = raw.shape
    agg = np.empty(n, np.float64)
    mu = np.empty(G, np.float64)
    sg = np.empty(G, np.float64)
    _load().orc_aggregate_unit(_p(raw), n, G, _p(agg), _p(mu), _p(sg))
    return agg, mu, sg


def kept_count(n: int, budget: int, sink: int, window: int) -> int:
    return int(_load().orc_kept_count(n, budget, sink, window))


def select_unit(agg: np.ndarray, budget: int, sink: int, window: int) -> np.ndarray:
    agg = _c(agg, np.float64)
    n = agg.shape[0]
    out = np.empty(max(n, 1), np.int32)
    K = _load().orc_select_unit(_p(agg), n, budget, sink, window, _p(out))
    if K < 0:
        raise ValueError("oracle select: bad arguments")
    return out[:K].copy()


def compact_rows(rows: np.ndarray, keep_idx: np.ndarray) -> np.ndarray:
    """Returns a compacted copy of rows (first K rows gathered, rest unchanged)."""
    out = np.array(rows, copy=True, order="C")
    rb = out.reshape(out.shape[0], -1).view(np.uint8).shape[1]
    ki = _c(keep_idx, np.int32)
    if _load().orc_compact_rows(_p(out), rb, _p(ki), len(ki)) != 0:
        raise MemoryError("oracle compact failed")
    return out


def compact_holefill(rows: np.ndarray, keep_idx: np.ndarray, n: int):
    """Hole-filling compaction of a copy of rows [n, ...]; returns (rows, moves)."""
    out = np.array(rows, copy=True, order="C")
    rb = out.reshape(out.shape[0], -1).view(np.uint8).shape[1]
    ki = _c(keep_idx, np.int32)
    moves = _load().orc_compact_holefill(_p(out), rb, _p(ki), len(ki), int(n))
    if moves < 0:
        raise MemoryError("oracle hole-fill compaction failed")
    return out, int(moves)


def decode_attention_unit(k_type: int, v_type: int, k_rows: np.ndarray, v_rows: np.ndarray,
                          hd: int, q: np.ndarray, scale: float) -> np.ndarray:
    """k_rows, v_rows: uint8 [n, row_bytes]; q: [G, hd].  Returns out [G, hd] fp64."""
    k_rows = _c(k_rows, np.uint8).reshape(-1, row_bytes(k_type, hd))
    v_rows = _c(v_rows, np.uint8).reshape(-1, row_bytes(v_type, hd))
    q = _c(q, np.float64).reshape(-1, hd)
    out = np.empty_like(q)
    rc = _load().orc_decode_attention_unit(k_type, v_type, _p(k_rows), _p(v_rows),
                                           k_rows.shape[0], hd, q.shape[0], _p(q), float(scale),
                                           _p(out))
    if rc != 0:
        raise ValueError("oracle decode attention failed")
    return out


def calib_stats(q: np.ndarray):
    """q: [T, H, hd] query values (any float dtype; fp16/fp32 widen exactly, a
    bfloat16 stream is passed as its float32 widening).  Returns fp64 arrays
    (q_re, q_im, q_abs, w), each [H, hd/2]."""
    q = _c(q, np.float64)
    T, H, hd = q.shape
    out = [np.empty((H, hd // 2), np.float64) for _ in range(4)]
    _load().orc_calib_stats(_p(q), T, H, hd, *[_p(x) for x in out])
    return tuple(out)


def evict(k_type: int, v_type: int, L: int, Hkv: int, Hq: int, hd: int, theta: float, offsets,
          k: np.ndarray, v: np.ndarray, pos: np.ndarray, n: int, budget: int, sink: int,
          window: int, q_re, q_im, w, want_raw=True, want_agg=True, compact=True,
          keep_mode: int = KEEP_UNIT, compact_mode: int = COMPACT_ORDERED):
    """Whole pass over a contiguous host cache [L][Hkv][cap][row] (in place).

    keep_mode: KEEP_UNIT, KEEP_KV_HEAD or KEEP_GLOBAL (who shares a keep set).
    compact_mode: COMPACT_ORDERED or COMPACT_HOLEFILL.
    Returns dict(kept, keep_idx [L,Hkv,K], raw [L,Hkv,n,G] or None, agg
    [L,Hkv,n] -- the score each unit's keep set was selected on -- or None).
    """
    assert k.flags.c_contiguous and v.flags.c_contiguous and pos.flags.c_contiguous
    cap = pos.shape[-1]
    G = Hq // Hkv
    K = kept_count(n, budget, sink, window)
    if K < 0:
        raise ValueError("bad budget/sink/window")
    keep = np.empty((L, Hkv, max(K, 1)), np.int32)
    raw = np.empty((L, Hkv, n, G), np.float64) if want_raw else None
    agg = np.empty((L, Hkv, n), np.float64) if want_agg else None
    q_re, q_im, w = (_c(x, np.float32) for x in (q_re, q_im, w))
    offs = _c(offsets, np.int64)
    rc = _load().orc_evict_ex(int(keep_mode), int(compact_mode), k_type, v_type, L, Hkv, Hq, hd,
                              float(theta), _p(offs), len(offs), _p(k), _p(v), _p(pos), cap, n,
                              budget, sink, window, _p(q_re), _p(q_im), _p(w), _p(keep), _p(raw),
                              _p(agg), 1 if compact else 0)
    if rc < 0:
        raise RuntimeError("oracle evict failed")
    return {"kept": int(rc), "keep_idx": keep[:, :, :K], "raw": raw, "agg": agg}
