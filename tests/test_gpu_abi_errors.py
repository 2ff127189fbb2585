"""Argument errors on a live context: every entry point returns its code before
anything is enqueued, so the caller's cache is left byte for byte as it was and
the context stays usable (the boundary's error contract in include/tria.h)."""
import ctypes
import dataclasses

import pytest
import torch

import parity_util as pu
from kv_cache_eviction_tria_amd import synth, tria

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
INVAL, UNSUP = tria.TRIA_E_INVAL, tria.TRIA_E_UNSUPPORTED


def _p(t, off=0):
    """Device address of a tensor, moved by off bytes (a misaligned pointer is
    refused before anything is read through it)."""
    return ctypes.c_void_p(t.data_ptr() + off) if t is not None else None


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_contiguous_entry_points_reject_bad_arguments():
    wl = synth.WORKLOADS["tiny_1x1_4k_f16"]
    n = 1000
    case = synth.make_case(wl, device="cpu", n=n, cap=n)
    stats = (case["q_re"], case["q_im"], case["w"])
    ctx = pu.make_ctx(wl, stats)
    k, v, pos = case["k"].to(DEV), case["v"].to(DEV), case["pos"].to(DEV)
    k0, v0, p0 = k.clone(), v.clone(), pos.clone()
    raw = torch.zeros(1, 1, n + 1, wl.G, dtype=torch.float32, device=DEV)
    keep = torch.zeros(1, 1, n + 1, dtype=torch.int32, device=DEV)
    q = torch.zeros(1, wl.Hq, wl.hd, dtype=torch.float32, device=DEV)
    out = torch.zeros_like(q)
    L = tria.lib()
    h = ctx.handle
    good = tria.Cache(_p(k), _p(v), _p(pos), n)
    no_k = tria.Cache(None, _p(v), _p(pos), n)
    k_off8 = tria.Cache(_p(k, 8), _p(v), _p(pos), n)
    v_off2 = tria.Cache(_p(k), _p(v, 2), _p(pos), n)
    pos_off2 = tria.Cache(_p(k), _p(v), _p(pos, 2), n)
    s = _stream()
    cases = {
        "evict k not 16-byte aligned": (
            lambda: L.tria_evict(h, ctypes.byref(k_off8), n, 100, 4, 16, s), INVAL),
        "evict v not 16-byte aligned": (
            lambda: L.tria_evict(h, ctypes.byref(v_off2), n, 100, 4, 16, s), INVAL),
        "evict pos not 4-byte aligned": (
            lambda: L.tria_evict(h, ctypes.byref(pos_off2), n, 100, 4, 16, s), INVAL),
        "noalloc k not 16-byte aligned": (
            lambda: L.tria_evict_noalloc(h, ctypes.byref(k_off8), n, 100, 4, 16, s), INVAL),
        "score raw not 16-byte aligned": (
            lambda: L.tria_score(h, ctypes.byref(good), n, _p(raw, 4), s), INVAL),
        "score k not 16-byte aligned": (
            lambda: L.tria_score(h, ctypes.byref(k_off8), n, _p(raw), s), INVAL),
        "select raw not 16-byte aligned": (
            lambda: L.tria_select(h, _p(raw, 8), n, 100, 4, 16, _p(keep), None, s), INVAL),
        "select keep not 4-byte aligned": (
            lambda: L.tria_select(h, _p(raw), n, 100, 4, 16, _p(keep, 2), None, s), INVAL),
        "select agg not 4-byte aligned": (
            lambda: L.tria_select(h, _p(raw), n, 100, 4, 16, _p(keep), _p(out, 2), s), INVAL),
        "compact keep not 4-byte aligned": (
            lambda: L.tria_compact(h, ctypes.byref(good), n, _p(keep, 1), 10, s), INVAL),
        "compact v not 16-byte aligned": (
            lambda: L.tria_compact(h, ctypes.byref(v_off2), n, _p(keep), 10, s), INVAL),
        "attention q not 4-byte aligned": (
            lambda: L.tria_decode_attention(h, ctypes.byref(good), n, _p(q, 2), ctypes.c_float(0.1),
                                            _p(out), s), INVAL),
        "attention out not 4-byte aligned": (
            lambda: L.tria_decode_attention(h, ctypes.byref(good), n, _p(q), ctypes.c_float(0.1),
                                            _p(out, 1), s), INVAL),
        "evict n > cap": (lambda: L.tria_evict(h, ctypes.byref(good), n + 1, 100, 4, 16, s), INVAL),
        "evict n < 0": (lambda: L.tria_evict(h, ctypes.byref(good), -1, 100, 4, 16, s), INVAL),
        "evict budget < 0": (lambda: L.tria_evict(h, ctypes.byref(good), n, -1, 4, 16, s), INVAL),
        "evict sink < 0": (lambda: L.tria_evict(h, ctypes.byref(good), n, 100, -1, 16, s), INVAL),
        "evict window < 0": (lambda: L.tria_evict(h, ctypes.byref(good), n, 100, 4, -1, s), INVAL),
        "evict null k": (lambda: L.tria_evict(h, ctypes.byref(no_k), n, 100, 4, 16, s), INVAL),
        "evict null cache": (lambda: L.tria_evict(h, None, n, 100, 4, 16, s), INVAL),
        "score n > cap": (lambda: L.tria_score(h, ctypes.byref(good), n + 1, _p(raw), s), INVAL),
        "score null raw": (lambda: L.tria_score(h, ctypes.byref(good), n, None, s), INVAL),
        "select budget < 0": (lambda: L.tria_select(h, _p(raw), n, -1, 4, 16, _p(keep), None, s),
                              INVAL),
        "select sink < 0": (lambda: L.tria_select(h, _p(raw), n, 100, -1, 16, _p(keep), None, s),
                            INVAL),
        "select window < 0": (lambda: L.tria_select(h, _p(raw), n, 100, 4, -1, _p(keep), None, s),
                              INVAL),
        "select null keep_idx": (lambda: L.tria_select(h, _p(raw), n, 100, 4, 16, None, None, s),
                                 INVAL),
        "select null raw": (lambda: L.tria_select(h, None, n, 100, 4, 16, _p(keep), None, s),
                            INVAL),
        "select past the row limit": (lambda: L.tria_select(h, _p(raw), tria.TRIA_MAX_ROWS + 1,
                                                            100, 4, 16, _p(keep), None, s), UNSUP),
        "compact n > cap": (lambda: L.tria_compact(h, ctypes.byref(good), n + 1, _p(keep), 10, s),
                            INVAL),
        "compact kept > n": (lambda: L.tria_compact(h, ctypes.byref(good), n, _p(keep), n + 1, s),
                             INVAL),
        "compact kept < 0": (lambda: L.tria_compact(h, ctypes.byref(good), n, _p(keep), -1, s),
                             INVAL),
        "compact null keep_idx": (lambda: L.tria_compact(h, ctypes.byref(good), n, None, 10, s),
                                  INVAL),
        "attention n > cap": (lambda: L.tria_decode_attention(h, ctypes.byref(good), n + 1, _p(q),
                                                               ctypes.c_float(0.1), _p(out), s),
                              INVAL),
        "attention null q": (lambda: L.tria_decode_attention(h, ctypes.byref(good), n, None,
                                                              ctypes.c_float(0.1), _p(out), s),
                             INVAL),
        "noalloc n > cap": (lambda: L.tria_evict_noalloc(h, ctypes.byref(good), n + 1, 100, 4, 16,
                                                          s), INVAL),
        "noalloc budget < 0": (lambda: L.tria_evict_noalloc(h, ctypes.byref(good), n, -1, 4, 16,
                                                             s), INVAL),
        "compaction workgroups < 0": (lambda: L.tria_set_compaction_workgroups(h, -1), INVAL),
        "compaction mode 7": (lambda: L.tria_set_compaction(h, 7), INVAL),
        "keep mode 9": (lambda: L.tria_set_keep_mode(h, 9), INVAL),
    }
    for name, (call, code) in cases.items():
        pu.say("case %s" % name)
        assert call() == code, name
    torch.cuda.synchronize()
    assert torch.equal(k, k0) and torch.equal(v, v0) and torch.equal(pos, p0)
    assert not raw.any() and not keep.any() and not out.any()
    # the context still runs a pass afterwards
    assert tria.tria_evict(ctx, k, v, pos, n, 300, 4, 64) == 300
    tria.tria_device_status(ctx)
    ctx.close()


def test_paged_batch_rejects_bad_arguments():
    wl = synth.WORKLOADS["paged16_qwen3_8b_q8"]
    wl = dataclasses.replace(wl, L=2, Hkv=2, Hq=8)
    lens = [700, 300, 1200]
    pg = synth.gen_paged(wl.L, wl.Hkv, wl.hd, wl.k_type, wl.v_type, lens, 3, DEV)
    stats = synth.gen_stats(wl.L, wl.Hq, wl.hd, 3)
    ctx = pu.make_ctx(wl, stats)
    snap = {x: pg[x].clone() for x in ("k_pool", "v_pool", "pos_pool")}
    bt = pg["block_table"]
    L = tria.lib()
    h = ctx.handle
    s = _stream()
    pc = tria.PagedCache(_p(pg["k_pool"]), _p(pg["v_pool"]), _p(pg["pos_pool"]), pg["n_blocks"],
                         _p(bt), bt.shape[1])
    no_bt = tria.PagedCache(_p(pg["k_pool"]), _p(pg["v_pool"]), _p(pg["pos_pool"]),
                            pg["n_blocks"], None, bt.shape[1])
    k_off = tria.PagedCache(_p(pg["k_pool"], 4), _p(pg["v_pool"]), _p(pg["pos_pool"]),
                            pg["n_blocks"], _p(bt), bt.shape[1])
    bt_off = tria.PagedCache(_p(pg["k_pool"]), _p(pg["v_pool"]), _p(pg["pos_pool"]),
                             pg["n_blocks"], _p(bt, 2), bt.shape[1])

    def arr(vals):
        return (ctypes.c_int64 * len(vals))(*vals)

    kept = arr([0] * 70)
    big = tria.TRIA_MAX_SEQ + 1
    cases = {
        "n_seq > max": (lambda: L.tria_evict_paged_batch(h, ctypes.byref(pc), big, arr([100] * big),
                                                         arr([50] * big), 0, 16, kept, s), INVAL),
        "n_seq 0": (lambda: L.tria_evict_paged_batch(h, ctypes.byref(pc), 0, arr([1]), arr([1]), 0,
                                                     16, kept, s), INVAL),
        "budget < 0": (lambda: L.tria_evict_paged_batch(h, ctypes.byref(pc), 3, arr(lens),
                                                        arr([100, -1, 100]), 0, 16, kept, s), INVAL),
        "sink < 0": (lambda: L.tria_evict_paged_batch(h, ctypes.byref(pc), 3, arr(lens),
                                                      arr([100] * 3), -1, 16, kept, s), INVAL),
        "window < 0": (lambda: L.tria_evict_paged_batch(h, ctypes.byref(pc), 3, arr(lens),
                                                        arr([100] * 3), 0, -1, kept, s), INVAL),
        "n past the block table": (lambda: L.tria_evict_paged_batch(
            h, ctypes.byref(pc), 3, arr([700, 300, bt.shape[1] * 16 + 1]), arr([100] * 3), 0, 16,
            kept, s), INVAL),
        "n < 0": (lambda: L.tria_evict_paged_batch(h, ctypes.byref(pc), 3, arr([700, -5, 1200]),
                                                   arr([100] * 3), 0, 16, kept, s), INVAL),
        "null block table": (lambda: L.tria_evict_paged_batch(h, ctypes.byref(no_bt), 3, arr(lens),
                                                              arr([100] * 3), 0, 16, kept, s),
                             INVAL),
        "null kept_out": (lambda: L.tria_evict_paged_batch(h, ctypes.byref(pc), 3, arr(lens),
                                                           arr([100] * 3), 0, 16, None, s), INVAL),
        "k_pool not 16-byte aligned": (
            lambda: L.tria_evict_paged_batch(h, ctypes.byref(k_off), 3, arr(lens), arr([100] * 3),
                                             0, 16, kept, s), INVAL),
        "block table not 4-byte aligned": (
            lambda: L.tria_evict_paged_batch(h, ctypes.byref(bt_off), 3, arr(lens),
                                             arr([100] * 3), 0, 16, kept, s), INVAL),
    }
    for name, (call, code) in cases.items():
        pu.say("case paged %s" % name)
        assert call() == code, name
    torch.cuda.synchronize()
    for x in snap:
        assert torch.equal(pg[x], snap[x]), x
    # a valid batch still runs
    got = tria.tria_evict_paged_batch(ctx, pg["k_pool"], pg["v_pool"], pg["pos_pool"], bt, lens,
                                      [200, 300, 400], 0, 16)
    assert got == [200, 300, 400]
    tria.tria_device_status(ctx)
    ctx.close()


def test_calibration_rejects_misaligned_queries():
    """Query rows must start on their element size; a refused add leaves the
    accumulators and the token count as they were."""
    hd, Hq = 64, 4
    cal = tria.TriaCalib(1, Hq, hd)
    q32 = torch.randn(9, Hq * hd, dtype=torch.float32, device=DEV)
    q16 = q32.to(torch.float16)
    L = tria.lib()
    s = _stream()
    assert L.tria_calib_add(cal.handle, 0, _p(q32, 2), tria.TRIA_Q_F32, 8, Hq * hd, s) == INVAL
    assert L.tria_calib_add(cal.handle, 0, _p(q16, 1), tria.TRIA_Q_F16, 8, Hq * hd, s) == INVAL
    assert cal.tokens(0) == 0
    # element-aligned but not vector-aligned rows take the element-wise kernel
    assert L.tria_calib_add(cal.handle, 0, _p(q16, 2), tria.TRIA_Q_F16, 8, Hq * hd, s) == 0
    assert cal.tokens(0) == 8
    torch.cuda.synchronize()
    cal.close()



def test_calibration_add_layers_refusals():
    """Layers past the object, no layers, and overlapping layers are refused and
    leave every token count as it was."""
    hd, Hq, L, T = 64, 4, 3, 8
    cal = tria.TriaCalib(L, Hq, hd)
    q = torch.randn(L, T, Hq * hd, dtype=torch.float32, device=DEV)
    lib = tria.lib()
    s = _stream()
    row, lay = Hq * hd, T * Hq * hd
    assert lib.tria_calib_add_layers(cal.handle, 1, L, _p(q, 0), tria.TRIA_Q_F32, T, row, lay,
                                     s) == INVAL
    assert lib.tria_calib_add_layers(cal.handle, -1, 2, _p(q, 0), tria.TRIA_Q_F32, T, row, lay,
                                     s) == INVAL
    assert lib.tria_calib_add_layers(cal.handle, 0, 0, _p(q, 0), tria.TRIA_Q_F32, T, row, lay,
                                     s) == INVAL
    assert lib.tria_calib_add_layers(cal.handle, 0, 2, _p(q, 0), tria.TRIA_Q_F32, T, row,
                                     lay - 1, s) == INVAL
    assert lib.tria_calib_add_layers(cal.handle, 0, 2, _p(q, 2), tria.TRIA_Q_F32, T, row, lay,
                                     s) == INVAL
    # a row count whose span overflows 64 bits
    assert lib.tria_calib_add_layers(cal.handle, 0, 2, _p(q, 0), tria.TRIA_Q_F32, 1 << 62, row,
                                     lay, s) == INVAL
    assert [cal.tokens(l) for l in range(L)] == [0, 0, 0]
    # one layer ignores the layer stride
    assert lib.tria_calib_add_layers(cal.handle, 2, 1, _p(q, 0), tria.TRIA_Q_F32, T, row, 0,
                                     s) == 0
    assert lib.tria_calib_add_layers(cal.handle, 0, 2, _p(q, 0), tria.TRIA_Q_F32, T, row, lay,
                                     s) == 0
    assert [cal.tokens(l) for l in range(L)] == [T, T, T]
    torch.cuda.synchronize()
    cal.close()
