"""Python access to the float64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
baseline use it; the GPU path never imports it.  Every function here only
marshals arguments; the arithmetic is in oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# The selection contract: positions whose float64 score lies within this
# relative distance of the k-th score may differ between implementations.
TIE_BAND = 1e-3


def build(force: bool = False) -> str:
    """Compile liboracle.so (plain C, -O2 without fast-math so sums keep their order)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
                               "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Batch(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("cu_q", ctypes.c_void_p), ("seqlens_k", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
                ("page_size", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i32, i64, dbl, ci = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double,
                                 ctypes.c_int)
        bp = ctypes.POINTER(_Batch)
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = dbl
        L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_decode.restype = dbl
        L.oracle_row_visible.argtypes = [bp, i32]
        L.oracle_row_visible.restype = i64
        L.oracle_index_score.argtypes = [bp, i64, i32, i32, vp, vp, vp, vp, vp, vp, i32, vp, i64, ci]
        L.oracle_masked_mha.argtypes = [bp, i64, i32, vp, vp, vp, vp, vp, vp, i32, dbl, vp, i32,
                                        vp, vp, ci]
        L.oracle_topk.argtypes = [vp, i64, i32, dbl, vp, vp, vp]
        L.oracle_topk.restype = i32
        L.oracle_topk_rows.argtypes = [vp, i64, vp, i32, i32, dbl, vp, vp, i64, vp, vp, ci]
        L.oracle_sparse_mla.argtypes = [bp, i64, i32, i32, i32, vp, vp, vp, i32, dbl, vp, i32, vp, vp,
                                        ci]
        L.oracle_dense_mla.argtypes = [bp, i64, i32, i32, i32, vp, vp, dbl, vp, i32, vp, vp, ci]
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_cache_append.argtypes = [bp, i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_transform_index.argtypes = [bp, i32, i32, vp, vp, vp, i32, i32, vp]
        L.oracle_layer_schedule.argtypes = [i32, i32, i32, vp, vp]
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


class Meta:
    """Batch metadata kept alive for the C struct."""

    def __init__(self, cu_seqlens_q, seqlens_k, page_table, page_size=64):
        self.cu = np.ascontiguousarray(cu_seqlens_q, np.int32)
        self.L = np.ascontiguousarray(seqlens_k, np.int32)
        self.pt = np.ascontiguousarray(page_table, np.int32)
        if self.pt.ndim == 1:
            self.pt = self.pt.reshape(len(self.L), -1)
        self.s = _Batch(len(self.L), _p(self.cu).value, _p(self.L).value, _p(self.pt).value,
                        self.pt.shape[1] if self.pt.ndim == 2 else 0, page_size)

    @classmethod
    def of(cls, batch):
        return cls(batch.cu_seqlens_q, batch.seqlens_k, batch.page_table)

    def ref(self):
        return ctypes.byref(self.s)

    def visible(self, t: int) -> int:
        return int(lib().oracle_row_visible(self.ref(), int(t)))


def e4m3_decode(code: int) -> float:
    return float(lib().oracle_e4m3_decode(int(code)))


def bf16_decode(bits: int) -> float:
    return float(lib().oracle_bf16_decode(int(bits)))


def e4m3_encode(x: float) -> int:
    """OCP e4m3fn code of the float32 value x (nearest, ties to even, saturating)."""
    return int(lib().oracle_e4m3_encode(float(x)))


def cache_append(meta: Meta, num_pages: int, k_new, kv_new, k8, k_scale, kv):
    """Writes the batch's new tokens into copies of the caches and returns them:
    k_new uint16 (bf16) [T, 128], kv_new uint16 [T, 576]; k8 uint8 [pages, 64, 128],
    k_scale float32 [pages, 64], kv uint16 [pages, 64, 576]."""
    k_new = np.ascontiguousarray(k_new, np.uint16)
    kv_new = np.ascontiguousarray(kv_new, np.uint16)
    k8 = np.array(k8, np.uint8, copy=True, order="C")
    k_scale = np.array(k_scale, np.float32, copy=True, order="C")
    kv = np.array(kv, np.uint16, copy=True, order="C")
    lib().oracle_cache_append(meta.ref(), int(num_pages), k_new.shape[-1], kv_new.shape[-1],
                              _p(k_new), _p(kv_new), _p(k8), _p(k_scale), _p(kv))
    return k8, k_scale, kv


def index_score(meta: Meta, q8, q_scale, w, k8, k_scale, rows, ld=None, threads=0):
    """float64 scores [len(rows), ld]; entries s >= v_t are NaN.  The pool
    holds k8.shape[0] pages; positions on a page id outside it score -inf."""
    q8 = np.ascontiguousarray(q8, np.uint8)
    H, D = q8.shape[1], q8.shape[2]
    rows = np.ascontiguousarray(rows, np.int32)
    if ld is None:
        ld = max([meta.visible(t) for t in rows] + [1])
    out = np.full((len(rows), ld), np.nan, np.float64)
    qs = np.ascontiguousarray(q_scale, np.float32)
    ww = np.ascontiguousarray(w, np.float32)
    kk = np.ascontiguousarray(k8, np.uint8)
    ks = np.ascontiguousarray(k_scale, np.float32)
    lib().oracle_index_score(meta.ref(), kk.shape[0], H, D, _p(q8), _p(qs), _p(ww), _p(kk), _p(ks),
                             _p(rows), len(rows), _p(out), ld, threads)
    return out


def topk(scores_rows, visible, k, band=TIE_BAND, threads=0):
    """Stable top-k of each row (ties to the lower position).

    Returns (sel [n, k] int32 with -1 padding, flags [n, ld] uint8, kth [n], K [n]).
    """
    sc = np.ascontiguousarray(scores_rows, np.float64)
    n, ld = sc.shape
    v = np.ascontiguousarray(visible, np.int64)
    sel = np.empty((n, k), np.int32)
    flags = np.zeros((n, ld), np.uint8)
    kth = np.empty(n, np.float64)
    K = np.empty(n, np.int32)
    lib().oracle_topk_rows(_p(sc), ld, _p(v), n, k, band, _p(sel), _p(flags), ld, _p(kth), _p(K),
                           threads)
    return sel, flags, kth, K


def sparse_mla(meta: Meta, q, kv, idx, rows, sm_scale, dv=512, threads=0):
    """float64 (out [n, H, dv], lse [n, H]) over the positions idx[i] (-1 = none);
    positions on a page id outside the kv.shape[0] pages of the pool are left out."""
    q = np.ascontiguousarray(q, np.uint16)
    kv = np.ascontiguousarray(kv, np.uint16)
    H, D = q.shape[1], q.shape[2]
    idx = np.ascontiguousarray(idx, np.int32)
    rows = np.ascontiguousarray(rows, np.int32)
    out = np.empty((len(rows), H, dv), np.float64)
    lse = np.empty((len(rows), H), np.float64)
    lib().oracle_sparse_mla(meta.ref(), kv.shape[0], H, D, dv, _p(q), _p(kv), _p(idx),
                            idx.shape[1], float(sm_scale), _p(rows), len(rows), _p(out), _p(lse),
                            threads)
    return out, lse


def dense_mla(meta: Meta, q, kv, rows, sm_scale, dv=512, threads=0):
    q = np.ascontiguousarray(q, np.uint16)
    kv = np.ascontiguousarray(kv, np.uint16)
    H, D = q.shape[1], q.shape[2]
    rows = np.ascontiguousarray(rows, np.int32)
    out = np.empty((len(rows), H, dv), np.float64)
    lse = np.empty((len(rows), H), np.float64)
    lib().oracle_dense_mla(meta.ref(), kv.shape[0], H, D, dv, _p(q), _p(kv), float(sm_scale),
                           _p(rows), len(rows), _p(out), _p(lse), threads)
    return out, lse


def masked_mha(meta: Meta, q_nope, q_rope, w_uk, w_uv, kv, idx, rows, sm_scale, threads=0):
    """float64 (out [n, H, 128], lse [n, H]) of the expanded multi-head form
    over the positions idx[i] (-1 = none), or every visible position when idx
    is None; positions on a page id outside the pool are left out."""
    qn = np.ascontiguousarray(q_nope, np.uint16)
    qr = np.ascontiguousarray(q_rope, np.uint16)
    wk = np.ascontiguousarray(w_uk, np.uint16)
    wv = np.ascontiguousarray(w_uv, np.uint16)
    kv = np.ascontiguousarray(kv, np.uint16)
    H = qn.shape[1]
    rows = np.ascontiguousarray(rows, np.int32)
    k = 0
    ip = None
    if idx is not None:
        idx = np.ascontiguousarray(idx, np.int32)
        k = idx.shape[1]
        ip = _p(idx)
    out = np.empty((len(rows), H, 128), np.float64)
    lse = np.empty((len(rows), H), np.float64)
    lib().oracle_masked_mha(meta.ref(), kv.shape[0], H, _p(qn), _p(qr), _p(wk), _p(wv), _p(kv),
                            ip, k, float(sm_scale), _p(rows), len(rows), _p(out), _p(lse), threads)
    return out, lse


def selection_check(gpu_idx, sel, flags, K):
    """The selection contract for one row: same count, and identical
    membership for every position outside the flagged tie band.

    Returns a list of problems (empty when the row passes)."""
    g = np.asarray(gpu_idx)
    probs = []
    if np.any(g < -1):
        probs.append("entries below -1 (neither a position nor padding)")
    g = g[g >= 0]
    if len(g) != int(K):
        probs.append(f"count {len(g)} != {int(K)}")
    if len(np.unique(g)) != len(g):
        probs.append("duplicate positions")
    o = np.asarray(sel)[: int(K)]
    gs, os_ = set(g.tolist()), set(o.tolist())
    for s in gs.symmetric_difference(os_):
        if s < 0 or s >= len(flags) or not flags[s]:
            probs.append(f"position {s} {'extra' if s in gs else 'missing'} outside tie band")
            if len(probs) > 8:
                break
    return probs


def transform_index(meta: Meta, num_pages: int, space: int, idx, rows, kv_offsets=None):
    """Selections idx int32 [len(rows), k] (logical positions, -1 padding) in
    index space 0 (logical), 1 (physical slot) or 2 (kv_offsets[b] + s)."""
    idx = np.ascontiguousarray(idx, np.int32)
    rows = np.ascontiguousarray(rows, np.int32)
    off = np.ascontiguousarray(kv_offsets if kv_offsets is not None else np.zeros(1), np.int32)
    out = np.empty_like(idx)
    lib().oracle_transform_index(meta.ref(), int(num_pages), int(space), _p(off), _p(idx),
                                 _p(rows), len(rows), idx.shape[1], _p(out))
    return out


def layer_schedule(n_layers: int, retention: int, mli: bool):
    """(produces, attends) per layer: the selection a layer makes (-1: none)
    and the selection its attention reads, numbered in the order made."""
    produces = np.empty(n_layers, np.int32)
    attends = np.empty(n_layers, np.int32)
    lib().oracle_layer_schedule(int(n_layers), int(retention), int(bool(mli)), _p(produces),
                                _p(attends))
    return produces, attends
