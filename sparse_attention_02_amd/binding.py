"""ctypes binding of libdsa.so (the C ABI declared in include/dsa.h).

Argument marshalling only: tensors are passed as device pointers
(torch.Tensor.data_ptr()) and streams as HIP stream handles.  Every step of
the path runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdsa.so")
# libdsa_checked.so: the same kernels compiled with device checks (bad page
# ids, index entries, NaN scores and metadata are recorded in a device word
# that dsa_device_check reports).  DSA_DEVICE_CHECKS=1 in the environment
# makes lib() load it instead of libdsa.so.
_LIB_CHECKED_PATH = os.path.join(_HERE, "libdsa_checked.so")
if os.environ.get("DSA_DEVICE_CHECKS", "0") not in ("", "0"):
    _LIB_PATH = _LIB_CHECKED_PATH

(DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP,
 DSA_ERR_DEVICE_CHECK) = range(6)
DSA_CHECK_PAGE_ID, DSA_CHECK_INDEX, DSA_CHECK_NAN_SCORE, DSA_CHECK_METADATA = 1, 2, 4, 8
DSA_OP_TOPK, DSA_OP_SPARSE_MLA, DSA_OP_DECODE_STEP, DSA_OP_DENSE_MLA = 1, 2, 3, 4
DSA_OP_MASKED_MHA = 5
DSA_MODE_FUSED, DSA_MODE_MLI = 0, 1
DSA_STAGE_INDEX_SCORE, DSA_STAGE_TOPK, DSA_STAGE_ATTENTION, DSA_NUM_STAGES = 0, 1, 2, 3
DSA_IDX_LOGICAL, DSA_IDX_PAGED, DSA_IDX_RAGGED = 0, 1, 2
PAGE_SIZE, IDX_HEADS, IDX_DIM, MLA_HEADS, MLA_DIM, MLA_DV, MAX_TOPK = 64, 64, 128, 128, 576, 512, 8192

EXPORTS = ["dsa_index_score", "dsa_topk", "dsa_sparse_mla_decode", "dsa_decode_step",
           "dsa_cache_append", "dsa_topk_transform", "dsa_sparse_mla_decode_paged",
           "dsa_decode_layers", "dsa_dense_mla_decode", "dsa_decode_step_noalloc",
           "dsa_masked_mha_prefill",
           "dsa_workspace_size", "dsa_default_splits", "dsa_status_string", "dsa_last_error",
           "dsa_device_check", "dsa_device_checks_enabled",
           # measurement kernels (include/dsa_bench.h)
           "dsa_bench_stream_read", "dsa_bench_key_stream_read"]


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class dsa_batch_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_tokens", ctypes.c_int32),
                ("max_q", ctypes.c_int32), ("max_seqlen_k", ctypes.c_int32),
                ("max_pages_per_req", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("cu_seqlens_q", ctypes.c_void_p), ("seqlens_k", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p)]


class dsa_indexer_inputs_t(ctypes.Structure):
    _fields_ = [("q8", ctypes.c_void_p), ("q_scale", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("k8_cache", ctypes.c_void_p), ("k_scale", ctypes.c_void_p)]


class dsa_mla_inputs_t(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("kv_cache", ctypes.c_void_p),
                ("sm_scale", ctypes.c_float)]


class dsa_layer_t(ctypes.Structure):
    _fields_ = [("ix", dsa_indexer_inputs_t), ("mla", dsa_mla_inputs_t),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


class dsa_step_opts_t(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("n_split", ctypes.c_int32),
                ("attend_idx", ctypes.c_void_p), ("stage_events", ctypes.c_void_p)]


_lib = None
_loaded = {}


def lib() -> ctypes.CDLL:
    """Load libdsa.so (or libdsa_checked.so, see above); raises if it has not
    been built."""
    global _lib
    if _lib is None:
        _lib = _load(_LIB_PATH)
    return _lib


@contextlib.contextmanager
def checked():
    """Within the block every call goes to libdsa_checked.so."""
    global _lib
    prev = lib()
    _lib = _load(_LIB_CHECKED_PATH)
    try:
        yield _lib
    finally:
        _lib = prev


def _load(path: str) -> ctypes.CDLL:
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                             ctypes.c_float)
    bp = ctypes.POINTER(dsa_batch_t)
    L.dsa_index_score.argtypes = [bp, vp, vp, vp, vp, vp, vp, i64, vp]
    L.dsa_topk.argtypes = [bp, vp, i64, i32, vp, vp, sz, vp]
    L.dsa_sparse_mla_decode.argtypes = [bp, vp, vp, vp, i32, f32, vp, vp, i32, vp, sz, vp]
    L.dsa_decode_step.argtypes = [bp, ctypes.POINTER(dsa_indexer_inputs_t),
                                  ctypes.POINTER(dsa_mla_inputs_t), i32,
                                  ctypes.POINTER(dsa_step_opts_t), vp, vp, vp, vp, sz, vp, vp]
    L.dsa_cache_append.argtypes = [bp, vp, vp, vp, vp, vp, vp]
    L.dsa_topk_transform.argtypes = [bp, vp, i64, i32, i32, vp, vp, vp, sz, vp]
    L.dsa_sparse_mla_decode_paged.argtypes = [bp, vp, vp, vp, i32, f32, vp, vp, i32, vp, sz, vp]
    L.dsa_decode_layers.argtypes = [bp, i32, ctypes.POINTER(dsa_layer_t), i32, i32, i32, i32,
                                    vp, vp, sz, vp, vp]
    L.dsa_dense_mla_decode.argtypes = [bp, vp, vp, f32, vp, vp, i32, vp, sz, vp]
    L.dsa_decode_step_noalloc.argtypes = [bp, ctypes.POINTER(dsa_indexer_inputs_t),
                                          ctypes.POINTER(dsa_mla_inputs_t), i32,
                                          ctypes.POINTER(dsa_step_opts_t), vp, vp, vp, vp]
    L.dsa_masked_mha_prefill.argtypes = [bp, vp, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp]
    for f in ("dsa_index_score", "dsa_topk", "dsa_sparse_mla_decode", "dsa_decode_step",
              "dsa_cache_append", "dsa_topk_transform", "dsa_sparse_mla_decode_paged",
              "dsa_decode_layers", "dsa_dense_mla_decode", "dsa_decode_step_noalloc",
              "dsa_masked_mha_prefill"):
        getattr(L, f).restype = ctypes.c_int
    L.dsa_workspace_size.argtypes = [ctypes.c_int, bp, i32, i32]
    L.dsa_workspace_size.restype = sz
    L.dsa_default_splits.argtypes = [bp, i32]
    L.dsa_default_splits.restype = i32
    L.dsa_status_string.argtypes = [ctypes.c_int]
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_last_error.argtypes = []
    L.dsa_last_error.restype = ctypes.c_char_p
    L.dsa_device_check.argtypes = [ctypes.POINTER(ctypes.c_uint32), vp]
    L.dsa_device_check.restype = ctypes.c_int
    L.dsa_device_checks_enabled.argtypes = []
    L.dsa_device_checks_enabled.restype = i32
    L.dsa_bench_stream_read.argtypes = [vp, sz, vp, vp]
    L.dsa_bench_stream_read.restype = ctypes.c_int
    L.dsa_bench_key_stream_read.argtypes = [vp, i32, vp, i32, i32, vp, i32, vp, vp]
    L.dsa_bench_key_stream_read.restype = ctypes.c_int
    _loaded[path] = L
    return L


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc: int):
    if rc != DSA_OK:
        msg = lib().dsa_last_error().decode() or lib().dsa_status_string(rc).decode()
        raise DsaError(rc, msg)


class Batch:
    """Batch metadata on the device plus its host scalars (dsa_batch_t)."""

    def __init__(self, cu_seqlens_q: torch.Tensor, seqlens_k: torch.Tensor,
                 page_table: torch.Tensor, num_pages: int, max_q: int, max_seqlen_k: int):
        self.cu_seqlens_q = cu_seqlens_q
        self.seqlens_k = seqlens_k
        self.page_table = page_table
        B = int(seqlens_k.shape[0])
        T = int(cu_seqlens_q[-1].item()) if B else 0
        self.c = dsa_batch_t(B, T, int(max_q), int(max_seqlen_k),
                             int(page_table.shape[1]) if page_table.dim() == 2 else 0,
                             int(num_pages), _ptr(cu_seqlens_q), _ptr(seqlens_k),
                             _ptr(page_table))

    @property
    def T(self) -> int:
        return int(self.c.num_tokens)

    def ref(self):
        return ctypes.byref(self.c)


def dsa_device_check(stream=None) -> int:
    """Reads and clears the device check word (synchronising the stream);
    returns its DSA_CHECK_* flags (0 in normal builds)."""
    flags = ctypes.c_uint32(0)
    rc = lib().dsa_device_check(ctypes.byref(flags), _stream(stream))
    if rc not in (DSA_OK, DSA_ERR_DEVICE_CHECK):
        _check(rc)
    return int(flags.value)


def dsa_bench_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Measurement kernel: reads all of src once (include/dsa_bench.h)."""
    _check(lib().dsa_bench_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                       _stream(stream)))


def dsa_bench_key_stream_read(batch: "Batch", k8_cache, sink, stream=None):
    """Measurement kernel: reads the batch's indexer-key pages the way the
    scan does and nothing else (include/dsa_bench.h)."""
    c = batch.c
    _check(lib().dsa_bench_key_stream_read(_ptr(k8_cache), c.num_pages, c.page_table, c.batch,
                                           c.max_pages_per_req, c.seqlens_k, c.max_seqlen_k,
                                           _ptr(sink), _stream(stream)))


def dsa_device_checks_enabled() -> bool:
    return bool(lib().dsa_device_checks_enabled())


def dsa_workspace_size(op: int, batch: Batch, k: int, n_split: int = 0) -> int:
    return int(lib().dsa_workspace_size(op, batch.ref(), k, n_split))


def dsa_default_splits(batch: Batch, k: int) -> int:
    return int(lib().dsa_default_splits(batch.ref(), k))


def dsa_index_score(batch: Batch, q8, q_scale, w, k8_cache, k_scale, scores, ld: int,
                    stream=None):
    _check(lib().dsa_index_score(batch.ref(), _ptr(q8), _ptr(q_scale), _ptr(w), _ptr(k8_cache),
                                 _ptr(k_scale), _ptr(scores), int(ld), _stream(stream)))


def dsa_cache_append(batch: Batch, k_new, kv_new, k8_cache, k_scale, kv_cache, stream=None):
    _check(lib().dsa_cache_append(batch.ref(), _ptr(k_new), _ptr(kv_new), _ptr(k8_cache),
                                  _ptr(k_scale), _ptr(kv_cache), _stream(stream)))


def dsa_topk(batch: Batch, scores, ld: int, k: int, idx, ws, ws_bytes: int, stream=None):
    _check(lib().dsa_topk(batch.ref(), _ptr(scores), int(ld), int(k), _ptr(idx), _ptr(ws),
                          int(ws_bytes), _stream(stream)))


def dsa_topk_transform(batch: Batch, scores, ld: int, k: int, space: int, kv_offsets, idx, ws,
                       ws_bytes: int, stream=None):
    _check(lib().dsa_topk_transform(batch.ref(), _ptr(scores), int(ld), int(k), int(space),
                                    _ptr(kv_offsets), _ptr(idx), _ptr(ws), int(ws_bytes),
                                    _stream(stream)))


def dsa_sparse_mla_decode_paged(batch: Batch, q, kv_cache, slots, k: int, sm_scale: float, out,
                                lse, n_split: int, ws, ws_bytes: int, stream=None):
    _check(lib().dsa_sparse_mla_decode_paged(batch.ref(), _ptr(q), _ptr(kv_cache), _ptr(slots),
                                             int(k), float(sm_scale), _ptr(out), _ptr(lse),
                                             int(n_split), _ptr(ws), int(ws_bytes),
                                             _stream(stream)))


def dsa_masked_mha_prefill(batch: Batch, q_nope, q_rope, w_uk, w_uv, kv_cache, idx, k: int,
                           sm_scale: float, out, lse, ws, ws_bytes: int, stream=None):
    _check(lib().dsa_masked_mha_prefill(batch.ref(), _ptr(q_nope), _ptr(q_rope), _ptr(w_uk),
                                        _ptr(w_uv), _ptr(kv_cache), _ptr(idx), int(k),
                                        float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws),
                                        int(ws_bytes), _stream(stream)))


def dsa_dense_mla_decode(batch: Batch, q, kv_cache, sm_scale: float, out, lse, n_split: int, ws,
                         ws_bytes: int, stream=None):
    _check(lib().dsa_dense_mla_decode(batch.ref(), _ptr(q), _ptr(kv_cache), float(sm_scale),
                                      _ptr(out), _ptr(lse), int(n_split), _ptr(ws), int(ws_bytes),
                                      _stream(stream)))


def dsa_sparse_mla_decode(batch: Batch, q, kv_cache, idx, k: int, sm_scale: float, out, lse,
                          n_split: int, ws, ws_bytes: int, stream=None):
    _check(lib().dsa_sparse_mla_decode(batch.ref(), _ptr(q), _ptr(kv_cache), _ptr(idx), int(k),
                                       float(sm_scale), _ptr(out), _ptr(lse), int(n_split),
                                       _ptr(ws), int(ws_bytes), _stream(stream)))


def dsa_decode_step(batch: Batch, ix: dict, mla: dict, k: int, mode: int, n_split: int,
                    attend_idx, idx_out, out, lse, ws, ws_bytes: int, stream_main=None,
                    stream_aux=None, stage_events=None):
    """ix: q8, q_scale, w, k8_cache, k_scale; mla: q, kv_cache, sm_scale.
    stage_events: None or 2 * DSA_NUM_STAGES raw hipEvent_t handles (ints)."""
    evs = None
    if stage_events is not None:
        if len(stage_events) != 2 * DSA_NUM_STAGES or not all(stage_events):
            raise ValueError(f"stage_events needs {2 * DSA_NUM_STAGES} event handles")
        evs = (ctypes.c_void_p * len(stage_events))(*stage_events)
    ixs = dsa_indexer_inputs_t(_ptr(ix["q8"]), _ptr(ix["q_scale"]), _ptr(ix["w"]),
                               _ptr(ix["k8_cache"]), _ptr(ix["k_scale"]))
    ms = dsa_mla_inputs_t(_ptr(mla["q"]), _ptr(mla["kv_cache"]), float(mla["sm_scale"]))
    opts = dsa_step_opts_t(int(mode), int(n_split), _ptr(attend_idx),
                           None if evs is None else ctypes.cast(evs, ctypes.c_void_p))
    aux = None if stream_aux is None else _stream(stream_aux)
    _check(lib().dsa_decode_step(batch.ref(), ctypes.byref(ixs), ctypes.byref(ms), int(k),
                                 ctypes.byref(opts), _ptr(idx_out), _ptr(out), _ptr(lse),
                                 _ptr(ws), int(ws_bytes), _stream(stream_main), aux))


def dsa_decode_step_noalloc(batch: Batch, ix: dict, mla: dict, k: int, n_split: int, idx_out, out,
                            lse, stream=None, stage_events=None):
    """dsa_decode_step (FUSED) in the library's static scratch: no workspace."""
    evs = None
    if stage_events is not None:
        if len(stage_events) != 2 * DSA_NUM_STAGES or not all(stage_events):
            raise ValueError(f"stage_events needs {2 * DSA_NUM_STAGES} event handles")
        evs = (ctypes.c_void_p * len(stage_events))(*stage_events)
    ixs = dsa_indexer_inputs_t(_ptr(ix["q8"]), _ptr(ix["q_scale"]), _ptr(ix["w"]),
                               _ptr(ix["k8_cache"]), _ptr(ix["k_scale"]))
    ms = dsa_mla_inputs_t(_ptr(mla["q"]), _ptr(mla["kv_cache"]), float(mla["sm_scale"]))
    opts = dsa_step_opts_t(DSA_MODE_FUSED, int(n_split), None,
                           None if evs is None else ctypes.cast(evs, ctypes.c_void_p))
    _check(lib().dsa_decode_step_noalloc(batch.ref(), ctypes.byref(ixs), ctypes.byref(ms), int(k),
                                         ctypes.byref(opts), _ptr(idx_out), _ptr(out), _ptr(lse),
                                         _stream(stream)))


def dsa_decode_layers(batch: Batch, layers: list, k: int, retention: int, mli: int, n_split: int,
                      sel, ws, ws_bytes: int, stream_main=None, stream_aux=None):
    """layers: dicts with ix (q8, q_scale, w, k8_cache, k_scale; may be None on
    layers without an indexer), mla (q, kv_cache, sm_scale), out and lse."""
    arr = (dsa_layer_t * len(layers))()
    for i, ly in enumerate(layers):
        ix = ly.get("ix") or {}
        arr[i].ix = dsa_indexer_inputs_t(_ptr(ix.get("q8")), _ptr(ix.get("q_scale")),
                                         _ptr(ix.get("w")), _ptr(ix.get("k8_cache")),
                                         _ptr(ix.get("k_scale")))
        mla = ly["mla"]
        arr[i].mla = dsa_mla_inputs_t(_ptr(mla["q"]), _ptr(mla["kv_cache"]), float(mla["sm_scale"]))
        arr[i].out = _ptr(ly["out"])
        arr[i].lse = _ptr(ly.get("lse"))
    aux = None if stream_aux is None else _stream(stream_aux)
    _check(lib().dsa_decode_layers(batch.ref(), len(layers), arr, int(k), int(retention), int(mli),
                                   int(n_split), _ptr(sel), _ptr(ws), int(ws_bytes),
                                   _stream(stream_main), aux))
