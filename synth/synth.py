"""Seeded synthetic inputs for the DSA decode path (shared by the GPU tests,
the bench and the CPU oracle).

This module makes input bytes only: it draws values, encodes them to FP8
(OCP e4m3fn) and bf16, lays them out in the paged caches and builds the
batch metadata.  It computes nothing the method computes.  The workload
shapes follow the DeepSeek Sparse Attention description in "MTP and sparse
attention: NSA and DSA" (DSA bullet: 64 indexer heads x 128 dims in FP8, a
128-dim indexer key per token, top-2048, absorbed MLA over a 512 + 64
latent) and the batch metadata of "[SGLang] NSA" (cache lengths include the
draft tokens; cumulative query offsets; a page table of 64-token pages).

Layouts (all C-contiguous):
  cu_seqlens_q  int32 [B+1]      query rows of request b: cu[b] .. cu[b+1]-1
  seqlens_k     int32 [B]        cached tokens of request b, new rows included
  page_table    int32 [B, max_pages]  physical page ids (64 tokens per page)
  q8            uint8 [T, 64, 128]   indexer queries, e4m3fn codes
  q_scale       f32   [T]            one scale per query token
  w             f32   [T, 64]        per-(token, head) weights
  k8            uint8 [pages, 64, 128]  indexer keys at physical slots
  k_scale       f32   [pages, 64]
  q             uint16 [T, 128, 576]    absorbed MLA queries, bf16 bits
  kv            uint16 [pages, 64, 576] latent cache (512 latent + 64 rope), bf16 bits
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

PAGE = 64
IDX_HEADS, IDX_DIM = 64, 128
MLA_HEADS, MLA_DIM, MLA_DV = 128, 576, 512
TOPK = 2048
SM_SCALE = 1.0 / math.sqrt(192.0)

# stream ids of the counter-based generator
S_IDX_Q, S_W, S_KEYS, S_PERM, S_LENS, S_NOISE = 1, 2, 3, 5, 9, 8
S_MLA_Q, S_KV = 6, 7  # + 16 * layer
S_HEAVY = 0x100  # + request
S_QN, S_QR, S_WUK, S_WUV = 0x201, 0x202, 0x203, 0x204  # expanded-form inputs


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (plain C, no GPU code)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        u64, i64, i32, dbl, vp, ci = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                      ctypes.c_double, ctypes.c_void_p, ctypes.c_int)
        L.synth_uniform.argtypes = [u64, u64, i64, vp]
        L.synth_normal.argtypes = [u64, u64, i64, vp]
        L.synth_permutation.argtypes = [u64, u64, i32, vp]
        L.synth_distinct.argtypes = [u64, u64, i32, i32, vp]
        L.synth_distinct.restype = ci
        L.synth_bf16_normal.argtypes = [u64, u64, i64, dbl, vp, ci]
        L.synth_indexer_q.argtypes = [u64, u64, i32, i32, i32, vp, vp, vp, ci]
        L.synth_indexer_keys.argtypes = [u64, u64, u64, dbl, i32, i32, i32, vp, vp, vp, i32, vp,
                                         vp, dbl, vp, vp, ci]
        L.synth_e4m3_encode.argtypes = [dbl]
        L.synth_e4m3_encode.restype = ctypes.c_uint8
        L.synth_bf16_encode.argtypes = [dbl]
        L.synth_bf16_encode.restype = ctypes.c_uint16
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def uniform(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_uniform(seed, stream, n, _p(out))
    return out


def normal(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_normal(seed, stream, n, _p(out))
    return out


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_permutation(seed, stream, n, _p(out))
    return out


def distinct(seed: int, stream: int, n: int, count: int) -> np.ndarray:
    out = np.empty(count, np.int32)
    if lib().synth_distinct(seed, stream, n, count, _p(out)) != 0:
        raise ValueError("count > n")
    return out


def e4m3_encode(x: float) -> int:
    return int(lib().synth_e4m3_encode(float(x)))


def bf16_normal(seed: int, stream: int, shape, scale: float, threads: int = 0) -> np.ndarray:
    out = np.empty(shape, np.uint16)
    lib().synth_bf16_normal(seed, stream, out.size, scale, _p(out), threads)
    return out


@dataclass
class Batch:
    """Batch metadata plus the inputs of one or more layers."""
    n_q: np.ndarray            # int32 [B]
    seqlens_k: np.ndarray      # int32 [B]
    cu_seqlens_q: np.ndarray   # int32 [B+1]
    page_table: np.ndarray     # int32 [B, max_pages]
    num_pages: int
    q8: np.ndarray
    q_scale: np.ndarray
    w: np.ndarray
    k8: list = field(default_factory=list)        # per layer
    k_scale: list = field(default_factory=list)
    q: list = field(default_factory=list)         # MLA queries per layer
    kv: list = field(default_factory=list)        # latent cache per layer
    heavy: list = field(default_factory=list)     # per request: heavy positions
    name: str = ""

    @property
    def B(self) -> int:
        return int(self.n_q.shape[0])

    @property
    def T(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_q(self) -> int:
        return int(self.n_q.max()) if self.B else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(self.seqlens_k.max()) if self.B else 0

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    def row_request(self) -> np.ndarray:
        return np.repeat(np.arange(self.B, dtype=np.int32), self.n_q)

    def visible(self) -> np.ndarray:
        """Tokens row t sees (the extend rule of "[SGLang] NSA", init_forward_metadata)."""
        out = np.empty(self.T, np.int64)
        for b in range(self.B):
            lo, hi = int(self.cu_seqlens_q[b]), int(self.cu_seqlens_q[b + 1])
            L, nq = int(self.seqlens_k[b]), hi - lo
            out[lo:hi] = L - nq + 1 + np.arange(nq)
        return np.maximum(out, 0)


def make_batch(n_q, L, *, seed: int, paging: str = "identity", heavy=64, layers: int = 1,
               key_noise: float = 0.1, mla_scale: float = 1.0 / math.sqrt(576.0),
               with_mla: bool = True, threads: int = 0, name: str = "",
               pool_extra_pages: int = 0) -> Batch:
    """Generate one batch.

    n_q, L: per-request query rows and cached lengths (lists or ints broadcast
    to a common B).  heavy: tokens per request that get the query-aligned
    offset; an int, or a float in (0, 1) for a fraction of L (rounded).
    paging: "identity" (request pages laid out in order) or "shuffled" (a
    uniformly random permutation of the whole page pool).
    """
    n_q = np.atleast_1d(np.asarray(n_q, np.int32))
    L = np.atleast_1d(np.asarray(L, np.int64))
    B = max(len(n_q), len(L))
    n_q = np.broadcast_to(n_q, (B,)).astype(np.int32)
    L = np.broadcast_to(L, (B,)).astype(np.int32)
    if np.any((L < n_q) & (L != 0)):
        # L = 0 is a padding request (no visible tokens); otherwise the
        # cache holds the request's new rows
        raise ValueError("each request's cache must hold its new rows")
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(n_q)
    T = int(cu[-1])
    pages_per = (L.astype(np.int64) + PAGE - 1) // PAGE
    num_pages = max(int(pages_per.sum()) + pool_extra_pages, 1)
    max_pages = max(int(pages_per.max()) if B else 1, 1)
    pool = (permutation(seed, S_PERM, num_pages) if paging == "shuffled"
            else np.arange(num_pages, dtype=np.int32))
    page_table = np.zeros((B, max_pages), np.int32)
    off = 0
    for b in range(B):
        n = int(pages_per[b])
        page_table[b, :n] = pool[off:off + n]
        off += n

    L_ = lib()
    q8 = np.empty((T, IDX_HEADS, IDX_DIM), np.uint8)
    q_scale = np.empty(T, np.float32)
    head_sum = np.empty((T, IDX_DIM), np.float64)
    if T:
        L_.synth_indexer_q(seed, S_IDX_Q, T, IDX_HEADS, IDX_DIM, _p(q8), _p(q_scale), _p(head_sum),
                           threads)
    w = (uniform(seed, S_W, T * IDX_HEADS) / 64.0).astype(np.float32).reshape(T, IDX_HEADS)

    # heavy tokens: offset 2.0 * sqrt(128) * u_b, u_b the unit direction of the
    # request's summed (rows, heads) pre-quantisation indexer query
    key_off = np.zeros(B, np.int64)
    key_off[1:] = np.cumsum(L.astype(np.int64))[:-1]
    total_keys = int(L.astype(np.int64).sum())
    heavy_mask = np.zeros(total_keys, np.uint8)
    dirs = np.zeros((B, IDX_DIM), np.float64)
    heavy_pos = []
    for b in range(B):
        cnt = heavy if isinstance(heavy, (int, np.integer)) else int(round(float(heavy) * int(L[b])))
        cnt = min(int(cnt), int(L[b]))
        pos = distinct(seed, S_HEAVY + b, int(L[b]), cnt) if cnt > 0 else np.zeros(0, np.int32)
        heavy_pos.append(np.sort(pos))
        heavy_mask[key_off[b] + pos.astype(np.int64)] = 1
        v = head_sum[cu[b]:cu[b + 1]].sum(axis=0)
        nrm = float(np.sqrt((v * v).sum()))
        dirs[b] = v / nrm if nrm > 0 else 0.0
    gain = 2.0 * math.sqrt(IDX_DIM)

    batch = Batch(n_q=n_q, seqlens_k=L.astype(np.int32), cu_seqlens_q=cu, page_table=page_table,
                  num_pages=num_pages, q8=q8, q_scale=q_scale, w=w, heavy=heavy_pos, name=name)
    for layer in range(layers):
        k8 = np.zeros((num_pages, PAGE, IDX_DIM), np.uint8)
        ks = np.ones((num_pages, PAGE), np.float32)
        if B:
            L_.synth_indexer_keys(seed, S_KEYS, S_NOISE + 16 * layer, key_noise if layer else 0.0,
                                  B, IDX_DIM, PAGE, _p(L), _p(key_off), _p(page_table), max_pages,
                                  _p(dirs), _p(heavy_mask), gain, _p(k8), _p(ks), threads)
        batch.k8.append(k8)
        batch.k_scale.append(ks)
        if with_mla:
            batch.q.append(bf16_normal(seed, S_MLA_Q + 16 * layer, (T, MLA_HEADS, MLA_DIM),
                                       mla_scale, threads))
            batch.kv.append(bf16_normal(seed, S_KV + 16 * layer, (num_pages, PAGE, MLA_DIM),
                                        mla_scale, threads))
    return batch


def mha_inputs(seed: int, T: int, q_std: float = 1.0, w_std: float = 1.0, threads: int = 0):
    """Inputs of the expanded multi-head form as bf16 bits: q_nope [T, 128,
    128] and q_rope [T, 128, 64] with standard deviation q_std, and the key
    and value up-projections w_uk, w_uv [128, 128, 512] with w_std."""
    qn = bf16_normal(seed, S_QN, (T, MLA_HEADS, 128), q_std, threads)
    qr = bf16_normal(seed, S_QR, (T, MLA_HEADS, 64), q_std, threads)
    wk = bf16_normal(seed, S_WUK, (MLA_HEADS, 128, 512), w_std, threads)
    wv = bf16_normal(seed, S_WUV, (MLA_HEADS, 128, 512), w_std, threads)
    return qn, qr, wk, wv


# The five workloads.  Seeds: 0 for the single-request case, the workload's
# number for the others.
WORKLOADS = {
    0: dict(name="decode-b1-q1-ctx8192", n_q=1, L=8192, paging="identity", heavy=64, seed=0),
    1: dict(name="decode-b32-mtp1-ctx32768", n_q=[2] * 32, L=32768, paging="shuffled", heavy=64,
            seed=1),
    2: dict(name="decode-b64-mtp1-ctx131072", n_q=[2] * 64, L=131072, paging="shuffled",
            heavy=0.01, seed=2),
    3: dict(name="prefill-4096-on-61440", n_q=4096, L=65536, paging="identity", heavy=64, seed=3),
    4: dict(name="mli-b48-mtp1-ctx10k-196k", n_q=[2] * 48, L=None, paging="shuffled", heavy=64,
            seed=4, layers=2),
}


def workload_lengths(idx: int) -> np.ndarray:
    w = WORKLOADS[idx]
    if w["L"] is not None:
        return np.broadcast_to(np.asarray(w["L"], np.int64), (len(np.atleast_1d(w["n_q"])),)).copy()
    # log-uniform in [10240, 196608], rounded
    u = uniform(w["seed"], S_LENS, len(w["n_q"]))
    lo, hi = math.log(10240.0), math.log(196608.0)
    return np.rint(np.exp(lo + u * (hi - lo))).astype(np.int64)


def make_workload(idx: int, *, threads: int = 0, mla_scale: float = 1.0 / math.sqrt(576.0),
                  with_mla: bool = True, layers: int | None = None) -> Batch:
    w = WORKLOADS[idx]
    return make_batch(w["n_q"], workload_lengths(idx), seed=w["seed"], paging=w["paging"],
                      heavy=w["heavy"], layers=layers if layers is not None else w.get("layers", 1),
                      mla_scale=mla_scale, with_mla=with_mla, threads=threads, name=w["name"])
