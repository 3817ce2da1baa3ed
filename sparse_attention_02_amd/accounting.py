"""Algorithmic work of the DSA decode path: FLOPs and HBM bytes.

Per-pair costs and per-token cache sizes follow the DSA accounting of
"MTP and sparse attention: NSA and DSA" (section "Sparse attention: NSA and
DSA", the listing that compares DSA with dense MLA, and its printed table):
  - absorbed MLA scores a (query, key) pair over the 512 + 64 latent for
    each of 128 heads and accumulates 512 value dims: 2 FLOPs per
    multiply-add on both products;
  - expanded multi-head attention (dense prefill) uses 128 + 64 query/key
    dims and 128 value dims per head;
  - the lightning indexer dots 64 heads of 128 dims per pair;
  - a cached token holds the bf16 latent (576 x 2 bytes) plus an FP8
    indexer key of 128 bytes and its 4-byte fp32 scale.
"""
from __future__ import annotations

import math

MLA_HEADS = 128
LATENT = 512
ROPE = 64
EXPANDED_HEAD_DIM = 128
IDX_HEADS = 64
IDX_DIM = 128
TOPK = 2048


def mla_pair_flops(heads: int = MLA_HEADS, latent: int = LATENT, rope: int = ROPE) -> int:
    """Absorbed MLA: scores over latent+rope dims, values over latent dims."""
    qk = heads * (latent + rope)
    pv = heads * latent
    return 2 * (qk + pv)


def expanded_pair_flops(heads: int = MLA_HEADS, head_dim: int = EXPANDED_HEAD_DIM,
                        rope: int = ROPE) -> int:
    return 2 * (heads * (head_dim + rope) + heads * head_dim)


def indexer_pair_flops(heads: int = IDX_HEADS, dim: int = IDX_DIM) -> int:
    return 2 * heads * dim


def latent_bytes_per_token(latent: int = LATENT, rope: int = ROPE) -> int:
    return 2 * (latent + rope)


def indexer_bytes_per_token(dim: int = IDX_DIM) -> int:
    return dim + 4  # FP8 key + fp32 scale


def one_query(L: int, k: int = TOPK) -> dict:
    """Per-layer work of one query token over a context of L tokens."""
    sel = min(L, k)
    return {
        "decode_flops_dense": L * mla_pair_flops(),
        "decode_flops_dsa": L * indexer_pair_flops() + sel * mla_pair_flops(),
        "decode_bytes_dense": L * latent_bytes_per_token(),
        "decode_bytes_dsa": L * indexer_bytes_per_token() + sel * latent_bytes_per_token(),
        # prefill of L tokens: half the L x L pairs are causal-visible
        "prefill_flops_dense": (L * L / 2) * expanded_pair_flops(),
        "prefill_flops_dsa": (L * L / 2) * indexer_pair_flops() + L * sel * mla_pair_flops(),
    }


def batch_work(seqlens_k, n_q, k: int = TOPK, dv: int = LATENT, dim: int = LATENT + ROPE) -> dict:
    """Algorithmic FLOPs and HBM bytes of one pass of the path over a batch.

    Bytes are what the method itself must move (no implementation scratch):
      indexer: every cached key (128 + 4 bytes) once per request, the FP8
        queries with their scale and 64 weights, the page-table entries;
      attention: each row's selected latent rows (1152 bytes each), its
        576-wide bf16 query, its 512-wide bf16 output per head, the fp32 lse
        per head and the k int32 selected positions.
    FLOPs count only causal-visible pairs.
    """
    idx_bytes = 0
    attn_bytes = 0
    idx_flops = 0
    mla_flops = 0
    gather = 0
    rows = 0
    for L, nq in zip(seqlens_k, n_q):
        L, nq = int(L), int(nq)
        idx_bytes += L * indexer_bytes_per_token() + 4 * math.ceil(L / 64)
        for j in range(nq):
            v = max(L - nq + 1 + j, 0)
            K = min(k, v)
            rows += 1
            idx_flops += v * indexer_pair_flops()
            mla_flops += K * mla_pair_flops(latent=dv, rope=dim - dv)
            attn_bytes += K * latent_bytes_per_token(dv, dim - dv)
            gather += K * latent_bytes_per_token(dv, dim - dv)
    idx_bytes += rows * (IDX_HEADS * IDX_DIM + 4 + IDX_HEADS * 4)
    attn_bytes += rows * (MLA_HEADS * dim * 2 + MLA_HEADS * dv * 2 + MLA_HEADS * 4 + k * 4)
    return {"rows": rows, "indexer_bytes": idx_bytes, "attention_bytes": attn_bytes,
            "bytes": idx_bytes + attn_bytes, "indexer_flops": idx_flops, "mla_flops": mla_flops,
            "attention_gather_bytes": gather}
