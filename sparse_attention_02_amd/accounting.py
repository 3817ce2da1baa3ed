"""Algorithmic work of the DSA path over a batch: FLOPs and HBM bytes.

The model is the library's own.  Row j of a request with n query rows and L
cached tokens (new rows included) sees v = L - n + 1 + j tokens; the indexer
scores all v of them and the attention runs over K = min(k, v) of them (all
v for the dense form).  The per-pair and per-token costs follow from the
operand shapes of include/dsa.h:
  - indexer: a row's 64 x 128 FP8 queries against one 128-byte key (plus its
    4-byte fp32 scale): 64 * 128 multiply-adds per (row, token);
  - attention: 128 heads score the 576-wide latent row (512 latent + 64
    rope) and accumulate its first 512 dims: 128 * (576 + 512) multiply-adds
    per (row, selected token); a cached latent row is 576 bf16;
  - a multiply-add counts 2 FLOPs.
Bytes are what the method must move, not implementation scratch (scores,
histograms, split partials): the key cache once per request, each row's
selected latent rows, the queries, the outputs, the selection and the
page-table entries.  The page "MTP and sparse attention: NSA and DSA"
prints per-query figures of the same quantities; the tests reproduce that
table from this model.
"""
from __future__ import annotations

import math

PAGE = 64          # DSA_PAGE_SIZE
IDX_HEADS = 64     # DSA_IDX_HEADS
IDX_DIM = 128      # DSA_IDX_DIM (one FP8 byte per dim)
MLA_HEADS = 128    # DSA_MLA_HEADS
MLA_DIM = 576      # DSA_MLA_DIM: 512 latent + 64 rope, bf16
MLA_DV = 512       # DSA_MLA_DV
TOPK = 2048


def indexer_pair_flops() -> int:
    """One (row, token) of the indexer: the row's 64 x 128 queries dotted with one key."""
    return 2 * IDX_HEADS * IDX_DIM


def attention_pair_flops(heads: int = MLA_HEADS, dim: int = MLA_DIM, dv: int = MLA_DV) -> int:
    """One (row, selected token) of the attention: 128 score dots over 576 dims,
    128 value accumulations over 512 dims."""
    return 2 * heads * (dim + dv)


def expanded_pair_flops(heads: int = MLA_HEADS, qk_dim: int = 128 + 64, v_dim: int = 128) -> int:
    """One (row, token) of attention in expanded (non-absorbed) multi-head
    form: per head a 192-dim score (128 up-projected + 64 rope) and a 128-dim
    value."""
    return 2 * heads * (qk_dim + v_dim)


def indexer_token_bytes() -> int:
    """A cached indexer key: 128 FP8 bytes plus its fp32 scale."""
    return IDX_DIM + 4


def latent_token_bytes(dim: int = MLA_DIM) -> int:
    """A cached latent row in bf16."""
    return 2 * dim


def row_visible(seqlens_k, n_q):
    """(request, visible tokens) of every query row, in row order."""
    for b, (L, nq) in enumerate(zip(seqlens_k, n_q)):
        L, nq = int(L), int(nq)
        for j in range(nq):
            yield b, max(L - nq + 1 + j, 0)


def batch_work(seqlens_k, n_q, k: int = TOPK, dense: bool = False) -> dict:
    """Algorithmic FLOPs and HBM bytes of one pass of the path over a batch.

    dense: the attention runs over every visible token and there is no
    indexer (the dense form the sparse path replaces).
    Returned: rows; indexer_bytes (key cache once per request, queries,
    scales, weights, page-table entries); attention_bytes (selected latent
    rows per row, queries, outputs, lse, the selection); bytes (their sum);
    cache_read_bytes (key cache + gathered latent rows only);
    attention_gather_bytes; indexer_flops; mla_flops; flops."""
    rows = 0
    idx_flops = mla_flops = 0
    gather = 0
    keys = 0      # key cache bytes read once per request
    ptab = 0      # page-table entries the scan reads
    for L in seqlens_k:
        if not dense:
            keys += int(L) * indexer_token_bytes()
            ptab += 4 * math.ceil(int(L) / PAGE)
    for _, v in row_visible(seqlens_k, n_q):
        rows += 1
        K = v if dense else min(k, v)
        if not dense:
            idx_flops += v * indexer_pair_flops()
        mla_flops += K * attention_pair_flops()
        gather += K * latent_token_bytes()
    idx_bytes = 0 if dense else keys + ptab + rows * (IDX_HEADS * IDX_DIM + 4 + IDX_HEADS * 4)
    sel_bytes = 0 if dense else rows * k * 4
    attn_bytes = gather + rows * (MLA_HEADS * MLA_DIM * 2 + MLA_HEADS * MLA_DV * 2 +
                                  MLA_HEADS * 4) + sel_bytes
    return {"rows": rows, "indexer_bytes": idx_bytes, "attention_bytes": attn_bytes,
            "bytes": idx_bytes + attn_bytes,
            "cache_read_bytes": keys + gather,
            "attention_gather_bytes": gather, "indexer_flops": idx_flops,
            "mla_flops": mla_flops, "flops": idx_flops + mla_flops}
