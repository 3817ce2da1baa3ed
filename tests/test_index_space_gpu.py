"""Top-k fused with the index transform (dsa_topk_transform) and attention
over physical slots (dsa_sparse_mla_decode_paged), through the C ABI.
Index work is compared exactly: the transformed selection must equal the
oracle's transform of the GPU's own logical selection entry by entry (and
that selection passes the usual check against the oracle's), and attention
over the slots must equal attention over the positions bit for bit (the
kernels differ only in how the slot table is filled) and the oracle within
the attention bounds."""
import numpy as np
import pytest
import torch

from gpu_common import (K, O, bf16_to_f64, check_attention, check_selection, dsa, index_scores,
                        oracle_rows, sparse_mla, synth, sync, to_device, topk)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def _transform(d, scores, ld, space, offsets=None, k=K):
    ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_TOPK, d.meta, k)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    idx = torch.empty((d.meta.T, k), dtype=torch.int32, device="cuda")
    off = None if offsets is None else torch.from_numpy(offsets).cuda()
    dsa.dsa_topk_transform(d.meta, scores, ld, k, space, off, idx, ws, ws_bytes)
    return idx


def _paged_mla(d, slots, k=K, n_split=0):
    T = d.meta.T
    ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_SPARSE_MLA, d.meta, k, n_split)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, 128), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_mla_decode_paged(d.meta, d.q[0], d.kv[0], slots, k, synth.SM_SCALE, out, lse,
                                    n_split, ws, ws_bytes)
    return out, lse


def _check_spaces(b, d, k=K, rows=None):
    scores, ld = index_scores(d)
    logical = topk(d, scores, ld, k)
    same = _transform(d, scores, ld, dsa.DSA_IDX_LOGICAL, k=k)
    paged = _transform(d, scores, ld, dsa.DSA_IDX_PAGED, k=k)
    starts = np.concatenate([[0], np.cumsum(b.seqlens_k)[:-1]]).astype(np.int32)
    ragged = _transform(d, scores, ld, dsa.DSA_IDX_RAGGED, starts, k=k)
    sync()
    rows = list(range(b.T)) if rows is None else rows
    g = logical.cpu().numpy()
    assert np.array_equal(same.cpu().numpy(), g)
    meta = O.Meta.of(b)
    sub = g[rows]
    assert np.array_equal(paged.cpu().numpy()[rows],
                          O.transform_index(meta, b.num_pages, 1, sub, rows))
    assert np.array_equal(ragged.cpu().numpy()[rows],
                          O.transform_index(meta, b.num_pages, 2, sub, rows, starts))
    _, vis, sc, sel, flags, Ks = oracle_rows(b, rows)
    check_selection(sub, sel, flags, Ks)
    return logical, paged, rows, meta


SMALL = [
    dict(n_q=[1], L=[63]),
    dict(n_q=[2, 1], L=[64, 65]),
    dict(n_q=[3, 1, 2], L=[2047, 2048, 2049]),
    dict(n_q=[2, 2, 1, 5], L=[130, 5000, 0, 4100]),
    dict(n_q=[1, 2], L=[9000, 20000]),
]


@pytest.mark.parametrize("ci", range(len(SMALL)))
def test_topk_transform_and_paged_attention_small(ci):
    case = SMALL[ci]
    b = synth.make_batch(case["n_q"], case["L"], seed=700 + ci, paging="shuffled", heavy=16,
                         pool_extra_pages=3)
    d = to_device(b)
    logical, paged, rows, meta = _check_spaces(b, d)
    out_l, lse_l = sparse_mla(d, logical)
    out_p, lse_p = _paged_mla(d, paged)
    sync()
    assert torch.equal(out_p, out_l) and torch.equal(lse_p, lse_l)
    ref, ref_lse = O.sparse_mla(meta, b.q[0], b.kv[0], logical.cpu().numpy(), rows,
                                synth.SM_SCALE)
    check_attention(bf16_to_f64(out_p), ref, lse_p.cpu().numpy(), ref_lse)


@pytest.mark.device_check_flags
def test_paged_attention_skips_out_of_range_slots():
    b = synth.make_batch([2, 1], [3000, 5000], seed=71, paging="shuffled", heavy=16,
                         pool_extra_pages=3)
    d = to_device(b)
    scores, ld = index_scores(d)
    logical = topk(d, scores, ld)
    paged = _transform(d, scores, ld, dsa.DSA_IDX_PAGED)
    sync()
    # knock out a few entries of each row: -1 and a slot past the pool
    p = paged.cpu().numpy()
    lg = logical.cpu().numpy()
    for i in range(b.T):
        p[i, 3] = -7
        p[i, 100] = b.num_pages * 64 + 5
        lg[i, 3] = -1
        lg[i, 100] = -1
    out_l, lse_l = sparse_mla(d, torch.from_numpy(lg).cuda())
    out_p, lse_p = _paged_mla(d, torch.from_numpy(p).cuda())
    sync()
    assert torch.equal(out_p, out_l) and torch.equal(lse_p, lse_l)


def test_topk_transform_headline_workload():
    """The 128K decode batch at full size, the launch the bench times; rows
    sampled for the oracle checks."""
    b = synth.make_workload(2)
    d = to_device(b, layers=[0])
    rng = np.random.default_rng(2)
    rows = sorted({0, b.T - 1} | set(rng.choice(b.T, 4, replace=False).tolist()))
    logical, paged, rows, meta = _check_spaces(b, d, rows=rows)
    out_l, lse_l = sparse_mla(d, logical)
    out_p, lse_p = _paged_mla(d, paged)
    sync()
    assert torch.equal(out_p, out_l) and torch.equal(lse_p, lse_l)
