"""The short-sequence dense form, through the C ABI: dsa_dense_mla_decode
against the oracle's dense attention, and against the sparse attention over
the every-position selection bit for bit; dsa_decode_step on batches whose
contexts fit in k, which select without scanning and attend densely."""
import numpy as np
import pytest
import torch

from gpu_common import (K, O, bf16_to_f64, check_attention, check_selection, decode_step, dsa,
                        oracle_rows, sparse_mla, synth, sync, to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def _dense(d, n_split=0, layer=0):
    T = d.meta.T
    ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_DENSE_MLA, d.meta, 1, n_split)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, 128), dtype=torch.float32, device="cuda")
    dsa.dsa_dense_mla_decode(d.meta, d.q[layer], d.kv[layer], synth.SM_SCALE, out, lse, n_split,
                             ws, ws_bytes)
    return out, lse


def _all_positions(b, k):
    vis = b.visible()
    idx = np.full((b.T, k), -1, np.int32)
    for t, v in enumerate(vis):
        idx[t, :min(v, k)] = np.arange(min(v, k))
    return idx


CASES = [
    dict(n_q=[1], L=[1]),
    dict(n_q=[2, 1], L=[64, 65]),
    dict(n_q=[3, 1, 2], L=[700, 2048, 1500]),
    dict(n_q=[2, 2, 1, 5], L=[130, 2000, 0, 1100]),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
@pytest.mark.parametrize("n_split", [0, 1, 3])
def test_dense_mla_matches_oracle_and_sparse(ci, n_split):
    case = CASES[ci]
    b = synth.make_batch(case["n_q"], case["L"], seed=800 + ci, paging="shuffled", heavy=16,
                         pool_extra_pages=3)
    d = to_device(b)
    out, lse = _dense(d, n_split)
    k = max(1, int(max(case["L"])))
    idx = torch.from_numpy(_all_positions(b, k)).cuda()
    out_s, lse_s = sparse_mla(d, idx, k=k, n_split=n_split)
    sync()
    assert torch.equal(out, out_s) and torch.equal(lse, lse_s)
    rows = list(range(b.T))
    ref, ref_lse = O.dense_mla(O.Meta.of(b), b.q[0], b.kv[0], rows, synth.SM_SCALE)
    check_attention(bf16_to_f64(out), ref, lse.cpu().numpy(), ref_lse)


def test_dense_mla_long_rows():
    """Rows of 20K-40K tokens (many splits of 2048): still the oracle's dense attention."""
    b = synth.make_batch([1, 2], [20000, 40000], seed=81, paging="shuffled", heavy=16,
                         pool_extra_pages=3)
    d = to_device(b)
    out, lse = _dense(d)
    sync()
    rows = list(range(b.T))
    ref, ref_lse = O.dense_mla(O.Meta.of(b), b.q[0], b.kv[0], rows, synth.SM_SCALE)
    check_attention(bf16_to_f64(out), ref, lse.cpu().numpy(), ref_lse)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_decode_step_short_contexts_skip_the_scan(ci):
    case = CASES[ci]
    b = synth.make_batch(case["n_q"], case["L"], seed=820 + ci, paging="shuffled", heavy=16,
                         pool_extra_pages=3)
    d = to_device(b)
    assert b.max_seqlen_k <= K
    idx, out, lse = decode_step(d)
    sync()
    g = idx.cpu().numpy()
    assert np.array_equal(g, _all_positions(b, K))
    rows = list(range(b.T))
    meta, vis, sc, sel, flags, Ks = oracle_rows(b, rows)
    check_selection(g, sel, flags, Ks)
    out_s, lse_s = sparse_mla(d, idx)
    sync()
    assert torch.equal(out, out_s) and torch.equal(lse, lse_s)


def test_decode_step_short_context_batch_at_size():
    """64 requests x 2 rows onto 2048 cached tokens: the batch the bench
    times for the short-context form."""
    b = synth.make_batch([2] * 64, [2048] * 64, seed=83, paging="shuffled", heavy=16,
                         pool_extra_pages=3)
    d = to_device(b)
    idx, out, lse = decode_step(d)
    sync()
    assert np.array_equal(idx.cpu().numpy(), _all_positions(b, K))
    rows = [0, 1, 77, b.T - 1]
    ref, ref_lse = O.dense_mla(O.Meta.of(b), b.q[0], b.kv[0], rows, synth.SM_SCALE)
    check_attention(bf16_to_f64(out[rows]), ref, lse[rows].cpu().numpy(), ref_lse)
