"""GPU parity of the masked multi-head attention in the expanded form
(dsa_masked_mha_prefill) with the float64 oracle, through the C ABI.

Small batches cover several 64-position tiles and 128-row query blocks with
ragged tails: prefill chunks onto cached prefixes, a padding request, page
ids outside the pool, with and without a selection.  The 4096-row prefill on
an empty cache runs in the bench's configuration (the top-2048 selection of
the indexer, then the masked form) and is checked on sampled rows.  Bars as
for the latent attention (gpu_common); the expanded keys and values are
held in bf16, one more rounding than the latent form has."""
import numpy as np
import pytest
import torch

from gpu_common import (K, O, bf16_to_f64, check_attention, dsa, index_scores, record_margin,
                        synth, sync, to_device, topk)

pytestmark = pytest.mark.gpu

SMALL = [
    dict(n_q=[1], L=[1]),
    dict(n_q=[3], L=[70]),
    dict(n_q=[130], L=[130]),
    dict(n_q=[2, 1, 0, 5], L=[64, 300, 0, 1000]),
    dict(n_q=[200, 1], L=[1500, 129]),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def _inputs(b, seed):
    qn, qr, wk, wv = synth.mha_inputs(seed, b.T)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda()
    return (qn, qr, wk, wv), tuple(dev(a) for a in (qn, qr, wk, wv))


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()


def check_masked_mha(b, host, idx, rows, out, lse):
    """The contract's output bars, and bounds derived from this form's
    arithmetic.  The expanded keys and values are rounded once to bf16
    (relative error <= 2^-9), so a score moves by at most
        dz = sm_scale * 2^-8 * max_s sum_d |q_nope_d| |k_d(s)|
    over the attended positions (2^-8: the rounding plus fp32 sums), and the
    lse, a smooth maximum of the scores, by at most dz.  The weights move by
    at most (2 dz + 2^-9) of themselves (the scores, then P's bf16 rounding),
    the values by 2^-9 and the output by its bf16 rounding, so each output
    element moves by at most (2 dz + 2^-7) max_s |v(s)|_inf."""
    qn, qr, wk, wv = host
    meta = O.Meta.of(b)
    ref, ref_lse = O.masked_mha(meta, qn, qr, wk, wv, b.kv[0], idx, rows, synth.SM_SCALE)
    got, got_lse = bf16_to_f64(out[rows]), lse[rows].cpu().numpy().astype(np.float64)
    check_attention(got, ref, relative=False)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(got_lse)) and np.all(np.isneginf(got_lse[~fin]))
    assert np.all(got[~fin] == 0)
    kvf = _bf16(b.kv[0]).reshape(-1, 576)
    W_k, W_v = _bf16(wk), _bf16(wv)
    Q = np.abs(_bf16(qn))
    dz = np.zeros((len(rows), 128))
    vm = np.zeros((len(rows), 128))
    req = [int(np.searchsorted(b.cu_seqlens_q, t, side="right") - 1) for t in rows]
    for bi in range(b.B):
        mine = [i for i in range(len(rows)) if req[i] == bi]
        L = int(b.seqlens_k[bi])
        if not mine or L == 0:
            continue
        pos = np.arange(L)
        pg = b.page_table[bi, pos // 64]
        ok = (pg >= 0) & (pg < b.num_pages)
        pos = pos[ok]
        c = kvf[pg[ok].astype(np.int64) * 64 + pos % 64, :512]
        att = np.zeros((len(mine), len(pos)), bool)  # attended, among the valid positions
        for j, i in enumerate(mine):
            v = meta.visible(rows[i])
            if idx is None:
                att[j] = pos < v
            else:
                lst = idx[i][(idx[i] >= 0) & (idx[i] < v)]
                att[j] = np.isin(pos, lst)
        qrows = Q[[rows[i] for i in mine]]
        for h in range(128):
            kn = np.abs(c @ W_k[h].T)                          # [n, 128]
            vv = np.abs(c @ W_v[h].T).max(axis=1)             # [n]
            A = qrows[:, h, :] @ kn.T                          # [rows, n]
            dz[mine, h] = np.where(att, A, 0.0).max(axis=1, initial=0.0)
            vm[mine, h] = np.where(att, vv[None, :], 0.0).max(axis=1, initial=0.0)
    dz *= synth.SM_SCALE * 2.0 ** -8
    lerr = np.where(fin, np.abs(got_lse - np.where(fin, ref_lse, 0.0)), 0.0)
    oerr = np.abs(got - ref).max(axis=2)
    lbound = dz + 1e-5
    obound = (2 * dz + 2.0 ** -7) * vm + 1e-30
    assert np.all(lerr <= lbound), float((lerr / lbound).max())
    assert np.all(oerr <= obound), float((oerr / obound).max())
    worst_l = float((lerr / lbound).max())
    worst_o = float((oerr / obound).max())
    record_margin("masked MHA lse error / derived bound", worst_l, 1.0)
    record_margin("masked MHA output error / derived bound", worst_o, 1.0)


def masked_mha(d, dv_in, idx=None, k=1):
    T = d.meta.T
    ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_MASKED_MHA, d.meta, 1, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, 128, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, 128), dtype=torch.float32, device="cuda")
    qn, qr, wk, wv = dv_in
    dsa.dsa_masked_mha_prefill(d.meta, qn, qr, wk, wv, d.kv[0], idx, k, synth.SM_SCALE, out, lse,
                               ws, ws_bytes)
    return out, lse


def _with_bad_pages(b):
    bad = b.page_table.copy()
    bad[0, 0] = -1 if b.page_table.shape[1] < 2 else b.num_pages + 3
    if b.page_table.shape[1] > 2:
        bad[0, 2] = -7
    b.page_table = bad
    return b


@pytest.mark.device_check_flags
@pytest.mark.parametrize("ci", range(len(SMALL)))
@pytest.mark.parametrize("mode", ["causal", "selection", "bad_pages"])
def test_masked_mha_small(ci, mode):
    case = SMALL[ci]
    b = synth.make_batch(case["n_q"], case["L"], seed=400 + ci, paging="shuffled", heavy=8,
                         pool_extra_pages=2)
    if mode == "bad_pages":
        b = _with_bad_pages(b)
    d = to_device(b)
    host, dev = _inputs(b, 500 + ci)
    idx = None
    k = 1
    if mode == "selection":
        # a random half of each row's visible positions (unsorted), -1 padded
        rng = np.random.default_rng(600 + ci)
        meta = O.Meta.of(b)
        k = 96
        idx = np.full((b.T, k), -1, np.int32)
        for t in range(b.T):
            v = meta.visible(t)
            pick = rng.choice(v, min(k, (v + 1) // 2), replace=False) if v else []
            idx[t, :len(pick)] = pick
    out, lse = masked_mha(d, dev, None if idx is None else torch.from_numpy(idx).cuda(), k)
    sync()
    check_masked_mha(b, host, idx, list(range(b.T)), out, lse)


def test_masked_mha_full_selection_is_causal_bitwise():
    """A selection listing every visible position of every row (in any
    order) gives the causal result, bit for bit."""
    b = synth.make_batch([300], [700], seed=410, paging="shuffled", heavy=8)
    d = to_device(b)
    _, dev = _inputs(b, 510)
    meta = O.Meta.of(b)
    rng = np.random.default_rng(7)
    idx = np.full((b.T, 700), -1, np.int32)
    for t in range(b.T):
        idx[t, :meta.visible(t)] = rng.permutation(meta.visible(t))
    o1, l1 = masked_mha(d, dev)
    o2, l2 = masked_mha(d, dev, torch.from_numpy(idx).cuda(), 700)
    sync()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_masked_mha_prefill_4096_with_topk_selection():
    """The 4096-row prefill on an empty cache (row j sees j + 1 tokens): the
    indexer's top-2048 selection, then the masked form over it; sampled rows
    on both sides of the 2048-token mark against the oracle."""
    n = 4096
    b = synth.make_batch([n], [n], seed=84, paging="identity", heavy=64, pool_extra_pages=1)
    d = to_device(b)
    host, dev = _inputs(b, 520)
    scores, ld = index_scores(d)
    idx = topk(d, scores, ld)
    del scores
    out, lse = masked_mha(d, dev, idx, K)
    sync()
    rows = [0, 1, 1000, 2046, 2047, 2048, 2049, 3000, 4095]
    check_masked_mha(b, host, idx[rows].cpu().numpy(), rows, out, lse)
