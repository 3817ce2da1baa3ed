"""Parity of the HIP path with the float64 oracle, through the C ABI.

Small cases span several tiles and ragged tails (L around the 64-token page
and the 2048-token selection, 1-5 rows per request, padding requests);
the five workloads run at their full sizes with the launch configuration
the bench uses, checked on sampled rows.  The bars:
  * scores: within SCORE_RTOL of the row's largest float64 score;
  * selection: identical to the oracle's outside its flagged tie band
    (bit-exact when both sides rank the same float32 scores);
  * attention: bf16 output within max-abs 2e-2 and mean-abs 2e-3 (also
    relative to the reference rms), lse within 1e-3.
"""
import numpy as np
import pytest
import torch

from gpu_common import (K, O, bf16_to_f64, check_attention, check_scores, check_selection,
                        decode_step, dsa, index_scores, oracle_rows, sparse_mla, synth, sync,
                        to_device, topk)

pytestmark = pytest.mark.gpu

SMALL = [
    dict(n_q=[1], L=[1]),
    dict(n_q=[1], L=[63]),
    dict(n_q=[2, 1], L=[64, 65]),
    dict(n_q=[3, 1, 2], L=[2047, 2048, 2049]),
    dict(n_q=[2, 2, 1, 5], L=[130, 5000, 0, 4100]),
    dict(n_q=[1, 2], L=[9000, 20000]),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def _small(case, seed, paging="shuffled", mla_scale=None, heavy=16):
    kw = {} if mla_scale is None else dict(mla_scale=mla_scale)
    return synth.make_batch(case["n_q"], case["L"], seed=seed, paging=paging, heavy=heavy,
                            pool_extra_pages=3, **kw)


@pytest.mark.parametrize("ci", range(len(SMALL)))
def test_index_score_small(ci):
    b = _small(SMALL[ci], 100 + ci)
    d = to_device(b)
    scores, ld = index_scores(d)
    sync()
    rows = list(range(b.T))
    meta, vis, sc, sel, flags, Ks = oracle_rows(b, rows)
    check_scores(scores.cpu().numpy().astype(np.float64), sc, vis)
    # positions past a row's visible length are not written
    g = scores.cpu().numpy()
    for i, v in enumerate(vis):
        assert np.isnan(g[i, v:]).all()


# SMALL cases with at most two rows per request (the scan form that gives
# each key page to one wave)
PAGE_FORM = [0, 1, 2, 5]


@pytest.mark.parametrize("ci", PAGE_FORM)
def test_index_score_unaligned_row_stride(ci):
    """ld not a multiple of 4: rows start unaligned and the scan writes them
    out element by element; nothing past a row's visible length is touched."""
    b = _small(SMALL[ci], 150 + ci)
    d = to_device(b)
    scores, ld = index_scores(d, ld=int(b.max_seqlen_k) + 5)
    sync()
    meta, vis, sc, *_ = oracle_rows(b, list(range(b.T)))
    got = scores.cpu().numpy().astype(np.float64)
    check_scores(got, sc, vis)
    for i, v in enumerate(vis):
        assert np.all(np.isnan(got[i, v:])), i


def _with_bad_pages(b):
    """Page ids outside the pool on three logical pages (one of the second
    request when there is one): -1, num_pages + 7 and -5."""
    bad = b.page_table.copy()
    bad[0, 1] = -1
    bad[0, 3] = b.num_pages + 7
    if b.B > 1:
        bad[1, 0] = -5
    b.page_table = bad
    return b


@pytest.mark.device_check_flags
@pytest.mark.parametrize("case", [dict(n_q=[2, 1], L=[5000, 3000]), dict(n_q=[1], L=[3000]),
                                  dict(n_q=[3, 1], L=[4000, 2500])])
def test_index_score_pages_with_invalid_ids_score_minus_inf(case):
    """A page id outside the pool names no key: its visible positions score
    -inf (both scan forms), every other score as the oracle's."""
    b = _with_bad_pages(_small(case, 160))
    meta, vis, sc, *_ = oracle_rows(b, list(range(b.T)))
    d = to_device(b)
    scores, ld = index_scores(d)
    sync()
    got = scores.cpu().numpy().astype(np.float64)
    n_inf = 0
    for i, v in enumerate(vis):
        ninf = np.isneginf(sc[i, :v])
        n_inf += int(ninf.sum())
        assert np.array_equal(np.isneginf(got[i, :v]), ninf), i
        got[i, :v][ninf] = 0.0
        sc[i, :v][ninf] = 0.0
    assert n_inf > 0
    check_scores(got, sc, vis)


@pytest.mark.device_check_flags
@pytest.mark.parametrize("case", [dict(n_q=[2, 1], L=[5000, 2100]), dict(n_q=[2, 2], L=[70001, 3000])])
def test_decode_step_with_invalid_page_ids_ignores_workspace_contents(case):
    """The step's selection and attention with page ids outside the pool do
    not depend on what the workspace held before the call (the scan writes
    -inf for every visible position it has no key for, so the top-k never
    reads a stale score): two calls over workspaces filled with different
    byte patterns agree bit for bit, and match the oracle.  The second case
    has rows longer than the one-pass top-k (scan histogram, collect and
    final kernels)."""
    b = _with_bad_pages(_small(case, 170))
    d = to_device(b)
    T = b.T
    ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_DECODE_STEP, d.meta, K, 0)
    res = []
    for fill in (0x00, 0x7F):  # 0x7F7F7F7F is a large positive float
        ws = torch.full((ws_bytes,), fill, dtype=torch.uint8, device="cuda")
        idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
        out = torch.empty((T, 128, 512), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((T, 128), dtype=torch.float32, device="cuda")
        ix = dict(q8=d.q8, q_scale=d.q_scale, w=d.w, k8_cache=d.k8[0], k_scale=d.k_scale[0])
        ml = dict(q=d.q[0], kv_cache=d.kv[0], sm_scale=synth.SM_SCALE)
        dsa.dsa_decode_step(d.meta, ix, ml, K, dsa.DSA_MODE_FUSED, 0, None, idx, out, lse, ws,
                            ws_bytes)
        sync()
        res.append((idx.clone(), out.clone(), lse.clone()))
    assert torch.equal(res[0][0], res[1][0])
    assert torch.equal(res[0][1], res[1][1]) and torch.equal(res[0][2], res[1][2])
    rows = list(range(T))
    meta, vis, sc, sel, flags, Ks = oracle_rows(b, rows)
    g = res[0][0].cpu().numpy()
    check_selection(g, sel, flags, Ks)
    ref, ref_lse = O.sparse_mla(meta, b.q[0], b.kv[0], g, rows, synth.SM_SCALE)
    check_attention(bf16_to_f64(res[0][1]), ref, res[0][2].cpu().numpy(), ref_lse)


@pytest.mark.parametrize("ci", range(len(SMALL)))
@pytest.mark.parametrize("k", [1, 37, 2048])
def test_topk_small_exact_on_same_scores(ci, k):
    """Given identical float32 scores the GPU selection equals the oracle's exactly."""
    b = _small(SMALL[ci], 200 + ci)
    d = to_device(b)
    scores, ld = index_scores(d)
    idx = topk(d, scores, ld, k)
    sync()
    s64 = scores.cpu().numpy().astype(np.float64)
    vis = b.visible()
    sel, flags, kth, Ks = O.topk(np.nan_to_num(s64, nan=-np.inf), vis, k, band=0.0)
    g = idx.cpu().numpy()
    for i in range(b.T):
        K_ = int(Ks[i])
        assert sorted(g[i, :K_].tolist()) == g[i, :K_].tolist()  # ascending
        assert set(g[i, :K_].tolist()) == set(sel[i, :K_].tolist()), i
        assert (g[i, K_:] == -1).all()


@pytest.mark.parametrize("pattern", ["all_equal", "few_values", "negative", "signed_zero",
                                     "heavy_ties"])
def test_topk_adversarial_scores(pattern):
    rng = np.random.default_rng(7)
    b = _small(dict(n_q=[1, 2, 1], L=[30000, 12000, 3000]), 300, heavy=0)
    d = to_device(b)
    T, ld = b.T, 30016
    vis = b.visible()
    if pattern == "all_equal":
        s = np.full((T, ld), 1.5, np.float32)
    elif pattern == "few_values":
        s = rng.integers(0, 5, (T, ld)).astype(np.float32)
    elif pattern == "negative":
        s = -np.abs(rng.normal(size=(T, ld))).astype(np.float32)
    elif pattern == "signed_zero":
        s = np.where(rng.random((T, ld)) < 0.5, np.float32(-0.0), np.float32(0.0))
        s[:, ::97] = 1.0
    else:
        s = np.round(rng.normal(size=(T, ld)), 1).astype(np.float32)
    for k in (1, 2048, 5000):
        idx = topk(d, torch.from_numpy(s).cuda(), ld, k)
        sync()
        sel, _, _, Ks = O.topk(s.astype(np.float64), vis, k, band=0.0)
        g = idx.cpu().numpy()
        for i in range(T):
            K_ = int(Ks[i])
            assert set(g[i, :K_].tolist()) == set(sel[i, :K_].tolist()), (pattern, k, i)
            assert (g[i, K_:] == -1).all()


def _meta(L, n_q=None):
    """Batch metadata only (identity page table): enough for the top-k."""
    n_q = n_q or [1] * len(L)
    cu = np.concatenate([[0], np.cumsum(n_q)]).astype(np.int32)
    mx = max(L)
    pages = max(1, -(-mx // 64))
    pt = np.tile(np.arange(pages, dtype=np.int32), (len(L), 1))
    dev = lambda a: torch.from_numpy(a).cuda()  # noqa: E731
    return dsa.Batch(dev(cu), dev(np.asarray(L, np.int32)), dev(pt), pages, max(n_q), mx)


@pytest.mark.parametrize("L", [[8192, 100], [8193, 40], [32768, 5000], [32769], [65536, 2049],
                               [65537, 3000], [131072, 70001], [200003]])
@pytest.mark.parametrize("k", [1, 2048, 8192])
@pytest.mark.parametrize("pattern", ["rounded", "few_values"])
def test_topk_one_pass_and_multi_pass_agree(L, k, pattern):
    """With scores 16-byte aligned and ld % 4 == 0, rows of at most 65536
    positions take the one-pass kernel (keys held in registers); longer rows,
    or an odd ld, go through the histogram, collect and final kernels (with
    few distinct values the final pass's candidates overflow its LDS stage
    and are read from the workspace list).  Both selections equal the
    oracle's on these float32 scores (rounded to 0.01, or 5 distinct values,
    so that many keys tie at the threshold), in ascending order."""
    rng = np.random.default_rng(sum(L) + k)
    meta = _meta(L)
    T, mx = len(L), max(L)
    if pattern == "rounded":
        s = np.round(rng.normal(size=(T, mx + 8)), 2).astype(np.float32)
    else:
        s = rng.integers(0, 5, (T, mx + 8)).astype(np.float32)
    vis = [min(x, mx) for x in L]
    sel, _, _, Ks = O.topk(s.astype(np.float64), vis, k, band=0.0)
    ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_TOPK, meta, k)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    got = []
    for ld in (mx + (-mx) % 4, mx + (-mx) % 4 + 1):
        x = torch.from_numpy(np.ascontiguousarray(s[:, :ld])).cuda()
        idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
        dsa.dsa_topk(meta, x, ld, k, idx, ws, ws_bytes)
        sync()
        g = idx.cpu().numpy()
        for i in range(T):
            K_ = int(Ks[i])
            assert g[i, :K_].tolist() == sorted(sel[i, :K_].tolist()), (ld, i)
            assert (g[i, K_:] == -1).all()
        got.append(g)
    assert np.array_equal(got[0], got[1])


@pytest.mark.parametrize("k", [1, 2048, 4096])
def test_topk_rows_longer_than_the_bitmap(k):
    """Rows of more than 393216 positions: the final pass gathers the
    selection into LDS and sorts it (k <= 4096); rounded scores put many
    keys at the threshold.  Equal to the oracle's selection, ascending."""
    L = [400000, 450001, 393216]
    rng = np.random.default_rng(k)
    meta = _meta(L)
    T, mx = len(L), max(L)
    ld = mx + (-mx) % 4
    s = np.round(rng.normal(size=(T, ld)), 2).astype(np.float32)
    sel, _, _, Ks = O.topk(s.astype(np.float64), L, k, band=0.0)
    ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_TOPK, meta, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(meta, torch.from_numpy(s).cuda(), ld, k, idx, ws, ws_bytes)
    sync()
    g = idx.cpu().numpy()
    for i in range(T):
        K_ = int(Ks[i])
        assert g[i, :K_].tolist() == sorted(sel[i, :K_].tolist()), i
        assert (g[i, K_:] == -1).all()


@pytest.mark.parametrize("ci", range(len(SMALL)))
def test_selection_end_to_end_small(ci):
    b = _small(SMALL[ci], 400 + ci)
    d = to_device(b)
    scores, ld = index_scores(d)
    idx = topk(d, scores, ld)
    sync()
    meta, vis, sc, sel, flags, Ks = oracle_rows(b, list(range(b.T)))
    check_selection(idx.cpu().numpy(), sel, flags, Ks)


@pytest.mark.parametrize("ci", [0, 2, 3, 4, 5])
@pytest.mark.parametrize("n_split", [1, 2, 7, 13, 64])
@pytest.mark.parametrize("stress", [False, True])
def test_sparse_mla_small_oracle_selection(ci, n_split, stress):
    """Attention fed the oracle's selection, for several split counts (the
    merge reads more than four splits in batches of eight: 7 is one partial
    batch, 13 a full and a partial one, 64 eight full ones);
    `stress` draws q and kv from N(0,1) so the absolute bound bites."""
    b = _small(SMALL[ci], 500 + ci, mla_scale=1.0 if stress else None)
    d = to_device(b)
    meta, vis, sc, sel, flags, Ks = oracle_rows(b, list(range(b.T)))
    idx = torch.from_numpy(sel).cuda()
    out, lse = sparse_mla(d, idx, n_split=n_split)
    sync()
    ref, ref_lse = O.sparse_mla(meta, b.q[0], b.kv[0], sel, list(range(b.T)), synth.SM_SCALE)
    check_attention(bf16_to_f64(out), ref, lse.cpu().numpy(), ref_lse, relative=not stress)


@pytest.mark.parametrize("n_split", [1, 3])
def test_sparse_mla_wide_logit_range(n_split):
    """Queries scaled by 2^6: logits spread over hundreds of units, so later
    tiles exceed the first tile's maximum by far more than the kernel lets
    its softmax weights grow, and it must take the exact maximum and start
    again."""
    b = _small(dict(n_q=[2, 1], L=[6000, 2500]), 650, mla_scale=1.0)
    q = b.q[0]
    f = (q.astype(np.uint32) << 16).view(np.float32) * np.float32(64.0)
    b.q[0] = (f.view(np.uint32) >> 16).astype(np.uint16)
    d = to_device(b)
    meta, vis, sc, sel, flags, Ks = oracle_rows(b, list(range(b.T)))
    idx = torch.from_numpy(sel).cuda()
    out, lse = sparse_mla(d, idx, n_split=n_split)
    sync()
    ref, ref_lse = O.sparse_mla(meta, b.q[0], b.kv[0], sel, list(range(b.T)), synth.SM_SCALE)
    assert np.abs(ref_lse[np.isfinite(ref_lse)]).max() > 100  # the case is wide
    check_attention(bf16_to_f64(out), ref, relative=False)
    # lse ~ a few hundred: fp32 sums of 576 products carry ~1e-6 relative
    g = lse.cpu().numpy().astype(np.float64)
    assert np.abs(g - ref_lse).max() <= 1e-3 + 4e-6 * np.abs(ref_lse).max()


def _weighted_abs_kv(b, sel, rows):
    """sum_s p_s |kv_s[0:512]| per (row, head): the softmax weights over the
    selection (float64 torch on the CPU) against the magnitudes of the value
    rows, and the largest |kv| per (row, 64-dim slice) over the selection."""
    kv = torch.from_numpy(b.kv[0].reshape(-1, 576).view(np.int16)).view(torch.bfloat16).double()
    q = torch.from_numpy(b.q[0].view(np.int16)).view(torch.bfloat16).double()
    A, S = [], []
    for i, t in enumerate(rows):
        bi = int(np.searchsorted(b.cu_seqlens_q, t, side="right") - 1)
        pos = torch.from_numpy(sel[i][sel[i] >= 0].astype(np.int64))
        slots = torch.from_numpy(b.page_table[bi].astype(np.int64))[pos // 64] * 64 + pos % 64
        rowsk = kv[slots]
        p = torch.softmax(synth.SM_SCALE * q[t] @ rowsk.T, dim=-1)
        A.append((p @ rowsk[:, :512].abs()).numpy())
        S.append(rowsk[:, :512].abs().reshape(-1, 8, 64).amax(dim=(0, 2)).numpy())
    return np.stack(A), np.stack(S)


def test_sparse_mla_split_invariance_and_determinism():
    """One split against four.  Each form rounds every softmax weight to bf16
    before the value product (relative error <= 2^-9 per weight, whatever
    reference maximum the split's online softmax holds) and rounds the output
    to bf16 (<= 2^-9 of |o|); with several splits each split's partial is held
    in fp16 scaled per 64-dim slice (<= 2^-11 of the slice's largest partial,
    itself at most the slice's largest |kv|).  So per element
      |o1 - o4| <= 2^-8 sum_s p_s |kv_s| + 2^-8 max(|o1|, |o4|) + 2^-11 max_slice |kv|,
    with p the exact softmax weights over the selection."""
    b = _small(SMALL[5], 600, mla_scale=1.0)
    d = to_device(b)
    rows = list(range(b.T))
    meta, vis, sc, sel, flags, Ks = oracle_rows(b, rows)
    idx = torch.from_numpy(sel).cuda()
    o1, l1 = sparse_mla(d, idx, n_split=1)
    o4, l4 = sparse_mla(d, idx, n_split=4)
    o4b, l4b = sparse_mla(d, idx, n_split=4)
    sync()
    assert torch.equal(o4, o4b) and torch.equal(l4, l4b)
    A, S = _weighted_abs_kv(b, sel, rows)  # [T, 128, 512], [T, 8]
    a, c = bf16_to_f64(o1), bf16_to_f64(o4)
    slice_max = np.repeat(S, 64, axis=1)[:, None, :]  # [T, 1, 512]
    bound = 2.0 ** -8 * A + 2.0 ** -8 * np.maximum(np.abs(a), np.abs(c)) + 2.0 ** -11 * slice_max
    diff = np.abs(a - c)
    from gpu_common import record_margin
    record_margin("split 1 vs 4: max |diff| / bound", float((diff / bound).max()), 1.0)
    assert np.all(diff <= bound), float((diff / bound).max())
    assert (l1 - l4).abs().max().item() <= 1e-4


@pytest.mark.device_check_flags
def test_sparse_mla_handles_unsorted_padded_and_invalid_positions():
    b = _small(dict(n_q=[2], L=[3000]), 700, mla_scale=1.0)
    d = to_device(b)
    rng = np.random.default_rng(1)
    sel = np.full((2, 256), -1, np.int32)
    pos = rng.choice(2999, 150, replace=False).astype(np.int32)
    sel[:, :150] = pos
    sel[0, 150] = 2999  # not visible to row 0: skipped
    sel[1, 150] = 2999
    sel[:, 151] = 5000  # past the cache: skipped
    rng.shuffle(sel[1])
    out, lse = sparse_mla(d, torch.from_numpy(sel).cuda(), k=256, n_split=3)
    sync()
    meta = O.Meta.of(b)
    ref, ref_lse = O.sparse_mla(meta, b.q[0], b.kv[0], sel, [0, 1], synth.SM_SCALE)
    check_attention(bf16_to_f64(out), ref, lse.cpu().numpy(), ref_lse, relative=False)


def test_page_permutation_invariance_bitwise():
    case = dict(n_q=[2, 1], L=[5000, 3000])
    b = _small(case, 800, paging="identity")
    d = to_device(b)
    idx1, out1, lse1 = decode_step(d)
    # same logical data, physical pages permuted
    perm = np.random.default_rng(3).permutation(b.num_pages).astype(np.int32)
    b2 = _small(case, 800, paging="identity")
    for lst in (b2.k8, b2.k_scale, b2.kv):
        x = lst[0].copy()
        lst[0][perm] = x
    b2.page_table = perm[b.page_table]
    d2 = to_device(b2)
    idx2, out2, lse2 = decode_step(d2)
    sync()
    assert torch.equal(idx1, idx2)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


@pytest.mark.parametrize("ci", range(len(SMALL)))
def test_decode_step_small(ci):
    b = _small(SMALL[ci], 900 + ci)
    d = to_device(b)
    idx, out, lse = decode_step(d)
    idx2, out2, lse2 = decode_step(d)
    sync()
    assert torch.equal(idx, idx2) and torch.equal(out, out2)  # deterministic
    rows = list(range(b.T))
    meta, vis, sc, sel, flags, Ks = oracle_rows(b, rows)
    g = idx.cpu().numpy()
    check_selection(g, sel, flags, Ks)
    ref, ref_lse = O.sparse_mla(meta, b.q[0], b.kv[0], g, rows, synth.SM_SCALE)
    check_attention(bf16_to_f64(out), ref, lse.cpu().numpy(), ref_lse)


# ------------------------------------------------------------ full workloads

_cache = {}


def _workload(i):
    if i not in _cache:
        _cache.clear()
        b = synth.make_workload(i)
        _cache[i] = (b, to_device(b))
    return _cache[i]


def _sample_rows(T, n, seed):
    rng = np.random.default_rng(seed)
    rows = {0, T - 1}
    rows.update(rng.choice(T, min(n, T), replace=False).tolist())
    return sorted(rows)


@pytest.mark.parametrize("wi", [0, 1, 2, 3])
def test_workload_decode_step(wi):
    """The workloads at full size in the bench's launch configuration.  The
    three decode workloads are checked on every row (the 128K batch's 128
    rows take the oracle about 8 s on 16 cores); the 4096-row prefill on
    sampled rows.  On the decode workloads the fused step's selection (scan
    with its histogram epilogue, then the top-k: one pass for rows of up to
    65536 positions, collect and final kernels beyond) must also equal, bit
    for bit, dsa_index_score followed by dsa_topk on the same inputs."""
    b, d = _workload(wi)
    print(f"workload {wi} {b.name}: T={b.T} pages={b.num_pages}", flush=True)
    idx, out, lse = decode_step(d)
    sync()
    if wi in (1, 2):
        scores, ld = index_scores(d)
        idx2 = topk(d, scores, ld)
        sync()
        assert torch.equal(idx, idx2)
        del scores
    rows = list(range(b.T)) if wi <= 2 else _sample_rows(b.T, 6, wi)
    meta, vis, sc, sel, flags, Ks = oracle_rows(b, rows)
    g = idx[rows].cpu().numpy()
    check_selection(g, sel, flags, Ks)
    ref, ref_lse = O.sparse_mla(meta, b.q[0], b.kv[0], g, rows, synth.SM_SCALE)
    check_attention(bf16_to_f64(out[rows]), ref, lse[rows].cpu().numpy(), ref_lse)
    # decode rows always select the heavy tokens (prefill rows need not: the
    # heavy direction follows the sum over all 4096 rows)
    for j, t in enumerate(rows if b.max_q <= 2 else []):
        bi = int(np.searchsorted(b.cu_seqlens_q, t, side="right") - 1)
        hv = set(b.heavy[bi].tolist())
        hv = {s for s in hv if s < vis[j]}
        assert hv <= set(g[j].tolist()) or len(hv) > K


def test_prefill_chunk_longer_than_the_one_pass_topk():
    """1024 new rows on a 68976-token prefix (70000 cached): the row-group
    scan in 128-page ranges with its histogram epilogue, then the
    multi-kernel top-k (rows of more than 65536 positions).  Scores,
    selection and attention on sampled rows against the oracle."""
    b = synth.make_batch([1024], [70000], seed=1600, paging="shuffled", heavy=64,
                         pool_extra_pages=3)
    d = to_device(b)
    idx, out, lse = decode_step(d)
    scores, ld = index_scores(d)
    sync()
    rows = sorted({0, 1023} | set(_sample_rows(b.T, 4, 16)))
    meta, vis, sc, sel, flags, Ks = oracle_rows(b, rows)
    check_scores(scores[rows].cpu().numpy().astype(np.float64), sc, vis)
    g = idx[rows].cpu().numpy()
    check_selection(g, sel, flags, Ks)
    ref, ref_lse = O.sparse_mla(meta, b.q[0], b.kv[0], g, rows, synth.SM_SCALE)
    check_attention(bf16_to_f64(out[rows]), ref, lse[rows].cpu().numpy(), ref_lse)


@pytest.mark.parametrize("wi", [1, 2])
def test_workload_index_scores(wi):
    b, d = _workload(wi)
    scores, ld = index_scores(d)
    sync()
    rows = _sample_rows(b.T, 3, 10 + wi)
    meta, vis, sc, sel, flags, Ks = oracle_rows(b, rows)
    check_scores(scores[rows].cpu().numpy().astype(np.float64), sc, vis)


def test_workload_mli_two_stream():
    """Two-layer ragged batch: layer l's attention over its selection runs on
    the main stream while layer l+1's indexer + top-k run on a second one."""
    b, d = _workload(4)
    print(f"workload 4 {b.name}: T={b.T} pages={b.num_pages}", flush=True)
    sel0, out0, lse0 = decode_step(d, layer=0)
    aux = torch.cuda.Stream()
    sel1, out_mli, lse_mli = decode_step(d, layer=1, mode=dsa.DSA_MODE_MLI, attend_idx=sel0,
                                         mla_layer=0, stream_aux=aux)
    # with the fused step's split count, the attention of the MLI step equals
    # the fused step's (same selection, same layer); by default MLI picks fewer
    ns = dsa.dsa_default_splits(d.meta, K)
    _, out_ns, lse_ns = decode_step(d, layer=1, mode=dsa.DSA_MODE_MLI, attend_idx=sel0,
                                    mla_layer=0, n_split=ns, stream_aux=aux)
    sync()
    assert torch.equal(out_ns, out0) and torch.equal(lse_ns, lse0)
    rows = _sample_rows(b.T, 6, 44)
    meta, vis, sc1, s1, f1, K1 = oracle_rows(b, rows, layer=1)
    check_selection(sel1[rows].cpu().numpy(), s1, f1, K1)
    g0 = sel0[rows].cpu().numpy()
    ref, ref_lse = O.sparse_mla(meta, b.q[0], b.kv[0], g0, rows, synth.SM_SCALE)
    check_attention(bf16_to_f64(out_mli[rows]), ref, lse_mli[rows].cpu().numpy(), ref_lse)
    # adjacent-layer selections overlap heavily (keys differ by 0.1 N(0,1) noise)
    a, c = sel0.cpu().numpy(), sel1.cpu().numpy()
    ov = [len(set(a[i][a[i] >= 0]) & set(c[i][c[i] >= 0])) / max(1, (a[i] >= 0).sum())
          for i in range(b.T)]
    print(f"selection overlap mean {np.mean(ov):.3f} min {np.min(ov):.3f}", flush=True)
    assert np.mean(ov) > 0.5
