"""Pins for the float64 CPU oracle: each check ties it to something other
than itself (the OCP FP8 definition as implemented by torch, library
routines on special cases, brute force, invariants, the pages' printed
numbers), so that a dropped term, a wrong index or a transposed operand in
the oracle fails at least one of them.  CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import oracle as O
from sparse_attention_02_amd import accounting

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- formats

def test_e4m3_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([O.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(ref[~nan], got[~nan])


def test_e4m3_named_values():
    # OCP 8-bit FP spec, E4M3: max normal 448, min normal 2^-6, min subnormal 2^-9
    assert O.e4m3_decode(0x7E) == 448.0
    assert O.e4m3_decode(0xFE) == -448.0
    assert O.e4m3_decode(0x08) == 2.0 ** -6
    assert O.e4m3_decode(0x01) == 2.0 ** -9
    assert O.e4m3_decode(0x38) == 1.0
    assert O.e4m3_decode(0x80) == 0.0


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, 4000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite values
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([O.bf16_decode(int(b)) for b in bits])
    assert np.array_equal(ref, got)


def test_synth_e4m3_encoder_matches_torch_rounding():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(0, 60, 3000), rng.normal(0, 0.01, 1000),
                        rng.uniform(-448, 448, 1000)]).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([synth.e4m3_encode(v) for v in x], np.uint8)
    assert np.array_equal(ref, got)
    assert synth.e4m3_encode(1000.0) == 0x7E  # saturates


def test_oracle_e4m3_encode_inverts_decode_on_every_code():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert O.e4m3_encode(O.e4m3_decode(c)) == c, hex(c)


def test_oracle_e4m3_encode_matches_torch_cast():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.normal(0, 60, 3000), rng.normal(0, 0.01, 1000),
                        rng.uniform(-448, 448, 1000), rng.normal(0, 2.0 ** -8, 500)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.e4m3_encode(float(v)) for v in x], np.uint8)
    assert np.array_equal(ref, got)


def test_oracle_e4m3_encode_ties_to_even_and_saturates():
    # midpoints between neighbouring codes go to the even code (even mantissa)
    for c in range(0, 0x7E):
        lo, hi = O.e4m3_decode(c), O.e4m3_decode(c + 1)
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # exact in float32
        assert O.e4m3_encode(float(mid)) == (c if c % 2 == 0 else c + 1)
        assert O.e4m3_encode(-float(mid)) == 0x80 | (c if c % 2 == 0 else c + 1)
    assert O.e4m3_encode(2.0 ** -10) == 0x00  # half the smallest subnormal: tie to 0
    assert O.e4m3_encode(448.0) == 0x7E
    assert O.e4m3_encode(460.0) == 0x7E
    assert O.e4m3_encode(1e30) == 0x7E and O.e4m3_encode(-1e30) == 0xFE
    assert O.e4m3_encode(-0.0) == 0x80 and O.e4m3_encode(0.0) == 0x00


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy() \
        .view(np.uint16)


def test_cache_append_places_quantises_and_leaves_other_slots():
    # three requests of 1, 2 and 3 new rows; the third mirrors the worked
    # example of "[SGLang] NSA" (3 rows onto kv_len 10: they are positions 7,
    # 8, 9); the second request's last page id is outside the pool
    rng = np.random.default_rng(5)
    P, num_pages = 64, 12
    L = np.array([70, 129, 10], np.int32)
    n = np.array([1, 2, 3])
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    T = int(cu[-1])
    pt = np.full((3, 3), -1, np.int32)
    pt[0, :2] = [7, 2]
    pt[1, :3] = [5, 9, num_pages + 4]
    pt[2, :1] = [3]
    meta = O.Meta(cu, L, pt)
    k_new = _bf16_bits(rng.normal(0, 1, (T, 128)) * rng.uniform(0.01, 100, (T, 1)))
    k_new[5] = 0  # an all-zero key
    kv_new = rng.integers(0, 1 << 16, (T, 576)).astype(np.uint16)
    k8 = np.full((num_pages, P, 128), 0xA5, np.uint8)
    ks = np.full((num_pages, P), -7.0, np.float32)
    kv = np.full((num_pages, P, 576), 0x1234, np.uint16)
    k8o, kso, kvo = O.cache_append(meta, num_pages, k_new, kv_new, k8, ks, kv)
    expect = {0: (2, 5), 3: (3, 7), 4: (3, 8), 5: (3, 9)}  # row -> (page, slot in page)
    # row 1 (request 1, position 127) lies on page 9; row 2 (position 128) on
    # the page outside the pool, which is not written
    expect[1] = (9, 63)
    touched = np.zeros((num_pages, P), bool)
    for t, (pg, s) in expect.items():
        touched[pg, s] = True
        x = torch.from_numpy(k_new[t].view(np.int16)).view(torch.bfloat16).float().numpy()
        amax = np.float32(np.abs(x).max())
        scale = np.float32(amax / np.float32(448)) if amax > 0 else np.float32(1)
        assert kso[pg, s] == scale
        qv = (x / scale).astype(np.float32)
        ref = torch.from_numpy(qv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(k8o[pg, s], ref)
        if amax > 0:
            assert np.abs(O.e4m3_decode(int(k8o[pg, s][np.argmax(np.abs(x))]))) == 448.0
            deq = np.array([O.e4m3_decode(int(c)) for c in k8o[pg, s]]) * float(scale)
            assert np.all(np.abs(deq - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * float(scale))
        else:
            assert scale == 1 and not k8o[pg, s].any()
        assert np.array_equal(kvo[pg, s], kv_new[t])
    assert np.all(k8o[~touched] == 0xA5) and np.all(kso[~touched] == -7.0)
    assert np.all(kvo[~touched] == 0x1234)


def test_transform_index_spaces():
    rng = np.random.default_rng(21)
    L = np.array([300, 130, 0, 64], np.int32)
    n = np.array([2, 1, 0, 1])
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    pages = (L + 63) // 64
    num_pages = int(pages.sum()) + 2
    perm = rng.permutation(num_pages).astype(np.int32)
    pt = np.full((4, int(pages.max())), -1, np.int32)
    off = 0
    for b, p_ in enumerate(pages):
        pt[b, :p_] = perm[off:off + p_]
        off += p_
    pt[1, 1] = num_pages + 3  # positions 64..127 of request 1 lie on a page outside the pool
    meta = O.Meta(cu, L, pt)
    rows = np.arange(int(cu[-1]), dtype=np.int32)
    k = 8
    idx = np.full((len(rows), k), -1, np.int32)
    req = np.searchsorted(cu, rows, side="right") - 1
    for i, t in enumerate(rows):
        v = meta.visible(int(t))
        sel = np.sort(rng.choice(v, size=min(k - 1, v), replace=False))
        idx[i, :len(sel)] = sel
    logical = O.transform_index(meta, num_pages, 0, idx, rows)
    assert np.array_equal(logical, idx)
    paged = O.transform_index(meta, num_pages, 1, idx, rows)
    inv = np.argsort(perm)  # pool page -> its place in the pool permutation
    for i, t in enumerate(rows):
        b = req[i]
        for j in range(k):
            s_ = idx[i, j]
            if s_ < 0:
                assert paged[i, j] == -1
            elif b == 1 and s_ // 64 == 1:
                assert paged[i, j] == -1  # page outside the pool
            else:
                # the slot's page is the request's page holding the position
                # (recovered through the pool permutation), same offset in it
                pg, o = divmod(int(paged[i, j]), 64)
                place = inv[pg] - int(pages[:b].sum())
                assert place == s_ // 64 and o == s_ % 64
    ident = O.Meta(cu, L, np.arange(pt.size, dtype=np.int32).reshape(pt.shape) * 0
                   + np.arange(pt.shape[1], dtype=np.int32)[None, :])
    assert np.array_equal(O.transform_index(ident, pt.shape[1], 1, idx, rows), idx)
    starts = np.concatenate([[0], np.cumsum(L)[:-1]]).astype(np.int32)
    rag = O.transform_index(meta, num_pages, 2, idx, rows, starts)
    live = idx >= 0
    assert np.array_equal(rag[live] - starts[req][:, None].repeat(k, 1)[live], idx[live])
    assert np.all(rag[~live] == -1) and np.all(rag[live] < int(L.sum()))


def test_layer_schedule_indexcache_and_mli():
    # every layer keeps an indexer, no MLI: each layer attends its own selection
    pr, at = O.layer_schedule(5, 1, False)
    assert pr.tolist() == [0, 1, 2, 3, 4] and at.tolist() == [0, 1, 2, 3, 4]
    # MLI alone (the two-stream step): layer l attends layer l-1's selection
    pr, at = O.layer_schedule(5, 1, True)
    assert pr.tolist() == [0, 1, 2, 3, 4] and at.tolist() == [0, 0, 1, 2, 3]
    # IndexCache at 1/4: layers 0 and 4 keep an indexer, the rest reuse
    pr, at = O.layer_schedule(8, 4, False)
    assert pr.tolist() == [0, -1, -1, -1, 1, -1, -1, -1]
    assert at.tolist() == [0, 0, 0, 0, 1, 1, 1, 1]
    # composed: layer 4 attends selection 0 while making selection 1
    pr, at = O.layer_schedule(9, 4, True)
    assert at.tolist() == [0, 0, 0, 0, 0, 1, 1, 1, 1]
    for n, r in ((12, 1), (12, 2), (12, 4), (13, 8), (3, 32)):
        for mli in (False, True):
            pr, at = O.layer_schedule(n, r, mli)
            # a fraction 1/r of the layers keeps an indexer
            assert (pr >= 0).sum() == -(-n // r)
            # no layer reads a selection made after it; every one is made
            made_at = {int(j): l for l, j in enumerate(pr) if j >= 0}
            assert all(made_at[int(j)] <= l for l, j in enumerate(at))
            # with MLI no indexer layer but the first waits for its own scan
            if mli:
                assert all(at[l] != pr[l] for l in range(1, n) if pr[l] >= 0)


# ------------------------------------------------------------- visibility

def test_visibility_worked_example():
    """An extend of 3 rows on a 10-token cache sees 8, 9, 10 tokens."""
    with open(os.path.join(GOLDEN, "p2_visibility.txt")) as f:
        line = [ln for ln in f if ln.strip() and not ln.startswith("#")][0]
    n, kv, *vis = map(int, line.split())
    meta = O.Meta([0, n], [kv], np.zeros((1, 1), np.int32))
    assert [meta.visible(t) for t in range(n)] == vis


# ----------------------------------------------------------- index score

def _tiny_index_batch(rng, H, D, L, n_q=1, pages=None):
    P = 64
    npages = (L + P - 1) // P
    pt = np.arange(npages, dtype=np.int32) if pages is None else pages
    q8 = rng.integers(0, 256, (n_q, H, D)).astype(np.uint8)
    q8[(q8 & 0x7F) == 0x7F] = 0x10  # no NaN codes
    k8 = rng.integers(0, 256, (npages, P, D)).astype(np.uint8)
    k8[(k8 & 0x7F) == 0x7F] = 0x21
    q_scale = rng.uniform(0.5, 2.0, n_q).astype(np.float32)
    k_scale = rng.uniform(0.5, 2.0, (npages, P)).astype(np.float32)
    w = rng.uniform(0, 1, (n_q, H)).astype(np.float32)
    meta = O.Meta([0, n_q], [L], pt.reshape(1, -1))
    return meta, q8, q_scale, w, k8, k_scale


def _dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


def test_index_score_single_head_is_relu_dot():
    """H = 1, w = 1: the score is ReLU of the textbook dot product."""
    rng = np.random.default_rng(2)
    meta, q8, qs, w, k8, ks = _tiny_index_batch(rng, 1, 128, 200)
    w[:] = 1.0
    got = O.index_score(meta, q8, qs, w, k8, ks, [0])[0, :200]
    q = _dec(q8[0, 0]) * float(qs[0])
    keys = _dec(k8.reshape(-1, 128)[:200]) * ks.reshape(-1)[:200, None].astype(np.float64)
    ref = np.maximum(keys @ q, 0.0)
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-12)
    assert (ref == 0).any() and (ref > 0).any()


@pytest.mark.parametrize("head", [0, 17, 63])
def test_index_score_one_hot_weight_isolates_head(head):
    """w = e_head: the score is ReLU(q_head . k); catches a wrong head index."""
    rng = np.random.default_rng(3 + head)
    meta, q8, qs, w, k8, ks = _tiny_index_batch(rng, 64, 128, 130)
    w[:] = 0.0
    w[0, head] = 1.0
    got = O.index_score(meta, q8, qs, w, k8, ks, [0])[0, :130]
    q = _dec(q8[0, head]) * float(qs[0])
    keys = _dec(k8.reshape(-1, 128)[:130]) * ks.reshape(-1)[:130, None].astype(np.float64)
    assert np.allclose(got, np.maximum(keys @ q, 0.0), rtol=1e-13, atol=1e-12)


def test_index_score_relu_per_head_not_after_sum():
    """Scores are additive in w (ReLU acts per head, before the weighted sum),
    and a head whose dot product is negative contributes nothing."""
    rng = np.random.default_rng(4)
    meta, q8, qs, w, k8, ks = _tiny_index_batch(rng, 64, 128, 100)
    w1 = rng.uniform(0, 1, w.shape).astype(np.float32)
    w2 = rng.uniform(0, 1, w.shape).astype(np.float32)
    w12 = (w1.astype(np.float64) + w2).astype(np.float32)
    exact = (w12.astype(np.float64) == w1.astype(np.float64) + w2)
    w1, w2, w12 = np.where(exact, w1, 0), np.where(exact, w2, 0), np.where(exact, w12, 0)
    a = O.index_score(meta, q8, qs, w1, k8, ks, [0])[0, :100]
    b = O.index_score(meta, q8, qs, w2, k8, ks, [0])[0, :100]
    c = O.index_score(meta, q8, qs, w12, k8, ks, [0])[0, :100]
    assert np.allclose(a + b, c, rtol=1e-12)
    # q = -k on every head: all dot products <= 0 -> score 0
    k8n = k8.copy()
    q8n = np.broadcast_to((k8[0, 5] ^ 0x80)[None, None, :], q8.shape).copy()
    s = O.index_score(meta, q8n, qs, w1, k8n, ks, [0])[0]
    assert s[5] == 0.0
    # and a negative w flips sign only through the weight
    neg = O.index_score(meta, q8, qs, -w1, k8, ks, [0])[0, :100]
    assert np.array_equal(neg, -a)


def test_index_score_scales_factor_out():
    rng = np.random.default_rng(5)
    meta, q8, qs, w, k8, ks = _tiny_index_batch(rng, 64, 128, 90)
    a = O.index_score(meta, q8, qs, w, k8, ks, [0])[0, :90]
    b = O.index_score(meta, q8, qs * 2, w, k8, ks * 4, [0])[0, :90]
    assert np.allclose(b, 8 * a, rtol=1e-13)


def test_index_score_page_permutation_invariant_bitwise():
    rng = np.random.default_rng(6)
    L, P = 64 * 5 + 17, 64
    meta, q8, qs, w, k8, ks = _tiny_index_batch(rng, 64, 128, L)
    a = O.index_score(meta, q8, qs, w, k8, ks, [0])[0, :L]
    perm = rng.permutation(k8.shape[0]).astype(np.int32)  # logical page i -> physical perm[i]
    k8p = np.empty_like(k8)
    ksp = np.empty_like(ks)
    k8p[perm] = k8
    ksp[perm] = ks
    meta2 = O.Meta([0, 1], [L], perm.reshape(1, -1))
    b = O.index_score(meta2, q8, qs, w, k8p, ksp, [0])[0, :L]
    assert np.array_equal(a, b)


def test_index_score_mtp_rows_visibility():
    """Row j of a 2-row request sees L-1+j tokens: changing the last token's key
    leaves row 0's scores unchanged and its score is not written for row 0."""
    b = synth.make_batch([2], [300], seed=11, with_mla=False)
    meta = O.Meta.of(b)
    s1 = O.index_score(meta, b.q8, b.q_scale, b.w, b.k8[0], b.k_scale[0], [0, 1])
    assert np.isnan(s1[0, 299]) and not np.isnan(s1[1, 299])
    k8 = b.k8[0].copy().reshape(-1, 128)
    slot = int(b.page_table[0, 299 // 64]) * 64 + 299 % 64
    k8[slot] = 0x38  # every dim 1.0
    s2 = O.index_score(meta, b.q8, b.q_scale, b.w, k8.reshape(b.k8[0].shape), b.k_scale[0], [0, 1])
    assert np.array_equal(s1[0, :299], s2[0, :299])
    assert s1[1, 299] != s2[1, 299]


# -------------------------------------------------------------------- top-k

def _brute_selected(scores, K):
    n = len(scores)
    out = set()
    for s in range(n):
        better = sum(1 for s2 in range(n) if scores[s2] > scores[s] or
                     (scores[s2] == scores[s] and s2 < s))
        if better < K:
            out.add(s)
    return out


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_rank(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 90))
    k = int(rng.integers(1, 40))
    vals = rng.integers(0, 12, n).astype(np.float64) * 0.25  # many ties
    sel, flags, kth, K = O.topk(vals[None, :], [n], k)
    K = int(K[0])
    assert K == min(n, k)
    assert set(sel[0, :K].tolist()) == _brute_selected(vals.tolist(), K)
    assert (sel[0, K:] == -1).all()


def test_topk_matches_numpy_stable_sort():
    rng = np.random.default_rng(7)
    vals = np.round(rng.normal(size=5000), 2)
    k = 700
    sel, _, kth, K = O.topk(vals[None, :], [5000], k)
    order = np.lexsort((np.arange(5000), -vals))[:k]
    assert sel[0].tolist() == order.tolist()
    assert kth[0] == vals[order[-1]]


def test_topk_all_equal_and_short_rows():
    sel, flags, kth, K = O.topk(np.full((1, 50), 3.0), [50], 10)
    assert sel[0].tolist() == list(range(10))
    assert flags[0].all()  # every position ties with the k-th
    sel, flags, kth, K = O.topk(np.arange(7.0)[None, :], [7], 10)
    assert sorted(sel[0, :7].tolist()) == list(range(7)) and (sel[0, 7:] == -1).all()
    sel, flags, kth, K = O.topk(np.arange(7.0)[None, :], [0], 4)
    assert (sel == -1).all() and K[0] == 0


def test_topk_tie_band_flags():
    vals = np.array([10.0, 5.0, 5.004, 4.9999, 5.0, 1.0])
    sel, flags, kth, K = O.topk(vals[None, :], [6], 3)
    assert kth[0] == 5.0 and sel[0].tolist() == [0, 2, 1]
    # band 1e-3 * 5 = 0.005 around 5.0: positions 1, 2, 3, 4
    assert flags[0].tolist() == [0, 1, 1, 1, 1, 0]


def _contract_case():
    """Twelve visible positions (two rows' worth of columns, ld 14), k = 5.
    The top five are 0, 7, 2, 11, 5; the k-th score is 5.0004, so the 1e-3
    band holds positions 5 (5.0004), 4 (5.0) and 10 (4.9998)."""
    vals = np.array([9.0, 1.0, 7.0, 3.0, 5.0, 5.0004, 2.0, 8.0, 4.0, 0.5, 4.9998, 6.0, 10.0, 11.0])
    sel, flags, kth, K = O.topk(vals[None, :], [12], 5)
    assert sel[0].tolist() == [0, 7, 2, 11, 5] and K[0] == 5 and kth[0] == 5.0004
    assert np.nonzero(flags[0])[0].tolist() == [4, 5, 10]
    return sel[0], flags[0], int(K[0])


@pytest.mark.parametrize("gpu, ok", [
    ([11, 5, 2, 7, 0], True),              # the oracle's set, another order
    ([0, 7, 2, 11, 5, -1, -1], True),      # with -1 padding
    ([0, 7, 2, 11, 4], True),              # swap inside the tie band
    ([10, 7, 2, 11, 0], True),             # the other band member
    ([0, 7, 2, 4, 5], False),              # 11 (outside the band) missing
    ([0, 7, 2, 11, 8], False),             # 8 (outside the band) extra
    ([0, 7, 2, 11, 11], False),            # duplicate
    ([0, 7, 2, 11, 13], False),            # position past the row's 12 visible
    ([0, 7, 2, 11], False),                # short count
    ([0, 7, 2, 11, 5, 4], False),          # one too many
    ([0, 7, 2, 11, -5], False),            # an entry that is neither a position nor -1
])
def test_selection_check_rejects_known_bad_selections(gpu, ok):
    """The index contract of the DSA bullet of "MTP and sparse attention: NSA
    and DSA" (each row keeps its top 2048) with the 1e-3 tie band: the checker
    accepts the oracle's set in any order and swaps inside the band, and
    reports every planted defect."""
    sel, flags, K = _contract_case()
    probs = O.selection_check(np.array(gpu, np.int32), sel, flags, K)
    assert (probs == []) == ok, probs


def test_index_score_pages_outside_pool_score_minus_inf():
    """A page id outside the pool (negative, or >= num_pages) names no key:
    every visible position on it scores -inf; all other scores are unchanged."""
    b = synth.make_batch([2], [300], seed=21, paging="shuffled", with_mla=False)
    meta = O.Meta.of(b)
    good = O.index_score(meta, b.q8, b.q_scale, b.w, b.k8[0], b.k_scale[0], [0, 1])
    pt = b.page_table.copy()
    pt[0, 1] = -1
    pt[0, 3] = b.num_pages
    bad = O.index_score(O.Meta(b.cu_seqlens_q, b.seqlens_k, pt), b.q8, b.q_scale, b.w, b.k8[0],
                        b.k_scale[0], [0, 1])
    invalid = np.zeros(bad.shape[1], bool)
    invalid[64:128] = invalid[192:256] = True
    for i, v in enumerate([299, 300]):
        assert np.all(np.isneginf(bad[i, :v][invalid[:v]]))
        assert np.array_equal(bad[i, :v][~invalid[:v]], good[i, :v][~invalid[:v]])
        assert np.all(np.isfinite(good[i, :v]))
    # the top-k ranks them last: a row with fewer keyed positions than k
    # takes every keyed one, then the -inf positions by position
    sel, flags, kth, K = O.topk(np.nan_to_num(bad, nan=-np.inf), [299, 300], 200)
    keyed = set(np.nonzero(~invalid[:300])[0].tolist())
    assert keyed - {299} <= set(sel[0, :K[0]].tolist())


# ---------------------------------------------------------------- attention

def _mla_case(rng, L, n_q=1, scale=1.0, pages=None):
    b = synth.make_batch([n_q], [L], seed=int(rng.integers(1 << 30)), paging="shuffled",
                         mla_scale=scale)
    return b


def _torch_attention(q, keys, sm):
    """softmax attention with torch float64 library calls."""
    qt = torch.from_numpy(q)
    kt = torch.from_numpy(keys)
    z = (qt @ kt.T) * sm
    p = torch.softmax(z, dim=-1)
    o = p @ kt[:, :512]
    lse = torch.logsumexp(z, dim=-1)
    return o.numpy(), lse.numpy()


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(
        torch.float64).numpy()


def _logical_rows(b, layer=0):
    """latent rows of request 0 in logical order (float64)."""
    L = int(b.seqlens_k[0])
    slots = b.page_table[0, np.arange(L) // 64].astype(np.int64) * 64 + np.arange(L) % 64
    return _bf16(b.kv[layer].reshape(-1, 576)[slots])


def test_dense_mla_matches_torch_softmax():
    rng = np.random.default_rng(8)
    b = _mla_case(rng, 300, n_q=2, scale=1.0)
    meta = O.Meta.of(b)
    out, lse = O.dense_mla(meta, b.q[0], b.kv[0], [0, 1], synth.SM_SCALE)
    keys = _logical_rows(b)
    for j in range(2):
        v = 300 - 2 + 1 + j
        ro, rl = _torch_attention(_bf16(b.q[0][j]), keys[:v], synth.SM_SCALE)
        assert np.allclose(out[j], ro, rtol=1e-10, atol=1e-12)
        assert np.allclose(lse[j], rl, rtol=1e-12)


def test_sparse_mla_with_k_at_least_context_is_dense():
    rng = np.random.default_rng(9)
    b = _mla_case(rng, 250, n_q=2, scale=1.0)
    meta = O.Meta.of(b)
    sc = O.index_score(meta, b.q8, b.q_scale, b.w, b.k8[0], b.k_scale[0], [0, 1])
    sel, _, _, K = O.topk(np.nan_to_num(sc, nan=-np.inf), [249, 250], 2048)
    so, sl = O.sparse_mla(meta, b.q[0], b.kv[0], sel, [0, 1], synth.SM_SCALE)
    do, dl = O.dense_mla(meta, b.q[0], b.kv[0], [0, 1], synth.SM_SCALE)
    assert np.allclose(so, do, rtol=1e-12, atol=1e-15) and np.allclose(sl, dl, rtol=1e-13)


def test_sparse_mla_special_cases():
    rng = np.random.default_rng(10)
    b = _mla_case(rng, 200, scale=1.0)
    meta = O.Meta.of(b)
    keys = _logical_rows(b)
    # one selected token: the output is that token's 512 latent dims
    idx = np.full((1, 16), -1, np.int32)
    idx[0, 3] = 77
    o, l = O.sparse_mla(meta, b.q[0], b.kv[0], idx, [0], synth.SM_SCALE)
    assert np.allclose(o[0], np.broadcast_to(keys[77, :512], o[0].shape), rtol=0, atol=0)
    # q = 0: uniform weights, the mean of the selected rows, lse = ln n
    sel = np.array([[5, 9, 150, 33, -1, 199]], np.int32)
    q0 = np.zeros_like(b.q[0])
    o, l = O.sparse_mla(meta, q0, b.kv[0], sel, [0], synth.SM_SCALE)
    mean = keys[[5, 9, 150, 33, 199], :512].mean(axis=0)
    assert np.allclose(o[0], mean[None, :], rtol=1e-13, atol=1e-15)
    assert np.allclose(l[0], math.log(5), rtol=1e-14)
    # all selected rows equal: output is that row
    kv = b.kv[0].copy().reshape(-1, 576)
    slots = [int(b.page_table[0, s // 64]) * 64 + s % 64 for s in (5, 9, 150)]
    kv[slots] = kv[slots[0]]
    o, l = O.sparse_mla(meta, b.q[0], kv.reshape(b.kv[0].shape), sel[:, :3], [0], synth.SM_SCALE)
    assert np.allclose(o[0], np.broadcast_to(keys[5, :512], o[0].shape), rtol=1e-13, atol=1e-15)
    # empty selection: zeros and -inf
    o, l = O.sparse_mla(meta, b.q[0], b.kv[0], np.full((1, 8), -1, np.int32), [0], synth.SM_SCALE)
    assert (o == 0).all() and np.isneginf(l).all()


def test_sparse_mla_page_permutation_invariant():
    rng = np.random.default_rng(12)
    b = _mla_case(rng, 330, scale=1.0)
    meta = O.Meta.of(b)
    sel = rng.choice(330, 100, replace=False).astype(np.int32)[None, :]
    o1, l1 = O.sparse_mla(meta, b.q[0], b.kv[0], sel, [0], synth.SM_SCALE)
    n = b.num_pages
    perm = rng.permutation(n).astype(np.int32)  # old physical page p -> perm[p]
    kv2 = np.empty_like(b.kv[0])
    kv2[perm] = b.kv[0]
    pt2 = perm[b.page_table]
    o2, l2 = O.sparse_mla(O.Meta(b.cu_seqlens_q, b.seqlens_k, pt2), b.q[0], kv2, sel, [0],
                          synth.SM_SCALE)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_sparse_mla_ignores_positions_outside_visible_range():
    rng = np.random.default_rng(13)
    b = _mla_case(rng, 100, n_q=2, scale=1.0)
    meta = O.Meta.of(b)
    sel = np.array([[1, 2, 99], [1, 2, 99]], np.int32)  # row 0 sees 99 tokens
    o, l = O.sparse_mla(meta, b.q[0], b.kv[0], sel, [0, 1], synth.SM_SCALE)
    o0, l0 = O.sparse_mla(meta, b.q[0], b.kv[0], sel[:, :2], [0, 1], synth.SM_SCALE)
    assert np.array_equal(o[0], o0[0]) and not np.array_equal(o[1], o0[1])


def test_sparse_mla_leaves_out_pages_outside_pool():
    """Selected positions on a page id outside the pool have no latent row:
    the attention over them equals the attention over the rest, bit for bit."""
    rng = np.random.default_rng(14)
    b = _mla_case(rng, 330, scale=1.0)
    pt = b.page_table.copy()
    pt[0, 2] = -3
    pt[0, 4] = b.num_pages + 9
    meta_bad = O.Meta(b.cu_seqlens_q, b.seqlens_k, pt)
    sel = np.array([[5, 130, 140, 200, 260, 300, 329]], np.int32)
    keep = np.array([[5, 200, 329, -1, -1, -1, -1]], np.int32)
    o1, l1 = O.sparse_mla(meta_bad, b.q[0], b.kv[0], sel, [0], synth.SM_SCALE)
    o2, l2 = O.sparse_mla(O.Meta.of(b), b.q[0], b.kv[0], keep, [0], synth.SM_SCALE)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    d1, dl1 = O.dense_mla(meta_bad, b.q[0], b.kv[0], [0], synth.SM_SCALE)
    live = np.array([s for s in range(330) if s // 64 not in (2, 4)], np.int32)[None, :]
    d2, dl2 = O.sparse_mla(O.Meta.of(b), b.q[0], b.kv[0], live, [0], synth.SM_SCALE)
    assert np.array_equal(d1, d2) and np.array_equal(dl1, dl2)


# ---------------------------------------------------------------- accounting

def test_accounting_reproduces_printed_table():
    """The per-pair costs and the decode columns of the printed DSA-versus-
    dense table of "MTP and sparse attention: NSA and DSA" follow from the
    library's per-row model (one query row over L cached tokens; dense =
    attention over every visible token, no indexer).  The prefill columns
    follow the page's own counting: L*L/2 indexer pairs, L*min(L, k)
    absorbed-attention pairs, and L*L/2 expanded-attention pairs for dense."""
    with open(os.path.join(GOLDEN, "p1_dsa_accounting.txt")) as f:
        lines = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    pair = lines[0]
    assert pair[0] == "pair"
    assert round(accounting.attention_pair_flops() / 1e3) == int(pair[1])
    assert round(accounting.indexer_pair_flops() / 1e3) == int(pair[2])
    assert round(100 * accounting.indexer_token_bytes() /
                 accounting.latent_token_bytes()) == int(pair[3])
    for row in lines[1:]:
        L = int(row[0]) * 1024
        vals = list(map(float, row[1:]))
        sparse = accounting.batch_work([L], [1])  # one query row seeing L tokens
        dense = accounting.batch_work([L], [1], dense=True)
        assert sparse["rows"] == dense["rows"] == 1
        pairs, sel = L * L / 2, min(L, accounting.TOPK)
        pre_dense = pairs * accounting.expanded_pair_flops()
        pre_dsa = pairs * accounting.indexer_pair_flops() + L * sel * accounting.attention_pair_flops()
        got = [
            round(dense["flops"] / 1e9, 2), round(sparse["flops"] / 1e9, 2),
            round(dense["flops"] / sparse["flops"], 1),
            round(dense["cache_read_bytes"] / 2 ** 20, 1),
            round(sparse["cache_read_bytes"] / 2 ** 20, 1),
            round(dense["cache_read_bytes"] / sparse["cache_read_bytes"], 1),
            round(pre_dense / 1e12, 1), round(pre_dsa / 1e12, 1), round(pre_dense / pre_dsa, 1),
        ]
        assert got == vals, (L, got, vals)


def test_batch_work_headline_workload():
    w = accounting.batch_work([131072] * 64, [2] * 64)
    assert w["rows"] == 128
    assert w["indexer_bytes"] == 64 * (131072 * 132 + 4 * 2048) + 128 * (8192 + 4 + 256)
    assert w["indexer_flops"] == sum(16384 * v for v in [131071, 131072] * 64)
    assert w["mla_flops"] == 128 * 2048 * 278528
    assert w["bytes"] == 1447657984  # the figure the bench divides by


# ------------------------------------------- masked MHA (expanded multi-head form)

def _mha_inputs(rng, T, H=128, integral=False):
    """q_nope, q_rope, w_uk, w_uv as bf16 bits.  integral: q_nope and w_uk in
    {-1, 0, 1}, so that w_uk^T q_nope is an integer of magnitude <= 128,
    exact in bf16."""
    if integral:
        qn = rng.integers(-1, 2, size=(T, H, 128)).astype(np.float32)
        wk = rng.integers(-1, 2, size=(H, 128, 512)).astype(np.float32)
    else:
        qn = rng.standard_normal((T, H, 128)).astype(np.float32)
        wk = (rng.standard_normal((H, 128, 512)) / math.sqrt(512)).astype(np.float32)
    qr = rng.standard_normal((T, H, 64)).astype(np.float32)
    wv = (rng.standard_normal((H, 128, 512)) / math.sqrt(512)).astype(np.float32)
    return _bf16_bits(qn), _bf16_bits(qr), _bf16_bits(wk), _bf16_bits(wv)


@pytest.mark.parametrize("with_idx", [False, True])
def test_masked_mha_is_the_up_projected_absorbed_attention(with_idx):
    """The expanded form against the absorbed one (the oracle's latent
    attention, pinned above): with q_latent(h) = W_UK(h)^T q_nope(h) both
    give the same scores, so the expanded output is W_UV(h) times the
    absorbed 512-dim output and the lse is the same -- a transposed weight,
    a dropped rope term or a wrong head fails it."""
    rng = np.random.default_rng(30)
    b = _mla_case(rng, 300, n_q=2, scale=0.05)
    meta = O.Meta.of(b)
    qn, qr, wk, wv = _mha_inputs(rng, 2, integral=True)
    q_lat = np.einsum("hdc,thd->thc", _bf16(wk), _bf16(qn))
    assert np.all(q_lat == np.round(q_lat)) and np.abs(q_lat).max() <= 128
    q_abs = np.concatenate([_bf16_bits(q_lat), qr], axis=-1)
    assert np.array_equal(_bf16(q_abs[..., :512]), q_lat)
    idx = None
    if with_idx:
        idx = np.full((2, 96), -1, np.int32)
        idx[0, :80] = rng.choice(299, 80, replace=False)
        idx[1, :90] = rng.choice(300, 90, replace=False)
        lo, ll = O.sparse_mla(meta, q_abs, b.kv[0], idx, [0, 1], synth.SM_SCALE)
    else:
        lo, ll = O.dense_mla(meta, q_abs, b.kv[0], [0, 1], synth.SM_SCALE)
    eo, el = O.masked_mha(meta, qn, qr, wk, wv, b.kv[0], idx, [0, 1], synth.SM_SCALE)
    ref = np.einsum("hdc,thc->thd", _bf16(wv), lo)
    assert np.allclose(eo, ref, rtol=1e-9, atol=1e-12)
    assert np.allclose(el, ll, rtol=1e-12, atol=1e-12)


def test_masked_mha_matches_torch_attention():
    """Random (non-integral) weights: the expanded keys and values by torch
    float64 matmuls, then torch's softmax and logsumexp."""
    rng = np.random.default_rng(31)
    b = _mla_case(rng, 140, n_q=1, scale=0.5)
    meta = O.Meta.of(b)
    qn, qr, wk, wv = _mha_inputs(rng, 1)
    eo, el = O.masked_mha(meta, qn, qr, wk, wv, b.kv[0], None, [0], synth.SM_SCALE)
    keys = torch.from_numpy(_logical_rows(b))              # [140, 576]
    kn = torch.einsum("hdc,sc->hsd", torch.from_numpy(_bf16(wk)), keys[:, :512])
    vn = torch.einsum("hdc,sc->hsd", torch.from_numpy(_bf16(wv)), keys[:, :512])
    z = (torch.einsum("hd,hsd->hs", torch.from_numpy(_bf16(qn[0])), kn) +
         torch.from_numpy(_bf16(qr[0])) @ keys[:, 512:].T) * synth.SM_SCALE
    o = torch.einsum("hs,hsd->hd", torch.softmax(z, dim=-1), vn)
    assert np.allclose(eo[0], o.numpy(), rtol=1e-10, atol=1e-13)
    assert np.allclose(el[0], torch.logsumexp(z, dim=-1).numpy(), rtol=1e-12)


def test_masked_mha_special_cases():
    rng = np.random.default_rng(32)
    b = _mla_case(rng, 200, scale=0.5)
    meta = O.Meta.of(b)
    qn, qr, wk, wv = _mha_inputs(rng, 1)
    keys = _logical_rows(b)
    W = _bf16(wv)
    # one selected position: its up-projected value row, for every head
    idx = np.full((1, 16), -1, np.int32)
    idx[0, 5] = 77
    o, l = O.masked_mha(meta, qn, qr, wk, wv, b.kv[0], idx, [0], synth.SM_SCALE)
    assert np.allclose(o[0], W @ keys[77, :512], rtol=1e-12, atol=1e-14)
    # zero queries: uniform weights, the mean of the value rows, lse = ln n
    sel = np.array([[5, 9, 150, 33, -1, 199, 250]], np.int32)  # 250 is past the row
    z = np.zeros_like(qn), np.zeros_like(qr)
    o, l = O.masked_mha(meta, z[0], z[1], wk, wv, b.kv[0], sel, [0], synth.SM_SCALE)
    mean = W @ keys[[5, 9, 150, 33, 199], :512].mean(axis=0)
    assert np.allclose(o[0], mean, rtol=1e-12, atol=1e-14)
    assert np.allclose(l[0], math.log(5), rtol=1e-14)
    # a position the row does not attend leaves the result alone
    kv = b.kv[0].copy().reshape(-1, 576)
    kv[int(b.page_table[0, 100 // 64]) * 64 + 100 % 64] = kv[0]
    o1, l1 = O.masked_mha(meta, qn, qr, wk, wv, b.kv[0], sel[:, :4], [0], synth.SM_SCALE)
    o2, l2 = O.masked_mha(meta, qn, qr, wk, wv, kv.reshape(b.kv[0].shape), sel[:, :4], [0],
                          synth.SM_SCALE)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # every visible position listed equals no list (plain causal)
    full = np.arange(200, dtype=np.int32)[None, :]
    o1, l1 = O.masked_mha(meta, qn, qr, wk, wv, b.kv[0], full, [0], synth.SM_SCALE)
    o2, l2 = O.masked_mha(meta, qn, qr, wk, wv, b.kv[0], None, [0], synth.SM_SCALE)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # nothing attended: zeros and -inf
    o, l = O.masked_mha(meta, qn, qr, wk, wv, b.kv[0], np.full((1, 4), -1, np.int32), [0],
                        synth.SM_SCALE)
    assert (o == 0).all() and np.isneginf(l).all()


def test_masked_mha_page_permutation_invariant():
    rng = np.random.default_rng(33)
    b = _mla_case(rng, 330, scale=0.5)
    meta = O.Meta.of(b)
    qn, qr, wk, wv = _mha_inputs(rng, 1)
    o1, l1 = O.masked_mha(meta, qn, qr, wk, wv, b.kv[0], None, [0], synth.SM_SCALE)
    perm = rng.permutation(b.num_pages).astype(np.int32)
    kv2 = np.empty_like(b.kv[0])
    kv2[perm] = b.kv[0]
    o2, l2 = O.masked_mha(O.Meta(b.cu_seqlens_q, b.seqlens_k, perm[b.page_table]), qn, qr, wk,
                          wv, kv2, None, [0], synth.SM_SCALE)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
