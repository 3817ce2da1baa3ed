"""Device checks (libdsa_checked.so, built with DSA_DEVICE_CHECKS): each kind
of bad device data planted on its own raises its flag in the device check
word, which dsa_device_check reports as DSA_ERR_DEVICE_CHECK and clears; a
clean step raises none and computes exactly what libdsa.so computes.  The
page tables checked are those of "[SGLang] NSA" (NSAMetadata)."""
import numpy as np
import pytest
import torch

from gpu_common import K, decode_step, dsa, index_scores, sparse_mla, synth, sync, to_device, topk

pytestmark = [pytest.mark.gpu, pytest.mark.device_check_flags]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with dsa.checked() as L:
        assert L.dsa_device_checks_enabled() == 1
    dsa.lib()


def _batch(seed, n_q=(2, 1), L=(5000, 3000)):
    return synth.make_batch(list(n_q), list(L), seed=seed, paging="shuffled", heavy=16,
                            pool_extra_pages=3)


def _flags():
    """Read and clear the check word; also checks the status code agrees."""
    import ctypes
    from sparse_attention_02_amd import binding as B
    v = ctypes.c_uint32(0)
    rc = B.lib().dsa_device_check(ctypes.byref(v), B._stream(None))
    assert rc == (B.DSA_ERR_DEVICE_CHECK if v.value else B.DSA_OK), (rc, v.value)
    return int(v.value)


def test_clean_step_raises_nothing_and_matches_the_normal_build():
    b = _batch(1800)
    d = to_device(b)
    idx0, out0, lse0 = decode_step(d)
    sync()
    with dsa.checked():
        _flags()  # start clean
        idx1, out1, lse1 = decode_step(d)
        sync()
        assert _flags() == 0
        # a long request: scan histogram, collect and final kernels
        b2 = _batch(1801, n_q=(2,), L=(70001,))
        d2 = to_device(b2)
        decode_step(d2)
        sync()
        assert _flags() == 0
    assert torch.equal(idx0, idx1) and torch.equal(out0, out1) and torch.equal(lse0, lse1)


@pytest.mark.parametrize("bad_id", ["negative", "past_pool"])
def test_page_id_outside_the_pool(bad_id):
    b = _batch(1802)
    b.page_table = b.page_table.copy()
    b.page_table[0, 2] = -4 if bad_id == "negative" else b.num_pages + 1
    d = to_device(b)
    with dsa.checked():
        _flags()
        idx, out, lse = decode_step(d)
        sync()
        f = _flags()
        assert f & dsa.DSA_CHECK_PAGE_ID, f
        assert _flags() == 0  # the read cleared the word
    # the same batch through the normal build flags nothing (checks compiled out)
    if not dsa.dsa_device_checks_enabled():
        decode_step(d)
        sync()
        assert dsa.dsa_device_check() == 0


def test_attention_index_entries_out_of_range():
    b = _batch(1803, n_q=(2,), L=(3000,))
    d = to_device(b)
    for bad in (2999, 5000, -5):  # not visible to row 0; past the cache; below -1
        sel = np.full((2, 64), -1, np.int32)
        sel[:, :10] = np.arange(10)
        sel[0, 10] = bad
        with dsa.checked():
            _flags()
            sparse_mla(d, torch.from_numpy(sel).cuda(), k=64, n_split=2)
            sync()
            f = _flags()
        assert f == dsa.DSA_CHECK_INDEX, (bad, f)
    # padding (-1) and visible positions are fine
    sel = np.full((2, 64), -1, np.int32)
    sel[:, :10] = np.arange(10)
    with dsa.checked():
        _flags()
        sparse_mla(d, torch.from_numpy(sel).cuda(), k=64, n_split=2)
        sync()
        assert _flags() == 0


@pytest.mark.parametrize("L", [(30000, 12000), (70001, 3000)])
def test_nan_score_given_to_the_topk(L):
    """Both top-k paths (one pass, and histogram / collect / final)."""
    b = _batch(1804, n_q=(1, 1), L=L)
    d = to_device(b)
    scores, ld = index_scores(d)
    sync()
    scores[0, 17] = float("nan")
    with dsa.checked():
        _flags()
        topk(d, scores, ld)
        sync()
        f = _flags()
    assert f == dsa.DSA_CHECK_NAN_SCORE, f


def test_nan_in_the_indexer_inputs():
    """A NaN key scale makes that key's scores NaN.  (NaN e4m3fn codes in the
    key bytes are outside the contract: the FP8 MFMA does not carry them
    into its sums, and the cache append only writes finite codes.)"""
    b = _batch(1805)
    b.k_scale[0] = b.k_scale[0].copy()
    b.k_scale[0][int(b.page_table[0, 1]), 5] = np.nan
    d = to_device(b)
    with dsa.checked():
        _flags()
        index_scores(d)
        sync()
        f = _flags()
    assert f == dsa.DSA_CHECK_NAN_SCORE, f


def test_metadata_cached_length_past_max_seqlen():
    b = _batch(1806)
    d = to_device(b)
    d.meta.seqlens_k[1] = int(b.max_seqlen_k) + 100  # device value past the host bound
    with dsa.checked():
        _flags()
        index_scores(d)
        sync()
        f = _flags()
    assert f & dsa.DSA_CHECK_METADATA, f


def test_cache_append_to_a_page_outside_the_pool():
    b = _batch(1807, n_q=(2, 1), L=(300, 200))
    b.page_table = b.page_table.copy()
    b.page_table[1, 3] = -1  # request 1's row lands at position 199 (page 3)
    d = to_device(b)
    T = b.T
    k_new = torch.zeros((T, 128), dtype=torch.bfloat16, device="cuda")
    kv_new = torch.zeros((T, 576), dtype=torch.bfloat16, device="cuda")
    with dsa.checked():
        _flags()
        dsa.dsa_cache_append(d.meta, k_new, kv_new, d.k8[0], d.k_scale[0], d.kv[0])
        sync()
        f = _flags()
    assert f == dsa.DSA_CHECK_PAGE_ID, f
