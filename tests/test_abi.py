"""CPU-only checks of the C ABI: the library loads, exports every function
include/dsa.h declares, and rejects bad host arguments before it touches
the device (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

from sparse_attention_02_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
HEADERS = sorted(os.path.join(ROOT, "include", h) for h in os.listdir(os.path.join(ROOT, "include"))
                 if h.endswith(".h"))


def _declared(headers=None):
    names = set()
    for h in headers or HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(B._LIB_PATH):
        from sparse_attention_02_amd import build
        build.build()
    return B.lib()


def test_header_declares_the_four_entry_points():
    d = _declared([HEADER])
    for name in ("dsa_index_score", "dsa_topk", "dsa_sparse_mla_decode", "dsa_decode_step"):
        assert name in d


def test_library_exports_every_declared_symbol(L):
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(B.EXPORTS) == _declared()


def _batch(B_=2, T=4, max_q=2, max_seqlen_k=300, max_pages=5, num_pages=10, ptrs=True):
    fake = 0x1000 if ptrs else None
    return B.dsa_batch_t(B_, T, max_q, max_seqlen_k, max_pages, num_pages, fake, fake, fake)


def _err(L):
    return L.dsa_last_error().decode()


def test_bench_kernels_refuse_bad_arguments(L):
    """The measurement kernels check their host arguments like the path's
    entry points (nothing launched here)."""
    sink = 0x1000
    assert L.dsa_bench_stream_read(0x1008, 64, sink, None) == B.DSA_ERR_INVALID_ARG
    assert L.dsa_bench_stream_read(0x1000, 63, sink, None) == B.DSA_ERR_INVALID_ARG
    assert L.dsa_bench_stream_read(0x1000, 0, sink, None) == B.DSA_OK
    assert L.dsa_bench_key_stream_read(0x1000, 10, 0x2000, 2, 1, 0x3000, 300, sink, None) == \
        B.DSA_ERR_INVALID_ARG  # 1 page per row cannot hold 300 tokens
    assert L.dsa_bench_key_stream_read(0x1000, 10, 0x2000, 0, 5, 0x3000, 300, sink, None) == B.DSA_OK


def test_status_strings(L):
    assert L.dsa_status_string(0) == b"ok"
    assert L.dsa_status_string(3) == b"workspace too small"
    assert L.dsa_status_string(B.DSA_ERR_DEVICE_CHECK) == b"device check failed"


def test_device_check_calls_in_both_builds(L):
    """libdsa.so compiles the checks out: the query returns DSA_OK with no
    flags and touches no device; libdsa_checked.so exports the same symbols
    and reports that its checks are on."""
    import ctypes as C
    assert L.dsa_device_checks_enabled() == 0
    v = C.c_uint32(7)
    assert L.dsa_device_check(C.byref(v), None) == B.DSA_OK and v.value == 0
    if not os.path.exists(B._LIB_CHECKED_PATH):
        from sparse_attention_02_amd import build
        build.build()
    Lc = B._load(B._LIB_CHECKED_PATH)
    assert Lc.dsa_device_checks_enabled() == 1
    assert all(hasattr(Lc, n) for n in _declared())


def test_batch_validation(L):
    P = 0x1000
    rc = L.dsa_topk(None, P, 300, 16, P, P, 1 << 30, None)
    assert rc == B.DSA_ERR_INVALID_ARG and "batch" in _err(L)
    b = _batch(max_pages=4)  # 4 * 64 < 300
    assert L.dsa_topk(ctypes.byref(b), P, 300, 16, P, P, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    b = _batch(max_q=5)  # max_q > T
    assert L.dsa_topk(ctypes.byref(b), P, 300, 16, P, P, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    b = _batch(ptrs=False)
    assert L.dsa_topk(ctypes.byref(b), P, 300, 16, P, P, 1 << 30, None) == B.DSA_ERR_INVALID_ARG


def test_topk_argument_checks(L):
    P = 0x1000
    b = _batch()
    for k in (0, -3, 8193):
        assert L.dsa_topk(ctypes.byref(b), P, 300, k, P, P, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    assert L.dsa_topk(ctypes.byref(b), P, 299, 16, P, P, 1 << 30, None) == B.DSA_ERR_INVALID_ARG
    need = L.dsa_workspace_size(B.DSA_OP_TOPK, ctypes.byref(b), 16, 0)
    assert need > 0
    rc = L.dsa_topk(ctypes.byref(b), P, 300, 16, P, P, need - 1, None)
    assert rc == B.DSA_ERR_WORKSPACE
    assert L.dsa_topk(ctypes.byref(b), P, 300, 16, None, P, need, None) == B.DSA_ERR_INVALID_ARG
    # rows longer than the final pass's bitmap (393216 positions) are sorted
    # in LDS, which holds 4096 selections: a larger k is refused up front
    long = _batch(max_seqlen_k=400000, max_pages=6250)
    need = L.dsa_workspace_size(B.DSA_OP_TOPK, ctypes.byref(long), 4097, 0)
    assert L.dsa_topk(ctypes.byref(long), P, 400000, 4097, P, P, need, None) == \
        B.DSA_ERR_UNSUPPORTED
    assert "4096" in _err(L)


def test_index_score_argument_checks(L):
    P = 0x1000
    b = _batch()
    assert L.dsa_index_score(ctypes.byref(b), P, P, P, P, P, P, 10, None) == B.DSA_ERR_INVALID_ARG
    assert L.dsa_index_score(ctypes.byref(b), None, P, P, P, P, P, 300, None) == \
        B.DSA_ERR_INVALID_ARG


def test_cache_append_argument_checks(L):
    P = 0x1000
    b = _batch()
    ok = (P, P, P, P, P)
    for i in range(5):  # each tensor pointer NULL in turn
        args = list(ok)
        args[i] = None
        assert L.dsa_cache_append(ctypes.byref(b), *args, None) == B.DSA_ERR_INVALID_ARG
    # kv_new / kv_cache 16-byte, k_new / k_scale 4-byte, k8_cache 2-byte alignment
    for i, off in ((1, 8), (4, 8), (0, 2), (3, 2), (2, 1)):
        args = list(ok)
        args[i] = P + off
        assert L.dsa_cache_append(ctypes.byref(b), *args, None) == B.DSA_ERR_INVALID_ARG
        assert "alignment" in _err(L)
    empty = _batch(B_=0, T=0, max_q=0, max_seqlen_k=0, ptrs=False)
    assert L.dsa_cache_append(ctypes.byref(empty), None, None, None, None, None, None) == B.DSA_OK
    assert L.dsa_cache_append(None, *ok, None) == B.DSA_ERR_INVALID_ARG


def test_topk_transform_argument_checks(L):
    P = 0x1000
    b = _batch()
    need = L.dsa_workspace_size(B.DSA_OP_TOPK, ctypes.byref(b), 16, 0)
    for space in (-1, 3):
        assert L.dsa_topk_transform(ctypes.byref(b), P, 300, 16, space, P, P, P, need, None) == \
            B.DSA_ERR_INVALID_ARG
        assert "space" in _err(L)
    assert L.dsa_topk_transform(ctypes.byref(b), P, 300, 16, B.DSA_IDX_RAGGED, None, P, P, need,
                                None) == B.DSA_ERR_INVALID_ARG
    assert "kv_offsets" in _err(L)
    assert L.dsa_topk_transform(ctypes.byref(b), P, 300, 16, B.DSA_IDX_PAGED, None, P, P,
                                need - 1, None) == B.DSA_ERR_WORKSPACE


def test_sparse_mla_paged_argument_checks(L):
    P = 0x1000
    b = _batch()
    assert L.dsa_sparse_mla_decode_paged(ctypes.byref(b), P, P, P, 0, 0.1, P, None, 0, P, 1 << 30,
                                         None) == B.DSA_ERR_INVALID_ARG
    assert L.dsa_sparse_mla_decode_paged(ctypes.byref(b), P, None, P, 16, 0.1, P, None, 1, P,
                                         1 << 30, None) == B.DSA_ERR_INVALID_ARG
    need = L.dsa_workspace_size(B.DSA_OP_SPARSE_MLA, ctypes.byref(b), 2048, 4)
    assert L.dsa_sparse_mla_decode_paged(ctypes.byref(b), P, P, P, 2048, 0.1, P, None, 4, P,
                                         need - 1, None) == B.DSA_ERR_WORKSPACE


def test_decode_layers_argument_checks(L):
    P = 0x1000
    b = _batch()
    assert ctypes.sizeof(B.dsa_layer_t) == 80
    assert B.dsa_layer_t.out.offset == 64 and B.dsa_layer_t.lse.offset == 72
    full = B.dsa_layer_t(B.dsa_indexer_inputs_t(P, P, P, P, P), B.dsa_mla_inputs_t(P, P, 0.07), P,
                         None)
    bare = B.dsa_layer_t(B.dsa_indexer_inputs_t(), B.dsa_mla_inputs_t(P, P, 0.07), P, None)
    need = L.dsa_workspace_size(B.DSA_OP_DECODE_STEP, ctypes.byref(b), 64, 0)

    def call(layers, retention=2, mli=0, aux=None, ws=need):
        arr = (B.dsa_layer_t * len(layers))(*layers)
        return L.dsa_decode_layers(ctypes.byref(b), len(layers), arr, 64, retention, mli, 0, P, P,
                                   ws, None, aux)

    assert L.dsa_decode_layers(ctypes.byref(b), 0, None, 64, 1, 0, 0, P, P, need, None, None) == \
        B.DSA_ERR_INVALID_ARG
    assert call([full, bare], retention=0) == B.DSA_ERR_INVALID_ARG
    assert call([full, bare], mli=2) == B.DSA_ERR_INVALID_ARG
    assert call([full, bare], mli=1) == B.DSA_ERR_INVALID_ARG  # no second stream
    assert call([full, bare, bare], retention=2) == B.DSA_ERR_INVALID_ARG  # layer 2 has no indexer
    assert "indexer" in _err(L)
    no_out = B.dsa_layer_t(B.dsa_indexer_inputs_t(), B.dsa_mla_inputs_t(P, P, 0.07), None, None)
    assert call([full, no_out]) == B.DSA_ERR_INVALID_ARG
    # layers without an indexer may leave its inputs NULL: validation passes
    # and the call stops at the (too small) workspace, before any launch
    assert call([full, bare, full, bare], retention=2, ws=need - 1) == B.DSA_ERR_WORKSPACE


def test_dense_mla_argument_checks(L):
    P = 0x1000
    b = _batch()
    need = L.dsa_workspace_size(B.DSA_OP_DENSE_MLA, ctypes.byref(b), 1, 4)
    assert need >= 4 * 4 * 128 * 512 * 2  # 4 splits of 4 rows, fp16 partials
    assert L.dsa_dense_mla_decode(ctypes.byref(b), None, P, 0.1, P, None, 4, P, need, None) == \
        B.DSA_ERR_INVALID_ARG
    assert L.dsa_dense_mla_decode(ctypes.byref(b), P, P, 0.1, P, None, 4, P, need - 1, None) == \
        B.DSA_ERR_WORKSPACE
    long = _batch(max_seqlen_k=131073, max_pages=2049)
    assert L.dsa_workspace_size(B.DSA_OP_DENSE_MLA, ctypes.byref(long), 1, 0) == 0
    assert L.dsa_dense_mla_decode(ctypes.byref(long), P, P, 0.1, P, None, 0, P, 1 << 40, None) == \
        B.DSA_ERR_UNSUPPORTED


def test_masked_mha_argument_checks(L):
    P = 0x1000
    b = _batch()  # B = 2, T = 4, max_seqlen_k = 300
    need = L.dsa_workspace_size(B.DSA_OP_MASKED_MHA, ctypes.byref(b), 1, 0)
    lp = 320  # 300 rounded up to 64
    assert need >= 2 * 128 * lp * 128 * 2 * 2 + 2 * lp * 64 * 2 + 4 * (lp // 32) * 4
    ok = (ctypes.byref(b), P, P, P, P, P, P, 64, 0.1, P, None, P, need, None)
    for i in (1, 2, 3, 4, 9):  # each required pointer NULL in turn
        args = list(ok)
        args[i] = None
        assert L.dsa_masked_mha_prefill(*args) == B.DSA_ERR_INVALID_ARG, i
    args = list(ok)
    args[1] = P + 8  # q_nope off the 16-byte grid
    assert L.dsa_masked_mha_prefill(*args) == B.DSA_ERR_INVALID_ARG
    args = list(ok)
    args[7] = 0  # k with a selection
    assert L.dsa_masked_mha_prefill(*args) == B.DSA_ERR_INVALID_ARG
    args = list(ok)
    args[12] = need - 1
    assert L.dsa_masked_mha_prefill(*args) == B.DSA_ERR_WORKSPACE
    long = _batch(max_seqlen_k=65537, max_pages=1025)
    assert L.dsa_workspace_size(B.DSA_OP_MASKED_MHA, ctypes.byref(long), 1, 0) == 0
    args = list(ok)
    args[0] = ctypes.byref(long)
    args[12] = 1 << 40
    assert L.dsa_masked_mha_prefill(*args) == B.DSA_ERR_UNSUPPORTED


def test_sparse_mla_argument_checks(L):
    P = 0x1000
    b = _batch()
    assert L.dsa_sparse_mla_decode(ctypes.byref(b), P, P, P, 16, 0.1, P, None, 65, P, 1 << 30,
                                   None) == B.DSA_ERR_INVALID_ARG
    need = L.dsa_workspace_size(B.DSA_OP_SPARSE_MLA, ctypes.byref(b), 2048, 4)
    assert need >= 4 * 4 * 128 * 512 * 2  # fp16 partials of 4 splits x 4 rows
    assert L.dsa_sparse_mla_decode(ctypes.byref(b), P, P, P, 2048, 0.1, P, None, 4, P, need - 1,
                                   None) == B.DSA_ERR_WORKSPACE
    # a single split needs no workspace
    assert L.dsa_workspace_size(B.DSA_OP_SPARSE_MLA, ctypes.byref(b), 2048, 1) == 0


def test_decode_step_argument_checks(L):
    P = 0x1000
    b = _batch()
    ix = B.dsa_indexer_inputs_t(P, P, P, P, P)
    ml = B.dsa_mla_inputs_t(P, P, 0.07)
    need = L.dsa_workspace_size(B.DSA_OP_DECODE_STEP, ctypes.byref(b), 64, 0)
    bad_mode = B.dsa_step_opts_t(7, 0, None)
    assert L.dsa_decode_step(ctypes.byref(b), ctypes.byref(ix), ctypes.byref(ml), 64,
                             ctypes.byref(bad_mode), P, P, None, P, need, None, None) == \
        B.DSA_ERR_INVALID_ARG
    mli = B.dsa_step_opts_t(B.DSA_MODE_MLI, 0, None)  # no attend_idx
    assert L.dsa_decode_step(ctypes.byref(b), ctypes.byref(ix), ctypes.byref(ml), 64,
                             ctypes.byref(mli), P, P, None, P, need, None, 0x2000) == \
        B.DSA_ERR_INVALID_ARG
    mli = B.dsa_step_opts_t(B.DSA_MODE_MLI, 0, P)
    assert L.dsa_decode_step(ctypes.byref(b), ctypes.byref(ix), ctypes.byref(ml), 64,
                             ctypes.byref(mli), P, P, None, P, need, 0x2000, 0x2000) == \
        B.DSA_ERR_INVALID_ARG  # same stream twice
    fused = B.dsa_step_opts_t(B.DSA_MODE_FUSED, 0, None)
    assert L.dsa_decode_step(ctypes.byref(b), ctypes.byref(ix), ctypes.byref(ml), 64,
                             ctypes.byref(fused), P, P, None, P, need - 1, None, None) == \
        B.DSA_ERR_WORKSPACE


def test_mli_step_refuses_attend_idx_overlapping_idx_out(L):
    """In MLI mode the aux stream's top-k writes idx_out while the main
    stream's attention reads attend_idx: overlapping ranges are refused
    before anything is enqueued; disjoint ones pass the check (the call then
    fails later only on the workspace size given here)."""
    P = 0x10000
    b = _batch()  # T = 4
    k = 64
    span = 4 * k * 4  # T * k int32
    ix = B.dsa_indexer_inputs_t(P, P, P, P, P)
    ml = B.dsa_mla_inputs_t(P, P, 0.07)
    need = L.dsa_workspace_size(B.DSA_OP_DECODE_STEP, ctypes.byref(b), k, 0)
    idx_out = 0x200000
    for attend, overlapping in ((idx_out, True), (idx_out + span - 4, True),
                                (idx_out - span + 4, True), (idx_out + span, False),
                                (idx_out - span, False)):
        mli = B.dsa_step_opts_t(B.DSA_MODE_MLI, 0, attend)
        rc = L.dsa_decode_step(ctypes.byref(b), ctypes.byref(ix), ctypes.byref(ml), k,
                               ctypes.byref(mli), idx_out, P, None, P, need - 1, 0x2000, 0x3000)
        if overlapping:
            assert rc == B.DSA_ERR_INVALID_ARG and "overlaps" in _err(L), (hex(attend), rc)
        else:
            assert rc == B.DSA_ERR_WORKSPACE, (hex(attend), rc, _err(L))


def test_noalloc_step_argument_checks(L):
    """The static-scratch step runs FUSED steps only and refuses, before any
    device call, a batch whose step needs more than its 64 MiB."""
    P = 0x10000
    ix = B.dsa_indexer_inputs_t(P, P, P, P, P)
    ml = B.dsa_mla_inputs_t(P, P, 0.07)
    fused = B.dsa_step_opts_t(B.DSA_MODE_FUSED, 0, None)
    mli = B.dsa_step_opts_t(B.DSA_MODE_MLI, 0, P)
    small = _batch()
    assert L.dsa_decode_step_noalloc(ctypes.byref(small), ctypes.byref(ix), ctypes.byref(ml), 64,
                                     ctypes.byref(mli), P, P, None, None) == B.DSA_ERR_INVALID_ARG
    assert "FUSED" in _err(L)
    assert L.dsa_decode_step_noalloc(ctypes.byref(small), ctypes.byref(ix), ctypes.byref(ml), 64,
                                     None, P, P, None, None) == B.DSA_ERR_INVALID_ARG
    big = B.dsa_batch_t(64, 128, 2, 131072, 2048, 131072, P, P, P)
    need = L.dsa_workspace_size(B.DSA_OP_DECODE_STEP, ctypes.byref(big), 2048, 0)
    assert need > 64 << 20
    assert L.dsa_decode_step_noalloc(ctypes.byref(big), ctypes.byref(ix), ctypes.byref(ml), 2048,
                                     ctypes.byref(fused), P, P, None, None) == B.DSA_ERR_WORKSPACE
    assert "64 MiB" in _err(L)
    empty = B.dsa_batch_t(0, 0, 0, 0, 0, 0, None, None, None)
    assert L.dsa_decode_step_noalloc(ctypes.byref(empty), ctypes.byref(ix), ctypes.byref(ml), 64,
                                     ctypes.byref(fused), None, None, None, None) == B.DSA_OK


def test_empty_batch_is_a_no_op(L):
    b = B.dsa_batch_t(0, 0, 0, 0, 0, 0, None, None, None)
    assert L.dsa_topk(ctypes.byref(b), None, 0, 16, None, None, 0, None) == B.DSA_OK
    assert L.dsa_sparse_mla_decode(ctypes.byref(b), None, None, None, 16, 0.1, None, None, 0,
                                   None, 0, None) == B.DSA_OK
    assert L.dsa_index_score(ctypes.byref(b), None, None, None, None, None, None, 0, None) == \
        B.DSA_OK


def test_workspace_sizes_grow_with_the_batch(L):
    small = _batch(T=4, max_seqlen_k=300)
    big = _batch(T=4, max_seqlen_k=600, max_pages=10)
    for op in (B.DSA_OP_TOPK, B.DSA_OP_DECODE_STEP):
        assert L.dsa_workspace_size(op, ctypes.byref(big), 64, 0) > \
            L.dsa_workspace_size(op, ctypes.byref(small), 64, 0)
    assert L.dsa_workspace_size(99, ctypes.byref(small), 64, 0) == 0
    # at most 256 work-groups, at least 4 tiles of 32 tokens per split
    assert L.dsa_default_splits(ctypes.byref(_batch(T=96, max_seqlen_k=300)), 2048) == 2
    assert L.dsa_default_splits(ctypes.byref(_batch(T=300, max_seqlen_k=300)), 2048) == 1
    assert L.dsa_default_splits(ctypes.byref(small), 2048) == 16
    assert L.dsa_default_splits(ctypes.byref(_batch(T=128, max_seqlen_k=300)), 2048) == 2
    assert L.dsa_default_splits(ctypes.byref(_batch(T=32, max_seqlen_k=300)), 2048) == 8
    assert L.dsa_default_splits(ctypes.byref(small), 100) == 1


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ("DSA_MODE_FUSED", "DSA_MODE_MLI", "DSA_STAGE_INDEX_SCORE", "DSA_STAGE_TOPK",
                 "DSA_STAGE_ATTENTION", "DSA_NUM_STAGES", "DSA_OP_TOPK", "DSA_OP_SPARSE_MLA",
                 "DSA_OP_DECODE_STEP", "DSA_OP_DENSE_MLA", "DSA_IDX_LOGICAL", "DSA_IDX_PAGED",
                 "DSA_IDX_RAGGED"):
        m = re.search(rf"\b{name}\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == getattr(B, name), name


def test_step_opts_layout():
    # mode, n_split, attend_idx, stage_events: 4 + 4 + 8 + 8 bytes
    assert ctypes.sizeof(B.dsa_step_opts_t) == 24
    assert B.dsa_step_opts_t.stage_events.offset == 16


def test_stage_events_argument_checked():
    with pytest.raises(ValueError):
        B.dsa_decode_step(None, {}, {}, 16, 0, 0, None, None, None, None, None, 0,
                          stage_events=[1, 2, 3])


def test_misaligned_pointers_are_refused(L):
    """The kernels move queries, keys, latent rows, outputs and partials in
    16-byte pieces: a pointer off that grid is an argument error, caught
    before anything is launched (fake addresses; nothing is dereferenced)."""
    P, M = 0x1000, 0x1008
    b = _batch()
    need = L.dsa_workspace_size(B.DSA_OP_SPARSE_MLA, ctypes.byref(b), 16, 2)
    for q, kv, out, ws in [(M, P, P, P), (P, M, P, P), (P, P, M, P), (P, P, P, M)]:
        assert L.dsa_sparse_mla_decode(ctypes.byref(b), q, kv, P, 16, 0.1, out, None, 2, ws,
                                       need, None) == B.DSA_ERR_INVALID_ARG
        assert "16-byte" in _err(L)
        assert L.dsa_dense_mla_decode(ctypes.byref(b), q, kv, 0.1, out, None, 2, ws, 1 << 30,
                                      None) == B.DSA_ERR_INVALID_ARG
    for q8, k8, sc in [(M, P, P), (P, M, P), (P, P, P + 2)]:
        assert L.dsa_index_score(ctypes.byref(b), q8, P, P, k8, P, sc, 300, None) == \
            B.DSA_ERR_INVALID_ARG
        assert "alignment" in _err(L)
    opts = B.dsa_step_opts_t(B.DSA_MODE_FUSED, 0, None)
    need = L.dsa_workspace_size(B.DSA_OP_DECODE_STEP, ctypes.byref(b), 64, 0)
    for q8, q, out, ws in [(M, P, P, P), (P, M, P, P), (P, P, M, P), (P, P, P, M)]:
        ix = B.dsa_indexer_inputs_t(q8, P, P, P, P)
        ml = B.dsa_mla_inputs_t(q, P, 0.07)
        assert L.dsa_decode_step(ctypes.byref(b), ctypes.byref(ix), ctypes.byref(ml), 64,
                                 ctypes.byref(opts), P, out, None, ws, need, None, None) == \
            B.DSA_ERR_INVALID_ARG
        assert "alignment" in _err(L)
    b = _batch()
    need = L.dsa_workspace_size(B.DSA_OP_TOPK, ctypes.byref(b), 16, 0)
    assert L.dsa_topk(ctypes.byref(b), P, 300, 16, P, M, need, None) == B.DSA_ERR_INVALID_ARG
    assert "16-byte" in _err(L)
