"""Out-of-bounds writes, through the C ABI: every output and workspace
buffer sits between two 4 KB guard zones filled with a byte pattern, and
after the call (fused step, MLI step, each stage alone, the dense form, the
cache append) the zones must be unchanged.  The batches cover ragged
requests, rows shorter than k, a padding request, page ids outside the pool
and the two top-k paths (rows up to 65536 positions and longer ones)."""
import numpy as np
import pytest
import torch

from gpu_common import K, dsa, synth, sync, to_device

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


class Guarded:
    """A device buffer of `nbytes` between two guard zones."""

    def __init__(self):
        self.bufs = []

    def bytes(self, nbytes):
        raw = torch.full((GUARD + max(nbytes, 1) + GUARD,), PATTERN, dtype=torch.uint8,
                         device="cuda")
        self.bufs.append((raw, max(nbytes, 1)))
        return raw[GUARD:GUARD + max(nbytes, 1)]

    def tensor(self, shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        return self.bytes(n).view(dtype).view(shape)

    def check(self):
        sync()
        for raw, n in self.bufs:
            head = raw[:GUARD]
            tail = raw[GUARD + n:]
            assert bool((head == PATTERN).all()), "write before the buffer"
            assert bool((tail == PATTERN).all()), "write past the buffer"


def _batch(n_q, L, seed, bad_page=False):
    b = synth.make_batch(n_q, L, seed=seed, paging="shuffled", heavy=16, pool_extra_pages=3)
    if bad_page:
        # one page id outside the pool: its positions are never scored,
        # gathered or written
        b.page_table[0, 1] = b.num_pages + 7
    return b, to_device(b)


CASES = [
    dict(n_q=[1, 2, 1], L=[63, 5000, 0], seed=1500, bad=False),
    dict(n_q=[2, 1, 3], L=[2049, 30000, 700], seed=1501, bad=True),
    dict(n_q=[2, 2], L=[70001, 140000], seed=1502, bad=False),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
@pytest.mark.parametrize("mode", ["fused", "mli"])
def test_decode_step_writes_stay_in_bounds(ci, mode, request):
    c = CASES[ci]
    if c["bad"] or mode == "mli":
        # a page id outside the pool; in MLI mode the previous selection also
        # names positions past some rows' visible length (skipped)
        request.applymarker(pytest.mark.device_check_flags)
    b, d = _batch(c["n_q"], c["L"], c["seed"], c["bad"])
    T = d.meta.T
    g = Guarded()
    ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_DECODE_STEP, d.meta, K, 0)
    ws = g.bytes(ws_bytes)
    idx = g.tensor((T, K), torch.int32)
    out = g.tensor((T, 128, 512), torch.bfloat16)
    lse = g.tensor((T, 128), torch.float32)
    ix = dict(q8=d.q8, q_scale=d.q_scale, w=d.w, k8_cache=d.k8[0], k_scale=d.k_scale[0])
    ml = dict(q=d.q[0], kv_cache=d.kv[0], sm_scale=synth.SM_SCALE)
    if mode == "fused":
        dsa.dsa_decode_step(d.meta, ix, ml, K, dsa.DSA_MODE_FUSED, 0, None, idx, out, lse, ws,
                            ws_bytes)
    else:
        prev = g.tensor((T, K), torch.int32)
        prev.copy_(torch.full((T, K), -1, dtype=torch.int32, device="cuda"))
        prev[:, :5] = torch.arange(5, dtype=torch.int32, device="cuda")
        aux = torch.cuda.Stream()
        dsa.dsa_decode_step(d.meta, ix, ml, K, dsa.DSA_MODE_MLI, 0, prev, idx, out, lse, ws,
                            ws_bytes, stream_aux=aux)
    g.check()


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_stages_write_in_bounds(ci, request):
    c = CASES[ci]
    if c["bad"]:
        request.applymarker(pytest.mark.device_check_flags)
    b, d = _batch(c["n_q"], c["L"], c["seed"], c["bad"])
    T = d.meta.T
    g = Guarded()
    mx = int(d.meta.c.max_seqlen_k)
    for ld in (mx + (-mx) % 4, mx + 1):  # the one-pass and the multi-kernel top-k
        scores = g.tensor((T, ld), torch.float32)
        dsa.dsa_index_score(d.meta, d.q8, d.q_scale, d.w, d.k8[0], d.k_scale[0], scores, ld)
        tk = dsa.dsa_workspace_size(dsa.DSA_OP_TOPK, d.meta, K)
        ws_t = g.bytes(tk)
        idx = g.tensor((T, K), torch.int32)
        dsa.dsa_topk(d.meta, scores, ld, K, idx, ws_t, tk)
        slots = g.tensor((T, K), torch.int32)
        dsa.dsa_topk_transform(d.meta, scores, ld, K, dsa.DSA_IDX_PAGED, None, slots, ws_t, tk)
    for n_split in (0, 3):
        mk = dsa.dsa_workspace_size(dsa.DSA_OP_SPARSE_MLA, d.meta, K, n_split)
        ws_m = g.bytes(mk)
        out = g.tensor((T, 128, 512), torch.bfloat16)
        lse = g.tensor((T, 128), torch.float32)
        dsa.dsa_sparse_mla_decode(d.meta, d.q[0], d.kv[0], idx, K, synth.SM_SCALE, out, lse,
                                  n_split, ws_m, mk)
        dsa.dsa_sparse_mla_decode_paged(d.meta, d.q[0], d.kv[0], slots, K, synth.SM_SCALE, out,
                                        lse, n_split, ws_m, mk)
    if mx <= 131072:
        dk = dsa.dsa_workspace_size(dsa.DSA_OP_DENSE_MLA, d.meta, 1, 0)
        ws_d = g.bytes(dk)
        out = g.tensor((T, 128, 512), torch.bfloat16)
        lse = g.tensor((T, 128), torch.float32)
        dsa.dsa_dense_mla_decode(d.meta, d.q[0], d.kv[0], synth.SM_SCALE, out, lse, 0, ws_d, dk)
    g.check()


def test_cache_append_writes_only_its_slots():
    """The appended rows' slots change; every other byte of the three pools,
    and the guard zones around them, does not."""
    b, d = _batch([2, 1, 3], [130, 64, 2000], 1503, bad_page=False)
    T = d.meta.T
    g = Guarded()
    P = b.num_pages
    k8 = g.tensor((P, 64, 128), torch.uint8)
    ks = g.tensor((P, 64), torch.float32)
    kv = g.tensor((P, 64, 576), torch.bfloat16)
    k8.copy_(d.k8[0])
    ks.copy_(d.k_scale[0])
    kv.copy_(d.kv[0])
    before = (k8.clone(), ks.clone(), kv.clone())
    k_new = torch.randn((T, 128), device="cuda").to(torch.bfloat16)
    kv_new = torch.randn((T, 576), device="cuda").to(torch.bfloat16)
    dsa.dsa_cache_append(d.meta, k_new, kv_new, k8, ks, kv)
    g.check()
    # the slots the rows land on
    cu = b.cu_seqlens_q
    touched = np.zeros((P, 64), bool)
    for r in range(len(b.seqlens_k)):
        n = int(cu[r + 1] - cu[r])
        for j in range(n):
            p = int(b.seqlens_k[r]) - n + j
            pg = int(b.page_table[r, p // 64])
            if 0 <= pg < P:
                touched[pg, p % 64] = True
    keep = torch.from_numpy(~touched).cuda()
    assert torch.equal(k8[keep], before[0][keep])
    assert torch.equal(ks[keep], before[1][keep])
    assert torch.equal(kv[keep], before[2][keep])
