"""dsa_decode_step_noalloc (the step in the library's static scratch) against
dsa_decode_step with a caller workspace, through the C ABI: two calls in a
row, the second on a smaller batch, each bit for bit equal to the workspace
step (same kernels, same split count), and the first also checked against
the oracle."""
import numpy as np
import pytest
import torch

from gpu_common import (K, O, bf16_to_f64, check_attention, check_selection, dsa, oracle_rows,
                        synth, sync, to_device)

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsa.lib()


def _run(b, noalloc):
    d = to_device(b)
    T = b.T
    idx = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
    out = torch.full((T, 128, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, 128), 5.0, dtype=torch.float32, device="cuda")
    ix = dict(q8=d.q8, q_scale=d.q_scale, w=d.w, k8_cache=d.k8[0], k_scale=d.k_scale[0])
    ml = dict(q=d.q[0], kv_cache=d.kv[0], sm_scale=synth.SM_SCALE)
    need = dsa.dsa_workspace_size(dsa.DSA_OP_DECODE_STEP, d.meta, K, 0)
    assert 0 < need <= SCRATCH
    if noalloc:
        dsa.dsa_decode_step_noalloc(d.meta, ix, ml, K, 0, idx, out, lse)
    else:
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        dsa.dsa_decode_step(d.meta, ix, ml, K, dsa.DSA_MODE_FUSED, 0, None, idx, out, lse, ws,
                            need)
    sync()
    return idx, out, lse


def test_noalloc_step_equals_workspace_step_on_two_calls():
    # first call: a request longer than the one-pass top-k (histogram, collect
    # and final kernels in the scratch), ragged rows and a padding request;
    # second call: a smaller batch that the scratch serves after the first
    big = synth.make_batch([2, 1, 2, 1], [70001, 9000, 0, 4100], seed=1700, paging="shuffled",
                           heavy=16, pool_extra_pages=3)
    small = synth.make_batch([1, 2], [3000, 2500], seed=1701, paging="shuffled", heavy=16,
                             pool_extra_pages=3)
    for i, b in enumerate((big, small)):
        print(f"no-alloc call {i}: T={b.T} L={list(b.seqlens_k)}", flush=True)
        g = _run(b, noalloc=True)
        r = _run(b, noalloc=False)
        for x, y in zip(g, r):
            assert torch.equal(x, y), i
        if i == 0:
            rows = list(range(b.T))
            meta, vis, sc, sel, flags, Ks = oracle_rows(b, rows)
            gi = g[0].cpu().numpy()
            check_selection(gi, sel, flags, Ks)
            ref, ref_lse = O.sparse_mla(meta, b.q[0], b.kv[0], gi, rows, synth.SM_SCALE)
            check_attention(bf16_to_f64(g[1]), ref, g[2].cpu().numpy(), ref_lse)


def test_noalloc_step_refuses_a_batch_beyond_the_scratch():
    """A 64-row batch on 131072-token contexts needs far more than 64 MiB: the
    call fails with DSA_ERR_WORKSPACE before anything is enqueued (outputs
    untouched)."""
    cu = torch.arange(0, 65, dtype=torch.int32, device="cuda")
    L = torch.full((64,), 131072, dtype=torch.int32, device="cuda")
    pt = torch.zeros((64, 2048), dtype=torch.int32, device="cuda")
    meta = dsa.Batch(cu, L, pt, 2048, 1, 131072)
    z8 = torch.zeros(16, dtype=torch.uint8, device="cuda")
    zf = torch.zeros(16, dtype=torch.float32, device="cuda")
    zb = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    idx = torch.full((64, K), -7, dtype=torch.int32, device="cuda")
    out = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_decode_step_noalloc(meta, dict(q8=z8, q_scale=zf, w=zf, k8_cache=z8, k_scale=zf),
                                    dict(q=zb, kv_cache=zb, sm_scale=0.07), K, 0, idx, out, None)
    assert e.value.status == dsa.binding.DSA_ERR_WORKSPACE and "64 MiB" in str(e.value)
    sync()
    assert bool((idx == -7).all())
