"""The multi-layer indexer schedule (dsa_decode_layers) through the C ABI:
IndexCache retention 1/r composed with MLI over a stack of layers.  Each
selection a kept indexer makes is checked against the oracle's for that
layer's keys, and each layer's attention against the oracle's attention over
the selection the oracle's schedule says the layer reads."""
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


def _run_layers(d, layer_ids, retention, mli, k=K):
    T = d.meta.T
    n = len(layer_ids)
    outs = [torch.empty((T, 128, 512), dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    lses = [torch.empty((T, 128), dtype=torch.float32, device="cuda") for _ in range(n)]
    layers = []
    for i, li in enumerate(layer_ids):
        ix = dict(q8=d.q8, q_scale=d.q_scale, w=d.w, k8_cache=d.k8[li], k_scale=d.k_scale[li])
        layers.append(dict(ix=ix if i % retention == 0 else None,
                           mla=dict(q=d.q[li], kv_cache=d.kv[li], sm_scale=synth.SM_SCALE),
                           out=outs[i], lse=lses[i]))
    n_sel = -(-n // retention)
    sel = torch.full((n_sel, T, k), -5, dtype=torch.int32, device="cuda")
    ws_bytes = dsa.dsa_workspace_size(dsa.DSA_OP_DECODE_STEP, d.meta, k, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    aux = torch.cuda.Stream() if mli else None
    dsa.dsa_decode_layers(d.meta, layers, k, retention, mli, 0, sel, ws, ws_bytes, stream_aux=aux)
    sync()
    return sel, outs, lses


def _check_schedule(b, d, layer_ids, retention, mli, rows):
    sel, outs, lses = _run_layers(d, layer_ids, retention, mli)
    produces, attends = O.layer_schedule(len(layer_ids), retention, mli)
    for l, j in enumerate(produces):
        if j < 0:
            continue
        meta, vis, sc, osel, flags, Ks = oracle_rows(b, rows, layer=layer_ids[l])
        check_selection(sel[j][rows].cpu().numpy(), osel, flags, Ks)
    meta = O.Meta.of(b)
    for l, li in enumerate(layer_ids):
        g = sel[attends[l]][rows].cpu().numpy()
        ref, ref_lse = O.sparse_mla(meta, b.q[li], b.kv[li], g, rows, synth.SM_SCALE)
        check_attention(bf16_to_f64(outs[l][rows]), ref, lses[l][rows].cpu().numpy(), ref_lse)
    return sel, outs, lses, attends


@pytest.fixture(scope="module")
def small():
    b = synth.make_batch([2, 1, 2], [3000, 5000, 9000], seed=900, paging="shuffled", heavy=16,
                         layers=5, pool_extra_pages=3)
    return b, to_device(b)


@pytest.mark.parametrize("retention,mli", [(1, 0), (1, 1), (2, 0), (2, 1), (4, 1), (8, 1)])
def test_decode_layers_schedule_small(small, retention, mli):
    b, d = small
    rows = list(range(b.T))
    sel, outs, lses, attends = _check_schedule(b, d, list(range(5)), retention, mli, rows)
    # a layer's attention equals the standalone attention over the selection
    # the schedule gives it, bit for bit
    for l in range(5):
        out, lse = sparse_mla(d, sel[attends[l]], layer=l)
        sync()
        assert torch.equal(out, outs[l]) and torch.equal(lse, lses[l])


def test_decode_layers_every_layer_fused_equals_steps(small):
    b, d = small
    sel, outs, lses = _run_layers(d, list(range(5)), 1, 0)
    for l in range(5):
        idx, out, lse = decode_step(d, layer=l)
        sync()
        assert torch.equal(idx, sel[l]) and torch.equal(out, outs[l]) and torch.equal(lse, lses[l])


def test_decode_layers_mli_workload():
    """The two-layer ragged workload (48 requests, 10K-196K tokens) as a
    four-layer stack alternating its layers, retention 1/2 with MLI, at full
    size; rows sampled for the oracle."""
    b = synth.make_workload(4)
    d = to_device(b)
    rng = np.random.default_rng(4)
    rows = sorted({0, b.T - 1} | set(rng.choice(b.T, 2, replace=False).tolist()))
    _check_schedule(b, d, [0, 1, 0, 1], 2, 1, rows)
