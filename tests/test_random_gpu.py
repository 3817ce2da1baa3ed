"""Randomised decode steps against the float64 oracle.

Twelve seeded batches with a random request count (1-6), rows per request
(1-4: both scan forms, the page-per-wave one for at most two rows and the
row-group one beyond), cached lengths (0 to 20000, so rows shorter and
longer than k, single partial pages and empty requests occur), k cycling
through {1, 7, 64, 500, 2048, 3000} and a shuffled page pool.  Every row is checked:
the selection equals the oracle's outside its tie band, and the attention
over the selection is within the bf16 output bars.
"""
import numpy as np
import pytest
import torch

from gpu_common import (O, bf16_to_f64, check_attention, check_selection, decode_step, synth,
                        sync, to_device)

pytestmark = pytest.mark.gpu


def _config(seed):
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 7))
    n_q = rng.integers(1, 5, B)
    L = rng.integers(0, 20001, B)
    L = np.where(n_q == 1, L, np.maximum(L, n_q))  # an empty request has one row
    if seed % 3 == 0:
        L[rng.integers(0, B)] = rng.integers(1, 64)  # a single partial page
    n_q, L = [int(x) for x in n_q], [int(x) for x in L]
    if seed % 4 == 1:
        n_q.append(1)  # an empty request
        L.append(0)
    k = [1, 7, 64, 500, 2048, 3000][seed % 6]
    return n_q, L, k


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("seed", range(12))
def test_random_decode_step(seed):
    n_q, L, k = _config(seed)
    print(f"seed {seed}: n_q={n_q} L={L} k={k}", flush=True)
    b = synth.make_batch(n_q, L, seed=7000 + seed, paging="shuffled", heavy=16,
                         pool_extra_pages=3)
    d = to_device(b)
    idx, out, lse = decode_step(d, k=k)
    sync()
    rows = list(range(b.T))
    meta = O.Meta.of(b)
    vis = [meta.visible(t) for t in rows]
    sc = O.index_score(meta, b.q8, b.q_scale, b.w, b.k8[0], b.k_scale[0], rows,
                       ld=max(vis + [1]))
    sel, flags, _, Ks = O.topk(np.nan_to_num(sc, nan=-np.inf), vis, k)
    g = idx.cpu().numpy()
    check_selection(g, sel, flags, Ks)
    ref, ref_lse = O.sparse_mla(meta, b.q[0], b.kv[0], g, rows, synth.SM_SCALE)
    check_attention(bf16_to_f64(out), ref, lse.cpu().numpy(), ref_lse)
