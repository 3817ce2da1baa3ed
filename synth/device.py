"""Copy a generated batch to the GPU as torch tensors (input plumbing only)."""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import torch


def _t(a: np.ndarray, device, dtype=None) -> torch.Tensor:
    x = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        x = x.view(dtype)
    return x.to(device, non_blocking=False)


def to_device(batch, device="cuda", layers=None) -> SimpleNamespace:
    """Device tensors of a synth Batch.  bf16 tensors keep their bit patterns
    (torch.bfloat16 views of the uint16 host arrays); FP8 codes stay uint8."""
    from sparse_attention_02_amd import Batch as DevBatch

    layers = range(len(batch.k8)) if layers is None else layers
    cu = _t(batch.cu_seqlens_q, device)
    lens = _t(batch.seqlens_k, device)
    pt = _t(batch.page_table, device)
    d = SimpleNamespace()
    d.meta = DevBatch(cu, lens, pt, batch.num_pages, batch.max_q, batch.max_seqlen_k)
    d.q8 = _t(batch.q8, device)
    d.q_scale = _t(batch.q_scale, device)
    d.w = _t(batch.w, device)
    d.k8 = [_t(batch.k8[i], device) for i in layers]
    d.k_scale = [_t(batch.k_scale[i], device) for i in layers]
    d.q = [_t(batch.q[i].view(np.int16), device, torch.bfloat16) for i in layers if batch.q]
    d.kv = [_t(batch.kv[i].view(np.int16), device, torch.bfloat16) for i in layers if batch.kv]
    return d
