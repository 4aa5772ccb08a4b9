"""Drive the HIP library through its C ABI for the GPU tests."""
from __future__ import annotations

import numpy as np
import torch

from position_independent_attention_amd import pic
from position_independent_attention_amd.workloads import bf16_bits_to_f32

DEV = torch.device("cuda:0")


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.set_device(DEV)


def ctx_for(w) -> pic.Context:
    return pic.Context(w.num_q_heads, w.num_kv_heads, w.head_dim, w.rope_theta, w.max_position)


def dev(a) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return bf16_bits_to_f32(t.cpu().numpy().view(np.uint16))


def prefill(ctx, w, dc=None, with_lse=True):
    dc = dc if dc is not None else pic.to_device(w, DEV)
    out = torch.full((dc.total_q, w.num_q_heads, w.head_dim), 0x7fc0, dtype=torch.int16, device=DEV)
    lse = torch.full((dc.total_q, w.num_q_heads), float("nan"), dtype=torch.float32, device=DEV) if with_lse else None
    pic.pic_attn_prefill(ctx, dc, out, lse)
    torch.cuda.synchronize()
    return out, lse, dc


def select(ctx, w, dc, lse, ratio=None):
    sel_off = pic.pic_select_offsets(w.span_len, w.ratio if ratio is None else ratio)
    dc.sel_off = dev(sel_off)
    nsel = int(sel_off[-1])
    sel = torch.full((max(nsel, 1),), -7, dtype=torch.int32, device=DEV)
    mass = torch.full(w.kv_pos.shape, -1.0, dtype=torch.float32, device=DEV)
    pic.qc_score_select(ctx, dc, lse, nsel, sel, mass)
    torch.cuda.synchronize()
    return sel_off, sel.cpu().numpy()[:nsel], mass.cpu().numpy()


def req_offsets(w, sel_off) -> np.ndarray:
    """CSR of selections per request from the per-span CSR (spans are grouped
    by request in request order)."""
    off = np.zeros(w.batch + 1, np.int64)
    for s in range(len(w.span_req)):
        off[w.span_req[s] + 1] += sel_off[s + 1] - sel_off[s]
    return np.cumsum(off).astype(np.int32)


def fuse(ctx, dc, sel_idx, req_off, fresh_k, fresh_v):
    n = int(req_off[-1])
    mx = int(np.max(np.diff(req_off))) if len(req_off) > 1 else 0
    pic.kv_fuse_scatter(ctx, dc, dev(np.asarray(sel_idx, np.int32)) if n else None, dev(req_off),
                        dev(fresh_k[:n]) if n else None, dev(fresh_v[:n]) if n else None, n, mx)
    torch.cuda.synchronize()


def decode(ctx, w, dc=None):
    """One decode call over all requests: each request's single query token."""
    assert np.all(np.diff(w.q_start) == 1)
    dc = dc if dc is not None else pic.to_device(w, DEV)
    out = torch.full((w.batch, w.num_q_heads, w.head_dim), 0x7fc0, dtype=torch.int16, device=DEV)
    lse = torch.full((w.batch, w.num_q_heads), float("nan"), dtype=torch.float32, device=DEV)
    pic.pic_attn_decode(ctx, dc, dc.q, dc.q_pos, out, lse)
    torch.cuda.synchronize()
    return out, lse, dc
