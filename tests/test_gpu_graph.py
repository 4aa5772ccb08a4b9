"""The whole hot-path step (prefill with LSE, selection, fusion, prefill over the
fused cache, decode) captured once as a HIP graph and replayed: every replay,
with eager work and synchronisations in between, equals the eager step bit for
bit.  bench.py times the step this way."""
import numpy as np
import pytest
import torch

from position_independent_attention_amd import pic, workloads as W
from tests import hip_helpers as H

pytestmark = pytest.mark.gpu


def setup_module(_):
    H.require_gpu()


def test_graph_replays_match_eager_step():
    dev = H.DEV
    w = W.long_context(n_spans=4, span_tok=512, q_len=64)
    ctx = pic.Context(w.num_q_heads, w.num_kv_heads, w.head_dim, w.rope_theta, w.max_position)
    sel_off = pic.pic_select_offsets(w.span_len, w.ratio)
    nsel = int(sel_off[-1])
    dc = pic.to_device(w, dev, sel_off=sel_off)
    kv0 = dc.max_kv_len
    kv_fused = ((kv0 + 15) // 16) * 16 + nsel
    kv_pos0, kv_len0 = dc.kv_pos.clone(), dc.kv_len.clone()

    def t(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)

    out1 = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch.int16, device=dev)
    lse1 = torch.empty((w.total_q, w.num_q_heads), dtype=torch.float32, device=dev)
    out2 = torch.empty_like(out1)
    sel = torch.empty(nsel, dtype=torch.int32, device=dev)
    req_off = t(np.array([0, nsel], np.int32))
    fk, fv = t(w.fresh_k[:nsel]), t(w.fresh_v[:nsel])
    q_dec = dc.q[-1:].clone()
    qpos_dec = t(np.array([int(w.q_pos[-1]) + 1], np.int32))
    out3 = torch.empty_like(q_dec)
    dcd = pic.DeviceCache(dc.pool_k, dc.pool_v, dc.block_table, dc.kv_len, dc.kv_pos, kv_fused)
    req_fused = pic.PicReqTable(1, dc.block_table.shape[1], kv_fused, 0, 0, 0)
    need = max(pic.pic_workspace_bytes(ctx, op, r, dc.total_q, dc.max_q_len) for op, r in
               ((pic.PIC_OP_PREFILL, dc.req()), (pic.PIC_OP_PREFILL, req_fused),
                (pic.PIC_OP_SELECT, dc.req()), (pic.PIC_OP_DECODE, req_fused)))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def step(st):
        dc.kv_pos.copy_(kv_pos0)
        dc.kv_len.copy_(kv_len0)
        dc.max_kv_len = kv0
        pic.pic_attn_prefill(ctx, dc, out1, lse1, ws=ws, stream=st)
        pic.qc_score_select(ctx, dc, lse1, nsel, sel, None, ws=ws, stream=st)
        pic.kv_fuse_scatter(ctx, dc, sel, req_off, fk, fv, nsel, nsel, stream=st)
        dc.max_kv_len = kv_fused
        pic.pic_attn_prefill(ctx, dc, out2, None, ws=ws, stream=st)
        pic.pic_attn_decode(ctx, dcd, q_dec, qpos_dec, out3, None, ws=ws, stream=st)

    outs = (out1, lse1, sel, out2, out3)
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    assert int((sel >= 0).sum()) == nsel

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    scratch = torch.empty_like(out1)
    for rep in range(4):
        for o in outs:
            o.zero_()
        # eager work of the program's own between the replays
        dc.max_kv_len = kv0
        dc.kv_pos.copy_(kv_pos0)
        dc.kv_len.copy_(kv_len0)
        pic.pic_attn_prefill(ctx, dc, scratch, None, ws=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep}: output {i} differs from the eager step"
    del g
    ctx.close()
