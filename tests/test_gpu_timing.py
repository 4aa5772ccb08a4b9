"""Kernel timing through the C ABI (pic_timing_start / pic_timing_stop): the
recorded intervals come in call order with the op of each call, lie inside the
call's own event-timed span, stop at the capacity, and leave every output bit
for bit as it is with timing off."""
import numpy as np
import pytest
import torch

from position_independent_attention_amd import pic, workloads as W
from tests import hip_helpers as H

pytestmark = pytest.mark.gpu


def setup_module(_):
    H.require_gpu()


def _calls(ctx, w):
    sel_off = pic.pic_select_offsets(w.span_len, w.ratio)
    dc = pic.to_device(w, H.DEV, sel_off=sel_off)
    out = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch.int16, device=H.DEV)
    lse = torch.empty((w.total_q, w.num_q_heads), dtype=torch.float32, device=H.DEV)
    nsel = int(sel_off[-1])
    sel = torch.empty((max(nsel, 1),), dtype=torch.int32, device=H.DEV)
    q1, p1 = dc.q[-1:].clone(), torch.tensor([int(w.q_pos[-1]) + 1], dtype=torch.int32, device=H.DEV)
    o1 = torch.empty_like(q1)
    return [("prefill", pic.PIC_OP_PREFILL, lambda: pic.pic_attn_prefill(ctx, dc, out, lse), out),
            ("select", pic.PIC_OP_SELECT, lambda: pic.qc_score_select(ctx, dc, lse, nsel, sel), sel),
            ("decode", pic.PIC_OP_DECODE, lambda: pic.pic_attn_decode(ctx, dc, q1, p1, o1), o1)]


def test_timing_intervals_follow_the_calls():
    w = W.long_context(n_spans=8, span_tok=1024, q_len=128)
    print(f"timing {w.name}: kv {w.max_kv_len} q {w.total_q}", flush=True)
    ctx = H.ctx_for(w)
    calls = _calls(ctx, w)
    ref = []
    for _, _, fn, o in calls:
        fn()
        torch.cuda.synchronize()
        ref.append(o.clone())
    spans = []
    pic.pic_timing_start(ctx, 4)
    with pytest.raises(pic.PicError):
        pic.pic_timing_start(ctx, 4)          # already on
    for rep in range(2):                      # 6 calls, capacity 4
        for _, _, fn, o in calls:
            o.zero_()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            spans.append(a.elapsed_time(b))
    ms, ops = pic.pic_timing_stop(ctx, 16)
    with pytest.raises(pic.PicError):
        pic.pic_timing_stop(ctx, 16)          # already off
    assert len(ms) == 4
    assert ops.tolist() == [c[1] for c in calls] + [calls[0][1]]
    for i in range(4):
        assert 0.0 < ms[i] <= spans[i] * 1.001 + 1e-3, (i, ms[i], spans[i])
    # outputs of the last (untimed) round are those of the runs without timing
    for (_, _, _, o), r in zip(calls, ref):
        assert torch.equal(o, r)
    # timing off again: calls record nothing and a new session starts empty;
    # a call that launches no kernel (no query tokens) records nothing either
    calls[0][2]()
    pic.pic_timing_start(ctx, 2)
    dc = pic.to_device(w, H.DEV)
    empty = pic.DeviceCache(dc.pool_k, dc.pool_v, dc.block_table, dc.kv_len, dc.kv_pos, dc.max_kv_len, q=dc.q,
                            q_start=torch.zeros(2, dtype=torch.int32, device=H.DEV), q_pos=dc.q_pos, total_q=0,
                            max_q_len=0)
    o0 = torch.empty((1, w.num_q_heads, w.head_dim), dtype=torch.int16, device=H.DEV)
    pic.pic_attn_prefill(ctx, empty, o0)
    torch.cuda.synchronize()
    ms, ops = pic.pic_timing_stop(ctx, 2)
    assert len(ms) == 0
    ctx.close()
