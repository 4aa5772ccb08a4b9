"""qc_score_select_noalloc (the selection with the library's per-GPU scratch as
its workspace) against qc_score_select with a caller workspace, through the C
ABI: two calls in a row, the second on a smaller input, with and without the
caller's LSE; then a call whose workspace would exceed the scratch is refused
before any launch."""
import numpy as np
import pytest
import torch

from position_independent_attention_amd import pic, workloads as W
from tests import hip_helpers as H

pytestmark = pytest.mark.gpu


def setup_module(_):
    H.require_gpu()


def _run(ctx, w, lse_given, noalloc):
    sel_off = pic.pic_select_offsets(w.span_len, w.ratio)
    dc = pic.to_device(w, H.DEV, sel_off=sel_off)
    out = torch.empty((w.total_q, w.num_q_heads, w.head_dim), dtype=torch.int16, device=H.DEV)
    lse = torch.empty((w.total_q, w.num_q_heads), dtype=torch.float32, device=H.DEV)
    pic.pic_attn_prefill(ctx, dc, out, lse)
    nsel = int(sel_off[-1])
    sel = torch.full((max(nsel, 1),), -7, dtype=torch.int32, device=H.DEV)
    mass = torch.full(w.kv_pos.shape, -1.0, dtype=torch.float32, device=H.DEV)
    fn = pic.qc_score_select_noalloc if noalloc else pic.qc_score_select
    fn(ctx, dc, lse if lse_given else None, nsel, sel, mass)
    torch.cuda.synchronize()
    return sel.cpu().numpy()[:nsel], mass.cpu().numpy()


@pytest.mark.parametrize("lse_given", [True, False])
def test_noalloc_select_equals_workspace_select_twice(lse_given):
    big = W.long_context(n_spans=8, span_tok=1024, q_len=256)
    small = W.tiny()
    for w in (big, small):
        print(f"noalloc select {w.name}: kv {w.max_kv_len} q {w.total_q} lse_given={lse_given}", flush=True)
        ctx = H.ctx_for(w)
        a_sel, a_mass = _run(ctx, w, lse_given, noalloc=False)
        b_sel, b_mass = _run(ctx, w, lse_given, noalloc=True)
        ctx.close()
        assert np.array_equal(a_sel, b_sel)
        n = int(w.kv_len[0])
        assert np.array_equal(a_mass[0, :n], b_mass[0, :n])
        assert not np.any(b_sel == -7)


def test_noalloc_select_refuses_a_workspace_beyond_the_scratch():
    w = W.tiny()
    ctx = H.ctx_for(w)
    sel_off = pic.pic_select_offsets(w.span_len, w.ratio)
    dc = pic.to_device(w, H.DEV, sel_off=sel_off)
    # 64 requests of up to 65,536 slots: the partial and the summed masses
    # take 16 MiB each
    B, mb = 64, 4096
    dc.block_table = torch.full((B, mb), -1, dtype=torch.int32, device=H.DEV)
    dc.kv_pos = torch.full((B, mb * 16), -1, dtype=torch.int32, device=H.DEV)
    dc.kv_len = torch.zeros(B, dtype=torch.int32, device=H.DEV)
    dc.max_kv_len = mb * 16
    dc.q_start = torch.zeros(B + 1, dtype=torch.int32, device=H.DEV)
    need = pic.pic_workspace_bytes(ctx, pic.PIC_OP_SELECT, dc.req(), dc.total_q, dc.max_q_len)
    assert need > (16 << 20)
    sel = torch.full((int(sel_off[-1]),), -7, dtype=torch.int32, device=H.DEV)
    with pytest.raises(pic.PicError) as e:
        pic.qc_score_select_noalloc(ctx, dc, None, int(sel_off[-1]), sel, None)
    assert e.value.status == pic.PIC_ERR_WORKSPACE
    assert "scratch" in ctx.last_error()
    torch.cuda.synchronize()
    assert np.all(sel.cpu().numpy() == -7)
    ctx.close()
