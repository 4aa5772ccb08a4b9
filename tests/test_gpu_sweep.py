"""Seeded random small layouts through the whole path, against the oracle.

Each seed draws a head layout (G = 1 .. 8), d (64 or 128), 1 to 3 requests of
1 to 3 spans (lengths 1 .. 399, gaps 0 .. 49 positions), 1 .. 47 query tokens
and a selection ratio, and masks about a tenth of some requests' context
slots (pi = -1).  Every seed runs prefill with LSE, the selection (with that
LSE and with its own LSE pass), the fusion
of the oracle's own selection and attention over the fused cache; a second
set runs decode (one query token per request).  Bars as in
test_gpu_parity.py.
"""
import sys

import numpy as np
import pytest

import oracle
from position_independent_attention_amd import pic, workloads as W
from tests import hip_helpers as H
from tests.util import check_lse, check_mass, check_selection, out_within, parity_stats

pytestmark = pytest.mark.gpu

HEADS = [(8, 2), (4, 4), (16, 2), (2, 1), (32, 8), (8, 1)]


def setup_module(_):
    H.require_gpu()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def random_layout(seed, decode=False):
    rng = np.random.default_rng(seed)
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    d = int(rng.choice([64, 128]))
    batch = int(rng.integers(1, 4))
    span_lens = [[int(x) for x in rng.integers(1, 400, size=int(rng.integers(1, 4)))] for _ in range(batch)]
    gaps = [[int(x) for x in rng.integers(0, 50, size=len(s))] for s in span_lens]
    q_len = [1] * batch if decode else [int(rng.integers(1, 48)) for _ in range(batch)]
    w = W.custom(2000 + seed, Hq=hq, Hkv=hkv, d=d, theta=float(rng.choice([1e4, 5e5])), span_lens=span_lens,
                 gaps=gaps, q_len=q_len, ratio=float(rng.choice([0.1, 0.25, 0.5])), decode=decode)
    for r in range(batch):
        n = int(w.kv_len[r]) - q_len[r]
        if n > 10 and rng.random() < 0.5:
            w.kv_pos[r, rng.choice(n, size=n // 10, replace=False)] = -1
    return w


SHUFFLED_HEADS = [(8, 2), (4, 1), (16, 2), (8, 1)]


def shuffled_layout(seed, decode=False):
    """1 to 2 requests (seeds from 6 on) of 2 to 5 spans of 64 to 599 tokens
    whose position ranges are shuffled against their slot order (reused spans
    back at other offsets), 64 to 160 query tokens (several row blocks at
    G = 8) or one in decode; in half the prefill seeds the queries sit at
    sorted random context positions (the sparse recompute's queries), and in
    half about a tenth of the context slots are masked."""
    rng = np.random.default_rng(seed)
    hq, hkv = SHUFFLED_HEADS[int(rng.integers(len(SHUFFLED_HEADS)))]
    d = int(rng.choice([64, 128]))
    batch = 1 if seed < 6 else 2
    lens = [[int(x) for x in rng.integers(64, 600, size=int(rng.integers(2, 6)))] for _ in range(batch)]
    nq = [1 if decode else int(rng.integers(64, 161)) for _ in range(batch)]
    w = W.custom(3000 + seed, Hq=hq, Hkv=hkv, d=d, theta=float(rng.choice([1e4, 5e5])), span_lens=lens,
                 q_len=nq, ratio=float(rng.choice([0.1, 0.25, 0.5])), decode=decode)
    for r in range(batch):
        spans = [s for s in range(len(w.span_req)) if int(w.span_req[s]) == r]
        assert [int(w.span_len[s]) for s in spans] == lens[r]
        base, pos = {}, 0
        for s in rng.permutation(spans):
            base[int(s)] = pos
            pos += int(w.span_len[s])
        for s in spans:
            st, L = int(w.span_start[s]), int(w.span_len[s])
            w.kv_pos[r, st:st + L] = base[s] + np.arange(L)
        n_ctx = int(w.kv_len[r]) - (0 if decode else nq[r])
        if not decode and rng.random() < 0.5:
            ctx_pos = w.kv_pos[r, :n_ctx]
            q0 = int(w.q_start[r])
            w.q_pos[q0:q0 + nq[r]] = np.sort(rng.choice(ctx_pos[ctx_pos >= 0], size=nq[r], replace=False))
        if rng.random() < 0.5:
            w.kv_pos[r, rng.choice(n_ctx, size=n_ctx // 10, replace=False)] = -1
    return w


def describe(w):
    return (f"B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
            f"kv={w.kv_len.tolist()} q={np.diff(w.q_start).tolist()} ratio={w.ratio}")


def check_out(got, ref, what):
    mx, mean, rel = parity_stats(got, ref)
    say(f"  {what}: max {mx:.3e} mean {mean:.3e} rel {rel:.3e}")
    assert out_within(got, ref), (what, mx, mean, rel)


@pytest.mark.parametrize("seed", list(range(10)) + [f"shuffled{i}" for i in range(10)])
def test_random_layout_prefill_select_fuse(seed):
    w = shuffled_layout(int(seed[8:])) if isinstance(seed, str) else random_layout(seed)
    say(f"seed {seed}: {describe(w)}")
    ctx = H.ctx_for(w)
    out, lse, dc = H.prefill(ctx, w)
    ref_o, ref_l = oracle.attention(w)
    check_out(H.host_bf16(out), ref_o, "O")
    check_lse(w, lse.cpu().numpy(), ref_l)

    ref_m = oracle.mass(w)
    ref_off, ref_idx = oracle.select(w, ref_m)
    # with the prefill's LSE, and with the selection's own K-only LSE pass
    # (512-row workgroups above 256 rows per kv head at d = 128)
    for lse_in in (lse, None):
        sel_off, sel, mass = H.select(ctx, w, dc, lse_in)
        check_selection(sel_off, sel, ref_off, ref_idx, ref_m, w)
        check_mass(w, mass, ref_m, what=f"mass (caller's lse: {lse_in is not None})")

    # fuse the oracle's own selection on both sides, then attend again
    req_off = H.req_offsets(w, ref_off)
    n = int(req_off[-1])
    pk, pv, kp, kl = oracle.fuse(w, ref_idx, req_off, w.fresh_k[:n], w.fresh_v[:n])
    dcf = pic.to_device(w, H.DEV)
    H.fuse(ctx, dcf, ref_idx, req_off, w.fresh_k, w.fresh_v)
    assert np.array_equal(dcf.kv_len.cpu().numpy(), kl)
    assert np.array_equal(dcf.kv_pos.cpu().numpy(), kp)
    assert np.array_equal(dcf.pool_k.cpu().numpy().view(np.uint16), pk)
    assert np.array_equal(dcf.pool_v.cpu().numpy().view(np.uint16), pv)
    fused = w.copy()
    fused.pool_k, fused.pool_v, fused.kv_pos, fused.kv_len = pk, pv, kp, kl
    dcf.max_kv_len = int(kl.max())
    out2, lse2, _ = H.prefill(ctx, fused, dcf)
    ref2, refl2 = oracle.attention(fused)
    check_out(H.host_bf16(out2), ref2, "O fused")
    check_lse(fused, lse2.cpu().numpy(), refl2)


@pytest.mark.parametrize("seed", list(range(10, 16)) + [f"shuffled{i}" for i in range(20, 26)])
def test_random_layout_decode(seed):
    w = shuffled_layout(int(seed[8:]), decode=True) if isinstance(seed, str) else random_layout(seed, decode=True)
    say(f"seed {seed}: {describe(w)}")
    ctx = H.ctx_for(w)
    out, lse, _ = H.decode(ctx, w)
    ref_o, ref_l = oracle.attention(w)
    check_out(H.host_bf16(out), ref_o, "O")
    check_lse(w, lse.cpu().numpy(), ref_l)
