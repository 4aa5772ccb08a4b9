"""Helpers shared by the tests: hand-built paged layouts and parity metrics.

Nothing here computes attention; layouts are input structure and the metrics
compare two result arrays.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from position_independent_attention_amd.workloads import (BLOCK, Workload, bf16_bits_to_f32,
                                                          f32_to_bf16_bits)

# Parity bar for bf16 outputs (max abs / mean abs), with rel-L2 as an extra
# guard.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
O_REL_L2 = 1e-2
# LSE and selection mass: caps derived from the kernel's arithmetic for a row
# with few keys.  The rotated q and k are rounded to bf16 (unit roundoff
# u = 2^-8) before the MFMA, so a score carries an error
# ds = sum_i q_i k_i (e_qi + e_ki) / sqrt(d), standard deviation about 2.3e-3
# for unit-variance data (worst case 2u sum|q_i k_i| / sqrt(d)).  LSE error is a
# convex combination of score errors, so it is at most max|ds|: 1e-2 is about
# 4.5 standard deviations.  A key's mass is sum_r p_r, each p_r off by
# p_r (ds_r - dlse_r), so |dmass| <= 2 max|ds| mass: 2e-2 of the mass, plus
# 1e-5 for fp32 accumulation.  Each row and each slot is held to the smaller
# of its cap and its own bar from tests/error_model.py, which shrinks with the
# row's effective key count (and, for the mass, with the rows a slot sums).
LSE_ABS = 1e-2
MASS_REL = 2e-2
MASS_FLOOR = 1e-5
SEL_BAND = 1e-3


def lse_bar(w, rows=None) -> np.ndarray:
    """Per-row LSE bar: the row's own error bar, capped at LSE_ABS (NaN, for a
    row that sees nothing, stays NaN)."""
    from tests.error_model import bars
    return np.minimum(bars(w, rows), LSE_ABS)


def mass_bar(w, ref_mass) -> np.ndarray:
    """Per-slot mass bar [B, stride]: the slot's own error bar, capped at the
    uniform MASS_REL * mass + MASS_FLOOR."""
    from tests.error_model import bars
    _, mb = bars(w, with_mass=True)
    return np.minimum(mb, MASS_REL * np.abs(np.asarray(ref_mass, np.float64)) + MASS_FLOOR)


def lse_errors(w, got, ref, rows=None):
    """(max error, largest error / bar) over rows, after checking that rows
    which see nothing are -inf on both sides."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bar = lse_bar(w, rows)
    empty = np.isnan(bar)
    assert np.array_equal(np.isneginf(ref), empty), "oracle -inf rows differ from the rows that see nothing"
    assert np.all(np.isneginf(got[empty])), "a row that sees nothing must get lse = -inf"
    err = np.abs(got[~empty] - ref[~empty])
    return (float(err.max()) if err.size else 0.0), (float((err / bar[~empty]).max()) if err.size else 0.0)


def check_lse(w, got, ref, rows=None, what="LSE"):
    """LSE of every row (or of the sampled rows=(t, h)) within its own bar."""
    mx, ratio = lse_errors(w, got, ref, rows)
    print(f"  {what}: max err {mx:.3e}, largest err / bar {ratio:.3f}", flush=True)
    assert ratio <= 1.0, (what, mx, ratio)


def check_mass(w, got, ref, what="mass"):
    """Mass of every slot j < kv_len of every request within its own bar
    (a slot that holds no usable key must get 0 within 1e-7)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bar = np.maximum(mass_bar(w, ref), 1e-7)
    worst = 0.0
    for r in range(w.batch):
        n = int(w.kv_len[r])
        err = np.abs(got[r, :n] - ref[r, :n])
        assert np.all(err <= bar[r, :n]), (what, r, float(np.nanmax(err / bar[r, :n])), int(np.isnan(err).sum()))
        if n:
            worst = max(worst, float((err / bar[r, :n]).max()))
    print(f"  {what}: largest err / bar {worst:.3f}", flush=True)


def bf16(x) -> np.ndarray:
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def f32(b) -> np.ndarray:
    return bf16_bits_to_f32(b)


def dense_workload(*, Hq: int, Hkv: int, d: int, theta: float, keys: Sequence[np.ndarray],
                   values: Sequence[np.ndarray], pis: Sequence[Sequence[int]],
                   queries: Sequence[np.ndarray], qpos: Sequence[Sequence[int]],
                   spans: Sequence[Sequence[tuple]] = (), ratio: float = 0.25,
                   seed: int = 0, extra_blocks: int = 0, fuse_cap: Sequence[int] = ()) -> Workload:
    """Pack dense per-request key/value rows into a randomly placed paged pool.

    keys[r], values[r]: float arrays [n_r, Hkv, d] (rounded to bf16 here);
    pis[r]: logical positions of those rows (-1 = empty); queries[r]:
    [nq_r, Hq, d]; qpos[r]: their positions.  spans[r]: (start, len) pairs in
    request-sequence indices.  fuse_cap[r] rows of private blocks are appended.
    """
    rng = np.random.default_rng(seed)
    B = len(keys)
    caps = list(fuse_cap) if len(fuse_cap) else [0] * B
    nblk = [(len(keys[r]) + BLOCK - 1) // BLOCK + (caps[r] + BLOCK - 1) // BLOCK for r in range(B)]
    total = sum(nblk) + extra_blocks
    perm = rng.permutation(total).astype(np.int32)
    max_blocks = max(max(nblk), 1)
    bt = np.full((B, max_blocks), -1, np.int32)
    kv_pos = np.full((B, max_blocks * BLOCK), -1, np.int32)
    kv_len = np.zeros(B, np.int32)
    pool_k = bf16(rng.standard_normal((total, Hkv, BLOCK, d)))
    pool_v_tok = bf16(rng.standard_normal((total, Hkv, BLOCK, d)))
    nxt = 0
    for r in range(B):
        n = len(keys[r])
        kb = bf16(np.asarray(keys[r], np.float64).reshape(n, Hkv, d))
        vb = bf16(np.asarray(values[r], np.float64).reshape(n, Hkv, d))
        for i in range(nblk[r]):
            bt[r, i] = perm[nxt + i]
        for j in range(n):
            blk = bt[r, j // BLOCK]
            pool_k[blk, :, j % BLOCK, :] = kb[j]
            pool_v_tok[blk, :, j % BLOCK, :] = vb[j]
        kv_pos[r, :n] = np.asarray(pis[r], np.int32)
        kv_len[r] = n
        nxt += nblk[r]
    pool_v = np.ascontiguousarray(pool_v_tok.transpose(0, 1, 3, 2))
    q = np.concatenate([bf16(np.asarray(qq, np.float64).reshape(-1, Hq, d)) for qq in queries], 0)
    q_start = np.zeros(B + 1, np.int32)
    q_start[1:] = np.cumsum([len(qp) for qp in qpos])
    q_pos = np.concatenate([np.asarray(qp, np.int32) for qp in qpos])
    sr, ss, sl = [], [], []
    for r in range(B):
        for (st, L) in (spans[r] if len(spans) else []):
            sr.append(r)
            ss.append(st)
            sl.append(L)
    cap = int(sum(caps))
    return Workload(
        name="dense", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rope_theta=float(theta),
        max_position=65536, batch=B, pool_k=pool_k, pool_v=pool_v, block_table=bt,
        kv_len=kv_len, kv_pos=kv_pos, q=q, q_start=q_start, q_pos=q_pos,
        span_req=np.asarray(sr, np.int32), span_start=np.asarray(ss, np.int32),
        span_len=np.asarray(sl, np.int32), ratio=ratio,
        fresh_k=bf16(rng.standard_normal((cap, Hkv, d))), fresh_v=bf16(rng.standard_normal((cap, Hkv, d))),
        fuse_cap=np.asarray(caps, np.int32), shared_blocks=np.zeros(0, np.int32), seed=seed)


def gather_dense(w: Workload, r: int):
    """Request r's cached rows in sequence order: K [n, Hkv, d] and
    V [n, Hkv, d] as float64, and pi [n] (layout walk only)."""
    n = int(w.kv_len[r])
    K = np.zeros((n, w.num_kv_heads, w.head_dim))
    V = np.zeros((n, w.num_kv_heads, w.head_dim))
    for j in range(n):
        blk = w.block_table[r, j // BLOCK]
        K[j] = f32(w.pool_k[blk, :, j % BLOCK, :])
        V[j] = f32(w.pool_v[blk, :, :, j % BLOCK])
    return K, V, w.kv_pos[r, :n].astype(np.int64)


def parity_stats(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    rel = float(np.linalg.norm((got - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-30))
    return float(diff.max()) if diff.size else 0.0, float(diff.mean()) if diff.size else 0.0, rel


def out_within(got, ref) -> bool:
    mx, mean, rel = parity_stats(got, ref)
    return mx <= O_MAX_ABS and mean <= O_MEAN_ABS and rel <= O_REL_L2


def check_selection(gpu_off, gpu_idx, ref_off, ref_idx, ref_mass, w: Workload, band: float = None):
    """Selection contract: same CSR sizes; per span, every oracle-selected
    token outside the tie band is chosen and every oracle-rejected one outside
    the band is not; the output is ascending and in the span.

    band None (a mass selection): token j's band is the sum of its own mass
    bar and the boundary token's (the bars check_mass holds each slot to),
    at least SEL_BAND.  Two masses closer than that may come out in either
    order within their bars.  A float: that band for every token (scores
    with their own error bound, such as key norms)."""
    bars = mass_bar(w, ref_mass) if band is None else None
    gpu_off = np.asarray(gpu_off)
    ref_off = np.asarray(ref_off)
    assert np.array_equal(gpu_off, ref_off), "per-span counts differ"
    for s in range(len(w.span_req)):
        r, st, L = int(w.span_req[s]), int(w.span_start[s]), int(w.span_len[s])
        g = np.asarray(gpu_idx[gpu_off[s]:gpu_off[s + 1]])
        o = np.asarray(ref_idx[ref_off[s]:ref_off[s + 1]])
        k = len(o)
        assert len(g) == k
        if k == 0:
            continue
        assert np.all(np.diff(g) > 0), "not ascending / duplicates"
        assert g.min() >= st and g.max() < st + L
        assert np.all(w.kv_pos[r, g] >= 0)
        m = ref_mass[r]
        jb = int(o[np.argmin(m[o])])
        boundary = m[jb]
        cand = [j for j in range(st, st + L) if j < w.kv_len[r] and w.kv_pos[r, j] >= 0]
        gs, os_ = set(g.tolist()), set(o.tolist())
        for j in cand:
            tol = band if bars is None else max(SEL_BAND, float(bars[r, j] + bars[r, jb]))
            if abs(m[j] - boundary) <= tol:
                continue
            assert (j in gs) == (j in os_), f"span {s} token {j} mass {m[j]} boundary {boundary}"
