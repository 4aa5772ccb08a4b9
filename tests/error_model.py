"""Error bars of the GPU path's LSE (per query row) and selection mass (per
slot), derived from the rounding the kernels perform.

The kernels round the rotated query and the rotated key to bf16 (unit
roundoff u = 2^-8, round to nearest even) before the score MFMA, and round
the probabilities to bf16 before the MFMA that sums them (row sums in the
attention kernels, column sums in the mass kernel).  Every other step runs in
fp32 (cos/sin table rows, rotation, accumulation, exp2, merges) and adds
errors orders of magnitude smaller.  Write each rounding as x(1 + e) with
|e| <= u; RNE errors are zero-mean and independent from element to element,
with standard deviation at most u / sqrt(3).

LSE of one row (rotated query q', softmax probabilities p_j over its visible
rotated keys k'_j, kbar = sum_j p_j k'_j), to first order:
    dlse = sum_i q'_i e_qi kbar_i / sqrt(d)                (A, the query's roundings)
         + sum_j p_j sum_i q'_i k'_ij e_kij / sqrt(d)       (B, the keys' roundings)
         + sum_j p_j e_pj                                  (C, bf16 probabilities)
Each part is a sum of many independent zero-mean terms, so dlse is close to
normal with variance
    u^2/3 (sum_i q'_i^2 kbar_i^2 / d + sum_j p_j^2 sum_i q'_i^2 k'_ij^2 / d + sum_j p_j^2)
and the bar is Z standard deviations plus 1e-5.  A long row of near-uniform
weights has a small sum_j p_j^2, so the B and C parts shrink with its
effective key count 1 / sum_j p_j^2; the A part does not when kbar leans
towards q' (as it does for scores of unit variance).

Mass of one slot j of a request (sum over its query rows r of p_rj), with
dmass_j = sum_r p_rj (dscore_rj - dlse_r + e_prj):
  * the key's own rounding is shared by every row of its kv head g; that part
    is qbar_gj . (k'_gj o e_kgj) / sqrt(d) with qbar_gj = sum_{r in g} p_rj q'_r,
    variance u^2/3 sum_i qbar_gji^2 k'_gji^2 / d;
  * the rest (the row's query rounding, its LSE error, the probability's own
    rounding) is independent from row to row: variance
    sum_r p_rj^2 (u^2/3 (sum_i q'_ri^2 k'_ij^2 / d + 1) + var(dlse_r));
  * the bar is Z standard deviations of the sum, plus 2e-4 of the mass and
    1e-7 for the fp32 accumulation over many rows.

The quantities come from the inputs in float64 (the rotation below is the
half-split RoPE the method uses; the bars need only magnitudes of products of
rotated vectors).  This module computes tolerances, not reference outputs:
outputs are always compared with the oracle's.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from position_independent_attention_amd.workloads import BLOCK, bf16_bits_to_f32

U = 2.0 ** -8          # bf16 unit roundoff
Z = 5.5                # standard deviations (the models' variances take the RNE error as
                       # uniform on [-u, u], about 15% above its true spread)
LSE_FLOOR = 1e-5
MASS_REL_FLOOR = 2e-4
MASS_ABS_FLOOR = 1e-7


def _rotate(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-2.0 * np.arange(half) / d)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[:, :half], x[:, half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=1)


def _usable_slots(w, r: int):
    n = int(w.kv_len[r])
    j = np.arange(n)
    pi = w.kv_pos[r, :n].astype(np.int64)
    blk = w.block_table[r, j // BLOCK].astype(np.int64)
    ok = (pi >= 0) & (pi < w.max_position) & (blk >= 0) & (blk < w.pool_k.shape[0])
    return j[ok], pi[ok], blk[ok]


def _keys(w, r: int, g: int, slots, pis, blks) -> np.ndarray:
    k = bf16_bits_to_f32(w.pool_k[blks, g, slots % BLOCK, :]).astype(np.float64)
    return _rotate(k, pis, w.rope_theta)


def bars(w, rows: Optional[Tuple[np.ndarray, np.ndarray]] = None, with_mass: bool = False):
    """Model bars: lse [total_q, Hq] (or [n] for rows=(t, h)), NaN where a row
    sees nothing, and with with_mass the mass bar [B, max_blocks*16]."""
    d = int(w.head_dim)
    G = int(w.num_q_heads) // int(w.num_kv_heads)
    sq = np.sqrt(d)
    if rows is None:
        lse_bar = np.full((int(w.q.shape[0]), int(w.num_q_heads)), np.nan)
    else:
        rt, rh = np.asarray(rows[0]), np.asarray(rows[1])
        lse_bar = np.full(rt.shape[0], np.nan)
    mass_bar = np.zeros(w.kv_pos.shape) if with_mass else None
    q_all = bf16_bits_to_f32(w.q).astype(np.float64)
    for r in range(int(w.batch)):
        q0, q1 = int(w.q_start[r]), int(w.q_start[r + 1])
        if q1 == q0:
            continue
        slots, pis, blks = _usable_slots(w, r)
        var = np.zeros(slots.shape[0])
        msum = np.zeros(slots.shape[0])
        for g in range(int(w.num_kv_heads)):
            if rows is None:
                tt = np.repeat(np.arange(q0, q1), G)
                hh = np.tile(np.arange(g * G, (g + 1) * G), q1 - q0)
                where = None
            else:
                sel = (rt >= q0) & (rt < q1) & (rh // G == g)
                if not sel.any():
                    continue
                where = np.nonzero(sel)[0]
                tt, hh = rt[where], rh[where]
            pos = w.q_pos[tt].astype(np.int64)
            live = (pos >= 0) & (pos < w.max_position)
            if slots.shape[0] == 0 or not live.any():
                continue
            kr = _keys(w, r, g, slots, pis, blks)                       # [n, d]
            qr = _rotate(q_all[tt, hh], np.where(live, pos, 0), w.rope_theta)  # [R, d]
            vis = (pis[None, :] <= pos[:, None]) & live[:, None]
            s = np.where(vis, qr @ kr.T / sq, -np.inf)
            m = s.max(axis=1)
            seen = np.isfinite(m)
            e = np.where(vis, np.exp(s - np.where(seen, m, 0.0)[:, None]), 0.0)
            z = e.sum(axis=1)
            p = e / np.where(seen, z, 1.0)[:, None]                     # [R, n]
            kbar = p @ kr
            qk2 = (qr ** 2) @ (kr ** 2).T / d                           # [R, n]
            b2 = (p ** 2 * qk2).sum(axis=1)
            c2 = (p ** 2).sum(axis=1)
            var_lse = U ** 2 / 3.0 * (((qr * kbar) ** 2).sum(axis=1) / d + b2 + c2)
            bar = np.where(seen, Z * np.sqrt(var_lse) + LSE_FLOOR, np.nan)
            if where is None:
                lse_bar[tt, hh] = bar
            else:
                lse_bar[where] = bar
            if with_mass:
                qbar = p.T @ qr                                         # [n, d]
                var += U ** 2 / 3.0 * ((qbar * kr) ** 2).sum(axis=1) / d
                var += (p ** 2 * (U ** 2 / 3.0 * (qk2 + 1.0) + var_lse[:, None])).sum(axis=0)
                msum += p.sum(axis=0)
        if with_mass:
            mass_bar[r, slots] = Z * np.sqrt(var) + MASS_REL_FLOOR * msum + MASS_ABS_FLOOR
    return (lse_bar, mass_bar) if with_mass else lse_bar
