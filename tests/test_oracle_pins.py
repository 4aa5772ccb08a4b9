"""The CPU oracle against what the pages and the mathematics fix.

Every pin here uses a route other than the oracle's own code: a matrix
exponential for the rotation, the polar form and the relative-position form
for scores, dense textbook attention (torch SDPA on pre-rotated keys),
invariants (shift, permutation, normalisation, total mass), brute force on
tiny inputs and closed-form special cases.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from position_independent_attention_amd import workloads as W
from tests.util import BLOCK, dense_workload, f32, gather_dense, parity_stats

HERE = os.path.dirname(os.path.abspath(__file__))


def rot_generator(d, theta):
    """Skew generator whose exponential turns pair (i, i+d/2) by theta^(-2i/d)
    per unit of position, counter-clockwise."""
    A = np.zeros((d, d))
    for i in range(d // 2):
        w = theta ** (-2.0 * i / d)
        A[i + d // 2, i] = w
        A[i, i + d // 2] = -w
    return A


def rot_matrix(d, theta, pos):
    return scipy.linalg.expm(pos * rot_generator(d, theta))


# ---------------------------------------------------------------- rotation

@pytest.mark.parametrize("d", [2, 4, 8, 64])
@pytest.mark.parametrize("pos", [0, 1, 7, 1000, 40000])
def test_rope_equals_matrix_exponential(d, pos):
    rng = np.random.default_rng(d * 100 + pos)
    x = rng.standard_normal(d)
    want = rot_matrix(d, 1e4, pos) @ x
    got = oracle.rope(d, 1e4, pos, x)
    assert np.max(np.abs(got - want)) < 1e-9 * max(1.0, pos * 1e-3)


def test_rope_zero_position_is_identity_and_norm_preserving():
    rng = np.random.default_rng(3)
    x = rng.standard_normal(128)
    assert np.array_equal(oracle.rope(128, 5e5, 0, x), x)
    y = oracle.rope(128, 5e5, 12345, x)
    assert abs(np.linalg.norm(y) - np.linalg.norm(x)) < 1e-12


def test_closed_form_d2_golden():
    """tests/golden/rope_d2_closed_form.json: polar-form scores of a d = 2 case."""
    g = json.load(open(os.path.join(HERE, "golden", "rope_d2_closed_form.json")))
    keys = np.array(g["keys"], np.float64)[:, None, :]
    vals = np.array(g["values"], np.float64)[:, None, :]
    w = dense_workload(Hq=1, Hkv=1, d=2, theta=g["theta"], keys=[keys], values=[vals],
                       pis=[g["key_pos"]], queries=[np.array(g["q"])[None, None, :]],
                       qpos=[[g["q_pos"]]])
    out, lse = oracle.attention(w)
    assert abs(lse[0, 0] - g["expected_lse"]) < 1e-12
    assert np.max(np.abs(out[0, 0] - np.array(g["expected_out"]))) < 1e-12
    m = oracle.mass(w)[0, :len(g["keys"])]
    assert np.max(np.abs(m - np.array(g["expected_prob"]))) < 1e-12


# ------------------------------------------------------ dense formulations

def relative_form_attention(w, r):
    """Scores from the relative-position form: for each frequency pair,
    (q_a k_a + q_b k_b) cos(phi) + (q_b k_a - q_a k_b) sin(phi) with
    phi = (pi - t) * theta^(-2i/d); then softmax over visible keys."""
    K, V, pi = gather_dense(w, r)
    d, Hq, G = w.head_dim, w.num_q_heads, w.group
    half = d // 2
    freqs = w.rope_theta ** (-2.0 * np.arange(half) / d)
    outs, lses = [], []
    for t in range(w.q_start[r], w.q_start[r + 1]):
        pos = int(w.q_pos[t])
        vis = (pi >= 0) & (pi <= pos)
        phi = (pi[:, None] - pos) * freqs[None, :]
        c, s = np.cos(phi), np.sin(phi)
        o_t, l_t = [], []
        for h in range(Hq):
            q = f32(w.q[t, h]).astype(np.float64)
            k = K[:, h // G, :]
            qa, qb, ka, kb = q[:half], q[half:], k[:, :half], k[:, half:]
            sc = ((qa * ka + qb * kb) * c + (qb * ka - qa * kb) * s).sum(1) / math.sqrt(d)
            sc = np.where(vis, sc, -np.inf)
            mx = sc.max()
            p = np.exp(sc - mx)
            z = p.sum()
            o_t.append((p / z) @ V[:, h // G, :])
            l_t.append(mx + math.log(z))
        outs.append(o_t)
        lses.append(l_t)
    return np.array(outs), np.array(lses)


@pytest.mark.parametrize("make", [W.tiny, lambda: W.custom(7, Hq=8, Hkv=2, d=16, theta=1e4,
                                                            span_lens=[[40, 23], [16]],
                                                            gaps=[[5, 300], [1000]],
                                                            q_len=[5, 3], q_gap=[2, 0])])
def test_relative_position_form(make):
    w = make()
    out, lse = oracle.attention(w)
    for r in range(w.batch):
        o2, l2 = relative_form_attention(w, r)
        sl = slice(w.q_start[r], w.q_start[r + 1])
        assert np.max(np.abs(out[sl] - o2)) < 1e-10
        assert np.max(np.abs(lse[sl] - l2)) < 1e-10


def prerotated(w, r):
    """Request r rotated once, with complex multiplication (pair (i, i+d/2) as
    real and imaginary part): queries at t, keys at pi, float64.  Returns
    Q [Hq, nq, d], K and V [Hq, n, d] (kv heads repeated over their group)
    and the visibility mask [nq, n]."""
    K, V, pi = gather_dense(w, r)
    d, G = w.head_dim, w.group
    half = d // 2
    freqs = torch.tensor(w.rope_theta ** (-2.0 * np.arange(half) / d), dtype=torch.float64)

    def rot(x, pos):  # x [n, H, d], pos [n]
        x = torch.as_tensor(x, dtype=torch.float64)
        z = torch.complex(x[..., :half], x[..., half:])
        ang = torch.as_tensor(pos, dtype=torch.float64)[:, None, None] * freqs
        z = z * torch.polar(torch.ones_like(ang), ang)
        return torch.cat([z.real, z.imag], -1)

    sl = slice(int(w.q_start[r]), int(w.q_start[r + 1]))
    qpos = w.q_pos[sl].astype(np.int64)
    Q = rot(f32(w.q[sl]).astype(np.float64), qpos)              # [nq, Hq, d]
    Kr = rot(K, np.maximum(pi, 0))                             # [n, Hkv, d]
    Kr = Kr.repeat_interleave(G, dim=1)
    Vr = torch.as_tensor(V).repeat_interleave(G, dim=1)
    mask = torch.as_tensor((pi[None, :] >= 0) & (pi[None, :] <= qpos[:, None]))
    return Q.transpose(0, 1), Kr.transpose(0, 1), Vr.transpose(0, 1), mask


def prerotated_sdpa(w, r):
    """Textbook attention (torch scaled_dot_product_attention, CPU float64)
    with a boolean mask over the once-rotated tensors."""
    Q, K, V, mask = prerotated(w, r)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask[None])
    s = (Q @ K.transpose(1, 2)) / math.sqrt(w.head_dim)
    s = s.masked_fill(~mask[None], -math.inf)
    return o.transpose(0, 1).numpy(), torch.logsumexp(s, -1).transpose(0, 1).numpy()


def prerotated_mass(w, r):
    """Selection mass of request r by another route: torch.softmax over the
    masked scores of the once-rotated tensors, summed over the request's
    query tokens and every q head, per slot."""
    Q, K, _, mask = prerotated(w, r)
    s = (Q @ K.transpose(1, 2)) / math.sqrt(w.head_dim)
    p = torch.softmax(s.masked_fill(~mask[None], -math.inf), -1)
    return torch.nan_to_num(p, nan=0.0).sum((0, 1)).numpy()   # rows that see nothing add nothing


@pytest.mark.parametrize("name", ["tiny", "gqa_ragged", "mha"])
def test_prerotation_equivalence(name):
    """The in-kernel rotation is algebraically equivalent to re-rotating the
    cache hits and running standard attention (MiniPIC section 2.1)."""
    if name == "tiny":
        w = W.tiny()
    elif name == "gqa_ragged":
        w = W.custom(11, Hq=6, Hkv=2, d=32, theta=5e5, span_lens=[[33, 70, 16], [5]],
                     gaps=[[0, 9000, 1], [77]], q_len=[7, 2], q_gap=[0, 3])
    else:
        w = W.custom(12, Hq=2, Hkv=2, d=64, theta=1e4, span_lens=[[50]], q_len=[9])
    out, lse = oracle.attention(w)
    for r in range(w.batch):
        o2, l2 = prerotated_sdpa(w, r)
        sl = slice(w.q_start[r], w.q_start[r + 1])
        assert np.max(np.abs(out[sl] - o2)) < 1e-10
        assert np.max(np.abs(lse[sl] - l2)) < 1e-10


@pytest.mark.parametrize("seed", [21, 22])
def test_mass_equals_summed_softmax_per_slot(seed):
    """The mass of every slot, not only its total, against the summed
    probabilities of textbook softmax attention (QCFuse methodology B: the
    query's attention over the layer's keys scores each token); masked slots
    hold pi = -1 and get none."""
    w = W.custom(seed, Hq=6, Hkv=2, d=32, theta=5e5, span_lens=[[40, 17], [30]], gaps=[[0, 500], [3]],
                 q_len=[5, 3], q_gap=[0, 2])
    w.kv_pos[0, [3, 20, 41]] = -1
    mass = oracle.mass(w)
    for r in range(w.batch):
        n = int(w.kv_len[r])
        ref = prerotated_mass(w, r)
        assert np.max(np.abs(mass[r, :n] - ref)) < 1e-10
    assert np.all(mass[0, [3, 20, 41]] == 0)


def test_identity_positions_is_causal_rope_attention():
    """pi = identity with the queries as the last tokens: standard causal RoPE
    self-attention (every query sees itself and everything before it)."""
    rng = np.random.default_rng(5)
    n, nq, d, Hq, Hkv = 40, 6, 16, 4, 2
    K = rng.standard_normal((n, Hkv, d))
    V = rng.standard_normal((n, Hkv, d))
    Qx = rng.standard_normal((nq, Hq, d))
    w = dense_workload(Hq=Hq, Hkv=Hkv, d=d, theta=1e4, keys=[K], values=[V], pis=[list(range(n))],
                       queries=[Qx], qpos=[list(range(n - nq, n))])
    out, lse = oracle.attention(w)
    o2, l2 = prerotated_sdpa(w, 0)
    assert np.max(np.abs(out - o2)) < 1e-10
    # Built without a mask from pi: plain lower-triangular causality.
    Kd, Vd, _ = gather_dense(w, 0)
    half = d // 2
    fr = 1e4 ** (-2.0 * np.arange(half) / d)
    for t in range(nq):
        for h in range(Hq):
            q = f32(w.q[t, h]).astype(np.float64)
            qr = rot_matrix(d, 1e4, n - nq + t) @ q
            ks = np.stack([rot_matrix(d, 1e4, j) @ Kd[j, h // 2] for j in range(n - nq + t + 1)])
            sc = ks @ qr / math.sqrt(d)
            p = np.exp(sc - sc.max())
            assert abs(lse[t, h] - (sc.max() + math.log(p.sum()))) < 1e-10
            assert np.max(np.abs(out[t, h] - (p / p.sum()) @ Vd[:n - nq + t + 1, h // 2])) < 1e-10


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("c", [1, 1000, 2 ** 14])
def test_shift_invariance(c):
    """Only t - pi(j) matters: shifting every logical position leaves O, lse and
    the selection mass unchanged."""
    w = W.custom(21, Hq=4, Hkv=2, d=32, theta=1e4, span_lens=[[48, 31]], gaps=[[3, 100]],
                 q_len=[6], q_gap=[4])
    out, lse = oracle.attention(w)
    m = oracle.mass(w)
    w2 = w.copy()
    w2.kv_pos = np.where(w.kv_pos >= 0, w.kv_pos + c, -1).astype(np.int32)
    w2.q_pos = (w.q_pos + c).astype(np.int32)
    out2, lse2 = oracle.attention(w2)
    assert np.max(np.abs(out - out2)) < 1e-9
    assert np.max(np.abs(lse - lse2)) < 1e-9
    assert np.max(np.abs(m - oracle.mass(w2))) < 1e-9


def test_rows_sum_to_one_and_total_mass():
    w = W.custom(22, Hq=8, Hkv=2, d=32, theta=5e5, span_lens=[[64, 17], [20]],
                 gaps=[[0, 50], [9]], q_len=[5, 4])
    w1 = w.copy()
    w1.pool_v[:] = 0x3F80                                     # bf16 1.0 everywhere
    out, _ = oracle.attention(w1)
    assert np.max(np.abs(out - 1.0)) < 1e-12                  # sum_j p_j = 1 per row
    m = oracle.mass(w)
    for r in range(w.batch):
        nq = w.q_start[r + 1] - w.q_start[r]
        assert abs(m[r].sum() - nq * w.num_q_heads) < 1e-9
        assert np.all(m[r][: w.kv_len[r]][w.kv_pos[r, : w.kv_len[r]] < 0] == 0)


def test_span_permutation_and_placement_invariance():
    """Moving spans to other physical blocks and to other places in the request
    sequence, with their pi attached, leaves every output unchanged; the mass
    moves with its token (positional, not index-based, masking)."""
    rng = np.random.default_rng(9)
    d, Hq, Hkv = 16, 4, 1
    spans = [(rng.standard_normal((32, Hkv, d)), rng.standard_normal((32, Hkv, d)), 100 + 40 * i)
             for i in range(3)]
    own_k, own_v = rng.standard_normal((4, Hkv, d)), rng.standard_normal((4, Hkv, d))
    Qx = rng.standard_normal((4, Hq, d))

    def build(order, seed):
        K = np.concatenate([spans[i][0] for i in order] + [own_k])
        V = np.concatenate([spans[i][1] for i in order] + [own_v])
        pi = sum([list(range(spans[i][2], spans[i][2] + 32)) for i in order], []) + [300, 301, 302, 303]
        return dense_workload(Hq=Hq, Hkv=Hkv, d=d, theta=1e4, keys=[K], values=[V], pis=[pi],
                              queries=[Qx], qpos=[[300, 301, 302, 303]], seed=seed)

    a, b = build([0, 1, 2], 1), build([2, 0, 1], 2)
    oa, la = oracle.attention(a)
    ob, lb = oracle.attention(b)
    assert np.max(np.abs(oa - ob)) < 1e-12 and np.max(np.abs(la - lb)) < 1e-12
    ma, mb = oracle.mass(a)[0], oracle.mass(b)[0]
    # span 2 sits at 64..95 in a, at 0..31 in b
    assert np.max(np.abs(ma[64:96] - mb[0:32])) < 1e-12
    assert np.max(np.abs(ma[0:32] - mb[32:64])) < 1e-12


# ---------------------------------------------------------------- special cases

def test_single_visible_key_returns_its_value():
    rng = np.random.default_rng(13)
    K = rng.standard_normal((20, 1, 8))
    V = rng.standard_normal((20, 1, 8))
    pi = [50 + j for j in range(20)]
    pi[7] = 3                                                  # only this one precedes the query
    w = dense_workload(Hq=2, Hkv=1, d=8, theta=1e4, keys=[K], values=[V], pis=[pi],
                       queries=[rng.standard_normal((1, 2, 8))], qpos=[[10]])
    out, lse = oracle.attention(w)
    _, Vd, _ = gather_dense(w, 0)
    assert np.max(np.abs(out[0] - Vd[7, 0])) < 1e-14
    qr = rot_matrix(8, 1e4, 10) @ f32(w.q[0, 0]).astype(np.float64)
    kr = rot_matrix(8, 1e4, 3) @ gather_dense(w, 0)[0][7, 0]
    assert abs(lse[0, 0] - qr @ kr / math.sqrt(8)) < 1e-12


def test_zero_keys_give_uniform_weights():
    rng = np.random.default_rng(14)
    V = rng.standard_normal((30, 2, 8))
    pi = list(range(30))
    w = dense_workload(Hq=4, Hkv=2, d=8, theta=1e4, keys=[np.zeros((30, 2, 8))], values=[V],
                       pis=[pi], queries=[rng.standard_normal((2, 4, 8))], qpos=[[11, 29]])
    out, lse = oracle.attention(w)
    _, Vd, _ = gather_dense(w, 0)
    for t, pos in enumerate([11, 29]):
        for h in range(4):
            assert np.max(np.abs(out[t, h] - Vd[: pos + 1, h // 2].mean(0))) < 1e-12
            assert abs(lse[t, h] - math.log(pos + 1)) < 1e-12


def test_all_positions_zero_is_unrotated_attention():
    rng = np.random.default_rng(15)
    K = rng.standard_normal((24, 1, 16))
    V = rng.standard_normal((24, 1, 16))
    w = dense_workload(Hq=1, Hkv=1, d=16, theta=1e4, keys=[K], values=[V], pis=[[0] * 24],
                       queries=[rng.standard_normal((1, 1, 16))], qpos=[[0]])
    out, lse = oracle.attention(w)
    Kd, Vd, _ = gather_dense(w, 0)
    q = f32(w.q[0, 0]).astype(np.float64)
    sc = Kd[:, 0] @ q / 4.0
    p = np.exp(sc - sc.max())
    assert np.max(np.abs(out[0, 0] - (p / p.sum()) @ Vd[:, 0])) < 1e-12


def test_empty_visible_set():
    w = dense_workload(Hq=1, Hkv=1, d=4, theta=1e4, keys=[np.ones((3, 1, 4))],
                       values=[np.ones((3, 1, 4))], pis=[[5, 6, -1]],
                       queries=[np.ones((1, 1, 4))], qpos=[[2]])
    out, lse = oracle.attention(w)
    assert np.all(out == 0) and lse[0, 0] == -np.inf


# ---------------------------------------------------------------- brute force

def brute_force(w):
    """Explicit d x d rotation matrices (matrix exponential) and direct sums."""
    outs, lses, mass = [], [], np.zeros(w.kv_pos.shape)
    for r in range(w.batch):
        K, V, pi = gather_dense(w, r)
        for t in range(w.q_start[r], w.q_start[r + 1]):
            o_t, l_t = [], []
            for h in range(w.num_q_heads):
                g = h // w.group
                qr = rot_matrix(w.head_dim, w.rope_theta, int(w.q_pos[t])) @ f32(w.q[t, h]).astype(np.float64)
                sc = {}
                for j in range(len(pi)):
                    if 0 <= pi[j] <= w.q_pos[t]:
                        kr = rot_matrix(w.head_dim, w.rope_theta, int(pi[j])) @ K[j, g]
                        sc[j] = float(qr @ kr) / math.sqrt(w.head_dim)
                z = sum(math.exp(v) for v in sc.values())
                o = sum((math.exp(v) / z) * V[j, g] for j, v in sc.items())
                for j, v in sc.items():
                    mass[r, j] += math.exp(v) / z
                o_t.append(o)
                l_t.append(math.log(z))
            outs.append(o_t)
            lses.append(l_t)
    return np.array(outs), np.array(lses), mass


@pytest.mark.parametrize("d", [2, 4])
def test_brute_force_tiny(d):
    rng = np.random.default_rng(30 + d)
    K = rng.standard_normal((8, 1, d))
    V = rng.standard_normal((8, 1, d))
    pi = [3, 9, -1, 0, 14, 2, 7, 12]
    w = dense_workload(Hq=2, Hkv=1, d=d, theta=1e4, keys=[K], values=[V], pis=[pi],
                       queries=[rng.standard_normal((3, 2, d))], qpos=[[7, 12, 20]],
                       spans=[[(0, 8)]], ratio=0.4)
    out, lse = oracle.attention(w)
    bo, bl, bm = brute_force(w)
    assert np.max(np.abs(out - bo)) < 1e-12
    assert np.max(np.abs(lse - bl)) < 1e-12
    m = oracle.mass(w)
    assert np.max(np.abs(m[0, :8] - bm[0, :8])) < 1e-12
    # top-k by enumerating every k-subset of the candidates: the best subset
    # maximises total mass, ties to the lexicographically smallest index set.
    off, idx = oracle.select(w, m)
    cand = [j for j in range(8) if pi[j] >= 0]
    k = min(len(cand), int(math.floor(0.4 * 8 + 0.5)))
    best = max(itertools.combinations(cand, k),
               key=lambda S: (round(sum(m[0, j] for j in S), 12), [-j for j in S]))
    assert list(idx) == sorted(best)


def test_select_ties_go_to_lower_index_and_respect_masks():
    w = dense_workload(Hq=1, Hkv=1, d=2, theta=1e4, keys=[np.zeros((20, 1, 2))],
                       values=[np.zeros((20, 1, 2))], pis=[list(range(20))],
                       queries=[np.zeros((1, 1, 2))], qpos=[[30]],
                       spans=[[(0, 10), (10, 10)]], ratio=0.35)
    m = np.zeros(w.kv_pos.shape)
    m[0, :20] = [5, 1, 1, 1, 7, 1, 1, 1, 1, 2,  3, 3, 3, 3, 0, 0, 9, 3, 3, 3]
    w.kv_pos[0, 4] = -1                          # masked: never a candidate
    off, idx = oracle.select(w, m)
    # k = floor(0.35*10 + 0.5) = 4 per span
    assert list(off) == [0, 4, 8]
    assert list(idx[:4]) == [0, 1, 2, 9]         # 5, 2, then ties at 1 -> 1, 2
    assert list(idx[4:]) == [10, 11, 12, 16]     # 9, then the lowest three 3s


def test_select_budget_rounding_and_small_spans():
    w = dense_workload(Hq=1, Hkv=1, d=2, theta=1e4, keys=[np.zeros((40, 1, 2))],
                       values=[np.zeros((40, 1, 2))], pis=[list(range(40))],
                       queries=[np.zeros((1, 1, 2))], qpos=[[50]],
                       spans=[[(0, 10), (10, 1), (11, 3), (14, 26)]], ratio=0.15)
    m = np.random.default_rng(1).random(w.kv_pos.shape)
    w.kv_pos[0, 11:14] = [-1, -1, 12]
    off, _ = oracle.select(w, m)
    # 0.15*10+.5 = 2.0 -> 2; 0.15*1+.5 -> 0; 0.15*3+.5 = 0.95 -> 0; 0.15*26+.5 = 4.4 -> 4
    assert list(np.diff(off)) == [2, 0, 0, 4]


# ---------------------------------------------------------------- needles

def test_planted_needles_are_selected():
    """Keys built so that, after rotation to their pi, each aligns with one
    rotated query row must receive the largest mass in their span."""
    w = W.tiny()
    d, theta = w.head_dim, w.rope_theta
    needles = {5: (0, 1), 77: (3, 0), 140: (9, 2), 201: (15, 3)}   # slot -> (t, h)
    for j, (t0, h0) in needles.items():
        q = f32(w.q[t0, h0]).astype(np.float64)
        qr = rot_matrix(d, theta, int(w.q_pos[t0])) @ q
        blk = w.block_table[0, j // BLOCK]
        kk = 1.5 * rot_matrix(d, theta, int(w.kv_pos[0, j])).T @ qr
        w.pool_k[blk, 0, j % BLOCK, :] = W.f32_to_bf16_bits(kk.astype(np.float32))
    m = oracle.mass(w)
    off, idx = oracle.select(w, m)
    chosen = set(idx.tolist())
    for lo in (0, 128):
        mine = sorted(j for j in needles if lo <= j < lo + 128)
        top = np.argsort(-m[0, lo:lo + 128], kind="stable")[: len(mine)] + lo
        assert sorted(top.tolist()) == mine
        assert set(mine) <= chosen
    # Span 1 is stored at sequence slots 128..255 but sits at positions
    # 200..327: rotating its keys at the storage slot loses the alignment.
    w2 = w.copy()
    w2.kv_pos[0, :256] = np.arange(256)
    m2 = oracle.mass(w2)
    for j in (140, 201):
        assert m2[0, j] < 0.5 * m[0, j]


# ------------------------------------------------------ anchor key norm

def _slot(w, r, j):
    return int(w.block_table[r, j // BLOCK]), j % BLOCK


def test_key_norm_closed_form_per_head():
    """A slot whose key is the constant c_g on kv head g has squared norm
    d * sum_g c_g^2: every head counts, once (a dropped head, a mean over heads
    or a per-head maximum would all differ)."""
    w = W.custom(121, Hq=8, Hkv=4, d=64, theta=1e4, span_lens=[[40]], q_len=[2])
    consts = [0.5, -1.25, 2.0, 0.0]   # bf16-exact
    blk, off = _slot(w, 0, 7)
    for g, c in enumerate(consts):
        w.pool_k[blk, g, off, :] = W.f32_to_bf16_bits(np.full(64, c, np.float32))
    n = oracle.key_norm(w)
    assert n[0, 7] == 64 * sum(c * c for c in consts)


def test_key_norm_rotation_invariant_and_scaling():
    """RoPE is a rotation: the norm of the key rotated at its pi (through the
    oracle's own rope) equals the stored key's norm; doubling a key (exact in
    bf16) multiplies the squared norm by exactly 4."""
    w = W.tiny()
    n = oracle.key_norm(w)
    for j in (0, 3, 130, 255):
        blk, off = _slot(w, 0, j)
        tot = 0.0
        for g in range(w.num_kv_heads):
            k = f32(w.pool_k[blk, g, off]).astype(np.float64)
            tot += float(np.sum(oracle.rope(w.head_dim, w.rope_theta, int(w.kv_pos[0, j]), k) ** 2))
        assert abs(tot - n[0, j]) <= 1e-9 * n[0, j]
    w2 = w.copy()
    blk, off = _slot(w2, 0, 9)
    w2.pool_k[blk, :, off] = W.f32_to_bf16_bits(2.0 * f32(w2.pool_k[blk, :, off]))
    assert oracle.key_norm(w2)[0, 9] == 4.0 * n[0, 9]


def test_key_norm_masked_slots_and_planted_anchors():
    """Unusable slots score 0 and are never anchors; keys planted with a 4x
    larger scale are the anchors of their spans."""
    w = W.tiny()
    w.kv_pos[0, 20:24] = -1
    planted = {0: [3, 50, 99], 128: [130, 201, 250]}   # span start -> slots
    for js in planted.values():
        for j in js:
            blk, off = _slot(w, 0, j)
            w.pool_k[blk, :, off] = W.f32_to_bf16_bits(4.0 * f32(w.pool_k[blk, :, off]))
    n = oracle.key_norm(w)
    assert np.all(n[0, 20:24] == 0.0)
    off_, idx = oracle.select(w, n, ratio=3 / 128)   # k = 3 per span
    assert idx.tolist() == sorted(sum(planted.values(), []))
    big = oracle.select(w, n, ratio=1.0)[1]
    assert not set(range(20, 24)) & set(big.tolist())


# ---------------------------------------------------------------- fusion

def test_fuse_semantics_against_replaced_dense_rows():
    """Fusing recomputed rows into private blocks is equivalent to replacing
    the selected rows in place (positions kept): attention over the fused
    paged cache equals attention over the dense replaced sequence."""
    w = W.custom(41, Hq=4, Hkv=2, d=16, theta=1e4, span_lens=[[40, 25], [33]],
                 gaps=[[0, 7], [100]], q_len=[3, 2], ratio=0.3)
    m = oracle.mass(w)
    off, idx = oracle.select(w, m)
    req_off = np.zeros(w.batch + 1, np.int32)
    for s in range(len(w.span_req)):
        req_off[w.span_req[s] + 1] += off[s + 1] - off[s]
    req_off = np.cumsum(req_off).astype(np.int32)
    n = int(req_off[-1])
    fk, fv = w.fresh_k[:n], w.fresh_v[:n]
    pk, pv, kp, kl = oracle.fuse(w, idx, req_off, fk, fv)
    fused = w.copy()
    fused.pool_k, fused.pool_v, fused.kv_pos, fused.kv_len = pk, pv, kp, kl
    out_f, lse_f = oracle.attention(fused)
    # shared (span) blocks untouched, bit for bit
    used = set()
    for r in range(w.batch):
        for b in range((w.kv_len[r] + BLOCK - 1) // BLOCK):
            used.add(int(w.block_table[r, b]))
    for b in used:
        assert np.array_equal(pk[b], w.pool_k[b]) and np.array_equal(pv[b], w.pool_v[b])
    # dense replaced sequences
    keys, vals, pis, qs, qp = [], [], [], [], []
    for r in range(w.batch):
        K, V, pi = gather_dense(w, r)
        for i in range(req_off[r], req_off[r + 1]):
            K[idx[i]] = f32(fk[i])
            V[idx[i]] = f32(fv[i])
        keys.append(K)
        vals.append(V)
        pis.append(pi.tolist())
        sl = slice(w.q_start[r], w.q_start[r + 1])
        qs.append(f32(w.q[sl]))
        qp.append(w.q_pos[sl].tolist())
    dense = dense_workload(Hq=4, Hkv=2, d=16, theta=1e4, keys=keys, values=vals, pis=pis,
                           queries=qs, qpos=qp, seed=5)
    out_d, lse_d = oracle.attention(dense)
    assert np.max(np.abs(out_f - out_d)) < 1e-12 and np.max(np.abs(lse_f - lse_d)) < 1e-12
    # layout facts: stale slots masked, fresh slots carry the stale positions
    for r in range(w.batch):
        base = (w.kv_len[r] + BLOCK - 1) // BLOCK * BLOCK
        cnt = req_off[r + 1] - req_off[r]
        assert kl[r] == base + cnt
        assert np.all(kp[r, w.kv_len[r]:base] == -1)
        sel = idx[req_off[r]:req_off[r + 1]]
        assert np.all(kp[r, sel] == -1)
        assert np.array_equal(kp[r, base:base + cnt], w.kv_pos[r, sel])


# ------------------------------------------------------ negative controls

def _max_stats(a, b):
    return parity_stats(a, b)


def _fails_bar(a, b):
    mx, mean, rel = _max_stats(a, b)
    return mx > 2e-2 or mean > 2e-3 or rel > 1e-2


@pytest.mark.parametrize("make", [W.tiny, W.llama_layer])
@pytest.mark.parametrize("mutation", ["pi_off_by_one", "interleaved_pairs", "gqa_mod_map",
                                      "no_causal_mask", "storage_positions"])
def test_negative_controls_exceed_tolerance(make, mutation):
    """Plausible mistakes, planted in the oracle's inputs so that the oracle
    computes the mistaken variant, move the output beyond the parity bar."""
    w = make()
    if make is W.llama_layer:                       # a row sample keeps this quick
        rows = (np.repeat(np.arange(0, 64, 9), 32), np.tile(np.arange(32), 8))
    else:
        rows = None
    ref, _ = oracle.attention(w, rows)
    m = w.copy()
    d = w.head_dim
    if mutation == "pi_off_by_one":
        ctx = np.zeros_like(m.kv_pos, bool)
        for r in range(m.batch):
            ctx[r, : m.kv_len[r] - (m.q_start[r + 1] - m.q_start[r])] = True
        m.kv_pos = np.where(ctx & (m.kv_pos >= 0), m.kv_pos + 1, m.kv_pos).astype(np.int32)
    elif mutation == "interleaved_pairs":
        # pairing (2i, 2i+1) == half-split pairing after moving 2i -> i, 2i+1 -> i + d/2
        perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
        m.q = np.ascontiguousarray(m.q[..., perm])
        m.pool_k = np.ascontiguousarray(m.pool_k[..., perm])
    elif mutation == "gqa_mod_map":
        Hq, Hkv, G = m.num_q_heads, m.num_kv_heads, m.group
        if Hkv == 1:
            pytest.skip("one kv head: every map is the same")
        src = np.empty(Hq, np.int64)
        for h in range(Hq):
            src[(h % Hkv) * G + h // Hkv] = h
        m.q = np.ascontiguousarray(m.q[:, src])
    elif mutation == "no_causal_mask":
        for r in range(m.batch):
            nq = m.q_start[r + 1] - m.q_start[r]
            own = slice(m.kv_len[r] - nq, m.kv_len[r])
            m.kv_pos[r, own] = m.q_pos[m.q_start[r]]
    elif mutation == "storage_positions":
        # the RoPE conflict: each span keeps the rotation of the offset it was
        # cached at (its own start, 0) instead of its position in this request
        for s in range(len(m.span_req)):
            r, st, L = m.span_req[s], m.span_start[s], m.span_len[s]
            m.kv_pos[r, st:st + L] = np.where(m.kv_pos[r, st:st + L] >= 0, np.arange(L), -1)
    if mutation == "gqa_mod_map":
        # the mutated result for original head h sits at head (h % Hkv) * G + h // Hkv
        hp = lambda h: (h % m.num_kv_heads) * m.group + h // m.num_kv_heads
        if rows is None:
            got, _ = oracle.attention(m)
            got = got[:, [hp(h) for h in range(m.num_q_heads)]]
        else:
            got, _ = oracle.attention(m, (rows[0], np.array([hp(h) for h in rows[1]])))
    else:
        got, _ = oracle.attention(m, rows)
    assert _fails_bar(got, ref), _max_stats(got, ref)
