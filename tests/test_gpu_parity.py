"""HIP path vs the CPU oracle, element by element, through the C ABI.

Bar (tests/util.py): bf16 outputs max abs <= 2e-2 and mean abs <= 2e-3 (plus
rel-L2 <= 1e-2); the LSE of each row and the selection mass of each slot within
their own bars from the kernels' bf16 roundings (tests/error_model.py), capped
at 1e-2 and at 2% + 1e-5; selected sets identical outside a 1e-3 band around
each span's k-th mass (ties to the lower index); fusion bit-exact.  Small shapes compare every output; the full-size shapes compare
sampled rows and size-independent properties.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from position_independent_attention_amd import pic, workloads as W
from tests import hip_helpers as H
from tests.util import check_lse, check_mass, check_selection, out_within, parity_stats

pytestmark = pytest.mark.gpu


def setup_module(_):
    H.require_gpu()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def edge_workloads():
    return {
        # kv_len not a multiple of 16 or 64, ragged spans, big position gaps
        "ragged_gqa4_d128": lambda: W.custom(101, Hq=8, Hkv=2, d=128, theta=5e5,
                                             span_lens=[[100, 37, 300], [5, 64]], gaps=[[0, 3000, 7], [40, 1]],
                                             q_len=[19, 3], q_gap=[0, 50]),
        "mha_d64": lambda: W.custom(102, Hq=4, Hkv=4, d=64, theta=1e4, span_lens=[[70, 90]], q_len=[33]),
        "gqa8_d128": lambda: W.custom(103, Hq=16, Hkv=2, d=128, theta=5e5, span_lens=[[256, 128]], q_len=[40]),
        "gqa1_q1": lambda: W.custom(104, Hq=2, Hkv=2, d=128, theta=1e4, span_lens=[[17], [300, 1]],
                                    q_len=[1, 1]),
        "many_rows": lambda: W.custom(105, Hq=32, Hkv=8, d=128, theta=5e5, span_lens=[[512, 257]],
                                      q_len=[130]),
        "batch3_zero_q": lambda: W.custom(106, Hq=8, Hkv=2, d=64, theta=1e4, span_lens=[[64], [80, 16], [33]],
                                          q_len=[4, 0, 9]),
    }


def masked_inside_blocks():
    w = W.custom(107, Hq=8, Hkv=2, d=128, theta=5e5, span_lens=[[200, 150]], q_len=[24], q_gap=[5])
    rng = np.random.default_rng(7)
    n = int(w.kv_len[0]) - 24
    holes = rng.choice(n, size=60, replace=False)
    w.kv_pos[0, holes] = -1
    # garbage in masked slots (NaN in V, NaN and +inf in K) and in the pool
    # rows past the end of the sequence must not leak into the output
    blk = w.block_table[0, holes[0] // 16]
    w.pool_v[blk, :, :, holes[0] % 16] = 0x7fc0           # bf16 NaN
    for j, bits in ((holes[1], 0x7fc0), (holes[2], 0x7f80)):  # NaN, +inf
        w.pool_k[w.block_table[0, j // 16], :, j % 16, :] = bits
    end = int(w.kv_len[0])
    assert end % 16, "the last block must be partial"
    last = w.block_table[0, end // 16]
    w.pool_k[last, :, end % 16:, :] = 0x7fc0
    w.pool_v[last, :, :, end % 16:] = 0x7fc0
    return w


def compare_out(got, ref, what):
    mx, mean, rel = parity_stats(got, ref)
    say(f"  {what}: max {mx:.3e} mean {mean:.3e} rel {rel:.3e}")
    assert out_within(got, ref), (what, mx, mean, rel)


# --------------------------------------------------------------- prefill

@pytest.mark.parametrize("name", ["tiny", "llama_layer"] + list(edge_workloads()) + ["masked_inside_blocks"])
def test_prefill_parity(name):
    w = {"tiny": W.tiny, "llama_layer": W.llama_layer, "masked_inside_blocks": masked_inside_blocks,
         **edge_workloads()}[name]()
    say(f"prefill {name}: B={w.batch} Hq={w.num_q_heads} Hkv={w.num_kv_heads} d={w.head_dim} "
        f"kv={w.kv_len.tolist()} q={np.diff(w.q_start).tolist()}")
    ctx = H.ctx_for(w)
    out, lse, _ = H.prefill(ctx, w)
    ref_o, ref_l = oracle.attention(w)
    compare_out(H.host_bf16(out), ref_o, "O")
    check_lse(w, lse.cpu().numpy(), ref_l)


def test_prefill_row_without_visible_keys():
    w = W.custom(108, Hq=4, Hkv=1, d=64, theta=1e4, span_lens=[[40]], q_len=[3])
    w.q_pos[0] = 0                     # its own key (pi = 0) is visible ...
    n = int(w.kv_len[0])
    w.kv_pos[0, n - 3] = 5             # ... unless it moves after the query
    w.kv_pos[0, :40] += 10             # and the context too
    ctx = H.ctx_for(w)
    out, lse, _ = H.prefill(ctx, w)
    o = H.host_bf16(out)
    ref_o, ref_l = oracle.attention(w)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse.cpu().numpy()[0]))
    assert np.all(np.isneginf(ref_l[0]))
    compare_out(o, ref_o, "O")


def score_jumps(decode=False):
    """Keys placed so that one (query, head) row each scores 10 to 24 log2
    units above everything it has seen before, at slots past the first tiles
    (the start and the middle of 64-key tiles and 16-key blocks): the
    softmax reference of those rows moves after keys were already
    accumulated.  Each key is c * R(pos - pi) q for its row's query q, i.e.
    after rotation it points along the rotated query; c sets the score."""
    w = W.custom(118, Hq=8, Hkv=2, d=128, theta=5e5, span_lens=[[1000], [300, 400]],
                 q_len=[1, 1] if decode else [40, 9], decode=decode)
    d, G = w.head_dim, w.num_q_heads // w.num_kv_heads
    sc = np.log2(np.e) / np.sqrt(d)
    k = W.bf16_bits_to_f32(w.pool_k)
    # (request, key slot, query row in the request, head, score in log2 units)
    for r, j, tt, h, jump in [(0, 194, 0, 0, 12.), (0, 385, 5, 3, 16.), (0, 609, 11, 5, 20.), (0, 800, 39, 6, 24.),
                              (0, 450, 20, 1, 10.), (1, 130, 0, 2, 12.), (1, 322, 3, 7, 18.), (1, 512, 8, 4, 22.)]:
        t = int(w.q_start[r]) + (0 if decode else tt)
        q = W.bf16_bits_to_f32(w.q[t, h]).astype(np.float64)
        turn = int(w.q_pos[t]) - int(w.kv_pos[r, j])
        k[w.block_table[r, j // 16], h // G, j % 16, :] = jump / sc / np.dot(q, q) * oracle.rope(d, w.rope_theta, turn, q)
    w.pool_k = W.f32_to_bf16_bits(k)
    return w


@pytest.mark.parametrize("op", ["prefill", "decode"])
def test_score_jumps_move_the_softmax_reference(op):
    """Bar: O as everywhere; LSE per row within the worst-case effect of the
    bf16 rounding of the rotated q and k (relative 2^-9 each) on any score,
    2^-8 |q| max_j |k_j| / sqrt(d) by Cauchy-Schwarz, plus 2^-8 for the
    bf16 probabilities.  A reference mix-up is off by 2^8 or more in the
    weights, i.e. by order |V| in O and 5 or more in the LSE."""
    w = score_jumps(decode=op == "decode")
    ctx = H.ctx_for(w)
    out, lse, _ = H.prefill(ctx, w) if op == "prefill" else H.decode(ctx, w)
    ref_o, ref_l = oracle.attention(w)
    say(f"{op} score jumps: lse range {ref_l.min():.1f} .. {ref_l.max():.1f}")
    compare_out(H.host_bf16(out), ref_o, "O")
    G = w.num_q_heads // w.num_kv_heads
    qn = np.linalg.norm(W.bf16_bits_to_f32(w.q).astype(np.float64), axis=-1)             # [t][h]
    kn = np.linalg.norm(W.bf16_bits_to_f32(w.pool_k).astype(np.float64), axis=-1)        # [blk][g][slot]
    err = np.abs(lse.cpu().numpy() - ref_l)
    for r in range(w.batch):
        blocks = w.block_table[r, :(int(w.kv_len[r]) + 15) // 16]
        kmax = kn[blocks].max(axis=(0, 2))                                               # [g]
        for t in range(int(w.q_start[r]), int(w.q_start[r + 1])):
            bound = 2.0 ** -8 * qn[t] * np.repeat(kmax, G) / np.sqrt(w.head_dim) + 2.0 ** -8
            assert np.all(err[t] <= bound), (t, err[t], bound)
    say(f"  LSE: max {err.max():.3e}")


def far_scores(q_len, decode=False):
    """Every score a (query, head) row sees sits near one value per head, far
    below or above zero, beside unusable slots with NaN / inf garbage inside
    the tiles.  Queries and keys live in the lowest-frequency RoPE pair
    (index 63 and 127 at d = 128), whose angle moves by about 2.4e-6 per
    position at theta 5e5, so over these few hundred positions the rotation
    is within 2e-3 of the identity and every score of a head is
    -c m_h / sqrt(d) up to that.  In log2 units the heads of kv head 0 sit at
    -20, -200, -8.5 and +30, those of kv head 1 at -10, -140, +2 and -40:
    references far below zero, one past exp2's range, one just past the
    slack, and positive ones."""
    w = W.custom(119, Hq=8, Hkv=2, d=128, theta=5e5, span_lens=[[200, 150, 333]], gaps=[[0, 9, 2]],
                 q_len=[q_len], decode=decode)
    d = w.head_dim
    log2e = np.log2(np.e)
    c = 20.0 * np.sqrt(d) / log2e                     # m = 1 <-> -20 in log2 units
    m = np.array([1.0, 10.0, 0.425, -1.5, 0.5, 7.0, -0.1, 2.0])
    q = np.zeros((w.total_q, w.num_q_heads, d), np.float32)
    q[:, :, 63] = m
    w.q = W.f32_to_bf16_bits(q)
    k = np.zeros(W.bf16_bits_to_f32(w.pool_k).shape, np.float32)
    k[..., 63] = -c
    w.pool_k = W.f32_to_bf16_bits(k)
    # unusable slots inside the context, with garbage in K and V
    rng = np.random.default_rng(9)
    n = int(w.kv_len[0]) - (0 if decode else q_len)
    holes = rng.choice(n, size=40, replace=False)
    w.kv_pos[0, holes] = -1
    for j, bits in ((holes[0], 0x7fc0), (holes[1], 0x7f80), (holes[2], 0xff80)):   # NaN, +inf, -inf
        w.pool_k[w.block_table[0, j // 16], :, j % 16, :] = bits
        w.pool_v[w.block_table[0, j // 16], :, :, j % 16] = bits
    return w


@pytest.mark.parametrize("case", ["prefill_320_rows", "prefill_160_rows", "prefill_20_rows", "decode"])
def test_scores_far_from_zero_beside_unusable_keys(case):
    """Bars: O as everywhere (the weights are near uniform, so the output is
    near the mean of the visible values); LSE per row within the worst-case
    effect of the bf16 rounding of the rotated q and k, as in the score-jump
    test; the selection's mass and picks as in the selection tests, with and
    without the caller's LSE.  Counting an unusable key at the weight exp2(-reference) would move
    the LSE by up to 200 log2 units, and an inf weight against a zero value
    row would make O NaN."""
    # 320 rows per kv head: two 256-row blocks of the prefill, one 512-row
    # block of the selection's own LSE pass
    q_len = {"prefill_320_rows": 80, "prefill_160_rows": 40, "prefill_20_rows": 5, "decode": 1}[case]
    w = far_scores(q_len, decode=case == "decode")
    ctx = H.ctx_for(w)
    out, lse, dc = H.prefill(ctx, w) if case != "decode" else H.decode(ctx, w)
    ref_o, ref_l = oracle.attention(w)
    say(f"{case}: lse range {ref_l.min():.1f} .. {ref_l.max():.1f}")
    o = H.host_bf16(out)
    assert np.all(np.isfinite(o))
    compare_out(o, ref_o, "O")
    G = w.num_q_heads // w.num_kv_heads
    qn = np.linalg.norm(W.bf16_bits_to_f32(w.q).astype(np.float64), axis=-1)             # [t][h]
    kmax = 20.0 * np.sqrt(w.head_dim) / np.log2(np.e) * 1.01
    err = np.abs(lse.cpu().numpy() - ref_l)
    bound = 2.0 ** -8 * qn * kmax / np.sqrt(w.head_dim) + 2.0 ** -8
    assert np.all(err <= bound), (float((err / bound).max()), np.unravel_index(np.argmax(err / bound), err.shape))
    say(f"  LSE: max {err.max():.3e}, largest err / bound {(err / bound).max():.3f}")
    if case == "decode":
        return
    # the selection over the same scores, with the caller's LSE and with its
    # own K-only LSE pass (which shares the prefill's reference handling)
    ref_m = oracle.mass(w)
    ref_off, ref_idx = oracle.select(w, ref_m)
    for lse_given in (True, False):
        sel_off, sel, mass = H.select(ctx, w, dc, lse if lse_given else None)
        check_selection(sel_off, sel, ref_off, ref_idx, ref_m, w)
        check_mass(w, mass, ref_m, what=f"mass (caller's lse: {lse_given})")


def out_of_range_values(decode):
    """Device-side values outside their ranges, with max_position 4096: block
    ids past the pool and negative, key positions at and past max_position, a
    query at max_position - 1 (the table's last row) that sees a key there,
    and a query at max_position.  Returns the workload the kernels get and the
    one the oracle gets: the same, with those positions set to -1 (the
    header's convention: such a key is unusable and such a row sees nothing;
    the oracle already treats a block id outside the pool as unusable)."""
    mp = 4096
    w = W.custom(121, Hq=8, Hkv=2, d=128, theta=5e5, span_lens=[[200, 150], [300]], gaps=[[0, 11], [5]],
                 q_len=[1, 1] if decode else [20, 5], decode=decode, max_position=mp)
    nb = w.pool_k.shape[0]
    w.block_table[0, 3] = nb + 5
    w.block_table[0, 6] = -7
    w.block_table[1, 2] = 2 ** 30
    w.kv_pos[0, [20, 21, 150]] = [mp, mp + 100, 2 ** 30]
    w.kv_pos[1, 40] = mp
    # request 1: its first query moves to the table's last row and sees a key
    # placed there; its last query (request 0's in decode) moves past the table
    t1 = int(w.q_start[1])
    w.q_pos[t1] = mp - 1
    w.kv_pos[1, 77] = mp - 1
    t_out = int(w.q_start[1]) - 1
    w.q_pos[t_out] = mp
    ref = dataclasses.replace(w, kv_pos=np.where(w.kv_pos >= mp, -1, w.kv_pos),
                              q_pos=np.where(w.q_pos >= mp, -1, w.q_pos))
    return w, ref, t_out


@pytest.mark.parametrize("op", ["prefill", "decode"])
def test_out_of_range_device_values(op):
    """Bars as everywhere; the row whose query sits past the table sees
    nothing (O = 0, LSE = -inf on both sides)."""
    w, ref, t_out = out_of_range_values(op == "decode")
    ctx = H.ctx_for(w)
    out, lse, _ = H.prefill(ctx, w) if op == "prefill" else H.decode(ctx, w)
    ref_o, ref_l = oracle.attention(ref)
    o = H.host_bf16(out)
    assert np.all(np.isfinite(o))
    assert np.all(o[t_out] == 0) and np.all(np.isneginf(lse.cpu().numpy()[t_out]))
    assert np.all(np.isneginf(ref_l[t_out]))
    compare_out(o, ref_o, "O")
    check_lse(ref, lse.cpu().numpy(), ref_l)


@pytest.mark.parametrize("name", ["shared_serving", "long_context"])
def test_prefill_full_size_sampled(name):
    w = {"shared_serving": W.shared_serving, "long_context": W.long_context}[name]()
    say(f"prefill full {name}: B={w.batch} kv={w.max_kv_len} q={w.max_q_len}")
    ctx = H.ctx_for(w)
    out, lse, _ = H.prefill(ctx, w)
    rng = np.random.default_rng(5)
    nr = 48
    reqs = rng.choice(w.batch, size=min(w.batch, 3), replace=False)
    ts, hs = [], []
    for i in range(nr):
        r = reqs[i % len(reqs)]
        ts.append(int(rng.integers(w.q_start[r], w.q_start[r + 1])))
        hs.append(int(rng.integers(0, w.num_q_heads)))
    ts[0], hs[0] = int(w.q_start[reqs[0]]), 0     # first query of a request (fewest own keys)
    ref_o, ref_l = oracle.attention(w, (np.array(ts), np.array(hs)))
    o = H.host_bf16(out)[ts, hs]
    compare_out(o, ref_o, "O sampled")
    check_lse(w, lse.cpu().numpy()[ts, hs], ref_l, rows=(ts, hs))
    assert np.all(np.isfinite(H.host_bf16(out)))


def test_longest_context_prefill_select_decode():
    """The largest context the default RoPE table holds: 63 reused 1024-token
    spans + 256 query tokens = 64,768 slots, positions up to 64,767 of 65,536.
    Prefill on sampled rows against the oracle, the selection's size-independent
    properties, and a one-token decode over the same spans against the oracle."""
    w = W.long_context(n_spans=63)
    assert w.max_kv_len == 64768 and int(w.q_pos.max()) < w.max_position
    say(f"longest context: kv={w.max_kv_len} q={w.max_q_len} max pos {int(w.q_pos.max())}")
    ctx = H.ctx_for(w)
    out, lse, dc = H.prefill(ctx, w)
    rng = np.random.default_rng(11)
    ts = np.concatenate([[0, w.total_q - 1], rng.integers(0, w.total_q, 14)])
    hs = rng.integers(0, w.num_q_heads, len(ts))
    ref_o, ref_l = oracle.attention(w, (ts, hs))
    compare_out(H.host_bf16(out)[ts, hs], ref_o, "O sampled")
    check_lse(w, lse.cpu().numpy()[ts, hs], ref_l, rows=(ts, hs))
    sel_off, sel, mass = H.select(ctx, w, dc, lse)
    n = int(w.kv_len[0])
    total = float(mass[0, :n].astype(np.float64).sum())
    say(f"  mass sum {total:.3f} expected {w.total_q * w.num_q_heads}")
    assert abs(total - w.total_q * w.num_q_heads) <= 1e-4 * w.total_q * w.num_q_heads
    for s in range(len(w.span_req)):
        st, L = int(w.span_start[s]), int(w.span_len[s])
        k = int(sel_off[s + 1] - sel_off[s])
        order = sorted(range(st, st + L), key=lambda j: (-float(mass[0, j]), j))
        assert list(sel[sel_off[s]:sel_off[s + 1]]) == sorted(order[:k])
    wd = W.long_context(n_spans=63, q_len=1)
    dout, dlse, _ = H.decode(ctx, wd)
    ref_o, ref_l = oracle.attention(wd)
    compare_out(H.host_bf16(dout), ref_o, "decode O")
    check_lse(wd, dlse.cpu().numpy(), ref_l)


# ---------------------------------------------------------------- decode

@pytest.mark.parametrize("name", ["small", "small_private", "edge_g8", "masked_garbage", "d64", "d64_irregular"])
def test_decode_parity(name):
    if name == "small":
        w = W.decode_heavy(batch=5, n_spans=3, span_tok=80)
    elif name == "small_private":
        w = W.decode_heavy(batch=3, n_spans=2, span_tok=1024, private_spans=True, Hq=32)
    elif name.startswith("d64"):
        w = W.custom(116, Hq=8, Hkv=2, d=64, theta=1e4, span_lens=[[300, 45], [1000], [2]],
                     gaps=[[0, 7], [3], [0]], q_len=[1, 1, 1], decode=True)
        if name == "d64_irregular":
            # positions shuffled inside every other block of request 1
            rng = np.random.default_rng(117)
            for b in range(0, 1000 // 16, 2):
                w.kv_pos[1, 16 * b:16 * b + 16] = rng.permutation(w.kv_pos[1, 16 * b:16 * b + 16])
    else:
        w = W.custom(109, Hq=16, Hkv=2, d=128, theta=5e5, span_lens=[[2500, 3], [1], [700, 700]],
                     gaps=[[0, 9], [3], [0, 0]], q_len=[1, 1, 1], decode=True)
        w.kv_pos[2, 100:140] = -1
        if name == "masked_garbage":
            # NaN / +inf in the masked slots' K and V and past every sequence's
            # end: none of it may reach the output
            for j in range(100, 140):
                blk = w.block_table[2, j // 16]
                w.pool_k[blk, :, j % 16, :] = 0x7fc0 if j % 2 else 0x7f80
                w.pool_v[blk, :, :, j % 16] = 0x7fc0
            for r in range(w.batch):
                end = int(w.kv_len[r])
                if end % 16:
                    last = w.block_table[r, end // 16]
                    w.pool_k[last, :, end % 16:, :] = 0x7fc0
                    w.pool_v[last, :, :, end % 16:] = 0x7fc0
    say(f"decode {name}: B={w.batch} kv={w.kv_len.tolist()[:6]}")
    ctx = H.ctx_for(w)
    out, lse, _ = H.decode(ctx, w)
    ref_o, ref_l = oracle.attention(w)
    compare_out(H.host_bf16(out), ref_o, "O")
    check_lse(w, lse.cpu().numpy(), ref_l)


def test_decode_full_size_sampled():
    w = W.decode_heavy()
    say(f"decode full: B={w.batch} kv={w.max_kv_len}")
    ctx = H.ctx_for(w)
    out, lse, _ = H.decode(ctx, w)
    reqs = [0, 17, 63]
    ts = np.repeat(reqs, w.num_q_heads)
    hs = np.tile(np.arange(w.num_q_heads), len(reqs))
    ref_o, ref_l = oracle.attention(w, (ts, hs))
    compare_out(H.host_bf16(out)[ts, hs], ref_o, "O sampled")
    check_lse(w, lse.cpu().numpy()[ts, hs], ref_l, rows=(ts, hs))


@pytest.mark.parametrize("name", ["one_request_32k", "two_requests_9k"])
def test_decode_many_splits(name):
    # few (request, kv head) rows over long contexts: the key range is cut into
    # more than 16 splits, merged by the one-workgroup-per-row merge
    if name == "one_request_32k":
        w = W.decode_heavy(batch=1, n_spans=32, span_tok=1024)
    else:
        w = W.decode_heavy(batch=2, n_spans=9, span_tok=1000, private_spans=True)
    say(f"decode {name}: B={w.batch} kv={w.kv_len.tolist()}")
    ctx = H.ctx_for(w)
    out, lse, _ = H.decode(ctx, w)
    ref_o, ref_l = oracle.attention(w)
    compare_out(H.host_bf16(out), ref_o, "O")
    check_lse(w, lse.cpu().numpy(), ref_l)


def test_decode_matches_prefill_with_one_query():
    w = W.decode_heavy(batch=4, n_spans=2, span_tok=300)
    ctx = H.ctx_for(w)
    o1, l1, _ = H.decode(ctx, w)
    o2, l2, _ = H.prefill(ctx, w)
    a, b = H.host_bf16(o1), H.host_bf16(o2)
    assert np.max(np.abs(a - b)) <= 1e-2
    # the prefill kernel sums bf16-rounded P (on the MFMA), decode sums fp32 p
    assert np.max(np.abs(l1.cpu().numpy() - l2.cpu().numpy())) <= 2e-3


def _irregular_decode():
    """Blocks whose usable keys do not sit at pi = base + offset (the decode
    kernel then rotates each key with its own table row), next to regular
    ones: positions shuffled inside every other block of request 0, a block
    whose base would be negative in request 1, and a hole inside a block of
    request 2 that the following slots do not skip."""
    w = W.decode_heavy(batch=3, n_spans=2, span_tok=300, private_spans=True, Hq=32)
    rng = np.random.default_rng(11)
    kp = w.kv_pos
    for b in range(0, int(w.kv_len[0]) // 16, 2):
        kp[0, 16 * b:16 * b + 16] = rng.permutation(kp[0, 16 * b:16 * b + 16])
    kp[1, 0:16] = np.concatenate([[-1, -1, -1], np.arange(13)])
    kp[2, 40] = -1
    kp[2, 41:48] -= 1
    return w


@pytest.mark.parametrize("name", ["irregular_blocks", "fused_long_context_small", "fused_shared_small"])
def test_decode_irregular_positions(name):
    if name == "irregular_blocks":
        w = _irregular_decode()
    else:
        # fresh rows sit in appended private blocks at the stale slots' scattered positions
        src = small_select_workloads()[name[len("fused_"):]]()
        ref_off, ref_idx = oracle.select(src, oracle.mass(src))
        req_off = H.req_offsets(src, ref_off)
        n = int(req_off[-1])
        pk, pv, kp, kl = oracle.fuse(src, ref_idx, req_off, src.fresh_k[:n], src.fresh_v[:n])
        fused = src.copy()
        fused.pool_k, fused.pool_v, fused.kv_pos, fused.kv_len = pk, pv, kp, kl
        w = _last_token_decode(fused)
    say(f"decode {name}: B={w.batch} kv={w.kv_len.tolist()[:6]}")
    ctx = H.ctx_for(w)
    out, lse, _ = H.decode(ctx, w)
    ref_o, ref_l = oracle.attention(w)
    compare_out(H.host_bf16(out), ref_o, "O")
    check_lse(w, lse.cpu().numpy(), ref_l)


# ------------------------------------------------------------- selection

def small_select_workloads():
    return {
        "tiny": W.tiny,
        "llama_layer": W.llama_layer,
        "long_context_small": lambda: W.long_context(n_spans=4, span_tok=512, q_len=64),
        "shared_small": lambda: W.shared_serving(batch=3, n_pool_spans=6, span_tok=256, spans_per_req=3,
                                                 q_len=32),
        "edge_spans": lambda: W.custom(110, Hq=8, Hkv=2, d=64, theta=1e4, span_lens=[[1, 2, 300, 7], [45]],
                                       q_len=[12, 5], ratio=0.34),
        # spans longer than the 2048 slots the top-k keeps in registers
        "long_spans": lambda: W.custom(111, Hq=8, Hkv=2, d=64, theta=1e4, span_lens=[[3000, 5], [2049, 2048]],
                                       q_len=[8, 4], ratio=0.2),
        # d = 64 with 160 rows per kv head: the 4-row-tile mass pass at d = 64
        "d64_many_rows": lambda: W.custom(115, Hq=8, Hkv=2, d=64, theta=1e4, span_lens=[[300, 200], [150]],
                                          q_len=[40, 33], ratio=0.2),
        # 16 kv heads (MHA): the fusion copies its heads in two passes of 8
        "mha16": lambda: W.custom(119, Hq=16, Hkv=16, d=128, theta=5e5, span_lens=[[200, 77], [90]],
                                  q_len=[9, 20], ratio=0.3),
        # NaN / inf in masked slots' K and V and past the sequence's end
        "masked_garbage": masked_inside_blocks,
        # the long-context head geometry (32/8, d 128) with more than one
        # 512-row block of the selection mass pass per kv head, as at the full
        # shape (1,024 rows): 800 rows (2 blocks) and 1,200 rows (3 blocks, the
        # last one ragged)
        "long_context_2rb": lambda: W.long_context(n_spans=3, span_tok=1024, q_len=200),
        "long_context_3rb": lambda: W.long_context(n_spans=2, span_tok=1024, q_len=300),
        # d = 64 with 400 and 612 rows per kv head: 2 and 3 of its 256-row blocks
        "d64_2rb": lambda: W.custom(132, Hq=8, Hkv=2, d=64, theta=1e4, span_lens=[[700, 300]],
                                    q_len=[100], ratio=0.2),
        "d64_3rb_batch2": lambda: W.custom(133, Hq=16, Hkv=4, d=64, theta=1e4,
                                           span_lens=[[500, 333], [900]], q_len=[153, 60], ratio=0.15),
    }


@pytest.mark.parametrize("lse_given", [True, False])
@pytest.mark.parametrize("name", list(small_select_workloads()))
def test_select_parity(name, lse_given):
    w = small_select_workloads()[name]()
    say(f"select {name} lse_given={lse_given}: spans={len(w.span_req)} ratio={w.ratio}")
    ctx = H.ctx_for(w)
    out, lse, dc = H.prefill(ctx, w)
    if lse_given and w.total_q * w.num_q_heads >= 4096:
        # the prefill behind the caller's lse, at the shapes with many row blocks
        ref_o, ref_l = oracle.attention(w)
        compare_out(H.host_bf16(out), ref_o, "O")
        check_lse(w, lse.cpu().numpy(), ref_l)
    sel_off, sel, mass = H.select(ctx, w, dc, lse if lse_given else None)
    ref_m = oracle.mass(w)
    ref_off, ref_idx = oracle.select(w, ref_m)
    check_selection(sel_off, sel, ref_off, ref_idx, ref_m, w)
    for r in range(w.batch):
        n = int(w.kv_len[r])
        err = np.abs(mass[r, :n] - ref_m[r, :n])
        rel = err / np.maximum(ref_m[r, :n], 1e-12)
        say(f"  mass r{r}: max abs err {err.max():.3e}, max rel err {rel.max():.3e} "
            f"(sum {mass[r, :n].sum():.4f} vs {ref_m[r, :n].sum():.4f})")
        assert abs(mass[r, :n].astype(np.float64).sum() - ref_m[r, :n].sum()) <= 1e-4 * ref_m[r, :n].sum()
    check_mass(w, mass, ref_m)


def test_select_ties_and_budget_edges():
    """Equal masses (all-zero keys give every visible key the same weight)
    resolve to the lower index; k = 0 and k = L spans."""
    w = W.custom(111, Hq=4, Hkv=1, d=64, theta=1e4, span_lens=[[32, 32, 48]], q_len=[4], ratio=0.25)
    w.pool_k[:] = 0
    ctx = H.ctx_for(w)
    _, lse, dc = H.prefill(ctx, w)
    for ratio in (0.25, 0.0, 1.0):
        sel_off, sel, mass = H.select(ctx, w, dc, lse, ratio=ratio)
        ref_m = oracle.mass(w)
        ref_off, ref_idx = oracle.select(w, ref_m, ratio)
        assert np.array_equal(sel_off, ref_off)
        assert np.array_equal(sel, ref_idx), (ratio, sel[:8], ref_idx[:8])


def test_select_fewer_candidates_than_budget_pads_with_minus_one():
    w = W.custom(112, Hq=4, Hkv=1, d=64, theta=1e4, span_lens=[[32]], q_len=[4], ratio=0.5)
    w.kv_pos[0, 4:30] = -1                                 # 6 candidates left, budget 16
    ctx = H.ctx_for(w)
    _, lse, dc = H.prefill(ctx, w)
    sel_off, sel, mass = H.select(ctx, w, dc, lse)
    ref_m = oracle.mass(w)
    ref_off, ref_idx = oracle.select(w, ref_m)
    assert sel_off[-1] == 16 and len(ref_idx) == 6
    assert np.array_equal(sel[:6], ref_idx) and np.all(sel[6:] == -1)


def test_select_full_size_properties():
    """Full 32k-context shape: every query row's probabilities sum to one, so
    the mass sums to n_q * Hq; masked slots get none; the selection is the
    per-span top-k of the returned mass with ties to the lower index."""
    w = W.long_context()
    ctx = H.ctx_for(w)
    _, lse, dc = H.prefill(ctx, w)
    sel_off, sel, mass = H.select(ctx, w, dc, lse)
    n = int(w.kv_len[0])
    total = float(mass[0, :n].astype(np.float64).sum())
    say(f"select full: mass sum {total:.3f} expected {w.total_q * w.num_q_heads}")
    assert abs(total - w.total_q * w.num_q_heads) <= 1e-4 * w.total_q * w.num_q_heads
    assert np.all(mass[0, :n] >= 0)
    for s in range(len(w.span_req)):
        st, L = int(w.span_start[s]), int(w.span_len[s])
        k = int(sel_off[s + 1] - sel_off[s])
        order = sorted(range(st, st + L), key=lambda j: (-float(mass[0, j]), j))
        assert list(sel[sel_off[s]:sel_off[s + 1]]) == sorted(order[:k])


@pytest.mark.parametrize("name", ["tiny", "shared_small", "edge_spans", "long_spans", "long_context_full"])
def test_select_without_mass_output_is_the_same_selection(name):
    """The mass output is optional: leaving it out must not change the
    selection by a bit, spans longer than the top-k's register cache
    included, both with and without the caller's lse."""
    w = W.long_context() if name == "long_context_full" else small_select_workloads()[name]()
    ctx = H.ctx_for(w)
    _, lse, dc = H.prefill(ctx, w)
    sel_off, _, _ = H.select(ctx, w, dc, lse)
    nsel = int(sel_off[-1])
    mass = torch.empty(w.kv_pos.shape, dtype=torch.float32, device=H.DEV)
    for lse_arg in (lse, None):
        picks = []
        for m in (mass, None):
            got = torch.full((max(nsel, 1),), -7, dtype=torch.int32, device=H.DEV)
            pic.qc_score_select(ctx, dc, lse_arg, nsel, got, m)
            torch.cuda.synchronize()
            picks.append(got.cpu().numpy()[:nsel])
        assert np.array_equal(picks[0], picks[1]), (name, lse_arg is None)
        assert not np.any(picks[1] == -7)


# ---------------------------------------------------------------- fusion

@pytest.mark.parametrize("name", ["tiny", "shared_small", "edge_spans", "mha16"])
def test_fuse_bit_exact_and_second_pass(name):
    """The oracle's own selection is fused by both sides: pool bytes, pi and
    kv_len must match bit for bit, shared blocks stay untouched, and attention
    over the fused cache matches the oracle over its fused copy."""
    w = small_select_workloads()[name]()
    ctx = H.ctx_for(w)
    ref_m = oracle.mass(w)
    ref_off, ref_idx = oracle.select(w, ref_m)
    req_off = H.req_offsets(w, ref_off)
    n = int(req_off[-1])
    pk, pv, kp, kl = oracle.fuse(w, ref_idx, req_off, w.fresh_k[:n], w.fresh_v[:n])
    dc = pic.to_device(w, H.DEV)
    H.fuse(ctx, dc, ref_idx, req_off, w.fresh_k, w.fresh_v)
    assert np.array_equal(dc.kv_len.cpu().numpy(), kl)
    assert np.array_equal(dc.kv_pos.cpu().numpy(), kp)
    gk = dc.pool_k.cpu().numpy().view(np.uint16)
    gv = dc.pool_v.cpu().numpy().view(np.uint16)
    assert np.array_equal(gk, pk) and np.array_equal(gv, pv)
    assert np.array_equal(gk[w.shared_blocks], w.pool_k[w.shared_blocks])
    fused = w.copy()
    fused.pool_k, fused.pool_v, fused.kv_pos, fused.kv_len = pk, pv, kp, kl
    dc.max_kv_len = int(kl.max())
    out2, lse2, _ = H.prefill(ctx, fused, dc)
    ref2, refl2 = oracle.attention(fused)
    compare_out(H.host_bf16(out2), ref2, "O fused")
    check_lse(fused, lse2.cpu().numpy(), refl2)


@pytest.mark.parametrize("d,q_len", [(128, 520), (64, 260)])
def test_fused_pass_with_many_rows_uses_tile_skipping(d, q_len):
    """Enough query rows for the tile-skipping kernel (8 or more row blocks).
    Over the fused cache its key range holds stale slots (pi = -1) in the
    spans, the query block (masked tiles), an alignment pad and the fused rows
    behind it.  All fused rows are visible to every row, so they run in the
    mask-free loop after the masked range."""
    w = W.custom(120 + d, Hq=8, Hkv=2, d=d, theta=5e5, span_lens=[[300, 203, 250]], gaps=[[0, 40, 9]],
                 q_len=[q_len], ratio=0.25)
    say(f"fused pass: d={d} q={q_len} kv={w.kv_len.tolist()} rows={q_len * 4}")
    ctx = H.ctx_for(w)
    ref_m = oracle.mass(w)
    ref_off, ref_idx = oracle.select(w, ref_m)
    req_off = H.req_offsets(w, ref_off)
    n = int(req_off[-1])
    pk, pv, kp, kl = oracle.fuse(w, ref_idx, req_off, w.fresh_k[:n], w.fresh_v[:n])
    assert int(kl[0]) % 16 and int(w.kv_len[0]) % 16, "want a pad and a partial last block"
    dc = pic.to_device(w, H.DEV)
    H.fuse(ctx, dc, ref_idx, req_off, w.fresh_k, w.fresh_v)
    assert np.array_equal(dc.kv_pos.cpu().numpy(), kp)
    fused = w.copy()
    fused.pool_k, fused.pool_v, fused.kv_pos, fused.kv_len = pk, pv, kp, kl
    dc.max_kv_len = int(kl.max())
    out, lse, _ = H.prefill(ctx, fused, dc)
    ref_o, ref_l = oracle.attention(fused)
    compare_out(H.host_bf16(out), ref_o, "O fused")
    check_lse(fused, lse.cpu().numpy(), ref_l)


def test_fuse_full_size_with_seeded_selection():
    """Full 32k shape: a seeded selection (15% per span, from the test's own
    generator) fused on both sides; bitwise equal; then sampled rows of the
    second pass against the oracle over its fused copy."""
    w = W.long_context()
    ctx = H.ctx_for(w)
    rng = np.random.default_rng(44)
    sel = np.concatenate([np.sort(rng.choice(np.arange(st, st + L), size=154, replace=False))
                          for st, L in zip(w.span_start, w.span_len)]).astype(np.int32)
    req_off = np.array([0, len(sel)], np.int32)
    pk, pv, kp, kl = oracle.fuse(w, sel, req_off, w.fresh_k[:len(sel)], w.fresh_v[:len(sel)])
    dc = pic.to_device(w, H.DEV)
    H.fuse(ctx, dc, sel, req_off, w.fresh_k, w.fresh_v)
    assert np.array_equal(dc.kv_len.cpu().numpy(), kl) and np.array_equal(dc.kv_pos.cpu().numpy(), kp)
    assert np.array_equal(dc.pool_k.cpu().numpy().view(np.uint16), pk)
    assert np.array_equal(dc.pool_v.cpu().numpy().view(np.uint16), pv)
    fused = w.copy()
    fused.pool_k, fused.pool_v, fused.kv_pos, fused.kv_len = pk, pv, kp, kl
    dc.max_kv_len = int(kl.max())
    out2, lse2, _ = H.prefill(ctx, fused, dc)
    ts = np.array([0, 1, 77, 128, 255, 200, 31, 64])
    hs = np.array([0, 31, 5, 17, 9, 22, 3, 12])
    ref2, refl2 = oracle.attention(fused, (ts, hs))
    compare_out(H.host_bf16(out2)[ts, hs], ref2, "O fused sampled")
    check_lse(fused, lse2.cpu().numpy()[ts, hs], refl2, rows=(ts, hs))


# ------------------------------------------------------- anchor extraction

ANCHOR_RATIO = 0.05   # the pages call it a small fraction; declared, not given


def _anchors(ctx, w, dc, ratio):
    sel_off = pic.pic_select_offsets(w.span_len, ratio)
    dc.span_req, dc.span_start, dc.span_len = H.dev(w.span_req), H.dev(w.span_start), H.dev(w.span_len)
    dc.sel_off, dc.n_spans = H.dev(sel_off), len(w.span_req)
    nsel = int(sel_off[-1])
    sel = torch.full((max(nsel, 1),), -7, dtype=torch.int32, device=H.DEV)
    norm = torch.full(w.kv_pos.shape, -1.0, dtype=torch.float32, device=H.DEV)
    pic.qc_anchor_select(ctx, dc, nsel, sel, norm)
    torch.cuda.synchronize()
    return sel_off, sel.cpu().numpy()[:nsel], norm.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "llama_layer", "shared_small", "edge_spans", "long_spans"])
def test_anchor_parity(name):
    """Squared key norms within the fp32 accumulation bound of the oracle's,
    and the anchors are the oracle's up to that band at the k-th boundary."""
    w = small_select_workloads()[name]()
    w.kv_pos[0, 5:9] = -1                         # masked slots score 0, never anchors
    ctx = H.ctx_for(w)
    dc = pic.to_device(w, H.DEV)
    off, idx, norm = _anchors(ctx, w, dc, ANCHOR_RATIO)
    ref = oracle.key_norm(w)
    # bf16 squares are exact in fp32; the n = Hkv*d additions each round by at
    # most one unit in the last place of the partial sum
    rel = w.num_kv_heads * w.head_dim * 2.0 ** -24
    for r in range(w.batch):
        n = int(w.kv_len[r])
        assert np.all(np.abs(norm[r, :n] - ref[r, :n]) <= rel * ref[r, :n]), r
    ref_off, ref_idx = oracle.select(w, ref, ratio=ANCHOR_RATIO)
    band = rel * float(ref.max())
    check_selection(off, idx, ref_off, ref_idx, ref, w, band=band)
    req0 = np.concatenate([idx[off[s]:off[s + 1]] for s in range(len(w.span_req)) if w.span_req[s] == 0])
    assert not set(range(5, 9)) & set(req0.tolist())


def test_anchor_full_size_and_bitwise_repeatable():
    w = W.long_context()
    ctx = H.ctx_for(w)
    dc = pic.to_device(w, H.DEV)
    off, idx, norm = _anchors(ctx, w, dc, ANCHOR_RATIO)
    off2, idx2, norm2 = _anchors(ctx, w, dc, ANCHOR_RATIO)
    assert np.array_equal(norm, norm2) and np.array_equal(idx, idx2)
    ref = oracle.key_norm(w)
    n = int(w.kv_len[0])
    rel = w.num_kv_heads * w.head_dim * 2.0 ** -24
    assert np.all(np.abs(norm[0, :n] - ref[0, :n]) <= rel * ref[0, :n])
    ref_off, ref_idx = oracle.select(w, ref, ratio=ANCHOR_RATIO)
    check_selection(off, idx, ref_off, ref_idx, ref, w, band=rel * float(ref.max()))


# ------------------------------------------------ pre-rotated keys (ablation)

def _prerotated(w):
    """Copy of w whose K pool holds every usable slot's key rotated at its pi by
    the oracle's rope, rounded to bf16: the standard RoPE cache that the
    keys_prerotated mode reads.  Fails if a slot would need two positions
    (a block shared at different offsets cannot be pre-rotated)."""
    wp = w.copy()
    seen = {}
    for r in range(w.batch):
        for j in range(int(w.kv_len[r])):
            pi, blk = int(w.kv_pos[r, j]), int(w.block_table[r, j // 16])
            if pi < 0 or blk < 0:
                continue
            assert seen.setdefault((blk, j % 16), pi) == pi, "slot needed at two positions"
            if (blk, j % 16, "done") in seen:
                continue
            seen[(blk, j % 16, "done")] = True
            for g in range(w.num_kv_heads):
                k = W.bf16_bits_to_f32(w.pool_k[blk, g, j % 16]).astype(np.float64)
                kr = oracle.rope(w.head_dim, w.rope_theta, pi, k)
                wp.pool_k[blk, g, j % 16] = W.f32_to_bf16_bits(kr.astype(np.float32))
    return wp


def test_prerotated_mode_prefill_and_mass():
    """Ablation of the in-kernel rotation: keys stored rotated, used as stored;
    results equal the method's (the oracle on the unrotated cache)."""
    w = W.long_context(n_spans=4, span_tok=512, q_len=64)
    wp = _prerotated(w)
    ctx = pic.Context(w.num_q_heads, w.num_kv_heads, w.head_dim, w.rope_theta, w.max_position,
                      keys_prerotated=True)
    out, lse, dc = H.prefill(ctx, wp)
    ref_o, ref_l = oracle.attention(w)
    compare_out(H.host_bf16(out), ref_o, "O prerotated")
    check_lse(w, lse.cpu().numpy(), ref_l)
    _, _, mass = H.select(ctx, wp, dc, lse)
    check_mass(w, mass, oracle.mass(w))


def test_prerotated_mode_decode():
    w = W.decode_heavy(batch=3, n_spans=2, span_tok=512, private_spans=True, Hq=32)
    wp = _prerotated(w)
    ctx = pic.Context(w.num_q_heads, w.num_kv_heads, w.head_dim, w.rope_theta, w.max_position,
                      keys_prerotated=True)
    out, lse, _ = H.decode(ctx, wp)
    ref_o, ref_l = oracle.attention(w)
    compare_out(H.host_bf16(out), ref_o, "O prerotated decode")
    check_lse(w, lse.cpu().numpy(), ref_l)


# ------------------------------------------------------- sparse recompute

def _recompute_case(w, sel_idx, req_off, seed):
    """The oracle's fused cache, queried by the selected tokens at their
    pre-fusion logical positions (QCFuse's discrete-token recompute)."""
    n = int(req_off[-1])
    pk, pv, kp, kl = oracle.fuse(w, sel_idx, req_off, w.fresh_k[:n], w.fresh_v[:n])
    fused = w.copy()
    fused.pool_k, fused.pool_v, fused.kv_pos, fused.kv_len = pk, pv, kp, kl
    pos = [w.kv_pos[r, sel_idx[req_off[r]:req_off[r + 1]]] for r in range(w.batch)]
    return W.recompute_queries(fused, pos, seed)


@pytest.mark.parametrize("name", ["tiny", "long_context_small", "shared_small", "edge_spans"])
def test_recompute_parity(name):
    """Scattered query positions, causal by position, over the fused cache:
    every recomputed token sees the context before it and its own fresh row."""
    w = small_select_workloads()[name]()
    ref_off, ref_idx = oracle.select(w, oracle.mass(w))
    wr = _recompute_case(w, ref_idx, H.req_offsets(w, ref_off), 900)
    say(f"recompute {name}: queries per request {np.diff(wr.q_start).tolist()}")
    ctx = H.ctx_for(wr)
    out, lse, _ = H.prefill(ctx, wr)
    ref_o, ref_l = oracle.attention(wr)
    compare_out(H.host_bf16(out), ref_o, "O recompute")
    check_lse(wr, lse.cpu().numpy(), ref_l)


def test_recompute_full_size_sampled():
    """Long-context shape: 4,928 selected tokens (seeded, 154 per span) as
    queries over the fused 37,952-slot cache; sampled rows against the oracle."""
    w = W.long_context()
    rng = np.random.default_rng(45)
    sel = np.concatenate([np.sort(rng.choice(np.arange(st, st + L), size=154, replace=False))
                          for st, L in zip(w.span_start, w.span_len)]).astype(np.int32)
    wr = _recompute_case(w, sel, np.array([0, len(sel)], np.int32), 901)
    ctx = H.ctx_for(wr)
    out, lse, _ = H.prefill(ctx, wr)
    ts = np.array([0, 1, 999, 2500, 4927, 3333, 17, 4000])
    hs = np.array([0, 31, 5, 17, 9, 22, 3, 12])
    ref_o, ref_l = oracle.attention(wr, (ts, hs))
    compare_out(H.host_bf16(out)[ts, hs], ref_o, "O recompute sampled")
    check_lse(wr, lse.cpu().numpy()[ts, hs], ref_l, rows=(ts, hs))


def test_recompute_skips_tiles_no_row_sees():
    """Queries at scattered positions in more than 8 row blocks (the variant
    that skips tiles no row of a workgroup sees), over a context whose
    positions run backwards through the slots: row blocks early in position
    order need only late tiles, so the first tile they stage is not tile 0."""
    w = W.custom(112, Hq=8, Hkv=2, d=64, theta=1e4, span_lens=[[640, 512, 768, 384, 512]], q_len=[8])
    n = int(w.kv_len[0]) - 8
    ctx_slots = np.nonzero(w.kv_pos[0, :n] >= 0)[0]
    top = int(w.kv_pos[0, ctx_slots].max())
    w.kv_pos[0, ctx_slots] = top - w.kv_pos[0, ctx_slots]
    rng = np.random.default_rng(113)
    picked = np.sort(rng.choice(ctx_slots, size=845, replace=False))
    wr = W.recompute_queries(w, [w.kv_pos[0, picked]], 114)
    say(f"recompute skip: {wr.total_q} queries x {w.num_q_heads // w.num_kv_heads} heads per kv head")
    ctx = H.ctx_for(wr)
    out, lse, _ = H.prefill(ctx, wr)
    ref_o, ref_l = oracle.attention(wr)
    compare_out(H.host_bf16(out), ref_o, "O recompute skip")
    check_lse(wr, lse.cpu().numpy(), ref_l)


# ------------------------------------------- span reuse by block hashing

def test_block_hash_reuse_end_to_end():
    """Token streams with the same SSEP spans at different offsets: the block
    cache hands both requests the same physical blocks, K/V are written only
    for missed blocks, and attention over the shared pool equals the oracle
    and equals private copies bit for bit."""
    from tests.test_block_hash import PAD, SSEP, PDEP, padded, span
    sp = [padded(span(200 + i, 60 + 37 * i), SSEP) for i in range(3)]
    streams = [padded(span(300, 20)) + sp[0] + sp[1] + sp[2],
               padded(span(301, 70)) + sp[2] + sp[0] + padded(span(302, 5), PDEP)]
    Hq, Hkv, d = 8, 2, 64
    nb_pool = 64
    cache = pic.BlockCache(nb_pool)
    maps = [cache.map_request(np.asarray(t, np.int32), PAD, SSEP, PDEP) for t in streams]
    cache.close()
    assert sum(int(m[2].sum()) for m in maps) < sum(len(m[0]) for m in maps)   # something was reused
    rng = np.random.default_rng(303)
    pool_k = np.zeros((nb_pool, Hkv, 16, d), np.uint16)
    pool_v = np.zeros((nb_pool, Hkv, d, 16), np.uint16)
    for table, _, miss in maps:
        for b, m in zip(table, miss):
            if m:   # the caller computes K/V of a missed block once
                pool_k[b] = W.f32_to_bf16_bits(rng.standard_normal((Hkv, 16, d), dtype=np.float32))
                pool_v[b] = W.f32_to_bf16_bits(rng.standard_normal((Hkv, d, 16), dtype=np.float32))
    maxb = max(len(m[0]) for m in maps)
    bt = np.full((2, maxb), -1, np.int32)
    kvp = np.full((2, maxb * 16), -1, np.int32)
    kvl = np.zeros(2, np.int32)
    for r, (table, pos, _) in enumerate(maps):
        bt[r, :len(table)] = table
        kvp[r, :len(pos)] = pos
        kvl[r] = len(pos)
    q_len = 6
    q_pos = np.concatenate([np.arange(q_len) + int(kvp[r].max()) + 1 for r in range(2)]).astype(np.int32)
    w = dataclasses.replace(W.tiny(), name="block_hash", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d,
                            rope_theta=1e4, batch=2, pool_k=pool_k, pool_v=pool_v, block_table=bt,
                            kv_len=kvl, kv_pos=kvp,
                            q=W.fresh_queries(2 * q_len, Hq, d, seed=304),
                            q_start=np.array([0, q_len, 2 * q_len], np.int32), q_pos=q_pos)
    ctx = H.ctx_for(w)
    out, lse, _ = H.prefill(ctx, w)
    ref_o, ref_l = oracle.attention(w)
    compare_out(H.host_bf16(out), ref_o, "O block-hash reuse")
    check_lse(w, lse.cpu().numpy(), ref_l)
    # private copies of request 1's blocks give the same bits
    wp = w.copy()
    n1 = len(maps[1][0])
    fresh_ids = np.arange(nb_pool - n1, nb_pool)
    wp.pool_k[fresh_ids] = w.pool_k[bt[1, :n1]]
    wp.pool_v[fresh_ids] = w.pool_v[bt[1, :n1]]
    wp.block_table[1, :n1] = fresh_ids
    out2, _, _ = H.prefill(ctx, wp)
    assert np.array_equal(out.cpu().numpy(), out2.cpu().numpy())


# ------------------------------------------------------- sharing / repeat

def test_shared_pool_untouched_and_runs_bitwise_repeatable():
    w = W.shared_serving(batch=4, n_pool_spans=8, span_tok=256, spans_per_req=4, q_len=48)
    ctx = H.ctx_for(w)
    dc = pic.to_device(w, H.DEV)
    ck = dc.pool_k.clone()
    cv = dc.pool_v.clone()
    o1, l1, _ = H.prefill(ctx, w, dc)
    s1 = H.select(ctx, w, dc, l1)
    o2, l2, _ = H.prefill(ctx, w, dc)
    s2 = H.select(ctx, w, dc, l2)
    od1, ld1, _ = H.decode(ctx, _last_token_decode(w), None)
    od2, ld2, _ = H.decode(ctx, _last_token_decode(w), None)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert np.array_equal(s1[1], s2[1]) and np.array_equal(s1[2], s2[2])
    assert torch.equal(od1, od2) and torch.equal(ld1, ld2)
    assert torch.equal(ck, dc.pool_k) and torch.equal(cv, dc.pool_v)


def _last_token_decode(w):
    """The same requests with only their last query token (decode shape)."""
    d = w.copy()
    last = w.q_start[1:] - 1
    d.q = w.q[last]
    d.q_pos = w.q_pos[last]
    d.q_start = np.arange(w.batch + 1, dtype=np.int32)
    return d


def test_shared_blocks_at_different_offsets_match_private_copies():
    """Two requests reading the same physical blocks at different logical
    offsets give what each would get from private copies of those blocks."""
    w = W.shared_serving(batch=2, n_pool_spans=3, span_tok=128, spans_per_req=3, q_len=16, seed=77)
    ctx = H.ctx_for(w)
    out, lse, _ = H.prefill(ctx, w)
    for r in range(2):
        solo = W.custom(0, Hq=w.num_q_heads, Hkv=w.num_kv_heads, d=w.head_dim, theta=w.rope_theta,
                        span_lens=[[128] * 3], q_len=[16])
        n = int(w.kv_len[r])
        nb = (n + 15) // 16
        solo.pool_k = np.ascontiguousarray(w.pool_k[w.block_table[r, :nb]])
        solo.pool_v = np.ascontiguousarray(w.pool_v[w.block_table[r, :nb]])
        solo.block_table = np.arange(nb, dtype=np.int32)[None, :]
        solo.kv_pos = w.kv_pos[r:r + 1, :nb * 16].copy()
        solo.kv_len = w.kv_len[r:r + 1].copy()
        sl = slice(w.q_start[r], w.q_start[r + 1])
        solo.q, solo.q_pos = w.q[sl].copy(), w.q_pos[sl].copy()
        solo.q_start = np.array([0, 16], np.int32)
        o2, l2, _ = H.prefill(ctx, solo)
        # equal up to the split-merge order, which depends on the batch size
        assert np.max(np.abs(H.host_bf16(out[sl]) - H.host_bf16(o2))) <= 1e-2
        assert np.max(np.abs(lse[sl].cpu().numpy() - l2.cpu().numpy())) <= 1e-4


# ------------------------------------------------------------ validation

def test_argument_errors_return_status_before_launch():
    w = W.tiny()
    ctx = H.ctx_for(w)
    dc = pic.to_device(w, H.DEV)
    out = torch.empty(w.q.shape, dtype=torch.int16, device=H.DEV)
    pool, req, qs = dc.pool(), dc.req(), dc.queries()
    h = pic.lib()
    import ctypes as C
    bad = pic.PicReqTable(req.batch, req.max_blocks, req.max_blocks * 16 + 1, req.block_table, req.kv_len,
                          req.kv_pos)
    assert h.pic_attn_prefill(ctx.handle, C.byref(pool), C.byref(bad), C.byref(qs), out.data_ptr(), None,
                              None, 0, None) == pic.PIC_ERR_INVALID_ARG
    bigq = pic.PicQueries(qs.q, qs.q_start, qs.q_pos, qs.total_q, qs.total_q + 1)
    assert h.pic_attn_prefill(ctx.handle, C.byref(pool), C.byref(req), C.byref(bigq), out.data_ptr(), None,
                              None, 0, None) == pic.PIC_ERR_INVALID_ARG
    # a workspace-needing shape without workspace
    wl = W.llama_layer()
    ctx2 = H.ctx_for(wl)
    dc2 = pic.to_device(wl, H.DEV)
    need = pic.pic_workspace_bytes(ctx2, pic.PIC_OP_PREFILL, dc2.req(), dc2.total_q, dc2.max_q_len)
    assert need > 0
    out2 = torch.empty(wl.q.shape, dtype=torch.int16, device=H.DEV)
    assert h.pic_attn_prefill(ctx2.handle, C.byref(dc2.pool()), C.byref(dc2.req()), C.byref(dc2.queries()),
                              out2.data_ptr(), None, None, 0, None) == pic.PIC_ERR_WORKSPACE
    assert "workspace" in ctx2.last_error()
    # decode with more than 16 q heads per kv head is declined
    ctx3 = pic.Context(64, 2, 128, 1e4, 1024)
    assert h.pic_attn_decode(ctx3.handle, C.byref(pool), C.byref(req), qs.q, qs.q_pos, out.data_ptr(), None,
                             None, 0, None) == pic.PIC_ERR_UNSUPPORTED
    torch.cuda.synchronize()
