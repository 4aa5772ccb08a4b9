"""Seeded generator: determinism, layout invariants, bf16 encoding."""
import numpy as np
import pytest
import torch

from position_independent_attention_amd import workloads as W

SMALL = {
    "tiny": W.tiny,
    "llama_layer": W.llama_layer,
    "shared_serving": lambda: W.shared_serving(batch=3, n_pool_spans=6, span_tok=64, spans_per_req=3,
                                               q_len=16),
    "long_context": lambda: W.long_context(n_spans=4, span_tok=128, q_len=32),
    "decode_heavy": lambda: W.decode_heavy(batch=4, n_spans=3, span_tok=64),
    "decode_heavy_private": lambda: W.decode_heavy(batch=3, n_spans=2, span_tok=64, private_spans=True),
}


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -3.0e-39, 65504.0], np.float32)])
    mine = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(W.bf16_bits_to_f32(mine), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("name", list(SMALL))
def test_deterministic(name):
    a, b = SMALL[name](), SMALL[name]()
    for f in ("pool_k", "pool_v", "block_table", "kv_pos", "kv_len", "q", "q_pos", "q_start",
              "span_start", "fresh_k"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f


@pytest.mark.parametrize("name", list(SMALL))
def test_layout_invariants(name):
    w = SMALL[name]()
    B = w.batch
    assert w.q_start[0] == 0 and w.q_start[-1] == w.total_q and np.all(np.diff(w.q_start) >= 0)
    for r in range(B):
        n = w.kv_len[r]
        nb = (n + 15) // 16
        assert np.all(w.block_table[r, :nb] >= 0) and np.all(w.block_table[r, :nb] < w.num_blocks)
        pi = w.kv_pos[r, :n]
        # every query sees its own key: the last q_len slots carry the query positions
        nq = w.q_start[r + 1] - w.q_start[r]
        assert np.array_equal(pi[n - nq:], w.q_pos[w.q_start[r]:w.q_start[r + 1]])
        assert np.all(w.kv_pos[r, n:] == -1)
        # logical positions are distinct among visible keys and precede the queries
        vis = pi[pi >= 0]
        assert len(np.unique(vis)) == len(vis)
        assert vis[: n - nq].max(initial=-1) < w.q_pos[w.q_start[r]]
        # fused-row capacity: private blocks appended after the sequence
        extra = (w.fuse_cap[r] + 15) // 16
        assert np.all(w.block_table[r, nb:nb + extra] >= 0)
    # each 16-token block belongs to exactly one span (padding to block boundaries)
    for s in range(len(w.span_req)):
        assert w.span_start[s] % 16 == 0
    # span blocks are never also used as private blocks
    priv = set()
    for r in range(B):
        nq = w.q_start[r + 1] - w.q_start[r]
        n = w.kv_len[r]
        first_own = (n - nq) // 16
        last = (n + 15) // 16 + (w.fuse_cap[r] + 15) // 16
        priv.update(int(b) for b in w.block_table[r, first_own:last])
    assert not (priv & set(w.shared_blocks.tolist()))


def test_shared_spans_appear_at_different_offsets():
    w = SMALL["shared_serving"]()
    first = {}
    moved = 0
    for r in range(w.batch):
        for b in range((w.kv_len[r] - 16) // 16):
            blk = int(w.block_table[r, b])
            pos = int(w.kv_pos[r, b * 16])
            if blk in first and first[blk] != pos:
                moved += 1
            first.setdefault(blk, pos)
    assert moved > 0


def test_decode_offsets_not_block_aligned():
    w = SMALL["decode_heavy"]()
    assert np.any(w.kv_pos[:, 0] % 16 != 0)
    assert np.all(np.diff(w.q_start) == 1)


def test_recompute_queries_layout():
    w = W.tiny()
    pos = [np.array([456, 3, 200, 17], np.int32)]
    a = W.recompute_queries(w, pos, seed=5)
    b = W.recompute_queries(w, pos, seed=5)
    assert a.q.shape == (4, w.num_q_heads, w.head_dim) and a.q.dtype == np.uint16
    assert np.array_equal(a.q, b.q)                       # seeded
    assert a.q_pos.tolist() == [3, 17, 200, 456]          # ordered by position
    assert a.q_start.tolist() == [0, 4]
    assert a.pool_k is w.pool_k and a.kv_pos is w.kv_pos  # cache shared, not copied
    e = W.recompute_queries(w, [np.zeros(0, np.int32)], seed=5)
    assert e.total_q == 0 and e.q_start.tolist() == [0, 0]
