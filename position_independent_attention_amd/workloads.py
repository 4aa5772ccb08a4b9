"""Seeded synthetic inputs for position-independent attention over reused KV spans.

This module builds input *data and structure* only: a paged pool of unrotated
K and V, per-request block tables, per-request logical-position maps (pi),
query tokens and their positions, span descriptors and fresh K/V rows for
cache fusion.  It computes none of the method's arithmetic (no rotation, no
softmax, no selection budget), so both the HIP path and the CPU oracle can
take their inputs from here without sharing any of the computation.

Shapes follow the workloads the pages describe:
  * MiniPIC (gist.science 2606.13126, section 2.1): documents ("spans") cached
    once with unrotated keys and reused at other logical offsets, with the same
    physical blocks referenced by concurrent requests at different offsets.
  * MiniPIC section 2.2 (Padding): spans are padded to KV-block boundaries, so
    every 16-token block belongs to exactly one span.
  * QCFuse (gist.science 2604.08585, methodology B/C): retrieved chunks that
    overlap across queries; a fraction of each chunk's tokens is recomputed
    and mixed back into the cache, which needs request-private blocks.

Layouts (all little-endian, bf16 stored as uint16 bit patterns):
  pool_k      uint16 [num_blocks][Hkv][16][d]   unrotated keys, token-major
  pool_v      uint16 [num_blocks][Hkv][d][16]   values, head-dim-major per block
  block_table int32  [B][max_blocks]            physical block of logical block
  kv_len      int32  [B]                        tokens in each request sequence
  kv_pos      int32  [B][max_blocks*16]         pi: logical position, -1 = empty
  q           uint16 [total_q][Hq][d]           unrotated queries
  q_start     int32  [B+1]                      CSR of queries per request
  q_pos       int32  [total_q]                  logical position of each query
  spans       int32  span_req/span_start/span_len (request-sequence indices)
  fresh_k/v   uint16 [cap][Hkv][d]              recomputed rows for fusion
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Input encoding only; finite inputs assumed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rope_theta: float
    max_position: int
    batch: int
    pool_k: np.ndarray
    pool_v: np.ndarray
    block_table: np.ndarray
    kv_len: np.ndarray
    kv_pos: np.ndarray
    q: np.ndarray
    q_start: np.ndarray
    q_pos: np.ndarray
    span_req: np.ndarray
    span_start: np.ndarray
    span_len: np.ndarray
    ratio: float
    fresh_k: np.ndarray
    fresh_v: np.ndarray
    fuse_cap: np.ndarray          # int32 [B]: rows that fit in the appended private blocks
    shared_blocks: np.ndarray     # int32: physical ids of span blocks (never to be written)
    decode: bool = False
    seed: int = 0

    # ---- derived sizes -------------------------------------------------
    @property
    def block_size(self) -> int:
        return BLOCK

    @property
    def num_blocks(self) -> int:
        return int(self.pool_k.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def max_q_len(self) -> int:
        return int(np.max(np.diff(self.q_start))) if self.batch else 0

    @property
    def max_kv_len(self) -> int:
        return int(np.max(self.kv_len)) if self.batch else 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def copy(self) -> "Workload":
        out = dataclasses.replace(self)
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            if isinstance(v, np.ndarray):
                setattr(out, f.name, v.copy())
        return out


@dataclasses.dataclass
class Piece:
    """A run of tokens placed contiguously in a request's sequence.

    `blocks` are logical pool-block indices (before the physical permutation);
    the piece occupies len(blocks) whole blocks of the request and its first
    `ntok` tokens get logical positions pos0, pos0+1, ...
    """
    blocks: List[int]
    pos0: int
    ntok: int
    span: bool            # a reusable span (a selection candidate)


def _normal_bf16(rng: np.random.Generator, shape: Tuple[int, ...], scale: float = 1.0,
                 chunk: int = 1 << 24) -> np.ndarray:
    """N(0, scale^2) samples drawn as float32 and rounded to bf16, in chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[s:e] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def assemble(name: str, *, seed: int, Hq: int, Hkv: int, d: int, theta: float,
             requests: Sequence[Sequence[Piece]], q_len: Sequence[int],
             q_pos0: Sequence[int], n_logical_blocks: int, shared_logical: Sequence[int],
             kv_scale: float = 1.0, ratio: float = 0.25, fuse_cap: Optional[Sequence[int]] = None,
             decode: bool = False, max_position: int = 65536,
             rng: Optional[np.random.Generator] = None, pool_values: bool = True) -> Workload:
    """Lay pieces out into a paged pool and per-request tables.

    Draw order from `rng` (PCG64 seeded with `seed` unless given): block-id
    permutation, K pool, V pool, q, fresh K, fresh V.  With pool_values=False
    the K and V pools are not drawn: pool_k / pool_v are read-only zero views
    of the pool's shape that hold no memory, for callers that fill a pool of
    that layout themselves (a multi-GiB timing pool drawn on the device).  Each request gets
    `q_len[r]` own query tokens at positions q_pos0[r].., whose (unrotated) K/V
    live in request-private blocks at the end of its sequence, plus
    ceil(fuse_cap[r]/16) more private blocks appended (reserved for fused rows).
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    B = len(requests)
    fuse_cap = list(fuse_cap) if fuse_cap is not None else [0] * B

    # Private blocks: the query block of each request, then the fusion blocks.
    next_logical = n_logical_blocks
    own_blocks, fuse_blocks = [], []
    for r in range(B):
        nb = (q_len[r] + BLOCK - 1) // BLOCK
        own_blocks.append(list(range(next_logical, next_logical + nb)))
        next_logical += nb
    for r in range(B):
        nb = (fuse_cap[r] + BLOCK - 1) // BLOCK
        fuse_blocks.append(list(range(next_logical, next_logical + nb)))
        next_logical += nb
    n_total = next_logical
    perm = rng.permutation(n_total).astype(np.int32)   # logical block -> physical id

    seq_blocks = []
    for r in range(B):
        nb = sum(len(p.blocks) for p in requests[r]) + len(own_blocks[r]) + len(fuse_blocks[r])
        seq_blocks.append(nb)
    max_blocks = max(seq_blocks) if B else 1
    block_table = np.full((B, max_blocks), -1, dtype=np.int32)
    kv_pos = np.full((B, max_blocks * BLOCK), -1, dtype=np.int32)
    kv_len = np.zeros(B, dtype=np.int32)
    span_req, span_start, span_len = [], [], []
    for r in range(B):
        cur = 0
        for p in requests[r]:
            for i, lb in enumerate(p.blocks):
                block_table[r, cur // BLOCK + i] = perm[lb]
            kv_pos[r, cur:cur + p.ntok] = np.arange(p.pos0, p.pos0 + p.ntok, dtype=np.int32)
            if p.span:
                span_req.append(r)
                span_start.append(cur)
                span_len.append(p.ntok)
            cur += len(p.blocks) * BLOCK
        for i, lb in enumerate(own_blocks[r]):
            block_table[r, cur // BLOCK + i] = perm[lb]
        kv_pos[r, cur:cur + q_len[r]] = np.arange(q_pos0[r], q_pos0[r] + q_len[r], dtype=np.int32)
        kv_len[r] = cur + q_len[r]
        cur2 = cur + len(own_blocks[r]) * BLOCK
        for i, lb in enumerate(fuse_blocks[r]):
            block_table[r, cur2 // BLOCK + i] = perm[lb]

    if pool_values:
        pool_k = _normal_bf16(rng, (n_total, Hkv, BLOCK, d), kv_scale)
        v_tok = _normal_bf16(rng, (n_total, Hkv, BLOCK, d), kv_scale)
        pool_v = np.ascontiguousarray(v_tok.transpose(0, 1, 3, 2))
        del v_tok
    else:
        pool_k = np.broadcast_to(np.uint16(0), (n_total, Hkv, BLOCK, d))
        pool_v = np.broadcast_to(np.uint16(0), (n_total, Hkv, d, BLOCK))

    total_q = int(sum(q_len))
    q = _normal_bf16(rng, (total_q, Hq, d))
    q_start = np.zeros(B + 1, dtype=np.int32)
    q_start[1:] = np.cumsum(np.asarray(q_len, dtype=np.int64))
    q_pos = np.concatenate([np.arange(q_pos0[r], q_pos0[r] + q_len[r], dtype=np.int32)
                            for r in range(B)]) if total_q else np.zeros(0, np.int32)
    cap = int(sum(fuse_cap))
    fresh_k = _normal_bf16(rng, (cap, Hkv, d))
    fresh_v = _normal_bf16(rng, (cap, Hkv, d))
    shared = np.array(sorted(int(perm[b]) for b in shared_logical), dtype=np.int32)
    return Workload(
        name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, rope_theta=float(theta),
        max_position=max_position, batch=B, pool_k=pool_k, pool_v=pool_v,
        block_table=block_table, kv_len=kv_len, kv_pos=kv_pos, q=q, q_start=q_start,
        q_pos=q_pos, span_req=np.asarray(span_req, np.int32),
        span_start=np.asarray(span_start, np.int32), span_len=np.asarray(span_len, np.int32),
        ratio=float(ratio), fresh_k=fresh_k, fresh_v=fresh_v,
        fuse_cap=np.asarray(fuse_cap, np.int32), shared_blocks=shared, decode=decode, seed=seed)


def _cap_for(span_lens: Sequence[int], ratio: float) -> int:
    # Storage upper bound for fused rows: ceil(ratio*L)+1 per span is always
    # at least the selection budget, whichever rounding rule the selector uses.
    return int(sum(math.ceil(ratio * L) + 1 for L in span_lens))


def _blocks(n_tok: int) -> int:
    return (n_tok + BLOCK - 1) // BLOCK


# ---------------------------------------------------------------------------
# The five workload shapes and their controls.
# ---------------------------------------------------------------------------

def tiny(seed: int = 1001) -> Workload:
    """1 request, 4 q heads / 1 kv head, d 64, theta 1e4; two 128-token spans at
    logical offsets 0 and 200; 16 query tokens at 456..471; top-25% per span."""
    rng = np.random.default_rng(seed)
    pieces = [Piece(list(range(0, 8)), 0, 128, True), Piece(list(range(8, 16)), 200, 128, True)]
    return assemble("tiny", seed=seed, Hq=4, Hkv=1, d=64, theta=1e4, requests=[pieces],
                    q_len=[16], q_pos0=[456], n_logical_blocks=16, shared_logical=range(16),
                    ratio=0.25, fuse_cap=[_cap_for([128, 128], 0.25)], rng=rng)


def llama_layer(seed: int = 1002, ratio: float = 0.25) -> Workload:
    """32/8 heads, d 128, theta 5e5; 64-token private prefix at 0..63, then eight
    512-token spans in a random order at contiguous offsets; 64 query tokens;
    K,V ~ N(0,1)*0.5; batch 1."""
    rng = np.random.default_rng(seed)
    order = rng.permutation(8)
    spb = 512 // BLOCK
    pieces = [Piece(list(range(8 * spb, 8 * spb + 4)), 0, 64, False)]   # private prefix
    pos = 64
    for s in order:
        pieces.append(Piece(list(range(int(s) * spb, (int(s) + 1) * spb)), pos, 512, True))
        pos += 512
    return assemble("llama_layer", seed=seed, Hq=32, Hkv=8, d=128, theta=5e5, requests=[pieces],
                    q_len=[64], q_pos0=[pos], n_logical_blocks=8 * spb + 4,
                    shared_logical=range(8 * spb), kv_scale=0.5, ratio=ratio,
                    fuse_cap=[_cap_for([512] * 8, ratio)], rng=rng)


def shared_serving(seed: int = 1003, batch: int = 16, n_pool_spans: int = 64, span_tok: int = 1024,
                   spans_per_req: int = 8, q_len: int = 128, ratio: float = 0.25) -> Workload:
    """A pool of 64 spans x 1024 tokens stored once; 16 requests each pick 8
    distinct spans in a random order (so the same physical blocks appear at
    different logical offsets); 128 query tokens each; 32/8 heads, d 128."""
    rng = np.random.default_rng(seed)
    spb = span_tok // BLOCK
    reqs = []
    for _ in range(batch):
        pick = rng.choice(n_pool_spans, size=spans_per_req, replace=False)
        pieces, pos = [], 0
        for s in pick:
            pieces.append(Piece(list(range(int(s) * spb, (int(s) + 1) * spb)), pos, span_tok, True))
            pos += span_tok
        reqs.append(pieces)
    ctx = spans_per_req * span_tok
    return assemble("shared_serving", seed=seed, Hq=32, Hkv=8, d=128, theta=5e5, requests=reqs,
                    q_len=[q_len] * batch, q_pos0=[ctx] * batch,
                    n_logical_blocks=n_pool_spans * spb, shared_logical=range(n_pool_spans * spb),
                    ratio=ratio, fuse_cap=[_cap_for([span_tok] * spans_per_req, ratio)] * batch,
                    rng=rng)


def long_context(seed: int = 1004, n_spans: int = 32, span_tok: int = 1024, q_len: int = 256,
                 ratio: float = 0.15) -> Workload:
    """32 spans x 1024 = 32k context in a random order, 256 query tokens,
    32/8 heads, d 128; keep the top 15% per span for recompute."""
    rng = np.random.default_rng(seed)
    spb = span_tok // BLOCK
    order = rng.permutation(n_spans)
    pieces, pos = [], 0
    for s in order:
        pieces.append(Piece(list(range(int(s) * spb, (int(s) + 1) * spb)), pos, span_tok, True))
        pos += span_tok
    return assemble("long_context", seed=seed, Hq=32, Hkv=8, d=128, theta=5e5, requests=[pieces],
                    q_len=[q_len], q_pos0=[pos], n_logical_blocks=n_spans * spb,
                    shared_logical=range(n_spans * spb), ratio=ratio,
                    fuse_cap=[_cap_for([span_tok] * n_spans, ratio)], rng=rng)


def decode_heavy(seed: int = 1005, batch: int = 64, n_spans: int = 16, span_tok: int = 1024,
                 private_spans: bool = False, Hq: int = 64, pool_values: bool = True) -> Workload:
    """Batch 64, one query token per request, 16k context built from 16 shared
    1024-token spans in a per-request random order starting at a per-request
    random offset b_r in [0, 1024); 64 q / 8 kv heads, d 128.

    private_spans=True is the unshared control: every request owns its own
    16 spans, so the pool (4 GiB at the default shape) exceeds on-chip caches.
    """
    rng = np.random.default_rng(seed)
    spb = span_tok // BLOCK
    reqs, q_pos0 = [], []
    for r in range(batch):
        order = rng.permutation(n_spans)
        base = int(rng.integers(0, 1024))
        pieces, pos = [], base
        off = r * n_spans if private_spans else 0
        for s in order:
            lb0 = (off + int(s)) * spb
            pieces.append(Piece(list(range(lb0, lb0 + spb)), pos, span_tok, True))
            pos += span_tok
        reqs.append(pieces)
        q_pos0.append(pos)
    n_log = (batch if private_spans else 1) * n_spans * spb
    return assemble("decode_heavy_private" if private_spans else "decode_heavy", seed=seed,
                    Hq=Hq, Hkv=8, d=128, theta=5e5, requests=reqs, q_len=[1] * batch,
                    q_pos0=q_pos0, n_logical_blocks=n_log,
                    shared_logical=range(0 if private_spans else n_log), decode=True, rng=rng,
                    pool_values=pool_values)


def custom(seed: int, *, Hq: int, Hkv: int, d: int, theta: float, span_lens: Sequence[Sequence[int]],
           gaps: Optional[Sequence[Sequence[int]]] = None, q_len: Sequence[int],
           q_gap: Sequence[int] = (), ratio: float = 0.25, kv_scale: float = 1.0,
           decode: bool = False, max_position: int = 65536) -> Workload:
    """Small shape-parametrised layouts for edge and tail cases.

    Request r holds spans of lengths span_lens[r] (any length; the tail of a
    span's last block stays empty, pi = -1), each starting gaps[r][i] positions
    after the previous one ends, then q_len[r] query tokens q_gap[r] positions
    after the last span.
    """
    rng = np.random.default_rng(seed)
    B = len(span_lens)
    reqs, qp0, nlog = [], [], 0
    for r in range(B):
        pieces, pos = [], 0
        for i, L in enumerate(span_lens[r]):
            if gaps is not None:
                pos += int(gaps[r][i])
            nb = _blocks(L)
            pieces.append(Piece(list(range(nlog, nlog + nb)), pos, int(L), True))
            nlog += nb
            pos += int(L)
        reqs.append(pieces)
        qp0.append(pos + (int(q_gap[r]) if len(q_gap) else 0))
    caps = [_cap_for(span_lens[r], ratio) for r in range(B)]
    return assemble("custom", seed=seed, Hq=Hq, Hkv=Hkv, d=d, theta=theta, requests=reqs,
                    q_len=list(q_len), q_pos0=qp0, n_logical_blocks=nlog,
                    shared_logical=range(nlog), kv_scale=kv_scale, ratio=ratio, fuse_cap=caps,
                    decode=decode, max_position=max_position, rng=rng)



def fresh_queries(n: int, Hq: int, d: int, seed: int) -> np.ndarray:
    """n recomputed query tokens, N(0,1) rounded to bf16 bits [n][Hq][d]."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((n, Hq, d), dtype=np.float32))


def recompute_queries(w: Workload, q_pos_per_req: Sequence[np.ndarray], seed: int) -> Workload:
    """Discrete-token recompute (QCFuse's sparse recompute): each request's
    recomputed tokens become its query tokens at their own logical positions,
    over the cache held in `w` (normally the fused cache).  Fresh queries are
    N(0,1) rounded to bf16; a request's queries are ordered by position (any
    order gives the same per-query result).  The returned workload shares w's
    cache arrays and spans."""
    pos = [np.sort(np.asarray(p, np.int32)) for p in q_pos_per_req]
    assert len(pos) == w.batch
    q_start = np.zeros(w.batch + 1, np.int32)
    q_start[1:] = np.cumsum([len(p) for p in pos])
    n = int(q_start[-1])
    q = fresh_queries(n, w.num_q_heads, w.head_dim, seed)
    out = dataclasses.replace(w)
    out.name = w.name + "_recompute"
    out.q = q
    out.q_start = q_start
    out.q_pos = np.concatenate(pos).astype(np.int32) if n else np.zeros(0, np.int32)
    out.decode = False
    return out

CONFIGS = {
    "tiny": tiny,
    "llama_layer": llama_layer,
    "shared_serving": shared_serving,
    "long_context": long_context,
    "decode_heavy": decode_heavy,
}
