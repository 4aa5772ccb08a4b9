"""Plain reference of MiniPIC's block-hash primitives (TEST INFRASTRUCTURE ONLY).

The product package never imports this module; only the test suite uses it.
It shares no code with the library's C++ implementation.

What it computes.  [MiniPIC: "Resumen Tecnico: MiniPIC ...", section 2.2:
user-controlled reuse primitives implemented as special tokens that change
how KV blocks are hashed.]

  - Padding: the user pads spans to KV-block boundaries so that the special
    tokens open a block.  Reading: a PAD token's slot holds no key (pi = -1)
    and does not advance the logical position.
  - SSEP at the start of a block restarts the hash chain from the root,
    h_i = H(h_0, x_i): the span is cacheable whatever precedes it.  Reading:
    the following blocks chain on the restarted hash as usual.
  - PDEP at the start of a block makes its hash depend on the whole preceding
    prompt, h_i = H(h_0, x_<=i).  Reading: the unbroken chain over every token
    of the request up to and including the block.
  - Otherwise a block chains on its predecessor (prefix caching).

Readings the page leaves open: H is 64-bit FNV-1a (Fowler-Noll-Vo, published
definition) over the 8 little-endian bytes of the parent hash followed by the
4 little-endian bytes of each token id; h_0 is the FNV-1a offset basis; only
full blocks are cacheable (a partial last block is always private); a miss
takes the lowest free block id; SSEP / PDEP are ordinary tokens for positions.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1
BLOCK = 16


def fnv1a64(data: bytes, h: int = FNV_OFFSET) -> int:
    """64-bit FNV-1a: for each byte, xor it in, then multiply by the prime."""
    for b in data:
        h ^= b
        h = (h * FNV_PRIME) & MASK64
    return h


def chain(parent: int, tokens: Sequence[int]) -> int:
    """H(parent, tokens): FNV-1a over the parent hash and the token ids."""
    data = parent.to_bytes(8, "little") + b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens)
    return fnv1a64(data)


def block_hashes(tokens: Sequence[int], ssep: int, pdep: int) -> List[int]:
    """Hash of every full block of one request's token stream."""
    out = []
    h = FNV_OFFSET      # the chain that SSEP restarts
    g = FNV_OFFSET      # the unbroken chain over the whole prompt
    for b in range(len(tokens) // BLOCK):
        x = list(tokens[b * BLOCK:(b + 1) * BLOCK])
        g = chain(g, x)
        if x[0] == ssep:
            h = chain(FNV_OFFSET, x)
        elif x[0] == pdep:
            h = g
        else:
            h = chain(h, x)
        out.append(h)
    return out


class BlockCache:
    """hash -> physical block id, with the lowest free id taken on a miss."""

    def __init__(self, num_blocks: int):
        self.free = list(range(num_blocks))
        self.by_hash: Dict[int, int] = {}

    def take(self) -> int:
        if not self.free:
            raise MemoryError("no free block")
        self.free.sort()
        return self.free.pop(0)

    def map_request(self, tokens: Sequence[int], pad: int, ssep: int, pdep: int
                    ) -> Tuple[List[int], List[int], List[int]]:
        """(block_table, kv_pos, miss): miss[b] = 1 when block b was newly taken
        (its K/V must be computed), 0 when an equal cached block is reused."""
        hashes = block_hashes(tokens, ssep, pdep)
        nblk = (len(tokens) + BLOCK - 1) // BLOCK
        table, miss = [], []
        for b in range(nblk):
            if b < len(hashes) and hashes[b] in self.by_hash:
                table.append(self.by_hash[hashes[b]])
                miss.append(0)
                continue
            blk = self.take()
            if b < len(hashes):
                self.by_hash[hashes[b]] = blk
            table.append(blk)
            miss.append(1)
        pos, p = [], 0
        for t in tokens:
            if t == pad:
                pos.append(-1)
            else:
                pos.append(p)
                p += 1
        return table, pos, miss
