"""MiniPIC's block-hash primitives (padding, SSEP, PDEP): the plain reference
pinned to the published FNV-1a vectors and to the reuse rules section 2.2 of
the MiniPIC page states, then the library's C++ implementation against it."""
import numpy as np
import pytest

from oracle import block_hash as BH
from position_independent_attention_amd import pic

PAD, SSEP, PDEP = -1, 1, 2


def span(seed, n):
    """n ordinary tokens (ids >= 10) from a seeded generator."""
    return np.random.default_rng(seed).integers(10, 50000, n).tolist()


def padded(tokens, first=None):
    """A span opened by a special token and padded to a block boundary."""
    t = ([first] if first is not None else []) + list(tokens)
    return t + [PAD] * ((-len(t)) % BH.BLOCK)


# ------------------------------------------------------------ the reference

def test_fnv1a64_published_vectors():
    assert BH.fnv1a64(b"") == 0xCBF29CE484222325
    assert BH.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert BH.fnv1a64(b"foobar") == 0x85944171F73967E8


def test_plain_prefix_caching_without_markers():
    c = BH.BlockCache(64)
    common = span(1, 32)
    t1, _, m1 = c.map_request(common + span(2, 32), PAD, SSEP, PDEP)
    t2, _, m2 = c.map_request(common + span(3, 32), PAD, SSEP, PDEP)
    assert t2[:2] == t1[:2] and m2[:2] == [0, 0]          # shared prefix blocks
    assert not set(t2[2:]) & set(t1) and m2[2:] == [1, 1]


def test_ssep_span_is_reused_at_any_offset():
    s = padded(span(4, 40), SSEP)                          # 3 blocks
    c = BH.BlockCache(64)
    t1, p1, _ = c.map_request(padded(span(5, 16)) + s, PAD, SSEP, PDEP)
    t2, p2, m2 = c.map_request(padded(span(6, 48)) + s, PAD, SSEP, PDEP)
    assert t2[3:6] == t1[1:4] and m2[3:6] == [0, 0, 0]    # same blocks at another offset
    assert p1[16] == 16 and p2[48] == 48                   # positions follow the request
    # the same span without SSEP chains on its context: no reuse
    c2 = BH.BlockCache(64)
    plain = padded(span(4, 40), 7)
    a, _, _ = c2.map_request(padded(span(5, 16)) + plain, PAD, SSEP, PDEP)
    b, _, mb = c2.map_request(padded(span(6, 48)) + plain, PAD, SSEP, PDEP)
    assert not set(b[3:]) & set(a) and mb[3:] == [1, 1, 1]


def test_pdep_block_depends_on_the_whole_prompt():
    s = padded(span(7, 30), SSEP)
    suffix = padded(span(8, 10), PDEP)
    c = BH.BlockCache(64)
    t1, _, _ = c.map_request(padded(span(9, 16)) + s + suffix, PAD, SSEP, PDEP)
    t2, _, m2 = c.map_request(padded(span(10, 16)) + s + suffix, PAD, SSEP, PDEP)
    assert t2[1:3] == t1[1:3]                               # the SSEP span is shared
    assert t2[3] != t1[3] and m2[3] == 1                    # the PDEP block is not
    t3, _, m3 = c.map_request(padded(span(9, 16)) + s + suffix, PAD, SSEP, PDEP)
    assert t3 == t1 and m3 == [0, 0, 0, 0]                  # same prompt: all hits
    assert BH.block_hashes(padded(span(9, 16)) + s + suffix, SSEP, PDEP)[3] == \
        BH.chain(BH.chain(BH.chain(BH.chain(BH.FNV_OFFSET, (padded(span(9, 16)) + s)[:16]),
                                   s[:16]), s[16:32]), suffix)


def test_pad_slots_are_masked_and_partial_blocks_never_shared():
    toks = padded(span(11, 5), SSEP) + span(12, 20)        # 16 + 20 tokens: last block partial
    c = BH.BlockCache(8)
    t1, p1, m1 = c.map_request(toks, PAD, SSEP, PDEP)
    assert p1[:6] == [0, 1, 2, 3, 4, 5] and all(x == -1 for x in p1[6:16])
    assert p1[16] == 6 and p1[-1] == 6 + 19
    t2, _, m2 = c.map_request(toks, PAD, SSEP, PDEP)
    assert t2[:2] == t1[:2] and m2[:2] == [0, 0]
    assert t2[2] != t1[2] and m2[2] == 1                    # the partial block is private
    s = padded(span(13, 16), SSEP)                          # 17 tokens -> 2 blocks
    t3, _, m3 = BH.BlockCache(8).map_request(s + span(14, 3) + [PAD] * 13 + s, PAD, SSEP, PDEP)
    assert t3[3:5] == t3[0:2] and m3 == [1, 1, 1, 0, 0]     # repeated span inside one request


# -------------------------------------------------------- the C++ library

def random_requests(seed, n_req):
    rng = np.random.default_rng(seed)
    pool = [padded(span(100 + i, int(rng.integers(1, 60))), SSEP) for i in range(6)]
    reqs = []
    for _ in range(n_req):
        t = padded(span(int(rng.integers(1000, 2000)), int(rng.integers(1, 40))))
        for _ in range(int(rng.integers(1, 5))):
            t += pool[int(rng.integers(0, 6))]
        if rng.random() < 0.5:
            t += padded(span(int(rng.integers(3000, 3010)), int(rng.integers(1, 30))), PDEP)
        t += span(int(rng.integers(4000, 5000)), int(rng.integers(0, 40)))
        reqs.append(t)
    return reqs


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_library_matches_reference(seed):
    reqs = random_requests(seed, 12)
    ref = BH.BlockCache(4096)
    cache = pic.BlockCache(4096)
    for t in reqs:
        rt, rp, rm = ref.map_request(t, PAD, SSEP, PDEP)
        gt, gp, gm = cache.map_request(np.asarray(t, np.int32), PAD, SSEP, PDEP)
        assert gt.tolist() == rt and gp.tolist() == rp and gm.tolist() == rm
    cache.close()


def test_library_reports_exhausted_pool():
    cache = pic.BlockCache(2)
    with pytest.raises(pic.PicError):
        cache.map_request(np.asarray(span(1, 40), np.int32), PAD, SSEP, PDEP)
    cache.close()
