// Host-side block hashing for user-controlled span reuse (MiniPIC,
// gist.science 2606.13126, section 2.2: padding, SSEP and PDEP special tokens
// change how KV blocks are hashed).  Turns a request's token stream into the
// block table and per-slot logical positions the attention entry points take,
// reusing cached blocks wherever the hash chain says the content is the same.
//
//  - A block's hash chains on its predecessor's (prefix caching).
//  - A block opened by SSEP restarts the chain from the root: the span is
//    cacheable whatever precedes it, so one physical block serves it at any
//    offset (the kernels rotate keys at each request's own positions).
//  - A block opened by PDEP takes the unbroken chain over every token of the
//    request so far: it only matches an identical prompt.
//  - H is 64-bit FNV-1a over the parent hash (8 bytes, little-endian) and the
//    block's token ids (4 bytes each, little-endian); the root is the FNV
//    offset basis.  Only full blocks are cacheable; PAD slots hold no key
//    (pi = -1) and do not advance the position; a miss takes the lowest free
//    block id.
#include <cstdint>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "pic_attn.h"

struct pic_block_cache {
    std::unordered_map<uint64_t, int32_t> by_hash;
    std::set<int32_t> free_ids;
};

namespace {

constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

inline uint64_t fnv_byte(uint64_t h, uint8_t b) { return (h ^ b) * kFnvPrime; }

// H(parent, tokens[0..n))
uint64_t chain(uint64_t parent, const int32_t *tokens, int n) {
    uint64_t h = kFnvOffset;
    for (int i = 0; i < 8; ++i) h = fnv_byte(h, (uint8_t)(parent >> (8 * i)));
    for (int t = 0; t < n; ++t) {
        const uint32_t u = (uint32_t)tokens[t];
        for (int i = 0; i < 4; ++i) h = fnv_byte(h, (uint8_t)(u >> (8 * i)));
    }
    return h;
}

}  // namespace

extern "C" {

pic_status pic_block_cache_create(int32_t num_blocks, pic_block_cache **out) {
    if (!out) return PIC_ERR_INVALID_ARG;
    *out = nullptr;
    if (num_blocks <= 0) return PIC_ERR_INVALID_ARG;
    pic_block_cache *c = new (std::nothrow) pic_block_cache;
    if (!c) return PIC_ERR_HIP;
    for (int32_t i = 0; i < num_blocks; ++i) c->free_ids.insert(c->free_ids.end(), i);
    *out = c;
    return PIC_OK;
}

void pic_block_cache_destroy(pic_block_cache *cache) { delete cache; }

pic_status pic_block_map(pic_block_cache *cache, const int32_t *tokens, int32_t n_tokens, int32_t pad_token,
                         int32_t ssep_token, int32_t pdep_token, int32_t *block_table, int32_t max_blocks,
                         int32_t *kv_pos, int32_t *miss, int32_t *n_blocks) {
    if (!cache || !n_blocks || n_tokens < 0 || (n_tokens > 0 && !tokens) || max_blocks < 0)
        return PIC_ERR_INVALID_ARG;
    const int32_t nblk = (int32_t)(((int64_t)n_tokens + PIC_BLOCK_SIZE - 1) / PIC_BLOCK_SIZE);
    if (nblk > max_blocks || (nblk > 0 && (!block_table || !kv_pos || !miss))) return PIC_ERR_INVALID_ARG;
    const int32_t nfull = n_tokens / PIC_BLOCK_SIZE;

    // hashes of the full blocks
    std::vector<uint64_t> hs((size_t)nfull);
    uint64_t h = kFnvOffset, g = kFnvOffset;
    for (int32_t b = 0; b < nfull; ++b) {
        const int32_t *x = tokens + (size_t)b * PIC_BLOCK_SIZE;
        g = chain(g, x, PIC_BLOCK_SIZE);
        if (x[0] == ssep_token) h = chain(kFnvOffset, x, PIC_BLOCK_SIZE);
        else if (x[0] == pdep_token) h = g;
        else h = chain(h, x, PIC_BLOCK_SIZE);
        hs[(size_t)b] = h;
    }
    // fresh blocks this request needs (a hash repeated inside the request is
    // taken once); refuse before changing anything if the pool is short
    size_t need = (size_t)(nblk - nfull);
    {
        std::unordered_map<uint64_t, int> seen;
        for (int32_t b = 0; b < nfull; ++b)
            if (!cache->by_hash.count(hs[(size_t)b]) && seen.emplace(hs[(size_t)b], 1).second) ++need;
    }
    if (need > cache->free_ids.size()) return PIC_ERR_WORKSPACE;

    for (int32_t b = 0; b < nblk; ++b) {
        if (b < nfull) {
            auto it = cache->by_hash.find(hs[(size_t)b]);
            if (it != cache->by_hash.end()) {
                block_table[b] = it->second;
                miss[b] = 0;
                continue;
            }
        }
        const int32_t id = *cache->free_ids.begin();
        cache->free_ids.erase(cache->free_ids.begin());
        if (b < nfull) cache->by_hash.emplace(hs[(size_t)b], id);
        block_table[b] = id;
        miss[b] = 1;
    }
    int32_t p = 0;
    for (int32_t t = 0; t < n_tokens; ++t) kv_pos[t] = tokens[t] == pad_token ? -1 : p++;
    for (int64_t t = n_tokens; t < (int64_t)nblk * PIC_BLOCK_SIZE; ++t) kv_pos[t] = -1;
    *n_blocks = nblk;
    return PIC_OK;
}

}  // extern "C"
