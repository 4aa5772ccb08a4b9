// Prefill-style kernels for gfx950: attention of many query tokens over a
// request's paged, unrotated KV cache with RoPE applied in-kernel at each
// key's logical position (MiniPIC, gist.science 2606.13126, section 2.1 score
// equation), in three modes sharing one tile pipeline:
//   kAttn  online-softmax attention -> O (bf16) and LSE, or split partials
//   kLse   the same scores, only the running max / sum -> LSE
//   kMass  p = exp(s - lse) column-summed over the query rows -> per-key
//          selection mass (QCFuse, gist.science 2604.08585, methodology B)
//
// Work decomposition
//   A workgroup (4 or 8 wave64) owns one (request, kv head, key split, row
//   block).
//   The G query heads of a kv head are packed with the request's query tokens
//   into "rows" (row = token * G + head-in-group), so one rotated K tile feeds
//   G * n_q rows.  Each wave owns 16*QG rows.
//
//   The scores are computed transposed, S^T = K Q^T, with
//   v_mfma_f32_16x16x32_bf16: K rows are the MFMA rows, query rows the MFMA
//   columns.  A lane then holds all the scores of its own query column, so
//   the softmax statistics, the O^T accumulator and the rescale all stay in
//   the lane's own column.  The two 16-key MFMA tiles of a 32-key half are
//   fed with interleaved key rows (tile T, row m -> key 8*(m/4) + 4*T + m%4),
//   which leaves every lane with 8 consecutive keys: exactly the B operand
//   layout that P^T needs for O^T += V^T P^T, with no shuffle.
//
// Pipeline per 64-key tile (LDS double-buffered, one barrier per tile)
//   - block ids and pi are loaded two tiles ahead, so the K / V / cos / sin
//     loads of the next tile are issued at the top of the iteration without
//     waiting on them;
//   - the current tile is computed from LDS in two 32-key halves;
//   - the next tile's K is rotated in registers with the fp32 cos/sin row of
//     each key's pi (every key rotated once per workgroup however many rows
//     read it), rounded to bf16 and written to the other LDS buffer with the
//     V^T tile (a plain copy: V is stored head-dim-major per block);
//   - unusable keys (pi = -1, no block, past the end) are cut without a
//     per-score test: their K rows load as zeros and the QK^T accumulators
//     start at each key's bias (0, or -inf for an unusable key);
//   - a pre-pass over the workgroup's key range finds the first and the last
//     usable key that some row does not see yet; tiles outside that range
//     take a mask-free fast path (in attention; the mass kernel's pre-pass
//     also counts unusable keys as needing the mask).
//   Softmax uses a lazy rescale: the running column max only moves (and O is
//   rescaled) when a tile's max exceeds it by more than 2^8, so exp2 of
//   (score*scale - max) stays below 256 and the O accumulator is almost never
//   touched by VALU.
#include "pic_internal.h"

#include <cfloat>
#include <type_traits>

namespace pic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr int kNeedWords = 256;         // tile bit mask of a workgroup: up to 8,192 tiles

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};   // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Finite test on the bit pattern: the kernel sources are built with
// -fno-honor-nans, under which a float compare may not reject a NaN.
__device__ __forceinline__ bool finite_bits(float x) { return (__float_as_uint(x) & 0x7fffffffu) < 0x7f800000u; }

#ifndef PIC_SCHED_HINTS
#define PIC_SCHED_HINTS 0
#endif
// Ask the scheduler for `n` groups of (1 MFMA, v VALU) in the current region.
template <int n, int v>
__device__ __forceinline__ void interleave_hint() {
#if PIC_SCHED_HINTS
#pragma unroll
    for (int i = 0; i < n; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, v, 0);
    }
#endif
}

// Rotate 8 RoPE pairs: lo holds x[i..i+7], hi holds x[i+d/2..i+d/2+7] (bf16),
// c/s the cos/sin of pos * theta^(-2(i+e)/d).  Result times scale (fp32),
// rounded to bf16.
__device__ __forceinline__ void rope8(u32x4 &lo, u32x4 &hi, const f32x4 c0, const f32x4 c1,
                                      const f32x4 s0, const f32x4 s1, float scale = 1.f) {
    const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    u32x4 ro, rh;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float a0 = bf_lo(lo[e]), a1 = bf_hi(lo[e]);
        const float b0 = bf_lo(hi[e]), b1 = bf_hi(hi[e]);
        const float cc0 = c[2 * e], cc1 = c[2 * e + 1], ss0 = s[2 * e], ss1 = s[2 * e + 1];
        ro[e] = pack2(fmaf(a0, cc0, -b0 * ss0) * scale, fmaf(a1, cc1, -b1 * ss1) * scale);
        rh[e] = pack2(fmaf(a0, ss0, b0 * cc0) * scale, fmaf(a1, ss1, b1 * cc1) * scale);
    }
    lo = ro;
    hi = rh;
}

// Workgroups are dispatched round-robin over the 8 XCDs.  Renumber them so
// that consecutive logical ids (which share K/V tiles) run on the same XCD
// and hit the same L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int X = 8;
    const int xcd = bid % X, idx = bid / X;
    const int q = n / X, rem = n % X;
    return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

// Column reductions over the 4 lane groups (16-lane rows) that hold the
// same query column: v_permlane16_swap / v_permlane32_swap with both operands
// equal leave the lane's value and its partner's in the two results.
__device__ __forceinline__ float col_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int WAVES>
struct Geo {
    static constexpr int NT = 64 * WAVES;        // threads per workgroup
    static constexpr int NC = D / 32;            // 32-wide MFMA k chunks along d
    static constexpr int HALF = D / 2;
    static constexpr int PC = D / 16;            // 8-pair chunks per key
    static constexpr int KTASK = kTileN * PC / NT;   // K staging tasks per thread
    static constexpr int VCH = 8 * D / NT;       // V 16-byte chunks per thread
    static constexpr int KBUF = kTileN * D;      // one K tile (bf16 elements), chunk-major
    static constexpr int VBUF = D * kTileN;      // one V^T tile, chunk-major
    static_assert(KTASK >= 1 && VCH >= 1, "staging needs at least one task per thread");
};

// K tile key k = 32*kh + 8*a + 4*T + b lives in LDS row
// krow(k) = 32*kh + 16*T + 4*a + b: the 16 keys that one MFMA operand read
// takes (MFMA row m = 4a + b of tile T) are 16 consecutive rows.
__device__ __forceinline__ int krow(int k) {
    return (k & ~31) | (((k >> 2) & 1) << 4) | (((k >> 3) & 3) << 2) | (k & 3);
}

// LDS tile layouts (gfx950 measured: a ds_read_b128 is conflict-free when
// each 16 consecutive lanes read one aligned 256-byte block in any
// XOR-permuted order; a ds_write_b128 when each 8 consecutive lanes write one
// aligned 128-byte block).  Both tiles are chunk-major: the 16-byte chunks of
// 64 consecutive rows form one 1 KB run, with the row index XOR-ed in its low
// three bits by a function of the chunk.
//  K tile, rows = keys (krow order), chunk ch = elements 8ch..8ch+7 of d.
//  The XOR spreads one key's PC chunks (one 8-lane write group) over the
//  eight 16-byte slots of a 128-byte block.
template <int D>
__device__ __forceinline__ int kxor(int ch) { return (ch % (D / 16)) * (8 / (D / 16)); }
template <int D>
__device__ __forceinline__ int koff(int r, int ch) { return ch * (kTileN * 8) + ((r ^ kxor<D>(ch)) * 8); }
//  V^T tile, rows = d, chunk ch = keys 8ch..8ch+7; rows in 64-row halves.
__device__ __forceinline__ int voff(int d, int ch) {
    return (d >> 6) * (64 * kTileN) + ch * (64 * 8) + (((d & 63) ^ (ch & 7)) * 8);
}
// V staging lane map: each 8 consecutive lanes take 8 consecutive d rows of
// one 8-key chunk (one 128-byte LDS block per write group).
__device__ __forceinline__ void vmap(int tid, int &half, int &dd) {
    const int l = tid & 63;
    half = (l >> 3) & 1;
    dd = (l & 7) | ((l >> 4) << 3);
}

// Staging geometry: staging task u of a thread covers key
// kk = tid / PC + u * (NT / PC) of the 64-key tile, channels 8pc..8pc+7 of
// each half of d (pc = tid % PC).  One wave's keys of one task are 64 / PC
// consecutive keys (8 or 16) starting at a multiple of 64 / PC, so they lie in
// one pool block: the block id is wave-uniform (a scalar load) and a lane's
// row inside the block never changes from tile to tile.
template <int D, int WAVES>
__device__ __forceinline__ int task_key0(int wave, int u) {   // first key of (wave, task u)
    using GG = Geo<D, WAVES>;
    return wave * (64 / GG::PC) + u * (GG::NT / GG::PC);
}

// Word 3 of a raw buffer resource on this architecture: 32-bit data format
// (with a zero format every load would return 0), no swizzle or index stride.
// A raw load whose byte offset lies past the resource's size returns zeros.
constexpr int kRsrcWord3 = 0x00020000;

// Block ids / positions of one tile for this thread's staging tasks, as
// loaded (at clamped indices); the range check is applied where they are used,
// one tile later, so that no wait for these loads sits at the tile start.
template <int D, int WAVES>
struct Meta {
    int32_t kblk[Geo<D, WAVES>::KTASK];   // wave-uniform
    int32_t kpi[Geo<D, WAVES>::KTASK];
    int32_t vblk;      // wave-uniform
    int32_t vkey_pi;   // lanes 0..15: pi of key lane of this wave's V block
};

// Data of one tile for this thread's staging tasks.
template <int D, int WAVES>
struct Data {
    u32x4 klo[Geo<D, WAVES>::KTASK], khi[Geo<D, WAVES>::KTASK];
    f32x4 cs[Geo<D, WAVES>::KTASK][4];     // cos0, cos1, sin0, sin1
    int32_t kpi[Geo<D, WAVES>::KTASK];     // pi if the key is usable, else -1
    u32x4 v[Geo<D, WAVES>::VCH];
    int32_t vmask;                         // bit e: key e of the V chunk is unusable
};

// Unconditional loads at clamped indices, then select: no divergent branches.
// Blocks past the range clamp to the block of the last key; kv_stride (a
// multiple of 16) bounds every position index, since a clamped block index
// times 16 plus a row below 16 stays below it.
template <int D, int WAVES>
__device__ __forceinline__ void meta_load(Meta<D, WAVES> &m, const int32_t *bt, const int32_t *pis, int tile,
                                          int key_end, int tid) {
    using GG = Geo<D, WAVES>;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lastb = (key_end - 1) >> 4;   // key_end >= 1
#pragma unroll
    for (int u = 0; u < GG::KTASK; ++u) {
        const int kb = tile + task_key0<D, WAVES>(wave, u);
        const int bc = min(kb >> 4, lastb);
        m.kblk[u] = bt[bc];
        m.kpi[u] = pis[(uint32_t)(bc * 16 + (kb & 15) + lane / GG::PC)];
    }
    // V staging: every lane of this wave covers keys of tile block (wave & 3)
    const int bv = min((tile >> 4) + (wave & 3), lastb);
    m.vblk = bt[bv];
    m.vkey_pi = pis[(uint32_t)(bv * 16 + (lane & 15))];
}

// ZERO: the K rows of unusable keys are read as zeros (their offsets fall
// outside the range of the block's buffer resource, and such loads return 0),
// so that whatever those pool rows hold cannot turn a score into NaN.
template <int D, int WAVES, bool ZERO = false>
__device__ __forceinline__ void data_load(const FwdParams &p, Data<D, WAVES> &dt, const Meta<D, WAVES> &m, int g,
                                          int tile, int key_end, int tid, bool need_v) {
    using GG = Geo<D, WAVES>;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int pc = lane % GG::PC;
#pragma unroll
    for (int u = 0; u < GG::KTASK; ++u) {
        const int kb = tile + task_key0<D, WAVES>(wave, u);
        const int row = (kb & 15) + lane / GG::PC;   // row inside the block
        const int blk = __builtin_amdgcn_readfirstlane(m.kblk[u]), pi = m.kpi[u];
        const bool bok = (unsigned)blk < (unsigned)p.num_blocks;
        const bool ok = bok && (kb & ~15) + row < key_end && (unsigned)pi < (unsigned)p.max_pos;
        dt.kpi[u] = ok ? pi : -1;
        // an unusable block reads the zero page; unusable keys of a usable
        // block are masked (scores) and zeroed (V) downstream
        const uint16_t *kbase = bok ? p.k_pool + ((size_t)blk * p.hkv + g) * (kBlock * D) : p.zero_page;
        const uint32_t off = (uint32_t)(row * D + 8 * pc);
        if constexpr (ZERO) {
            constexpr int kBytes = kBlock * D * 2;   // one (block, kv head) of K
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(kbase), (short)0, kBytes, kRsrcWord3);
            const int bo = ok ? (int)(2 * off) : 2 * kBytes;
            dt.klo[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, bo, 0, 0));
            dt.khi[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, bo + GG::HALF * 2, 0, 0));
        } else {
            dt.klo[u] = *reinterpret_cast<const u32x4 *>(kbase + off);
            dt.khi[u] = *reinterpret_cast<const u32x4 *>(kbase + off + GG::HALF);
        }
    }
    if (!need_v) return;
    int half, dd;
    vmap(tid, half, dd);
    const int jb = tile + 16 * (wave & 3);
    const int vblk = __builtin_amdgcn_readfirstlane(m.vblk);
    const bool bok = jb < key_end && (unsigned)vblk < (unsigned)p.num_blocks;
    // validity of the block's 16 keys: lanes 0..15 hold their pi; the ballot
    // lands in scalar registers
    const bool kv_ok = jb + (lane & 15) < key_end && (unsigned)m.vkey_pi < (unsigned)p.max_pos;
    const uint32_t okmask = (uint32_t)__ballot(kv_ok) & 0xffffu;
    dt.vmask = bok ? (int32_t)((~okmask >> (8 * half)) & 0xffu) : 0xff;
    const uint16_t *vb = bok ? p.v_pool + ((size_t)vblk * p.hkv + g) * (D * kBlock) : p.zero_page;
#pragma unroll
    for (int u = 0; u < GG::VCH; ++u) {
        const int d = dd + 32 * ((tid >> 8) + u * (GG::NT / 256));
        dt.v[u] = *reinterpret_cast<const u32x4 *>(vb + (uint32_t)(d * kBlock + 8 * half));
    }
}

// cos/sin rows of the staged keys (row 0 for unusable keys, whose data is 0).
template <int D, int WAVES, bool ROT>
__device__ __forceinline__ void cs_load(const FwdParams &p, Data<D, WAVES> &dt, int tid) {
    using GG = Geo<D, WAVES>;
    if constexpr (!ROT) return;   // keys stored rotated: no table rows
#pragma unroll
    for (int u = 0; u < GG::KTASK; ++u) {
        const int pc = tid % GG::PC;
        const int pi = dt.kpi[u];
        const uint32_t off = (uint32_t)((pi >= 0 ? pi : 0) * GG::HALF + 8 * pc);
        dt.cs[u][0] = *reinterpret_cast<const f32x4 *>(p.cos_tab + off);
        dt.cs[u][1] = *reinterpret_cast<const f32x4 *>(p.cos_tab + off + 4);
        dt.cs[u][2] = *reinterpret_cast<const f32x4 *>(p.sin_tab + off);
        dt.cs[u][3] = *reinterpret_cast<const f32x4 *>(p.sin_tab + off + 4);
    }
}

// Positions and block ids of the first two steps of first_bad_key, requested
// before the workgroup's earliest position is known.
struct FbPre {
    i32x4 pi[2];
    int32_t blk[2];
};

// Steps past the range read index 0 (every request row has a first block);
// those values are not used.
template <int NT>
__device__ __forceinline__ FbPre fb_preload(const int32_t *bt, const int32_t *pis, int key_begin, int key_end,
                                            int tid) {
    FbPre f;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int j0 = key_begin + 4 * tid + 4 * NT * s;
        const int jc = j0 < key_end ? j0 : 0;
        f.pi[s] = *reinterpret_cast<const i32x4 *>(pis + jc);
        f.blk[s] = bt[jc >> 4];
    }
    return f;
}

// First key of [key_begin, key_end) that needs the per-score mask (INT_MAX
// if none), and with last_bad the last such key (-1 if none).  With KEYBIAS
// only a usable key that the row with the smallest position does not see
// needs it (unusable keys are then cut by their score bias); otherwise also
// every unusable key.  Four keys per thread and step with no early exit, so
// the loads of all steps can be in flight at once.
// key_begin is a multiple of 64 and kv_stride of 16, so each 4-key load is
// aligned and stays inside the request's position row.  With s_need, also
// sets bit t of s_need for every 64-key tile t holding a usable key that the
// row with the largest position (max_row) sees.
// The first two steps use the rows preloaded by fb_preload.
template <int NT, bool KEYBIAS>
__device__ __forceinline__ int first_bad_key(const FwdParams &p, const int32_t *bt, const int32_t *pis,
                                             const FbPre &pre, int key_begin, int key_end, int min_pos, int tid,
                                             int *last_bad = nullptr, int max_row = -1,
                                             uint32_t *s_need = nullptr) {
    int bad = 0x7fffffff, last = -1;
    auto step = [&](int j0, const i32x4 pi, int blk) {
        const bool bok = blk >= 0 && blk < p.num_blocks;
        bool need = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool usable = j0 + i < key_end && bok && pi[i] >= 0 && pi[i] < p.max_pos;
            const bool b = KEYBIAS ? usable && pi[i] > min_pos : j0 + i < key_end && !(usable && pi[i] <= min_pos);
            if (b) {
                bad = min(bad, j0 + i);
                last = max(last, j0 + i);
            }
            need = need || (usable && pi[i] <= max_row);
        }
        if (s_need && need) {
            const int t = (j0 - key_begin) >> 6;   // the 4 keys share a tile
            atomicOr(&s_need[t >> 5], 1u << (t & 31));
        }
    };
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int j0 = key_begin + 4 * tid + 4 * NT * s;
        if (j0 < key_end) step(j0, pre.pi[s], pre.blk[s]);
    }
#pragma unroll 4
    for (int j0 = key_begin + 4 * tid + 8 * NT; j0 < key_end; j0 += 4 * NT)
        step(j0, *reinterpret_cast<const i32x4 *>(pis + j0), bt[j0 >> 4]);
    if (last_bad) *last_bad = last;
    return bad;
}

// Rotate and write one tile into an LDS buffer.  With s_bias, also writes
// each key's score bias (0 if usable, -inf if not); with K rows of unusable
// keys loaded as zeros their scores are then exactly -inf without a
// per-score test.  With s_mask, also each key's weight in the row sums as a
// bf16 1 (usable) or 0.
template <int D, int WAVES, bool ROT>
__device__ __forceinline__ void data_store(Data<D, WAVES> &dt, uint16_t *Ks, uint16_t *Vs, int32_t *s_pi, int tid,
                                           bool need_v, float *s_bias = nullptr, uint16_t *s_mask = nullptr) {
    using GG = Geo<D, WAVES>;
#pragma unroll
    for (int u = 0; u < GG::KTASK; ++u) {
        const int kk = tid / GG::PC + u * (GG::NT / GG::PC);
        const int pc = tid % GG::PC;
        const int pi = dt.kpi[u];
        u32x4 lo = dt.klo[u], hi = dt.khi[u];
        if constexpr (ROT) rope8(lo, hi, dt.cs[u][0], dt.cs[u][1], dt.cs[u][2], dt.cs[u][3]);
        const int kr = krow(kk);
        *reinterpret_cast<u32x4 *>(Ks + koff<D>(kr, pc)) = lo;
        *reinterpret_cast<u32x4 *>(Ks + koff<D>(kr, GG::PC + pc)) = hi;
        // masked-path visibility is one compare: unusable keys get INT_MAX
        if (pc == 0) s_pi[kk] = pi >= 0 ? pi : 0x7fffffff;
        if (s_bias && pc == 0) s_bias[kk] = pi >= 0 ? 0.f : -INFINITY;
        if (s_mask && pc == 0) s_mask[kk] = pi >= 0 ? 0x3f80 : 0;
    }
    if (need_v) {
        int half, dd;
        vmap(tid, half, dd);
        const int b = (tid >> 6) & 3;
        const int vm = dt.vmask;
        // unusable keys are zeroed so that 0 * garbage cannot poison O; the
        // masks are only built when some chunk of the wave needs them
        if (__any(vm != 0)) {
            uint32_t keep[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                keep[e] = ((vm >> (2 * e)) & 1 ? 0u : 0x0000ffffu) | ((vm >> (2 * e + 1)) & 1 ? 0u : 0xffff0000u);
#pragma unroll
            for (int u = 0; u < GG::VCH; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) dt.v[u][e] &= keep[e];
        }
#pragma unroll
        for (int u = 0; u < GG::VCH; ++u) {
            const u32x4 v = dt.v[u];
            const int d = dd + 32 * ((tid >> 8) + u * (GG::NT / 256));
            *reinterpret_cast<u32x4 *>(Vs + voff(d, 2 * b + half)) = v;
        }
    }
}

// SKIP: skip the tiles whose keys no row of the workgroup sees (launched for
// requests with many row blocks, whose positions differ from block to block).
template <int D, int QG, int WAVES, int MODE, bool SKIP, bool ROT>
__global__ __launch_bounds__(64 * WAVES) void fwd_kernel(FwdParams p) {
    using GG = Geo<D, WAVES>;
    constexpr int BM = 16 * QG * WAVES;
    constexpr bool kV = MODE == kAttn;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * GG::KBUF];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[kV ? 2 * GG::VBUF : 8];
    __shared__ __attribute__((aligned(16))) int32_t s_pi[2 * kTileN];
    // score bias of each staged key: 0, or -inf for an unusable key
    __shared__ __attribute__((aligned(16))) float s_bias[2 * kTileN];
    // weight of each staged key in the row sums: bf16 1, or 0 if unusable
    __shared__ __attribute__((aligned(16))) uint16_t s_maskb[2 * kTileN];
    // the QK accumulator start of each query column per row tile, -u (4
    // equal values): the 4 lanes of a column read it before every QK and
    // rewrite it (the same value) when u moves
    __shared__ __attribute__((aligned(16))) f32x4 s_negmu[MODE == kMass ? 1 : WAVES * QG * 16];
    __shared__ float s_red[MODE == kMass ? 2 * WAVES * kTileN : 1];
    __shared__ int32_t s_minpos, s_firstbad, s_lastbad, s_maxpos;
    // bit t: tile t holds a key that some row of the workgroup sees
    __shared__ uint32_t s_need[SKIP ? kNeedWords : 1];

    const int nwg = p.row_blocks * p.hkv * p.num_splits * p.batch;
    int lid = xcd_remap(blockIdx.x, nwg);
    // With tile skipping the row blocks of position-sorted queries see more
    // keys the later they come: dispatch them last first, so that the
    // longest workgroups start at once and the short ones fill the tail.
    const int rb = SKIP ? p.row_blocks - 1 - lid % p.row_blocks : lid % p.row_blocks;
    lid /= p.row_blocks;
    const int g = lid % p.hkv;
    lid /= p.hkv;
    const int sp = lid % p.num_splits;
    const int r = lid / p.num_splits;

    const int kv_stride = p.max_blocks * kBlock;
    const int kv_cap = min(kv_stride, p.max_kv_len);
    const int key_begin = sp * p.split_len;
    const int32_t *bt = p.block_table + (size_t)r * p.max_blocks;
    const int32_t *pis = p.kv_pos + (size_t)r * kv_stride;
    const int tid = threadIdx.x;

    // ---- requests that need nothing loaded go first: block ids and
    // positions of tiles 0 and 1 and of the masking pre-pass, at indices
    // clamped by the split's host-side bound (all inside the request's rows),
    // in the same round trip as kv_len; the true range is applied where the
    // values are used.  Tile 0's K / V / table rows follow them, and the
    // queries' rows follow the queries' positions, so the prologue waits on
    // about two round trips.
    const int key_end_h = min(kv_cap, key_begin + p.split_len);
    Meta<D, WAVES> m1, m2;
    Data<D, WAVES> dnext;
    if (key_end_h > key_begin) {
        meta_load<D, WAVES>(m1, bt, pis, key_begin, key_end_h, tid);
        meta_load<D, WAVES>(m2, bt, pis, key_begin + kTileN, key_end_h, tid);
    }
    const FbPre fb = fb_preload<GG::NT>(bt, pis, key_begin, key_end_h, tid);

    const int q0 = p.q_start[r];
    const int nq = p.q_start[r + 1] - q0;
    const int nrows = nq * p.group;
    if (rb * BM >= nrows) return;
    int kvl = p.kv_len[r];
    kvl = kvl < 0 ? 0 : (kvl > kv_cap ? kv_cap : kvl);
    const int key_end = min(kvl, key_begin + p.split_len);

    const int wave = tid >> 6, lane = tid & 63;
    const int lc = lane & 15, lg = lane >> 4;
    if (tid == 0) {
        s_minpos = 0x7fffffff;
        s_firstbad = 0x7fffffff;
        s_lastbad = -1;
        s_maxpos = -1;
    }
    if constexpr (SKIP)
        for (int w = tid; w < kNeedWords; w += GG::NT) s_need[w] = 0u;
    const int ntiles = key_end > key_begin ? (key_end - key_begin + kTileN - 1) / kTileN : 0;

    // ---- this lane's query columns: load, rotate at q_pos, scale by
    // log2(e)/sqrt(d) in fp32, round to bf16 and keep as B operands: the QK
    // MFMAs then give the scores in log2 units
    const float sc = p.scale_log2;
    u32x4 qop[QG][GG::NC];
    int qpos[QG], qt[QG], qh[QG];
    bool qvalid[QG];
    int my_min = 0x7fffffff, my_max = -1;
    // query token and head of this lane's column in row tile qg (recomputed
    // for the epilogue rather than kept live through the tile loop)
    auto row_of = [&](int qg, int &t, int &h) -> bool {
        const int row = rb * BM + wave * 16 * QG + 16 * qg + lc;
        const bool v = row < nrows;
        t = q0 + (v ? row / p.group : 0);
        h = g * p.group + (v ? row % p.group : 0);
        return v;
    };
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        qvalid[qg] = row_of(qg, qt[qg], qh[qg]);
        int pos = qvalid[qg] ? p.q_pos[qt[qg]] : -1;
        if (pos >= p.max_pos) pos = -1;
        qpos[qg] = pos;
        if (qvalid[qg]) {
            my_min = min(my_min, pos);
            my_max = max(my_max, pos);
        }
    }
    if (ntiles > 0) {
        data_load<D, WAVES, true>(p, dnext, m1, g, key_begin, key_end, tid, kV);
        cs_load<D, WAVES, ROT>(p, dnext, tid);
    }
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        const int pos = qpos[qg];
#pragma unroll
        for (int c = 0; c < GG::NC; ++c) qop[qg][c] = u32x4{0, 0, 0, 0};
        if (pos >= 0) {
            const uint16_t *src = p.q + ((size_t)qt[qg] * p.hq + qh[qg]) * D;
#pragma unroll
            for (int c = 0; c < GG::NC / 2; ++c) {
                const int i0 = 32 * c + 8 * lg;
                u32x4 lo = *reinterpret_cast<const u32x4 *>(src + i0);
                u32x4 hi = *reinterpret_cast<const u32x4 *>(src + GG::HALF + i0);
                const float *cr = p.cos_tab + (size_t)pos * GG::HALF + i0;
                const float *sr = p.sin_tab + (size_t)pos * GG::HALF + i0;
                rope8(lo, hi, *reinterpret_cast<const f32x4 *>(cr), *reinterpret_cast<const f32x4 *>(cr + 4),
                      *reinterpret_cast<const f32x4 *>(sr), *reinterpret_cast<const f32x4 *>(sr + 4), sc);
                qop[qg][c] = lo;
                qop[qg][c + GG::NC / 2] = hi;
            }
        }
    }

    // Running max in log2 units: a finite -1e30 until the column has seen a
    // usable key.
    float m_run[QG], lse2[QG];
    f32x4 acc[kV ? QG : 1][kV ? D / 16 : 1];
    // Row sums of P on the MFMA pipe: A = 16 x 32 whose every row holds the
    // keys' weights (1, or 0 for an unusable key), so each row of acc_l[qg]
    // accumulates sum_k w_k P^T[k][col].
    f32x4 acc_l[MODE == kMass ? 1 : QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        m_run[qg] = -1e30f;
        if constexpr (MODE != kMass) acc_l[qg] = f32x4{0.f, 0.f, 0.f, 0.f};
        lse2[qg] = INFINITY;
        if constexpr (MODE == kMass) {
            if (qpos[qg] >= 0) {
                const float ls = p.lse_in[(size_t)qt[qg] * p.hq + qh[qg]];
                // -inf (nothing visible), +inf or NaN: contribute nothing
                lse2[qg] = finite_bits(ls) ? ls * 1.4426950408889634f : INFINITY;
            }
        }
    }
    if constexpr (kV) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) acc[qg][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    __syncthreads();
    atomicMin(&s_minpos, my_min);
    if constexpr (SKIP) atomicMax(&s_maxpos, my_max);
    // Staging pipeline: the data of tile t+2 (and the block ids of t+3) are
    // requested next to the QK of tile t+1, about a tile before they are
    // rotated and stored; indices past the range are clamped and such keys
    // read the zero page, so the requests need no branch.  Tiles 0 and 1 are
    // requested before it is known which tiles the rows need.
    __syncthreads();
    const int min_pos = s_minpos;
    // Tiles with no key that any row sees are skipped (not in mass mode, which
    // writes every key's partial sum); so is every tile when too many for the
    // bit mask.
    const bool skip = SKIP && MODE != kMass && ntiles <= kNeedWords * 32;
    // First and last key of this workgroup's range that some row does not see
    // although it is usable (pi and block ids are small and L2-resident):
    // tiles outside that range need no per-score mask.
    {
        int last = -1;
        const int bad = SKIP ? first_bad_key<GG::NT, true>(p, bt, pis, fb, key_begin, key_end, min_pos, tid, &last,
                                                           s_maxpos, skip ? s_need : nullptr)
                             : first_bad_key<GG::NT, true>(p, bt, pis, fb, key_begin, key_end, min_pos, tid, &last);
        if (bad != 0x7fffffff) {
            atomicMin(&s_firstbad, bad);
            atomicMax(&s_lastbad, last);
        }
    }
    __syncthreads();
    const int first_bad = s_firstbad, last_bad = s_lastbad;
    // Whether the rows need every tile (the usual case): then the tile order
    // is plain, with no look-up in the mask.  Each wave checks the whole mask.
    bool every = !skip;
    if (SKIP && skip) {
        bool miss = false;
        for (int w = lane; w < kNeedWords; w += 64) {
            const int lo = 32 * w, n = min(max(ntiles - lo, 0), 32);
            const uint32_t want = n == 32 ? 0xffffffffu : ((1u << n) - 1u);
            miss = miss || (s_need[w] & want) != want;
        }
        every = !__any(miss);
    }
    // next needed tile after i (ntiles if none)
    auto next_tile = [&](int i) -> int {
        if (every) return min(i + 1, ntiles);
        for (int t = i + 1; t < ntiles; t = (t | 31) + 1) {
            const uint32_t w = __builtin_amdgcn_readfirstlane(s_need[t >> 5]) >> (t & 31);
            if (w) return min(t + __builtin_ctz(w), ntiles);
        }
        return ntiles;
    };
    const int it0 = SKIP ? next_tile(-1) : 0, it1 = SKIP ? next_tile(it0) : 1, it2 = SKIP ? next_tile(it1) : 2;
    if (SKIP && it0 < ntiles && (it0 != 0 || it1 != 1)) {
        // the rows skip tile 0 or 1: request the first two tiles they need
        meta_load<D, WAVES>(m1, bt, pis, key_begin + it0 * kTileN, key_end, tid);
        meta_load<D, WAVES>(m2, bt, pis, key_begin + it1 * kTileN, key_end, tid);
        data_load<D, WAVES, true>(p, dnext, m1, g, key_begin + it0 * kTileN, key_end, tid, kV);
        cs_load<D, WAVES, ROT>(p, dnext, tid);
    }
    if (SKIP ? it0 < ntiles : ntiles > 0) {
        data_store<D, WAVES, ROT>(dnext, Ks, Vs, s_pi, tid, kV, s_bias, s_maskb);
        __syncthreads();
    }
    // The softmax reference of each column: m_ref, the max the accumulators
    // are in (-1e30 until a usable key is seen).  The QK accumulators start
    // at -u (negmu), u = m_ref once set, else 0, so every score arrives as
    // s' = s - u and P = exp2(s') needs no VALU op before the exp.  An
    // unusable key (K row zero) then scores exactly -u: its P is finite while
    // -u <= the slack and it is weighted 0 in the row sums (V row zero);
    // a larger -u trips the reference check, whose rare path adds the key
    // bias (-inf) before forming P.  thr: the check's threshold on the
    // half's lane max, the slack once set, else -FLT_MAX (any visible key).
    float m_ref[QG], thr[QG];
    f32x4 *negmu = s_negmu + (MODE == kMass ? 0 : wave * QG * 16 + lc);   // row tile qg at [16 qg]
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        m_ref[qg] = m_run[qg];
        thr[qg] = -FLT_MAX;
        if constexpr (MODE != kMass) negmu[16 * qg] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- software pipeline over 32-key halves.  Per tile:
    //   R1  QK(half 1)            || softmax(half 0)
    //   R2  PV(half 0)            || softmax(half 1)
    //   R3  PV(half 1)            || rotate + stage the next tile
    //   --  barrier
    //   R4  QK(next tile, half 0)
    // Every softmax uses the reference the accumulators are in; when a
    // half's max passes it by more than 2^8 (rare after the first keys), the
    // reference moves, the accumulators follow before that half's PV, and the
    // half's scores (and those of the other half in flight) are shifted and
    // its P is formed again.
    // buf: LDS buffer of the tile.  The accumulators start at -u of their
    // column (attention, LSE) or at the keys' score bias (mass: -inf cuts an
    // unusable key, whose K row is zero).
    auto qk_half = [&](int buf, int kh, f32x4 (&sacc)[QG][2]) {
        const uint16_t *Kb = Ks + buf * GG::KBUF;
        // sacc[.][T][i] holds key 32 kh + 8 lg + 4 T + i
        f32x4 b0, b1, nm[QG];
        if constexpr (MODE == kMass) {
            const float *bb = s_bias + buf * kTileN + 32 * kh + 8 * lg;
            b0 = *reinterpret_cast<const f32x4 *>(bb);
            b1 = *reinterpret_cast<const f32x4 *>(bb + 4);
        } else {
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) nm[qg] = negmu[16 * qg];
        }
        // d-chunk outermost: 2*QG independent accumulators separate the
        // dependent MFMAs of one accumulator chain
        // rows 32*kh + 16*T + lc (T = 0, 1), chunk 4c + lg: the XOR stays
        // inside lc, so the row offset is an immediate
#pragma unroll
        for (int c = 0; c < GG::NC; ++c) {
            const int ch = 4 * c + lg;
            const uint16_t *k0 = Kb + ch * (kTileN * 8) + ((lc ^ kxor<D>(ch)) * 8) + (32 * kh) * 8;
            const u32x4 a0 = *reinterpret_cast<const u32x4 *>(k0);
            const u32x4 a1 = *reinterpret_cast<const u32x4 *>(k0 + 16 * 8);
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
                if constexpr (MODE == kMass) {
                    sacc[qg][0] = mfma16(a0, qop[qg][c], c == 0 ? b0 : sacc[qg][0]);
                    sacc[qg][1] = mfma16(a1, qop[qg][c], c == 0 ? b1 : sacc[qg][1]);
                } else {
                    sacc[qg][0] = mfma16(a0, qop[qg][c], c == 0 ? nm[qg] : sacc[qg][0]);
                    sacc[qg][1] = mfma16(a1, qop[qg][c], c == 0 ? nm[qg] : sacc[qg][1]);
                }
            }
        }
    };
    // Scores of one half (log2 units) -> masked exp2 -> bf16 P^T operands
    // (attn / lse) or column sums (mass).  Returns the lane maxima of the
    // shifted scores in mx.
    auto softmax_half = [&](auto full_c, const f32x4 (&sacc)[QG][2], const int32_t *pib, int kh,
                            u32x4 (&pb)[QG], float (&mx)[QG], float (&cs)[16]) {
        constexpr bool FULL = decltype(full_c)::value;
        int kp[8];
        if constexpr (!FULL) {
            const i32x4 a = *reinterpret_cast<const i32x4 *>(pib + 32 * kh + 8 * lg);
            const i32x4 b = *reinterpret_cast<const i32x4 *>(pib + 32 * kh + 8 * lg + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kp[i] = a[i];
                kp[4 + i] = b[i];
            }
        }
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
            float s[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] = sacc[qg][e >> 2][e & 3];
            if constexpr (!FULL) {
#pragma unroll
                for (int e = 0; e < 8; ++e) s[e] = kp[e] <= qpos[qg] ? s[e] : -INFINITY;
            }
            if constexpr (MODE == kMass) {
#pragma unroll
                for (int e = 0; e < 8; ++e) cs[kh * 8 + e] += fast_exp2(s[e] - lse2[qg]);
            } else {
                u32x4 pq;
#pragma unroll
                for (int e = 0; e < 4; ++e) pq[e] = pack2(fast_exp2(s[2 * e]), fast_exp2(s[2 * e + 1]));
                pb[qg] = pq;
                // lane-local maximum of the shifted scores; the column
                // maximum is only formed when some lane passes the check
                mx[qg] = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
            }
        }
    };
    auto pv_half = [&](const uint16_t *Vb, const uint16_t *mb, int kh, const u32x4 (&pb)[QG]) {
        if constexpr (MODE != kMass) {
            // the weights of keys 32 kh + 8 lg + e: the A operand of every row
            const u32x4 w = *reinterpret_cast<const u32x4 *>(mb + 32 * kh + 8 * lg);
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) acc_l[qg] = mfma16(w, pb[qg], acc_l[qg]);
        }
        if constexpr (kV) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                const int ch = 4 * kh + lg;
                const u32x4 a = *reinterpret_cast<const u32x4 *>(
                    Vb + (dt >> 2) * (64 * kTileN) + ch * (64 * 8) + (lc ^ ch) * 8 + (dt & 3) * 16 * 8);
#pragma unroll
                for (int qg = 0; qg < QG; ++qg) acc[qg][dt] = mfma16(a, pb[qg], acc[qg][dt]);
            }
        }
    };
    // Bring the accumulators from reference `from` to `to` (per lane).
    auto rescale = [&](int qg, float from, float to) {
        const float alpha = fast_exp2(from - to);
        acc_l[qg] *= alpha;
        if constexpr (kV) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) acc[qg][dt] *= alpha;
        }
    };
    // After a half whose lane maxima of the shifted scores are mx: only when
    // some lane passes thr (wave-uniform branch, rare once the first keys are
    // seen) are the column maxima formed.  In a mask-free tile the scores
    // first take the key bias, so that unusable keys count nowhere.  Columns
    // whose maximum passed move their reference there; the accumulators
    // follow at once (nothing of this half is in them yet), this half's
    // scores and, with SHIFT_OTHER, those of the other half already issued
    // are shifted to the new reference, and the half's P is formed again.
    // The common path is one compare per column and no branch target inside
    // the MFMA / VALU regions.
    auto settle = [&](auto full_c, auto shift_other_c, f32x4 (&sacc)[QG][2], f32x4 (&other)[QG][2],
                      const int32_t *pib, const float *bb, int kh, u32x4 (&pb)[QG], const float (&mx)[QG],
                      float (&cs)[16]) {
        constexpr bool FULL = decltype(full_c)::value;
        bool need = false;
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) need = need || mx[qg] > thr[qg];
        if (__builtin_expect(__any(need), 0)) {
            float lm[QG];
            if constexpr (FULL) {
                const f32x4 b0 = *reinterpret_cast<const f32x4 *>(bb + 32 * kh + 8 * lg);
                const f32x4 b1 = *reinterpret_cast<const f32x4 *>(bb + 32 * kh + 8 * lg + 4);
#pragma unroll
                for (int qg = 0; qg < QG; ++qg) {
                    sacc[qg][0] += b0;
                    sacc[qg][1] += b1;
                    float m = sacc[qg][0][0];
#pragma unroll
                    for (int e = 1; e < 8; ++e) m = fmaxf(m, sacc[qg][e >> 2][e & 3]);
                    lm[qg] = m;
                }
            } else {
#pragma unroll
                for (int qg = 0; qg < QG; ++qg) lm[qg] = mx[qg];
            }
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
                const float cm = col_max(lm[qg]);
                const bool was = thr[qg] > 0.f;
                const bool move = cm > thr[qg];
                const float u = was ? m_ref[qg] : 0.f;
                const float m_new = move ? u + cm : m_ref[qg];
                // before a column has seen a usable key its accumulators are
                // zero and exp2(-1e30 - m_new) = 0 keeps them so
                rescale(qg, m_ref[qg], m_new);
                const bool now = was || move;
                const float un = now ? m_new : 0.f;
                const float delta = un - u;
                m_ref[qg] = m_new;
                thr[qg] = now ? kRescaleSlack : -FLT_MAX;
                negmu[16 * qg] = f32x4{-un, -un, -un, -un};
                sacc[qg][0] -= delta;
                sacc[qg][1] -= delta;
                if constexpr (decltype(shift_other_c)::value) {
                    other[qg][0] -= delta;
                    other[qg][1] -= delta;
                }
            }
            float mx2[QG];
            softmax_half(full_c, sacc, pib, kh, pb, mx2, cs);
        }
    };

    f32x4 sA[QG][2], sB[QG][2];
    if (SKIP ? it0 < ntiles : ntiles > 0) {
        qk_half(0, 0, sA);
        data_load<D, WAVES, true>(p, dnext, m2, g, key_begin + it1 * kTileN, key_end, tid, kV);
        meta_load<D, WAVES>(m2, bt, pis, key_begin + it2 * kTileN, key_end, tid);
    }

    // One tile: the k-th processed, tile index it; n1, n2, n3 the next three
    // needed tiles.  MORE: n1 exists (stage it), FULL: no per-score mask
    // (every usable key is visible to every row).
    // Each region is straight-line code so the MFMA / VALU interleave hints
    // apply to it.
    auto tile_body = [&](auto more_c, auto full_c, int k, int it, int n1, int n2, int n3) {
        constexpr bool MORE = decltype(more_c)::value;
        const int cur = (SKIP ? k : it) & 1;
        const int tile = key_begin + it * kTileN;
        const uint16_t *Vc = Vs + (kV ? cur * GG::VBUF : 0);
        const int32_t *pc_ = s_pi + cur * kTileN;
        const float *bc = s_bias + cur * kTileN;
        const uint16_t *mc = s_maskb + cur * kTileN;
        u32x4 pb0[QG], pb1[QG];
        float mx0[QG], mx1[QG];
        float cs[16];   // kMass: column sums of this lane's 16 keys
#pragma unroll
        for (int u = 0; u < 16; ++u) cs[u] = 0.f;

        // R1: QK(half 1) || softmax(half 0)
        qk_half(cur, 1, sB);
        softmax_half(full_c, sA, pc_, 0, pb0, mx0, cs);
        interleave_hint<2 * QG * GG::NC, 4>();
        if constexpr (MODE != kMass) settle(full_c, std::true_type{}, sA, sB, pc_, bc, 0, pb0, mx0, cs);

        // R2: PV(half 0) || softmax(half 1)
        pv_half(Vc, mc, 0, pb0);
        if constexpr (MORE) cs_load<D, WAVES, ROT>(p, dnext, tid);
        softmax_half(full_c, sB, pc_, 1, pb1, mx1, cs);
        if constexpr (MODE != kMass) {
            interleave_hint<QG * (D / 16 + 1), 4>();
            settle(full_c, std::false_type{}, sB, sB, pc_, bc, 1, pb1, mx1, cs);
        }

        // R3: PV(half 1) || rotate + stage the next tile
        pv_half(Vc, mc, 1, pb1);
        if constexpr (MODE == kMass) {
            // Sum the 16 columns of the lane group: butterfly reduce-scatter,
            // afterwards lane lc holds the total of value index u = lc.
#pragma unroll
            for (int off = 8, n = 8; off >= 1; off >>= 1, n >>= 1) {
                const bool upper = (lc & off) != 0;
#pragma unroll
                for (int e = 0; e < n; ++e) {
                    const float send = upper ? cs[e] : cs[e + n];
                    const float keep = upper ? cs[e + n] : cs[e];
                    cs[e] = keep + __shfl_xor(send, off);
                }
            }
            const int key = 32 * (lc >> 3) + 8 * lg + 4 * ((lc >> 2) & 1) + (lc & 3);
            s_red[(cur * WAVES + wave) * kTileN + key] = cs[0];
        }
        if constexpr (MORE)
            data_store<D, WAVES, ROT>(dnext, Ks + (cur ^ 1) * GG::KBUF, Vs + (kV ? (cur ^ 1) * GG::VBUF : 0),
                                      s_pi + (cur ^ 1) * kTileN, tid, kV, s_bias + (cur ^ 1) * kTileN,
                                      s_maskb + (cur ^ 1) * kTileN);
        if constexpr (MODE != kMass) interleave_hint<QG * (D / 16 + 1), 3>();
        __syncthreads();

        if constexpr (MODE == kMass) {
            if (tid < kTileN) {
                const float *sr = s_red + cur * WAVES * kTileN;
                float tot = 0.f;
#pragma unroll
                for (int w = 0; w < WAVES; ++w) tot += sr[w * kTileN + tid];
                const int j = tile + tid;
                if (j < key_end)
                    p.mass_part[(((size_t)r * p.hkv + g) * p.row_blocks + rb) * p.mass_stride + j] = tot;
            }
        }
        // R4: request the tile after the next one || QK(next tile, half 0).
        // The requests go first: they fill the wait for the K operands that
        // every wave reads from LDS right after the barrier.
        if constexpr (MORE) {
            data_load<D, WAVES, true>(p, dnext, m2, g, SKIP ? key_begin + n2 * kTileN : tile + 2 * kTileN, key_end, tid,
                                kV);
            meta_load<D, WAVES>(m2, bt, pis, SKIP ? key_begin + n3 * kTileN : tile + 3 * kTileN, key_end, tid);
            qk_half(cur ^ 1, 0, sA);
        }
        (void)n1;
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    // Tiles [t1, t2) hold the usable keys some row does not see and run
    // masked; the rest run mask-free (before that range: the shared context,
    // after it: rows appended behind the query block, such as fused rows).
    // Each loop keeps its own register allocation; the outer loops run at
    // most twice.
    const int t1 = first_bad == 0x7fffffff ? ntiles : (first_bad - key_begin) / kTileN;
    const int t2 = last_bad < 0 ? ntiles : (last_bad - key_begin) / kTileN + 1;
    auto full_tile = [&](int i) { return i < t1 || i >= t2; };
    if constexpr (SKIP) {
        // the needed tiles in order: (it, n1, n2) advance together
        int k = 0, it = it0, n1 = it1, n2 = it2;
        for (; n1 < ntiles && full_tile(it); ++k) {
            const int n3 = next_tile(n2);
            tile_body(T_{}, T_{}, k, it, n1, n2, n3);
            it = n1, n1 = n2, n2 = n3;
        }
        for (; n1 < ntiles && !full_tile(it); ++k) {
            const int n3 = next_tile(n2);
            tile_body(T_{}, F_{}, k, it, n1, n2, n3);
            it = n1, n1 = n2, n2 = n3;
        }
        for (; n1 < ntiles; ++k) {
            const int n3 = next_tile(n2);
            tile_body(T_{}, T_{}, k, it, n1, n2, n3);
            it = n1, n1 = n2, n2 = n3;
        }
        if (it < ntiles) {
            if (full_tile(it)) tile_body(F_{}, T_{}, k, it, ntiles, ntiles, ntiles);
            else tile_body(F_{}, F_{}, k, it, ntiles, ntiles, ntiles);
        }
    } else {
        const int nl = ntiles - 1;   // tiles with a successor to stage
        int it = 0;
        for (; it < nl && full_tile(it); ++it) tile_body(T_{}, T_{}, it, it, 0, 0, 0);
        for (; it < nl && !full_tile(it); ++it) tile_body(T_{}, F_{}, it, it, 0, 0, 0);
        for (; it < nl; ++it) tile_body(T_{}, T_{}, it, it, 0, 0, 0);
        if (ntiles > 0) {
            if (full_tile(nl)) tile_body(F_{}, T_{}, nl, nl, 0, 0, 0);
            else tile_body(F_{}, F_{}, nl, nl, 0, 0, 0);
        }
    }
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) m_run[qg] = m_ref[qg];
    if constexpr (MODE == kMass) return;

    // ---- epilogue: per-lane partial sums -> column totals
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        // rows 0, 4, 8 and 12 (element 0 of the four lane groups) each hold
        // the row sum: their total is exactly 4 times it
        const float lt = col_sum(acc_l[qg][0]) * 0.25f;
        int t, h;
        if (!row_of(qg, t, h)) continue;
        const size_t rowid = (size_t)t * p.hq + h;
        if (p.num_splits == 1) {
            const bool any = lt > 0.f;
            if constexpr (kV) {
                const float inv = any ? 1.f / lt : 0.f;
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt) {
                    const f32x4 o = acc[qg][dt] * inv;
                    uint2 w;
                    w.x = pack2(o[0], o[1]);
                    w.y = pack2(o[2], o[3]);
                    *reinterpret_cast<uint2 *>(p.out + rowid * D + 16 * dt + 4 * lg) = w;
                }
            }
            if (p.lse && lg == 0)
                p.lse[rowid] = any ? (m_run[qg] + __log2f(lt)) * 0.6931471805599453f : -INFINITY;
        } else {
            const size_t prow = (size_t)sp * p.total_q * p.hq + rowid;
            if constexpr (kV) {
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt)
                    *reinterpret_cast<f32x4 *>(p.part_o + prow * D + 16 * dt + 4 * lg) = acc[qg][dt];
            }
            if (lg == 0) {
                p.part_ml[prow * 2 + 0] = lt > 0.f ? m_run[qg] : -INFINITY;
                p.part_ml[prow * 2 + 1] = lt;
            }
        }
    }
}

// Selection mass (QCFuse, gist.science 2604.08585, methodology B): for
// every key j of the workgroup's range, sum over its query rows of
// p = exp(s - lse), written per row block to mass_part.
//
// Unlike the attention pipeline the scores are computed untransposed,
// S = Q K^T (the same operand registers with A and B swapped), so a lane holds
// 4 query rows x 1 key per 16 x 16 MFMA tile.  The 8 probabilities of a lane
// over the wave's two row tiles are then exactly its slice of a 32 (rows) x
// 16 (keys) B operand, and the sum over the 32 rows runs on the MFMA pipe
// against an A operand whose row 0 is ones: no cross-lane reduction.  The
// staging (tile loads two ahead, rotation, LDS double buffer) is the
// attention kernel's.
template <int D, int QG, int WAVES, bool ROT>
__global__ __launch_bounds__(64 * WAVES) void mass_kernel(FwdParams p) {
    static_assert(QG % 2 == 0, "the 32-row MFMA column sum packs pairs of row tiles");
    using GG = Geo<D, WAVES>;
    constexpr int BM = 16 * QG * WAVES;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * GG::KBUF];
    __shared__ __attribute__((aligned(16))) int32_t s_pi[2 * kTileN];
    __shared__ float s_red[2][WAVES][kTileN];
    __shared__ int32_t s_minpos, s_firstbad;
    uint16_t *const Vs = nullptr;   // no V in this pass

    const int nwg = p.row_blocks * p.hkv * p.num_splits * p.batch;
    int lid = xcd_remap(blockIdx.x, nwg);
    const int rb = lid % p.row_blocks;
    lid /= p.row_blocks;
    const int g = lid % p.hkv;
    lid /= p.hkv;
    const int sp = lid % p.num_splits;
    const int r = lid / p.num_splits;

    const int kv_stride = p.max_blocks * kBlock;
    const int kv_cap = min(kv_stride, p.max_kv_len);
    const int key_begin = sp * p.split_len;
    const int32_t *bt = p.block_table + (size_t)r * p.max_blocks;
    const int32_t *pis = p.kv_pos + (size_t)r * kv_stride;
    const int tid = threadIdx.x;

    // ---- requests that need nothing loaded first, clamped by the split's
    // host-side bound (as in fwd_kernel)
    const int key_end_h = min(kv_cap, key_begin + p.split_len);
    Meta<D, WAVES> m1, m2;
    Data<D, WAVES> dnext;
    if (key_end_h > key_begin) {
        meta_load<D, WAVES>(m1, bt, pis, key_begin, key_end_h, tid);
        meta_load<D, WAVES>(m2, bt, pis, key_begin + kTileN, key_end_h, tid);
    }
    const FbPre fb = fb_preload<GG::NT>(bt, pis, key_begin, key_end_h, tid);

    const int q0 = p.q_start[r];
    const int nq = p.q_start[r + 1] - q0;
    const int nrows = nq * p.group;
    if (rb * BM >= nrows) return;
    int kvl = p.kv_len[r];
    kvl = kvl < 0 ? 0 : (kvl > kv_cap ? kv_cap : kvl);
    const int key_end = min(kvl, key_begin + p.split_len);

    const int wave = tid >> 6, lane = tid & 63;
    const int lc = lane & 15, lg = lane >> 4;
    if (tid == 0) {
        s_minpos = 0x7fffffff;
        s_firstbad = 0x7fffffff;
    }
    const int row0 = rb * BM + wave * 16 * QG;   // first row of this wave
    const int ntiles = key_end > key_begin ? (key_end - key_begin + kTileN - 1) / kTileN : 0;

    // ---- A operands: query row lc of each row tile, rotated at its q_pos
    u32x4 qop[QG][GG::NC];
    int qpos[QG], qtk[QG], qhd[QG];
    int my_min = 0x7fffffff;
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        const int row = row0 + 16 * qg + lc;
        const bool valid = row < nrows;
        qtk[qg] = q0 + (valid ? row / p.group : 0);
        qhd[qg] = g * p.group + (valid ? row % p.group : 0);
        int pos = valid ? p.q_pos[qtk[qg]] : -1;
        if (pos >= p.max_pos) pos = -1;
        if (valid) my_min = min(my_min, pos);
        qpos[qg] = pos;
    }
    // ---- the rows this lane's scores belong to: 4*lg + i of each row tile.
    // Rows past the end read the first row's LSE (in range); the value is
    // not used.  Every score accumulator starts at -lse (log2 units) and the
    // queries carry the scale log2(e)/sqrt(d), so an S tile holds exactly the
    // exp2 argument s * scale - lse.
    const float sc = p.scale_log2;
    float lse2[QG][4];
    int rpos[QG][4];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = row0 + 16 * qg + 4 * lg + i;
            const bool valid = row < nrows;
            const int qt = q0 + (valid ? row / p.group : 0);
            const int qh = g * p.group + (valid ? row % p.group : 0);
            int pos = valid ? p.q_pos[qt] : -1;
            const float ls = p.lse_in[(size_t)qt * p.hq + qh];
            if (pos >= p.max_pos) pos = -1;
            rpos[qg][i] = pos;
            // invalid rows, and rows whose lse is not finite (-inf: nothing
            // visible; NaN), contribute exp2(-inf) = 0
            lse2[qg][i] = pos >= 0 && finite_bits(ls) ? ls * 1.4426950408889634f : INFINITY;
        }
    f32x4 s_init[QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) s_init[qg] = f32x4{-lse2[qg][0], -lse2[qg][1], -lse2[qg][2], -lse2[qg][3]};
    if (ntiles > 0) {
        data_load<D, WAVES>(p, dnext, m1, g, key_begin, key_end, tid, false);
        cs_load<D, WAVES, ROT>(p, dnext, tid);
    }
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        const int pos = qpos[qg], qt = qtk[qg], qh = qhd[qg];
#pragma unroll
        for (int c = 0; c < GG::NC; ++c) qop[qg][c] = u32x4{0, 0, 0, 0};
        if (pos >= 0) {
            const uint16_t *src = p.q + ((size_t)qt * p.hq + qh) * D;
#pragma unroll
            for (int c = 0; c < GG::NC / 2; ++c) {
                const int i0 = 32 * c + 8 * lg;
                u32x4 lo = *reinterpret_cast<const u32x4 *>(src + i0);
                u32x4 hi = *reinterpret_cast<const u32x4 *>(src + GG::HALF + i0);
                const float *cr = p.cos_tab + (size_t)pos * GG::HALF + i0;
                const float *sr = p.sin_tab + (size_t)pos * GG::HALF + i0;
                rope8(lo, hi, *reinterpret_cast<const f32x4 *>(cr), *reinterpret_cast<const f32x4 *>(cr + 4),
                      *reinterpret_cast<const f32x4 *>(sr), *reinterpret_cast<const f32x4 *>(sr + 4), sc);
                qop[qg][c] = lo;
                qop[qg][c + GG::NC / 2] = hi;
            }
        }
    }
    const u32x4 ones_a = lc == 0 ? u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u} : u32x4{0, 0, 0, 0};

    __syncthreads();
    atomicMin(&s_minpos, my_min);
    __syncthreads();
    const int min_pos = s_minpos;
    {
        const int bad = first_bad_key<GG::NT, false>(p, bt, pis, fb, key_begin, key_end, min_pos, tid);
        if (bad != 0x7fffffff) atomicMin(&s_firstbad, bad);
    }
    __syncthreads();
    const int first_bad = s_firstbad;
    if (ntiles > 0) {
        data_store<D, WAVES, ROT>(dnext, Ks, Vs, s_pi, tid, false);
        __syncthreads();
        data_load<D, WAVES>(p, dnext, m2, g, key_begin + kTileN, key_end, tid, false);
        meta_load<D, WAVES>(m2, bt, pis, key_begin + 2 * kTileN, key_end, tid);
    }

    // S tile (kh, T): rows 16*qg + 4*lg + i, key column lc = LDS K row
    // 32*kh + 16*T + lc, i.e. key 32*kh + 8*(lc/4) + 4*T + lc%4
    auto qk = [&](const uint16_t *Kb, int kh, f32x4 (&sacc)[QG][2]) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) sacc[qg][0] = sacc[qg][1] = s_init[qg];
#pragma unroll
        for (int c = 0; c < GG::NC; ++c) {
            const int ch = 4 * c + lg;
            const uint16_t *k0 = Kb + ch * (kTileN * 8) + ((lc ^ kxor<D>(ch)) * 8) + (32 * kh) * 8;
            const u32x4 b0 = *reinterpret_cast<const u32x4 *>(k0);
            const u32x4 b1 = *reinterpret_cast<const u32x4 *>(k0 + 16 * 8);
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
                sacc[qg][0] = mfma16(qop[qg][c], b0, sacc[qg][0]);
                sacc[qg][1] = mfma16(qop[qg][c], b1, sacc[qg][1]);
            }
        }
    };
    // probabilities of one half -> column sums of its two 16-key tiles
    auto colsum = [&](auto full_c, const f32x4 (&sacc)[QG][2], const int32_t *pib, int kh, f32x4 (&ds)[2]) {
        constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            int kp = 0;
            if constexpr (!FULL) kp = pib[32 * kh + 8 * (lc >> 2) + 4 * T + (lc & 3)];
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q2 = 0; q2 < QG; q2 += 2) {
                // two row tiles make one 32-row B operand
                u32x4 pb;
#pragma unroll
                for (int qq = 0; qq < 2; ++qq)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int qg = q2 + qq;
                        float pr[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int i = 2 * h2 + e;
                            float x = sacc[qg][T][i];
                            if constexpr (!FULL) x = kp <= rpos[qg][i] ? x : -INFINITY;
                            pr[e] = fast_exp2(x);
                        }
                        pb[2 * qq + h2] = pack2(pr[0], pr[1]);
                    }
                d = mfma16(ones_a, pb, d);
            }
            ds[T] = d;
        }
    };
    auto tile_body = [&](auto more_c, auto full_c, int it) {
        constexpr bool MORE = decltype(more_c)::value;
        const int cur = it & 1;
        const int tile = key_begin + it * kTileN;
        const uint16_t *Kc = Ks + cur * GG::KBUF;
        const int32_t *pc_ = s_pi + cur * kTileN;
        f32x4 sA[QG][2], sB[QG][2], d0[2], d1[2];
        qk(Kc, 0, sA);
        qk(Kc, 1, sB);
        colsum(full_c, sA, pc_, 0, d0);
        if constexpr (MORE) cs_load<D, WAVES, ROT>(p, dnext, tid);
        colsum(full_c, sB, pc_, 1, d1);
        if (lg == 0) {
#pragma unroll
            for (int T = 0; T < 2; ++T) {
                const int key = 8 * (lc >> 2) + 4 * T + (lc & 3);
                s_red[cur][wave][key] = d0[T][0];
                s_red[cur][wave][32 + key] = d1[T][0];
            }
        }
        if constexpr (MORE)
            data_store<D, WAVES, ROT>(dnext, Ks + (cur ^ 1) * GG::KBUF, Vs, s_pi + (cur ^ 1) * kTileN, tid, false);
        __syncthreads();
        if (tid < kTileN) {
            float tot = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) tot += s_red[cur][w][tid];
            const int j = tile + tid;
            if (j < key_end) p.mass_part[(((size_t)r * p.hkv + g) * p.row_blocks + rb) * p.mass_stride + j] = tot;
        }
        if constexpr (MORE) {
            data_load<D, WAVES>(p, dnext, m2, g, tile + 2 * kTileN, key_end, tid, false);
            meta_load<D, WAVES>(m2, bt, pis, tile + 3 * kTileN, key_end, tid);
        }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    const int t_split = first_bad == 0x7fffffff ? ntiles : (first_bad - key_begin) / kTileN;
    const bool last_partial = ntiles > 0 && key_end - (key_begin + (ntiles - 1) * kTileN) < kTileN;
    const int nf = min(t_split, ntiles - 1);
    int it = 0;
    for (; it < nf; ++it) tile_body(T_{}, T_{}, it);
    for (; it < ntiles - 1; ++it) tile_body(T_{}, F_{}, it);
    if (ntiles > 0) {
        if (t_split >= ntiles && !last_partial) tile_body(F_{}, T_{}, ntiles - 1);
        else tile_body(F_{}, F_{}, ntiles - 1);
    }
}

// LSE-weighted merge of split partials.  One thread per (row, 4 channels).
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
    constexpr int TPR = D / 4;   // threads per row
    const int gtid = blockIdx.x * 256 + threadIdx.x;
    const int row = gtid / TPR, part = gtid % TPR;
    if (row >= p.rows) return;
    constexpr int kMax = 16;
    const int S = p.num_splits;
    float M = -INFINITY, L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if (S <= kMax) {
        // the usual case: all of a thread's loads are issued before the sums,
        // which run in split order
        float2 ml[kMax];
        f32x4 po[kMax];
#pragma unroll
        for (int s = 0; s < kMax; ++s) {
            if (s < S) {
                const size_t pr = (size_t)s * p.rows + row;
                ml[s] = *reinterpret_cast<const float2 *>(p.part_ml + pr * 2);
                if (p.part_o) po[s] = *reinterpret_cast<const f32x4 *>(p.part_o + pr * D + 4 * part);
            }
        }
#pragma unroll
        for (int s = 0; s < kMax; ++s)
            if (s < S) M = fmaxf(M, ml[s].x);
        const float Mu = M == -INFINITY ? 0.f : M;
#pragma unroll
        for (int s = 0; s < kMax; ++s) {
            if (s < S) {
                const float w = fast_exp2(ml[s].x - Mu);
                L += w * ml[s].y;
                if (p.part_o) o += w * po[s];
            }
        }
    } else {
        for (int s = 0; s < S; ++s) M = fmaxf(M, p.part_ml[((size_t)s * p.rows + row) * 2]);
        const float Mu = M == -INFINITY ? 0.f : M;
        for (int s = 0; s < S; ++s) {
            const size_t pr = (size_t)s * p.rows + row;
            const float w = fast_exp2(p.part_ml[pr * 2] - Mu);
            L += w * p.part_ml[pr * 2 + 1];
            if (p.part_o) o += w * *reinterpret_cast<const f32x4 *>(p.part_o + pr * D + 4 * part);
        }
    }
    const bool any = L > 0.f;
    if (p.out) {
        const float inv = any ? 1.f / L : 0.f;
        o *= inv;
        uint2 w;
        w.x = pack2(o[0], o[1]);
        w.y = pack2(o[2], o[3]);
        *reinterpret_cast<uint2 *>(p.out + (size_t)row * D + 4 * part) = w;
    }
    if (p.lse && part == 0) p.lse[row] = any ? (M + __log2f(L)) * 0.6931471805599453f : -INFINITY;
}

// LSE-weighted merge for many splits and few rows (decode): one workgroup
// per row; the split maxima / weights are staged in LDS and the splits of
// each channel quad are spread over the workgroup's threads.
template <int D>
__global__ __launch_bounds__(256) void merge_many_kernel(MergeParams p) {
    constexpr int NQ4 = D / 4;             // channel quads per row
    constexpr int NSUB = 256 / NQ4;        // split subsets
    __shared__ float s_w[kMergeMaxSplits];
    __shared__ float s_red[256];
    __shared__ f32x4 s_o[NSUB][NQ4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const int S = p.num_splits;
    float m = -INFINITY;
    for (int s = tid; s < S; s += 256) {
        const float v = p.part_ml[((size_t)s * p.rows + row) * 2];
        s_w[s] = v;
        m = fmaxf(m, v);
    }
    s_red[tid] = m;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (tid < off) s_red[tid] = fmaxf(s_red[tid], s_red[tid + off]);
        __syncthreads();
    }
    const float M = s_red[0];
    const float Mu = M == -INFINITY ? 0.f : M;
    __syncthreads();
    float l = 0.f;
    for (int s = tid; s < S; s += 256) {
        const float w = fast_exp2(s_w[s] - Mu);
        s_w[s] = w;
        l += w * p.part_ml[((size_t)s * p.rows + row) * 2 + 1];
    }
    s_red[tid] = l;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (tid < off) s_red[tid] += s_red[tid + off];
        __syncthreads();
    }
    const float L = s_red[0];
    const bool any = L > 0.f;
    if (p.lse && tid == 0) p.lse[row] = any ? (M + __log2f(L)) * 0.6931471805599453f : -INFINITY;
    if (!p.out || !p.part_o) return;
    const int q4 = tid % NQ4, sub = tid / NQ4;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = sub; s < S; s += NSUB)
        o += s_w[s] * *reinterpret_cast<const f32x4 *>(p.part_o + ((size_t)s * p.rows + row) * D + 4 * q4);
    s_o[sub][q4] = o;
    __syncthreads();
    if (sub != 0) return;
#pragma unroll
    for (int k = 1; k < NSUB; ++k) o += s_o[k][q4];
    const float inv = any ? 1.f / L : 0.f;
    o *= inv;
    uint2 w;
    w.x = pack2(o[0], o[1]);
    w.y = pack2(o[2], o[3]);
    *reinterpret_cast<uint2 *>(p.out + (size_t)row * D + 4 * q4) = w;
}

// ROT: keys are rotated at pi while staged (the method's path); without it
// the pool holds keys already rotated at their positions (ablation mode) and
// no table row is read.  A compile-time choice, so that no branch splits the
// MFMA / VALU regions of the tile loop.
template <int D, int QG, int WAVES, int MODE, bool SKIP>
hipError_t launch_one(const FwdParams &p, hipStream_t s, const KernelEvents &ev) {
    const int nwg = p.row_blocks * p.hkv * p.num_splits * p.batch;
    if (nwg <= 0) return hipSuccess;
    const dim3 grid(nwg), block(64 * WAVES);
    void (*k)(FwdParams);
    if constexpr (MODE == kMass && QG % 2 == 0)
        k = p.rotate_k ? mass_kernel<D, QG, WAVES, true> : mass_kernel<D, QG, WAVES, false>;
    else
        k = p.rotate_k ? fwd_kernel<D, QG, WAVES, MODE, SKIP, true> : fwd_kernel<D, QG, WAVES, MODE, SKIP, false>;
    if (ev.start)
        hipExtLaunchKernelGGL(k, grid, block, 0, s, ev.start, ev.stop, 0, p);
    else
        hipLaunchKernelGGL(k, grid, block, 0, s, p);
    return hipGetLastError();
}

// Variants: shape 0 = (QG 1, 4 waves): 64 rows per workgroup; shape 1 =
// (QG 2, 8 waves): 256 rows at d = 128, (QG 2, 4 waves): 128 rows at d = 64;
// shape 2 = shape 1 that skips tiles no row of the workgroup sees (not in
// mass mode).
template <int D, int MODE>
hipError_t launch_shape(const FwdParams &p, int shape, hipStream_t s, const KernelEvents &ev) {
    constexpr bool S = MODE != kMass;
    if (shape == 0) return launch_one<D, 1, 4, MODE, false>(p, s, ev);
    // the mass pass of larger requests: QG 4 (mass_rows_per_block rows), or
    // QG 2 (shape 3, d = 128: up to 256 rows per kv head)
    if constexpr (MODE == kMass) {
        if constexpr (D == 128) {
            if (shape == 3) return launch_one<D, 2, 8, MODE, false>(p, s, ev);
        }
        return launch_one<D, 4, D == 128 ? 8 : 4, MODE, false>(p, s, ev);
    }
    else {
        // the LSE pass keeps no O accumulator: 4 row tiles per wave (shape 4,
        // d = 128)
        if constexpr (MODE == kLse && D == 128) {
            if (shape == 4) return launch_one<D, 4, 8, MODE, false>(p, s, ev);
        }
        if constexpr (D == 128)
            return shape == 2 ? launch_one<D, 2, 8, MODE, S>(p, s, ev) : launch_one<D, 2, 8, MODE, false>(p, s, ev);
        else
            return shape == 2 ? launch_one<D, 2, 4, MODE, S>(p, s, ev) : launch_one<D, 2, 4, MODE, false>(p, s, ev);
    }
}

template <int D>
hipError_t launch_mode(const FwdParams &p, int mode, int shape, hipStream_t s, const KernelEvents &ev) {
    switch (mode) {
    case kAttn: return launch_shape<D, kAttn>(p, shape, s, ev);
    case kLse: return launch_shape<D, kLse>(p, shape, s, ev);
    default: return launch_shape<D, kMass>(p, shape, s, ev);
    }
}

}  // namespace

int fwd_rows_per_block(int head_dim, int shape) {
    if (shape == 4) return 512;   // the LSE pass with 4 row tiles per wave (d = 128)
    return shape == 0 ? 64 : (head_dim == 128 ? 256 : 128);   // 2 as 1
}
int mass_rows_per_block(int head_dim, int shape) {
    return head_dim == 128 ? (shape == 3 ? 256 : 512) : 256;
}

hipError_t launch_fwd(const FwdParams &p, int head_dim, int mode, int shape, hipStream_t s, KernelEvents ev) {
    return head_dim == 64 ? launch_mode<64>(p, mode, shape, s, ev) : launch_mode<128>(p, mode, shape, s, ev);
}

hipError_t launch_merge(const MergeParams &p, int head_dim, hipStream_t s) {
    if (p.rows <= 0) return hipSuccess;
    if (p.num_splits > 16 && p.num_splits <= kMergeMaxSplits) {
        if (head_dim == 64)
            hipLaunchKernelGGL(merge_many_kernel<64>, dim3(p.rows), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL(merge_many_kernel<128>, dim3(p.rows), dim3(256), 0, s, p);
        return hipGetLastError();
    }
    const int tpr = head_dim / 4;
    const long long threads = (long long)p.rows * tpr;
    const int grid = (int)((threads + 255) / 256);
    if (head_dim == 64)
        hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace pic
