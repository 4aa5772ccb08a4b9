// Query-centric selection and cache fusion for gfx950.
//
//   mass_reduce  sums the per-(kv head, row block) partial column masses that
//                the mass pass writes, in a fixed order (deterministic), into
//                mass[r][j] = sum over the request's query rows of the
//                softmax probability of key j (QCFuse, gist.science
//                2604.08585, methodology B: the query's attention over one
//                layer's K picks the tokens to recompute).
//   span_topk    one workgroup per span: radix select (4 x 8-bit digits of the
//                fp32 bit pattern, which orders non-negative floats) of the
//                k-th largest mass, then an in-order pass that keeps every
//                larger key and the lowest-index keys equal to the threshold;
//                output ascending.
//   fuse_scatter writes recomputed K/V rows bit for bit into the
//                request-private blocks appended after the sequence and
//                rewrites pi (QCFuse "Lo esencial" step 4 / phase 4: recomputed
//                tokens mixed into the stored cache; MiniPIC, gist.science
//                2606.13126, section 2.1: shared blocks are never written).
#include "pic_internal.h"

namespace pic {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mass_reduce_kernel(SelectParams p) {
    const int r = blockIdx.y;
    const int j = blockIdx.x * 256 + threadIdx.x;
    int kvl = p.kv_len[r];
    kvl = kvl < 0 ? 0 : (kvl > p.mass_stride ? p.mass_stride : kvl);
    if (j >= kvl) return;
    const int nrows = (p.q_start[r + 1] - p.q_start[r]) * p.group;
    const int nrb = min(p.row_blocks, (nrows + p.rows_per_block - 1) / p.rows_per_block);
    // partials in (kv head, row block) order, summed in that order; the loads
    // of a group of 16 are all in flight before the first add
    const int n = p.hkv * nrb;
    const float *mp = p.mass_part + (size_t)r * p.hkv * p.row_blocks * p.mass_stride + j;
    auto at = [&](int i) { return mp[((size_t)(i / nrb) * p.row_blocks + i % nrb) * p.mass_stride]; };
    float s = 0.f;
    int i = 0;
    for (; i + 16 <= n; i += 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = at(i + u);
#pragma unroll
        for (int u = 0; u < 16; ++u) s += v[u];
    }
    for (; i < n; ++i) s += at(i);
    p.mass[(size_t)r * p.kv_stride + j] = s;
}

constexpr int kTopkCache = 8;   // keys per thread kept in registers: spans up to 2048 slots

// Per-span top-k of the mass (QCFuse selection): a 4 x 8-bit radix select
// finds the k-th largest key (masses are >= 0, so their float bits order
// like the values), then one in-order pass keeps the keys above it and the
// first of the keys equal to it (ties go to the lower slot index).  Spans of
// up to 2048 slots keep their keys in registers.  Barriers: two per radix
// pass (the histograms are double-buffered and every wave scans all 256 bins
// itself, so no digit is broadcast) and one per 256-key chunk of the output
// pass (each wave publishes its counts of larger and of equal keys, from
// which every thread places its own).
__global__ __launch_bounds__(256) void span_topk_kernel(SelectParams p) {
    __shared__ __attribute__((aligned(16))) int s_hist[2][256];
    __shared__ int s_cnt[2][kWaves][2];   // per chunk parity and wave: keys larger than, equal to the threshold
    const int s = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = p.span_req[s], st = p.span_start[s], L = p.span_len[s];
    const int k = p.sel_off[s + 1] - p.sel_off[s];
    int32_t *out = p.sel_idx + p.sel_off[s];
    if (r < 0 || r >= p.batch || k <= 0) return;
    const int32_t *pis = p.kv_pos + (size_t)r * p.kv_stride;
    const float *mass = p.mass + (size_t)r * p.kv_stride;
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;   // the lanes under this one
    // A span that fits in registers requests its slots (clamped into the
    // request's row) beside the request's length, not after it.
    const int lo = max(st, 0), hi_span = min(st + max(L, 0), p.kv_stride);
    const bool cached = hi_span - lo <= 256 * kTopkCache;
    int32_t cpi[kTopkCache];
    uint32_t cms[kTopkCache];
    if (cached) {
#pragma unroll
        for (int u = 0; u < kTopkCache; ++u) {
            const int jc = min(lo + 256 * u + tid, max(hi_span - 1, 0));   // in the row for any u
            cpi[u] = pis[jc];
            cms[u] = __float_as_uint(mass[jc]);
        }
    }
    int kvl = p.kv_len[r];
    kvl = kvl < 0 ? 0 : (kvl > p.kv_stride ? p.kv_stride : kvl);
    const int hi = min(hi_span, kvl);

    uint32_t ck[kTopkCache];
    bool cc[kTopkCache];
    // visit(j, key, is_candidate) over this thread's slots, in chunk order;
    // every thread visits the same number of chunks
    auto visit = [&](auto &&f) {
        if (cached) {
#pragma unroll
            for (int u = 0; u < kTopkCache; ++u) {
                if (lo + 256 * u >= hi) break;
                f(lo + 256 * u + tid, ck[u], cc[u]);
            }
        } else {
            for (int base = lo; base < hi; base += 256) {
                const int j = base + tid;
                const bool c = j < hi && pis[j] >= 0;
                f(j, c ? __float_as_uint(mass[j]) : 0u, c);
            }
        }
    };
    if (cached) {
#pragma unroll
        for (int u = 0; u < kTopkCache; ++u) {
            const int j = lo + 256 * u + tid;
            const bool c = j < hi && cpi[u] >= 0;
            cc[u] = c;
            ck[u] = c ? cms[u] : 0u;
        }
    }
    s_hist[0][tid] = 0;
    s_hist[1][tid] = 0;
    __syncthreads();

    // Radix passes.  The first one histograms every candidate, so its bins
    // also give their number.
    uint32_t prefix = 0, pmask = 0, thr = 0;
    int rem = 0, kk = 0, take_eq = 0;
    bool take_all = false;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        int *h = s_hist[pass & 1];
        visit([&](int, uint32_t key, bool c) {
            if (c && (key & pmask) == prefix) atomicAdd(&h[(key >> shift) & 255], 1);
        });
        __syncthreads();   // the histogram is complete
        // lane l of every wave: digits 255-4l .. 252-4l, counted from the top
        const int4 hv = *reinterpret_cast<const int4 *>(h + 252 - 4 * lane);
        // the other buffer, last read in the previous pass, is the next one's
        s_hist[(pass + 1) & 1][tid] = 0;
        const int t = hv.x + hv.y + hv.z + hv.w;
        int incl = t;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        if (pass == 0) {
            const int total = __shfl(incl, 63);
            kk = min(k, total);
            take_all = kk == total;   // the same in every wave
            rem = kk;
            if (take_all) break;
        }
        const int excl = incl - t;
        const int c3 = excl + hv.w, c2 = c3 + hv.z, c1 = c2 + hv.y;
        // the digit where the count from the top first reaches rem, and the
        // count of keys with a larger digit
        int dig, above;
        if (c3 >= rem) {
            dig = 255 - 4 * lane;
            above = excl;
        } else if (c2 >= rem) {
            dig = 254 - 4 * lane;
            above = c3;
        } else if (c1 >= rem) {
            dig = 253 - 4 * lane;
            above = c2;
        } else {
            dig = 252 - 4 * lane;
            above = c1;
        }
        const uint64_t m = __ballot(excl < rem && incl >= rem);
        const int src = m ? (int)__builtin_ctzll(m) : 63;
        prefix |= (uint32_t)__shfl(dig, src) << shift;
        pmask |= 255u << shift;
        rem -= __shfl(above, src);
        __syncthreads();   // the next histogram is cleared before its atomics
    }
    if (!take_all) {
        thr = prefix;
        take_eq = rem;
    }
    // in-order pass: larger than the threshold, or equal and among the first
    // take_eq equal ones (lowest indices)
    int out_base = 0, eq_base = 0, chunk = 0;
    visit([&](int j, uint32_t key, bool cand) {
        const bool gt = cand && (take_all || key > thr);
        const bool eq = cand && !take_all && key == thr;
        const uint64_t gm = __ballot(gt), em = __ballot(eq);
        int(*cnt)[2] = s_cnt[chunk & 1];
        if (lane == 0) {
            cnt[wave][0] = __popcll(gm);
            cnt[wave][1] = __popcll(em);
        }
        __syncthreads();
        int gt_lo = 0, eq_lo = 0, gt_tot = 0, eq_tot = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int g = cnt[w][0], e = cnt[w][1];
            gt_lo += w < wave ? g : 0;
            eq_lo += w < wave ? e : 0;
            gt_tot += g;
            eq_tot += e;
        }
        const int eq_room = max(take_eq - eq_base, 0);   // equal keys still to take, in index order
        const bool take = gt || (eq && eq_lo + __popcll(em & below) < eq_room);
        const uint64_t tm = __ballot(take);
        const int pos = out_base + gt_lo + min(eq_lo, eq_room) + __popcll(tm & below);
        if (take && p.sel_off[s] + pos < p.max_sel) out[pos] = j;
        out_base += gt_tot + min(eq_tot, eq_room);
        eq_base += eq_tot;
        ++chunk;
    });
    for (int i = kk + tid; i < k; i += 256)
        if (p.sel_off[s] + i < p.max_sel) out[i] = -1;
}

// One workgroup per (fused block fb, group of kFuseHeads kv heads, request r):
// fresh K rows are copied 16 bytes at a time; fresh V rows are staged in LDS
// with 16-byte loads and written channel-major, 8 slots (16 bytes) per store.
// Only the fresh slots of a partial last block are written.  Every load of a
// workgroup is issued before its first store, so it waits on one round trip;
// the small workgroups (16 KB moved at d 128) keep several resident per CU.
// The head-group-0 workgroups also rewrite the request's positions.
constexpr int kFuseHeads = 2;

template <int D>
__global__ __launch_bounds__(256) void fuse_kernel(FuseParams p) {
    constexpr int CPR = D / 8;   // 16-byte chunks per row
    static_assert(kBlock * CPR <= 256, "one row chunk per thread");
    __shared__ __attribute__((aligned(16))) uint16_t s_v[kFuseHeads][kBlock][D + 8];
    const int fb = blockIdx.x, g0 = blockIdx.y * kFuseHeads, r = blockIdx.z, tid = threadIdx.x;
    const int row0 = max(0, p.sel_req_off[r]);
    const int cnt = min(p.sel_req_off[r + 1], p.n_sel) - row0;
    const int kv_stride = p.max_blocks * kBlock;
    int kvl = p.kv_len[r];
    kvl = kvl < 0 ? 0 : (kvl > kv_stride ? kv_stride : kvl);
    const int base = (kvl + kBlock - 1) / kBlock * kBlock;
    int32_t *pis = p.kv_pos + (size_t)r * kv_stride;
    if (fb == 0 && g0 == 0) {
        for (int j = kvl + tid; j < base; j += 256) pis[j] = -1;
    }
    const int n_here = min(kBlock, cnt - kBlock * fb);
    if (n_here <= 0 || g0 >= p.hkv) return;
    const int bidx = base / kBlock + fb;
    if (bidx >= p.max_blocks) return;
    const int blk = p.block_table[(size_t)r * p.max_blocks + bidx];
    if (blk < 0 || blk >= p.num_blocks) return;
    const int rowb = row0 + kBlock * fb;
    const int ng = min(kFuseHeads, p.hkv - g0);
    // this thread's chunk: slot sl, 16-byte column c
    const int sl = tid / CPR, c = tid % CPR;
    const bool has = tid < kBlock * CPR;
    const bool fresh = has && sl < n_here;

    u32x4 kc[kFuseHeads], vc[kFuseHeads];
#pragma unroll
    for (int gi = 0; gi < kFuseHeads; ++gi) {
        kc[gi] = vc[gi] = u32x4{0u, 0u, 0u, 0u};
        if (gi < ng && fresh) {
            const size_t src = ((size_t)(rowb + sl) * p.hkv + g0 + gi) * D + 8 * c;
            kc[gi] = *reinterpret_cast<const u32x4 *>(p.k_new + src);
            vc[gi] = *reinterpret_cast<const u32x4 *>(p.v_new + src);
        }
    }
#pragma unroll
    for (int gi = 0; gi < kFuseHeads; ++gi) {
        if (gi < ng && fresh)   // K rows: token-major in the pool
            *reinterpret_cast<u32x4 *>(p.k_pool + (((size_t)blk * p.hkv + g0 + gi) * kBlock + sl) * D + 8 * c) =
                kc[gi];
        if (gi < ng && has) *reinterpret_cast<u32x4 *>(&s_v[gi][sl][8 * c]) = vc[gi];
    }
    __syncthreads();
    // V: channel-major, thread -> (head, channel d, slots 8h .. 8h+7)
    for (int t = tid; t < ng * 2 * D; t += 256) {
        const int gi = t / (2 * D), d = (t >> 1) % D, h = t & 1;
        uint16_t *dst = p.v_pool + (((size_t)blk * p.hkv + g0 + gi) * D + d) * kBlock + 8 * h;
        if (8 * h + 8 <= n_here) {
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = (uint32_t)s_v[gi][8 * h + 2 * e][d] | ((uint32_t)s_v[gi][8 * h + 2 * e + 1][d] << 16);
            *reinterpret_cast<u32x4 *>(dst) = w;
        } else {
            for (int i = 0; i < 8 && 8 * h + i < n_here; ++i) dst[i] = s_v[gi][8 * h + i][d];
        }
    }
    // positions: fresh slot takes the stale slot's pi, the stale slot is masked
    if (g0 == 0 && tid < n_here) {
        const int i = kBlock * fb + tid;
        const int sel = p.sel_idx[row0 + i];
        const int slot = base + i;
        if (sel >= 0 && sel < kvl) {
            pis[slot] = pis[sel];
            pis[sel] = -1;
        } else {
            pis[slot] = -1;
        }
    }
}

__global__ void fuse_len_kernel(FuseParams p) {
    const int r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= p.batch) return;
    const int kv_stride = p.max_blocks * kBlock;
    int kvl = p.kv_len[r];
    kvl = kvl < 0 ? 0 : (kvl > kv_stride ? kv_stride : kvl);
    const int base = (kvl + kBlock - 1) / kBlock * kBlock;
    const int row0 = max(0, p.sel_req_off[r]);
    const int cnt = max(0, min(p.sel_req_off[r + 1], p.n_sel) - row0);
    p.kv_len[r] = min(base + cnt, kv_stride);
}

// Anchor score of every slot of a request (QCFuse, gist.science 2604.08585,
// methodology A / phase 1: anchors are the tokens with the highest key norms):
// the squared norm of the stored (unrotated) key over all kv heads, 0 for
// unusable slots.  One workgroup per 16-slot block, each 16-lane group one
// slot; a lane sums the squares of its 16-byte chunks of the slot's key (bf16
// squares are exact in fp32), chunks i, i + 16, ... in that order, and a
// fixed-order butterfly adds the 16 lanes: deterministic.  The block id comes
// first; every chunk of a lane is then requested before the first add, so a
// workgroup waits on two memory round trips.  HBM-bound: every usable key is
// read once.
template <int D>
__global__ __launch_bounds__(256) void key_norm_kernel(NormParams p) {
    const int b = blockIdx.x, r = blockIdx.y;
    const int kv_stride = p.max_blocks * kBlock;
    int kvl = p.kv_len[r];
    kvl = kvl < 0 ? 0 : (kvl > kv_stride ? kv_stride : kvl);
    if (b * kBlock >= kvl) return;
    const int blk = p.block_table[(size_t)r * p.max_blocks + b];
    const bool bok = (unsigned)blk < (unsigned)p.num_blocks;
    const int lane = threadIdx.x & 15;
    const int off = threadIdx.x >> 4, j = b * kBlock + off;   // slot of this lane's group
    const int pi = p.kv_pos[(size_t)r * kv_stride + j];       // j < kv_stride: b < max_blocks
    constexpr int CPR = D / 8;               // 16-byte chunks per head row
    constexpr int BATCH = 8;                 // chunks of a lane requested together
    const int nch = p.hkv * CPR;             // chunks of one slot's key
    float acc = 0.f;
    if (bok) {
        for (int c0 = lane; c0 < nch; c0 += 16 * BATCH) {
            u32x4 v[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int c = c0 + 16 * u;
                const int cl = c < nch ? c : 0;   // a chunk of the key: every load stays in the row
                const int g = cl / CPR, cc = cl % CPR;
                const u32x4 x = *reinterpret_cast<const u32x4 *>(
                    p.k_pool + (((size_t)blk * p.hkv + g) * kBlock + off) * D + 8 * cc);
                v[u] = c < nch ? x : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int u = 0; u < BATCH; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = __uint_as_float(v[u][e] << 16), hi = __uint_as_float(v[u][e] & 0xffff0000u);
                    acc = fmaf(lo, lo, acc);
                    acc = fmaf(hi, hi, acc);
                }
        }
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
    const bool ok = bok && (unsigned)pi < (unsigned)p.max_pos;
    if (lane == 0 && j < kvl) p.norm[(size_t)r * kv_stride + j] = ok ? acc : 0.f;
}

}  // namespace

hipError_t launch_key_norm(const NormParams &p, int head_dim, hipStream_t s) {
    if (p.batch <= 0 || p.max_blocks <= 0) return hipSuccess;
    const dim3 grid(p.max_blocks, p.batch);
    if (head_dim == 64)
        hipLaunchKernelGGL(key_norm_kernel<64>, grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(key_norm_kernel<128>, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_mass_reduce(const SelectParams &p, hipStream_t s) {
    if (p.batch <= 0 || p.mass_stride <= 0) return hipSuccess;
    hipLaunchKernelGGL(mass_reduce_kernel, dim3((p.mass_stride + 255) / 256, p.batch), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_topk(const SelectParams &p, hipStream_t s) {
    if (p.n_spans <= 0) return hipSuccess;
    hipLaunchKernelGGL(span_topk_kernel, dim3(p.n_spans), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_fuse(const FuseParams &p, int head_dim, hipStream_t s) {
    if (p.batch <= 0) return hipSuccess;
    const int nfb = p.max_rows > 0 ? (p.max_rows + kBlock - 1) / kBlock : 1;
    const dim3 grid(nfb, (p.hkv + kFuseHeads - 1) / kFuseHeads, p.batch);
    if (head_dim == 64)
        hipLaunchKernelGGL(fuse_kernel<64>, grid, dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL(fuse_kernel<128>, grid, dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fuse_len_kernel, dim3((p.batch + 255) / 256), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace pic
