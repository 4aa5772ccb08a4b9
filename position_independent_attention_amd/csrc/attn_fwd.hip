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
//   A workgroup (4 x wave64) owns one (request, kv head, key split, row block).
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
//   Per 64-key tile the whole workgroup stages K once: global -> registers ->
//   RoPE with the fp32 cos/sin table row of the key's pi -> bf16 -> LDS, so
//   every key is rotated once per workgroup however many rows read it.  V is
//   stored in the pool head-dim-major per block ([d][16]), so V^T tiles are
//   plain 16-byte copies.  Global loads of the next tile are issued before the
//   current tile's MFMA work.
#include "pic_internal.h"

namespace pic {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

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

// Rotate 8 RoPE pairs: lo holds x[i..i+7], hi holds x[i+d/2..i+d/2+7] (bf16),
// c/s the cos/sin of pos * theta^(-2(i+e)/d).  Result rounded to bf16.
__device__ __forceinline__ void rope8(u32x4 &lo, u32x4 &hi, const f32x4 c0, const f32x4 c1,
                                      const f32x4 s0, const f32x4 s1) {
    const float c[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
    const float s[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    u32x4 ro, rh;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float a0 = bf_lo(lo[e]), a1 = bf_hi(lo[e]);
        const float b0 = bf_lo(hi[e]), b1 = bf_hi(hi[e]);
        const float cc0 = c[2 * e], cc1 = c[2 * e + 1], ss0 = s[2 * e], ss1 = s[2 * e + 1];
        ro[e] = pack2(fmaf(a0, cc0, -b0 * ss0), fmaf(a1, cc1, -b1 * ss1));
        rh[e] = pack2(fmaf(a0, ss0, b0 * cc0), fmaf(a1, ss1, b1 * cc1));
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

template <int D>
struct Geo {
    static constexpr int NC = D / 32;            // 32-wide MFMA k chunks along d
    static constexpr int HALF = D / 2;
    static constexpr int PC = D / 16;            // 8-pair chunks per key
    static constexpr int KTASK = kTileN * PC / kThreads;   // K staging tasks per thread
    static constexpr int VCH = D / 32;           // V chunks per thread
    static constexpr int KS = D + 8;             // LDS row stride of K (bf16)
    static constexpr int VS = kTileN + 8;        // LDS row stride of V^T (bf16)
};

// One thread's share of a tile's global loads, kept in registers while the
// previous tile is being computed.
template <int D>
struct Stage {
    u32x4 klo[Geo<D>::KTASK], khi[Geo<D>::KTASK];
    int32_t kpi[Geo<D>::KTASK];     // pi if the key is usable, else -1
    u32x4 v[Geo<D>::VCH];
    int32_t vmask;                  // bit e set: key e of this thread's V chunk is unusable
};

template <int D>
__device__ __forceinline__ void stage_load(const FwdParams &p, Stage<D> &st, int r, int g, int tile,
                                           int key_end, int tid) {
    using GG = Geo<D>;
    const int32_t *bt = p.block_table + (size_t)r * p.max_blocks;
    const int32_t *pis = p.kv_pos + (size_t)r * p.max_blocks * kBlock;
#pragma unroll
    for (int u = 0; u < GG::KTASK; ++u) {
        const int kk = tid / GG::PC + u * (kThreads / GG::PC);
        const int pc = tid % GG::PC;
        const int j = tile + kk;
        int pi = -1, blk = -1;
        if (j < key_end) {
            blk = bt[j >> 4];
            pi = pis[j];
        }
        const bool ok = blk >= 0 && blk < p.num_blocks && pi >= 0 && pi < p.max_pos;
        st.kpi[u] = ok ? pi : -1;
        st.klo[u] = u32x4{0, 0, 0, 0};
        st.khi[u] = u32x4{0, 0, 0, 0};
        if (ok) {
            const uint16_t *row = p.k_pool + (((size_t)blk * p.hkv + g) * kBlock + (j & 15)) * D;
            st.klo[u] = *reinterpret_cast<const u32x4 *>(row + 8 * pc);
            st.khi[u] = *reinterpret_cast<const u32x4 *>(row + GG::HALF + 8 * pc);
        }
    }
    // V^T chunks: this thread covers keys 16*b + 8*half .. +7 of the tile for
    // d = dd + 32*u.
    const int half = tid & 1, dd = (tid >> 1) & 31, b = (tid >> 6) & 3;
    const int j0 = tile + 16 * b + 8 * half;
    int blk = -1;
    if (j0 < key_end) blk = bt[j0 >> 4];
    const bool bok = blk >= 0 && blk < p.num_blocks;
    int32_t vm = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int j = j0 + e;
        bool ok = bok && j < key_end;
        if (ok) {
            const int pi = pis[j];
            ok = pi >= 0 && pi < p.max_pos;
        }
        vm |= ok ? 0 : (1 << e);
    }
    st.vmask = vm;
#pragma unroll
    for (int u = 0; u < GG::VCH; ++u) {
        const int d = dd + 32 * u;
        st.v[u] = u32x4{0, 0, 0, 0};
        if (bok && vm != 0xff)
            st.v[u] = *reinterpret_cast<const u32x4 *>(
                p.v_pool + (((size_t)blk * p.hkv + g) * D + d) * kBlock + 8 * half);
    }
}

template <int D>
__device__ __forceinline__ void stage_store(const FwdParams &p, Stage<D> &st, uint16_t *Ks,
                                            uint16_t *Vs, int32_t *s_pi, int tid, bool need_v) {
    using GG = Geo<D>;
    const int half_n = GG::HALF;
#pragma unroll
    for (int u = 0; u < GG::KTASK; ++u) {
        const int kk = tid / GG::PC + u * (kThreads / GG::PC);
        const int pc = tid % GG::PC;
        const int pi = st.kpi[u];
        u32x4 lo = st.klo[u], hi = st.khi[u];
        if (pi >= 0) {
            const float *cr = p.cos_tab + (size_t)pi * half_n + 8 * pc;
            const float *sr = p.sin_tab + (size_t)pi * half_n + 8 * pc;
            const f32x4 c0 = *reinterpret_cast<const f32x4 *>(cr);
            const f32x4 c1 = *reinterpret_cast<const f32x4 *>(cr + 4);
            const f32x4 s0 = *reinterpret_cast<const f32x4 *>(sr);
            const f32x4 s1 = *reinterpret_cast<const f32x4 *>(sr + 4);
            rope8(lo, hi, c0, c1, s0, s1);
        }
        *reinterpret_cast<u32x4 *>(Ks + kk * GG::KS + 8 * pc) = lo;
        *reinterpret_cast<u32x4 *>(Ks + kk * GG::KS + GG::HALF + 8 * pc) = hi;
        if (pc == 0) s_pi[kk] = pi;
    }
    if (need_v) {
        const int half = tid & 1, dd = (tid >> 1) & 31, b = (tid >> 6) & 3;
        const int vm = st.vmask;
#pragma unroll
        for (int u = 0; u < GG::VCH; ++u) {
            u32x4 v = st.v[u];
            if (vm) {   // zero unusable keys so that 0 * garbage cannot poison O
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t w = v[e];
                    if (vm & (1 << (2 * e))) w &= 0xffff0000u;
                    if (vm & (1 << (2 * e + 1))) w &= 0x0000ffffu;
                    v[e] = w;
                }
            }
            const int d = dd + 32 * u;
            *reinterpret_cast<u32x4 *>(Vs + d * GG::VS + 16 * b + 8 * half) = v;
        }
    }
}

template <int D, int QG, int MODE>
__global__ __launch_bounds__(kThreads) void fwd_kernel(FwdParams p) {
    using GG = Geo<D>;
    constexpr int BM = 16 * QG * kWaves;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[kTileN * GG::KS];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[MODE == kAttn ? D * GG::VS : 8];
    __shared__ int32_t s_pi[kTileN];
    __shared__ float s_red[MODE == kMass ? kWaves * kTileN : 1];

    const int nwg = p.row_blocks * p.hkv * p.num_splits * p.batch;
    int lid = xcd_remap(blockIdx.x, nwg);
    const int rb = lid % p.row_blocks;
    lid /= p.row_blocks;
    const int g = lid % p.hkv;
    lid /= p.hkv;
    const int sp = lid % p.num_splits;
    const int r = lid / p.num_splits;

    const int q0 = p.q_start[r];
    const int nq = p.q_start[r + 1] - q0;
    const int nrows = nq * p.group;
    if (rb * BM >= nrows) return;
    const int kv_stride = p.max_blocks * kBlock;
    const int kv_cap = min(kv_stride, p.max_kv_len);
    int kvl = p.kv_len[r];
    kvl = kvl < 0 ? 0 : (kvl > kv_cap ? kv_cap : kvl);
    const int key_begin = sp * p.split_len;
    const int key_end = min(kvl, key_begin + p.split_len);

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int lc = lane & 15, lg = lane >> 4;

    // ---- this lane's query columns: load, rotate at q_pos, keep as B operands
    u32x4 qop[QG][GG::NC];
    int qpos[QG], qt[QG], qh[QG];
    bool qvalid[QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        const int row = rb * BM + wave * 16 * QG + 16 * qg + lc;
        qvalid[qg] = row < nrows;
        const int tl = qvalid[qg] ? row / p.group : 0;
        qt[qg] = q0 + tl;
        qh[qg] = g * p.group + (qvalid[qg] ? row % p.group : 0);
        int pos = qvalid[qg] ? p.q_pos[qt[qg]] : -1;
        if (pos >= p.max_pos) pos = -1;
        qpos[qg] = pos;
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
                      *reinterpret_cast<const f32x4 *>(sr), *reinterpret_cast<const f32x4 *>(sr + 4));
                qop[qg][c] = lo;
                qop[qg][c + GG::NC / 2] = hi;
            }
        }
    }

    float m_run[QG], l_run[QG], lse2[QG];
    f32x4 acc[MODE == kAttn ? QG : 1][MODE == kAttn ? D / 16 : 1];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        m_run[qg] = -INFINITY;
        l_run[qg] = 0.f;
        lse2[qg] = INFINITY;
        if constexpr (MODE == kMass) {
            if (qpos[qg] >= 0) {
                const float ls = p.lse_in[(size_t)qt[qg] * p.hq + qh[qg]];
                // -inf (nothing visible) or NaN: contribute nothing
                lse2[qg] = (ls > -INFINITY) ? ls * 1.4426950408889634f : INFINITY;
            }
        }
    }
    if constexpr (MODE == kAttn) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) acc[qg][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int ntiles = key_end > key_begin ? (key_end - key_begin + kTileN - 1) / kTileN : 0;
    Stage<D> st;
    if (ntiles > 0) stage_load<D>(p, st, r, g, key_begin, key_end, tid);

    for (int it = 0; it < ntiles; ++it) {
        const int tile = key_begin + it * kTileN;
        __syncthreads();
        stage_store<D>(p, st, Ks, Vs, s_pi, tid, MODE == kAttn);
        __syncthreads();
        if (it + 1 < ntiles) stage_load<D>(p, st, r, g, tile + kTileN, key_end, tid);

        // ---- S^T = K Q^T for the 64-key tile: sacc[qg][kh][T]
        f32x4 sacc[QG][2][2];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int T = 0; T < 2; ++T) sacc[qg][kh][T] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
            for (int T = 0; T < 2; ++T) {
                const int key = 32 * kh + 8 * (lc >> 2) + 4 * T + (lc & 3);
#pragma unroll
                for (int c = 0; c < GG::NC; ++c) {
                    const u32x4 a = *reinterpret_cast<const u32x4 *>(Ks + key * GG::KS + 32 * c + 8 * lg);
#pragma unroll
                    for (int qg = 0; qg < QG; ++qg) sacc[qg][kh][T] = mfma16(a, qop[qg][c], sacc[qg][kh][T]);
                }
            }
        }
        // pi of this lane's 16 keys: u = kh*8 + T*4 + i  ->  key 32kh + 8lg + 4T + i
        int kp[16];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            const i32x4 a = *reinterpret_cast<const i32x4 *>(s_pi + 32 * kh + 8 * lg);
            const i32x4 b = *reinterpret_cast<const i32x4 *>(s_pi + 32 * kh + 8 * lg + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kp[kh * 8 + i] = a[i];
                kp[kh * 8 + 4 + i] = b[i];
            }
        }

        if constexpr (MODE == kMass) {
            float cs[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) cs[u] = 0.f;
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const float s = sacc[qg][u >> 3][(u >> 2) & 1][u & 3];
                    const bool vis = kp[u] >= 0 && kp[u] <= qpos[qg];
                    cs[u] += vis ? fast_exp2(s * p.scale_log2 - lse2[qg]) : 0.f;
                }
            }
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
            s_red[wave * kTileN + key] = cs[0];
            __syncthreads();
            if (tid < kTileN) {
                const float tot = ((s_red[tid] + s_red[kTileN + tid]) + s_red[2 * kTileN + tid]) +
                                  s_red[3 * kTileN + tid];
                const int j = tile + tid;
                if (j < key_end)
                    p.mass_part[(((size_t)r * p.hkv + g) * p.row_blocks + rb) * p.mass_stride + j] = tot;
            }
        } else {
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) {
                float sv[16];
                float mx = -INFINITY;
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const float s = sacc[qg][u >> 3][(u >> 2) & 1][u & 3];
                    const bool vis = kp[u] >= 0 && kp[u] <= qpos[qg];
                    sv[u] = vis ? s * p.scale_log2 : -INFINITY;
                    mx = fmaxf(mx, sv[u]);
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run[qg], mx);
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = fast_exp2(m_run[qg] - m_use);
                m_run[qg] = m_new;
                float ls = 0.f;
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    sv[u] = fast_exp2(sv[u] - m_use);
                    ls += sv[u];
                }
                l_run[qg] = l_run[qg] * alpha + ls;
                if constexpr (MODE == kAttn) {
#pragma unroll
                    for (int dt = 0; dt < D / 16; ++dt) acc[qg][dt] *= alpha;
#pragma unroll
                    for (int kh = 0; kh < 2; ++kh) {
                        u32x4 pb;
#pragma unroll
                        for (int e = 0; e < 4; ++e) pb[e] = pack2(sv[kh * 8 + 2 * e], sv[kh * 8 + 2 * e + 1]);
#pragma unroll
                        for (int dt = 0; dt < D / 16; ++dt) {
                            const u32x4 a =
                                *reinterpret_cast<const u32x4 *>(Vs + (16 * dt + lc) * GG::VS + 32 * kh + 8 * lg);
                            acc[qg][dt] = mfma16(a, pb, acc[qg][dt]);
                        }
                    }
                }
            }
        }
    }
    if constexpr (MODE == kMass) return;

    // ---- epilogue: per-lane partial sums -> column totals
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
        float lt = l_run[qg];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        if (!qvalid[qg]) continue;
        const size_t rowid = (size_t)qt[qg] * p.hq + qh[qg];
        if (p.num_splits == 1) {
            const bool any = lt > 0.f;
            if constexpr (MODE == kAttn) {
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
            if constexpr (MODE == kAttn) {
#pragma unroll
                for (int dt = 0; dt < D / 16; ++dt)
                    *reinterpret_cast<f32x4 *>(p.part_o + prow * D + 16 * dt + 4 * lg) = acc[qg][dt];
            }
            if (lg == 0) {
                p.part_ml[prow * 2 + 0] = m_run[qg];
                p.part_ml[prow * 2 + 1] = lt;
            }
        }
    }
}

// LSE-weighted merge of split partials.  One thread per (row, 4 channels).
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
    constexpr int TPR = D / 4;   // threads per row
    const int gtid = blockIdx.x * 256 + threadIdx.x;
    const int row = gtid / TPR, part = gtid % TPR;
    if (row >= p.rows) return;
    float M = -INFINITY;
    for (int s = 0; s < p.num_splits; ++s) M = fmaxf(M, p.part_ml[((size_t)s * p.rows + row) * 2]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.num_splits; ++s) {
        const size_t pr = (size_t)s * p.rows + row;
        const float w = fast_exp2(p.part_ml[pr * 2] - Mu);
        L += w * p.part_ml[pr * 2 + 1];
        if (p.part_o) o += w * *reinterpret_cast<const f32x4 *>(p.part_o + pr * D + 4 * part);
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

template <int D, int QG, int MODE>
hipError_t launch_one(const FwdParams &p, hipStream_t s) {
    const int nwg = p.row_blocks * p.hkv * p.num_splits * p.batch;
    if (nwg <= 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_kernel<D, QG, MODE>), dim3(nwg), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <int D, int MODE>
hipError_t launch_qg(const FwdParams &p, int qg, hipStream_t s) {
    switch (qg) {
    case 1: return launch_one<D, 1, MODE>(p, s);
    case 2: return launch_one<D, 2, MODE>(p, s);
    default: return launch_one<D, 4, MODE>(p, s);
    }
}

template <int D>
hipError_t launch_mode(const FwdParams &p, int mode, int qg, hipStream_t s) {
    switch (mode) {
    case kAttn: return launch_qg<D, kAttn>(p, qg, s);
    case kLse: return launch_qg<D, kLse>(p, qg, s);
    default: return launch_qg<D, kMass>(p, qg, s);
    }
}

}  // namespace

hipError_t launch_fwd(const FwdParams &p, int head_dim, int mode, int qg, hipStream_t s) {
    return head_dim == 64 ? launch_mode<64>(p, mode, qg, s) : launch_mode<128>(p, mode, qg, s);
}

hipError_t launch_merge(const MergeParams &p, int head_dim, hipStream_t s) {
    if (p.rows <= 0) return hipSuccess;
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
