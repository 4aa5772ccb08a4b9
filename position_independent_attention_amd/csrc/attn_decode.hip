// Decode (one query token per request) over the paged, unrotated KV cache,
// with RoPE applied in-kernel at each key's logical position (MiniPIC,
// gist.science 2606.13126, section 2.1 score equation).
//
// Bound by HBM bytes: every cached key and value is read once per
// (request, kv head) and feeds only G = Hq/Hkv query rows.  So there is no
// LDS staging: each wave streams its own 32-key steps straight from global
// memory into MFMA operand registers, rotates the K operand in registers with
// the fp32 cos/sin row of the key's pi, and runs the same transposed
// S^T = K Q^T / O^T += V^T P^T scheme as the prefill kernel (the G query heads
// are the MFMA columns; columns >= G are masked).  The next step's loads are
// issued before the current step's math.  A workgroup (4 waves) covers 1024
// keys of one (request, kv head); waves are merged through LDS and splits by
// the LSE merge kernel.
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
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int X = 8;
    const int xcd = bid % X, idx = bid / X;
    const int q = n / X, rem = n % X;
    return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

// One 32-key step's operands for one lane.
template <int D>
struct Step {
    static constexpr int NC = D / 32;
    u32x4 k[2][NC];          // A operand rows (before rotation), tiles T = 0, 1
    f32x4 cs[2][NC / 2][4];  // cos0, cos1, sin0, sin1 for the rotated pairs
    int32_t kpi[2];          // pi of the A row keys (-1 unusable)
    u32x4 v[D / 16];         // V^T operand, channel 16*dt + lc, keys 8lg..8lg+7
    int32_t spi[8];          // pi of this lane's 8 score keys (-1 unusable)
};

template <int D>
__device__ __forceinline__ void step_load(const DecodeParams &p, Step<D> &st, const int32_t *bt,
                                          const int32_t *pis, int g, int kb, int key_end, int lc,
                                          int lg) {
    constexpr int NC = D / 32, HALF = D / 2;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
        const int j = kb + 8 * (lc >> 2) + 4 * T + (lc & 3);
        int pi = -1, blk = -1;
        if (j < key_end) {
            blk = bt[j >> 4];
            pi = pis[j];
        }
        const bool ok = blk >= 0 && blk < p.num_blocks && pi >= 0 && pi < p.max_pos;
        st.kpi[T] = ok ? pi : -1;
        const uint16_t *row = p.k_pool + (((size_t)(ok ? blk : 0) * p.hkv + g) * kBlock + (j & 15)) * D;
        const float *cr = p.cos_tab + (size_t)(ok ? pi : 0) * HALF;
        const float *sr = p.sin_tab + (size_t)(ok ? pi : 0) * HALF;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            st.k[T][c] = ok ? *reinterpret_cast<const u32x4 *>(row + 32 * c + 8 * lg) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < NC / 2; ++c) {
            const int i0 = 32 * c + 8 * lg;
            st.cs[T][c][0] = *reinterpret_cast<const f32x4 *>(cr + i0);
            st.cs[T][c][1] = *reinterpret_cast<const f32x4 *>(cr + i0 + 4);
            st.cs[T][c][2] = *reinterpret_cast<const f32x4 *>(sr + i0);
            st.cs[T][c][3] = *reinterpret_cast<const f32x4 *>(sr + i0 + 4);
        }
    }
    const int j0 = kb + 8 * lg;
    int blk = -1;
    if (j0 < key_end) blk = bt[j0 >> 4];
    const bool bok = blk >= 0 && blk < p.num_blocks;
    bool all = bok && j0 + 8 <= key_end;
    if (all) {
        const i32x4 a = *reinterpret_cast<const i32x4 *>(pis + j0);
        const i32x4 b = *reinterpret_cast<const i32x4 *>(pis + j0 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            st.spi[i] = a[i];
            st.spi[4 + i] = b[i];
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) st.spi[e] = (bok && j0 + e < key_end) ? pis[j0 + e] : -1;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if (st.spi[e] >= p.max_pos) st.spi[e] = -1;
    const uint16_t *vb = p.v_pool + ((size_t)(bok ? blk : 0) * p.hkv + g) * D * kBlock + (j0 & 15);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        st.v[dt] = bok ? *reinterpret_cast<const u32x4 *>(vb + (size_t)(16 * dt + lc) * kBlock)
                       : u32x4{0, 0, 0, 0};
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams p) {
    constexpr int NC = D / 32, HALF = D / 2;
    constexpr int WAVE_KEYS = kDecodeSplit / kWaves;
    __shared__ float s_o[kWaves][D][16];
    __shared__ float s_m[kWaves][16], s_l[kWaves][16];

    const int nwg = p.hkv * p.num_splits * p.batch;
    int lid = xcd_remap(blockIdx.x, nwg);
    const int g = lid % p.hkv;
    lid /= p.hkv;
    const int sp = lid % p.num_splits;
    const int r = lid / p.num_splits;

    const int kv_stride = p.max_blocks * kBlock;
    const int kv_cap = min(kv_stride, p.max_kv_len);
    int kvl = p.kv_len[r];
    kvl = kvl < 0 ? 0 : (kvl > kv_cap ? kv_cap : kvl);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lc = lane & 15, lg = lane >> 4;
    const int wbeg = sp * kDecodeSplit + wave * WAVE_KEYS;
    const int key_end = min(kvl, wbeg + WAVE_KEYS);
    const int32_t *bt = p.block_table + (size_t)r * p.max_blocks;
    const int32_t *pis = p.kv_pos + (size_t)r * kv_stride;

    // query column lc: head g*G + lc of request r
    const bool qv = lc < p.group;
    const int h = g * p.group + (qv ? lc : 0);
    int pos = qv ? p.q_pos[r] : -1;
    if (pos >= p.max_pos) pos = -1;
    u32x4 qop[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) qop[c] = u32x4{0, 0, 0, 0};
    if (pos >= 0) {
        const uint16_t *src = p.q + ((size_t)r * p.hq + h) * D;
#pragma unroll
        for (int c = 0; c < NC / 2; ++c) {
            const int i0 = 32 * c + 8 * lg;
            u32x4 lo = *reinterpret_cast<const u32x4 *>(src + i0);
            u32x4 hi = *reinterpret_cast<const u32x4 *>(src + HALF + i0);
            const float *cr = p.cos_tab + (size_t)pos * HALF + i0;
            const float *sr = p.sin_tab + (size_t)pos * HALF + i0;
            rope8(lo, hi, *reinterpret_cast<const f32x4 *>(cr), *reinterpret_cast<const f32x4 *>(cr + 4),
                  *reinterpret_cast<const f32x4 *>(sr), *reinterpret_cast<const f32x4 *>(sr + 4));
            qop[c] = lo;
            qop[c + NC / 2] = hi;
        }
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nsteps = key_end > wbeg ? (key_end - wbeg + 31) / 32 : 0;
    Step<D> cur;
    if (nsteps > 0) step_load<D>(p, cur, bt, pis, g, wbeg, key_end, lc, lg);
    for (int it = 0; it < nsteps; ++it) {
        Step<D> nxt;
        if (it + 1 < nsteps) step_load<D>(p, nxt, bt, pis, g, wbeg + 32 * (it + 1), key_end, lc, lg);

        f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            if (cur.kpi[T] >= 0) {
#pragma unroll
                for (int c = 0; c < NC / 2; ++c)
                    rope8(cur.k[T][c], cur.k[T][c + NC / 2], cur.cs[T][c][0], cur.cs[T][c][1],
                          cur.cs[T][c][2], cur.cs[T][c][3]);
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) sacc[T] = mfma16(cur.k[T][c], qop[c], sacc[T]);
        }
        float sv[8];
        float mx = -INFINITY;
        bool any_bad = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int kp = cur.spi[e];
            const bool vis = kp >= 0 && kp <= pos;
            any_bad |= kp < 0;
            sv[e] = vis ? sacc[e >> 2][e & 3] * p.scale_log2 : -INFINITY;
            mx = fmaxf(mx, sv[e]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            sv[e] = fast_exp2(sv[e] - m_use);
            ls += sv[e];
        }
        l_run = l_run * alpha + ls;
        u32x4 pb;
#pragma unroll
        for (int e = 0; e < 4; ++e) pb[e] = pack2(sv[2 * e], sv[2 * e + 1]);
        // any unusable key in the step: zero its V channel entries so that
        // 0 * garbage cannot poison O
        const bool wave_bad = __any(any_bad);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
            u32x4 a = cur.v[dt];
            if (wave_bad) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t w = a[e];
                    if (cur.spi[2 * e] < 0) w &= 0xffff0000u;
                    if (cur.spi[2 * e + 1] < 0) w &= 0x0000ffffu;
                    a[e] = w;
                }
            }
            acc[dt] = mfma16(a, pb, acc[dt] * alpha);
        }
        if (it + 1 < nsteps) cur = nxt;
    }

    // ---- merge the 4 waves of the workgroup through LDS
    float lt = l_run;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_o[wave][16 * dt + 4 * lg + i][lc] = acc[dt][i];
    if (lg == 0) {
        s_m[wave][lc] = m_run;
        s_l[wave][lc] = lt;
    }
    __syncthreads();
    // thread -> (column, 8 channels)
    const int col = tid & 15, d0 = (tid >> 4) * (D / 16);
    if (col >= p.group) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][col]);
    const float Mu = M == -INFINITY ? 0.f : M;
    float wgt[kWaves], L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        wgt[w] = fast_exp2(s_m[w][col] - Mu);
        L += wgt[w] * s_l[w][col];
    }
    float o[D / 16];
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
        float a = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) a += wgt[w] * s_o[w][d0 + i][col];
        o[i] = a;
    }
    const size_t rowid = (size_t)r * p.hq + g * p.group + col;
    if (p.num_splits == 1) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
        for (int i = 0; i < D / 16; i += 2)
            *reinterpret_cast<uint32_t *>(p.out + rowid * D + d0 + i) = pack2(o[i] * inv, o[i + 1] * inv);
        if (p.lse && tid < 16)
            p.lse[rowid] = L > 0.f ? (M + __log2f(L)) * 0.6931471805599453f : -INFINITY;
    } else {
        const size_t prow = (size_t)sp * p.batch * p.hq + rowid;
#pragma unroll
        for (int i = 0; i < D / 16; i += 4)
            *reinterpret_cast<f32x4 *>(p.part_o + prow * D + d0 + i) = f32x4{o[i], o[i + 1], o[i + 2], o[i + 3]};
        if (tid < 16) {
            p.part_ml[prow * 2] = M;
            p.part_ml[prow * 2 + 1] = L;
        }
    }
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int head_dim, hipStream_t s) {
    const int nwg = p.hkv * p.num_splits * p.batch;
    if (nwg <= 0) return hipSuccess;
    if (head_dim == 64)
        hipLaunchKernelGGL(decode_kernel<64>, dim3(nwg), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL(decode_kernel<128>, dim3(nwg), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace pic
