// Decode (one query token per request) over the paged, unrotated KV cache,
// with RoPE applied in-kernel at each key's logical position (MiniPIC,
// gist.science 2606.13126, section 2.1 score equation).
//
// Bound by HBM bytes: every cached key and value is read once per
// (request, kv head) and feeds only G = Hq/Hkv query rows.  So there is no
// LDS staging of K/V: each wave streams its own 32-key steps straight from
// global memory into MFMA operand registers (the next step's K, V and
// positions are requested before the current step's math), rotates the K
// operand in registers, and runs the same transposed S^T = K Q^T /
// O^T += V^T P^T scheme as the prefill kernel (the G query heads are the MFMA
// columns; columns >= G are masked).
//
// Rotation of key j at position pi uses R(pi) = R(pi - dl) R(dl) with dl the
// key's offset inside its 16-key block (capped at pi): the keys of a block
// that holds consecutive positions then all read the one table row pi - dl,
// which stays in L1, and R(dl) for dl = 0..15 (rows 0..15 of the same table)
// sits in LDS.  Any dl in 0..pi gives the same rotation, so blocks holding
// arbitrary positions are handled by the same code.
//
// A workgroup (4 waves) covers split_len keys of one (request, kv head);
// waves are merged through LDS and splits by the LSE merge kernel.
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

// Rotate 4 RoPE pairs: words 2*hh, 2*hh+1 of lo hold x[i..i+3] (first
// halves, two bf16 per word), the same words of hi the second halves x[i+d/2..];
// c/s the cos/sin of the 4 pairs.  Result rounded to bf16.
template <int hh>
__device__ __forceinline__ void rope4(u32x4 &lo, u32x4 &hi, const f32x4 c, const f32x4 s) {
    const uint32_t l0 = lo[2 * hh], l1 = lo[2 * hh + 1], h0 = hi[2 * hh], h1 = hi[2 * hh + 1];
    const float a0 = bf_lo(l0), a1 = bf_hi(l0), a2 = bf_lo(l1), a3 = bf_hi(l1);
    const float b0 = bf_lo(h0), b1 = bf_hi(h0), b2 = bf_lo(h1), b3 = bf_hi(h1);
    lo[2 * hh] = pack2(fmaf(a0, c[0], -b0 * s[0]), fmaf(a1, c[1], -b1 * s[1]));
    lo[2 * hh + 1] = pack2(fmaf(a2, c[2], -b2 * s[2]), fmaf(a3, c[3], -b3 * s[3]));
    hi[2 * hh] = pack2(fmaf(a0, s[0], b0 * c[0]), fmaf(a1, s[1], b1 * c[1]));
    hi[2 * hh + 1] = pack2(fmaf(a2, s[2], b2 * c[2]), fmaf(a3, s[3], b3 * c[3]));
}

__device__ __forceinline__ int xcd_remap(int bid, int n) {
    const int X = 8;
    const int xcd = bid % X, idx = bid / X;
    const int q = n / X, rem = n % X;
    return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

// One 32-key step's operands for one lane (cos/sin are fetched at use).
template <int D>
struct Step {
    static constexpr int NC = D / 32;
    u32x4 k[2][NC];      // A operand rows (before rotation), tiles T = 0, 1
    int32_t kpi[2];      // pi of the A row keys (-1 unusable)
    u32x4 v[D / 16];     // V^T operand, channel 16*dt + lc, keys 8lg..8lg+7
    int32_t spi[8];      // pi of this lane's 8 score keys (-1 unusable)
};

// Unconditional loads at clamped indices (key_end >= 1; kv_stride, a multiple
// of 16, bounds every index), then selects: unusable keys read the zero page.
template <int D>
__device__ __forceinline__ void step_load(const DecodeParams &p, Step<D> &st, const int32_t *bt,
                                          const int32_t *pis, int g, int kb, int key_end, int lc, int lg) {
    constexpr int NC = D / 32;
    const int last = key_end - 1;
#pragma unroll
    for (int T = 0; T < 2; ++T) {
        const int j = kb + 8 * (lc >> 2) + 4 * T + (lc & 3);
        const int jc = min(j, last);
        const int blk = bt[jc >> 4], pi = pis[jc];
        const bool ok = j < key_end && (unsigned)blk < (unsigned)p.num_blocks && (unsigned)pi < (unsigned)p.max_pos;
        st.kpi[T] = ok ? pi : -1;
        const uint16_t *row = ok ? p.k_pool + (((size_t)blk * p.hkv + g) * kBlock + (j & 15)) * D : p.zero_page;
#pragma unroll
        for (int c = 0; c < NC; ++c) st.k[T][c] = *reinterpret_cast<const u32x4 *>(row + 32 * c + 8 * lg);
    }
    const int j0 = kb + 8 * lg;                 // multiple of 8
    const int j0c = min(j0, last & ~7);         // 8 positions from here stay inside the row
    const int blk = bt[j0c >> 4];
    const bool bok = j0 < key_end && (unsigned)blk < (unsigned)p.num_blocks;
    const i32x4 a = *reinterpret_cast<const i32x4 *>(pis + j0c);
    const i32x4 b = *reinterpret_cast<const i32x4 *>(pis + j0c + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        st.spi[i] = (bok && j0 + i < key_end && (unsigned)a[i] < (unsigned)p.max_pos) ? a[i] : -1;
        st.spi[4 + i] = (bok && j0 + 4 + i < key_end && (unsigned)b[i] < (unsigned)p.max_pos) ? b[i] : -1;
    }
    const uint16_t *vb = bok ? p.v_pool + ((size_t)blk * p.hkv + g) * D * kBlock + (j0 & 15) : p.zero_page;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        st.v[dt] = *reinterpret_cast<const u32x4 *>(vb + (size_t)(16 * dt + lc) * kBlock);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(DecodeParams p) {
    constexpr int NC = D / 32, HALF = D / 2, NQ = HALF / 4;
    // R(dl) for dl = 0..15, laid out [frequency quad][dl]: the 16 lanes of a
    // lane group read one 256-byte block
    __shared__ f32x4 s_dc[NQ][16], s_ds[NQ][16];
    __shared__ float s_o[kWaves][D][16];
    __shared__ float s_m[kWaves][16], s_l[kWaves][16];

    const int nwg = p.hkv * p.num_splits * p.batch;
    int lid = xcd_remap(blockIdx.x, nwg);
    const int g = lid % p.hkv;
    lid /= p.hkv;
    const int sp = lid % p.num_splits;
    const int r = lid / p.num_splits;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lc = lane & 15, lg = lane >> 4;
    for (int t = tid; t < NQ * 16; t += kThreads) {
        const int dl = t & 15, q4 = t >> 4;
        const bool in = dl < p.max_pos;
        s_dc[q4][dl] = in ? *reinterpret_cast<const f32x4 *>(p.cos_tab + dl * HALF + 4 * q4) : f32x4{1.f, 1.f, 1.f, 1.f};
        s_ds[q4][dl] = in ? *reinterpret_cast<const f32x4 *>(p.sin_tab + dl * HALF + 4 * q4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int kv_stride = p.max_blocks * kBlock;
    const int kv_cap = min(kv_stride, p.max_kv_len);
    int kvl = p.kv_len[r];
    kvl = kvl < 0 ? 0 : (kvl > kv_cap ? kv_cap : kvl);
    const int wave_keys = p.split_len / kWaves;
    const int wbeg = sp * p.split_len + wave * wave_keys;
    const int key_end = min(kvl, wbeg + wave_keys);
    const int32_t *bt = p.block_table + (size_t)r * p.max_blocks;
    const int32_t *pis = p.kv_pos + (size_t)r * kv_stride;

    // query column lc: head g*G + lc of request r (branch-free: columns past
    // G and invalid positions rotate a clamped row and are zeroed)
    const bool qv = lc < p.group;
    const int h = g * p.group + (qv ? lc : 0);
    int pos = qv ? p.q_pos[r] : -1;
    if (pos >= p.max_pos) pos = -1;
    const int posc = pos >= 0 ? pos : 0;
    u32x4 qop[NC];
    {
        const uint16_t *src = p.q + ((size_t)r * p.hq + h) * D;
#pragma unroll
        for (int c = 0; c < NC / 2; ++c) {
            const int i0 = 32 * c + 8 * lg;
            u32x4 lo = *reinterpret_cast<const u32x4 *>(src + i0);
            u32x4 hi = *reinterpret_cast<const u32x4 *>(src + HALF + i0);
            const float *cr = p.cos_tab + (size_t)posc * HALF + i0;
            const float *sr = p.sin_tab + (size_t)posc * HALF + i0;
            rope4<0>(lo, hi, *reinterpret_cast<const f32x4 *>(cr), *reinterpret_cast<const f32x4 *>(sr));
            rope4<1>(lo, hi, *reinterpret_cast<const f32x4 *>(cr + 4), *reinterpret_cast<const f32x4 *>(sr + 4));
            const u32x4 z = {0u, 0u, 0u, 0u};
            qop[c] = pos >= 0 ? lo : z;
            qop[c + NC / 2] = pos >= 0 ? hi : z;
        }
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();   // R(dl) table

    // wave-uniform step count (the compiler cannot tell on its own)
    const int nsteps = __builtin_amdgcn_readfirstlane(key_end > wbeg ? (key_end - wbeg + 31) / 32 : 0);
    auto process = [&](Step<D> &cur) {
        f32x4 sacc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            // key offset inside its block (the step start is a multiple of 32)
            const int off = (8 * (lc >> 2) + 4 * T + (lc & 3)) & 15;
            const int pi = cur.kpi[T];
            const int dl = pi >= 0 ? min(off, pi) : 0;
            const int row = pi >= 0 ? pi - dl : 0;
            const float *cr = p.cos_tab + (size_t)row * HALF;
            const float *sr = p.sin_tab + (size_t)row * HALF;
            // cos/sin of 4 frequencies i0..i0+3 at pi: R(pi - dl) R(dl)
            auto rot = [&](int i0, f32x4 &cc, f32x4 &ss) {
                const f32x4 cp = *reinterpret_cast<const f32x4 *>(cr + i0);
                const f32x4 sn = *reinterpret_cast<const f32x4 *>(sr + i0);
                const f32x4 cd = s_dc[i0 >> 2][dl], sd = s_ds[i0 >> 2][dl];
                cc = cp * cd - sn * sd;
                ss = sn * cd + cp * sd;
            };
            if (p.rotate_k) {   // else the keys are stored rotated (ablation mode)
#pragma unroll
                for (int c = 0; c < NC / 2; ++c) {
                    f32x4 c0, s0, c1, s1;
                    rot(32 * c + 8 * lg, c0, s0);
                    rot(32 * c + 8 * lg + 4, c1, s1);
                    rope4<0>(cur.k[T][c], cur.k[T][c + NC / 2], c0, s0);
                    rope4<1>(cur.k[T][c], cur.k[T][c + NC / 2], c1, s1);
                }
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
        if (__any(any_bad)) {
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t w = cur.v[dt][e];
                    if (cur.spi[2 * e] < 0) w &= 0xffff0000u;
                    if (cur.spi[2 * e + 1] < 0) w &= 0x0000ffffu;
                    cur.v[dt][e] = w;
                }
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) acc[dt] = mfma16(cur.v[dt], pb, acc[dt] * alpha);
    };
    // two step buffers in turn; the step after the range is requested too
    // (clamped indices, zero page) so that no branch guards the requests
    Step<D> sa, sb;
    if (nsteps > 0) step_load<D>(p, sa, bt, pis, g, wbeg, key_end, lc, lg);
    for (int it = 0; it < nsteps; it += 2) {
        step_load<D>(p, sb, bt, pis, g, wbeg + 32 * (it + 1), key_end, lc, lg);
        process(sa);
        if (it + 1 >= nsteps) break;
        step_load<D>(p, sa, bt, pis, g, wbeg + 32 * (it + 2), key_end, lc, lg);
        process(sb);
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
    // thread -> (column, D/16 channels)
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
