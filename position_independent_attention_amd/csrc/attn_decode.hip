// Decode (one query token per request) over the paged, unrotated KV cache,
// with RoPE applied in-kernel at each key's logical position (MiniPIC,
// gist.science 2606.13126, section 2.1 score equation).
//
// Bound by HBM bytes: every cached key and value is read once per
// (request, kv head) and feeds only G = Hq/Hkv query rows.  So there is no
// LDS staging of K/V: each wave walks its range one pool block (16 keys) at a
// time, loading the block's keys and values straight into MFMA operand
// registers.  Scores are S^T = K Q^T (16x16x32 bf16, the G query heads are
// the MFMA columns, columns >= G are masked); the S^T accumulator layout is
// exactly the B operand of the 16x16x16 bf16 MFMA, so O^T += V^T P^T takes
// the probabilities without any data movement, and V^T comes 8 bytes per
// lane from the block's channel-major value layout.
//
// Rotation of key j at position pi: when the usable keys of a block sit at
// pi = base + offset (the usual case, also for a span reused at another
// offset), R(pi) = R(base) R(offset); the block's base cos/sin row (512 bytes
// at d = 128) is requested with the block and passed through LDS, and R(o)
// for o = 0..15 sits in LDS for the whole kernel.  Any other block computes
// each key's cos/sin from its angle (fp64 reduction to one revolution, then
// the hardware sin/cos), so that it needs no memory request at all.
// Positions are requested two blocks ahead, so a block's path and base row
// are known when its keys are requested, and every load of a block is issued
// before the previous block's math (memory requests retire in order, so a
// load issued later would also wait for the prefetch).
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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

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
__device__ __forceinline__ f32x4 mfma_k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}
constexpr float kSlack = 8.f;
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

// Positions of one 16-key step (one pool block), requested two steps ahead.
struct Pos {
    i32x4 a;        // pi of keys 4lg .. 4lg+3 (raw)
    int32_t x;      // pi of key lc (raw)
    int32_t blk;    // pool block id (raw, uniform)
};

// One 16-key step's operands for one lane, requested one step ahead.
template <int D>
struct Step {
    static constexpr int NC = D / 32;
    u32x4 k[NC];        // S^T A operand: key lc, channels 32c + 8lg .. +7 (before rotation)
    u32x2 v[D / 16];    // O^T A operand: channel 16dt + lc, keys 4lg .. 4lg+3
    f32x2 row;          // two entries of the cos (lanes of even half-groups) or sin row at the block base
    int32_t spi[4];     // pi of keys 4lg .. 4lg+3 (-1 unusable)
    int32_t kpi;        // pi of key lc (-1 unusable)
    int32_t fast;       // every usable key of the block sits at pi = base + offset
};

// kb is a multiple of 16 and wave-uniform; lastb = (key_end - 1) & ~15 bounds
// every index (kv_stride is a multiple of 16), so the loads need no branch.
__device__ __forceinline__ void pos_load(Pos &q, const int32_t *bt, const int32_t *pis, int kb, int lastb, int lc,
                                         int lg) {
    const int kbc = min(kb, lastb);
    q.a = *reinterpret_cast<const i32x4 *>(pis + kbc + 4 * lg);
    q.x = pis[kbc + lc];
    q.blk = bt[kbc >> 4];
}

// Validate a step's positions, pick its rotation path and request its K, V
// and base cos/sin row.  Unusable blocks read the zero page.
template <int D>
__device__ __forceinline__ void step_issue(const DecodeParams &p, Step<D> &st, const Pos &q, int g, int kb,
                                           int key_end, int lane, int lc, int lg) {
    constexpr int NC = D / 32, HALF = D / 2;
    const int blk = __builtin_amdgcn_readfirstlane(q.blk);
    const bool bok = (unsigned)blk < (unsigned)p.num_blocks;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        st.spi[i] = (bok && kb + 4 * lg + i < key_end && (unsigned)q.a[i] < (unsigned)p.max_pos) ? q.a[i] : -1;
    st.kpi = (bok && kb + lc < key_end && (unsigned)q.x < (unsigned)p.max_pos) ? q.x : -1;
    // base = pi - offset, the same for every usable key of the block?
    const bool use = st.kpi >= 0;
    const int cand = st.kpi - lc;
    const uint64_t um = __ballot(use);
    int base = 0, fast = 1;
    if (um) {
        base = __builtin_amdgcn_readlane(cand, (int)__builtin_ctzll(um));
        fast = base >= 0 && __ballot(use && cand != base) == 0;
    }
    st.fast = fast;
    const int rb = fast ? base : 0;
    const float *tab = ((lane / (HALF / 2)) & 1) ? p.sin_tab : p.cos_tab;
    st.row = *reinterpret_cast<const f32x2 *>(tab + (size_t)rb * HALF + 2 * (lane % (HALF / 2)));
    const uint16_t *kr = bok ? p.k_pool + (((size_t)blk * p.hkv + g) * kBlock + lc) * D : p.zero_page;
#pragma unroll
    for (int c = 0; c < NC; ++c) st.k[c] = *reinterpret_cast<const u32x4 *>(kr + 32 * c + 8 * lg);
    const uint16_t *vb = bok ? p.v_pool + ((size_t)blk * p.hkv + g) * D * kBlock : p.zero_page;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        st.v[dt] = *reinterpret_cast<const u32x2 *>(vb + (size_t)(16 * dt + lc) * kBlock + 4 * lg);
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_kernel(DecodeParams p) {
    constexpr int NC = D / 32, HALF = D / 2, NQ = HALF / 4;
    // R(o) for block offsets o = 0..15, laid out [frequency quad][o]: the 16
    // lanes of a lane group read one 256-byte block
    __shared__ f32x4 s_dc[NQ][16], s_ds[NQ][16];
    // each wave's current block-base row: cos, then sin
    __shared__ f32x4 s_row[kWaves][2][NQ];
    // revolutions per position of each frequency, theta^(-2i/d) / (2 pi)
    __shared__ double s_rf[HALF];
    __shared__ float s_o[kWaves][D][16];
    __shared__ float s_m[kWaves][16], s_l[kWaves][16];

    const int nwg = p.hkv * p.num_splits * p.batch;
    int lid = xcd_remap(blockIdx.x, nwg);
    const int g = lid % p.hkv;
    lid /= p.hkv;
    const int sp = lid % p.num_splits;
    const int r = lid / p.num_splits;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lc = lane & 15, lg = lane >> 4;
    for (int t = tid; t < HALF; t += kThreads) s_rf[t] = p.rev_freq[t];
    for (int t = tid; t < NQ * 16; t += kThreads) {
        const int o = t & 15, q4 = t >> 4;
        const bool in = o < p.max_pos;
        s_dc[q4][o] = in ? *reinterpret_cast<const f32x4 *>(p.cos_tab + o * HALF + 4 * q4) : f32x4{1.f, 1.f, 1.f, 1.f};
        s_ds[q4][o] = in ? *reinterpret_cast<const f32x4 *>(p.sin_tab + o * HALF + 4 * q4) : f32x4{0.f, 0.f, 0.f, 0.f};
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

    // running max: a per-column reference raised only when a score passes it
    // by more than kSlack (log2 units), so most steps skip the rescale
    float m_ref = -1e30f, l_run = 0.f;
    f32x4 acc[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();   // R(o) and revolution tables

    auto process = [&](Step<D> &st) {
        if (p.rotate_k) {   // else the keys are stored rotated (ablation mode)
            if (st.fast) {
                // R(base + lc) = R(base) R(lc): the base row goes through the
                // wave's LDS slot, R(lc) comes from the shared table
                if (lane < HALF)
                    *reinterpret_cast<f32x2 *>(reinterpret_cast<float *>(&s_row[wave][0][0]) +
                                               ((lane / (HALF / 2)) & 1) * HALF + 2 * (lane % (HALF / 2))) = st.row;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int c = 0; c < NC / 2; ++c) {
                    const int q0 = 8 * c + 2 * lg;
                    const f32x4 cb0 = s_row[wave][0][q0], sb0 = s_row[wave][1][q0];
                    const f32x4 cb1 = s_row[wave][0][q0 + 1], sb1 = s_row[wave][1][q0 + 1];
                    const f32x4 co0 = s_dc[q0][lc], so0 = s_ds[q0][lc];
                    const f32x4 co1 = s_dc[q0 + 1][lc], so1 = s_ds[q0 + 1][lc];
                    rope4<0>(st.k[c], st.k[c + NC / 2], cb0 * co0 - sb0 * so0, sb0 * co0 + cb0 * so0);
                    rope4<1>(st.k[c], st.k[c + NC / 2], cb1 * co1 - sb1 * so1, sb1 * co1 + cb1 * so1);
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
            } else {
                // positions that do not follow the block offsets: cos/sin of
                // each key's own angle, computed here rather than read from
                // the table (a table read issued now would also wait for the
                // next step's requests): pi * theta_i / (2 pi) in fp64, its
                // fractional part, then the hardware sin/cos of a fraction of
                // a revolution
                const double pd = (double)(st.kpi >= 0 ? st.kpi : 0);
                auto angle_cs = [&](int f0, f32x4 &cc, f32x4 &ss) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        double rv = pd * s_rf[f0 + e];
                        rv -= __builtin_rint(rv);
                        const float r = (float)rv;
                        cc[e] = __builtin_amdgcn_cosf(r);
                        ss[e] = __builtin_amdgcn_sinf(r);
                    }
                };
#pragma unroll
                for (int c = 0; c < NC / 2; ++c) {
                    f32x4 c0, s0, c1, s1;
                    angle_cs(32 * c + 8 * lg, c0, s0);
                    angle_cs(32 * c + 8 * lg + 4, c1, s1);
                    rope4<0>(st.k[c], st.k[c + NC / 2], c0, s0);
                    rope4<1>(st.k[c], st.k[c + NC / 2], c1, s1);
                }
            }
        }
        f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) sacc = mfma16(st.k[c], qop[c], sacc);
        // lane holds keys 4lg .. 4lg+3 of column lc
        float sv[4];
        float mx = -INFINITY;
        bool any_bad = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int kp = st.spi[e];
            const bool vis = kp >= 0 && kp <= pos;
            any_bad |= kp < 0;
            sv[e] = vis ? sacc[e] * p.scale_log2 : -INFINITY;
            mx = fmaxf(mx, sv[e]);
        }
        if (__any(mx > m_ref + kSlack)) {
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_ref, mx);
            const float alpha = fast_exp2(m_ref - m_new);
            m_ref = m_new;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) acc[dt] *= alpha;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sv[e] = fast_exp2(sv[e] - m_ref);
            l_run += sv[e];
        }
        const u32x2 pb = {pack2(sv[0], sv[1]), pack2(sv[2], sv[3])};
        // any unusable key in the step: zero its V entries so that
        // 0 * garbage cannot poison O
        if (__any(any_bad)) {
            const uint32_t m0 = (st.spi[0] < 0 ? 0u : 0xffffu) | (st.spi[1] < 0 ? 0u : 0xffff0000u);
            const uint32_t m1 = (st.spi[2] < 0 ? 0u : 0xffffu) | (st.spi[3] < 0 ? 0u : 0xffff0000u);
#pragma unroll
            for (int dt = 0; dt < D / 16; ++dt) {
                st.v[dt][0] &= m0;
                st.v[dt][1] &= m1;
            }
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) acc[dt] = mfma_k16(st.v[dt], pb, acc[dt]);
    };

    // Positions run two steps ahead of K/V so that a step's rotation path and
    // base row are known when its K/V are requested; everything a step needs
    // is then requested before the previous step's math.  The steps after the
    // range are requested too (clamped, all keys unusable), so no branch
    // guards the requests.
    const int nsteps = __builtin_amdgcn_readfirstlane(key_end > wbeg ? (key_end - wbeg + 15) / 16 : 0);
    if (nsteps > 0) {
        const int wb = __builtin_amdgcn_readfirstlane(wbeg);
        const int lastb = __builtin_amdgcn_readfirstlane((key_end - 1) & ~15);
        Pos pe, po;
        Step<D> sa, sb;
        pos_load(pe, bt, pis, wb, lastb, lc, lg);
        pos_load(po, bt, pis, wb + 16, lastb, lc, lg);
        step_issue<D>(p, sa, pe, g, wb, key_end, lane, lc, lg);
        for (int it = 0; it < nsteps; it += 2) {
            pos_load(pe, bt, pis, wb + 16 * (it + 2), lastb, lc, lg);
            step_issue<D>(p, sb, po, g, wb + 16 * (it + 1), key_end, lane, lc, lg);
            process(sa);
            if (it + 1 >= nsteps) break;
            pos_load(po, bt, pis, wb + 16 * (it + 3), lastb, lc, lg);
            step_issue<D>(p, sa, pe, g, wb + 16 * (it + 2), key_end, lane, lc, lg);
            process(sb);
        }
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
        s_m[wave][lc] = lt > 0.f ? m_ref : -INFINITY;
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

hipError_t launch_decode(const DecodeParams &p, int head_dim, hipStream_t s, KernelEvents ev) {
    const int nwg = p.hkv * p.num_splits * p.batch;
    if (nwg <= 0) return hipSuccess;
    auto k = head_dim == 64 ? decode_kernel<64> : decode_kernel<128>;
    if (ev.start)
        hipExtLaunchKernelGGL(k, dim3(nwg), dim3(kThreads), 0, s, ev.start, ev.stop, 0, p);
    else
        hipLaunchKernelGGL(k, dim3(nwg), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace pic
