// Internal declarations of the gfx950 library: launch parameter blocks and the
// host-side launchers implemented in the kernel translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pic {

constexpr int kBlock = 16;        // tokens per pool block
constexpr int kTileN = 64;            // keys per staged tile in the prefill-style kernels
constexpr int kMergeMaxSplits = 4096;  // splits the many-split merge stages in LDS
constexpr int kThreads = 256;     // 4 wave64 per workgroup
constexpr int kWaves = 4;

enum Mode : int { kAttn = 0, kLse = 1, kMass = 2 };

// Everything one prefill-style launch needs.  Pointers are device pointers.
struct FwdParams {
    const uint16_t *zero_page;  // >= 16*d zero bf16, read in place of unusable keys
    const uint16_t *k_pool;
    const uint16_t *v_pool;
    int32_t num_blocks;
    const int32_t *block_table;
    const int32_t *kv_len;
    const int32_t *kv_pos;
    int32_t max_blocks;
    const uint16_t *q;
    const int32_t *q_start;   // [B+1]
    const int32_t *q_pos;     // [total_q]
    int32_t batch, total_q;
    int32_t hq, hkv, group;
    const float *cos_tab;     // [max_pos][d/2]
    const float *sin_tab;
    int32_t rotate_k;         // 0: keys are stored rotated (ablation mode)
    int32_t max_pos;
    float scale_log2;         // log2(e) / sqrt(d)
    int32_t max_kv_len;       // host bound on kv_len (clamps every key range)
    int32_t split_len;        // keys per split, multiple of kTileN
    int32_t num_splits;
    int32_t row_blocks;       // workgroups along the packed (token, head) rows
    // outputs
    uint16_t *out;            // [total_q][hq][d] bf16 (num_splits == 1)
    float *lse;               // [total_q][hq] natural log, nullable
    float *part_o;            // [num_splits][total_q][hq][d]
    float *part_ml;           // [num_splits][total_q][hq][2] (max in log2 units, sum)
    // selection mass
    const float *lse_in;      // [total_q][hq] natural log
    float *mass_part;         // [B][hkv][row_blocks][mass_stride]
    int32_t mass_stride;
};

struct DecodeParams {
    const uint16_t *zero_page;
    const uint16_t *k_pool;
    const uint16_t *v_pool;
    int32_t num_blocks;
    const int32_t *block_table;
    const int32_t *kv_len;
    const int32_t *kv_pos;
    int32_t max_blocks;
    const uint16_t *q;        // [B][hq][d]
    const int32_t *q_pos;     // [B]
    int32_t batch;
    int32_t hq, hkv, group;
    const float *cos_tab;
    const float *sin_tab;
    const double *rev_freq;   // [d/2] theta^(-2i/d) / (2 pi): revolutions per position
    int32_t rotate_k;         // 0: keys are stored rotated (ablation mode)
    int32_t max_pos;
    float scale_log2;
    int32_t max_kv_len;
    int32_t split_len;        // keys per workgroup, a multiple of 4 * 32
    int32_t num_splits;
    uint16_t *out;
    float *lse;
    float *part_o;            // [num_splits][B][hq][d]
    float *part_ml;           // [num_splits][B][hq][2]
};

struct MergeParams {
    const float *part_o;      // may be null (lse-only partials)
    const float *part_ml;
    int32_t num_splits;
    int32_t rows;             // total_q * hq
    uint16_t *out;            // nullable
    float *lse;               // nullable
};

struct SelectParams {
    const float *mass_part;   // [B][hkv][row_blocks][mass_stride]
    int32_t hkv, row_blocks, mass_stride;
    const int32_t *q_start;
    int32_t group, rows_per_block;
    const int32_t *kv_len;
    const int32_t *kv_pos;
    int32_t kv_stride;        // max_blocks * 16
    int32_t batch;
    float *mass;              // [B][kv_stride]
    const int32_t *span_req, *span_start, *span_len, *sel_off;
    int32_t n_spans;
    int32_t *sel_idx;
    int32_t max_sel;          // capacity of sel_idx (host value)
};

// Anchor key norms (QCFuse anchor extraction).
struct NormParams {
    const uint16_t *k_pool;
    int32_t num_blocks, hkv;
    const int32_t *block_table;
    const int32_t *kv_len;
    const int32_t *kv_pos;
    int32_t max_blocks, max_pos;
    int32_t batch;
    float *norm;              // [B][max_blocks * 16]
};

struct FuseParams {
    uint16_t *k_pool;
    uint16_t *v_pool;
    int32_t num_blocks, hkv;
    const int32_t *block_table;
    int32_t *kv_len;
    int32_t *kv_pos;
    int32_t max_blocks;
    const int32_t *sel_idx;
    const int32_t *sel_req_off;
    const uint16_t *k_new;
    const uint16_t *v_new;
    int32_t batch;
    int32_t max_rows;         // bound of rows per request
    int32_t n_sel;            // rows in k_new / v_new / sel_idx
};

// Kernel timing: when `start` is set, the main kernel of a launcher is
// launched with hipExtLaunchKernelGGL, which stamps the two events with the
// kernel's own start and end.
struct KernelEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};

// Launchers (return the launch's hipError_t).
// shape 0: 64 rows per workgroup; shape 1: 256 rows (d = 128) / 128 rows (d = 64);
// shape 2: shape 1 skipping the tiles that no row of a workgroup sees; shape 4
// (LSE mode at d = 128 only): 4 row tiles per wave, 512 rows
int fwd_rows_per_block(int head_dim, int shape);
// rows per workgroup of the mass pass at shape >= 1: 4 row tiles per wave, or
// 2 at shape 3 (d = 128 only)
int mass_rows_per_block(int head_dim, int shape);
hipError_t launch_fwd(const FwdParams &p, int head_dim, int mode, int shape, hipStream_t s,
                      KernelEvents ev = KernelEvents{});
hipError_t launch_decode(const DecodeParams &p, int head_dim, hipStream_t s, KernelEvents ev = KernelEvents{});
hipError_t launch_merge(const MergeParams &p, int head_dim, hipStream_t s);
hipError_t launch_mass_reduce(const SelectParams &p, hipStream_t s);
hipError_t launch_topk(const SelectParams &p, hipStream_t s);
hipError_t launch_key_norm(const NormParams &p, int head_dim, hipStream_t s);
hipError_t launch_fuse(const FuseParams &p, int head_dim, hipStream_t s);

}  // namespace pic
