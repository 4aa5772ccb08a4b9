// Host side of the C ABI declared in include/pic_attn.h: context and RoPE
// table, argument validation, launch planning, workspace carving and the
// launches of the gfx950 kernels.  No entry point allocates device memory
// except pic_ctx_create (pic_timing_start creates HIP events); no entry
// point synchronises the stream except pic_timing_stop.
#include "pic_attn.h"
#include "pic_internal.h"

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

// Device scratch of qc_score_select_noalloc: one copy per GPU, held until the
// process ends.  Host code never uses this name as an address (on the host it
// is only a handle of the symbol); it uses the per-device address that
// hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[PIC_NOALLOC_SCRATCH_BYTES];

struct pic_ctx {
    int device = 0;
    pic_config cfg{};
    float *cos_d = nullptr;
    float *sin_d = nullptr;
    double *rev_d = nullptr;      // [d/2] theta^(-2i/d) / (2 pi): revolutions per position
    uint16_t *zero_d = nullptr;   // zero page read in place of unusable keys
    void *scratch_d = nullptr;    // this device's address of `scratch`
    std::string err;
    // kernel timing (pic_timing_start / pic_timing_stop): event pairs in call order
    bool timing = false;
    std::vector<hipEvent_t> tev;  // 2 * capacity
    std::vector<int32_t> top;     // op of each recorded interval
};

namespace {

using pic::kBlock;

constexpr size_t kAlign = 256;
constexpr int kCUs = 256;   // compute units of an MI355X

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

pic_status fail(pic_ctx *ctx, pic_status s, const char *fmt, const char *detail = "") {
    if (ctx) {
        char buf[512];
        std::snprintf(buf, sizeof buf, fmt, detail);
        ctx->err = buf;
    }
    return s;
}

pic_status hip_fail(pic_ctx *ctx, hipError_t e, const char *where) {
    if (ctx) ctx->err = std::string(where) + ": " + hipGetErrorString(e);
    return PIC_ERR_HIP;
}

// Launch geometry of the prefill-style kernels.
struct FwdPlan {
    int shape = 0;        // kernel variant (0, 1, 2: 1 with tile skipping), see pic::launch_fwd
    int rows_per_block = 64;
    int row_blocks = 0;
    int split_len = pic::kTileN;
    int num_splits = 1;
};

// Splits of the key range so that base workgroups x splits fill the GPU.
void set_splits(FwdPlan &pl, const pic_config &c, int batch, int max_kv_len) {
    const long long base = (long long)pl.row_blocks * c.num_kv_heads * batch;
    // the big shape runs one 512-thread workgroup per CU, the small one several
    const long long target = pl.shape >= 1 && c.head_dim == 128 ? kCUs : 2 * kCUs;
    int splits = 1;
    if (base > 0 && max_kv_len > 0) {
        const long long want = (target + base - 1) / base;
        const long long cap = std::max(1, (max_kv_len + 255) / 256);   // >= 4 tiles per split
        splits = (int)std::max(1LL, std::min(want, cap));
    }
    const int per = max_kv_len > 0 ? (max_kv_len + splits - 1) / splits : pic::kTileN;
    pl.split_len = std::max(pic::kTileN, (per + pic::kTileN - 1) / pic::kTileN * pic::kTileN);
    pl.num_splits = max_kv_len > 0 ? (max_kv_len + pl.split_len - 1) / pl.split_len : 1;
}

FwdPlan plan_fwd(const pic_config &c, int batch, int max_q_len, int max_kv_len) {
    FwdPlan pl;
    const int G = c.num_q_heads / c.num_kv_heads;
    const long long rows = (long long)max_q_len * G;
    pl.shape = rows >= 128 ? 1 : 0;
    pl.rows_per_block = pic::fwd_rows_per_block(c.head_dim, pl.shape);
    pl.row_blocks = (int)((rows + pl.rows_per_block - 1) / pl.rows_per_block);
    // many row blocks hold queries at many different positions: take the
    // variant that skips the tiles no row of a workgroup sees
    if (pl.shape == 1 && pl.row_blocks >= 8) pl.shape = 2;
    set_splits(pl, c, batch, max_kv_len);
    return pl;
}

// The selection's own LSE pass (lse == NULL): it keeps no O accumulator, so
// at d = 128 a request with more than 256 rows per kv head takes 4 row tiles
// per wave (shape 4, 512-row workgroups) unless it has the many row blocks of
// the tile-skipping variant.  Up to 256 rows a 512-row workgroup would leave
// half its waves on rows that do not exist.
FwdPlan plan_lse(const pic_config &c, int batch, int max_q_len, int max_kv_len) {
    FwdPlan pl = plan_fwd(c, batch, max_q_len, max_kv_len);
    const long long rows = (long long)max_q_len * (c.num_q_heads / c.num_kv_heads);
    if (pl.shape != 1 || c.head_dim != 128 || rows <= 256) return pl;
    pl.shape = 4;
    pl.rows_per_block = pic::fwd_rows_per_block(c.head_dim, 4);
    pl.row_blocks = (int)((rows + pl.rows_per_block - 1) / pl.rows_per_block);
    set_splits(pl, c, batch, max_kv_len);
    return pl;
}

// The selection mass pass: at shape >= 1 its workgroups hold twice the rows
// (4 row tiles per wave: it keeps no O accumulator), and it never skips
// tiles.  At d = 128 a request of at most 256 rows per kv head takes 2 row
// tiles per wave (shape 3): a 512-row workgroup would leave half its waves
// computing rows that do not exist.
FwdPlan plan_mass(const pic_config &c, int batch, int max_q_len, int max_kv_len) {
    FwdPlan pl = plan_fwd(c, batch, max_q_len, max_kv_len);
    if (pl.shape == 0) return pl;
    const long long rows = (long long)max_q_len * (c.num_q_heads / c.num_kv_heads);
    pl.shape = c.head_dim == 128 && rows <= 256 ? 3 : 1;
    pl.rows_per_block = pic::mass_rows_per_block(c.head_dim, pl.shape);
    pl.row_blocks = (int)((rows + pl.rows_per_block - 1) / pl.rows_per_block);
    set_splits(pl, c, batch, max_kv_len);
    return pl;
}

// Decode: about four 256-thread workgroups per CU in total (or one resident
// round when that would leave a second round mostly idle), each covering
// split_len keys (a multiple of 4 waves x 32 keys, at least 512) of one
// (request, kv head).
struct DecodePlan {
    int split_len = 512;
    int num_splits = 1;
};

DecodePlan plan_decode(int batch, int hkv, int max_kv_len) {
    DecodePlan d;
    if (max_kv_len <= 0 || batch <= 0) return d;
    const long long rows = (long long)batch * hkv;
    const long long per = (rows * max_kv_len + 4LL * kCUs - 1) / (4LL * kCUs);
    long long len = (per + 127) / 128 * 128;
    len = std::max(512LL, std::min(len, ((long long)max_kv_len + 127) / 128 * 128));
    // Two workgroups per CU are resident at once.  A plan that overflows one
    // such round by less than a whole round would leave its second round
    // mostly idle: take one round of longer splits instead.
    const long long resident = 2LL * kCUs;
    const long long nwg = rows * ((max_kv_len + len - 1) / len);
    if (nwg > resident && nwg < 2 * resident) {
        const long long per_row = std::max(1LL, resident / rows);
        len = ((max_kv_len + per_row - 1) / per_row + 127) / 128 * 128;
        len = std::max(512LL, len);
    }
    d.split_len = (int)len;
    d.num_splits = (int)((max_kv_len + len - 1) / len);
    return d;
}

// Workspace layouts (byte offsets, 256-aligned).
struct PrefillWs {
    size_t part_o = 0, part_ml = 0, total = 0;
};
PrefillWs prefill_ws(const pic_config &c, const FwdPlan &pl, int total_q) {
    PrefillWs w;
    if (pl.num_splits > 1) {
        const size_t rows = (size_t)total_q * c.num_q_heads;
        w.part_o = 0;
        w.part_ml = align_up((size_t)pl.num_splits * rows * c.head_dim * sizeof(float));
        w.total = w.part_ml + align_up((size_t)pl.num_splits * rows * 2 * sizeof(float));
    }
    return w;
}

struct DecodeWs {
    size_t part_o = 0, part_ml = 0, total = 0;
};
DecodeWs decode_ws(const pic_config &c, int batch, int splits) {
    DecodeWs w;
    if (splits > 1) {
        const size_t rows = (size_t)batch * c.num_q_heads;
        w.part_ml = align_up((size_t)splits * rows * c.head_dim * sizeof(float));
        w.total = w.part_ml + align_up((size_t)splits * rows * 2 * sizeof(float));
    }
    return w;
}

struct SelectWs {
    size_t lse = 0, lse_ml = 0, mass_part = 0, mass = 0, total = 0;
};
SelectWs select_ws(const pic_config &c, const FwdPlan &pl, const FwdPlan &plm, int batch, int max_blocks,
                   int total_q, int max_kv_len) {
    SelectWs w;
    size_t off = 0;
    const size_t rows = (size_t)total_q * c.num_q_heads;
    w.lse = off;
    off += align_up(rows * sizeof(float));
    w.lse_ml = off;
    if (pl.num_splits > 1) off += align_up((size_t)pl.num_splits * rows * 2 * sizeof(float));
    w.mass_part = off;
    off += align_up((size_t)batch * c.num_kv_heads * plm.row_blocks * (size_t)max_kv_len * sizeof(float));
    w.mass = off;
    off += align_up((size_t)batch * max_blocks * kBlock * sizeof(float));
    w.total = off;
    return w;
}

pic_status check_ctx(const pic_ctx *ctx) { return ctx ? PIC_OK : PIC_ERR_INVALID_ARG; }

// Kernel timing: the next free event pair (if timing is on and the capacity
// holds another interval), stamped by the launch with the main kernel's own
// start and end; the interval counts once the launch has succeeded.
struct TimedSpan {
    pic_ctx *ctx;
    pic_op op;
    pic::KernelEvents ev;
    TimedSpan(pic_ctx *c, pic_op o) : ctx(c), op(o) {
        if (!ctx->timing || ctx->top.size() * 2 >= ctx->tev.size()) return;
        ev.start = ctx->tev[2 * ctx->top.size()];
        ev.stop = ctx->tev[2 * ctx->top.size() + 1];
    }
    void commit() {
        if (ev.start) ctx->top.push_back((int32_t)op);
    }
};

// Device address of `scratch` on the current device, looked up once per
// device (the lookup loads the library's code object there if needed).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(int device, void **out) {
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void *ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[device] = ptr;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

pic_status check_pool_req(pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req) {
    if (!pool || !req) return fail(ctx, PIC_ERR_INVALID_ARG, "pool or request table is NULL%s");
    if (!pool->k || !pool->v) return fail(ctx, PIC_ERR_INVALID_ARG, "pool k/v pointer is NULL%s");
    if (pool->num_blocks < 0) return fail(ctx, PIC_ERR_INVALID_ARG, "num_blocks < 0%s");
    if (req->batch < 0) return fail(ctx, PIC_ERR_INVALID_ARG, "batch < 0%s");
    if (req->max_blocks <= 0) return fail(ctx, PIC_ERR_INVALID_ARG, "max_blocks must be > 0%s");
    if (req->max_blocks > (1 << 26)) return fail(ctx, PIC_ERR_INVALID_ARG, "max_blocks too large%s");
    if (req->max_kv_len < 0 || (long long)req->max_kv_len > (long long)req->max_blocks * kBlock)
        return fail(ctx, PIC_ERR_INVALID_ARG, "max_kv_len outside [0, max_blocks*16]%s");
    if (req->batch > 0 && (!req->block_table || !req->kv_len || !req->kv_pos))
        return fail(ctx, PIC_ERR_INVALID_ARG, "block_table / kv_len / kv_pos is NULL%s");
    return PIC_OK;
}

pic_status check_queries(pic_ctx *ctx, const pic_queries *qs, int batch) {
    if (!qs) return fail(ctx, PIC_ERR_INVALID_ARG, "queries descriptor is NULL%s");
    if (qs->total_q < 0 || qs->max_q_len < 0)
        return fail(ctx, PIC_ERR_INVALID_ARG, "total_q / max_q_len < 0%s");
    if (qs->total_q > 0 && qs->max_q_len == 0)
        return fail(ctx, PIC_ERR_INVALID_ARG, "total_q > 0 but max_q_len == 0%s");
    if (qs->max_q_len > qs->total_q) return fail(ctx, PIC_ERR_INVALID_ARG, "max_q_len > total_q%s");
    if (batch > 0 && !qs->q_start) return fail(ctx, PIC_ERR_INVALID_ARG, "q_start is NULL%s");
    if (qs->total_q > 0 && (!qs->q || !qs->q_pos)) return fail(ctx, PIC_ERR_INVALID_ARG, "q / q_pos is NULL%s");
    return PIC_OK;
}

void fill_fwd_common(pic::FwdParams &p, const pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req,
                     const pic_queries *qs, const FwdPlan &pl) {
    const pic_config &c = ctx->cfg;
    std::memset(&p, 0, sizeof p);
    p.k_pool = pool->k;
    p.v_pool = pool->v;
    p.num_blocks = pool->num_blocks;
    p.block_table = req->block_table;
    p.kv_len = req->kv_len;
    p.kv_pos = req->kv_pos;
    p.max_blocks = req->max_blocks;
    p.q = qs->q;
    p.q_start = qs->q_start;
    p.q_pos = qs->q_pos;
    p.batch = req->batch;
    p.total_q = qs->total_q;
    p.hq = c.num_q_heads;
    p.hkv = c.num_kv_heads;
    p.group = c.num_q_heads / c.num_kv_heads;
    p.cos_tab = ctx->cos_d;
    p.sin_tab = ctx->sin_d;
    p.rotate_k = c.keys_prerotated ? 0 : 1;
    p.max_pos = c.max_position;
    p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
    p.max_kv_len = req->max_kv_len;
    p.split_len = pl.split_len;
    p.num_splits = pl.num_splits;
    p.row_blocks = pl.row_blocks;
    p.zero_page = ctx->zero_d;
}

}  // namespace

extern "C" {

const char *pic_status_str(pic_status s) {
    switch (s) {
    case PIC_OK: return "PIC_OK";
    case PIC_ERR_INVALID_ARG: return "PIC_ERR_INVALID_ARG";
    case PIC_ERR_UNSUPPORTED: return "PIC_ERR_UNSUPPORTED";
    case PIC_ERR_WORKSPACE: return "PIC_ERR_WORKSPACE";
    case PIC_ERR_HIP: return "PIC_ERR_HIP";
    }
    return "PIC_ERR_UNKNOWN";
}

const char *pic_ctx_last_error(const pic_ctx *ctx) { return ctx ? ctx->err.c_str() : ""; }

pic_status pic_ctx_create(const pic_config *cfg, pic_ctx **out) {
    if (!out) return PIC_ERR_INVALID_ARG;
    *out = nullptr;
    if (!cfg) return PIC_ERR_INVALID_ARG;
    if (cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0 || cfg->num_q_heads % cfg->num_kv_heads != 0)
        return PIC_ERR_INVALID_ARG;
    if (cfg->max_position <= 0 || cfg->max_position > (1 << 22)) return PIC_ERR_INVALID_ARG;
    if (!(cfg->rope_theta > 0.0) || !std::isfinite(cfg->rope_theta)) return PIC_ERR_INVALID_ARG;
    if (cfg->head_dim != 64 && cfg->head_dim != 128) return PIC_ERR_UNSUPPORTED;
    if (cfg->block_size != PIC_BLOCK_SIZE) return PIC_ERR_UNSUPPORTED;
    if (cfg->keys_prerotated != 0 && cfg->keys_prerotated != 1) return PIC_ERR_INVALID_ARG;

    pic_ctx *ctx = new (std::nothrow) pic_ctx;
    if (!ctx) return PIC_ERR_HIP;
    ctx->cfg = *cfg;
    if (hipGetDevice(&ctx->device) != hipSuccess) {
        delete ctx;
        return PIC_ERR_HIP;
    }
    // cos/sin(p * theta^(-2i/d)) in double, stored as fp32
    const int half = cfg->head_dim / 2;
    const size_t n = (size_t)cfg->max_position * half;
    std::vector<float> cs(n), sn(n);
    std::vector<double> inv(half);
    for (int i = 0; i < half; ++i) inv[i] = std::pow(cfg->rope_theta, -2.0 * i / cfg->head_dim);
    for (int p = 0; p < cfg->max_position; ++p)
        for (int i = 0; i < half; ++i) {
            const double a = (double)p * inv[i];
            cs[(size_t)p * half + i] = (float)std::cos(a);
            sn[(size_t)p * half + i] = (float)std::sin(a);
        }
    std::vector<double> rev(half);
    for (int i = 0; i < half; ++i) rev[i] = inv[i] / (2.0 * 3.14159265358979323846);
    hipError_t e = hipMalloc(&ctx->cos_d, n * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(&ctx->sin_d, n * sizeof(float));
    if (e == hipSuccess) e = hipMalloc(&ctx->rev_d, half * sizeof(double));
    if (e == hipSuccess) e = hipMemcpy(ctx->cos_d, cs.data(), n * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(ctx->sin_d, sn.data(), n * sizeof(float), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(ctx->rev_d, rev.data(), half * sizeof(double), hipMemcpyHostToDevice);
    const size_t zbytes = (size_t)cfg->head_dim * PIC_BLOCK_SIZE * sizeof(uint16_t);
    if (e == hipSuccess) e = hipMalloc(&ctx->zero_d, zbytes);
    if (e == hipSuccess) e = hipMemset(ctx->zero_d, 0, zbytes);
    if (e == hipSuccess) e = scratch_address(ctx->device, &ctx->scratch_d);
    if (e != hipSuccess) {
        pic_ctx_destroy(ctx);
        return PIC_ERR_HIP;
    }
    *out = ctx;
    return PIC_OK;
}

void pic_ctx_destroy(pic_ctx *ctx) {
    if (!ctx) return;
    for (hipEvent_t ev : ctx->tev) (void)hipEventDestroy(ev);
    if (ctx->cos_d) (void)hipFree(ctx->cos_d);
    if (ctx->sin_d) (void)hipFree(ctx->sin_d);
    if (ctx->rev_d) (void)hipFree(ctx->rev_d);
    if (ctx->zero_d) (void)hipFree(ctx->zero_d);
    delete ctx;
}

pic_status pic_timing_start(pic_ctx *ctx, int32_t capacity) {
    if (check_ctx(ctx) != PIC_OK) return PIC_ERR_INVALID_ARG;
    if (ctx->timing) return fail(ctx, PIC_ERR_INVALID_ARG, "timing is already on%s");
    if (capacity < 1 || capacity > 65536) return fail(ctx, PIC_ERR_INVALID_ARG, "timing capacity out of range%s");
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != ctx->device) e = hipSetDevice(ctx->device);
    ctx->tev.assign(2 * (size_t)capacity, nullptr);
    for (size_t i = 0; e == hipSuccess && i < ctx->tev.size(); ++i) e = hipEventCreate(&ctx->tev[i]);
    if (cur != ctx->device) (void)hipSetDevice(cur);
    if (e != hipSuccess) {
        for (hipEvent_t ev : ctx->tev)
            if (ev) (void)hipEventDestroy(ev);
        ctx->tev.clear();
        return hip_fail(ctx, e, "timing events");
    }
    ctx->top.clear();
    ctx->top.reserve(capacity);
    ctx->timing = true;
    return PIC_OK;
}

pic_status pic_timing_stop(pic_ctx *ctx, float *ms, int32_t *ops, int32_t cap, int32_t *count) {
    if (check_ctx(ctx) != PIC_OK) return PIC_ERR_INVALID_ARG;
    if (!ctx->timing) return fail(ctx, PIC_ERR_INVALID_ARG, "timing is off%s");
    if (cap < 0 || !count) return fail(ctx, PIC_ERR_INVALID_ARG, "cap / count invalid%s");
    const int32_t n = (int32_t)ctx->top.size();
    hipError_t e = n > 0 ? hipEventSynchronize(ctx->tev[2 * (size_t)n - 1]) : hipSuccess;
    for (int32_t i = 0; e == hipSuccess && i < n && i < cap; ++i) {
        float t = 0.f;
        e = hipEventElapsedTime(&t, ctx->tev[2 * (size_t)i], ctx->tev[2 * (size_t)i + 1]);
        if (ms) ms[i] = t;
        if (ops) ops[i] = ctx->top[i];
    }
    for (hipEvent_t ev : ctx->tev) (void)hipEventDestroy(ev);
    ctx->tev.clear();
    ctx->top.clear();
    ctx->timing = false;
    *count = n;
    if (e != hipSuccess) return hip_fail(ctx, e, "timing read");
    return PIC_OK;
}

// Anchor extraction: the per-slot score when the caller passes no buffer.
size_t anchor_ws(int batch, int max_blocks) {
    return align_up((size_t)batch * max_blocks * kBlock * sizeof(float));
}

pic_status pic_workspace_bytes(const pic_ctx *ctx, pic_op op, const pic_req_table *req, int32_t total_q,
                               int32_t max_q_len, size_t *bytes) {
    if (!ctx || !req || !bytes) return PIC_ERR_INVALID_ARG;
    if (req->batch < 0 || req->max_kv_len < 0 || req->max_blocks <= 0) return PIC_ERR_INVALID_ARG;
    const pic_config &c = ctx->cfg;
    switch (op) {
    case PIC_OP_PREFILL: {
        if (total_q < 0 || max_q_len < 0) return PIC_ERR_INVALID_ARG;
        *bytes = prefill_ws(c, plan_fwd(c, req->batch, max_q_len, req->max_kv_len), total_q).total;
        return PIC_OK;
    }
    case PIC_OP_DECODE:
        *bytes = decode_ws(c, req->batch, plan_decode(req->batch, c.num_kv_heads, req->max_kv_len).num_splits).total;
        return PIC_OK;
    case PIC_OP_SELECT: {
        if (total_q < 0 || max_q_len < 0) return PIC_ERR_INVALID_ARG;
        const FwdPlan pl = plan_lse(c, req->batch, max_q_len, req->max_kv_len);
        const FwdPlan plm = plan_mass(c, req->batch, max_q_len, req->max_kv_len);
        *bytes = select_ws(c, pl, plm, req->batch, req->max_blocks, total_q, req->max_kv_len).total;
        return PIC_OK;
    }
    case PIC_OP_ANCHOR:
        *bytes = anchor_ws(req->batch, req->max_blocks);
        return PIC_OK;
    }
    return PIC_ERR_INVALID_ARG;
}

pic_status pic_select_offsets(int32_t n_spans, const int32_t *span_len_host, double ratio,
                              int32_t *sel_off_host) {
    if (n_spans < 0 || !sel_off_host || (n_spans > 0 && !span_len_host)) return PIC_ERR_INVALID_ARG;
    if (!(ratio >= 0.0 && ratio <= 1.0)) return PIC_ERR_INVALID_ARG;
    long long acc = 0;
    sel_off_host[0] = 0;
    for (int32_t s = 0; s < n_spans; ++s) {
        if (span_len_host[s] < 0) return PIC_ERR_INVALID_ARG;
        const long long k = (long long)std::floor(ratio * (double)span_len_host[s] + 0.5);
        acc += std::min<long long>(k, span_len_host[s]);
        if (acc > 0x7fffffffLL) return PIC_ERR_INVALID_ARG;
        sel_off_host[s + 1] = (int32_t)acc;
    }
    return PIC_OK;
}

pic_status pic_attn_prefill(pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req,
                            const pic_queries *qs, uint16_t *out, float *lse, void *ws, size_t ws_bytes,
                            void *stream) {
    if (check_ctx(ctx) != PIC_OK) return PIC_ERR_INVALID_ARG;
    pic_status st = check_pool_req(ctx, pool, req);
    if (st != PIC_OK) return st;
    if ((st = check_queries(ctx, qs, req->batch)) != PIC_OK) return st;
    if (qs->total_q > 0 && !out) return fail(ctx, PIC_ERR_INVALID_ARG, "out is NULL%s");
    if (req->batch == 0 || qs->total_q == 0) return PIC_OK;
    const pic_config &c = ctx->cfg;
    const FwdPlan pl = plan_fwd(c, req->batch, qs->max_q_len, req->max_kv_len);
    const PrefillWs w = prefill_ws(c, pl, qs->total_q);
    if (w.total > 0 && (!ws || ws_bytes < w.total))
        return fail(ctx, PIC_ERR_WORKSPACE, "workspace too small for prefill%s");
    hipStream_t s = (hipStream_t)stream;
    pic::FwdParams p;
    fill_fwd_common(p, ctx, pool, req, qs, pl);
    p.out = out;
    p.lse = lse;
    if (pl.num_splits > 1) {
        p.part_o = (float *)((char *)ws + w.part_o);
        p.part_ml = (float *)((char *)ws + w.part_ml);
    }
    TimedSpan ts(ctx, PIC_OP_PREFILL);
    hipError_t e = pic::launch_fwd(p, c.head_dim, pic::kAttn, pl.shape, s, ts.ev);
    if (e != hipSuccess) return hip_fail(ctx, e, "prefill launch");
    ts.commit();
    if (pl.num_splits > 1) {
        pic::MergeParams m{p.part_o, p.part_ml, pl.num_splits, qs->total_q * c.num_q_heads, out, lse};
        e = pic::launch_merge(m, c.head_dim, s);
        if (e != hipSuccess) return hip_fail(ctx, e, "prefill merge launch");
    }
    return PIC_OK;
}

pic_status pic_attn_decode(pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req, const uint16_t *q,
                           const int32_t *q_pos, uint16_t *out, float *lse, void *ws, size_t ws_bytes,
                           void *stream) {
    if (check_ctx(ctx) != PIC_OK) return PIC_ERR_INVALID_ARG;
    pic_status st = check_pool_req(ctx, pool, req);
    if (st != PIC_OK) return st;
    if (req->batch > 0 && (!q || !q_pos || !out)) return fail(ctx, PIC_ERR_INVALID_ARG, "q / q_pos / out is NULL%s");
    const pic_config &c = ctx->cfg;
    if (c.num_q_heads / c.num_kv_heads > 16)
        return fail(ctx, PIC_ERR_UNSUPPORTED, "decode supports up to 16 q heads per kv head%s");
    if (req->batch == 0) return PIC_OK;
    const DecodePlan dp = plan_decode(req->batch, c.num_kv_heads, req->max_kv_len);
    const int splits = dp.num_splits;
    const DecodeWs w = decode_ws(c, req->batch, splits);
    if (w.total > 0 && (!ws || ws_bytes < w.total))
        return fail(ctx, PIC_ERR_WORKSPACE, "workspace too small for decode%s");
    hipStream_t s = (hipStream_t)stream;
    pic::DecodeParams p;
    std::memset(&p, 0, sizeof p);
    p.zero_page = ctx->zero_d;
    p.k_pool = pool->k;
    p.v_pool = pool->v;
    p.num_blocks = pool->num_blocks;
    p.block_table = req->block_table;
    p.kv_len = req->kv_len;
    p.kv_pos = req->kv_pos;
    p.max_blocks = req->max_blocks;
    p.q = q;
    p.q_pos = q_pos;
    p.batch = req->batch;
    p.hq = c.num_q_heads;
    p.hkv = c.num_kv_heads;
    p.group = c.num_q_heads / c.num_kv_heads;
    p.cos_tab = ctx->cos_d;
    p.sin_tab = ctx->sin_d;
    p.rev_freq = ctx->rev_d;
    p.rotate_k = c.keys_prerotated ? 0 : 1;
    p.max_pos = c.max_position;
    p.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
    p.max_kv_len = req->max_kv_len;
    p.split_len = dp.split_len;
    p.num_splits = splits;
    p.out = out;
    p.lse = lse;
    if (splits > 1) {
        p.part_o = (float *)((char *)ws + w.part_o);
        p.part_ml = (float *)((char *)ws + w.part_ml);
    }
    TimedSpan ts(ctx, PIC_OP_DECODE);
    hipError_t e = pic::launch_decode(p, c.head_dim, s, ts.ev);
    if (e != hipSuccess) return hip_fail(ctx, e, "decode launch");
    ts.commit();
    if (splits > 1) {
        pic::MergeParams m{p.part_o, p.part_ml, splits, req->batch * c.num_q_heads, out, lse};
        e = pic::launch_merge(m, c.head_dim, s);
        if (e != hipSuccess) return hip_fail(ctx, e, "decode merge launch");
    }
    return PIC_OK;
}

pic_status qc_score_select(pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req, const pic_queries *qs,
                           const float *lse, const pic_spans *spans, int32_t max_sel, int32_t *sel_idx,
                           float *mass, void *ws, size_t ws_bytes, void *stream) {
    if (check_ctx(ctx) != PIC_OK) return PIC_ERR_INVALID_ARG;
    pic_status st = check_pool_req(ctx, pool, req);
    if (st != PIC_OK) return st;
    if ((st = check_queries(ctx, qs, req->batch)) != PIC_OK) return st;
    if (!spans || spans->n_spans < 0) return fail(ctx, PIC_ERR_INVALID_ARG, "spans descriptor invalid%s");
    if (spans->n_spans > 0 && (!spans->span_req || !spans->span_start || !spans->span_len || !spans->sel_off))
        return fail(ctx, PIC_ERR_INVALID_ARG, "span arrays are NULL%s");
    if (max_sel < 0 || (max_sel > 0 && !sel_idx)) return fail(ctx, PIC_ERR_INVALID_ARG, "sel_idx / max_sel invalid%s");
    if (req->batch == 0) return PIC_OK;
    const pic_config &c = ctx->cfg;
    const FwdPlan pl = plan_lse(c, req->batch, qs->max_q_len, req->max_kv_len);
    const FwdPlan plm = plan_mass(c, req->batch, qs->max_q_len, req->max_kv_len);
    const SelectWs w = select_ws(c, pl, plm, req->batch, req->max_blocks, qs->total_q, req->max_kv_len);
    if (!ws || ws_bytes < w.total) return fail(ctx, PIC_ERR_WORKSPACE, "workspace too small for selection%s");
    hipStream_t s = (hipStream_t)stream;
    char *wb = (char *)ws;
    pic::FwdParams p;
    fill_fwd_common(p, ctx, pool, req, qs, pl);
    hipError_t e;
    const float *lse_use = lse;
    if (!lse && qs->total_q > 0) {
        // the query rows' log-sum-exp over the same keys (K only)
        float *lse_ws = (float *)(wb + w.lse);
        pic::FwdParams pl_lse = p;
        pl_lse.lse = lse_ws;
        if (pl.num_splits > 1) pl_lse.part_ml = (float *)(wb + w.lse_ml);
        e = pic::launch_fwd(pl_lse, c.head_dim, pic::kLse, pl.shape, s);
        if (e != hipSuccess) return hip_fail(ctx, e, "selection lse launch");
        if (pl.num_splits > 1) {
            pic::MergeParams m{nullptr, pl_lse.part_ml, pl.num_splits, qs->total_q * c.num_q_heads, nullptr, lse_ws};
            e = pic::launch_merge(m, c.head_dim, s);
            if (e != hipSuccess) return hip_fail(ctx, e, "selection lse merge launch");
        }
        lse_use = lse_ws;
    }
    float *mass_out = mass ? mass : (float *)(wb + w.mass);
    float *mass_part = (float *)(wb + w.mass_part);
    pic::SelectParams sp;
    std::memset(&sp, 0, sizeof sp);
    sp.mass_part = mass_part;
    sp.hkv = c.num_kv_heads;
    sp.row_blocks = plm.row_blocks;
    sp.mass_stride = req->max_kv_len;
    sp.q_start = qs->q_start;
    sp.group = c.num_q_heads / c.num_kv_heads;
    sp.rows_per_block = plm.rows_per_block;
    sp.kv_len = req->kv_len;
    sp.kv_pos = req->kv_pos;
    sp.kv_stride = req->max_blocks * kBlock;
    sp.batch = req->batch;
    sp.mass = mass_out;
    sp.span_req = spans->span_req;
    sp.span_start = spans->span_start;
    sp.span_len = spans->span_len;
    sp.sel_off = spans->sel_off;
    sp.n_spans = spans->n_spans;
    sp.sel_idx = sel_idx;
    sp.max_sel = max_sel;
    if (qs->total_q > 0 && req->max_kv_len > 0) {
        pic::FwdParams pm = p;
        pm.lse_in = lse_use;
        pm.mass_part = mass_part;
        pm.mass_stride = req->max_kv_len;
        pm.split_len = plm.split_len;
        pm.num_splits = plm.num_splits;
        pm.row_blocks = plm.row_blocks;
        TimedSpan ts(ctx, PIC_OP_SELECT);
        e = pic::launch_fwd(pm, c.head_dim, pic::kMass, plm.shape, s, ts.ev);
        if (e != hipSuccess) return hip_fail(ctx, e, "selection mass launch");
        ts.commit();
    }
    e = pic::launch_mass_reduce(sp, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "mass reduce launch");
    if (max_sel > 0) {
        e = pic::launch_topk(sp, s);
        if (e != hipSuccess) return hip_fail(ctx, e, "top-k launch");
    }
    return PIC_OK;
}

pic_status qc_score_select_noalloc(pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req,
                                   const pic_queries *qs, const float *lse, const pic_spans *spans,
                                   int32_t max_sel, int32_t *sel_idx, float *mass, void *stream) {
    if (check_ctx(ctx) != PIC_OK) return PIC_ERR_INVALID_ARG;
    if (!ctx->scratch_d) return fail(ctx, PIC_ERR_HIP, "no scratch address for this device%s");
    pic_status st = check_pool_req(ctx, pool, req);
    if (st != PIC_OK) return st;
    if ((st = check_queries(ctx, qs, req->batch)) != PIC_OK) return st;
    const pic_config &c = ctx->cfg;
    const FwdPlan pl = plan_lse(c, req->batch, qs->max_q_len, req->max_kv_len);
    const FwdPlan plm = plan_mass(c, req->batch, qs->max_q_len, req->max_kv_len);
    const size_t need = select_ws(c, pl, plm, req->batch, req->max_blocks, qs->total_q, req->max_kv_len).total;
    if (need > (size_t)PIC_NOALLOC_SCRATCH_BYTES) {
        char buf[160];
        std::snprintf(buf, sizeof buf, "selection needs %zu bytes of scratch, more than the %zu bytes the "
                      "no-allocation entry point holds%%s", need, (size_t)PIC_NOALLOC_SCRATCH_BYTES);
        return fail(ctx, PIC_ERR_WORKSPACE, buf);
    }
    // The selection's scratch needs no clearing: every partial the later
    // kernels read is written first by an earlier kernel of the same call.
    return qc_score_select(ctx, pool, req, qs, lse, spans, max_sel, sel_idx, mass, ctx->scratch_d,
                           (size_t)PIC_NOALLOC_SCRATCH_BYTES, stream);
}

pic_status qc_anchor_select(pic_ctx *ctx, const pic_kv_pool *pool, const pic_req_table *req,
                            const pic_spans *spans, int32_t max_sel, int32_t *sel_idx, float *norm, void *ws,
                            size_t ws_bytes, void *stream) {
    if (check_ctx(ctx) != PIC_OK) return PIC_ERR_INVALID_ARG;
    pic_status st = check_pool_req(ctx, pool, req);
    if (st != PIC_OK) return st;
    if (!spans || spans->n_spans < 0) return fail(ctx, PIC_ERR_INVALID_ARG, "spans descriptor invalid%s");
    if (spans->n_spans > 0 && (!spans->span_req || !spans->span_start || !spans->span_len || !spans->sel_off))
        return fail(ctx, PIC_ERR_INVALID_ARG, "span arrays are NULL%s");
    if (max_sel < 0 || (max_sel > 0 && !sel_idx)) return fail(ctx, PIC_ERR_INVALID_ARG, "sel_idx / max_sel invalid%s");
    if (req->batch > 65535) return fail(ctx, PIC_ERR_UNSUPPORTED, "anchor extraction supports up to 65535 requests%s");
    if (req->batch == 0) return PIC_OK;
    const size_t need = norm ? 0 : anchor_ws(req->batch, req->max_blocks);
    if (need > 0 && (!ws || ws_bytes < need)) return fail(ctx, PIC_ERR_WORKSPACE, "workspace too small for anchors%s");
    const pic_config &c = ctx->cfg;
    hipStream_t s = (hipStream_t)stream;
    float *score = norm ? norm : (float *)ws;
    pic::NormParams np;
    std::memset(&np, 0, sizeof np);
    np.k_pool = pool->k;
    np.num_blocks = pool->num_blocks;
    np.hkv = c.num_kv_heads;
    np.block_table = req->block_table;
    np.kv_len = req->kv_len;
    np.kv_pos = req->kv_pos;
    np.max_blocks = req->max_blocks;
    np.max_pos = c.max_position;
    np.batch = req->batch;
    np.norm = score;
    hipError_t e = pic::launch_key_norm(np, c.head_dim, s);
    if (e != hipSuccess) return hip_fail(ctx, e, "key norm launch");
    if (max_sel > 0) {
        pic::SelectParams sp;
        std::memset(&sp, 0, sizeof sp);
        sp.kv_len = req->kv_len;
        sp.kv_pos = req->kv_pos;
        sp.kv_stride = req->max_blocks * kBlock;
        sp.batch = req->batch;
        sp.mass = score;
        sp.span_req = spans->span_req;
        sp.span_start = spans->span_start;
        sp.span_len = spans->span_len;
        sp.sel_off = spans->sel_off;
        sp.n_spans = spans->n_spans;
        sp.sel_idx = sel_idx;
        sp.max_sel = max_sel;
        e = pic::launch_topk(sp, s);
        if (e != hipSuccess) return hip_fail(ctx, e, "anchor top-k launch");
    }
    return PIC_OK;
}

pic_status kv_fuse_scatter(pic_ctx *ctx, pic_kv_pool *pool, pic_req_table *req, const int32_t *sel_idx,
                           const int32_t *sel_req_off, const uint16_t *k_new, const uint16_t *v_new, int32_t n_sel,
                           int32_t max_rows_per_req, void *stream) {
    if (check_ctx(ctx) != PIC_OK) return PIC_ERR_INVALID_ARG;
    pic_status st = check_pool_req(ctx, pool, req);
    if (st != PIC_OK) return st;
    if (n_sel < 0 || max_rows_per_req < 0 || max_rows_per_req > n_sel)
        return fail(ctx, PIC_ERR_INVALID_ARG, "n_sel / max_rows_per_req invalid%s");
    if (req->batch > 0 && !sel_req_off) return fail(ctx, PIC_ERR_INVALID_ARG, "sel_req_off is NULL%s");
    if (req->batch > 65535) return fail(ctx, PIC_ERR_UNSUPPORTED, "kv_fuse_scatter supports up to 65535 requests%s");
    if (n_sel > 0 && (!sel_idx || !k_new || !v_new))
        return fail(ctx, PIC_ERR_INVALID_ARG, "sel_idx / k_new / v_new is NULL%s");
    if (req->batch == 0) return PIC_OK;
    pic::FuseParams p;
    std::memset(&p, 0, sizeof p);
    p.k_pool = pool->k;
    p.v_pool = pool->v;
    p.num_blocks = pool->num_blocks;
    p.hkv = ctx->cfg.num_kv_heads;
    p.block_table = req->block_table;
    p.kv_len = req->kv_len;
    p.kv_pos = req->kv_pos;
    p.max_blocks = req->max_blocks;
    p.sel_idx = sel_idx;
    p.sel_req_off = sel_req_off;
    p.k_new = k_new;
    p.v_new = v_new;
    p.batch = req->batch;
    p.max_rows = max_rows_per_req;
    p.n_sel = n_sel;
    hipError_t e = pic::launch_fuse(p, ctx->cfg.head_dim, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(ctx, e, "fuse launch");
    return PIC_OK;
}

}  // extern "C"
