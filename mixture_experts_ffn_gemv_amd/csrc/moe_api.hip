// Host side of the C ABI declared in include/moe.h: the context (scratch,
// slot table, host arena), argument checks, and the launch sequence of one
// MoE layer call on a HIP stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstring>
#include <mutex>
#include <new>
#include <type_traits>
#include <vector>

#include "moe.h"
#include "moe_common.h"
#include "moe_internal.h"

using namespace moe;

thread_local LaunchTimer* moe::g_launch_timer = nullptr;

namespace {

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// bump allocator over one device allocation
struct Carver {
    size_t off = 0;
    template <typename TT>
    size_t take(size_t count) {
        const size_t o = align_up(off, 256);
        off = o + count * sizeof(TT);
        return o;
    }
};

}  // namespace

struct moe_ctx {
    moe_cfg cfg;
    int device = 0;
    int n_cu = 256;          // compute units of the device
    bool decode_ok = false;  // the decode-path kernels fit this shape
    bool mmq_ok = false;     // the MMQ tiles fit this shape
    bool mixed = false;      // groups of <= GEMV_ROWS rows on the GEMV kernels when the MMQ path runs
    int max_pairs = 0;
    int max_chunks = 0;   // chunk-list capacity
    uint8_t* dev = nullptr;
    // scratch views
    float* logits = nullptr;
    int logit_rows = 0;      // rows of the logits scratch: room for the router's split-K partials
    int32_t* idx = nullptr;
    float* gw = nullptr;
    int8_t* xq = nullptr;
    float* xd = nullptr;
    int32_t* xs16 = nullptr;
    float* xs16f = nullptr;
    uint16_t* xs16b = nullptr;   // [M][D/256][48] bf16 planes of xs16f (MMQ)
    int32_t* offsets = nullptr;
    int32_t* active = nullptr;
    int32_t* n_active = nullptr;
    int32_t* n_chunks = nullptr;
    int32_t* perm = nullptr;
    int32_t* inv = nullptr;
    Chunk* chunks = nullptr;
    Chunk* wave_chunks = nullptr;     // one slot wave's chunks (lists compacted, same bases)
    int32_t* wave_n_chunks = nullptr;
    float* h_routed = nullptr;
    uint8_t* hrec = nullptr;
    float* h_shared = nullptr;
    int8_t* hq_routed = nullptr;
    float* hd_routed = nullptr;
    int32_t* hs_routed = nullptr;
    int8_t* hq_shared = nullptr;
    float* hd_shared = nullptr;
    int32_t* hs_shared = nullptr;
    // the bf16 shared expert runs on a side stream: fork after the call's input is
    // ready, join before the combine
    hipStream_t side = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    float* e_rows = nullptr;
    float* ys = nullptr;
    int32_t* err = nullptr;
    uint32_t* arrive = nullptr;   // the one-token router launch's arrival counters (0 between calls)
    int32_t* slot_table_dev = nullptr;
    // slots
    uint8_t* arena = nullptr;
    int n_slots = 0;
    size_t slot_bytes = 0, off_w1 = 0, off_w3 = 0, off_w2 = 0;
    int32_t* slot_host = nullptr;   // pinned mirror of the table
    std::vector<int32_t> slot_owner; // slot -> expert or -1
    bool table_dirty = true;
    hipEvent_t table_ev = nullptr;
    bool table_ev_pending = false;
    // host arena and the miss streaming (copies on their own stream, fenced by events)
    const uint8_t* host_arena = nullptr;
    size_t host_stride = 0;
    hipStream_t copy = nullptr;
    int32_t* idx_host = nullptr;    // pinned read-back of the picks
    int32_t* view_host = nullptr;   // pinned per-wave slot tables, [E][E]
    std::vector<uint64_t> slot_tick; // slot -> last call that used it (least recently used goes first)
    uint64_t tick = 0;
    std::vector<hipEvent_t> ev_copy, ev_wave, ev_c0, ev_c1;   // per wave
    mutable std::vector<std::pair<hipEvent_t, hipEvent_t>> fetch_pending;
    // expert-compute time of calls with a host arena or with profiling on: an event
    // pair per call, read when the counters are read
    std::vector<hipEvent_t> ev_comp;
    size_t comp_next = 0;
    mutable std::vector<std::pair<hipEvent_t, hipEvent_t>> comp_pending;
    mutable moe_stats stats;
    // per-kernel timing
    bool prof = false;
    std::vector<hipEvent_t> ev_pool;
    size_t ev_next = 0;
    struct Mark {
        int kind;
        hipEvent_t a, b;
    };
    std::vector<Mark> marks;
    double k_ms[MOE_K_COUNT] = {};
    int64_t k_n[MOE_K_COUNT] = {};
};

namespace {

// The per-call device buffers of a context sized for M tokens, carved from one
// allocation at `base` (views set on ctx when base is not NULL); returns the
// bytes needed. decode_only: just what a call of M <= 8 tokens on the decode
// kernels (K-quant experts, every pick resident) touches, for the static
// scratch of moe_forward_static; the other views stay NULL.
size_t carve_scratch(moe_ctx* ctx, size_t M, bool decode_only, uint8_t* base) {
    const moe_cfg& c = ctx->cfg;
    const size_t E = c.n_routed, D = c.dim, I = c.inter;
    const size_t P = M * c.topk;
    const size_t m_small = std::min<size_t>(M, ROUTE_SMALL_MAX_M);
    Carver cv;
    auto view = [&](auto*& field, size_t off) {
        if (base != nullptr) field = reinterpret_cast<std::remove_reference_t<decltype(field)>>(base + off);
    };
    // first, at the same offset for every M: the arrival counters, which every call
    // leaves at 0 (the static scratch holds them across calls of any size)
    view(ctx->arrive, cv.take<uint32_t>(ROUTER_ARRIVE_WORDS));
    // the router's partial logits: up to 8 splits of m rows, within 4096 rows (one split at m <= 8)
    const int logit_rows = decode_only ? (int)M : (int)std::max<size_t>(M, std::min<size_t>(8 * M, 4096));
    if (base != nullptr) ctx->logit_rows = logit_rows;
    view(ctx->logits, cv.take<float>((size_t)logit_rows * E));
    view(ctx->idx, cv.take<int32_t>(P));
    view(ctx->gw, cv.take<float>(P));
    view(ctx->xq, cv.take<int8_t>(M * D));
    view(ctx->xd, cv.take<float>(M * D / QB));
    view(ctx->xs16, cv.take<int32_t>(M * D / 16));
    view(ctx->xs16f, cv.take<float>(M * D / 16));
    view(ctx->offsets, cv.take<int32_t>(E + 1));
    view(ctx->active, cv.take<int32_t>(E));
    view(ctx->n_active, cv.take<int32_t>(1));
    view(ctx->n_chunks, cv.take<int32_t>(PLAN_LISTS));
    view(ctx->perm, cv.take<int32_t>(P));
    view(ctx->inv, cv.take<int32_t>(P));
    view(ctx->chunks, cv.take<Chunk>(decode_only ? m_small * (c.topk + 1) + 1 : (size_t)ctx->max_chunks));
    view(ctx->h_shared, cv.take<float>(M * I));
    view(ctx->ys, cv.take<float>(M * D));
    view(ctx->hrec, cv.take<uint8_t>(m_small * (c.topk + 1) * decode_rec_bytes((int)I)));
    view(ctx->err, cv.take<int32_t>(STATUS_WORDS));
    if (!decode_only) {
        view(ctx->xs16b, cv.take<uint16_t>(M * D / QK * 48));
        view(ctx->wave_chunks, cv.take<Chunk>((size_t)ctx->max_chunks));
        view(ctx->wave_n_chunks, cv.take<int32_t>(PLAN_LISTS));
        view(ctx->h_routed, cv.take<float>(P * I));
        view(ctx->hq_routed, cv.take<int8_t>(P * I));
        view(ctx->hd_routed, cv.take<float>(P * I / QB));
        view(ctx->hs_routed, cv.take<int32_t>(P * I / 16));
        view(ctx->hq_shared, cv.take<int8_t>(M * I));
        view(ctx->hd_shared, cv.take<float>(M * I / QB));
        view(ctx->hs_shared, cv.take<int32_t>(M * I / 16));
        view(ctx->e_rows, cv.take<float>(P * D));
        view(ctx->slot_table_dev, cv.take<int32_t>(E));
    }
    return align_up(cv.off, 256);
}

int check_cfg(const moe_cfg* c) {
    if (c == nullptr) return MOE_EINVAL;
    if (c->dim < 256 || c->dim > 8192 || c->dim % 256) return MOE_EINVAL;
    if (c->inter < 256 || c->inter > 8192 || c->inter % 256) return MOE_EINVAL;
    if (c->n_routed < 1 || c->n_routed > 1024) return MOE_EINVAL;
    if (c->topk < 1 || c->topk > 64 || c->topk > c->n_routed) return MOE_EINVAL;
    if (!(c->gate_temp > 0.f)) return MOE_EINVAL;
    if (c->max_tokens < 1 || c->max_tokens > 65536) return MOE_EINVAL;
    if ((int64_t)c->max_tokens * c->topk > (1 << 22)) return MOE_EINVAL;
    if (c->expert_fmt != MOE_EXPERT_KQUANT && c->expert_fmt != MOE_EXPERT_MXFP4) return MOE_EINVAL;
    return MOE_OK;
}

void layout_of(const moe_cfg& c, size_t& slot, size_t& o1, size_t& o3, size_t& o2) {
    const size_t DI = (size_t)c.dim * c.inter;
    const bool fp4 = c.expert_fmt == MOE_EXPERT_MXFP4;   // codes (2 per byte) + one scale byte per 32
    const size_t n13 = fp4 ? DI / 2 + DI / 32 : (size_t)c.inter * (c.dim / QK) * Q2K_BYTES;
    const size_t n2 = fp4 ? DI / 2 + DI / 32 : (size_t)c.dim * (c.inter / QK) * Q3K_BYTES;
    o1 = 0;
    o3 = n13;
    o2 = 2 * n13;
    slot = 2 * n13 + n2;
}

// upper bound of routed chunks of at most `rows` token rows for m tokens:
// sum_e ceil(c_e / rows) <= (P + (rows - 1) * min(E, P)) / rows
int routed_chunk_bound(const moe_cfg& c, int m, int rows = GEMV_ROWS) {
    const int P = m * c.topk;
    const int act = std::min(c.n_routed, P);
    return (P + (rows - 1) * act) / rows + 1;
}

int shared_chunk_count(int m, int rows = GEMV_ROWS) { return (m + rows - 1) / rows; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

hipEvent_t prof_event(moe_ctx* ctx) {
    if (ctx->ev_next == ctx->ev_pool.size()) {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        ctx->ev_pool.push_back(e);
    }
    return ctx->ev_pool[ctx->ev_next++];
}

// with profiling on, the kernels `fn` launches (it returns hipError_t) carry
// start/stop events recorded as kernel class `kind`
struct ClassTimer final : LaunchTimer {
    moe_ctx* ctx;
    int kind;
    bool next_pair(hipEvent_t* start, hipEvent_t* stop) override {
        *start = prof_event(ctx);
        *stop = prof_event(ctx);
        if (*start == nullptr || *stop == nullptr) return false;
        ctx->marks.push_back({kind, *start, *stop});
        return true;
    }
};

template <typename F>
int timed(moe_ctx* ctx, hipStream_t, int kind, F fn) {
    if (!ctx->prof) return fn() == hipSuccess ? MOE_OK : MOE_EHIP;
    ClassTimer t;
    t.ctx = ctx;
    t.kind = kind;
    g_launch_timer = &t;
    const hipError_t e = fn();
    g_launch_timer = nullptr;
    return e == hipSuccess ? MOE_OK : MOE_EHIP;
}

int upload_table(moe_ctx* ctx, hipStream_t st) {
    if (!ctx->table_dirty) return MOE_OK;
    if (hipMemcpyAsync(ctx->slot_table_dev, ctx->slot_host, sizeof(int32_t) * ctx->cfg.n_routed,
                       hipMemcpyHostToDevice, st) != hipSuccess)
        return MOE_EHIP;
    if (hipEventRecord(ctx->table_ev, st) != hipSuccess) return MOE_EHIP;
    ctx->table_ev_pending = true;
    ctx->table_dirty = false;
    return MOE_OK;
}

// the pinned mirror may still be read by a queued upload: wait before changing it
int table_mutable(moe_ctx* ctx) {
    if (ctx->table_ev_pending) {
        if (hipEventSynchronize(ctx->table_ev) != hipSuccess) return MOE_EHIP;
        ctx->table_ev_pending = false;
    }
    return MOE_OK;
}

int check_weights(const moe_ctx* ctx, const moe_weights* w) {
    if (w == nullptr || w->router_w == nullptr || w->router_bias == nullptr) return MOE_EINVAL;
    if (!aligned(w->router_w, 16) || !aligned(w->router_bias, 4)) return MOE_EINVAL;
    if (w->shared_fmt == MOE_SHARED_NONE) return MOE_OK;
    if (w->shared_fmt != MOE_SHARED_BF16 && w->shared_fmt != MOE_SHARED_KQUANT) return MOE_EINVAL;
    if (w->shared_fmt == MOE_SHARED_KQUANT && ctx->cfg.expert_fmt == MOE_EXPERT_MXFP4) return MOE_EINVAL;
    if (w->shared_w1 == nullptr || w->shared_w3 == nullptr || w->shared_w2 == nullptr) return MOE_EINVAL;
    if (!aligned(w->shared_w1, 16) || !aligned(w->shared_w3, 16) || !aligned(w->shared_w2, 16)) return MOE_EINVAL;
    if (w->shared_fmt == MOE_SHARED_BF16 && ctx->cfg.dim > 8192) return MOE_EINVAL;
    return MOE_OK;
}

// How a call of m tokens runs: the routing kernels (small: one workgroup for the
// top-k and bucketing, m <= 8), the expert kernels (MMQ above 8 tokens where the
// tiles fit; the decode kernels for K-quant experts up to 8 tokens), and where a
// bf16 shared expert's rows go. Up to 8 tokens with every pick resident (no host
// arena) the bf16 shared expert rides in the routed launches: its gate/up rows as
// extra workgroups of the router launch, its down rows (into ys, added by the
// routed down kernel or, for MXFP4 experts, by the combine kernel) as extra
// workgroups of the top-k launch; with K-quant experts the second half of the
// down rows goes to the routed gate/up launch instead, whose workgroups leave CU
// slots free (the top-k launch is then shorter and gate/up hardly longer). No
// second stream then.
struct CallPlan {
    bool small, use_mmq, fp4, decode, shared_fused;
    bool fold_topk;   // up to 8 tokens on the decode kernels: the router launch also selects
    int sh_router_rows, sh_topk_rows, sh_gateup_rows;
};

CallPlan plan_call(const moe_ctx* ctx, int m, int shared_fmt) {
    const moe_cfg& c = ctx->cfg;
    CallPlan pl{};
    pl.small = m <= ROUTE_SMALL_MAX_M && m * c.topk <= ROUTE_SMALL_MAX_PAIRS;
    pl.use_mmq = !pl.small && ctx->mmq_ok;
    pl.fp4 = c.expert_fmt == MOE_EXPERT_MXFP4;
    pl.decode = pl.small && ctx->decode_ok;
    pl.fold_topk = pl.decode && !pl.fp4 && router_select_ok(c.n_routed, c.topk, m);
    pl.shared_fused = shared_fmt == MOE_SHARED_BF16 && pl.small && (ctx->decode_ok || pl.fp4) &&
                      ctx->host_arena == nullptr;
    if (pl.shared_fused) {
        pl.sh_router_rows = c.inter;
        pl.sh_gateup_rows = !ctx->decode_ok ? 0 : pl.fold_topk ? c.dim : c.dim - c.dim / 2;
        pl.sh_topk_rows = c.dim - pl.sh_gateup_rows;
    }
    return pl;
}

// router logits and the top-k into (idx, gw) (moe_route)
int run_route(moe_ctx* ctx, const moe_weights* w, const uint16_t* x, int m, int32_t* idx, float* gw, hipStream_t st) {
    const moe_cfg& c = ctx->cfg;
    int splits = 1;
    int rc = timed(ctx, st, MOE_K_ROUTER, [&] {
        if (m <= ROUTE_SMALL_MAX_M)
            return launch_router_quant(x, m, (const uint16_t*)w->router_w, c.dim, c.n_routed, ctx->logits, nullptr,
                                       nullptr, nullptr, nullptr, st);
        return launch_router_gemm(x, m, (const uint16_t*)w->router_w, c.dim, c.n_routed, ctx->logits,
                                  ctx->logit_rows, &splits, st);
    });
    if (rc != MOE_OK) return rc;
    return timed(ctx, st, MOE_K_TOPK, [&] {
        return launch_topk(ctx->logits, splits, w->router_bias, m, c.n_routed, c.topk, c.gate_temp,
                           c.norm_topk_prob, c.route_scale, idx, gw, ctx->err, st);
    });
}

}  // namespace

extern "C" {

const char* moe_strerror(int code) {
    switch (code) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_ENOMEM: return "out of memory";
        case MOE_EHIP: return "HIP runtime error";
        case MOE_ENONFINITE: return "NaN routing key";
        case MOE_ENOTRESIDENT: return "picked expert not resident";
        case MOE_ESTATE: return "required state not set";
        case MOE_ESCRATCH: return "call needs more than the static scratch holds";
        default: return "unknown status";
    }
}

int moe_expert_layout(const moe_cfg* cfg, size_t* slot_bytes, size_t* off_w1, size_t* off_w3, size_t* off_w2) {
    if (check_cfg(cfg) != MOE_OK || !slot_bytes || !off_w1 || !off_w3 || !off_w2) return MOE_EINVAL;
    layout_of(*cfg, *slot_bytes, *off_w1, *off_w3, *off_w2);
    return MOE_OK;
}

// One thread per block of a rows x nsb matrix of B-byte blocks (B even): block
// (r, s) moves from plain row order to the panel order of the slot layout.
__global__ __launch_bounds__(256) void pack_matrix_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                          int rows, int nsb, int B) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)rows * nsb) return;
    const int r = (int)(q / nsb), s = (int)(q % nsb);
    const uint16_t* in = reinterpret_cast<const uint16_t*>(src + q * B);
    uint16_t* out = reinterpret_cast<uint16_t*>(dst + panel_off(r, s, nsb, B));
    for (int i = 0; i < B / 2; ++i) out[i] = in[i];
}

// One thread per 32-weight piece of a rows x K MXFP4 matrix: its 16 code bytes
// and its scale byte move from plain row order to the tiles of the slot layout.
__global__ __launch_bounds__(256) void pack_fp4_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                       int rows, int K) {
    const int np = K / 32;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (q >= (int64_t)rows * np) return;
    const int r = (int)(q / np), p = (int)(q % np);
    const size_t cb = (size_t)rows * (K / 2);
    const uint16_t* in = reinterpret_cast<const uint16_t*>(src + q * 16);
    uint16_t* out = reinterpret_cast<uint16_t*>(dst + fp4_code_off(r, p, K));
    for (int i = 0; i < 8; ++i) out[i] = in[i];
    dst[cb + fp4_scale_off(r, p, K)] = src[cb + q];
}

int moe_pack_expert(const moe_cfg* cfg, const void* src, void* dst, void* stream) {
    if (check_cfg(cfg) != MOE_OK || src == nullptr || dst == nullptr) return MOE_EINVAL;
    if (((uintptr_t)src | (uintptr_t)dst) & 1) return MOE_EINVAL;
    size_t bytes, o1, o3, o2;
    layout_of(*cfg, bytes, o1, o3, o2);
    const uint8_t* s8 = (const uint8_t*)src;
    uint8_t* d8 = (uint8_t*)dst;
    if (s8 < d8 + bytes && d8 < s8 + bytes) return MOE_EINVAL;
    const hipStream_t st = (hipStream_t)stream;
    const int D = cfg->dim, I = cfg->inter;
    if (cfg->expert_fmt == MOE_EXPERT_MXFP4) {
        struct F { size_t off; int rows, K; } mats[3] = {{o1, I, D}, {o3, I, D}, {o2, D, I}};
        for (const F& m : mats) {
            const int64_t n = (int64_t)m.rows * (m.K / 32);
            if (hip_status(launch_kernel(pack_fp4_kernel, (int)((n + 255) / 256), 256, 0, st, s8 + m.off, d8 + m.off,
                                         m.rows, m.K)) != MOE_OK)
                return MOE_EHIP;
        }
        return MOE_OK;
    }
    struct M { size_t off; int rows, nsb, B; } mats[3] = {
        {o1, I, D / QK, Q2K_BYTES}, {o3, I, D / QK, Q2K_BYTES}, {o2, D, I / QK, Q3K_BYTES}};
    for (const M& m : mats) {
        const int64_t n = (int64_t)m.rows * m.nsb;
        if (hip_status(launch_kernel(pack_matrix_kernel, (int)((n + 255) / 256), 256, 0, st, s8 + m.off, d8 + m.off,
                                     m.rows, m.nsb, m.B)) != MOE_OK)
            return MOE_EHIP;
    }
    return MOE_OK;
}

int moe_create(const moe_cfg* cfg, moe_ctx** out) {
    if (out == nullptr) return MOE_EINVAL;
    const int rc = check_cfg(cfg);
    if (rc != MOE_OK) return rc;
    moe_ctx* ctx = new (std::nothrow) moe_ctx();
    if (ctx == nullptr) return MOE_ENOMEM;
    ctx->cfg = *cfg;
    std::memset(&ctx->stats, 0, sizeof(ctx->stats));
    if (hipGetDevice(&ctx->device) != hipSuccess) {
        delete ctx;
        return MOE_EHIP;
    }
    const moe_cfg& c = ctx->cfg;
    {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, ctx->device) == hipSuccess && prop.multiProcessorCount > 0)
            ctx->n_cu = prop.multiProcessorCount;
    }
    // K-quant experts: the decode and MMQ kernels where their tiles fit this shape;
    // MXFP4 experts: their own chunked GEMV kernels up to 8 tokens, their
    // matrix-core kernels above
    const bool fp4 = c.expert_fmt == MOE_EXPERT_MXFP4;
    if (fp4 && !fp4_supported(c.dim, c.inter)) {
        delete ctx;
        return MOE_EINVAL;
    }
    ctx->decode_ok = !fp4 && decode_supported(c.dim, c.inter);
    ctx->mmq_ok = fp4 ? fp4_mmq_supported(c.dim, c.inter) : mmq_supported(c.dim, c.inter);
    const size_t M = c.max_tokens;
    ctx->max_pairs = (int)(M * c.topk);
    // room for the GEMV list, the MMQ plan of any m <= max_tokens (both grow with
    // m) and the single-row chunks of the small-batch routing
    const int m_small = (int)std::min<size_t>(M, ROUTE_SMALL_MAX_M);
    ctx->max_chunks = std::max(routed_chunk_bound(c, (int)M) + shared_chunk_count((int)M) + 1,
                               std::max(mmq_chunk_plan((int)M, c.topk, c.n_routed, true, false).total(),
                                        mmq_chunk_plan((int)M, c.topk, c.n_routed, true, true).total()));
    ctx->max_chunks = std::max(ctx->max_chunks, m_small * (c.topk + 1) + 1);
    layout_of(c, ctx->slot_bytes, ctx->off_w1, ctx->off_w3, ctx->off_w2);

    const size_t total = carve_scratch(ctx, M, false, nullptr);
    if (hipMalloc((void**)&ctx->dev, total) != hipSuccess) {
        delete ctx;
        return MOE_ENOMEM;
    }
    carve_scratch(ctx, M, false, ctx->dev);
    if (hipMemset(ctx->dev, 0, total) != hipSuccess) {
        moe_destroy(ctx);
        return MOE_EHIP;
    }
    const size_t E = c.n_routed;
    if (hipHostMalloc((void**)&ctx->slot_host, sizeof(int32_t) * E, hipHostMallocDefault) != hipSuccess) {
        moe_destroy(ctx);
        return MOE_ENOMEM;
    }
    for (size_t e = 0; e < E; ++e) ctx->slot_host[e] = -1;
    if (hipEventCreateWithFlags(&ctx->table_ev, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ctx->ev_fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ctx->ev_join, hipEventDisableTiming) != hipSuccess ||
        hipStreamCreateWithFlags(&ctx->side, hipStreamNonBlocking) != hipSuccess) {
        moe_destroy(ctx);
        return MOE_EHIP;
    }
    ctx->table_dirty = true;
    *out = ctx;
    return MOE_OK;
}

int moe_destroy(moe_ctx* ctx) {
    if (ctx == nullptr) return MOE_OK;
    (void)hipDeviceSynchronize();
    if (ctx->table_ev) (void)hipEventDestroy(ctx->table_ev);
    if (ctx->ev_fork) (void)hipEventDestroy(ctx->ev_fork);
    if (ctx->ev_join) (void)hipEventDestroy(ctx->ev_join);
    if (ctx->side) (void)hipStreamDestroy(ctx->side);
    if (ctx->copy) (void)hipStreamDestroy(ctx->copy);
    for (auto* v : {&ctx->ev_copy, &ctx->ev_wave, &ctx->ev_c0, &ctx->ev_c1})
        for (hipEvent_t e : *v) (void)hipEventDestroy(e);
    if (ctx->idx_host) (void)hipHostFree(ctx->idx_host);
    if (ctx->view_host) (void)hipHostFree(ctx->view_host);
    for (hipEvent_t e : ctx->ev_pool) (void)hipEventDestroy(e);
    for (hipEvent_t e : ctx->ev_comp) (void)hipEventDestroy(e);
    if (ctx->slot_host) (void)hipHostFree(ctx->slot_host);
    if (ctx->dev) (void)hipFree(ctx->dev);
    delete ctx;
    return MOE_OK;
}

int moe_set_slots(moe_ctx* ctx, void* arena_dev, int32_t n_slots) {
    if (ctx == nullptr || arena_dev == nullptr || n_slots < 1 || !aligned(arena_dev, 256)) return MOE_EINVAL;
    const int rc = table_mutable(ctx);
    if (rc != MOE_OK) return rc;
    ctx->arena = (uint8_t*)arena_dev;
    ctx->n_slots = n_slots;
    ctx->slot_owner.assign(n_slots, -1);
    ctx->slot_tick.assign(n_slots, 0);
    for (int e = 0; e < ctx->cfg.n_routed; ++e) ctx->slot_host[e] = -1;
    ctx->table_dirty = true;
    return MOE_OK;
}

int moe_slot_bind(moe_ctx* ctx, int32_t expert, int32_t slot) {
    if (ctx == nullptr) return MOE_EINVAL;
    if (ctx->arena == nullptr) return MOE_ESTATE;
    if (expert < 0 || expert >= ctx->cfg.n_routed || slot < 0 || slot >= ctx->n_slots) return MOE_EINVAL;
    const int owner = ctx->slot_owner[slot];
    if (owner >= 0 && owner != expert) return MOE_EINVAL;
    const int rc = table_mutable(ctx);
    if (rc != MOE_OK) return rc;
    const int old = ctx->slot_host[expert];
    if (old >= 0 && old != slot) ctx->slot_owner[old] = -1;
    ctx->slot_host[expert] = slot;
    ctx->slot_owner[slot] = expert;
    ctx->table_dirty = true;
    return MOE_OK;
}

int moe_slot_evict(moe_ctx* ctx, int32_t expert) {
    if (ctx == nullptr) return MOE_EINVAL;
    if (ctx->arena == nullptr) return MOE_ESTATE;
    if (expert < 0 || expert >= ctx->cfg.n_routed) return MOE_EINVAL;
    const int rc = table_mutable(ctx);
    if (rc != MOE_OK) return rc;
    const int old = ctx->slot_host[expert];
    if (old >= 0) ctx->slot_owner[old] = -1;
    ctx->slot_host[expert] = -1;
    ctx->table_dirty = true;
    return MOE_OK;
}

int moe_slot_of(const moe_ctx* ctx, int32_t expert, int32_t* slot) {
    if (ctx == nullptr || slot == nullptr || expert < 0 || expert >= ctx->cfg.n_routed) return MOE_EINVAL;
    *slot = ctx->slot_host[expert];
    return MOE_OK;
}

int moe_set_host_arena(moe_ctx* ctx, const void* pinned_host, size_t expert_stride) {
    if (ctx == nullptr) return MOE_EINVAL;
    if (pinned_host != nullptr && expert_stride < ctx->slot_bytes) return MOE_EINVAL;
    if (pinned_host != nullptr && ctx->copy == nullptr) {
        const size_t E = ctx->cfg.n_routed;
        if (hipStreamCreateWithFlags(&ctx->copy, hipStreamNonBlocking) != hipSuccess) return MOE_EHIP;
        if (hipHostMalloc((void**)&ctx->idx_host, sizeof(int32_t) * ctx->max_pairs, hipHostMallocDefault) != hipSuccess ||
            hipHostMalloc((void**)&ctx->view_host, sizeof(int32_t) * E * E, hipHostMallocDefault) != hipSuccess)
            return MOE_ENOMEM;
    }
    ctx->host_arena = (const uint8_t*)pinned_host;
    ctx->host_stride = expert_stride;
    return MOE_OK;
}

int moe_route(moe_ctx* ctx, const moe_weights* w, const void* x_bf16, int32_t m, float* weights_out,
              int32_t* idx_out, void* stream) {
    if (ctx == nullptr || x_bf16 == nullptr || weights_out == nullptr || idx_out == nullptr) return MOE_EINVAL;
    if (m < 1 || m > ctx->cfg.max_tokens || !aligned(x_bf16, 16)) return MOE_EINVAL;
    int rc = check_weights(ctx, w);
    if (rc != MOE_OK) return rc;
    return run_route(ctx, w, (const uint16_t*)x_bf16, m, idx_out, weights_out, (hipStream_t)stream);
}

// the routing copies of moe_forward_ex and the call count
static int finish_call(moe_ctx* ctx, float* weights_out, int32_t* idx_out, int P, hipStream_t st) {
    if (weights_out != nullptr &&
        hipMemcpyAsync(weights_out, ctx->gw, sizeof(float) * P, hipMemcpyDeviceToDevice, st) != hipSuccess)
        return MOE_EHIP;
    if (idx_out != nullptr &&
        hipMemcpyAsync(idx_out, ctx->idx, sizeof(int32_t) * P, hipMemcpyDeviceToDevice, st) != hipSuccess)
        return MOE_EHIP;
    ctx->stats.calls++;
    return MOE_OK;
}

// ---------------------------------------------------------------- miss streaming
// (metrale's ExpertLru and forward: route, read the picks back, gather the
// picked experts' slices into device slots, misses copied from the host arena
// on a side stream; MoeV41 struct documentation, forward / arena_of)

static hipEvent_t wave_event(std::vector<hipEvent_t>& pool, size_t w, bool timing) {
    while (pool.size() <= w) {
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, timing ? hipEventDefault : hipEventDisableTiming) != hipSuccess) return nullptr;
        pool.push_back(e);
    }
    return pool[w];
}

static void collect_fetch_times(const moe_ctx* ctx) {
    for (const auto& pr : ctx->fetch_pending) {
        float ms = 0.f;
        if (hipEventSynchronize(pr.second) == hipSuccess && hipEventElapsedTime(&ms, pr.first, pr.second) == hipSuccess)
            ctx->stats.fetch_ms += ms;
    }
    ctx->fetch_pending.clear();
    for (const auto& pr : ctx->comp_pending) {
        float ms = 0.f;
        if (hipEventSynchronize(pr.second) == hipSuccess && hipEventElapsedTime(&ms, pr.first, pr.second) == hipSuccess)
            ctx->stats.compute_ms += ms;
    }
    ctx->comp_pending.clear();
}

// the next start/stop pair for a call's expert-compute time (nullptr pair: none)
static std::pair<hipEvent_t, hipEvent_t> compute_events(moe_ctx* ctx) {
    if (ctx->comp_pending.size() >= 1024) collect_fetch_times(ctx);   // bounded: read the oldest back
    if (ctx->comp_pending.empty()) ctx->comp_next = 0;   // every pair was read back
    while (ctx->ev_comp.size() < ctx->comp_next + 2) {
        hipEvent_t e = nullptr;
        if (hipEventCreate(&e) != hipSuccess) return {nullptr, nullptr};
        ctx->ev_comp.push_back(e);
    }
    const size_t i = ctx->comp_next;
    ctx->comp_next += 2;
    return {ctx->ev_comp[i], ctx->ev_comp[i + 1]};
}

// Read the picks back (the one host wait of a streamed call) and split the
// distinct experts into waves that fit the slots: resident ones first, so no
// wave evicts an expert a later wave still finds resident; several waves take
// half the slots each, so one wave's copies never overwrite the slots the
// wave before it is still computing with.
static int plan_waves(moe_ctx* ctx, int P, hipStream_t st, std::vector<std::vector<int>>& waves) {
    waves.clear();
    const auto t0 = std::chrono::steady_clock::now();
    if (hipMemcpyAsync(ctx->idx_host, ctx->idx, sizeof(int32_t) * P, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
        return MOE_EHIP;
    ctx->stats.route_ms += std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t0).count();
    collect_fetch_times(ctx);
    std::vector<char> seen(ctx->cfg.n_routed, 0);
    std::vector<int> hits, misses;
    for (int p = 0; p < P; ++p) {
        const int e = ctx->idx_host[p];
        if (e < 0 || e >= ctx->cfg.n_routed || seen[e]) continue;
        seen[e] = 1;
    }
    for (int e = 0; e < ctx->cfg.n_routed; ++e)
        if (seen[e]) (ctx->slot_host[e] >= 0 ? hits : misses).push_back(e);
    ctx->stats.hits += hits.size();
    std::vector<int> order(hits);
    order.insert(order.end(), misses.begin(), misses.end());
    const int n = (int)order.size();
    const int cap = n <= ctx->n_slots ? ctx->n_slots : std::max(1, ctx->n_slots / 2);
    for (int i = 0; i < n; i += cap)
        waves.emplace_back(order.begin() + i, order.begin() + std::min(n, i + cap));
    return MOE_OK;
}

// Make wave w resident (least recently used slots outside this wave and the one
// before it are reused), then point the device table at it: the wave's experts
// at their slots, the experts of the other waves at SLOT_SKIP.
static int run_wave(moe_ctx* ctx, const std::vector<std::vector<int>>& waves, size_t w, hipStream_t st) {
    int rc = table_mutable(ctx);
    if (rc != MOE_OK) return rc;
    const int E = ctx->cfg.n_routed;
    std::vector<char> keep(ctx->n_slots, 0);
    for (size_t v = (w > 0 ? w - 1 : 0); v <= w; ++v)
        for (int e : waves[v])
            if (ctx->slot_host[e] >= 0) keep[ctx->slot_host[e]] = 1;
    ++ctx->tick;
    hipEvent_t c0 = wave_event(ctx->ev_c0, w, true), c1 = wave_event(ctx->ev_c1, w, true);
    hipEvent_t ec = wave_event(ctx->ev_copy, w, false);
    if (c0 == nullptr || c1 == nullptr || ec == nullptr) return MOE_EHIP;
    // the slots of wave w - 2 may be overwritten: wait until that wave's kernels are done
    if (w >= 2 && hipStreamWaitEvent(ctx->copy, ctx->ev_wave[w - 2], 0) != hipSuccess) return MOE_EHIP;
    bool copied = false;
    for (int e : waves[w]) {
        if (ctx->slot_host[e] < 0) {
            int victim = -1;
            for (int sl = 0; sl < ctx->n_slots; ++sl) {
                if (keep[sl]) continue;
                if (victim < 0 || (ctx->slot_owner[sl] < 0 && ctx->slot_owner[victim] >= 0) ||
                    ((ctx->slot_owner[sl] < 0) == (ctx->slot_owner[victim] < 0) && ctx->slot_tick[sl] < ctx->slot_tick[victim]))
                    victim = sl;
            }
            if (victim < 0) return MOE_ESTATE;   // cannot happen: a wave takes at most half the slots
            if (!copied && hipEventRecord(c0, ctx->copy) != hipSuccess) return MOE_EHIP;
            copied = true;
            if (ctx->slot_owner[victim] >= 0) ctx->slot_host[ctx->slot_owner[victim]] = SLOT_NONE;
            if (hipMemcpyAsync(ctx->arena + (size_t)victim * ctx->slot_bytes, ctx->host_arena + (size_t)e * ctx->host_stride,
                               ctx->slot_bytes, hipMemcpyHostToDevice, ctx->copy) != hipSuccess)
                return MOE_EHIP;
            ctx->slot_owner[victim] = e;
            ctx->slot_host[e] = victim;
            ctx->stats.misses++;
            ctx->stats.bytes_copied += ctx->slot_bytes;
        }
        keep[ctx->slot_host[e]] = 1;
        ctx->slot_tick[ctx->slot_host[e]] = ctx->tick;
    }
    if (copied) {
        if (hipEventRecord(c1, ctx->copy) != hipSuccess || hipEventRecord(ec, ctx->copy) != hipSuccess ||
            hipStreamWaitEvent(st, ec, 0) != hipSuccess)
            return MOE_EHIP;
        ctx->fetch_pending.emplace_back(c0, c1);
    }
    int32_t* view = ctx->view_host + w * (size_t)E;
    for (int e = 0; e < E; ++e) view[e] = ctx->slot_host[e];
    for (size_t v = 0; v < waves.size(); ++v)
        if (v != w)
            for (int e : waves[v]) view[e] = SLOT_SKIP;
    if (hipMemcpyAsync(ctx->slot_table_dev, view, sizeof(int32_t) * E, hipMemcpyHostToDevice, st) != hipSuccess)
        return MOE_EHIP;
    ctx->table_dirty = true;   // the next call uploads the residency table again
    ctx->stats.waves++;
    return MOE_OK;
}

int moe_forward_ex(moe_ctx* ctx, const moe_weights* w, const void* x_bf16, int32_t m, void* out_bf16,
                   float* weights_out, int32_t* idx_out, void* stream) {
    if (ctx == nullptr || x_bf16 == nullptr || out_bf16 == nullptr) return MOE_EINVAL;
    if (m < 1 || m > ctx->cfg.max_tokens) return MOE_EINVAL;
    if (!aligned(x_bf16, 16) || !aligned(out_bf16, 16)) return MOE_EINVAL;
    int rc = check_weights(ctx, w);
    if (rc != MOE_OK) return rc;
    if (ctx->arena == nullptr) return MOE_ESTATE;
    const moe_cfg& c = ctx->cfg;
    const hipStream_t st = (hipStream_t)stream;
    const uint16_t* x = (const uint16_t*)x_bf16;
    const int P = m * c.topk;

    rc = upload_table(ctx, st);
    if (rc != MOE_OK) return rc;
    const bool bf16_shared = w->shared_fmt == MOE_SHARED_BF16;
    const CallPlan pl = plan_call(ctx, m, w->shared_fmt);
    const bool small = pl.small, use_mmq = pl.use_mmq, fp4 = pl.fp4, shared_fused = pl.shared_fused;
    SharedRows sr_a{}, sr_b{}, sr_c{};
    if (shared_fused) {
        sr_a.w1 = (const uint16_t*)w->shared_w1;
        sr_a.w3 = (const uint16_t*)w->shared_w3;
        sr_a.x = x;
        sr_a.h = (uint16_t*)ctx->h_shared;
        sr_a.D = c.dim;
        sr_a.I = c.inter;
        sr_a.m = m;
        sr_a.limit = c.swiglu_limit;
        sr_b = sr_a;
        sr_a.row0 = 0;
        sr_a.rows = pl.sh_router_rows;
        sr_b.w1 = sr_b.w3 = nullptr;
        sr_b.w2 = (const uint16_t*)w->shared_w2;
        sr_b.ys = ctx->ys;
        sr_b.row0 = 0;
        sr_b.rows = pl.sh_topk_rows;
        sr_c = sr_b;
        sr_c.row0 = pl.sh_topk_rows;
        sr_c.rows = pl.sh_gateup_rows;
    }
    if (bf16_shared && !shared_fused) {
        // the shared expert needs only x: run it beside the routing and the routed experts
        if (hipEventRecord(ctx->ev_fork, st) != hipSuccess || hipStreamWaitEvent(ctx->side, ctx->ev_fork, 0) != hipSuccess)
            return MOE_EHIP;
        if (small) {
            rc = timed(ctx, ctx->side, MOE_K_SHARED_GATEUP, [&] {
                return launch_shared_bf16_gateup(x, m, c.dim, c.inter, (const uint16_t*)w->shared_w1,
                                                 (const uint16_t*)w->shared_w3, (uint16_t*)ctx->h_shared,
                                                 c.swiglu_limit, ctx->side);
            });
            if (rc != MOE_OK) return rc;
            rc = timed(ctx, ctx->side, MOE_K_SHARED_DOWN, [&] {
                return launch_shared_bf16_down((const uint16_t*)ctx->h_shared, m, c.dim, c.inter,
                                               (const uint16_t*)w->shared_w2, ctx->ys, ctx->side);
            });
        } else {
            rc = timed(ctx, ctx->side, MOE_K_SHARED_GATEUP, [&] {
                return launch_shared_bf16_gemm(x, m, c.dim, c.inter, (const uint16_t*)w->shared_w1,
                                               (const uint16_t*)w->shared_w3, (const uint16_t*)w->shared_w2,
                                               (uint16_t*)ctx->h_shared, ctx->ys, c.swiglu_limit, ctx->side);
            });
        }
        if (rc != MOE_OK) return rc;
        if (hipEventRecord(ctx->ev_join, ctx->side) != hipSuccess) return MOE_EHIP;
    }
    const bool kq = w->shared_fmt == MOE_SHARED_KQUANT;
    const ChunkPlan plan = mmq_chunk_plan(m, c.topk, c.n_routed, kq, ctx->mixed && !fp4);
    if (pl.fold_topk) {
        RouteSel ro{};
        ro.bias = w->router_bias;
        ro.E = c.n_routed;
        ro.k = c.topk;
        ro.gate_temp = c.gate_temp;
        ro.norm = c.norm_topk_prob;
        ro.route_scale = c.route_scale;
        ro.idx = ctx->idx;
        ro.gw = ctx->gw;
        ro.err = ctx->err;
        ro.shared_chunks = kq ? 1 : 0;
        ro.offsets = ctx->offsets;
        ro.active = ctx->active;
        ro.n_active = ctx->n_active;
        ro.perm = ctx->perm;
        ro.inv = ctx->inv;
        ro.chunks = ctx->chunks;
        ro.n_chunks = ctx->n_chunks;
        ro.slot_table = ctx->slot_table_dev;
        ro.arrive = ctx->arrive;
        rc = timed(ctx, st, MOE_K_ROUTER, [&] {
            return launch_router_select(x, m, (const uint16_t*)w->router_w, c.dim, ctx->logits, ctx->xq, ctx->xd,
                                        ctx->xs16, ctx->xs16f, ro, st, shared_fused ? &sr_a : nullptr);
        });
        if (rc != MOE_OK) return rc;
    } else if (small) {
        rc = timed(ctx, st, MOE_K_ROUTER, [&] {
            return launch_router_quant(x, m, (const uint16_t*)w->router_w, c.dim, c.n_routed, ctx->logits, ctx->xq,
                                       ctx->xd, ctx->xs16, ctx->xs16f, st, shared_fused ? &sr_a : nullptr);
        });
        if (rc != MOE_OK) return rc;
        rc = timed(ctx, st, MOE_K_TOPK, [&] {
            return launch_route_small(ctx->logits, w->router_bias, m, c.n_routed, c.topk, c.gate_temp,
                                      c.norm_topk_prob, c.route_scale, ctx->idx, ctx->gw, ctx->err, kq ? 1 : 0,
                                      ctx->offsets, ctx->active, ctx->n_active, ctx->perm, ctx->inv, ctx->chunks,
                                      ctx->n_chunks, ctx->slot_table_dev, st, shared_fused ? &sr_b : nullptr);
        });
        if (rc != MOE_OK) return rc;
    } else {
        int splits = 1;
        rc = timed(ctx, st, MOE_K_ROUTER, [&] {
            hipError_t e = launch_router_gemm(x, m, (const uint16_t*)w->router_w, c.dim, c.n_routed, ctx->logits,
                                              ctx->logit_rows, &splits, st);
            if (e != hipSuccess || fp4) return e;   // MXFP4 experts read x itself
            return launch_quantize_rows(x, m, c.dim, ctx->xq, ctx->xd, ctx->xs16, ctx->xs16f, ctx->xs16b, st);
        });
        if (rc != MOE_OK) return rc;
        rc = timed(ctx, st, MOE_K_TOPK, [&] {
            return launch_topk(ctx->logits, splits, w->router_bias, m, c.n_routed, c.topk, c.gate_temp,
                               c.norm_topk_prob, c.route_scale, ctx->idx, ctx->gw, ctx->err, st);
        });
        if (rc != MOE_OK) return rc;
        rc = timed(ctx, st, MOE_K_BUCKET, [&] {
            return launch_bucket(ctx->idx, m, c.topk, c.n_routed, kq ? 1 : 0, use_mmq ? &plan : nullptr, ctx->offsets, ctx->active,
                                 ctx->n_active, ctx->perm, ctx->inv, ctx->chunks, ctx->n_chunks, st);
        });
        if (rc != MOE_OK) return rc;
    }

    ExpertArgs a;
    a.chunks = ctx->chunks;
    a.n_chunks = ctx->n_chunks;
    a.perm = ctx->perm;
    a.inv = ctx->inv;
    a.topk = c.topk;
    a.slot_table = ctx->slot_table_dev;
    a.arena = ctx->arena;
    a.slot_bytes = ctx->slot_bytes;
    a.off_w1 = ctx->off_w1;
    a.off_w3 = ctx->off_w3;
    a.off_w2 = ctx->off_w2;
    a.sh_w1 = kq ? (const uint8_t*)w->shared_w1 : nullptr;
    a.sh_w3 = kq ? (const uint8_t*)w->shared_w3 : nullptr;
    a.sh_w2 = kq ? (const uint8_t*)w->shared_w2 : nullptr;
    a.x16 = x;
    a.xq = ctx->xq;
    a.xd = ctx->xd;
    a.xs16 = ctx->xs16;
    a.xs16f = ctx->xs16f;
    a.xs16b = ctx->xs16b;
    a.h_routed = ctx->h_routed;
    a.hrec = ctx->hrec;
    a.h_shared = ctx->h_shared;
    a.hq_routed = ctx->hq_routed;
    a.hd_routed = ctx->hd_routed;
    a.hs_routed = ctx->hs_routed;
    a.hq_shared = ctx->hq_shared;
    a.hd_shared = ctx->hd_shared;
    a.hs_shared = ctx->hs_shared;
    a.e_rows = ctx->e_rows;
    a.ys = ctx->ys;
    a.D = c.dim;
    a.I = c.inter;
    a.limit = c.swiglu_limit;
    a.err = ctx->err;
    const int chunks = routed_chunk_bound(c, m) + (kq ? shared_chunk_count(m) : 0);
    const float* ys = w->shared_fmt == MOE_SHARED_BF16 ? ctx->ys : nullptr;

    // with a host arena: read the picks back and stream the missing experts in
    std::vector<std::vector<int>> waves;
    if (ctx->host_arena != nullptr) {
        rc = plan_waves(ctx, P, st, waves);
        if (rc != MOE_OK) return rc;
        if (waves.size() == 1) {
            rc = run_wave(ctx, waves, 0, st);
            if (rc != MOE_OK) return rc;
            if (small && hip_status(launch_refresh_slots(ctx->chunks, ctx->n_chunks, ctx->slot_table_dev, st)) != MOE_OK)
                return MOE_EHIP;
        }
    }
    // the expert-compute time of this call (calls with a host arena or with profiling on)
    std::pair<hipEvent_t, hipEvent_t> comp{nullptr, nullptr};
    if (ctx->host_arena != nullptr || ctx->prof) {
        comp = compute_events(ctx);
        if (comp.first == nullptr || hipEventRecord(comp.first, st) != hipSuccess) return MOE_EHIP;
    }
    auto end_compute = [&]() -> int {
        if (comp.first == nullptr) return MOE_OK;
        if (hipEventRecord(comp.second, st) != hipSuccess) return MOE_EHIP;
        ctx->comp_pending.push_back(comp);
        return MOE_OK;
    };
    if (small && ctx->decode_ok && waves.size() <= 1) {
        // one single-row chunk per pick (and per token of a K-quant shared expert):
        // gate/up writes q8_1(h) records, down accumulates G E per token and stores bf16
        const int nch = P + (kq ? m : 0);
        rc = timed(ctx, st, MOE_K_GATEUP,
                   [&] { return launch_gateup_q8(a, P, nch, st, sr_c.rows > 0 ? &sr_c : nullptr); });
        if (rc != MOE_OK) return rc;
        if (bf16_shared && !shared_fused && hipStreamWaitEvent(st, ctx->ev_join, 0) != hipSuccess) return MOE_EHIP;
        rc = timed(ctx, st, MOE_K_DOWN, [&] {
            return launch_down_combine(a, P, m, nch, ys, (uint16_t*)out_bf16, st);
        });
        if (rc != MOE_OK) return rc;
        rc = end_compute();
        if (rc != MOE_OK) return rc;
        return finish_call(ctx, weights_out, idx_out, P, st);
    }
    // chunks of at most GEMV_ROWS rows, or single rows on the small-batch routing;
    // with several slot waves the kernels run once per wave and skip the other waves' experts
    const int rows_max = small ? 1 : std::min(m, GEMV_ROWS);
    const int nch = small ? P + (kq ? m : 0) : chunks;
    const size_t n_runs = std::max<size_t>(1, waves.size());
    const ExpertArgs a_all = a;   // each wave's launches take a copy (with its own chunk lists)
    for (size_t wv = 0; wv < n_runs; ++wv) {
        ExpertArgs a = a_all;
        if (waves.size() > 1) {
            rc = run_wave(ctx, waves, wv, st);
            if (rc != MOE_OK) return rc;
            if (use_mmq) {   // this wave's chunks only, so that its launches spread them over the XCDs
                if (hip_status(launch_compact_wave(a_all.chunks, a_all.n_chunks, ctx->slot_table_dev, wv == 0, plan,
                                                   ctx->wave_chunks, ctx->wave_n_chunks, st)) != MOE_OK)
                    return MOE_EHIP;
                a.chunks = ctx->wave_chunks;
                a.n_chunks = ctx->wave_n_chunks;
            }
        }
        if (use_mmq && fp4) {   // bf16 h, no q8_1 step
            rc = timed(ctx, st, MOE_K_GATEUP, [&] { return launch_fp4_mmq(a, plan, true, st); });
            if (rc != MOE_OK) return rc;
            rc = timed(ctx, st, MOE_K_DOWN, [&] { return launch_fp4_mmq(a, plan, false, st); });
            if (rc != MOE_OK) return rc;
        } else if (use_mmq) {
            // a mixed plan's small groups on the GEMV kernels, the rest on MMQ
            ExpertArgs ag = a;
            ag.chunks = a.chunks + plan.base[GEMV_LIST];
            ag.n_chunks = a.n_chunks + GEMV_LIST;
            if (plan.cap[GEMV_LIST] > 0) {
                rc = timed(ctx, st, MOE_K_GATEUP,
                           [&] { return launch_gateup_q2k(ag, GEMV_ROWS, plan.cap[GEMV_LIST], st); });
                if (rc != MOE_OK) return rc;
            }
            rc = timed(ctx, st, MOE_K_GATEUP, [&] { return launch_mmq(a, plan, true, st); });
            if (rc != MOE_OK) return rc;
            rc = timed(ctx, st, MOE_K_QUANT, [&] { return launch_quantize_h(a, P, kq ? m : 0, st); });
            if (rc != MOE_OK) return rc;
            if (plan.cap[GEMV_LIST] > 0) {
                rc = timed(ctx, st, MOE_K_DOWN,
                           [&] { return launch_down_q3k(ag, GEMV_ROWS, plan.cap[GEMV_LIST], st); });
                if (rc != MOE_OK) return rc;
            }
            rc = timed(ctx, st, MOE_K_DOWN, [&] { return launch_mmq(a, plan, false, st); });
            if (rc != MOE_OK) return rc;
        } else {
            if (c.expert_fmt == MOE_EXPERT_MXFP4) {   // bf16 h, no q8_1 step
                rc = timed(ctx, st, MOE_K_GATEUP, [&] { return launch_fp4(a, rows_max, nch, true, st); });
                if (rc != MOE_OK) return rc;
                rc = timed(ctx, st, MOE_K_DOWN, [&] { return launch_fp4(a, rows_max, nch, false, st); });
                if (rc != MOE_OK) return rc;
            } else {
                rc = timed(ctx, st, MOE_K_GATEUP, [&] { return launch_gateup_q2k(a, rows_max, nch, st); });
                if (rc != MOE_OK) return rc;
                rc = timed(ctx, st, MOE_K_QUANT, [&] { return launch_quantize_h(a, P, kq ? m : 0, st); });
                if (rc != MOE_OK) return rc;
                rc = timed(ctx, st, MOE_K_DOWN, [&] { return launch_down_q3k(a, rows_max, nch, st); });
                if (rc != MOE_OK) return rc;
            }
        }
        if (waves.size() > 1) {
            hipEvent_t ew = wave_event(ctx->ev_wave, wv, false);
            if (ew == nullptr || hipEventRecord(ew, st) != hipSuccess) return MOE_EHIP;
        }
    }
    if (bf16_shared && !shared_fused && hipStreamWaitEvent(st, ctx->ev_join, 0) != hipSuccess) return MOE_EHIP;
    const float* ys_all = w->shared_fmt == MOE_SHARED_NONE ? nullptr : ctx->ys;
    rc = timed(ctx, st, MOE_K_COMBINE, [&] {
        return launch_combine(ctx->e_rows, ys_all, ctx->gw, ctx->inv, m, c.topk, c.dim, (uint16_t*)out_bf16, st);
    });
    if (rc != MOE_OK) return rc;
    rc = end_compute();
    if (rc != MOE_OK) return rc;
    return finish_call(ctx, weights_out, idx_out, P, st);
}

int moe_forward(moe_ctx* ctx, const moe_weights* w, const void* x_bf16, int32_t m, void* out_bf16, void* stream) {
    return moe_forward_ex(ctx, w, x_bf16, m, out_bf16, nullptr, nullptr, stream);
}

int moe_plan_call(const moe_ctx* ctx, int32_t m, int32_t shared_fmt, moe_plan* out) {
    if (ctx == nullptr || out == nullptr || m < 1 || m > ctx->cfg.max_tokens) return MOE_EINVAL;
    if (shared_fmt != MOE_SHARED_NONE && shared_fmt != MOE_SHARED_BF16 && shared_fmt != MOE_SHARED_KQUANT)
        return MOE_EINVAL;
    const CallPlan pl = plan_call(ctx, m, shared_fmt);
    out->small_routing = pl.small ? 1 : 0;
    out->expert_path = pl.use_mmq ? MOE_PATH_MMQ : pl.decode ? MOE_PATH_DECODE : MOE_PATH_GEMV;
    out->shared_rows_router = pl.sh_router_rows;
    out->shared_rows_topk = pl.sh_topk_rows;
    out->shared_rows_gateup = pl.sh_gateup_rows;
    return MOE_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- the no-allocation variant
// Scratch of moe_forward_static: one copy per device (each GPU the library runs
// on holds it until the process ends). Host code never uses this name as an
// address: it takes the device's own address of the array from
// hipGetSymbolAddress, once per device, and passes that to the kernels.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_dev[MAX_DEVICES] = {};

// the current device's address of `scratch`, looked up on its first use there
int static_scratch(uint8_t** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
    if (dev < 0 || dev >= MAX_DEVICES) return MOE_EINVAL;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_EHIP;
        g_scratch_dev[dev] = static_cast<uint8_t*>(p);
    }
    *out = g_scratch_dev[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward_static(const moe_cfg* cfg, const moe_weights* w, const void* arena, const int32_t* slot_table,
                       const void* x_bf16, int32_t m, void* out_bf16, float* weights_out, int32_t* idx_out,
                       int32_t* status, void* stream) {
    if (check_cfg(cfg) != MOE_OK || cfg->expert_fmt != MOE_EXPERT_KQUANT || !decode_supported(cfg->dim, cfg->inter))
        return MOE_EINVAL;
    if (arena == nullptr || slot_table == nullptr || x_bf16 == nullptr || out_bf16 == nullptr) return MOE_EINVAL;
    if (m < 1 || m > ROUTE_SMALL_MAX_M || m * cfg->topk > ROUTE_SMALL_MAX_PAIRS) return MOE_EINVAL;
    if (!aligned(arena, 256) || !aligned(slot_table, 4) || !aligned(x_bf16, 16) || !aligned(out_bf16, 16) ||
        !aligned(status, 4))
        return MOE_EINVAL;
    // a context on the stack that owns nothing: the caller's arena and slot table,
    // and views into the static scratch sized for this call's m tokens
    moe_ctx tmp{};
    tmp.cfg = *cfg;
    tmp.cfg.max_tokens = m;
    tmp.decode_ok = true;
    tmp.mmq_ok = false;
    tmp.max_pairs = m * cfg->topk;
    tmp.max_chunks = m * (cfg->topk + 1) + 1;
    layout_of(tmp.cfg, tmp.slot_bytes, tmp.off_w1, tmp.off_w3, tmp.off_w2);
    tmp.arena = (uint8_t*)arena;
    tmp.slot_table_dev = const_cast<int32_t*>(slot_table);
    tmp.table_dirty = false;
    if (carve_scratch(&tmp, m, true, nullptr) > MOE_STATIC_SCRATCH_BYTES) return MOE_ESCRATCH;
    uint8_t* base = nullptr;
    const int rc = static_scratch(&base);
    if (rc != MOE_OK) return rc;
    carve_scratch(&tmp, m, true, base);
    if (status != nullptr) tmp.err = status;
    return moe_forward_ex(&tmp, w, x_bf16, m, out_bf16, weights_out, idx_out, stream);
}

int moe_quantize_q8_1(const void* x_bf16, int32_t rows, int32_t cols, int8_t* q_out, float* d_out, void* stream) {
    if (x_bf16 == nullptr || q_out == nullptr || d_out == nullptr || rows < 1 || cols < QB || cols % QB) return MOE_EINVAL;
    if (!aligned(x_bf16, 16) || !aligned(q_out, 16) || !aligned(d_out, 4)) return MOE_EINVAL;
    return hip_status(
        launch_quantize_rows((const uint16_t*)x_bf16, rows, cols, q_out, d_out, nullptr, nullptr, nullptr, (hipStream_t)stream));
}

int moe_check(moe_ctx* ctx, void* stream) {
    if (ctx == nullptr) return MOE_EINVAL;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOE_EHIP;
    int32_t word = 0;
    if (hipMemcpy(&word, ctx->err, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return MOE_EHIP;
    const int32_t zero = 0;
    if (hipMemcpy(ctx->err, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return MOE_EHIP;
    if (word & ERR_NONFINITE) return MOE_ENONFINITE;
    if (word & ERR_NOTRESIDENT) return MOE_ENOTRESIDENT;
    return MOE_OK;
}

int moe_set_dispatch(moe_ctx* ctx, int32_t mode) {
    if (ctx == nullptr || (mode != MOE_DISPATCH_MIXED && mode != MOE_DISPATCH_MMQ)) return MOE_EINVAL;
    ctx->mixed = mode == MOE_DISPATCH_MIXED;
    return MOE_OK;
}

int moe_set_profiling(moe_ctx* ctx, int32_t on) {
    if (ctx == nullptr) return MOE_EINVAL;
    if (ctx->prof && !on) {
        // drop what was recorded
        if (hipDeviceSynchronize() != hipSuccess) return MOE_EHIP;
        ctx->marks.clear();
        ctx->ev_next = 0;
    }
    ctx->prof = on != 0;
    for (int i = 0; i < MOE_K_COUNT; ++i) {
        ctx->k_ms[i] = 0.0;
        ctx->k_n[i] = 0;
    }
    return MOE_OK;
}

int moe_kernel_times(moe_ctx* ctx, double* ms_sum, int64_t* launches, int32_t n) {
    if (ctx == nullptr || ms_sum == nullptr || launches == nullptr || n < 0) return MOE_EINVAL;
    if (hipDeviceSynchronize() != hipSuccess) return MOE_EHIP;
    for (const auto& mk : ctx->marks) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, mk.a, mk.b) != hipSuccess) return MOE_EHIP;
        ctx->k_ms[mk.kind] += ms;
        ctx->k_n[mk.kind] += 1;
    }
    ctx->marks.clear();
    ctx->ev_next = 0;
    for (int i = 0; i < n && i < MOE_K_COUNT; ++i) {
        ms_sum[i] = ctx->k_ms[i];
        launches[i] = ctx->k_n[i];
        ctx->k_ms[i] = 0.0;
        ctx->k_n[i] = 0;
    }
    return MOE_OK;
}

int moe_get_stats(const moe_ctx* ctx, moe_stats* out) {
    if (ctx == nullptr || out == nullptr) return MOE_EINVAL;
    if (hipDeviceSynchronize() != hipSuccess) return MOE_EHIP;
    collect_fetch_times(ctx);
    uint32_t near = 0;
    if (hipMemcpy(&near, ctx->err + ERR_NEAR_TIES, sizeof(near), hipMemcpyDeviceToHost) != hipSuccess)
        return MOE_EHIP;
    *out = ctx->stats;
    out->near_ties = near;
    return MOE_OK;
}

int moe_reset_stats(moe_ctx* ctx) {
    if (ctx == nullptr) return MOE_EINVAL;
    if (hipDeviceSynchronize() != hipSuccess) return MOE_EHIP;
    collect_fetch_times(ctx);
    std::memset(&ctx->stats, 0, sizeof(ctx->stats));
    const uint32_t zero = 0;
    if (hipMemcpy(ctx->err + ERR_NEAR_TIES, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess)
        return MOE_EHIP;
    return MOE_OK;
}

}  // extern "C"
