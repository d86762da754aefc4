// Launchers shared between the kernel translation units and the host library.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_common.h"
#include "shared_rows.h"

namespace moe {

// Per-kernel timing. While a sink is installed on the calling thread, every
// launch below carries a start and a stop event that take the kernel's own
// begin and end timestamps (hipExtLaunchKernel), the interval a kernel trace
// reports; the sink supplies the events and remembers them.
struct LaunchTimer {
    virtual bool next_pair(hipEvent_t* start, hipEvent_t* stop) = 0;
};
extern thread_local LaunchTimer* g_launch_timer;

template <typename... P, typename... A>
hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t st, A... args) {
    if (g_launch_timer != nullptr) {
        hipEvent_t e0 = nullptr, e1 = nullptr;
        if (!g_launch_timer->next_pair(&e0, &e1)) return hipErrorOutOfMemory;
        hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, e0, e1, 0u, static_cast<P>(args)...);
    } else {
        hipLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, static_cast<P>(args)...);
    }
    return hipGetLastError();
}

struct GemvGeom {
    int P;          // rows processed in parallel
    int threads;    // workgroup size
    int R;          // rows per tile
    int tiles;      // tiles per chunk
    int lds_base;   // LDS bytes before the per-row-slot reduction area
    int lds_per_t;  // reduction bytes per token row
};

GemvGeom gateup_geom(int D, int I);
GemvGeom down_geom(int D, int I);

constexpr int MMQ_ROWS = 64;   // the most token rows one MMQ chunk holds (four 16-row sub-tiles)
// MMQ chunk classes by expert-group size: a group of <= 16 rows is one chunk of
// class 0 (one sub-tile), 17..32 rows one chunk of class 1 (two sub-tiles),
// more rows are 64-row chunks of class 2 (four sub-tiles, the last one
// ragged). Each class is launched with its own kernel instance, so chunks of
// lightly used experts do not carry the registers of four sub-tiles.
constexpr int MMQ_CLASSES = 3;
constexpr int MMQ_CLASS_MAX[MMQ_CLASSES] = {16, 32, MMQ_ROWS};
// A mixed plan (GEMVs for groups of up to GEMV_ROWS rows, MMQ above, as the
// pages dispatch by group size) adds a fourth list of GEMV chunks; the MMQ
// classes then hold groups of more than GEMV_ROWS rows only.
constexpr int GEMV_LIST = MMQ_CLASSES;
constexpr int PLAN_LISTS = MMQ_CLASSES + 1;
struct ChunkPlan {
    int base[PLAN_LISTS];   // first slot of each list in the chunk array
    int cap[PLAN_LISTS];    // slots reserved (an upper bound of the list's chunks)
    bool mixed;
    int total() const { return base[GEMV_LIST] + cap[GEMV_LIST]; }
};
// P = m * k picks over E experts; `shared` adds the K-quant shared expert's m rows
// (in the list its m rows fall in, like a routed group of m rows)
inline ChunkPlan mmq_chunk_plan(int m, int k, int E, bool shared, bool mixed) {
    const int P = m * k, act = P < E ? P : E;
    ChunkPlan pl;
    pl.mixed = mixed;
    const bool sh_gemv = shared && mixed && m <= GEMV_ROWS;
    const int g0 = mixed ? (P / (GEMV_ROWS + 1) < act ? P / (GEMV_ROWS + 1) : act) : act;
    pl.cap[0] = g0 + (shared && !sh_gemv && m <= 16 ? 1 : 0);
    pl.cap[1] = P / 17 + (shared && m > 16 && m <= 32 ? 1 : 0);
    // groups of v > 32 rows: sum ceil(v / 64) <= P / 64 + (number of such groups) <= P / 64 + P / 33
    pl.cap[2] = P / MMQ_ROWS + P / 33 + 1 + (shared && m > 32 ? (m + MMQ_ROWS - 1) / MMQ_ROWS : 0);
    pl.cap[GEMV_LIST] = mixed ? act + (sh_gemv ? 1 : 0) : 0;
    pl.base[0] = 0;
    for (int c = 1; c < PLAN_LISTS; ++c) pl.base[c] = pl.base[c - 1] + pl.cap[c - 1];
    return pl;
}

// router logits for m tokens, plus q8_1 of x in the same launch when xq != NULL (with
// the per-16 quant sums as i32 and as fp16(d) * sum in f32 when those are non-NULL)
hipError_t launch_router_quant(const uint16_t* x, int m, const uint16_t* wr, int D, int E, float* logits,
                               int8_t* xq, float* xd, int32_t* xs16, float* xs16f, hipStream_t st,
                               const SharedRows* sr = nullptr);
// The selection's parameters and outputs when the router launch selects (the
// top-k, its weights, the bucketing and the chunk list of route_m1 / route_small). `arrive`: ROUTER_ARRIVE_WORDS words of arrival
// counters (a top counter, then one per group of router workgroups, one 128-byte
// line apart), every one 0 between calls.
constexpr int ARRIVE_GROUPS = 16;
constexpr int ARRIVE_STRIDE = 32;
constexpr int ROUTER_ARRIVE_WORDS = (1 + ARRIVE_GROUPS) * ARRIVE_STRIDE;
struct RouteSel {
    const float* bias;
    int E, k;
    float gate_temp;
    int norm;
    float route_scale;
    int32_t* idx;
    float* gw;
    int32_t* err;
    int shared_chunks;
    int32_t *offsets, *active, *n_active, *perm, *inv;
    Chunk* chunks;
    int32_t* n_chunks;
    const int32_t* slot_table;
    uint32_t* arrive;
};
// Up to 8 tokens: the router launch also selects (its last router workgroup to
// finish runs the top-k, and at 2..8 tokens the bucketing), so that no top-k
// launch follows. k <= 64; E <= 1024 at one token, E <= 384 and m k <= 512 above.
bool router_select_ok(int E, int k, int m);
hipError_t launch_router_select(const uint16_t* x, int m, const uint16_t* wr, int D, float* logits, int8_t* xq,
                                float* xd, int32_t* xs16, float* xs16f, const RouteSel& ro, hipStream_t st,
                                const SharedRows* sr = nullptr);
// top-k and bucketing in one workgroup, for m * topk <= 512 and m <= 8
constexpr int ROUTE_SMALL_MAX_M = 8;
constexpr int ROUTE_SMALL_MAX_PAIRS = 512;
hipError_t launch_route_small(const float* logits, const float* bias, int m, int E, int k, float gate_temp,
                              int norm, float route_scale, int32_t* idx, float* gw, int32_t* err, int shared_chunks,
                              int32_t* offsets, int32_t* active, int32_t* n_active, int32_t* perm, int32_t* inv,
                              Chunk* chunks, int32_t* n_chunks, const int32_t* slot_table, hipStream_t st,
                              const SharedRows* sr = nullptr);
// (xs16b: the per-16 sums times d as three bf16 planes per superblock, for the MMQ min term; may be NULL)
hipError_t launch_quantize_rows(const uint16_t* x, int m, int D, int8_t* xq, float* xd, int32_t* xs16,
                                float* xs16f, uint16_t* xs16b, hipStream_t st);
// logits: `splits` partial arrays [m, E] (from launch_router_gemm), summed in order
hipError_t launch_topk(const float* logits, int splits, const float* bias, int m, int E, int k, float gate_temp,
                       int norm, float route_scale, int32_t* idx, float* gw, int32_t* err, hipStream_t st);
// plan == nullptr: one chunk list of at most GEMV_ROWS rows per chunk (n_chunks[0]);
// otherwise the plan's lists (three MMQ classes, and the GEMV list of a mixed plan)
// at plan->base[c], counts in n_chunks[c]
hipError_t launch_bucket(const int32_t* idx, int m, int k, int E, int shared_chunks, const ChunkPlan* plan,
                         int32_t* offsets, int32_t* active, int32_t* n_active, int32_t* perm, int32_t* inv,
                         Chunk* chunks, int32_t* n_chunks, hipStream_t st);
// the chunks of the plan's lists that one slot wave computes (the others' experts read
// SLOT_SKIP in its table), compacted list by list at the same bases, with their counts
hipError_t launch_compact_wave(const Chunk* chunks, const int32_t* n_chunks, const int32_t* slot_table, bool first_wave,
                               const ChunkPlan& plan, Chunk* out, int32_t* n_out, hipStream_t st);
// the small-batch chunks re-read their experts' slots (after miss streaming)
hipError_t launch_refresh_slots(Chunk* chunks, const int32_t* n_chunks, const int32_t* slot_table, hipStream_t st);
bool mmq_supported(int D, int I);
// one launch per class with reserved slots; a.chunks / a.n_chunks point at class 0
hipError_t launch_fp4_mmq(const ExpertArgs& a, const ChunkPlan& plan, bool gateup, hipStream_t st);
hipError_t launch_mmq(const ExpertArgs& a, const ChunkPlan& plan, bool gateup, hipStream_t st);
// logits [m, E] as `*splits` partial arrays one after another (split K, so that a
// small m still fills the chip); logits must hold max_rows x E floats
hipError_t launch_router_gemm(const uint16_t* x, int m, const uint16_t* wr, int D, int E, float* logits,
                              int max_rows, int* splits, hipStream_t st);
hipError_t launch_shared_bf16_gemm(const uint16_t* x, int m, int D, int I, const uint16_t* w1, const uint16_t* w3,
                                   const uint16_t* w2, uint16_t* h, float* ys, float limit, hipStream_t st);
hipError_t launch_gateup_q2k(const ExpertArgs& a, int rows_max, int max_chunks, hipStream_t st);
// MXFP4 experts: gate/up (h bf16 into h_routed) or down (E rows), chunks of <= rows_max rows
bool fp4_supported(int D, int I);
hipError_t launch_fp4(const ExpertArgs& a, int rows_max, int max_chunks, bool gateup, hipStream_t st);
// MXFP4 experts above 8 tokens: the MMQ chunk classes on bf16 matrix-core tiles
bool fp4_mmq_supported(int D, int I);
hipError_t launch_quantize_h(const ExpertArgs& a, int routed_rows, int shared_rows, hipStream_t st);
hipError_t launch_down_q3k(const ExpertArgs& a, int rows_max, int max_chunks, hipStream_t st);
// decode path (single-row chunks from the small-batch routing)
bool decode_supported(int D, int I);
size_t decode_rec_bytes(int I);
// gate/up writing the q8_1 records of h
hipError_t launch_gateup_q8(const ExpertArgs& a, int routed_rows, int max_chunks, hipStream_t st,
                            const SharedRows* sr = nullptr);
// down + weighted combine (+ the shared expert's f32 output ys when given), bf16 store
hipError_t launch_down_combine(const ExpertArgs& a, int routed_rows, int m, int max_chunks, const float* ys,
                               uint16_t* out, hipStream_t st);
hipError_t launch_shared_bf16_gateup(const uint16_t* x, int m, int D, int I, const uint16_t* w1,
                                     const uint16_t* w3, uint16_t* h_bf16, float limit, hipStream_t st);
hipError_t launch_shared_bf16_down(const uint16_t* h_bf16, int m, int D, int I, const uint16_t* w2, float* ys,
                                   hipStream_t st);
hipError_t launch_combine(const float* e_rows, const float* ys, const float* gw, const int32_t* inv, int m,
                          int k, int D, uint16_t* out, hipStream_t st);

}  // namespace moe
