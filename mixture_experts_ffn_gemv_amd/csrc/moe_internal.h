// Launchers shared between the kernel translation units and the host library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_common.h"

namespace moe {

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

// router logits for m tokens, plus q8_1 of x in the same launch when xq != NULL
hipError_t launch_router_quant(const uint16_t* x, int m, const uint16_t* wr, int D, int E, float* logits,
                               int8_t* xq, float* xd, int32_t* xs16, hipStream_t st);
// top-k and bucketing in one workgroup, for m * topk <= 512 and m <= 8
constexpr int ROUTE_SMALL_MAX_M = 8;
constexpr int ROUTE_SMALL_MAX_PAIRS = 512;
hipError_t launch_route_small(const float* logits, const float* bias, int m, int E, int k, float gate_temp,
                              int norm, float route_scale, int32_t* idx, float* gw, int32_t* err, int shared_chunks,
                              int32_t* offsets, int32_t* active, int32_t* n_active, int32_t* perm, int32_t* inv,
                              Chunk* chunks, int32_t* n_chunks, hipStream_t st);
hipError_t launch_quantize_rows(const uint16_t* x, int m, int D, int8_t* xq, float* xd, int32_t* xs16,
                                float* xs16f, hipStream_t st);
hipError_t launch_topk(const float* logits, const float* bias, int m, int E, int k, float gate_temp, int norm,
                       float route_scale, int32_t* idx, float* gw, int32_t* err, hipStream_t st);
// chunks of at most rows_per_chunk token rows (GEMV_ROWS for the GEMVs, MMQ_ROWS for the MMQ)
hipError_t launch_bucket(const int32_t* idx, int m, int k, int E, int shared_chunks, int rows_per_chunk,
                         int32_t* offsets, int32_t* active, int32_t* n_active, int32_t* perm, int32_t* inv,
                         Chunk* chunks, int32_t* n_chunks, hipStream_t st);
constexpr int MMQ_ROWS = 64;   // the most token rows one MMQ chunk holds (four 16-row sub-tiles)
// MMQ chunk height for a batch: the 16-row sub-tile count per chunk follows the
// mean rows per expert, so that chunks of lightly used experts do not carry the
// registers of four sub-tiles (a heavy expert is split into several chunks)
inline int mmq_chunk_rows(int m, int k, int E) {
    const long mean = ((long)m * k + E - 1) / E;
    return mean <= 16 ? 16 : mean <= 40 ? 32 : MMQ_ROWS;
}
bool mmq_supported(int D, int I);
hipError_t launch_mmq(const ExpertArgs& a, int rows_max, int max_chunks, bool gateup, hipStream_t st);
hipError_t launch_router_gemm(const uint16_t* x, int m, const uint16_t* wr, int D, int E, float* logits,
                              hipStream_t st);
hipError_t launch_shared_bf16_gemm(const uint16_t* x, int m, int D, int I, const uint16_t* w1, const uint16_t* w3,
                                   const uint16_t* w2, uint16_t* h, float* ys, float limit, hipStream_t st);
hipError_t launch_gateup_q2k(const ExpertArgs& a, int rows_max, int max_chunks, hipStream_t st);
hipError_t launch_quantize_h(const ExpertArgs& a, int routed_rows, int shared_rows, hipStream_t st);
hipError_t launch_down_q3k(const ExpertArgs& a, int rows_max, int max_chunks, hipStream_t st);
// streaming (persistent, software-pipelined) GEMVs for chunks of one row
bool stream_gemv_supported(int D, int I);
hipError_t launch_gateup_q2k_stream(const ExpertArgs& a, int n_wg, hipStream_t st);
hipError_t launch_down_q3k_stream(const ExpertArgs& a, int n_wg, hipStream_t st);
hipError_t launch_shared_bf16_gateup(const uint16_t* x, int m, int D, int I, const uint16_t* w1,
                                     const uint16_t* w3, uint16_t* h_bf16, float limit, hipStream_t st);
hipError_t launch_shared_bf16_down(const uint16_t* h_bf16, int m, int D, int I, const uint16_t* w2, float* ys,
                                   hipStream_t st);
hipError_t launch_combine(const float* e_rows, const float* ys, const float* gw, const int32_t* inv, int m,
                          int k, int D, uint16_t* out, hipStream_t st);

}  // namespace moe
