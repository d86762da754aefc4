// bf16 MFMA GEMM with f32 accumulation for the batched (m > 8) steps that are
// plain dense products: the router logits z = x W_R^T, and the bf16 shared
// expert (gate/up with the clamped-SwiGLU epilogue, then down). The pages use
// metrale's `gemm` / `gemm_f32out` kernels for these (kernel table of
// moe_v41.rs); the shared expert's math is the Open Model Atlas
// "Shared expert" equations with the Expert excerpt's clamps.
//
// C[M, N] = A[M, K] B[N, K]^T, both operands K-contiguous bf16. Workgroup tile
// 64 (A rows) x 128 (B rows) x 64 (K), four wavefronts, each owning 32 B rows;
// v_mfma_f32_16x16x32_bf16 tiles. Each K step's tiles go from global memory
// straight into LDS (global-to-LDS loads, 16 bytes per lane) in a ring of four
// buffers: steps k + 1 .. k + 3 are in flight while step k is multiplied (with
// one step in flight each workgroup waited out most of a load's latency per
// step). A tile row is 128 bytes
// (8 chunks of 16); chunk c of row r is stored at slot c ^ ((r >> 1) & 7), so
// the 16 rows one operand read touches fall on distinct banks. The f32 output
// may be split over K (grid z): split s sums K steps [s nk / S, (s + 1) nk / S)
// into its own partial array; the router's top-k adds them.
#include <algorithm>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int BM = 64, BN = 128, BK = 64;
constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
constexpr int NSTAGE = 4;   // K steps in LDS: one computed, three in flight

enum Epilogue { EPI_F32 = 0, EPI_SWIGLU = 1 };

MOE_DEV int swz(int row, int c) { return row * (BK * 2) + ((c ^ ((row >> 1) & 7)) << 4); }

}  // namespace

// EPI_F32:    out f32 [M, N] = A B^T           (B = wa, N rows)
// EPI_SWIGLU: out bf16 [M, N] = bf16(SwiGLU(A wa^T, A wb^T)); each workgroup takes
//             64 rows of wa and the same 64 rows of wb as its 128 B rows
template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const uint16_t* __restrict__ A, int M,
                                                        const uint16_t* __restrict__ wa,
                                                        const uint16_t* __restrict__ wb, int N, int K,
                                                        void* __restrict__ out, float limit) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int nk_all = K / BK, splits = gridDim.z, sidx = blockIdx.z;
    const int kt0 = sidx * nk_all / splits, nk = (sidx + 1) * nk_all / splits - kt0;
    if (EPI == EPI_F32) out = reinterpret_cast<float*>(out) + (size_t)sidx * M * N;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int m0 = blockIdx.y * BM;
    const int rows_per_b = EPI == EPI_SWIGLU ? BN / 2 : BN;
    const int n0 = blockIdx.x * rows_per_b;

    // this thread's 16-byte units: LDS slot p = 256 u + tid holds row p / 8, chunk
    // (p % 8) ^ ((row >> 1) & 7) of its tile (rows past the matrix repeat its last row;
    // their products are never stored)
    const uint16_t* srcA[2];
    const uint16_t* srcB[4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int p = u * 256 + tid, row = p >> 3, c = (p & 7) ^ ((row >> 1) & 7);
        srcA[u] = A + (size_t)(m0 + min(row, M - m0 - 1)) * K + kt0 * BK + c * 8;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int p = u * 256 + tid, row = p >> 3, c = (p & 7) ^ ((row >> 1) & 7);
        const uint16_t* base;
        if (EPI == EPI_SWIGLU) base = row < 64 ? wa + (size_t)(n0 + row) * K : wb + (size_t)(n0 + row - 64) * K;
        else base = wa + (size_t)(n0 + min(row, N - n0 - 1)) * K;
        srcB[u] = base + kt0 * BK + c * 8;
    }
    auto stage = [&](int kt, uint8_t* buf) {
#pragma unroll
        for (int u = 0; u < 2; ++u) load_lds16(srcA[u] + kt * BK, buf + (u * 256 + wv * 64) * 16);
#pragma unroll
        for (int u = 0; u < 4; ++u) load_lds16(srcB[u] + kt * BK, buf + A_BYTES + (u * 256 + wv * 64) * 16);
    };

    f32x4_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = (f32x4_t){0.f, 0.f, 0.f, 0.f};

    const int l16 = lane & 15, g = lane >> 4;
    stage(0, smem);
    if (nk > 1) stage(1, smem + STAGE);
    if (nk > 2) stage(2, smem + 2 * STAGE);
    for (int kt = 0; kt < nk; ++kt) {
        // step kt is in LDS (each later step in flight holds six loads per thread) ...
        if (kt + 2 < nk) wait_vm_loads<12>();
        else if (kt + 1 < nk) wait_vm_loads<6>();
        else wait_vm_loads<0>();
        barrier_lds();        // ... for every wave; the buffer of step kt - 1 is free
        const uint8_t* buf = smem + (kt % NSTAGE) * STAGE;
        if (kt + 3 < nk) stage(kt + 3, smem + ((kt + 3) % NSTAGE) * STAGE);
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {
            const int c = 4 * kk + g;   // this lane's K values 32 kk + 8 g .. + 7
            bf16x8_t af[4], bfr[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(buf + swz(16 * i + l16, c));
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // wave wv owns B rows {16 j' + ...}: for SwiGLU, rows 16 wv.. of wa and the same of wb
                const int brow = EPI == EPI_SWIGLU ? (j == 0 ? 16 * wv : 64 + 16 * wv) : 32 * wv + 16 * j;
                bfr[j] = *reinterpret_cast<const bf16x8_t*>(buf + A_BYTES + swz(brow + l16, c));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }
    wait_vm_loads<0>();   // no load into LDS outlives the workgroup

    // C layout: lane holds column (B row) lane % 16 of the 16x16 tile, rows 4 (lane / 16) + r
    const int col = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + 16 * i + 4 * (lane >> 4) + r;
            if (row >= M) continue;
            if (EPI == EPI_SWIGLU) {
                const int n = n0 + 16 * wv + col;
                const float h = swiglu(acc[i][0][r], acc[i][1][r], limit);
                reinterpret_cast<uint16_t*>(out)[(size_t)row * N + n] = (uint16_t)f32_to_bf16(h);
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int n = n0 + 32 * wv + 16 * j + col;
                    if (n < N) reinterpret_cast<float*>(out)[(size_t)row * N + n] = acc[i][j][r];
                }
            }
        }
    }
}

// logits f32 [m, E] = x W_R^T, split over K into up to 8 partial arrays while the
// tiles alone would not give every CU a workgroup and the scratch has room
hipError_t launch_router_gemm(const uint16_t* x, int m, const uint16_t* wr, int D, int E, float* logits,
                              int max_rows, int* splits, hipStream_t st) {
    const int tiles = ((E + BN - 1) / BN) * ((m + BM - 1) / BM);
    int s = (256 + tiles - 1) / tiles;
    s = std::max(1, std::min({s, 8, D / BK, max_rows / m}));
    *splits = s;
    dim3 grid((E + BN - 1) / BN, (m + BM - 1) / BM, s);
    return launch_kernel(gemm_bf16_kernel<EPI_F32>, grid, 256, NSTAGE * STAGE, st, x, m, wr, wr, E, D, logits, 0.f);
}

// h bf16 [m, I] = SwiGLU(x W1^T, x W3^T);  ys f32 [m, D] = h W2^T
hipError_t launch_shared_bf16_gemm(const uint16_t* x, int m, int D, int I, const uint16_t* w1, const uint16_t* w3,
                                   const uint16_t* w2, uint16_t* h, float* ys, float limit, hipStream_t st) {
    dim3 g1(I / (BN / 2), (m + BM - 1) / BM);
    hipError_t e = launch_kernel(gemm_bf16_kernel<EPI_SWIGLU>, g1, 256, NSTAGE * STAGE, st, x, m, w1, w3, I, D, h, limit);
    if (e != hipSuccess) return e;
    dim3 g2(D / BN, (m + BM - 1) / BM);
    return launch_kernel(gemm_bf16_kernel<EPI_F32>, g2, 256, NSTAGE * STAGE, st, h, m, w2, w2, D, I, ys, 0.f);
}

}  // namespace moe
