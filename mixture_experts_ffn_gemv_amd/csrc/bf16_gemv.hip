// bf16 shared-expert GEMVs for chunks of at most 8 tokens (metrale's `gemv`
// kernel: "the bf16 shared expert at one token"; the pages keep the shared
// expert resident in bf16 or K-quant).
//   gate/up (NM = 2): h = bf16(SwiGLU_clamped(W1s x, W3s x))   [m, I] bf16
//   down    (NM = 1): ys = W2s h                                 [m, D] f32
// Every lane owns 16 consecutive K elements (one 32-byte slice), so the rows
// stream with fully coalesced loads and the activations sit in registers; the
// products use v_dot2_f32_bf16 (f32 accumulation).
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

MOE_DEV float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                           false);
}

// Lanes: tid = pr * NM*L + mtx * L + kl, L = K/16.
template <int NM, int T>
__global__ __launch_bounds__(1024) void bf16_rows_kernel(const uint16_t* __restrict__ act, int m, int K,
                                                         const uint16_t* __restrict__ wa,
                                                         const uint16_t* __restrict__ wb, int N, int R, int P,
                                                         int RG, void* __restrict__ out, float limit) {
    extern __shared__ __align__(16) uint8_t smem[];
    float* red = reinterpret_cast<float*>(smem);   // [R][NM][L/RG][T]
    const int L = K / 16;
    const int tiles = N / R;
    const int tc = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int t0 = tc * GEMV_ROWS;
    const int nrows = min(GEMV_ROWS, m - t0);
    const int r0 = tile * R;
    const int tid = threadIdx.x;
    const int pr = tid / (NM * L), rem = tid % (NM * L);
    const int mtx = rem / L, kl = rem % L;
    const uint16_t* W = mtx == 0 ? wa : wb;

    uint32_t xv[T][8];
#pragma unroll
    for (int i = 0; i < T; ++i) {
        if (i < nrows) {
            const uint4* src = reinterpret_cast<const uint4*>(act + (size_t)(t0 + i) * K + 16 * kl);
            const uint4 u0 = src[0], u1 = src[1];
            xv[i][0] = u0.x; xv[i][1] = u0.y; xv[i][2] = u0.z; xv[i][3] = u0.w;
            xv[i][4] = u1.x; xv[i][5] = u1.y; xv[i][6] = u1.z; xv[i][7] = u1.w;
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) xv[i][q] = 0;
        }
    }
    const int ng = L / RG;
    constexpr int UNR = 4;
    for (int rb = pr; rb < R; rb += UNR * P) {
        uint4 wv[UNR][2];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int r = rb + u * P;
            if (r < R) {
                const uint4* src = reinterpret_cast<const uint4*>(W + (size_t)(r0 + r) * K + 16 * kl);
                wv[u][0] = src[0];
                wv[u][1] = src[1];
            }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int r = rb + u * P;
            if (r >= R) break;
            const uint32_t w[8] = {wv[u][0].x, wv[u][0].y, wv[u][0].z, wv[u][0].w,
                                   wv[u][1].x, wv[u][1].y, wv[u][1].z, wv[u][1].w};
            float part[T];
#pragma unroll
            for (int i = 0; i < T; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int q = 0; q < 8; ++q) acc = dot2_bf16(w[q], xv[i][q], acc);
                part[i] = acc;
            }
#pragma unroll
            for (int i = 0; i < T; ++i) {
                float v = part[i];
                for (int off = 1; off < RG; off <<= 1) v += __shfl_xor(v, off);
                part[i] = v;
            }
            if ((kl & (RG - 1)) == 0) {
#pragma unroll
                for (int i = 0; i < T; ++i) red[((r * NM + mtx) * ng + kl / RG) * T + i] = part[i];
            }
        }
    }
    __syncthreads();
    for (int q = tid; q < R * T; q += blockDim.x) {
        const int r = q / T, i = q % T;
        if (i >= nrows) continue;
        float y0 = 0.f, y1 = 0.f;
        for (int g = 0; g < ng; ++g) {
            y0 += red[((r * NM + 0) * ng + g) * T + i];
            if (NM == 2) y1 += red[((r * NM + 1) * ng + g) * T + i];
        }
        if (NM == 2) {
            uint16_t* h = reinterpret_cast<uint16_t*>(out);
            h[(size_t)(t0 + i) * N + r0 + r] = (uint16_t)f32_to_bf16(swiglu(y0, y1, limit));
        } else {
            float* ys = reinterpret_cast<float*>(out);
            ys[(size_t)(t0 + i) * N + r0 + r] = y0;
        }
    }
}

static int gcd_int(int a, int b) {
    while (b) {
        const int t = a % b;
        a = b;
        b = t;
    }
    return a;
}

template <int NM, int T>
static hipError_t launch_rows(const uint16_t* act, int m, int K, const uint16_t* wa, const uint16_t* wb, int N,
                              void* out, float limit, hipStream_t st) {
    const int L = K / 16;
    const int lanes = NM * L;
    int P = 1;
    while (lanes * P < 256 && lanes * (P + 1) <= 1024) ++P;
    while ((lanes * P) % 64 != 0 && lanes * (P + 1) <= 1024) ++P;
    int R = 8;
    while (R < P) R += 8;
    while (N % R) R += 8;
    const int RG = gcd_int(L, 64);
    const size_t lds = (size_t)R * NM * (L / RG) * T * sizeof(float);
    const int tiles = N / R;
    const int tchunks = (m + GEMV_ROWS - 1) / GEMV_ROWS;
    return launch_kernel(bf16_rows_kernel<NM, T>, tiles * tchunks, lanes * P, lds, st, act, m, K, wa, wb, N, R, P, RG, out, limit);
}

hipError_t launch_shared_bf16_gateup(const uint16_t* x, int m, int D, int I, const uint16_t* w1,
                                     const uint16_t* w3, uint16_t* h_bf16, float limit, hipStream_t st) {
    if (m <= 1) return launch_rows<2, 1>(x, m, D, w1, w3, I, h_bf16, limit, st);
    if (m <= 2) return launch_rows<2, 2>(x, m, D, w1, w3, I, h_bf16, limit, st);
    if (m <= 4) return launch_rows<2, 4>(x, m, D, w1, w3, I, h_bf16, limit, st);
    return launch_rows<2, 8>(x, m, D, w1, w3, I, h_bf16, limit, st);
}

hipError_t launch_shared_bf16_down(const uint16_t* h_bf16, int m, int D, int I, const uint16_t* w2, float* ys,
                                   hipStream_t st) {
    if (m <= 1) return launch_rows<1, 1>(h_bf16, m, I, w2, w2, D, ys, 0.f, st);
    if (m <= 2) return launch_rows<1, 2>(h_bf16, m, I, w2, w2, D, ys, 0.f, st);
    if (m <= 4) return launch_rows<1, 4>(h_bf16, m, I, w2, w2, D, ys, 0.f, st);
    return launch_rows<1, 8>(h_bf16, m, I, w2, w2, D, ys, 0.f, st);
}

}  // namespace moe
