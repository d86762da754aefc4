// The bf16 shared expert's rows as extra workgroups of other launches: its
// gate/up rows in the router launch (the routing kernels leave most of the
// chip idle; the shared expert needs only x), its down rows in the top-k launch
// and, with K-quant experts, half of them in the routed gate/up launch. h = bf16(SwiGLU_clamped(W1s x, W3s x)), as in the
// shared-expert GEMV of the pages (metrale `gemv`, the bf16 shared expert at
// one token).
#pragma once

#include "moe_common.h"

namespace moe {

struct SharedRows {
    const uint16_t* w1;   // gate/up rows: bf16 [I, D] row-major (NULL with w2 NULL: no shared rows)
    const uint16_t* w3;   // bf16 [I, D]
    const uint16_t* x;    // bf16 [m, D]
    uint16_t* h;          // bf16 [m, I] (written by gate/up rows, read by down rows)
    const uint16_t* w2;   // down rows instead: bf16 [D, I] row-major, ys = W2 h (f32 [m, D])
    float* ys;
    int32_t row0, rows;   // the rows [row0, row0 + rows) this launch computes (of h, or of ys)
    int32_t D, I, m;      // m <= 8
    float limit;
};

// Workgroups needed for the launch's rows with `threads` threads each: a gate/up
// row per two wavefronts, a down row per wavefront. (threads >= 128; the
// routing launches that carry shared rows use at least that)
inline int shared_rows_blocks(const SharedRows& sr, int threads) {
    const int rpw = sr.w2 != nullptr ? threads / 64 : threads / 128;
    return sr.rows <= 0 || rpw <= 0 ? 0 : (sr.rows + rpw - 1) / rpw;
}

// 16-byte pieces of a row a lane holds in registers at once (rows of up to 6144
// values in one round; longer rows take a second, synchronous round)
constexpr int SR_PIECES = 12;

MOE_DEV float dot2_bf16x(uint32_t a, uint32_t b, float c) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
}

// Workgroup `blk` of the shared rows: wavefront 2i takes row (row0 + blk * rpw + i)
// of W1, wavefront 2i + 1 the same row of W3 (rpw = wavefronts / 2). A lane
// holds 16-byte pieces lane, lane + 64, ... of its row (every load of the
// wavefront 1 KB contiguous; up to SR_PIECES per round), dots them with the
// same pieces of each token row of x, and the wavefront sums; the gate
// wavefront applies the SwiGLU.
MOE_DEV void shared_gateup_block(const SharedRows& sr, int blk) {
    __shared__ float up[16][8];
    const int nw = blockDim.x >> 6, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rpw = nw >> 1, rl = wv >> 1;
    const int rr = blk * rpw + rl;
    const bool valid = wv < 2 * rpw && rr < sr.rows;
    const int r = sr.row0 + rr;
    const int n16 = sr.D / 8;   // 16-byte pieces per row
    float dots[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) dots[t] = 0.f;
    if (valid) {
        const uint4* W = reinterpret_cast<const uint4*>(((wv & 1) ? sr.w3 : sr.w1) + (size_t)r * sr.D);
        for (int j0 = 0; j0 * 64 < n16; j0 += SR_PIECES) {
            uint4 wq[SR_PIECES];
#pragma unroll
            for (int j = 0; j < SR_PIECES; ++j) {
                const int k = lane + 64 * (j0 + j);
                wq[j] = k < n16 ? W[k] : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (t >= sr.m) break;
                const uint4* X = reinterpret_cast<const uint4*>(sr.x + (size_t)t * sr.D);
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < SR_PIECES; ++j) {
                    const int k = lane + 64 * (j0 + j);
                    if (k < n16) {
                        const uint4 xv = X[k];
                        acc = dot2_bf16x(wq[j].x, xv.x, acc);
                        acc = dot2_bf16x(wq[j].y, xv.y, acc);
                        acc = dot2_bf16x(wq[j].z, xv.z, acc);
                        acc = dot2_bf16x(wq[j].w, xv.w, acc);
                    }
                }
                dots[t] += acc;
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t >= sr.m) break;
            dots[t] = wave_sum(dots[t]);
        }
        if ((wv & 1) && lane == 0) {
#pragma unroll
            for (int t = 0; t < 8; ++t) up[rl][t] = dots[t];
        }
    }
    __syncthreads();
    if (valid && !(wv & 1) && lane == 0) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t >= sr.m) break;
            sr.h[(size_t)t * sr.I + r] = (uint16_t)f32_to_bf16(swiglu(dots[t], up[rl][t], sr.limit));
        }
    }
}

// Workgroup `blk` of the shared down rows: wavefront i takes output row
// row0 + blk * (wavefronts) + i of W2, 16-byte pieces lane, lane + 64, ... (every
// load of the wavefront 1 KB contiguous), dotted with the same pieces of each
// token's h; the wavefront sums and lane 0 writes ys. NP pieces per lane and
// round (fewer registers for launches that must stay lean).
template <int NP = SR_PIECES>
MOE_DEV void shared_down_block(const SharedRows& sr, int blk) {
    const int nw = blockDim.x >> 6, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rr = blk * nw + wv;
    if (rr >= sr.rows) return;
    const int r = sr.row0 + rr;
    const int n16 = sr.I / 8;   // 16-byte pieces per row
    const uint4* W = reinterpret_cast<const uint4*>(sr.w2 + (size_t)r * sr.I);
    float dots[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) dots[t] = 0.f;
    for (int j0 = 0; j0 * 64 < n16; j0 += NP) {
        uint4 wq[NP];
#pragma unroll
        for (int j = 0; j < NP; ++j) {
            const int k = lane + 64 * (j0 + j);
            wq[j] = k < n16 ? W[k] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t >= sr.m) break;
            const uint4* H = reinterpret_cast<const uint4*>(sr.h + (size_t)t * sr.I);
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const int k = lane + 64 * (j0 + j);
                if (k < n16) {
                    const uint4 hv = H[k];
                    acc = dot2_bf16x(wq[j].x, hv.x, acc);
                    acc = dot2_bf16x(wq[j].y, hv.y, acc);
                    acc = dot2_bf16x(wq[j].z, hv.z, acc);
                    acc = dot2_bf16x(wq[j].w, hv.w, acc);
                }
            }
            dots[t] += acc;
        }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        if (t >= sr.m) break;
        const float v = wave_sum(dots[t]);
        if (lane == 0) sr.ys[(size_t)t * sr.D + r] = v;
    }
}

// the launch's shared rows, gate/up or down
MOE_DEV void shared_rows_block(const SharedRows& sr, int blk) {
    if (sr.w2 != nullptr) shared_down_block(sr, blk);
    else shared_gateup_block(sr, blk);
}

}  // namespace moe
