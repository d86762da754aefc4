// The bf16 shared expert's gate/up, as extra workgroups of the routing
// launches (the routing kernels leave most of the chip idle; the shared
// expert needs only x). h = bf16(SwiGLU_clamped(W1s x, W3s x)), as in the
// shared-expert GEMV of the pages (metrale `gemv`, the bf16 shared expert at
// one token).
#pragma once

#include "moe_common.h"

namespace moe {

struct SharedRows {
    const uint16_t* w1;   // bf16 [I, D] row-major; NULL: no shared-expert rows in this launch
    const uint16_t* w3;   // bf16 [I, D]
    const uint16_t* x;    // bf16 [m, D]
    uint16_t* h;          // bf16 [m, I]
    int32_t row0, rows;   // the rows [row0, row0 + rows) this launch computes
    int32_t D, I, m;      // m <= 8
    float limit;
};

// Workgroups needed for `rows` rows with `threads` threads each (a row per two wavefronts).
// (threads >= 128; the routing launches that carry shared rows use at least that)
inline int shared_rows_blocks(int rows, int threads) {
    const int rpw = threads / 128;
    return rows <= 0 || rpw <= 0 ? 0 : (rows + rpw - 1) / rpw;
}

MOE_DEV float dot2_bf16x(uint32_t a, uint32_t b, float c) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
}

// Workgroup `blk` of the shared rows: wavefront 2i takes row (row0 + blk * rpw + i)
// of W1, wavefront 2i + 1 the same row of W3 (rpw = wavefronts / 2). A lane
// holds 16-byte pieces lane, lane + 64, ... of its row (every load of the
// wavefront is 1 KB contiguous), dots them with the same pieces of each token
// row of x, and the wavefront sums; the gate wavefront applies the SwiGLU.
MOE_DEV void shared_gateup_block(const SharedRows& sr, int blk) {
    __shared__ float up[16][8];
    const int nw = blockDim.x >> 6, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rpw = nw >> 1, rl = wv >> 1;
    const int rr = blk * rpw + rl;
    const bool valid = wv < 2 * rpw && rr < sr.rows;
    const int r = sr.row0 + rr;
    const int n16 = sr.D / 8;   // 16-byte pieces per row (D <= 8192: at most 16 per lane)
    float dots[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) dots[t] = 0.f;
    if (valid) {
        const uint4* W = reinterpret_cast<const uint4*>(((wv & 1) ? sr.w3 : sr.w1) + (size_t)r * sr.D);
        uint4 wq[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int k = lane + 64 * j;
            wq[j] = k < n16 ? W[k] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t >= sr.m) break;
            const uint4* X = reinterpret_cast<const uint4*>(sr.x + (size_t)t * sr.D);
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int k = lane + 64 * j;
                if (k < n16) {
                    const uint4 xv = X[k];
                    acc = dot2_bf16x(wq[j].x, xv.x, acc);
                    acc = dot2_bf16x(wq[j].y, xv.y, acc);
                    acc = dot2_bf16x(wq[j].z, xv.z, acc);
                    acc = dot2_bf16x(wq[j].w, xv.w, acc);
                }
            }
            dots[t] = wave_sum(acc);
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

}  // namespace moe
