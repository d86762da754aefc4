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
// the same for the down rows of the routing launches (rows of up to 3072 values in one round)
constexpr int SR_DOWN_PIECES = 6;

MOE_DEV float dot2_bf16x(uint32_t a, uint32_t b, float c) {
    typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), c, false);
}

// Workgroup `blk` of the shared rows: wavefront 2i takes row (row0 + blk * rpw + i)
// of W1, wavefront 2i + 1 the same row of W3 (rpw = wavefronts / 2). A lane
// holds 16-byte pieces lane, lane + 64, ... of its row (every load of the
// wavefront 1 KB contiguous; up to SR_PIECES per round) and dots them with the
// same pieces of each token row of x; the wavefront sums (lane t keeps token
// t's sum) and the gate wavefront applies the SwiGLU. The weights go straight
// into registers through a buffer resource over the row (pieces past its end
// read as zeros); each token's pieces of x come once per workgroup into LDS
// (buffer loads into LDS, requested before the weights for the first token;
// pieces past the row land as zeros), where the wavefronts read them.
MOE_DEV void shared_gateup_block(const SharedRows& sr, int blk) {
    __shared__ float up[16][8];
    __shared__ __align__(16) uint4 xs[SR_PIECES * 64];
    const int nw = blockDim.x >> 6, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rpw = nw >> 1, rl = wv >> 1;
    const int rr = blk * rpw + rl;
    const bool valid = wv < 2 * rpw && rr < sr.rows;
    const int r = sr.row0 + rr;
    const int n16 = sr.D / 8;   // 16-byte pieces per row
    const uint32_t row_bytes = (uint32_t)sr.D * 2;
    float mine = 0.f;   // lane t < m: token t's dot
    const auto W = buffer_rsrc(((wv & 1) ? sr.w3 : sr.w1) + (size_t)(valid ? r : sr.row0) * sr.D, row_bytes);
    // token t's pieces [p0, p0 + SR_PIECES * 64) of x into xs: 16 bytes per thread and
    // load (pieces past the row land as zeros)
    auto stage_x = [&](int t, int p0) {
        const auto X = buffer_rsrc(sr.x + (size_t)t * sr.D, row_bytes);
        for (int i = threadIdx.x; i < SR_PIECES * 64; i += blockDim.x) buffer_load_lds16(X, xs + (i - lane), 16 * (p0 + i));
    };
    for (int p0 = 0; p0 < n16; p0 += SR_PIECES * 64) {
        const uint32_t off = 16 * (p0 + lane);
        stage_x(0, p0);
        uint4 wq[SR_PIECES];
#pragma unroll
        for (int j = 0; j < SR_PIECES; ++j) wq[j] = buffer_load16(W, off + 1024 * j);
        for (int t = 0; t < sr.m; ++t) {
            if (t > 0) {
                __syncthreads();   // every wavefront is done with token t - 1's pieces
                stage_x(t, p0);
            }
            // this wavefront's DMA has landed (for the first token it was issued before
            // the weights, which may stay in flight)
            if (t == 0) wait_vm_loads<SR_PIECES>();
            else wait_vm_loads<0>();
            __syncthreads();
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < SR_PIECES; ++j) {
                const uint4 xv = xs[lane + 64 * j];
                acc = dot2_bf16x(wq[j].x, xv.x, acc);
                acc = dot2_bf16x(wq[j].y, xv.y, acc);
                acc = dot2_bf16x(wq[j].z, xv.z, acc);
                acc = dot2_bf16x(wq[j].w, xv.w, acc);
            }
            const float sum = wave_sum(acc);
            if (lane == t) mine += sum;
        }
        __syncthreads();   // xs is restaged by the next round
    }
    if (valid && (wv & 1) && lane < sr.m) up[rl][lane] = mine;
    __syncthreads();
    if (valid && !(wv & 1) && lane < sr.m)
        sr.h[(size_t)lane * sr.I + r] = (uint16_t)f32_to_bf16(swiglu(mine, up[rl][lane], sr.limit));
}

// Workgroup `blk` of the shared down rows: wavefront i takes output row
// row0 + blk * (wavefronts) + i of W2, 16-byte pieces lane, lane + 64, ... (every
// load of the wavefront 1 KB contiguous), dotted with the same pieces of each
// token's h; the wavefront sums and lane t writes token t's ys. NP pieces per
// lane and round (fewer registers for launches that must stay lean); loads are
// requested as in the gate/up rows.
template <int NP = SR_PIECES>
MOE_DEV void shared_down_block(const SharedRows& sr, int blk) {
    const int nw = blockDim.x >> 6, wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rr = blk * nw + wv;
    if (rr >= sr.rows) return;
    const int r = sr.row0 + rr;
    const uint32_t row_bytes = (uint32_t)sr.I * 2;
    const auto W = buffer_rsrc(sr.w2 + (size_t)r * sr.I, row_bytes);
    float mine = 0.f;   // lane t < m: token t's dot
    for (uint32_t o0 = 0; o0 < row_bytes; o0 += NP * 1024) {
        const uint32_t off = o0 + 16 * lane;
        uint4 hq[NP], wq[NP];
        const auto H0 = buffer_rsrc(sr.h, row_bytes);
#pragma unroll
        for (int j = 0; j < NP; ++j) hq[j] = buffer_load16(H0, off + 1024 * j);
#pragma unroll
        for (int j = 0; j < NP; ++j) wq[j] = buffer_load16(W, off + 1024 * j);
#pragma unroll 1
        for (int t = 0; t < sr.m; ++t) {
            if (t > 0) {
                const auto H = buffer_rsrc(sr.h + (size_t)t * sr.I, row_bytes);
#pragma unroll
                for (int j = 0; j < NP; ++j) hq[j] = buffer_load16(H, off + 1024 * j);
            }
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                acc = dot2_bf16x(wq[j].x, hq[j].x, acc);
                acc = dot2_bf16x(wq[j].y, hq[j].y, acc);
                acc = dot2_bf16x(wq[j].z, hq[j].z, acc);
                acc = dot2_bf16x(wq[j].w, hq[j].w, acc);
            }
            const float sum = wave_sum(acc);
            if (lane == t) mine += sum;
        }
    }
    if (lane < sr.m) sr.ys[(size_t)lane * sr.D + r] = mine;
}

}  // namespace moe
