// Expert-grouped MMQ for batched calls: the routed experts' products as
// int8 matrix-core tiles over the still-quantised blocks (metrale moe_v41
// module documentation: "by default MMQ above" eight rows; kernel table of
// moe_v41.rs: mmq_q2k_* / mmq_q3k_*).
//
// A chunk is one expert with up to MMQ_ROWS token rows (in three size classes,
// each launched with the sub-tile count it needs). One workgroup computes
// 64 output rows of one chunk: gate/up for 64 rows of W1 and the same rows of
// W3 (then the clamped SwiGLU), or down for 64 rows of W2. Tokens form the A
// operand (16-row sub-tiles of q8_1 quants), weights the B operand
// (v_mfma_i32_16x16x32_i8: K = 32 is exactly one q8_1 block, so each product is
// rescaled by that block's activation scale).
//  * Q2_K: the B bytes are sc_n * q (<= 45), so d * (B . A) covers the scale
//    part of the weight; the min part -dmin * m_n * sum(A) is added per
//    superblock from the per-16 sums of the activation quants.
//  * Q3_K: the B bytes are (32 - sc6_n) * q3 = -(sc6_n - 32) q3, which lies in
//    [-128, 124] (the unnegated product would reach +128), built with a
//    v_perm_b32 byte lookup from q3 + 4; the sign goes into d.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

namespace {

constexpr int TILE_ROWS = 64;   // weight rows per workgroup (16 per wavefront)

MOE_DEV i32x4_t mfma_i8(int64_t a, int64_t b) {
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, (i32x4_t){0, 0, 0, 0}, 0, 0, 0);
}

MOE_DEV int chunk_token_mmq(const ExpertArgs& a, const Chunk& ch, int i) {
    return ch.expert < 0 ? ch.row0 + i : a.perm[ch.row0 + i] / a.topk;
}

}  // namespace

// ------------------------------------------------------------------ Q2_K gate/up
// LDS: raw blocks of 64 W1 rows then 64 W3 rows, KS superblocks at a time.
template <int NS>
__global__ __launch_bounds__(256) void mmq_gateup_q2k_kernel(ExpertArgs a, int KS) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int nsb = D / QK;
    const int tiles = I / TILE_ROWS;
    const int c = blockIdx.x / tiles, rt = blockIdx.x % tiles;
    if (c >= *a.n_chunks) return;
    const Chunk ch = a.chunks[c];
    const bool shared = ch.expert < 0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r0 = rt * TILE_ROWS;
    float* hout = (shared ? a.h_shared : a.h_routed) + (size_t)ch.row0 * I;
    const uint8_t *w1, *w3;
    if (shared) {
        w1 = a.sh_w1;
        w3 = a.sh_w3;
    } else {
        const int slot = a.slot_table[ch.expert];
        if (slot == SLOT_SKIP) return;   // computed in another slot wave
        if (slot < 0) {
            if (tid == 0 && rt == 0) atomicOr(a.err, ERR_NOTRESIDENT);
            for (int q = tid; q < TILE_ROWS * ch.nrows; q += 256)
                hout[(size_t)(q / TILE_ROWS) * I + r0 + q % TILE_ROWS] = 0.f;
            return;
        }
        const uint8_t* base = a.arena + (size_t)slot * a.slot_bytes;
        w1 = base + a.off_w1;
        w3 = base + a.off_w3;
    }
    const size_t rowbytes = (size_t)nsb * Q2K_BYTES;
    const int seg_dw = KS * Q2K_BYTES / 4;              // dwords per row segment
    uint32_t* lds = reinterpret_cast<uint32_t*>(smem);   // [128 rows][seg_dw]

    // A rows: token of sub-tile s, row lane % 16; C rows: tokens 4 (lane / 16) + r
    const int g = lane >> 4, l16 = lane & 15;
    int tokA[NS], tokC[NS][4];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int ia = 16 * s + l16;
        tokA[s] = ia < ch.nrows ? chunk_token_mmq(a, ch, ia) : -1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ic = 16 * s + 4 * g + r;
            tokC[s][r] = ic < ch.nrows ? chunk_token_mmq(a, ch, ic) : -1;
        }
    }
    typedef float f4 __attribute__((ext_vector_type(4)));
    f4 accg[NS], accu[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) accg[s] = accu[s] = (f4){0.f, 0.f, 0.f, 0.f};
    const int ns = min(NS, (ch.nrows + 15) / 16);   // sub-tiles holding tokens

    const int wrow = 16 * wv + l16;   // this lane's weight row (B column) in the tile
    for (int sb0 = 0; sb0 < nsb; sb0 += KS) {
        const int ks = min(KS, nsb - sb0);
        const int sdw = ks * Q2K_BYTES / 4;
        // stage rows [r0, r0+64) of W1 and W3, superblocks [sb0, sb0+ks)
        for (int q = tid; q < 128 * sdw; q += 256) {
            const int row = q / sdw, dw = q % sdw;
            const uint8_t* src = (row < 64 ? w1 + (size_t)(r0 + row) * rowbytes
                                            : w3 + (size_t)(r0 + row - 64) * rowbytes) +
                                 (size_t)sb0 * Q2K_BYTES;
            lds[row * seg_dw + dw] = reinterpret_cast<const uint32_t*>(src)[dw];
        }
        __syncthreads();
        for (int sbi = 0; sbi < ks; ++sbi) {
            const int sb = sb0 + sbi;
            const uint32_t* bg = lds + wrow * seg_dw + sbi * (Q2K_BYTES / 4);
            const uint32_t* bu = lds + (64 + wrow) * seg_dw + sbi * (Q2K_BYTES / 4);
            const uint32_t ddg = bg[20], ddu = bu[20];
            const float dg = half_bits_to_f32(ddg & 0xFFFFu), dming = half_bits_to_f32(ddg >> 16);
            const float du = half_bits_to_f32(ddu & 0xFFFFu), dminu = half_bits_to_f32(ddu >> 16);
            f4 sg[NS], su[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) sg[s] = su[s] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
            for (int kb8 = 0; kb8 < 8; ++kb8) {
                const int hh = kb8 >> 2, j = kb8 & 3;
                // B: 8 weights at positions 8g..8g+7 of plane j, half hh; one sub-block
                const int n = 8 * hh + 2 * j + (g >> 1);
                const int qd = 4 + 8 * hh + 2 * g;   // dword of qs[32 hh + 8 g]
                const uint32_t scg = (bg[n >> 2] >> (8 * (n & 3))) & 15;
                const uint32_t scu = (bu[n >> 2] >> (8 * (n & 3))) & 15;
                const uint32_t bg0 = ((bg[qd] >> (2 * j)) & 0x03030303u) * scg;
                const uint32_t bg1 = ((bg[qd + 1] >> (2 * j)) & 0x03030303u) * scg;
                const uint32_t bu0 = ((bu[qd] >> (2 * j)) & 0x03030303u) * scu;
                const uint32_t bu1 = ((bu[qd + 1] >> (2 * j)) & 0x03030303u) * scu;
                const int64_t Bg = (int64_t)(((uint64_t)bg1 << 32) | bg0);
                const int64_t Bu = (int64_t)(((uint64_t)bu1 << 32) | bu0);
                const int kbg = sb * 8 + kb8;
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    if (s >= ns) break;
                    int64_t A = 0;
                    if (tokA[s] >= 0) A = *reinterpret_cast<const int64_t*>(a.xq + (size_t)tokA[s] * D + kbg * QB + 8 * g);
                    const i32x4_t cg = mfma_i8(A, Bg);
                    const i32x4_t cu = mfma_i8(A, Bu);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float dx = tokC[s][r] >= 0 ? a.xd[(size_t)tokC[s][r] * (D / QB) + kbg] : 0.f;
                        sg[s][r] = fmaf((float)cg[r], dx, sg[s][r]);
                        su[s][r] = fmaf((float)cu[r], dx, su[s][r]);
                    }
                }
            }
            // min part, -dmin * sum_n m_n * X16_n with X16_n = fp16(d of the q8_1 block)
            // times the sum of the sub-block's 16 quants: four f32 16x16x4 matrix-core
            // products per matrix (K = the 16 sub-blocks), accumulated straight into acc
            float bmg[4], bmu[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = 4 * q + g;
                bmg[q] = -dming * (float)((bg[n >> 2] >> (8 * (n & 3) + 4)) & 15);
                bmu[q] = -dminu * (float)((bu[n >> 2] >> (8 * (n & 3) + 4)) & 15);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (s >= ns) break;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    accg[s][r] = fmaf(dg, sg[s][r], accg[s][r]);
                    accu[s][r] = fmaf(du, su[s][r], accu[s][r]);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float x16 = tokA[s] >= 0 ? a.xs16f[(size_t)tokA[s] * (D / 16) + sb * 16 + 4 * q + g] : 0.f;
                    accg[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(x16, bmg[q], accg[s], 0, 0, 0);
                    accu[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(x16, bmu[q], accu[s], 0, 0, 0);
                }
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * s + 4 * g + r;
            if (i < ch.nrows) hout[(size_t)i * I + r0 + wrow] = swiglu(accg[s][r], accu[s][r], a.limit);
        }
    }
}

// ------------------------------------------------------------------ Q3_K down
// LDS: the raw blocks of 64 whole W2 rows (contiguous), then the 64-entry byte
// lookup table (32 - sc6) * (v - 4) for v = 0..7, indexed by sc6.
template <int NS>
__global__ __launch_bounds__(256) void mmq_down_q3k_kernel(ExpertArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int nsb = I / QK;
    const int rowbytes = nsb * Q3K_BYTES;
    const int tiles = D / TILE_ROWS;
    const int c = blockIdx.x / tiles, rt = blockIdx.x % tiles;
    if (c >= *a.n_chunks) return;
    const Chunk ch = a.chunks[c];
    const bool shared = ch.expert < 0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int r0 = rt * TILE_ROWS;
    float* eout = (shared ? a.ys : a.e_rows) + (size_t)ch.row0 * D;
    const uint8_t* w2;
    if (shared) {
        w2 = a.sh_w2;
    } else {
        const int slot = a.slot_table[ch.expert];
        if (slot == SLOT_SKIP) return;   // computed in another slot wave
        if (slot < 0) {
            for (int q = tid; q < TILE_ROWS * ch.nrows; q += 256)
                eout[(size_t)(q / TILE_ROWS) * D + r0 + q % TILE_ROWS] = 0.f;
            return;
        }
        w2 = a.arena + (size_t)slot * a.slot_bytes + a.off_w2;
    }
    uint32_t* lds = reinterpret_cast<uint32_t*>(smem);
    const int tile_bytes = TILE_ROWS * rowbytes;                 // multiple of 16 (64 * 110 * nsb)
    uint2* lut = reinterpret_cast<uint2*>(smem + tile_bytes + 16);   // [64]
    {
        const uint4* src = reinterpret_cast<const uint4*>(w2 + (size_t)r0 * rowbytes);
        uint4* dst = reinterpret_cast<uint4*>(smem);
        for (int q = tid; q < tile_bytes / 16; q += 256) dst[q] = src[q];
        if (tid < 64) {
            const int sneg = 32 - tid;   // -(sc6 - 32)
            uint32_t lo = 0, hi = 0;
            for (int v = 0; v < 4; ++v) lo |= ((uint32_t)((sneg * (v - 4)) & 0xFF)) << (8 * v);
            for (int v = 4; v < 8; ++v) hi |= ((uint32_t)((sneg * (v - 4)) & 0xFF)) << (8 * (v - 4));
            lut[tid] = make_uint2(lo, hi);
        }
    }
    __syncthreads();

    const int hq_ld = I;
    const int8_t* hq = shared ? a.hq_shared : a.hq_routed;
    const float* hd = shared ? a.hd_shared : a.hd_routed;
    const int g = lane >> 4, l16 = lane & 15;
    int rowA[NS], rowC[NS][4];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int ia = 16 * s + l16;
        rowA[s] = ia < ch.nrows ? ch.row0 + ia : -1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int ic = 16 * s + 4 * g + r;
            rowC[s][r] = ic < ch.nrows ? ch.row0 + ic : -1;
        }
    }
    typedef float f4 __attribute__((ext_vector_type(4)));
    f4 acc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = (f4){0.f, 0.f, 0.f, 0.f};
    const int ns = min(NS, (ch.nrows + 15) / 16);
    const int wrow = 16 * wv + l16;
    for (int sb = 0; sb < nsb; ++sb) {
        const int off = wrow * rowbytes + sb * Q3K_BYTES;   // 2-byte aligned
        const int A0 = off >> 2;
        const uint32_t sh = (uint32_t)(off & 3) * 8u;
        const uint32_t s0 = funnel(lds[A0 + 25], lds[A0 + 24], sh);
        const uint32_t s1 = funnel(lds[A0 + 26], lds[A0 + 25], sh);
        const uint32_t s2 = funnel(lds[A0 + 27], lds[A0 + 26], sh);
        const float dneg = -half_bits_to_f32((lds[A0 + 27] >> sh) & 0xFFFFu);
        f4 ss[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s) ss[s] = (f4){0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
        for (int kb8 = 0; kb8 < 8; ++kb8) {
            const int hh = kb8 >> 2, j = kb8 & 3;
            const int n = 8 * hh + 2 * j + (g >> 1);
            // six-bit scale of sub-block n
            const uint32_t low4 = (((n & 7) < 4 ? s0 : s1) >> (8 * (n & 3) + 4 * (n >> 3))) & 15;
            const uint32_t hi2 = (s2 >> (8 * (n & 3) + 2 * (n >> 2))) & 3;
            const uint2 L = lut[low4 | (hi2 << 4)];
            // q3 + 4 for positions 8g..8g+7 of plane j, half hh
            const int qdw = A0 + 8 + 8 * hh + 2 * g;   // qs[32 hh + 8 g] (before the realignment)
            const int hdw = A0 + 2 * g;                // hmask[8 g]
            const uint32_t q0 = funnel(lds[qdw + 1], lds[qdw], sh), q1 = funnel(lds[qdw + 2], lds[qdw + 1], sh);
            const uint32_t m0 = funnel(lds[hdw + 1], lds[hdw], sh), m1 = funnel(lds[hdw + 2], lds[hdw + 1], sh);
            const int hbit = 4 * hh + j;
            const uint32_t v0 = ((q0 >> (2 * j)) & 0x03030303u) | (((m0 >> hbit) & 0x01010101u) << 2);
            const uint32_t v1 = ((q1 >> (2 * j)) & 0x03030303u) | (((m1 >> hbit) & 0x01010101u) << 2);
            const uint32_t b0 = __builtin_amdgcn_perm(L.y, L.x, v0);
            const uint32_t b1 = __builtin_amdgcn_perm(L.y, L.x, v1);
            const int64_t B = (int64_t)(((uint64_t)b1 << 32) | b0);
            const int kbg = sb * 8 + kb8;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (s >= ns) break;
                int64_t A = 0;
                if (rowA[s] >= 0) A = *reinterpret_cast<const int64_t*>(hq + (size_t)rowA[s] * hq_ld + kbg * QB + 8 * g);
                const i32x4_t cc = mfma_i8(A, B);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float dx = rowC[s][r] >= 0 ? hd[(size_t)rowC[s][r] * (I / QB) + kbg] : 0.f;
                    ss[s][r] = fmaf((float)cc[r], dx, ss[s][r]);
                }
            }
        }
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[s][r] = fmaf(dneg, ss[s][r], acc[s][r]);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * s + 4 * g + r;
            if (i < ch.nrows) eout[(size_t)i * D + r0 + wrow] = acc[s][r];
        }
    }
}

// ------------------------------------------------------------------ launch
bool mmq_supported(int D, int I) {
    // whole 64-row tiles, and the W2 tile plus its lookup table within LDS
    return I % TILE_ROWS == 0 && D % TILE_ROWS == 0 &&
           (size_t)TILE_ROWS * (I / QK) * Q3K_BYTES + 16 + 64 * 8 <= 160 * 1024;
}

template <int NS>
static hipError_t launch_mmq_ns(const ExpertArgs& a, int max_chunks, bool gateup, hipStream_t st) {
    if (gateup) {
        const int KS = 4;
        const size_t lds = (size_t)128 * KS * Q2K_BYTES;
        return launch_kernel(mmq_gateup_q2k_kernel<NS>, max_chunks * (a.I / TILE_ROWS), 256, lds, st, a, KS);
    }
    const size_t lds = (size_t)TILE_ROWS * (a.I / QK) * Q3K_BYTES + 16 + 64 * 8;
    return launch_kernel(mmq_down_q3k_kernel<NS>, max_chunks * (a.D / TILE_ROWS), 256, lds, st, a);
}

hipError_t launch_mmq(const ExpertArgs& a, const ChunkPlan& plan, bool gateup, hipStream_t st) {
    for (int c = 0; c < MMQ_CLASSES; ++c) {
        if (plan.cap[c] <= 0) continue;
        ExpertArgs ac = a;
        ac.chunks = a.chunks + plan.base[c];
        ac.n_chunks = a.n_chunks + c;
        const hipError_t e = c == 0   ? launch_mmq_ns<1>(ac, plan.cap[c], gateup, st)
                             : c == 1 ? launch_mmq_ns<2>(ac, plan.cap[c], gateup, st)
                                      : launch_mmq_ns<4>(ac, plan.cap[c], gateup, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace moe
