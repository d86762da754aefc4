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


}  // namespace

// Workgroups are spread over the 8 XCDs round-robin by id; the tiles of one
// chunk are given consecutive logical ids on one XCD so that their shared
// activation rows are fetched into one L2 (nb_pad is a multiple of 8).
MOE_DEV int xcd_logical_block(int b, int nb_pad) { return (b & 7) * (nb_pad >> 3) + (b >> 3); }

// ------------------------------------------------------------------ Q2_K gate/up
// Rounds of KS = 2 superblocks. Per round the workgroup stages, through
// registers into LDS (the next round's loads in flight while the current
// round is computed): the raw blocks of its 64 W1 and 64 W3 rows, the q8_1
// quants of its token rows, their block scales and their per-16 sums (both
// transposed to [k][row] so a lane reads its four C rows at once).
namespace {
constexpr int GKS = 2;                        // superblocks per round
constexpr int GW_DW = GKS * Q2K_BYTES / 4;    // 42 dwords of one row per round
constexpr int GA_STRIDE = GKS * QK + 16;      // bytes per token row in LDS (padded against bank conflicts)

template <int NS>
struct GateupLds {
    static constexpr int rows = NS * 16;
    static constexpr int w_bytes = 128 * GW_DW * 4;
    static constexpr int a_off = w_bytes;
    static constexpr int dx_off = a_off + rows * GA_STRIDE;        // [GKS * 8][rows] f32
    static constexpr int x16_off = dx_off + GKS * 8 * rows * 4;    // [GKS * 16][rows] f32
    static constexpr int bytes = x16_off + GKS * 16 * rows * 4;
};
}  // namespace

template <int NS>
__global__ __launch_bounds__(256) void mmq_gateup_q2k_kernel(ExpertArgs a, int nb) {
    extern __shared__ __align__(16) uint8_t smem[];
    using LL = GateupLds<NS>;
    const int D = a.D, I = a.I;
    const int nsb = D / QK;
    const int tiles = I / TILE_ROWS;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    if (lb >= nb) return;
    const int c = lb / tiles, rt = lb % tiles;
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
    const int rounds = (nsb + GKS - 1) / GKS;

    // --- staging assignments (fixed over the rounds; the last round may hold one superblock)
    // weights: dword q = tid + 256 u of the [128 rows][ks * 21] segment
    // activations: 16-byte chunk q = tid + 256 u of the [rows][ks * 16] quants
    constexpr int NW = 128 * GW_DW / 256;          // 21
    constexpr int NA = (LL::rows * GKS * 16 + 255) / 256;
    uint32_t wr[NW];
    uint4 ar[NA];
    uint4 dxr, x16r0, x16r1;
    auto token_of = [&](int i) { return i < ch.nrows ? (shared ? ch.row0 + i : a.perm[ch.row0 + i] / a.topk) : -1; };
    auto stage_load = [&](int rd) {
        const int sb0 = rd * GKS, ks = min(GKS, nsb - sb0), seg = ks * 21;
        // weights: row = q / seg (magic multipliers, exact for q < 128 * 42)
#pragma unroll
        for (int u = 0; u < NW; ++u) {
            const int q = tid + 256 * u;
            const int row = ks == 2 ? (int)(((uint32_t)q * 24967u) >> 20) : (int)(((uint32_t)q * 49933u) >> 20);
            const int dw = q - row * seg;
            wr[u] = 0u;
            if (row < 128) {
                const uint8_t* src = (row < 64 ? w1 + (size_t)(r0 + row) * rowbytes
                                               : w3 + (size_t)(r0 + row - 64) * rowbytes) + (size_t)sb0 * Q2K_BYTES;
                wr[u] = reinterpret_cast<const uint32_t*>(src)[dw];
            }
        }
        const int cpr = ks * 16;   // 16-byte chunks of quants per token row
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int q = tid + 256 * u;
            const int row = q / cpr, col = q % cpr;
            ar[u] = make_uint4(0u, 0u, 0u, 0u);
            if (row < LL::rows) {
                const int t = token_of(row);
                if (t >= 0) ar[u] = reinterpret_cast<const uint4*>(a.xq + (size_t)t * D + sb0 * QK)[col];
            }
        }
        // scales: row = tid / (2 ks), 4 consecutive blocks; 16-sums: row = tid / (4 ks)
        dxr = make_uint4(0u, 0u, 0u, 0u);
        {
            const int row = tid / (2 * ks), col = tid % (2 * ks);
            if (row < LL::rows) {
                const int t = token_of(row);
                if (t >= 0) dxr = reinterpret_cast<const uint4*>(a.xd + (size_t)t * (D / QB) + sb0 * 8)[col];
            }
        }
        x16r0 = x16r1 = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int q = tid + 256 * u;
            const int row = q / (4 * ks), col = q % (4 * ks);
            if (row < LL::rows) {
                const int t = token_of(row);
                if (t >= 0) {
                    const uint4 v = reinterpret_cast<const uint4*>(a.xs16f + (size_t)t * (D / 16) + sb0 * 16)[col];
                    if (u == 0) x16r0 = v; else x16r1 = v;
                }
            }
        }
    };
    auto stage_store = [&](int rd) {
        const int sb0 = rd * GKS, ks = min(GKS, nsb - sb0), seg = ks * 21;
        uint32_t* wl = reinterpret_cast<uint32_t*>(smem);
#pragma unroll
        for (int u = 0; u < NW; ++u) {
            const int q = tid + 256 * u;
            const int row = ks == 2 ? (int)(((uint32_t)q * 24967u) >> 20) : (int)(((uint32_t)q * 49933u) >> 20);
            if (row < 128) wl[row * GW_DW + (q - row * seg)] = wr[u];
        }
        const int cpr = ks * 16;
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int q = tid + 256 * u;
            const int row = q / cpr, col = q % cpr;
            if (row < LL::rows) *reinterpret_cast<uint4*>(smem + LL::a_off + row * GA_STRIDE + col * 16) = ar[u];
        }
        float* dxl = reinterpret_cast<float*>(smem + LL::dx_off);
        {
            const int row = tid / (2 * ks), col = tid % (2 * ks);
            if (row < LL::rows) {
                dxl[(4 * col + 0) * LL::rows + row] = __uint_as_float(dxr.x);
                dxl[(4 * col + 1) * LL::rows + row] = __uint_as_float(dxr.y);
                dxl[(4 * col + 2) * LL::rows + row] = __uint_as_float(dxr.z);
                dxl[(4 * col + 3) * LL::rows + row] = __uint_as_float(dxr.w);
            }
        }
        float* xl = reinterpret_cast<float*>(smem + LL::x16_off);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int q = tid + 256 * u;
            const int row = q / (4 * ks), col = q % (4 * ks);
            const uint4 v = u == 0 ? x16r0 : x16r1;
            if (row < LL::rows) {
                xl[(4 * col + 0) * LL::rows + row] = __uint_as_float(v.x);
                xl[(4 * col + 1) * LL::rows + row] = __uint_as_float(v.y);
                xl[(4 * col + 2) * LL::rows + row] = __uint_as_float(v.z);
                xl[(4 * col + 3) * LL::rows + row] = __uint_as_float(v.w);
            }
        }
    };

    // A rows: token of sub-tile s, row lane % 16; C rows: tokens 4 (lane / 16) + r
    const int g = lane >> 4, l16 = lane & 15;
    typedef float f4 __attribute__((ext_vector_type(4)));
    f4 accg[NS], accu[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) accg[s] = accu[s] = (f4){0.f, 0.f, 0.f, 0.f};
    const int ns = min(NS, (ch.nrows + 15) / 16);   // sub-tiles holding tokens
    const int wrow = 16 * wv + l16;                   // this lane's weight row (B column) in the tile
    const uint32_t* wl = reinterpret_cast<const uint32_t*>(smem);
    const float* dxl = reinterpret_cast<const float*>(smem + LL::dx_off);
    const float* xl = reinterpret_cast<const float*>(smem + LL::x16_off);

    stage_load(0);
    for (int rd = 0; rd < rounds; ++rd) {
        if (rd > 0) __syncthreads();   // the previous round is consumed
        stage_store(rd);
        __syncthreads();
        if (rd + 1 < rounds) stage_load(rd + 1);   // in flight during this round's products
        const int ks = min(GKS, nsb - rd * GKS);
        for (int sbi = 0; sbi < ks; ++sbi) {
            const uint32_t* bg = wl + wrow * GW_DW + sbi * 21;
            const uint32_t* bu = wl + (64 + wrow) * GW_DW + sbi * 21;
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
                const int kk = sbi * 8 + kb8;   // block within the round
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    if (s >= ns) break;
                    const int64_t A = *reinterpret_cast<const int64_t*>(smem + LL::a_off + (16 * s + l16) * GA_STRIDE +
                                                                        kk * QB + 8 * g);
                    const i32x4_t cg = mfma_i8(A, Bg);
                    const i32x4_t cu = mfma_i8(A, Bu);
                    const f4 dx = *reinterpret_cast<const f4*>(dxl + kk * LL::rows + 16 * s + 4 * g);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        sg[s][r] = fmaf((float)cg[r], dx[r], sg[s][r]);
                        su[s][r] = fmaf((float)cu[r], dx[r], su[s][r]);
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
                    const float x16 = xl[(sbi * 16 + 4 * q + g) * LL::rows + 16 * s + l16];
                    accg[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(x16, bmg[q], accg[s], 0, 0, 0);
                    accu[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(x16, bmu[q], accu[s], 0, 0, 0);
                }
            }
        }
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
// LDS: the raw blocks of the 64 whole W2 rows (contiguous, staged once), the
// 64-entry byte lookup table (32 - sc6) * (v - 4) for v = 0..7 indexed by sc6,
// then per superblock the q8_1 quants of the chunk's h rows and their block
// scales ([k][row]), staged through registers one superblock ahead.
namespace {
constexpr int DA_STRIDE = QK + 16;  // bytes per h row in LDS (padded against bank conflicts)
template <int NS>
struct DownLds {
    static constexpr int rows = NS * 16;
    __host__ __device__ static int w_bytes(int I) { return TILE_ROWS * (I / QK) * Q3K_BYTES; }   // multiple of 16
    __host__ __device__ static int lut_off(int I) { return w_bytes(I) + 16; }
    __host__ __device__ static int a_off(int I) { return lut_off(I) + 64 * 8; }
    __host__ __device__ static int dx_off(int I) { return a_off(I) + rows * DA_STRIDE; }   // [8][rows] f32
    __host__ __device__ static int bytes(int I) { return dx_off(I) + 8 * rows * 4; }
};
}  // namespace

template <int NS>
__global__ __launch_bounds__(256) void mmq_down_q3k_kernel(ExpertArgs a, int nb) {
    extern __shared__ __align__(16) uint8_t smem[];
    using LL = DownLds<NS>;
    const int D = a.D, I = a.I;
    const int nsb = I / QK;
    const int rowbytes = nsb * Q3K_BYTES;
    const int tiles = D / TILE_ROWS;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    if (lb >= nb) return;
    const int c = lb / tiles, rt = lb % tiles;
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
    const int8_t* hq = shared ? a.hq_shared : a.hq_routed;
    const float* hd = shared ? a.hd_shared : a.hd_routed;
    const int rows_valid = ch.nrows;
    // per superblock: 16-byte chunk q = tid + 256 u of [rows][16] quants; scales: row = tid / 2
    constexpr int NA = (LL::rows * 16 + 255) / 256;
    uint4 ar[NA];
    uint4 dxr;
    auto stage_load = [&](int sb) {
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int q = tid + 256 * u;
            const int row = q >> 4, col = q & 15;
            ar[u] = make_uint4(0u, 0u, 0u, 0u);
            if (row < rows_valid && row < LL::rows)
                ar[u] = reinterpret_cast<const uint4*>(hq + (size_t)(ch.row0 + row) * I + sb * QK)[col];
        }
        dxr = make_uint4(0u, 0u, 0u, 0u);
        const int row = tid >> 1, col = tid & 1;
        if (row < rows_valid && row < LL::rows)
            dxr = reinterpret_cast<const uint4*>(hd + (size_t)(ch.row0 + row) * (I / QB) + sb * 8)[col];
    };
    auto stage_store = [&]() {
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int q = tid + 256 * u;
            const int row = q >> 4, col = q & 15;
            if (row < LL::rows) *reinterpret_cast<uint4*>(smem + LL::a_off(I) + row * DA_STRIDE + col * 16) = ar[u];
        }
        float* dxl = reinterpret_cast<float*>(smem + LL::dx_off(I));
        const int row = tid >> 1, col = tid & 1;
        if (row < LL::rows) {
            dxl[(4 * col + 0) * LL::rows + row] = __uint_as_float(dxr.x);
            dxl[(4 * col + 1) * LL::rows + row] = __uint_as_float(dxr.y);
            dxl[(4 * col + 2) * LL::rows + row] = __uint_as_float(dxr.z);
            dxl[(4 * col + 3) * LL::rows + row] = __uint_as_float(dxr.w);
        }
    };
    stage_load(0);
    uint32_t* lds = reinterpret_cast<uint32_t*>(smem);
    const int tile_bytes = LL::w_bytes(I);
    uint2* lut = reinterpret_cast<uint2*>(smem + LL::lut_off(I));   // [64]
    {
        const uint4* src = reinterpret_cast<const uint4*>(w2 + (size_t)r0 * rowbytes);
        uint4* dst = reinterpret_cast<uint4*>(smem);
        const int n16 = tile_bytes / 16;
        int q = tid;
        for (; q + 3 * 256 < n16; q += 4 * 256) {   // four loads in flight per step
            const uint4 v0 = src[q], v1 = src[q + 256], v2 = src[q + 512], v3 = src[q + 768];
            dst[q] = v0;
            dst[q + 256] = v1;
            dst[q + 512] = v2;
            dst[q + 768] = v3;
        }
        for (; q < n16; q += 256) dst[q] = src[q];
        if (tid < 64) {
            const int sneg = 32 - tid;   // -(sc6 - 32)
            uint32_t lo = 0, hi = 0;
            for (int v = 0; v < 4; ++v) lo |= ((uint32_t)((sneg * (v - 4)) & 0xFF)) << (8 * v);
            for (int v = 4; v < 8; ++v) hi |= ((uint32_t)((sneg * (v - 4)) & 0xFF)) << (8 * (v - 4));
            lut[tid] = make_uint2(lo, hi);
        }
    }

    const int g = lane >> 4, l16 = lane & 15;
    typedef float f4 __attribute__((ext_vector_type(4)));
    f4 acc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = (f4){0.f, 0.f, 0.f, 0.f};
    const int ns = min(NS, (ch.nrows + 15) / 16);
    const int wrow = 16 * wv + l16;
    const float* dxl = reinterpret_cast<const float*>(smem + LL::dx_off(I));
    for (int sb = 0; sb < nsb; ++sb) {
        if (sb > 0) __syncthreads();   // the previous superblock's activations are consumed
        stage_store();
        __syncthreads();
        if (sb + 1 < nsb) stage_load(sb + 1);
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
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (s >= ns) break;
                const int64_t A = *reinterpret_cast<const int64_t*>(smem + LL::a_off(I) + (16 * s + l16) * DA_STRIDE +
                                                                    kb8 * QB + 8 * g);
                const i32x4_t cc = mfma_i8(A, B);
                const f4 dx = *reinterpret_cast<const f4*>(dxl + kb8 * LL::rows + 16 * s + 4 * g);
#pragma unroll
                for (int r = 0; r < 4; ++r) ss[s][r] = fmaf((float)cc[r], dx[r], ss[s][r]);
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
    // whole 64-row tiles, and the W2 tile, its lookup table and the widest
    // class's activation rows within LDS
    return I % TILE_ROWS == 0 && D % TILE_ROWS == 0 && DownLds<4>::bytes(I) <= 160 * 1024;
}

template <int NS>
static hipError_t launch_mmq_ns(const ExpertArgs& a, int max_chunks, bool gateup, hipStream_t st) {
    const int nb = max_chunks * (gateup ? a.I / TILE_ROWS : a.D / TILE_ROWS);
    const int nb_pad = (nb + 7) / 8 * 8;
    if (gateup)
        return launch_kernel(mmq_gateup_q2k_kernel<NS>, nb_pad, 256, (size_t)GateupLds<NS>::bytes, st, a, nb);
    return launch_kernel(mmq_down_q3k_kernel<NS>, nb_pad, 256, (size_t)DownLds<NS>::bytes(a.I), st, a, nb);
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
