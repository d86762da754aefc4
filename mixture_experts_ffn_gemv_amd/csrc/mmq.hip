// Expert-grouped MMQ for batched calls: the routed experts' products as
// int8 matrix-core tiles over the still-quantised blocks (metrale moe_v41
// module documentation: "by default MMQ above" eight rows; kernel table of
// moe_v41.rs: mmq_q2k_* / mmq_q3k_*).
//
// A chunk is one expert with up to MMQ_ROWS token rows (in three size classes,
// each launched with the sub-tile count it needs). One workgroup computes
// 64 output rows of one chunk: gate/up for 64 rows of W1 and the same rows of
// W3 (then the clamped SwiGLU), or down for 64 rows of W2. Weights form the A
// operand (16 rows per wavefront), the chunk's tokens the B operand (16-column
// sub-tiles of q8_1 quants); v_mfma_i32_16x16x32_i8 has K = 32, exactly one
// q8_1 block, so each product is rescaled by that block's activation scale,
// one scalar per lane since a lane's accumulators share one token column.
//  * Q2_K: the A bytes are sc_n * q (<= 45), so d * (A . B) covers the scale
//    part of the weight; the min part -dmin * m_n * sum(B) is added per
//    superblock from the per-16 sums of the activation quants.
//  * Q3_K: the A bytes are (32 - sc6_n) * q3 = -(sc6_n - 32) q3, which lies in
//    [-128, 124] (the unnegated product would reach +128), built with a
//    byte lookup from q3 + 4; the sign goes into d.
// Weight tiles are whole 8-row panels (the slot layout stores a panel's rows
// of one superblock column as one contiguous run), streamed through LDS by the
// wavefront-wide global-to-LDS load path.
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


// ------------------------------------------------------------------ Q2_K gate/up
// Weights are the A operand (16 rows of W1 and the same 16 rows of W3 per
// wavefront, 64 per workgroup), the chunk's token rows the B operand (NS
// sub-tiles of 16 columns): C[row][token] = v_mfma_i32_16x16x32_i8 over one
// q8_1 block, rescaled by the token's block scale (C column = lane % 16, so
// one scalar per lane and block).
//  * Per superblock the workgroup's 2 x 64 weight rows (eight panels of each
//    matrix: one contiguous 672-byte run per panel) and the activations of
//    its token rows (quants, block scales, the min-term sums) go from global
//    memory straight into LDS with wavefront-wide loads; the weights land as
//    [matrix][row][84 bytes] (a 21-dword row stride: the 16 rows a wavefront
//    reads lie in distinct banks), the quants transposed to [16-byte
//    chunk][token], the block scales as [token][8 blocks], the min-term sums as
//    [token][96 bytes]. Two superblocks are in LDS: one is computed while the
//    next is in flight.
//  * Every sub-tile is computed whether or not the chunk fills it (rows past
//    the chunk repeat its last row and are never stored): no branches inside
//    the unrolled block loop. Each block's B reads (and scales) are issued one
//    block ahead, and each block is its own scheduling region, so the compiler
//    does not hold several blocks' products in registers at once.
//  * A lane (row = lane % 16, g = lane / 16) takes from its row's superblock
//    the sixteen scale bytes, d / dmin and the qs bytes 8g..8g+7 of both
//    halves, which hold its eight K values of all four planes. The A bytes
//    sc_n * q come from a byte lookup (v_perm_b32 on [3 sc, 2 sc, sc, 0]
//    indexed by 3 - q).
//  * The min part -dmin * sum_n m_n * X16_n (X16 = block scale times the sum
//    of 16 quants, an f32 with at most 24 significant bits) is a K = 16
//    product per superblock. With four sub-tiles it runs on the bf16 matrix
//    core: the quantiser stores each X16 as three bf16 pieces hi + mid + lo
//    (exact), and two v_mfma_f32_16x16x32_bf16 per matrix and sub-tile take
//    K = [16 sub-blocks x (hi, mid)] and [16 x (lo, -)] against A = m_n (exact
//    in bf16); the product goes out with -dmin of its rows, each sub-tile and
//    matrix in its own block region. With one or two sub-tiles the A operand
//    of that path would be built for too few products: there it is four
//    v_mfma_f32_16x16x4_f32 per matrix and sub-tile on the f32 sums, with
//    A = -dmin * m_n.
namespace {
constexpr int GW_UNITS = 2 * TILE_ROWS * Q2K_BYTES / 16;   // 16-byte units of one superblock column (672)
constexpr int GW_LOADS = (GW_UNITS + 255) / 256;           // per thread (3)
constexpr int X16_REC = 96;                                // bytes of one token's min-term sums per superblock

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));

template <int NS>
struct GateupLds {
    static constexpr int R = NS * 16;                        // token rows
    static constexpr int nbuf = 2;                           // superblocks in LDS: one computed, one in flight
    static constexpr int w_off = 0;                          // [2 matrices][64 rows][84 B] (+ overrun)
    static constexpr int q_off = w_off + GW_LOADS * 256 * 16;   // [16 chunks][R] x 16 B
    static constexpr int ndx = (8 * R + 255) / 256;          // dword loads per thread for the block scales
    static constexpr int dx_off = q_off + 16 * R * 16;       // [R][8 blocks] f32 (+ padding to ndx * 256)
    // the min-term sums: bf16 pieces [R][96 B] for four sub-tiles (16-byte loads; a wave
    // past the end skips, the last one's overrun is kept), else f32 [16 sub-blocks][R]
    static constexpr bool bf16_min = NS == 4;
    static constexpr int x16_units = R * X16_REC / 16;       // 16-byte units of the bf16 pieces
    static constexpr int nx16 = (x16_units + 255) / 256;     // loads per thread
    static constexpr int x16_off = dx_off + ndx * 256 * 4;
    static constexpr int buf_bytes = x16_off + (bf16_min ? (x16_units + 63) / 64 * 64 * 16 : 16 * R * 4);
    static constexpr int xch_off = nbuf * buf_bytes;         // [4 waves][d W1, d W3, -dmin W1, -dmin W3][16 rows] f32
    static constexpr int bytes = xch_off + 4 * 4 * 16 * 4;
};

// bf16 of two small non-negative integers (exact), packed low | high
MOE_DEV uint32_t bf16_pair(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
}  // namespace

template <int NS>
__global__ __launch_bounds__(256) void mmq_gateup_q2k_kernel(ExpertArgs a, int nb) {
    extern __shared__ __align__(16) uint8_t smem[];
    using LL = GateupLds<NS>;
    constexpr int R = LL::R;
    const int D = a.D, I = a.I;
    const int nsb = D / QK;
    const int tiles = I / TILE_ROWS;
    const int nb_act = min(nb, *a.n_chunks * tiles);   // blocks with work this call (nb: the grid's)
    const int lb = xcd_logical_block(blockIdx.x, nb_act);
    if (lb >= nb_act) return;
    const int c = lb / tiles, rt = lb % tiles;
    const Chunk ch = a.chunks[c];
    const bool shared = ch.expert < 0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15;
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
    // the token (x row) of chunk row t; rows past the chunk repeat its last row
    auto token_of = [&](int t) {
        const int tr = max(0, min(t, ch.nrows - 1));
        return shared ? ch.row0 + tr : a.perm[ch.row0 + tr] / a.topk;
    };

    // staging of one superblock into buffer bi (every thread issues LL::ndma loads)
    const int8_t* xq_row = a.xq + (size_t)token_of(tid & (R - 1)) * D;
    // block-scale unit i = 256 u + tid: block i % 8 of token row i / 8 (rows past R
    // repeat the last one)
    const float* xd_src[LL::ndx];
#pragma unroll
    for (int u = 0; u < LL::ndx; ++u) {
        const int i = u * 256 + tid;
        xd_src[u] = a.xd + (size_t)token_of(min(i >> 3, R - 1)) * (D / QB) + (i & 7);
    }
    // min-term unit i = 256 u + tid: 16-byte piece i % 6 of token row i / 6's record
    // (units past the end repeat the last one into the overrun)
    const uint8_t* x16_src[LL::bf16_min ? LL::nx16 : 1];
    if constexpr (LL::bf16_min) {
#pragma unroll
        for (int u = 0; u < LL::nx16; ++u) {
            const int i = min(u * 256 + tid, LL::x16_units - 1);
            x16_src[u] = reinterpret_cast<const uint8_t*>(a.xs16b) + (size_t)token_of(i / 6) * nsb * X16_REC +
                         (i % 6) * 16;
        }
    } else {   // f32 unit p = 256 u + tid: sub-block p / R of token row p % R (one row per thread)
        x16_src[0] = reinterpret_cast<const uint8_t*>(a.xs16f + (size_t)token_of(tid & (R - 1)) * (D / 16));
    }
    // weight unit f = 256 u + tid of a superblock column: matrix f / 336, panel (f % 336) / 42,
    // 16-byte piece f % 42 (units past the end repeat the last one into the overrun)
    const uint8_t* wsrc[GW_LOADS];
#pragma unroll
    for (int u = 0; u < GW_LOADS; ++u) {
        const int f = min(256 * u + tid, GW_UNITS - 1);
        const int m = f / (GW_UNITS / 2), rem = f % (GW_UNITS / 2);
        const int pp = rem / (PANEL * Q2K_BYTES / 16), k = rem % (PANEL * Q2K_BYTES / 16);
        wsrc[u] = (m ? w3 : w1) + (size_t)(r0 + PANEL * pp) * rowbytes + k * 16;
    }
    auto stage = [&](int sb, int bi) {
        uint8_t* buf = smem + bi * LL::buf_bytes;
#pragma unroll
        for (int u = 0; u < GW_LOADS; ++u)
            load_lds16(wsrc[u] + (size_t)sb * (PANEL * Q2K_BYTES), buf + LL::w_off + (u * 256 + wv * 64) * 16);
#pragma unroll
        for (int u = 0; u < NS; ++u) {   // unit p = u * 256 + tid: 16-byte chunk p / R of row p % R
            const int kc = (u * 256 + tid) / R;
            load_lds16(xq_row + (size_t)sb * QK + kc * 16, buf + LL::q_off + (u * 256 + wv * 64) * 16);
        }
#pragma unroll
        for (int u = 0; u < LL::ndx; ++u)
            load_lds4(xd_src[u] + (size_t)sb * 8, buf + LL::dx_off + (u * 256 + wv * 64) * 4);
        if constexpr (LL::bf16_min) {
#pragma unroll
            for (int u = 0; u < LL::nx16; ++u)
                if (u * 256 + wv * 64 < LL::x16_units)   // wave-uniform
                    load_lds16(x16_src[u] + (size_t)sb * X16_REC, buf + LL::x16_off + (u * 256 + wv * 64) * 16);
        } else {
#pragma unroll
            for (int u = 0; u < NS; ++u) {
                const int n = (u * 256 + tid) / R;
                load_lds4(x16_src[0] + ((size_t)sb * 16 + n) * 4, buf + LL::x16_off + (u * 256 + wv * 64) * 4);
            }
        }
    };

    // this lane's weight rows in LDS (dword offsets), W1 and W3
    const int wr = 16 * wv + l16;
    const int wo1 = wr * (Q2K_BYTES / 4);
    const int wo3 = wo1 + TILE_ROWS * (Q2K_BYTES / 4);

    typedef float f4 __attribute__((ext_vector_type(4)));
    f4 accg[NS], accu[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) accg[s] = accu[s] = (f4){0.f, 0.f, 0.f, 0.f};
    float* xch = reinterpret_cast<float*>(smem + LL::xch_off) + wv * 64;

    stage(0, 0);
    for (int sb = 0; sb < nsb; ++sb) {
        wait_vm_loads<0>();   // superblock sb is in LDS ...
        barrier_lds();        // ... for every wave; the buffer of superblock sb - 1 is free
        const int bcur = sb & 1;
        if (sb + 1 < nsb) stage(sb + 1, bcur ^ 1);
        const uint8_t* buf = smem + bcur * LL::buf_bytes;
        const uint32_t* wl = reinterpret_cast<const uint32_t*>(buf + LL::w_off);
        const float* dxl = reinterpret_cast<const float*>(buf + LL::dx_off);
        const uint8_t* x16l = buf + LL::x16_off;
        uint32_t cw[2][9];   // scales, qs 8g.. (2 dwords), qs 32 + 8g.. (2), d | dmin
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const uint32_t* p = wl + (m ? wo3 : wo1);
#pragma unroll
            for (int q = 0; q < 4; ++q) cw[m][q] = p[q];
            cw[m][4] = p[4 + 2 * g];
            cw[m][5] = p[5 + 2 * g];
            cw[m][6] = p[12 + 2 * g];
            cw[m][7] = p[13 + 2 * g];
            cw[m][8] = p[20];
        }
        // d and -dmin of the four C rows 4g..4g+3 (held by the lanes of those rows)
        if (g == 0) {
            xch[l16] = half_bits_to_f32(cw[0][8] & 0xFFFFu);
            xch[16 + l16] = half_bits_to_f32(cw[1][8] & 0xFFFFu);
            xch[32 + l16] = -half_bits_to_f32(cw[0][8] >> 16);
            xch[48 + l16] = -half_bits_to_f32(cw[1][8] >> 16);
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const f4 dG = *reinterpret_cast<const f4*>(xch + 4 * g);
        const f4 dU = *reinterpret_cast<const f4*>(xch + 16 + 4 * g);
        const f4 nG = *reinterpret_cast<const f4*>(xch + 32 + 4 * g);
        const f4 nU = *reinterpret_cast<const f4*>(xch + 48 + 4 * g);
        // min-part A operands: m_n of this lane's row for n = 8 (g % 2) + 0..7 as bf16
        // (first product: against the hi plane for g < 2, the mid plane for g >= 2;
        // second: the lo plane for g < 2, nothing for g >= 2)
        u32x4_v am[2], am2[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if constexpr (!LL::bf16_min) break;
            // scale bytes 8 (g % 2)..+7 (read again from LDS: a lane-dependent pick among
            // the registers would go through scratch memory)
            const uint2 sw = *reinterpret_cast<const uint2*>(wl + (m ? wo3 : wo1) + 2 * (g & 1));
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t nib = (h ? sw.y : sw.x) >> 4 & 0x0F0F0F0Fu;
                am[m][2 * h] = bf16_pair((float)(nib & 0xFFu), (float)(nib >> 8 & 0xFFu));
                am[m][2 * h + 1] = bf16_pair((float)(nib >> 16 & 0xFFu), (float)(nib >> 24));
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) am2[m][q] = g < 2 ? am[m][q] : 0u;
        }
        // B of block kb8: the 8 quants of this lane's token (column) and K slice, and
        // the token's scale of that block
        auto load_b = [&](int kb8, int64_t* B, float* dx) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                B[s] = *reinterpret_cast<const int64_t*>(
                    buf + LL::q_off + ((2 * kb8 + (g >> 1)) * R + 16 * s + l16) * 16 + 8 * (g & 1));
                dx[s] = dxl[(16 * s + l16) * 8 + kb8];
            }
        };
        // min-part B of sub-tile s: this lane's token's (hi | mid) and (lo | lo) pieces
        auto load_x16 = [&](int s, u32x4_v& b1, u32x4_v& b2) {
            const uint8_t* rec = x16l + (16 * s + l16) * X16_REC;
            b1 = *reinterpret_cast<const u32x4_v*>(rec + 16 * g);
            b2 = *reinterpret_cast<const u32x4_v*>(rec + 64 + 16 * (g & 1));
        };
        f4 sg[NS], su[NS];
        int64_t Bn[NS];
        float dxn[NS];
        u32x4_v xb1, xb2;
        f4 rmin = {0.f, 0.f, 0.f, 0.f};
        load_b(0, Bn, dxn);
        if constexpr (LL::bf16_min) load_x16(0, xb1, xb2);
#pragma unroll
        for (int kb8 = 0; kb8 < 8; ++kb8) {
            // one block per scheduling region (the next block's B reads issued first);
            // the empty asm statements below pin each block's rescaled sums in place, so
            // the compiler cannot sink the rescale past later blocks' products (which
            // would hold every block's results in registers at once)
            __builtin_amdgcn_sched_barrier(0);
            const int hh = kb8 >> 2, j = kb8 & 3;
            int64_t B[NS];
            float dxc[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                B[s] = Bn[s];
                dxc[s] = dxn[s];
            }
            if (kb8 < 7) load_b(kb8 + 1, Bn, dxn);
            // this lane's 8 weights: positions 8g..8g+7 of plane j, half hh (sub-block 8hh + 2j + g / 2)
            const int nsh = 8 * ((2 * j + (g >> 1)) & 3);
            int64_t Aw[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                // lookup bytes 3 sc, 2 sc, sc, 0, indexed by 3 - q (the inverted 2-bit field)
                const uint32_t sc = (cw[m][2 * hh + (j >> 1)] >> nsh) & 15u;
                const uint32_t lut = __umul24(sc, 0x010203u);
                const uint32_t s0 = ((cw[m][4 + 2 * hh] >> (2 * j)) & 0x03030303u) ^ 0x03030303u;
                const uint32_t s1 = ((cw[m][5 + 2 * hh] >> (2 * j)) & 0x03030303u) ^ 0x03030303u;
                const uint32_t b0 = __builtin_amdgcn_perm(lut, lut, s0);
                const uint32_t b1 = __builtin_amdgcn_perm(lut, lut, s1);
                Aw[m] = (int64_t)(((uint64_t)b1 << 32) | b0);
            }
            i32x4_t cg[NS], cu[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                cg[s] = mfma_i8(Aw[0], B[s]);
                cu[s] = mfma_i8(Aw[1], B[s]);
            }
            // the min part of the previous region's sub-tile and matrix goes out
            if (LL::bf16_min && kb8 > 0) {
                const int sp = (kb8 - 1) >> 1;
                f4& acc = (kb8 - 1) & 1 ? accu[sp] : accg[sp];
                const f4& nd = (kb8 - 1) & 1 ? nU : nG;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] = fmaf(nd[r], rmin[r], acc[r]);
            }
            // this region's: sub-tile kb8 / 2, matrix kb8 % 2
            if constexpr (LL::bf16_min) {
                const int m = kb8 & 1;
                rmin = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, am[m]),
                                                              __builtin_bit_cast(bf16x8_v, xb1),
                                                              (f4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                rmin = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, am2[m]),
                                                              __builtin_bit_cast(bf16x8_v, xb2), rmin, 0, 0, 0);
                if (m == 1 && (kb8 >> 1) + 1 < NS) load_x16((kb8 >> 1) + 1, xb1, xb2);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const float dx = dxc[s];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sg[s][r] = kb8 == 0 ? dx * (float)cg[s][r] : fmaf(dx, (float)cg[s][r], sg[s][r]);
                    su[s][r] = kb8 == 0 ? dx * (float)cu[s][r] : fmaf(dx, (float)cu[s][r], su[s][r]);
                    asm volatile("" : "+v"(sg[s][r]), "+v"(su[s][r]));
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (LL::bf16_min) {   // the last region's min part (sub-tile 3, W3)
#pragma unroll
            for (int r = 0; r < 4; ++r) accu[3][r] = fmaf(nU[r], rmin[r], accu[3][r]);
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                accg[s][r] = fmaf(dG[r], sg[s][r], accg[s][r]);
                accu[s][r] = fmaf(dU[r], su[s][r], accu[s][r]);
            }
        }
        if constexpr (!LL::bf16_min) {
            // min part on the f32 sums: A = -dmin * m_n of this lane's row for sub-block n = 4q + g
            const float* xl = reinterpret_cast<const float*>(x16l);
            float bmg[4], bmu[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bmg[q] = -half_bits_to_f32(cw[0][8] >> 16) * (float)((cw[0][q] >> (8 * g + 4)) & 15u);
                bmu[q] = -half_bits_to_f32(cw[1][8] >> 16) * (float)((cw[1][q] >> (8 * g + 4)) & 15u);
            }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float x16 = xl[(4 * q + g) * R + 16 * s + l16];
                    accg[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(bmg[q], x16, accg[s], 0, 0, 0);
                    accu[s] = __builtin_amdgcn_mfma_f32_16x16x4f32(bmu[q], x16, accu[s], 0, 0, 0);
                }
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the exchange slots are reused next superblock
    }
    wait_vm_loads<0>();   // no load into LDS outlives the workgroup
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int t = 16 * s + l16;
        if (t < ch.nrows) {
            f4 h;
#pragma unroll
            for (int r = 0; r < 4; ++r) h[r] = swiglu(accg[s][r], accu[s][r], a.limit);
            *reinterpret_cast<f4*>(hout + (size_t)t * I + r0 + 16 * wv + 4 * g) = h;
        }
    }
}

// ------------------------------------------------------------------ Q3_K down
// W2 rows are the A operand (16 per wavefront, 64 per workgroup), the chunk's
// q8_1 rows of h the B operand: C[row][token] per q8_1 block, rescaled by the
// token's block scale, times -d of the row per superblock.
//  * Per superblock the 64 rows' blocks (eight panels: one contiguous
//    880-byte run each) and the h quants and block scales go into LDS with
//    wavefront-wide loads, the weights as [row][110 bytes], the quants
//    transposed to [16-byte chunk][token], the block scales as [8
//    blocks][token]; two superblocks are in LDS, one computed while the next is
//    in flight. As for gate/up, every sub-tile is computed (no branches in the
//    block loop).
//  * A lane (row = lane % 16, g = lane / 16) realigns once per superblock the
//    hmask bytes 8g..8g+7, the qs bytes 8g.. of both halves and the scales
//    (superblocks are 110 bytes, so half of them start at 2 bytes past a dword).
//  * B bytes: (32 - sc6) * (q3 + 4 - 4), from a 64-entry lookup of the 8 values
//    per six-bit scale (v_perm_b32 on q3 + 4); the sign goes into d.
namespace {
constexpr int DW_UNITS = TILE_ROWS * Q3K_BYTES / 16;   // 16-byte units of one superblock column (440)
constexpr int DW_LOADS = (DW_UNITS + 255) / 256;       // per thread (2)

template <int NS>
struct DownLds {
    static constexpr int R = NS * 16;
    static constexpr int ndx = (8 * R + 255) / 256;
    static constexpr int w_bytes = DW_LOADS * 256 * 16;   // [64 rows][110 B] (+ overrun)
    static constexpr int q_off = w_bytes;
    static constexpr int dx_off = q_off + 16 * R * 16;    // [8 blocks][R] f32 (+ overrun)
    static constexpr int buf_bytes = dx_off + ndx * 256 * 4;
    static constexpr int lut_off = 2 * buf_bytes;
    static constexpr int xch_off = lut_off + 64 * 8;
    __host__ __device__ static int bytes(int) { return xch_off + 4 * 16 * 4; }
};
}  // namespace

template <int NS>
__global__ __launch_bounds__(256) void mmq_down_q3k_kernel(ExpertArgs a, int nb) {
    extern __shared__ __align__(16) uint8_t smem[];
    using LL = DownLds<NS>;
    constexpr int R = LL::R;
    const int D = a.D, I = a.I;
    const int nsb = I / QK;
    const int rowbytes = nsb * Q3K_BYTES;
    const int tiles = D / TILE_ROWS;
    const int nb_act = min(nb, *a.n_chunks * tiles);   // blocks with work this call (nb: the grid's)
    const int lb = xcd_logical_block(blockIdx.x, nb_act);
    if (lb >= nb_act) return;
    const int c = lb / tiles, rt = lb % tiles;
    const Chunk ch = a.chunks[c];
    const bool shared = ch.expert < 0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int g = lane >> 4, l16 = lane & 15, gh = g >> 1;
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

    // h rows of the chunk (rows past it repeat its last row; their products are never stored)
    const int srow = max(0, min(tid & (R - 1), ch.nrows - 1));
    const int8_t* hq_row = hq + (size_t)(ch.row0 + srow) * I;
    // block-scale unit i = 256 u + tid: block i / R of h row i % R (rows past the chunk
    // repeat its last row; units past the eight blocks repeat block 7 into the overrun),
    // laid out [block][row] as for gate/up
    const float* hd_src[LL::ndx];
#pragma unroll
    for (int u = 0; u < LL::ndx; ++u) {
        const int i = u * 256 + tid;
        const int tr = max(0, min(i % R, ch.nrows - 1));
        hd_src[u] = hd + (size_t)(ch.row0 + tr) * (I / QB) + min(i / R, 7);
    }
    // weight unit f = 256 u + tid of a superblock column: panel f / 55, piece f % 55
    const uint8_t* wsrc[DW_LOADS];
#pragma unroll
    for (int u = 0; u < DW_LOADS; ++u) {
        const int f = min(256 * u + tid, DW_UNITS - 1);
        const int pp = f / (PANEL * Q3K_BYTES / 16), k = f % (PANEL * Q3K_BYTES / 16);
        wsrc[u] = w2 + (size_t)(r0 + PANEL * pp) * rowbytes + k * 16;
    }
    auto stage = [&](int sb, int bi) {
        uint8_t* buf = smem + bi * LL::buf_bytes;
#pragma unroll
        for (int u = 0; u < DW_LOADS; ++u)
            load_lds16(wsrc[u] + (size_t)sb * (PANEL * Q3K_BYTES), buf + (u * 256 + wv * 64) * 16);
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int kc = (u * 256 + tid) / R;
            load_lds16(hq_row + (size_t)sb * QK + kc * 16, buf + LL::q_off + (u * 256 + wv * 64) * 16);
        }
#pragma unroll
        for (int u = 0; u < LL::ndx; ++u)
            load_lds4(hd_src[u] + (size_t)sb * 8, buf + LL::dx_off + (u * 256 + wv * 64) * 4);
    };
    stage(0, 0);
    // lookup: entry sc6 holds (32 - sc6) * (v - 4) for v = 0..7 (bytes; lies in [-128, 124])
    uint2* lut = reinterpret_cast<uint2*>(smem + LL::lut_off);
    if (tid < 64) {
        const int sneg = 32 - tid;
        uint32_t lo = 0, hi = 0;
        for (int v = 0; v < 4; ++v) lo |= ((uint32_t)((sneg * (v - 4)) & 0xFF)) << (8 * v);
        for (int v = 4; v < 8; ++v) hi |= ((uint32_t)((sneg * (v - 4)) & 0xFF)) << (8 * (v - 4));
        lut[tid] = make_uint2(lo, hi);
    }

    typedef float f4 __attribute__((ext_vector_type(4)));
    f4 acc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = (f4){0.f, 0.f, 0.f, 0.f};
    const int wrow = 16 * wv + l16;
    float* xch = reinterpret_cast<float*>(smem + LL::xch_off) + wv * 16;

    for (int sb = 0; sb < nsb; ++sb) {
        wait_vm_loads<0>();   // superblock sb is in LDS ...
        barrier_lds();        // ... for every wave; the buffer of superblock sb - 1 is free
        const int bi = sb & 1;
        if (sb + 1 < nsb) stage(sb + 1, bi ^ 1);
        const uint8_t* buf = smem + bi * LL::buf_bytes;
        const uint32_t* lds = reinterpret_cast<const uint32_t*>(buf);
        const float* dxl = reinterpret_cast<const float*>(buf + LL::dx_off);

        const int off = wrow * Q3K_BYTES;   // 2-byte aligned
        const int A0 = off >> 2;
        const uint32_t sh = (uint32_t)(off & 3) * 8u;        // 0 or 16
        uint32_t hm[2], q0[2], q1[2];
        {
            const uint32_t h0 = lds[A0 + 2 * g], h1 = lds[A0 + 2 * g + 1], h2 = lds[A0 + 2 * g + 2];
            hm[0] = funnel(h1, h0, sh);
            hm[1] = funnel(h2, h1, sh);
            const uint32_t a0 = lds[A0 + 8 + 2 * g], a1 = lds[A0 + 9 + 2 * g], a2 = lds[A0 + 10 + 2 * g];
            q0[0] = funnel(a1, a0, sh);
            q0[1] = funnel(a2, a1, sh);
            const uint32_t b0 = lds[A0 + 16 + 2 * g], b1 = lds[A0 + 17 + 2 * g], b2 = lds[A0 + 18 + 2 * g];
            q1[0] = funnel(b1, b0, sh);
            q1[1] = funnel(b2, b1, sh);
        }
        const uint32_t t24 = lds[A0 + 24], t25 = lds[A0 + 25], t26 = lds[A0 + 26], t27 = lds[A0 + 27];
        const uint32_t S0 = funnel(t25, t24, sh), S1 = funnel(t26, t25, sh), S2 = funnel(t27, t26, sh);
        const float dneg = -half_bits_to_f32((t27 >> sh) & 0xFFFFu);

        auto load_b = [&](int kb8, int64_t* B, float* dx) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                B[s] = *reinterpret_cast<const int64_t*>(
                    buf + LL::q_off + ((2 * kb8 + gh) * R + 16 * s + l16) * 16 + 8 * (g & 1));
                dx[s] = dxl[kb8 * R + 16 * s + l16];
            }
        };
        // the lookup entry of block kb8: six-bit scale of sub-block n = 8 hh + 2 j + g / 2
        // (low nibble of byte 2j + g/2, high nibble for hh = 1; two high bits from byte
        // 8 + n % 4)
        auto load_lut = [&](int kb8) {
            const int hh = kb8 >> 2, j = kb8 & 3;
            const int nb4 = (2 * j + gh) & 3;
            const uint32_t low4 = ((j < 2 ? S0 : S1) >> (8 * nb4 + 4 * hh)) & 15u;
            const uint32_t hi2 = (S2 >> (8 * nb4 + 2 * (2 * hh + (j >> 1)))) & 3u;
            return lut[low4 | (hi2 << 4)];
        };
        f4 ss[NS];
        int64_t Bn[NS];
        float dxn[NS];
        load_b(0, Bn, dxn);
        uint2 Ln = load_lut(0);
#pragma unroll
        for (int kb8 = 0; kb8 < 8; ++kb8) {
            // one block per scheduling region, as for gate/up (the next block's B reads and
            // lookup entry issued first)
            __builtin_amdgcn_sched_barrier(0);
            const int hh = kb8 >> 2, j = kb8 & 3;
            int64_t B[NS];
            float dxc[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                B[s] = Bn[s];
                dxc[s] = dxn[s];
            }
            const uint2 L = Ln;
            if (kb8 < 7) {
                load_b(kb8 + 1, Bn, dxn);
                Ln = load_lut(kb8 + 1);
            }
            // q3 + 4 for positions 8g..8g+7 of plane j, half hh
            const uint32_t* qh = hh ? q1 : q0;
            const int hbit = 4 * hh + j;
            const uint32_t v0 = ((qh[0] >> (2 * j)) & 0x03030303u) | (((hm[0] >> hbit) & 0x01010101u) << 2);
            const uint32_t v1 = ((qh[1] >> (2 * j)) & 0x03030303u) | (((hm[1] >> hbit) & 0x01010101u) << 2);
            const int64_t Aw = (int64_t)(((uint64_t)__builtin_amdgcn_perm(L.y, L.x, v1) << 32) |
                                         __builtin_amdgcn_perm(L.y, L.x, v0));
            i32x4_t cc[NS];
#pragma unroll
            for (int s = 0; s < NS; ++s) cc[s] = mfma_i8(Aw, B[s]);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const float dx = dxc[s];
#pragma unroll
                for (int r = 0; r < 4; ++r)
                {
                    ss[s][r] = kb8 == 0 ? dx * (float)cc[s][r] : fmaf(dx, (float)cc[s][r], ss[s][r]);
                    asm volatile("" : "+v"(ss[s][r]));
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // -d of the four C rows 4g..4g+3 (held by the lanes of those rows)
        if (g == 0) xch[l16] = dneg;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const f4 dn = *reinterpret_cast<const f4*>(xch + 4 * g);
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[s][r] = fmaf(dn[r], ss[s][r], acc[s][r]);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    wait_vm_loads<0>();   // no load into LDS outlives the workgroup
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int t = 16 * s + l16;
        if (t < ch.nrows) *reinterpret_cast<f4*>(eout + (size_t)t * D + r0 + 16 * wv + 4 * g) = acc[s];
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
