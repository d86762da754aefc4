// Expert kernels of the decode path (m <= 8 tokens). Every chunk is a single
// row: one (token, pick) pair of a routed expert, or one token of a K-quant
// shared expert, with its slot, token and routing weight resolved when the
// routing made it. The arithmetic is the GEMV of the pages (GGUF Q2_K / Q3_K
// superblocks read directly against q8_1 activations; metrale moe_v41 module
// documentation; kernel table of moe_v41.rs: mmvq_q2k_experts /
// mmvq_q3k_experts for all selected experts in one launch per projection,
// swiglu_q8 for the SwiGLU and the q8_1 rows of its output in one launch,
// accumulate / finish for the weighted sum).
//
//  gateup_q8_kernel:   one workgroup = one chunk x 32 rows of the inter
//      dimension, W1 and W3, streamed as four 8-row sub-tiles through LDS;
//      the epilogue applies the clamped SwiGLU and writes the q8_1 block the
//      32 values of h form (no f32 h in memory).
//  down_combine_kernel: one workgroup = 8 rows of the output dimension for
//      every chunk. It streams the chunks' Q3_K rows and q8_1(h) records in
//      groups, accumulates G * E per token in a fixed order (the chunks'
//      order, then the shared expert's f32 output), and stores bf16.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int GU_TILE = 32;   // rows of I per gate/up workgroup: one q8_1 block of h
constexpr int GU_SUB = 8;     // rows per sub-tile
constexpr int GU_NU = 6;      // 16-byte loads into LDS per thread per sub-tile (2 * 8 * 84 * nsb bytes over 16 * nsb lanes)
constexpr int GU_MAX_THREADS = 512;
constexpr int DC_ROWS = 8;    // output rows per down workgroup
constexpr int DC_GROUP = 2;   // chunks streamed together by the down workgroup
constexpr int DC_NPF = 3;     // 16-byte loads per thread per group

// bytes of one q8_1 record of an h row: quants, then the f32 scales, then the
// 16-value sums
MOE_DEV int rec_bytes(int I) { return I + (I / QB) * 4 + (I / 16) * 4; }

}  // namespace

// ------------------------------------------------------------------ Q2_K gate/up -> q8_1(h)
// One workgroup = one chunk x 32 rows of the inter dimension (one q8_1 block
// of h), W1 and W3. The 32 rows stream through LDS as four sub-tiles of 8 rows
// of each matrix, loaded straight from global memory into LDS (no register
// staging) into two LDS slots: sub-tile i + 1 is in flight while sub-tile i is
// computed, and sub-tile i + 2 is requested as soon as slot i & 1 is free.
// Lanes: tid = 16 * s + r: superblock column s of local row r of the sub-tile
// (rows 0..7 are W1, 8..15 are W3). A lane keeps the q8_1 block data of
// superblock s of x in registers for the whole tile and does every weight of
// one (row, superblock) per sub-tile: the four 2-bit planes of each qs dword
// are masked in place (planes 1 and 3 land at 4x, folded into the activation
// block scale), and the sub-block scales and mins are applied per 16 weights.
__global__ __launch_bounds__(GU_MAX_THREADS) void gateup_q8_kernel(ExpertArgs a, int routed_rows) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int L = D / QB;
    const int nsb = D / QK;
    const int rowbytes = nsb * Q2K_BYTES;
    const int tiles = I / GU_TILE;
    const int c = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int tid = threadIdx.x, bd = blockDim.x;
    const int slot_bytes = GU_NU * bd * 16;
    const int nch = *a.n_chunks;
    if (c >= nch) return;
    const Chunk ch = a.chunks[c];
    const int token = ch.token;

    // the lane's superblock of x: 256 quants, the eight block scales and the
    // 16-value sums (requested before the weights, used once the first sub-tile is in)
    const int r = tid & 15, s = tid >> 4;
    const bool live = s < nsb;
    const int sx = live ? s : 0;
    uint32_t xv[64];
    float4 d0, d1;
    int4 s16v[4];
    {
        const uint4* xs = reinterpret_cast<const uint4*>(a.xq + (size_t)token * D + (size_t)sx * QK);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const uint4 v = xs[q];
            xv[4 * q + 0] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
        }
        const float4* dp = reinterpret_cast<const float4*>(a.xd + (size_t)token * L + (size_t)sx * 8);
        d0 = dp[0];
        d1 = dp[1];
        const int4* sp = reinterpret_cast<const int4*>(a.xs16 + (size_t)token * 2 * L + (size_t)sx * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) s16v[q] = sp[q];
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // these loads stay ahead of the sub-tile requests

    const bool shared = ch.expert < 0;
    const int r0 = tile * GU_TILE;
    const int rec = rec_bytes(I);
    uint8_t* out = a.hrec + (size_t)(shared ? routed_rows + ch.row0 : ch.row0) * rec;
    const uint8_t *w1, *w3;
    if (shared) {
        w1 = a.sh_w1;
        w3 = a.sh_w3;
    } else {
        if (ch.slot < 0) {   // not resident: flag it, and this block of h is zero
            if (tid == 0 && tile == 0) atomicOr(a.err, ERR_NOTRESIDENT);
            if (tid < GU_TILE / 4) reinterpret_cast<uint32_t*>(out + r0)[tid] = 0u;
            if (tid == 0) {
                reinterpret_cast<float*>(out + I)[tile] = 0.f;
                reinterpret_cast<int32_t*>(out + I + (I / QB) * 4)[2 * tile] = 0;
                reinterpret_cast<int32_t*>(out + I + (I / QB) * 4)[2 * tile + 1] = 0;
            }
            return;
        }
        const uint8_t* base = a.arena + (size_t)ch.slot * a.slot_bytes;
        w1 = base + a.off_w1;
        w3 = base + a.off_w3;
    }
    // Sub-tile i = W1 rows [r0 + 8 i, r0 + 8 i + 8) then the same rows of W3:
    // 2 * n16 16-byte units, unit f of thread tid's u-th load being u * bd + tid.
    // Each wave's load writes 64 consecutive units of the slot; units past the
    // end re-read the last one into the slot's padding, so every wave issues
    // exactly GU_NU loads per sub-tile (the waits below count them).
    const int n16 = GU_SUB * rowbytes / 16;
    const int wave_unit = tid & ~63;
    auto issue = [&](int i) {
        uint8_t* dst = smem + (i & 1) * slot_bytes;
        const uint8_t* g1 = w1 + (size_t)(r0 + GU_SUB * i) * rowbytes;
        const uint8_t* g3 = w3 + (size_t)(r0 + GU_SUB * i) * rowbytes;
#pragma unroll
        for (int u = 0; u < GU_NU; ++u) {
            const int f = min(u * bd + tid, 2 * n16 - 1);
            const uint8_t* src = f < n16 ? g1 + (size_t)f * 16 : g3 + (size_t)(f - n16) * 16;
            load_lds16(src, dst + (size_t)(u * bd + wave_unit) * 16);
        }
    };
    issue(0);
    issue(1);
    float dxs[8], m16[16];
    {
        const float dx[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            m16[4 * q + 0] = dx[2 * q] * (float)s16v[q].x;
            m16[4 * q + 1] = dx[2 * q] * (float)s16v[q].y;
            m16[4 * q + 2] = dx[2 * q + 1] * (float)s16v[q].z;
            m16[4 * q + 3] = dx[2 * q + 1] * (float)s16v[q].w;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) dxs[t] = (t & 1) ? 0.25f * dx[t] : dx[t];
    }

    float* red = reinterpret_cast<float*>(smem + 2 * slot_bytes);   // [4 sub-tiles][16 rows][nsb]
    for (int i = 0; i < GU_TILE / GU_SUB; ++i) {
        if (i + 1 < GU_TILE / GU_SUB) wait_vm_loads<GU_NU>();   // sub-tile i is in LDS (i + 1 may not be)
        else wait_vm_loads<0>();
        barrier_lds();
        if (live) {
            const uint32_t* wp = reinterpret_cast<const uint32_t*>(smem + (i & 1) * slot_bytes +
                                                                   panel_off(r, s, nsb, Q2K_BYTES));
            uint32_t sc[4], qw[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) sc[q] = wp[q];
#pragma unroll
            for (int q = 0; q < 16; ++q) qw[q] = wp[4 + q];
            const uint32_t dd = wp[20];
            // qs byte b of half hh holds weight 128 hh + 32 j + b in bits 2j..2j+1
            // (sub-block 8 hh + 2 j + b / 16, activation block 4 hh + j); the first
            // product of each sub-block starts its sum
            int in[16];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    const uint32_t w = qw[8 * hh + cc], w4 = w >> 4;
                    const int nb = 8 * hh + (cc >> 2);
                    const bool first = (cc & 3) == 0;
                    in[nb + 0] = sdot4(w & 0x03030303u, xv[(4 * hh + 0) * 8 + cc], first ? 0 : in[nb + 0]);
                    in[nb + 2] = sdot4(w & 0x0C0C0C0Cu, xv[(4 * hh + 1) * 8 + cc], first ? 0 : in[nb + 2]);
                    in[nb + 4] = sdot4(w4 & 0x03030303u, xv[(4 * hh + 2) * 8 + cc], first ? 0 : in[nb + 4]);
                    in[nb + 6] = sdot4(w4 & 0x0C0C0C0Cu, xv[(4 * hh + 3) * 8 + cc], first ? 0 : in[nb + 6]);
                }
            }
            // scale bytes 4q .. 4q + 3 = sub-blocks 4q .. 4q + 3 (activation blocks 2q, 2q + 1):
            // low nibbles the scales, high nibbles the mins
            float fs = 0.f, ms = 0.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t sq = sc[q] & 0x0F0F0F0Fu, mq = (sc[q] >> 4) & 0x0F0F0F0Fu;
                const int is0 = __mul24((int)(sq & 0xFFu), in[4 * q]) + __mul24((int)((sq >> 8) & 0xFFu), in[4 * q + 1]);
                const int is1 = __mul24((int)((sq >> 16) & 0xFFu), in[4 * q + 2]) + __mul24((int)(sq >> 24), in[4 * q + 3]);
                fs = fmaf(dxs[2 * q], (float)is0, fs);
                fs = fmaf(dxs[2 * q + 1], (float)is1, fs);
                ms = fmaf((float)(mq & 0xFFu), m16[4 * q], ms);
                ms = fmaf((float)((mq >> 8) & 0xFFu), m16[4 * q + 1], ms);
                ms = fmaf((float)((mq >> 16) & 0xFFu), m16[4 * q + 2], ms);
                ms = fmaf((float)(mq >> 24), m16[4 * q + 3], ms);
            }
            const float d = half_bits_to_f32(dd & 0xFFFFu), dmin = half_bits_to_f32(dd >> 16);
            red[(i * 16 + r) * nsb + s] = fmaf(d, fs, -dmin * ms);
        }
        if (i + 2 < GU_TILE / GU_SUB) {
            barrier_lds();   // every lane is done with slot i & 1
            issue(i + 2);
        }
    }
    barrier_lds();
    // row t of the tile: W1 and W3 partials of sub-tile t / 8, local rows t % 8 and 8 + t % 8;
    // then the q8_1 block of the 32 values of h across lanes 0..31
    if (tid < GU_TILE) {
        const float* rg = red + ((tid >> 3) * 16 + (tid & 7)) * nsb;
        const float* ru = rg + 8 * nsb;
        float gs = 0.f, us = 0.f;
        for (int q = 0; q < nsb; ++q) {
            gs += rg[q];
            us += ru[q];
        }
        const float h = swiglu(gs, us, a.limit);
        float amax = fabsf(h);
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 32));
        const float d = amax / 127.0f;
        const int qi = (d == 0.f) ? 0 : (int)roundf(h / d);
        reinterpret_cast<int8_t*>(out + r0)[tid] = (int8_t)qi;
        int qs = qi;
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) qs += __shfl_xor(qs, off, 16);
        if (tid == 0) reinterpret_cast<float*>(out + I)[tile] = round_to_fp16(d);
        if ((tid & 15) == 0) reinterpret_cast<int32_t*>(out + I + (I / QB) * 4)[2 * tile + (tid >> 4)] = qs;
    }
}

// ------------------------------------------------------------------ Q3_K down + combine
// Lanes: tid = pr * L + kb (L = I / 32; pr = output row of the tile, 8 rows).
// LDS: per group of DC_GROUP chunks, each chunk's 8 W2 rows then its q8_1(h)
// record; the per-row partial sums; the per-token accumulators.
__global__ __launch_bounds__(1024) void down_combine_kernel(ExpertArgs a, int routed_rows, int m, int max_chunks,
                                                            const float* __restrict__ ys, uint16_t* __restrict__ out) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int L = I / QB;
    const int nsb = I / QK;
    const int rowbytes = nsb * Q3K_BYTES;
    const int r0 = blockIdx.x * DC_ROWS;
    const int tid = threadIdx.x, bd = blockDim.x;
    const int rec = rec_bytes(I);
    const int tile_bytes = DC_ROWS * rowbytes;   // a multiple of 16 (8 * 110 * nsb)
    const int unit = tile_bytes + rec;           // LDS bytes per chunk
    const int unit16 = unit / 16, tile16 = tile_bytes / 16;

    // the chunk list (records read once, kept in LDS)
    int* c_slot = reinterpret_cast<int*>(smem + DC_GROUP * unit + 16);
    int* c_row = c_slot + max_chunks;
    int* c_tok = c_row + max_chunks;
    float* c_w = reinterpret_cast<float*>(c_tok + max_chunks);
    float* red = c_w + max_chunks;                 // [DC_GROUP][DC_ROWS][nsb]
    float* acc = red + DC_GROUP * DC_ROWS * nsb;   // [m][DC_ROWS]
    const int nch = min(*a.n_chunks, max_chunks);
    for (int q = tid; q < nch; q += bd) {
        const Chunk ch = a.chunks[q];
        const bool sh = ch.expert < 0;
        c_slot[q] = sh ? -2 : ch.slot;
        c_row[q] = sh ? routed_rows + ch.row0 : ch.row0;
        c_tok[q] = ch.token;
        c_w[q] = ch.weight;
    }
    for (int q = tid; q < m * DC_ROWS; q += bd) acc[q] = 0.f;
    __syncthreads();

    // group loads: DC_GROUP units of [tile | record]; chunks past the end repeat the last one
    uint4 pf0, pf1, pf2;   // named registers (an array here was placed in scratch memory)
    static_assert(DC_NPF == 3, "the prefetch registers below");
#define DC_LOAD_ONE(g0, u, dst)                                                                              \
    {                                                                                                        \
        const int q = min(tid + (u) * bd, DC_GROUP * unit16 - 1);                                            \
        const int cc = q / unit16, o = q % unit16;                                                           \
        const int cidx = min((g0) + cc, nch - 1);                                                            \
        const int slot = c_slot[cidx];                                                                       \
        uint4 v = make_uint4(0u, 0u, 0u, 0u);                                                                \
        if (o < tile16) {                                                                                    \
            if (slot != -1) {                                                                                \
                const uint8_t* w2 = slot == -2 ? a.sh_w2 : a.arena + (size_t)slot * a.slot_bytes + a.off_w2;  \
                v = reinterpret_cast<const uint4*>(w2 + (size_t)r0 * rowbytes)[o];                          \
            }                                                                                                \
        } else {                                                                                             \
            v = reinterpret_cast<const uint4*>(a.hrec + (size_t)c_row[cidx] * rec)[o - tile16];              \
        }                                                                                                    \
        dst = v;                                                                                             \
    }
#define DC_LOAD_GROUP(g0) { DC_LOAD_ONE(g0, 0, pf0) DC_LOAD_ONE(g0, 1, pf1) DC_LOAD_ONE(g0, 2, pf2) }
    if (nch > 0) DC_LOAD_GROUP(0)

    const int pr = tid / L, kb = tid % L;
    const bool lane_live = pr < DC_ROWS;
    const int s = kb >> 3, hh = (kb >> 2) & 1, j = kb & 3;
    // per-lane constants for the two 6-bit scales of sub-blocks n = 8hh + 2j + {0,1}
    const int n_lo = 8 * hh + 2 * j;
    const int lo_byte0 = 2 * j, lo_shift = 4 * hh;
    const int hi_byte0 = 8 + (n_lo & 3), hi_byte1 = 8 + ((n_lo + 1) & 3);
    const int hi_shift = 2 * (n_lo >> 2);
    uint4* lds16 = reinterpret_cast<uint4*>(smem);
    const uint32_t* lds32 = reinterpret_cast<const uint32_t*>(smem);
    for (int g0 = 0; g0 < nch; g0 += DC_GROUP) {
        if (g0 > 0) __syncthreads();   // the previous group's units and partials are consumed
#define DC_STORE_ONE(u, src) \
    if (tid + (u) * bd < DC_GROUP * unit16) lds16[tid + (u) * bd] = src;
        DC_STORE_ONE(0, pf0) DC_STORE_ONE(1, pf1) DC_STORE_ONE(2, pf2)
#undef DC_STORE_ONE
        __syncthreads();
        if (g0 + DC_GROUP < nch) DC_LOAD_GROUP(g0 + DC_GROUP)
        const int ng = min(DC_GROUP, nch - g0);
        if (lane_live) {
            for (int cc = 0; cc < ng; ++cc) {
                const int ubase = cc * unit;
                const uint32_t* hq32 = lds32 + (ubase + tile_bytes) / 4;
                // the lane's q8_1 block of h: two 16-byte reads (dword reads at a
                // 32-byte lane stride conflicted on the LDS banks)
                const uint4 h0 = reinterpret_cast<const uint4*>(hq32)[2 * kb];
                const uint4 h1 = reinterpret_cast<const uint4*>(hq32)[2 * kb + 1];
                const uint32_t av[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
                const float dx = reinterpret_cast<const float*>(hq32 + I / 4)[kb];
                const int2 hs = reinterpret_cast<const int2*>(hq32 + I / 4 + L)[kb];
                const int slo = hs.x, shi = hs.y;
                const int sb = ubase + panel_off(pr, s, nsb, Q3K_BYTES);   // 2-byte aligned
                const int A = sb >> 2;
                const uint32_t sh = (uint32_t)(sb & 3) * 8u;              // 0 or 16
                uint32_t V[8];
                {
                    const int qo = A + 8 + 8 * hh;                           // qs[32 hh ..] at byte 32 + 32 hh
                    uint32_t prev = lds32[qo];
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const uint32_t next = lds32[qo + q + 1];
                        const uint32_t qs = funnel(next, prev, sh);
                        const uint32_t hm = funnel(lds32[A + q + 1], lds32[A + q], sh);
                        prev = next;
                        const uint32_t lo = (qs >> (2 * j)) & 0x03030303u;
                        const uint32_t hb = (hm >> (4 * hh + j)) & 0x01010101u;
                        V[q] = lo | (hb << 2);                               // q3 + 4, 0..7
                    }
                }
                const uint32_t s0 = funnel(lds32[A + 25], lds32[A + 24], sh);   // scale bytes 0..3
                const uint32_t s1 = funnel(lds32[A + 26], lds32[A + 25], sh);   // 4..7
                const uint32_t s2 = funnel(lds32[A + 27], lds32[A + 26], sh);   // 8..11
                const uint32_t dbits = (lds32[A + 27] >> sh) & 0xFFFFu;          // d at byte 108
                const uint32_t lo_word = (lo_byte0 < 4) ? s0 : s1;
                const int lsh = 8 * (lo_byte0 & 3);
                const int low4_lo = (lo_word >> (lsh + lo_shift)) & 15;
                const int low4_hi = (lo_word >> (lsh + 8 + lo_shift)) & 15;
                const int hi2_lo = (s2 >> (8 * (hi_byte0 - 8) + hi_shift)) & 3;
                const int hi2_hi = (s2 >> (8 * (hi_byte1 - 8) + hi_shift)) & 3;
                const int s6_lo = (low4_lo | (hi2_lo << 4)) - 32;
                const int s6_hi = (low4_hi | (hi2_hi << 4)) - 32;
                const float d = half_bits_to_f32(dbits);
                int il = 0, ih = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q) il = sdot4(V[q], av[q], il);
#pragma unroll
                for (int q = 4; q < 8; ++q) ih = sdot4(V[q], av[q], ih);
                il -= 4 * slo;
                ih -= 4 * shi;
                float part = dx * (d * (float)(__mul24(s6_lo, il) + __mul24(s6_hi, ih)));
                part = group8_sum(part);
                if ((kb & 7) == 7) red[(cc * DC_ROWS + pr) * nsb + s] = part;
            }
        }
        __syncthreads();
        if (tid < DC_ROWS) {   // row tid: this group's chunks in order
            for (int cc = 0; cc < ng; ++cc) {
                const float* re = red + (cc * DC_ROWS + tid) * nsb;
                float e = 0.f;
                for (int q = 0; q < nsb; ++q) e += re[q];
                const int c = g0 + cc;
                acc[c_tok[c] * DC_ROWS + tid] += c_slot[c] == -1 ? 0.f : c_w[c] * e;
            }
        }
    }
#undef DC_LOAD_GROUP
#undef DC_LOAD_ONE
    __syncthreads();
    for (int q = tid; q < m * DC_ROWS; q += bd) {
        const int t = q / DC_ROWS, r = q % DC_ROWS;
        float v = acc[q];
        if (ys != nullptr) v += ys[(size_t)t * D + r0 + r];
        out[(size_t)t * D + r0 + r] = (uint16_t)f32_to_bf16(v);
    }
}

// ------------------------------------------------------------------ launch
bool decode_supported(int D, int I) {
    // lanes: 16 per superblock of D for gate/up and 8 * I / 32 for down, within one workgroup
    return D % QK == 0 && I % QK == 0 && 16 * (D / QK) <= GU_MAX_THREADS && I / 4 <= 1024 && D % DC_ROWS == 0;
}

static int round64(int v) { return (v + 63) / 64 * 64; }

size_t decode_rec_bytes(int I) { return (size_t)I + (size_t)(I / QB) * 4 + (size_t)(I / 16) * 4; }

hipError_t launch_gateup_q8(const ExpertArgs& a, int routed_rows, int max_chunks, hipStream_t st) {
    if (max_chunks <= 0) return hipSuccess;
    const int nsb = a.D / QK;
    const int threads = round64(16 * nsb);
    const size_t lds = (size_t)2 * GU_NU * threads * 16 + (size_t)(GU_TILE / GU_SUB) * 16 * nsb * 4;
    return launch_kernel(gateup_q8_kernel, max_chunks * (a.I / GU_TILE), threads, lds, st, a, routed_rows);
}

hipError_t launch_down_combine(const ExpertArgs& a, int routed_rows, int m, int max_chunks, const float* ys,
                               uint16_t* out, hipStream_t st) {
    const int threads = round64(DC_ROWS * (a.I / QB));
    const int nsb = a.I / QK;
    const size_t unit = (size_t)DC_ROWS * nsb * Q3K_BYTES + decode_rec_bytes(a.I);
    const size_t lds = DC_GROUP * unit + 16 + (size_t)max_chunks * 16 + (size_t)DC_GROUP * DC_ROWS * nsb * 4 +
                       (size_t)m * DC_ROWS * 4;
    return launch_kernel(down_combine_kernel, a.D / DC_ROWS, threads, lds, st, a, routed_rows, m, max_chunks, ys, out);
}

}  // namespace moe
