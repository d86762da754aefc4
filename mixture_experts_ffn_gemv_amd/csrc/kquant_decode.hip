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
//      dimension (four 8-row panels), W1 and W3, every block loaded straight
//      into registers at the start; the epilogue applies the clamped SwiGLU and
//      writes the q8_1 block the 32 values of h form (no f32 h in memory).
//  down_combine_kernel: one workgroup = 8 rows of the output dimension for
//      one token's chunks (its picks, then its row of a K-quant shared expert).
//      It loads their q8_1(h) records into LDS and each lane's Q3_K block into
//      registers, accumulates G * E in a fixed order (the chunks' order, then
//      the bf16 shared expert's ys), and stores bf16.
#include <algorithm>

#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int GU_TILE = 32;   // rows of I per gate/up workgroup: one q8_1 block of h (four panels)
constexpr int DC_ROWS = 8;    // output rows per down workgroup: one panel

// bytes of one q8_1 record of an h row: quants, then the f32 scales, then the
// 16-value sums
MOE_DEV int rec_bytes(int I) { return I + (I / QB) * 4 + (I / 16) * 4; }

// a lane's value from another lane of its 16-lane row (DPP control CTRL)
template <int CTRL>
MOE_DEV int dpp16(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}


}  // namespace

// ------------------------------------------------------------------ Q2_K gate/up -> q8_1(h)
// One workgroup = one chunk x 32 rows of the inter dimension (four 8-row
// panels: one q8_1 block of h), W1 and W3. Lanes: tid = r + 8 (sl + NSL (m + 2 p)):
// row r of panel p of matrix m (0 = W1, 1 = W3), superblocks s = sl + NSL k,
// k < SPL. A lane loads its SPL 84-byte blocks straight from global memory into
// registers at the start: the 8 rows of a superblock column are one contiguous
// run, so each wavefront load covers whole runs (5 KB contiguous), and every
// weight of the tile is requested at once. The token's q8_1 activations come
// into LDS by the DMA path. Per block the four 2-bit planes of each qs dword
// are masked in place (planes 1 and 3 land at 4x, folded into the activation
// block scale) and the sub-block scales and mins applied per 16 weights; the
// per-row sums over the superblocks run in order, then the clamped SwiGLU and
// the q8_1 block of the 32 values of h across 32 lanes. Workgroups past the
// routed tiles (routed_blocks) compute rows of a bf16 shared expert's down
// product instead.
template <int SPL>
__global__ __launch_bounds__(1024) void gateup_q8_kernel(ExpertArgs a, int routed_rows, int routed_blocks,
                                                         SharedRows sr) {
    if ((int)blockIdx.x >= routed_blocks) {   // bf16 shared-expert down rows riding in this launch (5 pieces: <= 80 VGPRs)
        shared_down_block<5>(sr, blockIdx.x - routed_blocks);
        return;
    }
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int L = D / QB;
    const int nsb = D / QK;
    const int NSL = (nsb + SPL - 1) / SPL;
    const int rowbytes = nsb * Q2K_BYTES;
    const int tiles = I / GU_TILE;
    const int c = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int tid = threadIdx.x, bd = blockDim.x, wv = tid >> 6;
    // the chunk (in bounds: the grid covers the list's capacity) and the count,
    // requested together (the test reads both, so neither load waits for the other)
    const Chunk ch = a.chunks[c];
    const int nch = *a.n_chunks;
    if ((c >= nch) | (ch.nrows <= 0)) return;
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
                reinterpret_cast<int2*>(out + I + (I / QB) * 4)[tile] = make_int2(0, 0);
            }
            return;
        }
        const uint8_t* base = a.arena + (size_t)ch.slot * a.slot_bytes;
        w1 = base + a.off_w1;
        w3 = base + a.off_w3;
    }
    // the token's q8_1 activations: quants (D bytes), block scales (L f32),
    // fp16(d) times the 16-value sums (2L f32), requested first, through registers
    // into LDS. Each superblock's 256 quants are followed by 16 bytes of padding
    // (unit f at f + min(f / 16, nsb)): the lanes of a wavefront read 8 different
    // superblocks at once, 272 bytes apart, which falls on distinct banks where a
    // 256-byte stride would not.
    const int nx16 = (D + 4 * L + 8 * L) / 16;
    const int nxu = (nx16 + bd - 1) / bd;
    uint4 xv0 = make_uint4(0, 0, 0, 0);
    {
        const uint8_t* xq = reinterpret_cast<const uint8_t*>(a.xq + (size_t)ch.token * D);
        const uint8_t* xd = reinterpret_cast<const uint8_t*>(a.xd + (size_t)ch.token * L);
        const uint8_t* xs = reinterpret_cast<const uint8_t*>(a.xs16f + (size_t)ch.token * 2 * L);
        for (int u = 0; u < nxu; ++u) {
            const int f = u * bd + tid;
            if (f < nx16) {
                const uint8_t* src = f < D / 16 ? xq + (size_t)f * 16
                                   : f < D / 16 + L / 4 ? xd + (size_t)(f - D / 16) * 16
                                                        : xs + (size_t)(f - D / 16 - L / 4) * 16;
                const uint4 v = *reinterpret_cast<const uint4*>(src);
                if (u == 0) xv0 = v;   // stored after the weight loads are issued
                else reinterpret_cast<uint4*>(smem)[f + min(f >> 4, nsb)] = v;
            }
        }
    }
    // this lane's blocks, straight into registers (the waits for them are the
    // compiler's, placed at their first use, so the first block is computed
    // while the later ones arrive)
    const int r = tid & 7, rest = tid >> 3, sl = rest % NSL, mp = rest / NSL;
    const int m = mp & 1, p = mp >> 1;
    const bool live = p < GU_TILE / PANEL;
    uint32_t wq[SPL][21];
    {
        const uint8_t* panel = (m ? w3 : w1) + (size_t)(r0 + PANEL * (live ? p : 0)) * rowbytes;
#pragma unroll
        for (int k = 0; k < SPL; ++k) {
            const int s = min(sl + NSL * k, nsb - 1);
            const uint32_t* q = reinterpret_cast<const uint32_t*>(panel + (size_t)(s * PANEL + r) * Q2K_BYTES);
#pragma unroll
            for (int i = 0; i < 21; ++i) wq[k][i] = q[i];
        }
    }
    if (tid < nx16) reinterpret_cast<uint4*>(smem)[tid + min(tid >> 4, nsb)] = xv0;
    barrier_lds();

    const uint8_t* xl = smem;
    const uint8_t* xsc = xl + D + 16 * nsb;   // the block scales, then the 16-value terms
    float* red = reinterpret_cast<float*>(smem + (size_t)((nx16 + nsb + bd - 1) / bd) * bd * 16);   // [8 vectors x 4 panels... ][nsb]
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
        const int s = sl + NSL * k;
        if (!live || s >= nsb) continue;
        const uint32_t* sc = wq[k];
        const uint32_t* qw = wq[k] + 4;
        const uint32_t dd = wq[k][20];
        const uint32_t* xq32 = reinterpret_cast<const uint32_t*>(xl) + s * (QK / 4 + 4);
        const float* dxp = reinterpret_cast<const float*>(xsc) + s * 8;
        const float* s16p = reinterpret_cast<const float*>(xsc + 4 * L) + s * 16;
        float fs = 0.f, ms = 0.f;
        // q8_1 block t = 4 hh + j of x meets plane j of qs half hh: qs byte b of half
        // hh holds weight 128 hh + 32 j + b in bits 2j..2j+1 (sub-block 2t + b / 16)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int hh = t >> 2, j = t & 3;
            const uint4 x0 = reinterpret_cast<const uint4*>(xq32 + 8 * t)[0];
            const uint4 x1 = reinterpret_cast<const uint4*>(xq32 + 8 * t)[1];
            const uint32_t xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            int il = 0, ih = 0;
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                const uint32_t w = qw[8 * hh + cc];
                const uint32_t pl = j == 0 ? (w & 0x03030303u) : j == 1 ? (w & 0x0C0C0C0Cu)
                                  : j == 2 ? ((w >> 4) & 0x03030303u) : ((w >> 4) & 0x0C0C0C0Cu);
                if (cc < 4) il = sdot4(pl, xv[cc], il);
                else ih = sdot4(pl, xv[cc], ih);
            }
            const uint32_t sw = sc[t >> 1] >> (16 * (t & 1));   // scale bytes 2t, 2t + 1
            const int isum = __mul24((int)(sw & 15u), il) + __mul24((int)((sw >> 8) & 15u), ih);
            const float dx = dxp[t];
            const float2 s16 = reinterpret_cast<const float2*>(s16p)[t];   // fp16(d) * sum per 16
            fs = fmaf((j & 1) ? 0.25f * dx : dx, (float)isum, fs);
            ms = fmaf((float)((sw >> 4) & 15u), s16.x, ms);
            ms = fmaf((float)((sw >> 12) & 15u), s16.y, ms);
        }
        const float d = half_bits_to_f32(dd & 0xFFFFu), dmin = half_bits_to_f32(dd >> 16);
        red[((p * 2 + m) * PANEL + r) * nsb + s] = fmaf(d, fs, -dmin * ms);
    }
    barrier_lds();
    // row t of the tile (panel t / 8, row t % 8): the W1 and W3 sums, the clamped
    // SwiGLU, then the q8_1 block of the 32 values across lanes 0..31
    if (tid < GU_TILE) {
        const int pp = tid >> 3, rr = tid & 7;
        const float* rg = red + ((pp * 2 + 0) * PANEL + rr) * nsb;
        const float* ru = red + ((pp * 2 + 1) * PANEL + rr) * nsb;
        float gs = 0.f, us = 0.f;
        for (int q = 0; q < nsb; ++q) {
            gs += rg[q];
            us += ru[q];
        }
        const float h = swiglu(gs, us, a.limit);
        // the block's amax across the 32 lanes: within each 16 by DPP, then across the two
        float amax = fabsf(h);
        amax = fmaxf(amax, __int_as_float(dpp16<0xB1>(__float_as_int(amax))));    // quad_perm [1,0,3,2]
        amax = fmaxf(amax, __int_as_float(dpp16<0x4E>(__float_as_int(amax))));    // quad_perm [2,3,0,1]
        amax = fmaxf(amax, __int_as_float(dpp16<0x124>(__float_as_int(amax))));   // row_ror:4
        amax = fmaxf(amax, __int_as_float(dpp16<0x128>(__float_as_int(amax))));   // row_ror:8
        amax = fmaxf(amax, __shfl_xor(amax, 16, 32));
        const float d = amax / 127.0f;
        const int qi = (d == 0.f) ? 0 : (int)roundf(h / d);
        reinterpret_cast<int8_t*>(out + r0)[tid] = (int8_t)qi;
        int qs = qi;   // the 16-value sums, by DPP within each 16
        qs += dpp16<0xB1>(qs);
        qs += dpp16<0x4E>(qs);
        qs += dpp16<0x124>(qs);
        qs += dpp16<0x128>(qs);
        if (tid == 0) reinterpret_cast<float*>(out + I)[tile] = round_to_fp16(d);
        if ((tid & 15) == 0) reinterpret_cast<int32_t*>(out + I + (I / QB) * 4)[2 * tile + (tid >> 4)] = qs;
    }
    (void)wv;
}

// ------------------------------------------------------------------ Q3_K down + combine
// v + the weighted E of a pass's ng chunks g0.. that belong to token tsel and are
// resident, in chunk order (e: this row's E of chunk q at e[q * DC_ROWS]). Up to 8
// chunks every LDS read is requested before the first product.
MOE_DEV float combine_pass(float v, int g0, int ng, int tsel, const int* c_tok, const int* c_slot, const float* c_w,
                           const float* e) {
    if (ng <= 8) {
        bool use[8];
        float w[8], ev[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int c = g0 + min(q, ng - 1);
            use[q] = (q < ng) & (c_tok[c] == tsel) & (c_slot[c] != -1);   // no short circuit: reads batched
            w[q] = c_w[c];
            ev[q] = e[min(q, ng - 1) * DC_ROWS];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (use[q]) v = fmaf(w[q], ev[q], v);
        return v;
    }
    for (int q = 0; q < ng; ++q) {
        const int c = g0 + q;
        if (c_tok[c] == tsel && c_slot[c] != -1) v = fmaf(c_w[c], e[q * DC_ROWS], v);
    }
    return v;
}

// One workgroup = one panel of 8 output rows for one token (workgroup b: token
// b / (D / 8), panel b % (D / 8)); its chunks are the token's k picks (at m = 1
// every chunk in list order, else the positions inv[] gives, in pick order) and
// then its K-quant shared-expert row; a pass takes G of them at once. Lanes: tid = r + 8 (s + nsb cl): row r of the panel,
// superblock s, chunk cl of the pass. A lane loads its 110-byte block straight
// from global memory into registers (the 8 rows of a superblock column are one
// contiguous run, so a wavefront reads whole runs), realigns it (blocks start
// on 2-byte boundaries) and dots all 256 weights against the chunk's q8_1 h,
// whose records the pass loads into LDS. The per-(row, chunk) sums over the
// superblocks and the weighted sum over the chunks of each token run in a
// fixed order (chunks in list order, then the shared expert's f32 output ys,
// when given).
template <bool TOK>   // TOK: m > 1, a workgroup per (token, panel); else the one token's chunks in list order
__global__ __launch_bounds__(1024) void down_combine_kernel(ExpertArgs a, int routed_rows, int m, int max_chunks,
                                                            int G, const float* __restrict__ ys,
                                                            uint16_t* __restrict__ out) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int nsb = I / QK;
    const int rowbytes = nsb * Q3K_BYTES;
    const int panels = D / DC_ROWS;
    const int tsel = TOK ? blockIdx.x / panels : 0;
    const int r0 = (TOK ? blockIdx.x % panels : blockIdx.x) * DC_ROWS;
    const int tid = threadIdx.x, bd = blockDim.x;
    const int rec = rec_bytes(I);
    const int rec16 = rec / 16;                          // a multiple of 16 bytes (I a multiple of 256)
    const int nu = (G * rec16 + bd - 1) / bd;            // record loads per thread and pass
    constexpr int NR = 3;   // record units per thread held in registers; further ones load synchronously
    uint8_t* hrec = smem;                                // [G][rec] (+ the last loads' overrun), >= NR bd units
    int* c_slot = reinterpret_cast<int*>(smem + (size_t)max(nu, NR) * bd * 16);
    int* c_row = c_slot + max_chunks;
    int* c_tok = c_row + max_chunks;
    float* c_w = reinterpret_cast<float*>(c_tok + max_chunks);
    const int pst = (nsb + 3) & ~3;                      // partials per (chunk, row), padded to 16 bytes
    float* part = c_w + max_chunks;                      // [G][8][pst] (16-byte aligned: 4 arrays of max_chunks words)
    float* acc = part + G * DC_ROWS * pst;               // [8]
    float* esum = acc + DC_ROWS;                         // [G][8]
    const int k = a.topk;
    // this workgroup's chunks into LDS: one token's are the list's first entries
    // (max_chunks <= blockDim), staged whatever their count, which is requested
    // alongside (entries past it are never read)
    const int nch = TOK ? min(k + (a.sh_w2 != nullptr ? 1 : 0), max_chunks) : min(*a.n_chunks, max_chunks);
    for (int q = tid; q < (TOK ? nch : max_chunks); q += bd) {
        const int ci = !TOK ? q : q < k ? a.inv[tsel * k + q] : routed_rows + tsel;
        const Chunk ch = a.chunks[ci];
        const bool sh = ch.expert < 0;
        c_slot[q] = sh ? -2 : ch.slot;
        c_row[q] = sh ? routed_rows + ch.row0 : ch.row0;
        c_tok[q] = ch.token;
        c_w[q] = ch.weight;
    }
    for (int q = tid; q < DC_ROWS; q += bd) acc[q] = 0.f;
    // the shared expert's output for this workgroup's rows, requested now (it is added last)
    const float ysv = (ys != nullptr && tid < DC_ROWS) ? ys[(size_t)tsel * D + r0 + tid] : 0.f;
    // with every (chunk, row) of a pass in one wavefront, wavefront 0 finishes each pass
    // (lanes 0..7 carry the rows' sums across passes)
    const bool wave_sum = G * DC_ROWS <= 64;
    float accv = 0.f;
    // the chunk entries in LDS for every wavefront; the ys load stays in flight (a full
    // workgroup barrier would wait for it, behind the other workgroups' weight loads)
    barrier_lds();

    const int r = tid & 7, sc = tid >> 3, s = sc % nsb, cl = sc / nsb;
    const uint32_t* h32 = reinterpret_cast<const uint32_t*>(hrec) + (size_t)cl * (rec / 4);
    for (int g0 = 0; g0 < nch; g0 += G) {
        const int ng = min(G, nch - g0);
        // this pass's q8_1(h) records (units past the end repeat the last one), then this
        // lane's block, 28 dwords from the dword below its start (in bounds: a block that
        // starts on a dword ends 2 bytes before the next block of its column run), in
        // straight-line code (a lane without a block reads slot 0's). The records go into
        // LDS through registers before the block is requested: requested behind the
        // other workgroups' weight loads they arrive microseconds later than on their own.
        // The waits are exact, so a lane computes its block as soon as it has arrived.
        // Record units past NR per thread (other shapes) are staged first, synchronously.
        auto rec_unit = [&](int u) {
            const int f = min(u * bd + tid, ng * rec16 - 1);
            const int q = f / rec16, k = f % rec16;
            return reinterpret_cast<const uint4*>(a.hrec + (size_t)c_row[g0 + q] * rec + k * 16);
        };
        for (int u = NR; u < nu; ++u) reinterpret_cast<uint4*>(hrec)[u * bd + tid] = *rec_unit(u);
        uint4 R[NR];
#pragma unroll
        for (int u = 0; u < NR; ++u) R[u] = *rec_unit(u);
        const bool act = cl < ng;
        const int slot = act ? c_slot[g0 + cl] : -1;
        const uint8_t* w2 = slot == -2 ? a.sh_w2 : a.arena + (size_t)max(slot, 0) * a.slot_bytes + a.off_w2;
        const uint8_t* blk = w2 + (size_t)r0 * rowbytes + (size_t)(s * DC_ROWS + r) * Q3K_BYTES;
        const uint32_t mis = (uint32_t)((uintptr_t)blk & 3);
        const uint32_t sh = mis * 8u;
        const uint32_t* wp = reinterpret_cast<const uint32_t*>(blk - mis);   // pointer arithmetic keeps it global
#pragma unroll
        for (int u = 0; u < NR; ++u) reinterpret_cast<uint4*>(hrec)[u * bd + tid] = R[u];
        __atomic_signal_fence(__ATOMIC_SEQ_CST);   // the block's loads stay behind the records' stores
        uint32_t W[28];
#pragma unroll
        for (int q = 0; q < 28; ++q) W[q] = wp[q];
        barrier_lds();
        if (slot != -1) {
            // realigned block: hmask dwords 0..7, qs 8..23, scales 24..26, d in 27
            uint32_t B[28];
#pragma unroll
            for (int q = 0; q < 27; ++q) B[q] = funnel(W[q + 1], W[q], sh);
            B[27] = W[27] >> sh;
            const uint32_t* hq = h32 + s * (QK / 4);
            const float* hd = reinterpret_cast<const float*>(h32 + I / 4) + s * 8;
            const int* hs = reinterpret_cast<const int*>(h32 + I / 4 + I / QB) + s * 16;
            float fs = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {   // q8_1 block t of h: plane j = t % 4 of half hh = t / 4
                const int hh = t >> 2, j = t & 3;
                const uint4 x0 = reinterpret_cast<const uint4*>(hq + 8 * t)[0];
                const uint4 x1 = reinterpret_cast<const uint4*>(hq + 8 * t)[1];
                const uint32_t xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                int il = 0, ih = 0;
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    // q3 + 4 = low two bits | high bit << 2, for 4 weights (the hmask bit
                    // of plane 4 hh + j shifted straight to bit 2 of each byte)
                    const int hs = 4 * hh + j - 2;
                    const uint32_t hb = (hs >= 0 ? B[cc] >> hs : B[cc] << -hs) & 0x04040404u;
                    const uint32_t v = ((B[8 + 8 * hh + cc] >> (2 * j)) & 0x03030303u) | hb;
                    if (cc < 4) il = sdot4(v, xv[cc], il);
                    else ih = sdot4(v, xv[cc], ih);
                }
                const int2 s16 = reinterpret_cast<const int2*>(hs)[t];
                il -= 4 * s16.x;
                ih -= 4 * s16.y;
                // six-bit scales of sub-blocks n = 2t, 2t + 1: low nibble of byte n % 8
                // (high nibble for n >= 8), two high bits of byte 8 + n % 4 at 2 (n / 4)
                const int n0 = 2 * t, n1 = 2 * t + 1;
                const int lo0 = (B[24 + ((n0 & 7) >> 2)] >> (8 * (n0 & 3) + 4 * hh)) & 15;
                const int lo1 = (B[24 + ((n1 & 7) >> 2)] >> (8 * (n1 & 3) + 4 * hh)) & 15;
                const int hi0 = (B[26] >> (8 * (n0 & 3) + 2 * (n0 >> 2))) & 3;
                const int hi1 = (B[26] >> (8 * (n1 & 3) + 2 * (n1 >> 2))) & 3;
                const int isum = __mul24((lo0 | (hi0 << 4)) - 32, il) + __mul24((lo1 | (hi1 << 4)) - 32, ih);
                fs = fmaf(hd[t], (float)isum, fs);
            }
            part[(cl * DC_ROWS + r) * pst + s] = half_bits_to_f32(B[27] & 0xFFFFu) * fs;
        }
        barrier_lds();
        // E of (chunk q / 8, row q % 8): its superblock partials in order, read 16 bytes at a
        // time (up to 16 partials every read requested before the first add)
        auto e_of = [&](int q) {
            const float4* pe = reinterpret_cast<const float4*>(part + q * pst);
            const int n4 = pst / 4;
            float e = 0.f;
            auto add4 = [&](const float4& v, int k4) {
                e += v.x;   // 4 k4 < nsb for every k4 < n4
                if (4 * k4 + 1 < nsb) e += v.y;
                if (4 * k4 + 2 < nsb) e += v.z;
                if (4 * k4 + 3 < nsb) e += v.w;
            };
            if (n4 <= 4) {
                float4 v[4];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4) v[k4] = pe[min(k4, n4 - 1)];
#pragma unroll
                for (int k4 = 0; k4 < 4; ++k4)
                    if (k4 < n4) add4(v[k4], k4);
            } else {
                for (int k4 = 0; k4 < n4; ++k4) add4(pe[k4], k4);
            }
            return e;
        };
        if (wave_sum) {
            if (tid < 64) {
                // lane q: E of (chunk q / 8, row q % 8) into LDS; then row q % 8 (lanes 0..7) takes
                // this pass's chunks of the token in order, from LDS (one wavefront: its LDS
                // writes come before its reads)
                if (tid < ng * DC_ROWS) esum[tid] = e_of(tid);
                __builtin_amdgcn_wave_barrier();
                if (tid < DC_ROWS) accv = combine_pass(accv, g0, ng, tsel, c_tok, c_slot, c_w, esum + tid);
            }
        } else {
            // E of each (chunk, row): its superblock partials in order
            for (int q = tid; q < ng * DC_ROWS; q += bd) esum[q] = e_of(q);
            barrier_lds();
            if (tid < DC_ROWS)   // row tid: this pass's chunks of the token in order
                acc[tid] = combine_pass(acc[tid], g0, ng, tsel, c_tok, c_slot, c_w, esum + tid);
        }
        if (g0 + G < nch) barrier_lds();   // the records and partials are reused by the next pass
    }
    if (tid < DC_ROWS) {
        float v = wave_sum ? accv : acc[tid];
        if (ys != nullptr) v += ysv;
        out[(size_t)tsel * D + r0 + tid] = (uint16_t)f32_to_bf16(v);
    }
}

// ------------------------------------------------------------------ launch
bool decode_supported(int D, int I) {
    // lanes: 64 per superblock slot of D (at most two superblocks per lane) for gate/up,
    // 8 per superblock of I for down, within one workgroup
    return D % QK == 0 && I % QK == 0 && 32 * (D / QK) <= 1024 && DC_ROWS * (I / QK) <= 1024 && D % DC_ROWS == 0;
}

static int round64(int v) { return (v + 63) / 64 * 64; }

size_t decode_rec_bytes(int I) { return (size_t)I + (size_t)(I / QB) * 4 + (size_t)(I / 16) * 4; }

hipError_t launch_gateup_q8(const ExpertArgs& a, int routed_rows, int max_chunks, hipStream_t st,
                            const SharedRows* sr) {
    if (max_chunks <= 0) return hipSuccess;
    const int nsb = a.D / QK;
    const int spl = 64 * nsb <= 1024 ? 1 : 2;                 // superblocks per lane
    const int threads = round64(64 * ((nsb + spl - 1) / spl));  // 8 rows x slots x 2 matrices x 4 panels
    const int nx16 = (a.D + 12 * (a.D / QB)) / 16 + nsb;   // with one padding unit per superblock
    const size_t lds = (size_t)((nx16 + threads - 1) / threads) * threads * 16 + (size_t)64 * nsb * 4;
    const int grid = max_chunks * (a.I / GU_TILE);
    SharedRows none{};
    const SharedRows& s = sr ? *sr : none;
    const int nsh = sr ? shared_rows_blocks(*sr, threads) : 0;
    if (spl == 1) return launch_kernel(gateup_q8_kernel<1>, grid + nsh, threads, lds, st, a, routed_rows, grid, s);
    return launch_kernel(gateup_q8_kernel<2>, grid + nsh, threads, lds, st, a, routed_rows, grid, s);
}

hipError_t launch_down_combine(const ExpertArgs& a, int routed_rows, int m, int max_chunks, const float* ys,
                               uint16_t* out, hipStream_t st) {
    const int nsb = a.I / QK;
    const int lanes = DC_ROWS * nsb;                      // per chunk
    const int per_tok = std::min(max_chunks, a.topk + (a.sh_w2 != nullptr ? 1 : 0));
    const int G = std::max(1, std::min(per_tok, 1024 / lanes));
    const int threads = round64(lanes * G);
    const int rec16 = (int)(decode_rec_bytes(a.I) / 16);
    const int nu = (G * rec16 + threads - 1) / threads;
    const int pst = (nsb + 3) & ~3;
    const size_t lds = (size_t)std::max(nu, 3) * threads * 16 + (size_t)per_tok * 16 + (size_t)G * DC_ROWS * pst * 4 +
                       (size_t)DC_ROWS * 4 + (size_t)G * DC_ROWS * 4;
    if (m == 1)
        return launch_kernel(down_combine_kernel<false>, a.D / DC_ROWS, threads, lds, st, a, routed_rows, m, per_tok,
                             G, ys, out);
    return launch_kernel(down_combine_kernel<true>, (a.D / DC_ROWS) * m, threads, lds, st, a, routed_rows, m, per_tok,
                         G, ys, out);
}

}  // namespace moe
