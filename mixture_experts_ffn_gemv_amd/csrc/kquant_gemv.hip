// Expert GEMVs over K-quant blocks for chunks of at most 8 token rows:
//   gate/up: g = W1 q8_1(x), u = W3 q8_1(x) with Q2_K W1/W3, clamped SwiGLU
//            epilogue -> h (f32);
//   down:    E = W2 q8_1(h) with Q3_K W2 (q8_1(h) is formed in the prologue).
// Block formats: GGUF Q2_K (84 B) and Q3_K (110 B) superblocks, read as raw
// bytes. The pages describe this as GEMVs for groups of up to eight rows on
// the still-quantised blocks with q8_1 activations (metrale moe_v41 module
// documentation; kernel table of moe_v41.rs: mmvq_q2k / mmvq_q3k).
//
// Layout of the work (gfx950, wave64):
//  * one workgroup = one chunk x one tile of R weight rows; the tile's raw
//    blocks are copied HBM -> LDS with coalesced 16-byte loads;
//  * every lane owns one fixed 32-value q8_1 block of the K dimension (so its
//    activation quants stay in registers for all rows of the tile) and
//    computes its partial dot product for each row with v_dot4_i32_i8;
//  * the 8 lanes of a superblock are reduced with lane shuffles, the
//    superblocks of a row through LDS in a fixed order (deterministic).
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

// token rows of a chunk
struct ChunkRows {
    int tok[GEMV_ROWS];
    int nrows;
    bool shared;
};

MOE_DEV ChunkRows chunk_rows(const ExpertArgs& a, const Chunk& ch) {
    ChunkRows cr;
    cr.nrows = ch.nrows;
    cr.shared = ch.expert < 0;
#pragma unroll
    for (int i = 0; i < GEMV_ROWS; ++i) {
        int t = -1;
        if (i < ch.nrows) t = cr.shared ? ch.row0 + i : a.perm[ch.row0 + i] / a.topk;
        cr.tok[i] = t;
    }
    return cr;
}

// Copy chunks [0, n) of a then [0, n) of b (16 B each) to dst, which is 2n
// chunks long, with up to eight loads in flight per thread before the LDS
// writes. Named registers, not an array: an array here was placed in scratch
// memory. Indices past the end are clamped to the last chunk, which is then
// written several times with the same bytes.
MOE_DEV void stage_two(uint4* dst, const uint4* a, const uint4* b, int n, int tid, int bd) {
    const int total = (a == b) ? n : 2 * n;
    auto src = [&](int q) { return q < n ? a[q] : b[q - n]; };
    for (int q0 = tid; q0 < total; q0 += 8 * bd) {
        const int q1 = min(q0 + bd, total - 1), q2 = min(q0 + 2 * bd, total - 1);
        const int q3 = min(q0 + 3 * bd, total - 1), q4 = min(q0 + 4 * bd, total - 1);
        const int q5 = min(q0 + 5 * bd, total - 1), q6 = min(q0 + 6 * bd, total - 1);
        const int q7 = min(q0 + 7 * bd, total - 1);
        const uint4 v0 = src(q0), v1 = src(q1), v2 = src(q2), v3 = src(q3);
        const uint4 v4 = src(q4), v5 = src(q5), v6 = src(q6), v7 = src(q7);
        dst[q0] = v0;
        dst[q1] = v1;
        dst[q2] = v2;
        dst[q3] = v3;
        dst[q4] = v4;
        dst[q5] = v5;
        dst[q6] = v6;
        dst[q7] = v7;
    }
}

MOE_DEV const uint8_t* expert_base(const ExpertArgs& a, int expert) {
    const int slot = a.slot_table[expert];
    if (slot < 0) return nullptr;
    return a.arena + (size_t)slot * a.slot_bytes;
}

// ------------------------------------------------------------------ Q2_K gate/up
// Lanes: tid = pr * 2L + mtx * L + kb  (L = D/32; mtx 0 = W1, 1 = W3; pr = row slot).
template <int T>
__global__ __launch_bounds__(512) void gateup_q2k_kernel(ExpertArgs a, int R, int P) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int L = D / QB;
    const int nsb = D / QK;
    const int rowbytes = nsb * Q2K_BYTES;
    const int tiles = I / R;
    const int c = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    if (c >= *a.n_chunks) return;
    const Chunk ch = a.chunks[c];
    const int r0 = tile * R;
    const ChunkRows cr = chunk_rows(a, ch);
    float* hout = (cr.shared ? a.h_shared : a.h_routed) + (size_t)ch.row0 * I;
    const uint8_t *w1, *w3;
    if (cr.shared) {
        w1 = a.sh_w1;
        w3 = a.sh_w3;
    } else {
        if (a.slot_table[ch.expert] == SLOT_SKIP) return;   // computed in another slot wave
        const uint8_t* base = expert_base(a, ch.expert);
        if (base == nullptr) {
            if (threadIdx.x == 0 && tile == 0) atomicOr(a.err, ERR_NOTRESIDENT);
            for (int q = threadIdx.x; q < R * cr.nrows; q += blockDim.x)
                hout[(size_t)(q / R) * I + r0 + q % R] = 0.f;
            return;
        }
        w1 = base + a.off_w1;
        w3 = base + a.off_w3;
    }

    const int tid = threadIdx.x;
    const int pr = tid / (2 * L), rem = tid % (2 * L);
    const int mtx = rem / L, kb = rem % L;
    const int s = kb >> 3, hh = (kb >> 2) & 1, j = kb & 3;

    // the lane's activation block for each row of the chunk
    uint32_t av[T][8];
    float dx[T];
    int slo[T], shi[T];
#pragma unroll
    for (int i = 0; i < T; ++i) {
        if (i < cr.nrows) {
            const int t = cr.tok[i];
            const uint4* src = reinterpret_cast<const uint4*>(a.xq + (size_t)t * D + kb * QB);
            const uint4 u0 = src[0], u1 = src[1];
            av[i][0] = u0.x; av[i][1] = u0.y; av[i][2] = u0.z; av[i][3] = u0.w;
            av[i][4] = u1.x; av[i][5] = u1.y; av[i][6] = u1.z; av[i][7] = u1.w;
            dx[i] = a.xd[(size_t)t * L + kb];
            slo[i] = a.xs16[(size_t)t * 2 * L + 2 * kb];
            shi[i] = a.xs16[(size_t)t * 2 * L + 2 * kb + 1];
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) av[i][q] = 0;
            dx[i] = 0.f;
            slo[i] = shi[i] = 0;
        }
    }

    // stage W1 rows [r0, r0+R) then W3 rows [r0, r0+R) into LDS
    uint8_t* tw = smem;
    float* red = reinterpret_cast<float*>(smem + 2 * R * rowbytes);   // [R][2][nsb][T]
    {
        const int n16 = R * rowbytes / 16;
        const uint4* g1 = reinterpret_cast<const uint4*>(w1 + (size_t)r0 * rowbytes);
        const uint4* g3 = reinterpret_cast<const uint4*>(w3 + (size_t)r0 * rowbytes);
        uint4* dst = reinterpret_cast<uint4*>(tw);
        stage_two(dst, g1, g3, n16, tid, (int)blockDim.x);
    }
    __syncthreads();

    const uint32_t* tw32 = reinterpret_cast<const uint32_t*>(tw);
    for (int r = pr; r < R; r += P) {
        const int sb = mtx * R * rowbytes + panel_off(r, s, nsb, Q2K_BYTES);   // multiple of 4
        uint32_t W[8];
        const int qoff = (sb + 16 + 32 * hh) >> 2;
#pragma unroll
        for (int q = 0; q < 8; ++q) W[q] = (tw32[qoff + q] >> (2 * j)) & 0x03030303u;
        const uint32_t scw = tw32[(sb >> 2) + 2 * hh + (j >> 1)] >> (16 * (j & 1));
        const uint32_t ddm = tw32[(sb + 80) >> 2];
        const float d = half_bits_to_f32(ddm & 0xFFFFu), dmin = half_bits_to_f32(ddm >> 16);
        const int sc_lo = scw & 15, m_lo = (scw >> 4) & 15, sc_hi = (scw >> 8) & 15, m_hi = (scw >> 12) & 15;
        float part[T];
#pragma unroll
        for (int i = 0; i < T; ++i) {
            int il = 0, ih = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) il = sdot4(W[q], av[i][q], il);
#pragma unroll
            for (int q = 4; q < 8; ++q) ih = sdot4(W[q], av[i][q], ih);
            const int isum = __mul24(sc_lo, il) + __mul24(sc_hi, ih);
            const int msum = __mul24(m_lo, slo[i]) + __mul24(m_hi, shi[i]);
            part[i] = dx[i] * (d * (float)isum - dmin * (float)msum);
        }
#pragma unroll
        for (int i = 0; i < T; ++i) part[i] = group8_sum(part[i]);
        if ((kb & 7) == 7) {
#pragma unroll
            for (int i = 0; i < T; ++i) red[((r * 2 + mtx) * nsb + s) * T + i] = part[i];
        }
    }
    __syncthreads();
    for (int q = tid; q < R * T; q += blockDim.x) {
        const int r = q / T, i = q % T;
        if (i >= cr.nrows) continue;
        const float* rg = red + (size_t)(r * 2 + 0) * nsb * T + i;
        const float* ru = red + (size_t)(r * 2 + 1) * nsb * T + i;
        float g = 0.f, u = 0.f;
        int sbi = 0;
        for (; sbi + 4 <= nsb; sbi += 4) {   // four independent reads per step, summed in order
            const float g0 = rg[(sbi + 0) * T], g1 = rg[(sbi + 1) * T], g2 = rg[(sbi + 2) * T], g3 = rg[(sbi + 3) * T];
            const float u0 = ru[(sbi + 0) * T], u1 = ru[(sbi + 1) * T], u2 = ru[(sbi + 2) * T], u3 = ru[(sbi + 3) * T];
            g = (((g + g0) + g1) + g2) + g3;
            u = (((u + u0) + u1) + u2) + u3;
        }
        for (; sbi < nsb; ++sbi) {
            g += rg[sbi * T];
            u += ru[sbi * T];
        }
        hout[(size_t)i * I + r0 + r] = swiglu(g, u, a.limit);
    }
}

// ------------------------------------------------------------------ Q3_K down
// Lanes: tid = pr * L + kb (L = I/32). The prologue forms the lane's q8_1 block of h.
template <int T>
__global__ __launch_bounds__(640) void down_q3k_kernel(ExpertArgs a, int R, int P) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int L = I / QB;
    const int nsb = I / QK;
    const int rowbytes = nsb * Q3K_BYTES;
    const int tiles = D / R;
    const int c = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    if (c >= *a.n_chunks) return;
    const Chunk ch = a.chunks[c];
    const int r0 = tile * R;
    const ChunkRows cr = chunk_rows(a, ch);
    float* eout = (cr.shared ? a.ys : a.e_rows) + (size_t)ch.row0 * D;
    const uint8_t* w2;
    if (cr.shared) {
        w2 = a.sh_w2;
    } else {
        if (a.slot_table[ch.expert] == SLOT_SKIP) return;   // computed in another slot wave
        const uint8_t* base = expert_base(a, ch.expert);
        if (base == nullptr) {
            for (int q = threadIdx.x; q < R * cr.nrows; q += blockDim.x)
                eout[(size_t)(q / R) * D + r0 + q % R] = 0.f;
            return;
        }
        w2 = base + a.off_w2;
    }

    const int tid = threadIdx.x;
    const int pr = tid / L, kb = tid % L;
    const int s = kb >> 3, hh = (kb >> 2) & 1, j = kb & 3;

    uint32_t av[T][8];
    float dx[T];
    int slo[T], shi[T];
    const int8_t* hq = cr.shared ? a.hq_shared : a.hq_routed;
    const float* hd = cr.shared ? a.hd_shared : a.hd_routed;
    const int32_t* hs = cr.shared ? a.hs_shared : a.hs_routed;
#pragma unroll
    for (int i = 0; i < T; ++i) {
        if (i < cr.nrows) {
            const size_t row = (size_t)ch.row0 + i;
            const uint4* src = reinterpret_cast<const uint4*>(hq + row * I + kb * QB);
            const uint4 u0 = src[0], u1 = src[1];
            av[i][0] = u0.x; av[i][1] = u0.y; av[i][2] = u0.z; av[i][3] = u0.w;
            av[i][4] = u1.x; av[i][5] = u1.y; av[i][6] = u1.z; av[i][7] = u1.w;
            dx[i] = hd[row * L + kb];
            slo[i] = hs[row * 2 * L + 2 * kb];
            shi[i] = hs[row * 2 * L + 2 * kb + 1];
        } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) av[i][q] = 0;
            dx[i] = 0.f;
            slo[i] = shi[i] = 0;
        }
    }

    uint8_t* tw = smem;
    float* red = reinterpret_cast<float*>(smem + R * rowbytes + 16);   // [R][nsb][T]
    {
        const int n16 = R * rowbytes / 16;
        const uint4* g = reinterpret_cast<const uint4*>(w2 + (size_t)r0 * rowbytes);
        uint4* dst = reinterpret_cast<uint4*>(tw);
        stage_two(dst, g, g, n16, tid, (int)blockDim.x);   // second half empty: copies g[0, n16)
    }
    __syncthreads();

    // per-lane constants for the two 6-bit scales of sub-blocks n = 8hh + 2j + {0,1}
    const int n_lo = 8 * hh + 2 * j;
    const int lo_byte0 = 2 * j, lo_shift = 4 * hh;
    const int hi_byte0 = 8 + (n_lo & 3), hi_byte1 = 8 + ((n_lo + 1) & 3);
    const int hi_shift = 2 * (n_lo >> 2);
    const uint32_t* tw32 = reinterpret_cast<const uint32_t*>(tw);
    for (int r = pr; r < R; r += P) {
        const int sb = panel_off(r, s, nsb, Q3K_BYTES);    // 2-byte aligned
        const int A = sb >> 2;
        const uint32_t sh = (uint32_t)(sb & 3) * 8u;     // 0 or 16
        uint32_t V[8];
        {
            const int qo = A + 8 + 8 * hh;                  // qs[32hh ..] at byte 32 + 32hh
            uint32_t prev = tw32[qo];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t next = tw32[qo + q + 1];
                const uint32_t qs = funnel(next, prev, sh);
                const uint32_t hm = funnel(tw32[A + q + 1], tw32[A + q], sh);
                prev = next;
                const uint32_t lo = (qs >> (2 * j)) & 0x03030303u;
                const uint32_t hb = (hm >> (4 * hh + j)) & 0x01010101u;
                V[q] = lo | (hb << 2);                      // q3 + 4, 0..7
            }
        }
        const uint32_t s0 = funnel(tw32[A + 25], tw32[A + 24], sh);   // scale bytes 0..3
        const uint32_t s1 = funnel(tw32[A + 26], tw32[A + 25], sh);   // 4..7
        const uint32_t s2 = funnel(tw32[A + 27], tw32[A + 26], sh);   // 8..11
        const uint32_t dbits = (tw32[A + 27] >> sh) & 0xFFFFu;         // d at byte 108
        const uint32_t lo_word = (lo_byte0 < 4) ? s0 : s1;
        const int lsh = 8 * (lo_byte0 & 3);
        const int low4_lo = (lo_word >> (lsh + lo_shift)) & 15;
        const int low4_hi = (lo_word >> (lsh + 8 + lo_shift)) & 15;
        const int hi2_lo = (s2 >> (8 * (hi_byte0 - 8) + hi_shift)) & 3;
        const int hi2_hi = (s2 >> (8 * (hi_byte1 - 8) + hi_shift)) & 3;
        const int s6_lo = (low4_lo | (hi2_lo << 4)) - 32;
        const int s6_hi = (low4_hi | (hi2_hi << 4)) - 32;
        const float d = half_bits_to_f32(dbits);
        float part[T];
#pragma unroll
        for (int i = 0; i < T; ++i) {
            int il = 0, ih = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) il = sdot4(V[q], av[i][q], il);
#pragma unroll
            for (int q = 4; q < 8; ++q) ih = sdot4(V[q], av[i][q], ih);
            il -= 4 * slo[i];
            ih -= 4 * shi[i];
            part[i] = dx[i] * (d * (float)(__mul24(s6_lo, il) + __mul24(s6_hi, ih)));
        }
#pragma unroll
        for (int i = 0; i < T; ++i) part[i] = group8_sum(part[i]);
        if ((kb & 7) == 7) {
#pragma unroll
            for (int i = 0; i < T; ++i) red[(r * nsb + s) * T + i] = part[i];
        }
    }
    __syncthreads();
    for (int q = tid; q < R * T; q += blockDim.x) {
        const int r = q / T, i = q % T;
        if (i >= cr.nrows) continue;
        const float* re = red + (size_t)r * nsb * T + i;
        float e = 0.f;
        int sbi = 0;
        for (; sbi + 4 <= nsb; sbi += 4) {
            const float e0 = re[(sbi + 0) * T], e1 = re[(sbi + 1) * T], e2 = re[(sbi + 2) * T], e3 = re[(sbi + 3) * T];
            e = (((e + e0) + e1) + e2) + e3;
        }
        for (; sbi < nsb; ++sbi) e += re[sbi * T];
        eout[(size_t)i * D + r0 + r] = e;
    }
}

// ------------------------------------------------------------------ q8_1 of h
// One lane per 32-value block of the SwiGLU output rows (routed positions, then
// the K-quant shared expert's token rows): the activation of the down projection.
__global__ __launch_bounds__(256) void quantize_h_kernel(ExpertArgs a, int routed_rows, int shared_rows) {
    const int L = a.I / QB;
    const int b = blockIdx.x * 256 + threadIdx.x;
    const int total = (routed_rows + shared_rows) * L;
    if (b >= total) return;
    const bool sh = b >= routed_rows * L;
    const int bb = sh ? b - routed_rows * L : b;
    const float* src = (sh ? a.h_shared : a.h_routed) + (size_t)bb * QB;
    float v[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float4 f = reinterpret_cast<const float4*>(src)[q];
        v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    }
    uint32_t qv[8];
    float d;
    int sl, shs;
    q8_1_block(v, qv, d, sl, shs);
    uint4* dst = reinterpret_cast<uint4*>((sh ? a.hq_shared : a.hq_routed) + (size_t)bb * QB);
    dst[0] = make_uint4(qv[0], qv[1], qv[2], qv[3]);
    dst[1] = make_uint4(qv[4], qv[5], qv[6], qv[7]);
    (sh ? a.hd_shared : a.hd_routed)[bb] = d;
    int32_t* hs = (sh ? a.hs_shared : a.hs_routed) + 2 * (size_t)bb;
    hs[0] = sl;
    hs[1] = shs;
}

hipError_t launch_quantize_h(const ExpertArgs& a, int routed_rows, int shared_rows, hipStream_t st) {
    const int total = (routed_rows + shared_rows) * (a.I / QB);
    if (total == 0) return hipSuccess;
    return launch_kernel(quantize_h_kernel, (total + 255) / 256, 256, 0, st, a, routed_rows, shared_rows);
}

// ------------------------------------------------------------------ launch geometry
GemvGeom gateup_geom(int D, int I) {
    GemvGeom g;
    const int L2 = 2 * (D / QB);
    g.P = L2 >= 256 ? 1 : 256 / L2;
    g.threads = L2 * g.P;
    g.R = g.P > GEMV_ROWS ? g.P : GEMV_ROWS;
    g.tiles = I / g.R;
    const int rowbytes = (D / QK) * Q2K_BYTES;
    g.lds_base = 2 * g.R * rowbytes;
    g.lds_per_t = g.R * 2 * (D / QK) * 4;
    return g;
}

GemvGeom down_geom(int D, int I) {
    GemvGeom g;
    const int L = I / QB;
    int P = 1;
    while (L * P < 256 || (L * P) % 64 != 0) {
        if (L * (P + 1) > 640) break;     // the kernel's launch bound
        ++P;
    }
    g.P = P;
    g.threads = L * P;
    g.R = 2 * GEMV_ROWS;
    while (g.R < P) g.R += GEMV_ROWS;
    while (D % g.R) g.R += GEMV_ROWS;
    g.tiles = D / g.R;
    const int rowbytes = (I / QK) * Q3K_BYTES;
    g.lds_base = g.R * rowbytes + 16;
    g.lds_per_t = g.R * (I / QK) * 4;
    return g;
}

template <int T>
static hipError_t launch_pair(const ExpertArgs& a, int max_chunks, hipStream_t st) {
    const GemvGeom gu = gateup_geom(a.D, a.I);
    const size_t lds1 = gu.lds_base + (size_t)gu.lds_per_t * T;
    hipError_t e = launch_kernel(gateup_q2k_kernel<T>, max_chunks * gu.tiles, gu.threads, lds1, st, a, gu.R, gu.P);
    if (e != hipSuccess) return e;
    return hipSuccess;
}

template <int T>
static hipError_t launch_down(const ExpertArgs& a, int max_chunks, hipStream_t st) {
    const GemvGeom dg = down_geom(a.D, a.I);
    const size_t lds2 = dg.lds_base + (size_t)dg.lds_per_t * T;
    return launch_kernel(down_q3k_kernel<T>, max_chunks * dg.tiles, dg.threads, lds2, st, a, dg.R, dg.P);
}

hipError_t launch_gateup_q2k(const ExpertArgs& a, int rows_max, int max_chunks, hipStream_t st) {
    if (max_chunks <= 0) return hipSuccess;
    if (rows_max <= 1) return launch_pair<1>(a, max_chunks, st);
    if (rows_max <= 2) return launch_pair<2>(a, max_chunks, st);
    if (rows_max <= 4) return launch_pair<4>(a, max_chunks, st);
    return launch_pair<8>(a, max_chunks, st);
}

hipError_t launch_down_q3k(const ExpertArgs& a, int rows_max, int max_chunks, hipStream_t st) {
    if (max_chunks <= 0) return hipSuccess;
    if (rows_max <= 1) return launch_down<1>(a, max_chunks, st);
    if (rows_max <= 2) return launch_down<2>(a, max_chunks, st);
    if (rows_max <= 4) return launch_down<4>(a, max_chunks, st);
    return launch_down<8>(a, max_chunks, st);
}

}  // namespace moe
