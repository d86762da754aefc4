// Streaming expert GEMVs for chunks of one or two token rows (decode).
//   gate/up: g = W1 q8_1(x), u = W3 q8_1(x) over Q2_K blocks + clamped SwiGLU -> h
//   down:    E = W2 q8_1(h) over Q3_K blocks
// Same arithmetic as the general GEMVs (GGUF Q2_K / Q3_K superblocks against
// q8_1 activations; metrale moe_v41 module documentation: GEMVs for groups of
// up to eight rows; kernel table of moe_v41.rs: mmvq_q2k / mmvq_q3k /
// mmvq_*_experts), organised for bandwidth:
//  * persistent workgroups: the valid tiles (chunk x R weight rows) are split
//    into equal contiguous runs, one run per workgroup, so consecutive tiles
//    of a run are consecutive bytes of one expert;
//  * software pipelining: the next tile's raw blocks are loaded into registers
//    (coalesced 16-byte loads) while the current tile is computed from LDS;
//  * each lane owns half a superblock of the K dimension (four q8_1 blocks),
//    reads its weight bytes from LDS once for the four bit planes, and keeps
//    the four activation blocks in registers.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

// up to NPF 16-byte chunks per thread held in registers between the global
// loads and the LDS writes (named values: arrays of them ended up in scratch)
template <int NPF>
struct Prefetch {
    uint4 v0, v1, v2, v3, v4, v5;
};

// chunks [0, n) of a, then [0, n) of b when two_mats
template <int NPF>
MOE_DEV void prefetch_load(Prefetch<NPF>& pf, const uint4* a, const uint4* b, int n, bool two_mats, int tid, int bd) {
    static_assert(NPF >= 1 && NPF <= 6, "prefetch depth");
    const int total = two_mats ? 2 * n : n;
    auto src = [&](int q) {
        const int qq = min(q, total - 1);
        return qq < n ? a[qq] : b[qq - n];
    };
    pf.v0 = src(tid);
    if (NPF > 1) pf.v1 = src(tid + bd);
    if (NPF > 2) pf.v2 = src(tid + 2 * bd);
    if (NPF > 3) pf.v3 = src(tid + 3 * bd);
    if (NPF > 4) pf.v4 = src(tid + 4 * bd);
    if (NPF > 5) pf.v5 = src(tid + 5 * bd);
}

template <int NPF>
MOE_DEV void prefetch_store(const Prefetch<NPF>& pf, uint4* dst, int total, int tid, int bd) {
    dst[min(tid, total - 1)] = pf.v0;
    if (NPF > 1) dst[min(tid + bd, total - 1)] = pf.v1;
    if (NPF > 2) dst[min(tid + 2 * bd, total - 1)] = pf.v2;
    if (NPF > 3) dst[min(tid + 3 * bd, total - 1)] = pf.v3;
    if (NPF > 4) dst[min(tid + 4 * bd, total - 1)] = pf.v4;
    if (NPF > 5) dst[min(tid + 5 * bd, total - 1)] = pf.v5;
}

constexpr int GATEUP_NPF = 6;
constexpr int DOWN_NPF = 4;

// the run of valid tiles [first, last) of this workgroup
MOE_DEV void tile_run(int n_valid, int& first, int& last) {
    const int per = (n_valid + gridDim.x - 1) / gridDim.x;
    first = min((int)blockIdx.x * per, n_valid);
    last = min(first + per, n_valid);
}

// weights of a chunk: routed expert through the slot table, or the shared expert
MOE_DEV const uint8_t* chunk_weights(const ExpertArgs& a, const Chunk& ch, size_t off, const uint8_t* shared) {
    if (ch.expert < 0) return shared;
    const int slot = a.slot_table[ch.expert];
    if (slot < 0) return nullptr;
    return a.arena + (size_t)slot * a.slot_bytes + off;
}

MOE_DEV int chunk_token(const ExpertArgs& a, const Chunk& ch, int i) {
    return ch.expert < 0 ? ch.row0 + i : a.perm[ch.row0 + i] / a.topk;
}

// Sum over aligned groups of RG lanes (RG in {1, 2, 4, 8}); valid in the group's last lane.
MOE_DEV float group_sum(float v, int RG) {
    if (RG >= 2) v += dpp_quad_xor1(v);
    if (RG >= 4) v += dpp_quad_xor2(v);
    if (RG >= 8) v += dpp_row_ror4(v);
    return v;
}

}  // namespace

// ------------------------------------------------------------------ Q2_K gate/up
// Lanes: tid = pr * 2 L4 + mtx * L4 + sl, L4 = D / 128 (two lanes per superblock:
// sl = 2 s + hh), mtx 0 = W1, 1 = W3, pr = row slot (P slots).
template <int T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(3))) void gateup_q2k_stream_kernel(ExpertArgs a, int R, int P, int RG) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int L4 = D / 128;
    const int nsb = D / QK;
    const int rowbytes = nsb * Q2K_BYTES;
    const int TPC = I / R;
    const int n16 = R * rowbytes / 16;
    const int bd = blockDim.x, tid = threadIdx.x;
    int first, last;
    tile_run(*a.n_chunks * TPC, first, last);
    if (first >= last) return;

    const int pr = tid / (2 * L4), rem = tid % (2 * L4);
    const int mtx = rem / L4, sl = rem % L4;
    const int s = sl >> 1, hh = sl & 1;
    const int ngr = L4 / RG;
    uint8_t* tw = smem;
    float* red = reinterpret_cast<float*>(smem + 2 * R * rowbytes);   // [R][2][ngr][T]

    // activation blocks kb = 8 s + 4 hh + j: quants, d / f_j, and f_j * (16-value sums);
    // f_j = 1, 4, 16, 16 is the scale the bit-plane masks below leave on the quants
    uint32_t av[T][4][8];
    float dxs[T][4];
    int slo[T][4], shi[T][4];
    int cur_chunk = -1, nrows = 0;

    Chunk ch = a.chunks[first / TPC];
    const uint8_t* w1 = chunk_weights(a, ch, a.off_w1, a.sh_w1);
    const uint8_t* w3 = chunk_weights(a, ch, a.off_w3, a.sh_w3);
    Prefetch<GATEUP_NPF> pf;
    if (w1 != nullptr) {
        const size_t o = (size_t)(first % TPC) * R * rowbytes;
        prefetch_load(pf, reinterpret_cast<const uint4*>(w1 + o), reinterpret_cast<const uint4*>(w3 + o), n16, true,
                      tid, bd);
    }
    for (int tile = first; tile < last; ++tile) {
        const int c = tile / TPC, r0 = (tile % TPC) * R;
        const bool resident = w1 != nullptr;
        if (c != cur_chunk) {
            cur_chunk = c;
            nrows = ch.nrows;
#pragma unroll
            for (int i = 0; i < T; ++i) {
                const bool live = i < nrows;
                const int t = live ? chunk_token(a, ch, i) : 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kb = 8 * s + 4 * hh + j;
                    const int f = j == 0 ? 1 : (j == 1 ? 4 : 16);
                    if (live) {
                        const uint4* src = reinterpret_cast<const uint4*>(a.xq + (size_t)t * D + kb * QB);
                        const uint4 u0 = src[0], u1 = src[1];
                        av[i][j][0] = u0.x; av[i][j][1] = u0.y; av[i][j][2] = u0.z; av[i][j][3] = u0.w;
                        av[i][j][4] = u1.x; av[i][j][5] = u1.y; av[i][j][6] = u1.z; av[i][j][7] = u1.w;
                        dxs[i][j] = a.xd[(size_t)t * (D / QB) + kb] / (float)f;
                        slo[i][j] = f * a.xs16[(size_t)t * (D / 16) + 2 * kb];
                        shi[i][j] = f * a.xs16[(size_t)t * (D / 16) + 2 * kb + 1];
                    } else {
#pragma unroll
                        for (int q = 0; q < 8; ++q) av[i][j][q] = 0;
                        dxs[i][j] = 0.f;
                        slo[i][j] = shi[i][j] = 0;
                    }
                }
            }
        }
        float* hout = (ch.expert < 0 ? a.h_shared : a.h_routed) + (size_t)ch.row0 * I;
        if (resident) prefetch_store(pf, reinterpret_cast<uint4*>(tw), 2 * n16, tid, bd);
        __syncthreads();
        // issue the next tile's loads before computing this one
        const Chunk ch_this = ch;
        if (tile + 1 < last) {
            const int nc = (tile + 1) / TPC;
            if (nc != c) {
                ch = a.chunks[nc];
                w1 = chunk_weights(a, ch, a.off_w1, a.sh_w1);
                w3 = chunk_weights(a, ch, a.off_w3, a.sh_w3);
            }
            if (w1 != nullptr) {
                const size_t o = (size_t)((tile + 1) % TPC) * R * rowbytes;
                prefetch_load(pf, reinterpret_cast<const uint4*>(w1 + o), reinterpret_cast<const uint4*>(w3 + o), n16,
                              true, tid, bd);
            }
        }
        if (resident) {
            const uint32_t* tw32 = reinterpret_cast<const uint32_t*>(tw);
#pragma unroll 1
            for (int r = pr; r < R; r += P) {
                const int sb = ((mtx * R + r) * rowbytes + s * Q2K_BYTES) >> 2;   // dword index
                uint32_t Q[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) Q[q] = tw32[sb + 4 + 8 * hh + q];
                const uint32_t sc0 = tw32[sb + 2 * hh], sc1 = tw32[sb + 2 * hh + 1];
                const uint32_t ddm = tw32[sb + 20];
                const float d = half_bits_to_f32(ddm & 0xFFFFu), dmin = half_bits_to_f32(ddm >> 16);
                float part[T];
#pragma unroll
                for (int i = 0; i < T; ++i) part[i] = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t scw = (j < 2 ? sc0 : sc1) >> (16 * (j & 1));
                    const int sc_lo = scw & 15, m_lo = (scw >> 4) & 15;
                    const int sc_hi = (scw >> 8) & 15, m_hi = (scw >> 12) & 15;
                    uint32_t W[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q)
                        W[q] = j == 3 ? ((Q[q] >> 2) & 0x30303030u) : (Q[q] & (0x03030303u << (2 * j)));
#pragma unroll
                    for (int i = 0; i < T; ++i) {
                        int il = 0, ih = 0;
#pragma unroll
                        for (int q = 0; q < 4; ++q) il = sdot4(W[q], av[i][j][q], il);
#pragma unroll
                        for (int q = 4; q < 8; ++q) ih = sdot4(W[q], av[i][j][q], ih);
                        const int isum = __mul24(sc_lo, il) + __mul24(sc_hi, ih);
                        const int msum = __mul24(m_lo, slo[i][j]) + __mul24(m_hi, shi[i][j]);
                        part[i] = fmaf(dxs[i][j], fmaf(d, (float)isum, -dmin * (float)msum), part[i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < T; ++i) part[i] = group_sum(part[i], RG);
                if (sl % RG == RG - 1) {
#pragma unroll
                    for (int i = 0; i < T; ++i) red[((r * 2 + mtx) * ngr + sl / RG) * T + i] = part[i];
                }
            }
        }
        __syncthreads();
        for (int q = tid; q < R * T; q += bd) {
            const int r = q / T, i = q % T;
            if (i >= ch_this.nrows) continue;
            float h = 0.f;
            if (resident) {
                const float* rg = red + (size_t)(r * 2 + 0) * ngr * T + i;
                const float* ru = red + (size_t)(r * 2 + 1) * ngr * T + i;
                float g = 0.f, u = 0.f;
                for (int k = 0; k < ngr; ++k) {
                    g += rg[k * T];
                    u += ru[k * T];
                }
                h = swiglu(g, u, a.limit);
            } else if (q == 0 && r0 == 0) {
                atomicOr(a.err, ERR_NOTRESIDENT);
            }
            hout[(size_t)i * I + r0 + r] = h;
        }
    }
}

// ------------------------------------------------------------------ Q3_K down
// Lanes: tid = pr * L4 + sl, L4 = I / 128 (sl = 2 s + hh), pr = row slot.
template <int T>
__global__ __launch_bounds__(640) __attribute__((amdgpu_waves_per_eu(3))) void down_q3k_stream_kernel(ExpertArgs a, int R, int P, int RG) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int L4 = I / 128;
    const int nsb = I / QK;
    const int rowbytes = nsb * Q3K_BYTES;
    const int TPC = D / R;
    const int n16 = R * rowbytes / 16;
    const int bd = blockDim.x, tid = threadIdx.x;
    int first, last;
    tile_run(*a.n_chunks * TPC, first, last);
    if (first >= last) return;

    const int pr = tid / L4, sl = tid % L4;
    const bool lane_live = pr < P;
    const int s = sl >> 1, hh = sl & 1;
    const int ngr = L4 / RG;
    uint8_t* tw = smem;
    float* red = reinterpret_cast<float*>(smem + R * rowbytes + 16);   // [R][ngr][T]

    uint32_t av[T][4][8];
    float dx[T][4];
    int slo[T][4], shi[T][4];
    int cur_chunk = -1;

    // per-lane constants of the packed 6-bit scales for sub-blocks n = 8 hh + 2 j + {0, 1}
    Chunk ch = a.chunks[first / TPC];
    const uint8_t* w2 = chunk_weights(a, ch, a.off_w2, a.sh_w2);
    Prefetch<DOWN_NPF> pf;
    if (w2 != nullptr) {
        const size_t o = (size_t)(first % TPC) * R * rowbytes;
        const uint4* g = reinterpret_cast<const uint4*>(w2 + o);
        prefetch_load(pf, g, g, n16, false, tid, bd);
    }
    for (int tile = first; tile < last; ++tile) {
        const int c = tile / TPC, r0 = (tile % TPC) * R;
        const bool resident = w2 != nullptr;
        if (c != cur_chunk) {
            cur_chunk = c;
            const int8_t* hq = ch.expert < 0 ? a.hq_shared : a.hq_routed;
            const float* hd = ch.expert < 0 ? a.hd_shared : a.hd_routed;
            const int32_t* hs = ch.expert < 0 ? a.hs_shared : a.hs_routed;
#pragma unroll
            for (int i = 0; i < T; ++i) {
                const bool live = i < ch.nrows;
                const size_t row = (size_t)ch.row0 + i;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int kb = 8 * s + 4 * hh + j;
                    if (live && lane_live) {
                        const uint4* src = reinterpret_cast<const uint4*>(hq + row * I + kb * QB);
                        const uint4 u0 = src[0], u1 = src[1];
                        av[i][j][0] = u0.x; av[i][j][1] = u0.y; av[i][j][2] = u0.z; av[i][j][3] = u0.w;
                        av[i][j][4] = u1.x; av[i][j][5] = u1.y; av[i][j][6] = u1.z; av[i][j][7] = u1.w;
                        dx[i][j] = hd[row * (I / QB) + kb];
                        slo[i][j] = 4 * hs[row * (I / 16) + 2 * kb];
                        shi[i][j] = 4 * hs[row * (I / 16) + 2 * kb + 1];
                    } else {
#pragma unroll
                        for (int q = 0; q < 8; ++q) av[i][j][q] = 0;
                        dx[i][j] = 0.f;
                        slo[i][j] = shi[i][j] = 0;
                    }
                }
            }
        }
        float* eout = (ch.expert < 0 ? a.ys : a.e_rows) + (size_t)ch.row0 * D;
        if (resident) prefetch_store(pf, reinterpret_cast<uint4*>(tw), n16, tid, bd);
        __syncthreads();
        const Chunk ch_this = ch;
        if (tile + 1 < last) {
            const int nc = (tile + 1) / TPC;
            if (nc != c) {
                ch = a.chunks[nc];
                w2 = chunk_weights(a, ch, a.off_w2, a.sh_w2);
            }
            if (w2 != nullptr) {
                const uint4* g = reinterpret_cast<const uint4*>(w2 + (size_t)((tile + 1) % TPC) * R * rowbytes);
                prefetch_load(pf, g, g, n16, false, tid, bd);
            }
        }
        if (resident && lane_live) {
            const uint32_t* tw32 = reinterpret_cast<const uint32_t*>(tw);
#pragma unroll 1
            for (int r = pr; r < R; r += P) {
                const int sb = r * rowbytes + s * Q3K_BYTES;   // 2-byte aligned
                const int A = sb >> 2;
                const uint32_t sh = (uint32_t)(sb & 3) * 8u;
                uint32_t Qs[8], Hh[8];
                {
                    const int qo = A + 8 + 8 * hh;
                    uint32_t prevq = tw32[qo], prevh = tw32[A];
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const uint32_t nq = tw32[qo + q + 1], nh = tw32[A + q + 1];
                        Qs[q] = funnel(nq, prevq, sh);
                        Hh[q] = funnel(nh, prevh, sh) >> (4 * hh);   // high bits of planes j at bit j
                        prevq = nq;
                        prevh = nh;
                    }
                }
                const uint32_t s0 = funnel(tw32[A + 25], tw32[A + 24], sh);
                const uint32_t s1 = funnel(tw32[A + 26], tw32[A + 25], sh);
                const uint32_t s2 = funnel(tw32[A + 27], tw32[A + 26], sh);
                const float d = half_bits_to_f32((tw32[A + 27] >> sh) & 0xFFFFu);
                float part[T];
#pragma unroll
                for (int i = 0; i < T; ++i) part[i] = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // six-bit scales of sub-blocks n = 8 hh + 2 j + b: low nibble in byte 2 j + b
                    // (high half when hh = 1), top pair in byte 8 + (2 j + b) % 4 at bit 2 (2 hh + j / 2)
                    const uint32_t lo_word = j < 2 ? s0 : s1;
                    const int lsh = 16 * (j & 1) + 4 * hh;
                    const int hsh = 2 * (2 * hh + j / 2);
                    const int hb0 = 8 * ((2 * j) & 3), hb1 = 8 * ((2 * j + 1) & 3);
                    const int s6_lo = (int)(((lo_word >> lsh) & 15) | (((s2 >> (hb0 + hsh)) & 3) << 4)) - 32;
                    const int s6_hi = (int)(((lo_word >> (lsh + 8)) & 15) | (((s2 >> (hb1 + hsh)) & 3) << 4)) - 32;
                    uint32_t V[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const uint32_t lo = (Qs[q] >> (2 * j)) & 0x03030303u;
                        const uint32_t hb = j <= 2 ? (Hh[q] << (2 - j)) : (Hh[q] >> 1);
                        V[q] = (hb & 0x04040404u) | lo;   // q3 + 4, in 0..7
                    }
#pragma unroll
                    for (int i = 0; i < T; ++i) {
                        int il = 0, ih = 0;
#pragma unroll
                        for (int q = 0; q < 4; ++q) il = sdot4(V[q], av[i][j][q], il);
#pragma unroll
                        for (int q = 4; q < 8; ++q) ih = sdot4(V[q], av[i][j][q], ih);
                        const int isum = __mul24(s6_lo, il - slo[i][j]) + __mul24(s6_hi, ih - shi[i][j]);
                        part[i] = fmaf(dx[i][j] * d, (float)isum, part[i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < T; ++i) part[i] = group_sum(part[i], RG);
                if (sl % RG == RG - 1) {
#pragma unroll
                    for (int i = 0; i < T; ++i) red[(r * ngr + sl / RG) * T + i] = part[i];
                }
            }
        }
        __syncthreads();
        for (int q = tid; q < R * T; q += bd) {
            const int r = q / T, i = q % T;
            if (i >= ch_this.nrows) continue;
            float e = 0.f;
            if (resident) {
                const float* re = red + (size_t)r * ngr * T + i;
                for (int k = 0; k < ngr; ++k) e += re[k * T];
            }
            eout[(size_t)i * D + r0 + r] = e;
        }
    }
}

// ------------------------------------------------------------------ launch
static int pow2_divisor_cap8(int v) {
    int g = 1;
    while (g < 8 && v % (2 * g) == 0) g *= 2;
    return g;
}

struct StreamGeom {
    int P, threads, R, RG;
    size_t lds;
};

static StreamGeom gateup_stream_geom(int D, int I, int T) {
    StreamGeom g;
    const int pair = 2 * (D / 128);
    int P = 1;
    while (pair * P < 256 || (pair * P) % 64) {
        if (pair * (P + 1) > 512) break;
        ++P;
    }
    g.P = P;
    g.threads = pair * P;
    g.R = 8;
    while (g.R < P) g.R *= 2;
    g.RG = pow2_divisor_cap8(D / 128);
    const int rowbytes = (D / QK) * Q2K_BYTES;
    g.lds = (size_t)2 * g.R * rowbytes + (size_t)g.R * 2 * ((D / 128) / g.RG) * T * 4;
    return g;
}

static StreamGeom down_stream_geom(int D, int I, int T) {
    StreamGeom g;
    const int L4 = I / 128;
    int P = 1;
    while (L4 * P < 256 || (L4 * P) % 64) {
        if (L4 * (P + 1) > 640) break;
        ++P;
    }
    g.P = P;
    g.threads = L4 * P;
    g.R = 16;
    while (g.R < P) g.R *= 2;
    while (D % g.R) g.R /= 2;
    g.RG = pow2_divisor_cap8(L4);
    const int rowbytes = (I / QK) * Q3K_BYTES;
    g.lds = (size_t)g.R * rowbytes + 16 + (size_t)g.R * (L4 / g.RG) * T * 4;
    return g;
}

bool stream_gemv_supported(int D, int I) {
    // tiles of R rows must be whole 16-byte runs, and the per-thread prefetch
    // (GATEUP_NPF / DOWN_NPF chunks of 16 bytes) must cover a whole tile
    const StreamGeom gu = gateup_stream_geom(D, I, 1);
    const StreamGeom dn = down_stream_geom(D, I, 1);
    const int gu_bytes = 2 * gu.R * (D / QK) * Q2K_BYTES;
    const int dn_bytes = dn.R * (I / QK) * Q3K_BYTES;
    return I % gu.R == 0 && D % dn.R == 0 && gu.R % gu.P == 0 && dn.R % dn.P == 0 && gu_bytes % 16 == 0 &&
           dn_bytes % 16 == 0 && gu_bytes <= GATEUP_NPF * 16 * gu.threads && dn_bytes <= DOWN_NPF * 16 * dn.threads;
}

// one token row per chunk (the decode arm; wider chunks use the general GEMVs)
hipError_t launch_gateup_q2k_stream(const ExpertArgs& a, int n_wg, hipStream_t st) {
    const StreamGeom g = gateup_stream_geom(a.D, a.I, 1);
    launch_kernel(gateup_q2k_stream_kernel<1>, n_wg, g.threads, g.lds, st, a, g.R, g.P, g.RG);
    return hipGetLastError();
}

hipError_t launch_down_q3k_stream(const ExpertArgs& a, int n_wg, hipStream_t st) {
    const StreamGeom g = down_stream_geom(a.D, a.I, 1);
    launch_kernel(down_q3k_stream_kernel<1>, n_wg, g.threads, g.lds, st, a, g.R, g.P, g.RG);
    return hipGetLastError();
}

}  // namespace moe
