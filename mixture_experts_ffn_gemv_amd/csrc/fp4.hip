// Routed experts in MXFP4, the upstream checkpoint's own format (Open Model
// Atlas, "DeepSeek V4.1 · Mixture of experts": the experts' Linear layers hold
// float4_e2m1fn_x2 weights; config.json expert_dtype "fp4"). The pages give the
// element type only; the scales follow the OCP microscaling layout: per 32
// consecutive weights of a row one E8M0 scale 2^(E-127), each weight an e2m1
// code, two per byte (the even weight in the low nibble). A matrix [rows, cols]
// is its codes [rows, cols/2] followed by its scales [rows, cols/32]; an expert
// slice is [W1 | W3 | W2].
//
// The activations stay bf16, as in the excerpt's Linear layers: each lane turns
// a 16-byte piece of codes (one 32-weight block) into bf16 pairs with the
// gfx950 scaled conversion (exact: the codes have two significant bits and the
// scale is a power of two) and dots them with bf16 pairs of x (f32
// accumulation). h is rounded to bf16 before W2.
//
// A chunk holds up to T token rows of one expert (positions row0.. in
// expert-sorted pick order). The chunk's bf16 rows go into LDS once per
// workgroup; each wavefront then reads whole rows of the weights (coalesced
// 16-byte pieces).
//  fp4_gateup_kernel: a wavefront per row r of h, holding pieces of W1 row r
//      and W3 row r, so the clamped SwiGLU needs no exchange; h bf16 [pairs, I].
//  fp4_down_kernel:   a wavefront per output row of W2 against the chunk's h
//      rows; E f32 [pairs, D], summed per token by the combine kernel.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int FP4_BLOCK = 32;    // weights per E8M0 scale, and per lane piece (16 code bytes)
constexpr int FP4_WAVES = 8;     // rows per workgroup (one per wavefront)
constexpr int MAXP = 4;          // pieces of a row per lane: rows of at most 4 x 64 x 32 = 8192 weights

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

MOE_DEV float e8m0_scale(uint32_t e) { return e == 255u ? __builtin_nanf("") : ldexpf(1.f, (int)e - 127); }

// the 32 weights of a piece as 16 bf16 pairs (pair k: weights 2k, 2k + 1)
MOE_DEV void piece_to_bf16(const uint4& q, float sc, uint32_t (&w)[16]) {
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], sc, 0));
        w[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], sc, 1));
        w[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], sc, 2));
        w[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], sc, 3));
    }
}

MOE_DEV float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// the chunk's token rows of a bf16 matrix [*, K] into LDS (rows past nrows are zero)
template <int T>
MOE_DEV void stage_rows(uint4* dst, const uint16_t* src, const int (&row)[T], int nrows, int K) {
    const int k8 = K / 8;
    for (int u = threadIdx.x; u < T * k8; u += blockDim.x) {
        const int i = u / k8, k = u % k8;
        dst[u] = i < nrows ? reinterpret_cast<const uint4*>(src + (size_t)row[i] * K)[k] : make_uint4(0, 0, 0, 0);
    }
}

// one row of an MXFP4 matrix (K weights) against T bf16 rows in LDS: acc[t] += row . x[t]
template <int T>
MOE_DEV void row_dot(const uint8_t* codes, const uint8_t* scales, const uint4* xl, int K, float (&acc)[T]) {
    const int lane = threadIdx.x & 63, np = K / FP4_BLOCK, k8 = K / 8;
    uint4 q[MAXP];
    uint32_t e[MAXP];
#pragma unroll
    for (int j = 0; j < MAXP; ++j) {
        const int p = min(lane + 64 * j, np - 1);
        q[j] = reinterpret_cast<const uint4*>(codes)[p];
        e[j] = scales[p];
    }
#pragma unroll
    for (int j = 0; j < MAXP; ++j) {
        const int p = lane + 64 * j;
        if (p >= np) break;
        uint32_t w[16];
        piece_to_bf16(q[j], e8m0_scale(e[j]), w);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const uint4* xp = xl + (size_t)t * k8 + 4 * p;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 xv = xp[i];
                acc[t] = dot2(w[4 * i + 0], xv.x, acc[t]);
                acc[t] = dot2(w[4 * i + 1], xv.y, acc[t]);
                acc[t] = dot2(w[4 * i + 2], xv.z, acc[t]);
                acc[t] = dot2(w[4 * i + 3], xv.w, acc[t]);
            }
        }
    }
}

// the expert's slice, or nullptr (with the chunk's outputs to be zeroed or skipped)
MOE_DEV const uint8_t* chunk_slice(const ExpertArgs& a, const Chunk& ch, bool& skip) {
    const int slot = a.slot_table[ch.expert];
    skip = slot == SLOT_SKIP;   // computed in another slot wave
    if (skip || slot < 0) return nullptr;
    return a.arena + (size_t)slot * a.slot_bytes;
}

}  // namespace

template <int T>
__global__ __launch_bounds__(FP4_WAVES * 64) void fp4_gateup_kernel(ExpertArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int tiles = I / FP4_WAVES;
    const int c = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    if (c >= *a.n_chunks) return;
    const Chunk ch = a.chunks[c];
    const int lane = threadIdx.x & 63, r = tile * FP4_WAVES + (threadIdx.x >> 6);
    uint16_t* h = reinterpret_cast<uint16_t*>(a.h_routed);   // bf16 [pairs, I]
    bool skip;
    const uint8_t* base = chunk_slice(a, ch, skip);
    if (skip) return;
    if (base == nullptr) {   // not resident: flag it, and its rows of h are zero
        if (threadIdx.x == 0 && tile == 0) atomicOr(a.err, ERR_NOTRESIDENT);
        if (lane < ch.nrows) h[(size_t)(ch.row0 + lane) * I + r] = 0;
        return;
    }
    int tok[T];
#pragma unroll
    for (int i = 0; i < T; ++i) tok[i] = i < ch.nrows ? a.perm[ch.row0 + i] / a.topk : 0;
    uint4* xl = reinterpret_cast<uint4*>(smem);
    stage_rows<T>(xl, a.x16, tok, ch.nrows, D);
    __syncthreads();
    const size_t cb = (size_t)I * (D / 2);   // code bytes of W1 (scales follow)
    float g[T], u[T];
#pragma unroll
    for (int t = 0; t < T; ++t) g[t] = u[t] = 0.f;
    const uint8_t* w1 = base + a.off_w1;
    const uint8_t* w3 = base + a.off_w3;
    row_dot<T>(w1 + (size_t)r * (D / 2), w1 + cb + (size_t)r * (D / FP4_BLOCK), xl, D, g);
    row_dot<T>(w3 + (size_t)r * (D / 2), w3 + cb + (size_t)r * (D / FP4_BLOCK), xl, D, u);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float gs = wave_sum(g[t]), us = wave_sum(u[t]);
        if (lane == t && t < ch.nrows)
            h[(size_t)(ch.row0 + t) * I + r] = (uint16_t)f32_to_bf16(swiglu(gs, us, a.limit));
    }
}

template <int T>
__global__ __launch_bounds__(FP4_WAVES * 64) void fp4_down_kernel(ExpertArgs a) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int tiles = D / FP4_WAVES;
    const int c = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    if (c >= *a.n_chunks) return;
    const Chunk ch = a.chunks[c];
    const int lane = threadIdx.x & 63, d = tile * FP4_WAVES + (threadIdx.x >> 6);
    bool skip;
    const uint8_t* base = chunk_slice(a, ch, skip);
    if (skip) return;
    if (base == nullptr) {
        if (lane < ch.nrows) a.e_rows[(size_t)(ch.row0 + lane) * D + d] = 0.f;
        return;
    }
    int rows[T];
#pragma unroll
    for (int i = 0; i < T; ++i) rows[i] = ch.row0 + min(i, ch.nrows - 1);
    uint4* hl = reinterpret_cast<uint4*>(smem);
    stage_rows<T>(hl, reinterpret_cast<const uint16_t*>(a.h_routed), rows, ch.nrows, I);
    __syncthreads();
    const uint8_t* w2 = base + a.off_w2;
    const size_t cb = (size_t)D * (I / 2);
    float e[T];
#pragma unroll
    for (int t = 0; t < T; ++t) e[t] = 0.f;
    row_dot<T>(w2 + (size_t)d * (I / 2), w2 + cb + (size_t)d * (I / FP4_BLOCK), hl, I, e);
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const float es = wave_sum(e[t]);
        if (lane == t && t < ch.nrows) a.e_rows[(size_t)(ch.row0 + t) * D + d] = es;
    }
}

bool fp4_supported(int D, int I) {
    // a row fits MAXP pieces per lane; the row tiles divide both dims
    return D % 256 == 0 && I % 256 == 0 && D <= MAXP * 64 * FP4_BLOCK && I <= MAXP * 64 * FP4_BLOCK;
}

template <int T>
static hipError_t launch_fp4_t(const ExpertArgs& a, int max_chunks, bool gateup, hipStream_t st) {
    if (gateup)
        return launch_kernel(fp4_gateup_kernel<T>, max_chunks * (a.I / FP4_WAVES), FP4_WAVES * 64,
                             (size_t)T * a.D * 2, st, a);
    return launch_kernel(fp4_down_kernel<T>, max_chunks * (a.D / FP4_WAVES), FP4_WAVES * 64, (size_t)T * a.I * 2,
                         st, a);
}

hipError_t launch_fp4(const ExpertArgs& a, int rows_max, int max_chunks, bool gateup, hipStream_t st) {
    if (max_chunks <= 0) return hipSuccess;
    if (rows_max <= 1) return launch_fp4_t<1>(a, max_chunks, gateup, st);
    if (rows_max <= 2) return launch_fp4_t<2>(a, max_chunks, gateup, st);
    if (rows_max <= 4) return launch_fp4_t<4>(a, max_chunks, gateup, st);
    return launch_fp4_t<8>(a, max_chunks, gateup, st);
}

}  // namespace moe
