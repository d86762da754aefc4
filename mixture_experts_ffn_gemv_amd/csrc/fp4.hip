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

// ------------------------------------------------------------------ batched (matrix cores)
// Above 8 tokens the chunks of the MMQ size classes run on v_mfma_f32_16x16x32_bf16:
// the weights are the A operand (16 rows per wavefront, 64 per workgroup), the
// chunk's token rows the B operand (NS sub-tiles of 16). Per 128-wide K stage the
// workgroup's code bytes and scale bytes and the chunk's bf16 rows go from global
// memory straight into LDS (global-to-LDS loads, double-buffered); a lane turns
// its 8 weights of a 32-block (4 code bytes) into the bf16 A operand with the
// scaled conversion, so the block scale costs nothing beyond the conversion.

namespace {
constexpr int FM_ROWS = 64;    // weight rows per workgroup
constexpr int FM_K = 128;      // K per stage: 4 blocks of 32

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

template <int NS, int NM>
struct FmLds {   // per buffer: NM matrices' codes [m][row][64 B], scales [m][row][4 B], rows [R][256 B]
    static constexpr int R = NS * 16;
    static constexpr int codes = NM * FM_ROWS * (FM_K / 2);
    static constexpr int sc_off = codes;
    static constexpr int x_off = sc_off + NM * FM_ROWS * 4;
    static constexpr int buf = x_off + R * FM_K * 2;
    static constexpr int bytes = 2 * buf;
};

// the A operand: 8 weights (4 code bytes, one 32-block's scale) as bf16
MOE_DEV bf16x8_t fp4_operand(uint32_t codes, float sc) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    u4 w;
    w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
    w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
    w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
    w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
    return __builtin_bit_cast(bf16x8_t, w);
}

// One stage's loads into buffer `buf`: NM matrices' 64 rows x 64 code bytes and 4 scale
// bytes from rows r0.. of each matrix (codes then scales, row length K), and the R
// bf16 rows' 128 values from `xrow` (one pointer per 16-byte unit of this thread).
template <int NS, int NM>
MOE_DEV void fm_stage(uint8_t* buf, const uint8_t* const (&mat)[NM], int r0, int K, int Rows, int kt,
                      const uint16_t* const (&xsrc)[NS]) {
    using LL = FmLds<NS, NM>;
    const int tid = threadIdx.x, wv = tid >> 6;
    const size_t cb = (size_t)Rows * (K / 2);
#pragma unroll
    for (int u = 0; u < NM; ++u) {   // unit p = 256 u + tid: matrix u, row (tid / 4), 16-byte chunk tid % 4
        const int row = tid >> 2, c = tid & 3;
        load_lds16(mat[u] + (size_t)(r0 + row) * (K / 2) + kt * (FM_K / 2) + c * 16,
                   buf + (u * 256 + wv * 64) * 16);
    }
    if (tid < NM * FM_ROWS) {        // a lane per (matrix, row): its 4 scale bytes
        const int m = tid / FM_ROWS, row = tid % FM_ROWS;
        load_lds4(mat[m] + cb + (size_t)(r0 + row) * (K / 32) + kt * 4, buf + LL::sc_off + (wv * 64) * 4);
    }
#pragma unroll
    for (int u = 0; u < NS; ++u)     // unit p = 256 u + tid: token row p / 16, 16-byte chunk p % 16
        load_lds16(xsrc[u] + kt * FM_K, buf + LL::x_off + (u * 256 + wv * 64) * 16);
}
}  // namespace

template <int NS>
__global__ __launch_bounds__(256) void fp4_mmq_gateup_kernel(ExpertArgs a, int nb) {
    extern __shared__ __align__(16) uint8_t smem[];
    using LL = FmLds<NS, 2>;
    const int D = a.D, I = a.I;
    const int tiles = I / FM_ROWS;
    const int nb_act = min(nb, *a.n_chunks * tiles);
    const int lb = xcd_logical_block(blockIdx.x, nb_act);
    if (lb >= nb_act) return;
    const int c = lb / tiles, rt = lb % tiles;
    const Chunk ch = a.chunks[c];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, g = lane >> 4;
    const int r0 = rt * FM_ROWS;
    uint16_t* h = reinterpret_cast<uint16_t*>(a.h_routed);   // bf16 [pairs, I]
    bool skip;
    const uint8_t* base = chunk_slice(a, ch, skip);
    if (skip) return;
    if (base == nullptr) {
        if (tid == 0 && rt == 0) atomicOr(a.err, ERR_NOTRESIDENT);
        for (int q = tid; q < FM_ROWS * ch.nrows; q += 256)
            h[(size_t)(ch.row0 + q / FM_ROWS) * I + r0 + q % FM_ROWS] = 0;
        return;
    }
    const uint8_t* const mat[2] = {base + a.off_w1, base + a.off_w3};
    // this thread's token-row units: row (256 u + tid) / 16 (rows past the chunk repeat its last)
    const uint16_t* xsrc[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int p = u * 256 + tid, t = min(p / 16, ch.nrows - 1);
        xsrc[u] = a.x16 + (size_t)(a.perm[ch.row0 + t] / a.topk) * D + (p % 16) * 8;
    }
    const int ns = min(NS, (ch.nrows + 15) / 16);
    f4_t accg[NS], accu[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) accg[s] = accu[s] = (f4_t){0.f, 0.f, 0.f, 0.f};
    const int nk = D / FM_K;
    const int row = 16 * wv + l16;
    fm_stage<NS, 2>(smem, mat, r0, D, I, 0, xsrc);
    for (int kt = 0; kt < nk; ++kt) {
        wait_vm_loads<0>();   // stage kt is in LDS ...
        barrier_lds();        // ... for every wave; the other buffer is free
        const uint8_t* buf = smem + (kt & 1) * LL::buf;
        if (kt + 1 < nk) fm_stage<NS, 2>(smem + ((kt + 1) & 1) * LL::buf, mat, r0, D, I, kt + 1, xsrc);
        const uint32_t sw1 = reinterpret_cast<const uint32_t*>(buf + LL::sc_off)[row];
        const uint32_t sw3 = reinterpret_cast<const uint32_t*>(buf + LL::sc_off)[FM_ROWS + row];
#pragma unroll
        for (int b = 0; b < 4; ++b) {   // 32-block b of the stage: this lane's K values 8g..8g+7
            const uint32_t c1 = reinterpret_cast<const uint32_t*>(buf)[row * 16 + 4 * b + g];
            const uint32_t c3 = reinterpret_cast<const uint32_t*>(buf)[(FM_ROWS + row) * 16 + 4 * b + g];
            const bf16x8_t A1 = fp4_operand(c1, e8m0_scale((sw1 >> (8 * b)) & 255u));
            const bf16x8_t A3 = fp4_operand(c3, e8m0_scale((sw3 >> (8 * b)) & 255u));
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (s >= ns) break;
                const bf16x8_t B = *reinterpret_cast<const bf16x8_t*>(
                    buf + LL::x_off + (size_t)(16 * s + l16) * (FM_K * 2) + (32 * b + 8 * g) * 2);
                accg[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, accg[s], 0, 0, 0);
                accu[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A3, B, accu[s], 0, 0, 0);
            }
        }
    }
    wait_vm_loads<0>();   // no load into LDS outlives the workgroup
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int t = 16 * s + l16;
        if (t < ch.nrows) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                h[(size_t)(ch.row0 + t) * I + r0 + 16 * wv + 4 * g + i] =
                    (uint16_t)f32_to_bf16(swiglu(accg[s][i], accu[s][i], a.limit));
        }
    }
}

template <int NS>
__global__ __launch_bounds__(256) void fp4_mmq_down_kernel(ExpertArgs a, int nb) {
    extern __shared__ __align__(16) uint8_t smem[];
    using LL = FmLds<NS, 1>;
    const int D = a.D, I = a.I;
    const int tiles = D / FM_ROWS;
    const int nb_act = min(nb, *a.n_chunks * tiles);
    const int lb = xcd_logical_block(blockIdx.x, nb_act);
    if (lb >= nb_act) return;
    const int c = lb / tiles, rt = lb % tiles;
    const Chunk ch = a.chunks[c];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, g = lane >> 4;
    const int r0 = rt * FM_ROWS;
    bool skip;
    const uint8_t* base = chunk_slice(a, ch, skip);
    if (skip) return;
    if (base == nullptr) {
        for (int q = tid; q < FM_ROWS * ch.nrows; q += 256)
            a.e_rows[(size_t)(ch.row0 + q / FM_ROWS) * D + r0 + q % FM_ROWS] = 0.f;
        return;
    }
    const uint8_t* const mat[1] = {base + a.off_w2};
    const uint16_t* hb = reinterpret_cast<const uint16_t*>(a.h_routed);
    const uint16_t* xsrc[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int p = u * 256 + tid, t = min(p / 16, ch.nrows - 1);
        xsrc[u] = hb + (size_t)(ch.row0 + t) * I + (p % 16) * 8;
    }
    const int ns = min(NS, (ch.nrows + 15) / 16);
    f4_t acc[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = (f4_t){0.f, 0.f, 0.f, 0.f};
    const int nk = I / FM_K;
    const int row = 16 * wv + l16;
    fm_stage<NS, 1>(smem, mat, r0, I, D, 0, xsrc);
    for (int kt = 0; kt < nk; ++kt) {
        wait_vm_loads<0>();
        barrier_lds();
        const uint8_t* buf = smem + (kt & 1) * LL::buf;
        if (kt + 1 < nk) fm_stage<NS, 1>(smem + ((kt + 1) & 1) * LL::buf, mat, r0, I, D, kt + 1, xsrc);
        const uint32_t sw = reinterpret_cast<const uint32_t*>(buf + LL::sc_off)[row];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t c2 = reinterpret_cast<const uint32_t*>(buf)[row * 16 + 4 * b + g];
            const bf16x8_t A = fp4_operand(c2, e8m0_scale((sw >> (8 * b)) & 255u));
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (s >= ns) break;
                const bf16x8_t B = *reinterpret_cast<const bf16x8_t*>(
                    buf + LL::x_off + (size_t)(16 * s + l16) * (FM_K * 2) + (32 * b + 8 * g) * 2);
                acc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, acc[s], 0, 0, 0);
            }
        }
    }
    wait_vm_loads<0>();
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int t = 16 * s + l16;
        if (t < ch.nrows) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a.e_rows[(size_t)(ch.row0 + t) * D + r0 + 16 * wv + 4 * g + i] = acc[s][i];
        }
    }
}

bool fp4_mmq_supported(int D, int I) { return D % FM_K == 0 && I % FM_K == 0 && D % FM_ROWS == 0 && I % FM_ROWS == 0; }

template <int NS>
static hipError_t launch_fp4_mmq_ns(const ExpertArgs& a, int max_chunks, bool gateup, hipStream_t st) {
    const int nb = max_chunks * (gateup ? a.I / FM_ROWS : a.D / FM_ROWS);
    const int nb_pad = (nb + 7) / 8 * 8;
    if (gateup) return launch_kernel(fp4_mmq_gateup_kernel<NS>, nb_pad, 256, (size_t)FmLds<NS, 2>::bytes, st, a, nb);
    return launch_kernel(fp4_mmq_down_kernel<NS>, nb_pad, 256, (size_t)FmLds<NS, 1>::bytes, st, a, nb);
}

hipError_t launch_fp4_mmq(const ExpertArgs& a, const ChunkPlan& plan, bool gateup, hipStream_t st) {
    for (int c = 0; c < MMQ_CLASSES; ++c) {
        if (plan.cap[c] <= 0) continue;
        ExpertArgs ac = a;
        ac.chunks = a.chunks + plan.base[c];
        ac.n_chunks = a.n_chunks + c;
        const hipError_t e = c == 0   ? launch_fp4_mmq_ns<1>(ac, plan.cap[c], gateup, st)
                             : c == 1 ? launch_fp4_mmq_ns<2>(ac, plan.cap[c], gateup, st)
                                      : launch_fp4_mmq_ns<4>(ac, plan.cap[c], gateup, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
