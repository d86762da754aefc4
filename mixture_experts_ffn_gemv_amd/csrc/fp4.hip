// Routed experts in MXFP4, the upstream checkpoint's own format (Open Model
// Atlas, "DeepSeek V4.1 · Mixture of experts": the experts' Linear layers hold
// float4_e2m1fn_x2 weights; config.json expert_dtype "fp4"). The pages give the
// element type only; the scales follow the OCP microscaling layout: per 32
// consecutive weights of a row one E8M0 scale 2^(E-127), each weight an e2m1
// code, two per byte (the even weight in the low nibble). In plain order a matrix
// [rows, cols] is its codes [rows, cols/2] followed by its scales [rows, cols/32];
// an expert slice is [W1 | W3 | W2]. A slot holds each matrix in tiles of 64 rows
// x 128 columns (fp4_code_off / fp4_scale_off; moe_pack_expert writes them): a
// tile's 4096 code bytes are one contiguous run, so the batched kernel reads
// each K stage of its 64 rows as one block of HBM rather than 64 pieces 64
// bytes long, one per row (which left it near half the streaming rate).
//
// The activations stay bf16, as in the excerpt's Linear layers: a lane turns 4
// code bytes (8 weights of one 32-weight block) into a bf16 matrix-core operand
// with the gfx950 scaled conversion (exact: the codes have two significant bits
// and the scale is a power of two), and v_mfma_f32_16x16x32_bf16 takes 16 weight
// rows against 16 token rows (f32 accumulation). h is rounded to bf16 before W2.
//
// A chunk holds token rows of one expert (positions row0.. in expert-sorted pick
// order). Two kernels per matrix pair:
//  fp4_gemv_kernel<NM, T, SPW>: chunks of at most T <= 8 rows (decode, small batches); a
//      workgroup per 16 weight rows, its wavefronts splitting K, each with all
//      of its loads in flight at once; partial tiles summed in LDS.
//  fp4_mmq_kernel<NS, DOWN>: the MMQ size classes above 8 tokens; a workgroup
//      per 64 rows of W1 and of W3 (gate/up) or per 128 rows of W2 (down),
//      streaming K through double-buffered LDS.
// Gate/up (NM = 2) holds W1 and W3 rows side by side, so the clamped SwiGLU
// needs no exchange, and writes h bf16 [pairs, I]; down (NM = 1) writes E f32
// [pairs, D], summed per token by the combine kernel.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int FP4_BLOCK = 32;    // weights per E8M0 scale, and per lane piece (16 code bytes)

MOE_DEV float e8m0_scale(uint32_t e) { return e == 255u ? __builtin_nanf("") : ldexpf(1.f, (int)e - 127); }

// the expert's slice, or nullptr (with the chunk's outputs to be zeroed or skipped)
MOE_DEV const uint8_t* chunk_slice(const ExpertArgs& a, const Chunk& ch, bool& skip) {
    const int slot = a.slot_table[ch.expert];
    skip = slot == SLOT_SKIP;   // computed in another slot wave
    if (skip || slot < 0) return nullptr;
    return a.arena + (size_t)slot * a.slot_bytes;
}

}  // namespace

// ------------------------------------------------------------------ batched (matrix cores)
// Above 8 tokens the chunks of the MMQ size classes run on v_mfma_f32_16x16x32_bf16:
// the weights are the A operand (16 rows per wavefront, 64 per workgroup), the
// chunk's token rows the B operand (NS sub-tiles of 16). Per 128-wide K stage the
// workgroup's code bytes and scale bytes and the chunk's bf16 rows go from global
// memory straight into LDS (global-to-LDS loads, double-buffered). Lane group g
// (lanes 16g..16g+15) owns 32-block g of the stage: one 16-byte LDS read gives a
// lane its row's whole block, and MFMA step j takes the block's weights 8j..8j+7
// (the sum over K does not depend on which step adds which term), so the B
// operand of lane (t, g) at step j is token t's values 32g+8j..32g+8j+7. The
// scaled conversion turns 4 code bytes into the bf16 A operand with the block
// scale applied, so the scale costs nothing beyond the conversion.
// LDS banks: the 16 lanes of a group read one block from each of 16 rows, so code
// block c of row r is stored at slot c ^ ((r >> 2) & 3) of the row's 64 bytes; token
// rows are 256 bytes, so 16-byte chunk c of row t is stored at chunk c ^ (t & 15).
// Either way the 16 reads of a lane group fall on distinct banks.

namespace {
constexpr int FM_ROWS = 64;    // weight rows per workgroup
constexpr int FM_K = 128;      // K per stage: 4 blocks of 32

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int NS, int NM>
struct FmLds {   // per buffer: NM matrices' codes [m][row][64 B], scales [m][row][4 B], rows [R][256 B]
    static constexpr int R = NS * 16;
    static constexpr int codes = NM * FM_ROWS * (FM_K / 2);
    static constexpr int sc_off = codes;
    static constexpr int x_off = sc_off + NM * FM_ROWS * 4;
    static constexpr int buf = x_off + R * FM_K * 2;
    static constexpr int bytes = 2 * buf;
};

// the A operand: 8 weights (4 code bytes of one 32-block, its scale) as bf16
MOE_DEV bf16x8_t fp4_operand(uint32_t codes, float sc) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    u4 w;
    w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 0));
    w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 1));
    w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 2));
    w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, sc, 3));
    return __builtin_bit_cast(bf16x8_t, w);
}

// One stage's loads into buffer `buf`: NM 64-row tiles' 64 x 64 code bytes and 4 scale
// bytes per row (tile u: codes from cm[u], scales from sm[u], at rows r0.. of a
// matrix with rows of K weights), and the R bf16 rows' 128 values from `xsrc` (one
// pointer per 16-byte unit of this thread, already pointing at the swizzled chunk
// its LDS slot holds).
template <int NS, int NM>
MOE_DEV void fm_stage(uint8_t* buf, const uint8_t* const (&cm)[NM], const uint8_t* const (&sm)[NM], int r0, int K,
                      int kt, const uint16_t* const (&xsrc)[NS]) {
    using LL = FmLds<NS, NM>;
    const int tid = threadIdx.x, wv = tid >> 6;
#pragma unroll
    for (int u = 0; u < NM; ++u) {   // unit p = 256 u + tid: tile u, row tid / 4, slot tid % 4 (swizzled block)
        const int row = tid >> 2, c = (tid & 3) ^ ((row >> 2) & 3);
        load_lds16(cm[u] + fp4_code_off(r0 + row, 4 * kt + c, K), buf + (u * 256 + wv * 64) * 16);
    }
    if (tid < NM * FM_ROWS) {        // a lane per (tile, row): its 4 scale bytes
        const int m = tid / FM_ROWS, row = tid % FM_ROWS;
        load_lds4(sm[m] + fp4_scale_off(r0 + row, 4 * kt, K), buf + LL::sc_off + (wv * 64) * 4);
    }
#pragma unroll
    for (int u = 0; u < NS; ++u)     // unit p = 256 u + tid: token row p / 16, 16-byte chunk p % 16
        load_lds16(xsrc[u] + kt * FM_K, buf + LL::x_off + (u * 256 + wv * 64) * 16);
}
}  // namespace

// Gate/up (DOWN false): tile 0 is 64 rows of W1, tile 1 the same rows of W3, the
// B operand the tokens' x rows, and h = bf16(SwiGLU) of the two. Down (DOWN true):
// tiles 0 and 1 are 128 consecutive rows of W2 (r0.. and r0 + 64..), the B operand
// the chunk's bf16 h rows, and both tiles' products go to E f32 [pairs, D].
template <int NS, bool DOWN>
__global__ __launch_bounds__(256) void fp4_mmq_kernel(ExpertArgs a, int nb) {
    extern __shared__ __align__(16) uint8_t smem[];
    using LL = FmLds<NS, 2>;
    const int D = a.D, I = a.I;
    const int Rows = DOWN ? D : I, K = DOWN ? I : D;
    const int rows_wg = DOWN ? 2 * FM_ROWS : FM_ROWS;
    const int tiles = Rows / rows_wg;
    const int nb_act = min(nb, *a.n_chunks * tiles);
    const int lb = xcd_logical_block(blockIdx.x, nb_act);
    if (lb >= nb_act) return;
    const int c = lb / tiles, rt = lb % tiles;
    const Chunk ch = a.chunks[c];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, l16 = lane & 15, g = lane >> 4;
    const int r0 = rt * rows_wg;
    uint16_t* h = reinterpret_cast<uint16_t*>(a.h_routed);   // bf16 [pairs, I]
    bool skip;
    const uint8_t* base = chunk_slice(a, ch, skip);
    if (skip) return;
    if (base == nullptr) {   // not resident: flag it (gate/up), and the outputs are zero
        if (!DOWN && tid == 0 && rt == 0) atomicOr(a.err, ERR_NOTRESIDENT);
        for (int q = tid; q < rows_wg * ch.nrows; q += 256) {
            const size_t o = (size_t)(ch.row0 + q / rows_wg) * Rows + r0 + q % rows_wg;
            if (DOWN) a.e_rows[o] = 0.f;
            else h[o] = 0;
        }
        return;
    }
    const size_t cb = (size_t)Rows * (K / 2);   // code bytes of a matrix (its scales follow)
    const uint8_t* cm[2];
    const uint8_t* sm[2];
    if (DOWN) {   // the second tile: one tile row further on, in the codes and in the scales
        cm[0] = base + a.off_w2;
        cm[1] = cm[0] + (size_t)(K / FM_K) * 4096;
        sm[0] = cm[0] + cb;
        sm[1] = sm[0] + (size_t)(K / FM_K) * 256;
    } else {
        cm[0] = base + a.off_w1;
        cm[1] = base + a.off_w3;
        sm[0] = cm[0] + cb;
        sm[1] = cm[1] + cb;
    }
    // this thread's token-row units: LDS slot p = 256 u + tid is chunk p % 16 of row
    // t = p / 16 and holds that row's chunk (p % 16) ^ (t & 15) (rows past the chunk
    // repeat its last)
    const uint16_t* xsrc[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int p = u * 256 + tid, t = p / 16, tr = min(t, ch.nrows - 1);
        const int sw = ((p % 16) ^ (t & 15)) * 8;
        xsrc[u] = DOWN ? h + (size_t)(ch.row0 + tr) * I + sw
                       : a.x16 + (size_t)(a.perm[ch.row0 + tr] / a.topk) * D + sw;
    }
    const int ns = min(NS, (ch.nrows + 15) / 16);
    f4_t acc0[NS], acc1[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) acc0[s] = acc1[s] = (f4_t){0.f, 0.f, 0.f, 0.f};
    const int nk = K / FM_K;
    const int row = 16 * wv + l16;
    fm_stage<NS, 2>(smem, cm, sm, r0, K, 0, xsrc);
    for (int kt = 0; kt < nk; ++kt) {
        wait_vm_loads<0>();   // stage kt is in LDS ...
        barrier_lds();        // ... for every wave; the other buffer is free
        const uint8_t* buf = smem + (kt & 1) * LL::buf;
        if (kt + 1 < nk) fm_stage<NS, 2>(smem + ((kt + 1) & 1) * LL::buf, cm, sm, r0, K, kt + 1, xsrc);
        // block g of this lane's row in both tiles: 16 code bytes and a scale byte
        const int slot = g ^ ((row >> 2) & 3);   // row and FM_ROWS + row share (r >> 2) & 3
        const u32x4_t c0 = *reinterpret_cast<const u32x4_t*>(buf + (row * 4 + slot) * 16);
        const u32x4_t c1 = *reinterpret_cast<const u32x4_t*>(buf + ((FM_ROWS + row) * 4 + slot) * 16);
        const float s0 = e8m0_scale(buf[LL::sc_off + row * 4 + g]);
        const float s1 = e8m0_scale(buf[LL::sc_off + (FM_ROWS + row) * 4 + g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {   // step j: the block's weights 8j..8j+7
            const bf16x8_t A0 = fp4_operand(c0[j], s0);
            const bf16x8_t A1 = fp4_operand(c1[j], s1);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if (s >= ns) break;
                const bf16x8_t B = *reinterpret_cast<const bf16x8_t*>(
                    buf + LL::x_off + (16 * s + l16) * (FM_K * 2) + (((4 * g + j) ^ l16) * 16));
                acc0[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, acc0[s], 0, 0, 0);
                acc1[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, acc1[s], 0, 0, 0);
            }
        }
    }
    wait_vm_loads<0>();   // no load into LDS outlives the workgroup
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int t = 16 * s + l16;
        if (t < ch.nrows) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const size_t o = (size_t)(ch.row0 + t) * Rows + r0 + 16 * wv + 4 * g + i;
                if (DOWN) {
                    a.e_rows[o] = acc0[s][i];
                    a.e_rows[o + FM_ROWS] = acc1[s][i];
                } else {
                    h[o] = (uint16_t)f32_to_bf16(swiglu(acc0[s][i], acc1[s][i], a.limit));
                }
            }
        }
    }
}

// ------------------------------------------------------------------ small chunks (split K)
// A workgroup per (chunk, 16 weight rows); wavefront w takes K stages
// SPW w .. SPW w + SPW - 1 (of 128 columns), lane (l16, g) row l16 and
// block g of each stage, as in the batched kernels. All of a lane's code and
// scale loads are issued before anything waits (one contiguous 1 KB run per
// wavefront load: 16 rows x 64 bytes of a tile), then the chunk's token rows go
// into LDS (row stride K + 8 bf16), and each stage is 4 MFMA steps per matrix
// with token t's values in B column t (zero for t >= rows). The wavefronts'
// 16 x 16 partial tiles are summed in LDS.
constexpr int FG_ROWS = 16;   // weight rows per workgroup
// K stages per wavefront (at most 16 wavefronts for K <= 8192): gate/up 5 (8
// wavefronts at D = 5120), down 4, the faster of 3..6 for each at the real shape
constexpr int FG_SPW_GU = 5, FG_SPW_DN = 4;

template <int NM, int T, int SPW>
__global__ __launch_bounds__(1024) void fp4_gemv_kernel(ExpertArgs a, int nb) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int D = a.D, I = a.I;
    const int Rows = NM == 2 ? I : D, K = NM == 2 ? D : I;
    const int tiles = Rows / FG_ROWS;
    const int nb_act = min(nb, *a.n_chunks * tiles);
    const int lb = xcd_logical_block(blockIdx.x, nb_act);
    if (lb >= nb_act) return;
    const int c = lb / tiles, r0 = (lb % tiles) * FG_ROWS;
    const Chunk ch = a.chunks[c];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, nw = blockDim.x >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    uint16_t* h = reinterpret_cast<uint16_t*>(a.h_routed);   // bf16 [pairs, I]
    bool skip;
    const uint8_t* base = chunk_slice(a, ch, skip);
    if (skip) return;
    if (base == nullptr) {   // not resident: flag it, and its outputs are zero
        if (NM == 2 && tid == 0 && r0 == 0) atomicOr(a.err, ERR_NOTRESIDENT);
        for (int q = tid; q < FG_ROWS * ch.nrows; q += blockDim.x) {
            const size_t o = (size_t)(ch.row0 + q / FG_ROWS) * Rows + r0 + q % FG_ROWS;
            if (NM == 2) h[o] = 0;
            else a.e_rows[o] = 0.f;
        }
        return;
    }
    const int nk = K / FM_K, row = r0 + l16;
    const size_t cb = (size_t)Rows * (K / 2);
    const uint8_t* mat[NM];
    mat[0] = base + (NM == 2 ? a.off_w1 : a.off_w2);
    if (NM == 2) mat[NM - 1] = base + a.off_w3;
    u32x4_t q[NM][SPW];
    uint32_t e[NM][SPW];
#pragma unroll
    for (int s = 0; s < SPW; ++s) {   // stages past K repeat the last one (in bounds, not used)
        const int st = min(wv * SPW + s, nk - 1);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            q[m][s] = *reinterpret_cast<const u32x4_t*>(mat[m] + fp4_code_off(row, 4 * st + g, K));
            e[m][s] = mat[m][cb + fp4_scale_off(row, 4 * st + g, K)];
        }
    }
    // the chunk's token rows (T >= rows): thread i moves 8 values at units i and
    // i + blockDim of each (the workgroup has 64 ceil(nk / SPW) >= K / (8 XU)
    // threads; loads past the rows or past K repeat the last, in bounds and unused)
    constexpr int XU = (SPW + 3) / 4;
    const int ld = K + 8, k8 = K / 8, bd = blockDim.x;
    uint16_t* xl = reinterpret_cast<uint16_t*>(smem);
    uint4 xr[T][XU];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int tr = ch.row0 + min(t, ch.nrows - 1);
        const uint16_t* src = NM == 2 ? a.x16 + (size_t)(a.perm[tr] / a.topk) * D : h + (size_t)tr * I;
#pragma unroll
        for (int j = 0; j < XU; ++j) xr[t][j] = reinterpret_cast<const uint4*>(src)[min(tid + j * bd, k8 - 1)];
    }
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int j = 0; j < XU; ++j) {
            const int u = tid + j * bd;
            if (t < ch.nrows && u < k8) *reinterpret_cast<uint4*>(xl + t * ld + 8 * u) = xr[t][j];
        }
    __syncthreads();
    f4_t acc[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) acc[m] = (f4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
        const int st = wv * SPW + s;
        if (st >= nk) break;   // uniform per wavefront
        float sc[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) sc[m] = e8m0_scale(e[m][s]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8_t B = {};
            if (l16 < T && l16 < ch.nrows)
                B = *reinterpret_cast<const bf16x8_t*>(xl + l16 * ld + FM_K * st + 32 * g + 8 * j);
#pragma unroll
            for (int m = 0; m < NM; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp4_operand(q[m][s][j], sc[m]), B, acc[m], 0, 0, 0);
        }
    }
    // lane (l16, g) holds rows 4g..4g+3 of column l16; the token rows are done with
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);   // [wavefront][matrix][row 16][column 16]
    if (l16 < T && l16 < ch.nrows) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[((wv * NM + m) * 16 + 4 * g + i) * 16 + l16] = acc[m][i];
    }
    __syncthreads();
    for (int qq = tid; qq < FG_ROWS * ch.nrows; qq += blockDim.x) {
        const int rr = qq % FG_ROWS, t = qq / FG_ROWS;
        float v[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            v[m] = 0.f;
            for (int w = 0; w < nw; ++w) v[m] += red[((w * NM + m) * 16 + rr) * 16 + t];
        }
        const size_t o = (size_t)(ch.row0 + t) * Rows + r0 + rr;
        if (NM == 2) h[o] = (uint16_t)f32_to_bf16(swiglu(v[0], v[NM - 1], a.limit));
        else a.e_rows[o] = v[0];
    }
}

bool fp4_mmq_supported(int D, int I) { return D % FM_K == 0 && I % FM_K == 0 && D % (2 * FM_ROWS) == 0 && I % FM_ROWS == 0; }

template <int NS>
static hipError_t launch_fp4_mmq_ns(const ExpertArgs& a, int max_chunks, bool gateup, hipStream_t st) {
    const int nb = max_chunks * (gateup ? a.I / FM_ROWS : a.D / (2 * FM_ROWS));
    const int nb_pad = (nb + 7) / 8 * 8;
    if (gateup) return launch_kernel(fp4_mmq_kernel<NS, false>, nb_pad, 256, (size_t)FmLds<NS, 2>::bytes, st, a, nb);
    return launch_kernel(fp4_mmq_kernel<NS, true>, nb_pad, 256, (size_t)FmLds<NS, 2>::bytes, st, a, nb);
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
    // the 64 x 128 slot tiles divide both dims; a workgroup stays within 16 wavefronts
    return D % 256 == 0 && I % 256 == 0 && D <= FG_SPW_GU * 16 * FM_K && I <= FG_SPW_DN * 16 * FM_K;
}

template <int T>
static hipError_t launch_fp4_t(const ExpertArgs& a, int max_chunks, bool gateup, hipStream_t st) {
    const int K = gateup ? a.D : a.I, Rows = gateup ? a.I : a.D;
    const int spw = gateup ? FG_SPW_GU : FG_SPW_DN;
    const int nw = (K / FM_K + spw - 1) / spw;   // 64 nw XU >= K / 8 (XU units per thread)
    const int nb = max_chunks * (Rows / FG_ROWS);
    const int nb_pad = (nb + 7) / 8 * 8;   // whole rounds over the 8 XCDs
    const size_t lds = std::max((size_t)T * (K + 8) * 2, (size_t)nw * (gateup ? 2 : 1) * 256 * 4);
    if (gateup) return launch_kernel(fp4_gemv_kernel<2, T, FG_SPW_GU>, nb_pad, nw * 64, lds, st, a, nb);
    return launch_kernel(fp4_gemv_kernel<1, T, FG_SPW_DN>, nb_pad, nw * 64, lds, st, a, nb);
}

hipError_t launch_fp4(const ExpertArgs& a, int rows_max, int max_chunks, bool gateup, hipStream_t st) {
    if (max_chunks <= 0) return hipSuccess;
    if (rows_max <= 1) return launch_fp4_t<1>(a, max_chunks, gateup, st);
    if (rows_max <= 2) return launch_fp4_t<2>(a, max_chunks, gateup, st);
    if (rows_max <= 4) return launch_fp4_t<4>(a, max_chunks, gateup, st);
    return launch_fp4_t<8>(a, max_chunks, gateup, st);
}

}  // namespace moe
