// Device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int QK = 256;          // weights per K-quant superblock
constexpr int Q2K_BYTES = 84;    // scales[16] | qs[64] | d | dmin
constexpr int Q3K_BYTES = 110;   // hmask[32] | qs[64] | scales[12] | d
constexpr int QB = 32;           // values per q8_1 block
constexpr int GEMV_ROWS = 8;     // token rows per GEMV chunk

// Slot layout of a K-quant matrix (rows x nsb superblocks of B bytes): panels of
// PANEL consecutive rows; a panel holds its rows' superblock 0, then their
// superblock 1, and so on. A tile of whole panels is one contiguous byte
// range (as in plain row order), and each superblock column of a panel is one
// contiguous run of PANEL * B bytes.
constexpr int PANEL = 8;

// Byte offset of superblock s of row r from the start of r's panel group
// (r counted from a panel boundary).
MOE_DEV __host__ int panel_off(int r, int s, int nsb, int B) {
    return ((r / PANEL) * nsb + s) * PANEL * B + (r % PANEL) * B;
}

// MXFP4 slot layout: a matrix [rows, K] is stored in tiles of 64 rows x 128
// columns, tile (rows 64i.., columns 128s..) at index i * (K / 128) + s. A tile's
// code bytes are its 64 rows x 64 bytes, row after row (4096 bytes per tile);
// after all codes come the scale bytes, 64 rows x 4 per tile in the same order.
// Piece p of row r is the 16 code bytes and the scale of weights 32p..32p+31.
MOE_DEV __host__ size_t fp4_code_off(int r, int p, int K) {
    return ((size_t)((r >> 6) * (K >> 7) + (p >> 2)) * 64 + (r & 63)) * 64 + (p & 3) * 16;
}
MOE_DEV __host__ size_t fp4_scale_off(int r, int p, int K) {   // from the end of the codes
    return ((size_t)((r >> 6) * (K >> 7) + (p >> 2)) * 64 + (r & 63)) * 4 + (p & 3);
}

// device error word bits (word 0 of the context's status words)
constexpr int ERR_NONFINITE = 1;
constexpr int ERR_NOTRESIDENT = 2;
// word 1 of the status words: tokens whose k-th and (k+1)-th keys were a near
// tie (an unsigned count, added to by the top-k kernels)
constexpr int ERR_NEAR_TIES = 1;
constexpr int STATUS_WORDS = 2;
// slot-table entries: >= 0 a slot; -1 not resident (an error when picked);
// SLOT_SKIP: picked, but computed in another slot wave of this call (the kernels skip it)
constexpr int SLOT_NONE = -1;
constexpr int SLOT_SKIP = -2;

// One unit of expert work: up to GEMV_ROWS token rows of one expert.
// expert >= 0: routed expert; row0 is a position in the expert-sorted pair list.
// expert == -1: the shared expert; row0 is a token index.
struct Chunk {
    int32_t expert;   // routed expert id, or -1 for the K-quant shared expert
    int32_t row0;     // first position (routed: in expert-sorted pick order; shared: token)
    int32_t nrows;
    int32_t slot;     // decode chunks: the expert's slot when the chunk was made (-1: not resident)
    int32_t token;    // decode chunks (one row each): the row's token
    float weight;     // decode chunks: the row's routing weight (1 for the shared expert)
    int32_t pad0, pad1;
};

// Everything the expert kernels read and write.
struct ExpertArgs {
    const Chunk* chunks;
    const int32_t* n_chunks;
    const int32_t* perm;        // position -> pair (token * topk + pick)
    const int32_t* inv;         // pair -> position (its chunk, on the small-batch routing)
    int32_t topk;
    const int32_t* slot_table;  // expert -> slot or -1
    const uint8_t* arena;
    size_t slot_bytes, off_w1, off_w3, off_w2;
    const uint8_t* sh_w1;       // K-quant shared expert (NULL when bf16 / none)
    const uint8_t* sh_w3;
    const uint8_t* sh_w2;
    const uint16_t* x16;        // bf16 x [m, D] (MXFP4 experts read it unquantised)
    const int8_t* xq;           // q8_1 of x: int8 [m, D], d f32 [m, D/32], 16-sums i32 [m, D/16]
    const float* xd;
    const int32_t* xs16;
    const float* xs16f;         // fp16(d) * (sum of each 16 quants) of x, f32 [m, D/16] (decode min term)
    const uint16_t* xs16b;      // the same values split into three bf16 planes per superblock (MMQ min term):
                                // [m][D/256][hi 16 | mid 16 | lo 16], hi + mid + lo exactly the f32 value
    float* h_routed;            // f32 [pairs, I] in position order (bf16 [pairs, I] for MXFP4 experts)
    float* h_shared;            // f32 [m, I]
    int8_t* hq_routed;          // q8_1 of h_routed: int8 [pairs, I], d f32 [pairs, I/32], 16-sums i32 [pairs, I/16]
    float* hd_routed;
    int32_t* hs_routed;
    int8_t* hq_shared;          // q8_1 of h_shared (K-quant shared expert): [m, I] ...
    float* hd_shared;
    int32_t* hs_shared;
    float* e_rows;              // f32 [pairs, D] in position order
    float* ys;                  // f32 [m, D]
    uint8_t* hrec;              // decode path: q8_1 record of each h row, [quants I | d f32 I/32 | 16-sums i32 I/16]
    int32_t D, I;
    float limit;
    int32_t* err;
};

MOE_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
MOE_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// nearest-even f32 -> bf16 (NaN not special-cased)
MOE_DEV uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

MOE_DEV float half_bits_to_f32(uint32_t h) {
    _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
    return (float)v;
}

MOE_DEV float round_to_fp16(float f) { return (float)(_Float16)f; }

MOE_DEV int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// (hi:lo) >> sh for sh in {0, 16}
MOE_DEV uint32_t funnel(uint32_t hi, uint32_t lo, uint32_t sh) {
    return __builtin_amdgcn_alignbit(hi, lo, sh);
}

// Clamped SwiGLU: g <= L, -L <= u <= L when L > 0; h = g * sigmoid(g) * u.
MOE_DEV float swiglu(float g, float u, float limit) {
    if (limit > 0.f) {
        g = fminf(g, limit);
        u = fminf(fmaxf(u, -limit), limit);
    }
    return g / (1.0f + expf(-g)) * u;
}

// q8_1 of 32 f32 values held by one lane: d = amax / 127 (IEEE division),
// q = round-half-away(v / d) with the unrounded d, 0 when d == 0.
// Outputs the packed int8 quants, fp16(d) as f32, and the sums of the two
// 16-value halves of q.
MOE_DEV void q8_1_block(const float* v, uint32_t* q, float& d16, int& s_lo, int& s_hi) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    const float d = amax / 127.0f;
    int sl = 0, sh = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        uint32_t packed = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int qi = (d == 0.f) ? 0 : (int)roundf(v[4 * c + b] / d);
            packed |= ((uint32_t)(qi & 0xFF)) << (8 * b);
            if (c < 4) sl += qi; else sh += qi;
        }
        q[c] = packed;
    }
    d16 = round_to_fp16(d);
    s_lo = sl;
    s_hi = sh;
}

// DPP lane moves (GFX9 encodings): quad permutes, and a rotate by 4 inside a 16-lane row
MOE_DEV float dpp_quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
MOE_DEV float dpp_quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
MOE_DEV float dpp_row_ror4(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, true));
}

// Sum over each aligned group of 8 lanes; the result is valid in lanes 4..7 of the group.
MOE_DEV float group8_sum(float v) {
    v += dpp_quad_xor1(v);
    v += dpp_quad_xor2(v);
    v += dpp_row_ror4(v);
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wavefront with DPP row shifts
// and row broadcasts; lanes a move does not reach (outside the row, or rows the
// row mask leaves out) add 0.
template <int CTRL, int ROW_MASK>
MOE_DEV int dpp_or_zero(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}
MOE_DEV int wave_inclusive_scan(int v) {
    v += dpp_or_zero<0x111, 0xF>(v);   // row_shr:1
    v += dpp_or_zero<0x112, 0xF>(v);   // row_shr:2
    v += dpp_or_zero<0x114, 0xF>(v);   // row_shr:4
    v += dpp_or_zero<0x118, 0xF>(v);   // row_shr:8
    v += dpp_or_zero<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_or_zero<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return v;
}

// 16 bytes per lane from global memory straight into LDS (gfx950 global_load_lds_dwordx4).
// `lds` must be the same in every lane of the wave: lane l writes lds + 16 l.
// The load counts as a vector-memory load of the issuing wave (vmcnt).
MOE_DEV void load_lds16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// 4 bytes per lane from global memory straight into LDS (lane l writes lds + 4 l).
MOE_DEV void load_lds4(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (they complete in issue order); a compiler fence keeps LDS reads after it.
template <int N>
MOE_DEV void wait_vm_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations,
// leaves global loads (including loads into LDS) in flight.
MOE_DEV void barrier_lds() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt not waited
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroups are dispatched to the 8 XCDs round-robin by id (block b on XCD
// b % 8). The grid is sized for the most chunks a call can have; the nb_act
// blocks that have work this call are split into 8 contiguous ranges, one per
// XCD, so that every XCD gets an equal share and the tiles of one chunk sit on
// one XCD, whose L2 then holds the chunk's activation rows. Blocks past their
// XCD's range get nb_act (no work).
MOE_DEV int xcd_logical_block(int b, int nb_act) {
    const int per = (nb_act + 7) >> 3;
    const int i = b >> 3;
    return i < per ? min((b & 7) * per + i, nb_act) : nb_act;
}

// A raw buffer resource over [p, p + bytes) (bytes < 2^32): a load through it whose
// lane offset lies past the end returns zeros instead of reading memory. p and
// bytes must be the same in every lane of the wavefront: they are taken from the
// first active lane, so that the resource sits in scalar registers.
MOE_DEV __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), 0, n, 0x00020000);
}
// 16 bytes at byte offset `off` (a multiple of 16) of a buffer resource
MOE_DEV uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16 bytes per lane at byte offset `off` of a buffer resource straight into LDS (lane
// l writes lds + 16 l; lds is the same in every lane); past the end, zeros land
MOE_DEV void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)off, 0, 0, 0);
}

MOE_DEV float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

}  // namespace moe
