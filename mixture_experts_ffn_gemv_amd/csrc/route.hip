// Routing kernels: router logits, q8_1 of the input rows, the biased stable
// top-k with its weights, and the token -> expert bucketing.
//
// Semantics follow metrale's route_from_logits (moe_v41.rs source view):
// scores sqrt(softplus(z / gate_temp)) with softplus(v) = v above 20, keys
// score + bias ordered descending with ties to the lower expert id, weights the
// unbiased scores renormalised (sum + 1e-20) when norm_topk_prob and topk > 1,
// times route_scale; and the Open Model Atlas router equations for
// DeepSeek V4.1. The selection runs on the device (one wavefront per token)
// instead of the pages' host round trip.
#include <algorithm>

#include "moe_common.h"
#include "moe_internal.h"
#include "route_select.h"
#include "shared_rows.h"

namespace moe {

// one-token selection inside the router launch: bias and slot entries each router
// thread prefetches (256 threads: E <= 1024)
constexpr int M1_PREFETCH = 4;

// ---------------------------------------------------------------- router logits + q8_1(x)
// One launch, two kinds of workgroups. Blocks [0, E * ntg): router logits
// z[t, e] = sum_d x[t, d] * W_R[e, d] with f32 accumulation, one workgroup per
// (expert row, group of TT tokens); each thread walks 4-element chunks of the
// row so the row's bytes are read once per token group with coalesced loads.
// Blocks past that: q8_1 of x, one lane per 32-value block (int8 quants,
// fp16(d) as f32, and the two 16-value sums of the quants used by the Q2_K
// min term): d = amax / 127, q = round-half-away(x / d).
// v = hi + mid + lo exactly, three bf16 values (truncation splits: v's 24-bit significand
// in three 8-bit pieces), packed as the low halves of the three returned words
MOE_DEV void split3_bf16(float v, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const uint32_t vb = __float_as_uint(v);
    const float r = v - __uint_as_float(vb & 0xFFFF0000u);
    const uint32_t rb = __float_as_uint(r);
    const float l = r - __uint_as_float(rb & 0xFFFF0000u);   // at most 8 significant bits
    hi = vb >> 16;
    mid = rb >> 16;
    lo = __float_as_uint(l) >> 16;
}

MOE_DEV void quantize_block_bf16(const uint16_t* __restrict__ x, int b, int8_t* __restrict__ xq,
                                 float* __restrict__ xd, int32_t* __restrict__ xs16, float* __restrict__ xs16f = nullptr,
                                 uint16_t* __restrict__ xs16b = nullptr) {
    const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)b * QB);
    float v[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const uint4 u = src[c];
        v[8 * c + 0] = bf16_lo(u.x); v[8 * c + 1] = bf16_hi(u.x);
        v[8 * c + 2] = bf16_lo(u.y); v[8 * c + 3] = bf16_hi(u.y);
        v[8 * c + 4] = bf16_lo(u.z); v[8 * c + 5] = bf16_hi(u.z);
        v[8 * c + 6] = bf16_lo(u.w); v[8 * c + 7] = bf16_hi(u.w);
    }
    uint32_t q[8];
    float d;
    int sl, sh;
    q8_1_block(v, q, d, sl, sh);
    uint4* dst = reinterpret_cast<uint4*>(xq + (size_t)b * QB);
    dst[0] = make_uint4(q[0], q[1], q[2], q[3]);
    dst[1] = make_uint4(q[4], q[5], q[6], q[7]);
    xd[b] = d;
    if (xs16 != nullptr) {
        xs16[2 * b] = sl;
        xs16[2 * b + 1] = sh;
    }
    if (xs16f != nullptr) {   // exact: 11-bit scale times a sum of 16 quants
        xs16f[2 * b] = d * (float)sl;
        xs16f[2 * b + 1] = d * (float)sh;
    }
    if (xs16b != nullptr) {   // block b % 8 of its superblock: entries 2 (b % 8), + 1 of each plane
        uint32_t h0, m0, l0, h1, m1, l1;
        split3_bf16(d * (float)sl, h0, m0, l0);
        split3_bf16(d * (float)sh, h1, m1, l1);
        uint32_t* rec = reinterpret_cast<uint32_t*>(xs16b + (size_t)(b >> 3) * 48) + (b & 7);
        rec[0] = h0 | (h1 << 16);
        rec[8] = m0 | (m1 << 16);
        rec[16] = l0 | (l1 << 16);
    }
}

// the one-token selection by the last router workgroup (defined with the top-k
// kernels); b[i], sl[i]: bias and slot of expert threadIdx.x + 256 i
template <int KPL>
MOE_DEV void select_tail_m1(const float* scores_in, const RouteSel& ro, const float (&b)[M1_PREFETCH],
                            const int (&sl)[M1_PREFETCH]);

// the small-batch selection by one workgroup (defined with the top-k kernels)
template <int KPL, int NT, bool FROM_SCORES>
MOE_DEV void select_small(const float* src, const float* bias, int m, int E, int k, float gate_temp, int norm,
                          float route_scale, int32_t* idx, float* gw, int32_t* err, int shared_chunks,
                          int32_t* offsets, int32_t* active, int32_t* n_active, int32_t* perm, int32_t* inv,
                          Chunk* chunks, int32_t* n_chunks, const int32_t* slot_table);

// Thread 0 of router workgroup e (of E), after its scores are stored and waited
// for: counts the arrival in two levels and tells whether this workgroup was the
// last of all (the counters wrap to 0 after their last arrival).
MOE_DEV bool count_arrival(const RouteSel& ro, int e, int E) {
    const int g = e % ARRIVE_GROUPS, ng = min(E, ARRIVE_GROUPS);
    const unsigned n_in_g = (unsigned)((E - g + ARRIVE_GROUPS - 1) / ARRIVE_GROUPS);
    bool l = atomicInc(ro.arrive + ARRIVE_STRIDE * (1 + g), n_in_g - 1) == n_in_g - 1;
    if (l) l = atomicInc(ro.arrive, (unsigned)(ng - 1)) == (unsigned)(ng - 1);
    return l;
}

// KPL > 0 (the router launch also selects): each router workgroup counts its
// arrival after its scores are stored, and the last of the E to arrive runs the
// selection on all of them (no workgroup waits for another: the last one finds
// every score already written). One token: the top-k of route_m1; 2..8 tokens:
// the selection and bucketing of route_small. The count runs in two levels: workgroup e counts in group
// e % ARRIVE_GROUPS, the last of each group in the top counter (each counter on
// a cache line of its own), since increments of one address are performed one
// after another. Every router workgroup requests the bias and slot-table
// entries the selection needs at its start, so that the last one has them at hand.
template <int TT, int KPL = 0>
__global__ __launch_bounds__(512) void router_quant_kernel(const uint16_t* __restrict__ x, int m,
                                                           const uint16_t* __restrict__ wr, int D, int E, int ntg,
                                                           float* __restrict__ logits, int8_t* __restrict__ xq,
                                                           float* __restrict__ xd, int32_t* __restrict__ xs16, float* __restrict__ xs16f,
                                                           SharedRows sr, RouteSel ro) {
    const int nrouter = E * ntg, bd = blockDim.x;
    const int nq = xq == nullptr ? 0 : (m * (D / QB) + bd - 1) / bd;
    if ((int)blockIdx.x >= nrouter + nq) {   // the shared expert's gate/up rows
        shared_gateup_block(sr, blockIdx.x - nrouter - nq);
        return;
    }
    if ((int)blockIdx.x >= nrouter) {
        const int b = (blockIdx.x - nrouter) * bd + threadIdx.x;
        if (b < m * (D / QB)) quantize_block_bf16(x, b, xq, xd, xs16, xs16f);
        return;
    }
    if constexpr (TT > 1) {
        // 512 threads: thread i takes 16-byte units i and i + 512 of the expert's row
        // and of each token row (D / 8 <= 1024 units), every load requested at once
        // (units past the row and tokens past m repeat the last ones; not kept)
        constexpr int UM = 2;
        const int e = blockIdx.x % E, tid = threadIdx.x, nu = D / 8;
        const uint4* w4 = reinterpret_cast<const uint4*>(wr + (size_t)e * D);
        uint4 wv[UM], xv[UM][TT];
#pragma unroll
        for (int i = 0; i < UM; ++i) {
            const int c = min(tid + 512 * i, nu - 1);
            wv[i] = w4[c];
#pragma unroll
            for (int t = 0; t < TT; ++t) xv[i][t] = reinterpret_cast<const uint4*>(x + (size_t)min(t, m - 1) * D)[c];
        }
        float acc[TT];
#pragma unroll
        for (int t = 0; t < TT; ++t) acc[t] = 0.f;
#pragma unroll
        for (int i = 0; i < UM; ++i) {
            if (tid + 512 * i >= nu) break;
            const uint32_t w8[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const uint32_t x8[4] = {xv[i][t].x, xv[i][t].y, xv[i][t].z, xv[i][t].w};
                float a = acc[t];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    a = fmaf(bf16_lo(x8[q]), bf16_lo(w8[q]), a);
                    a = fmaf(bf16_hi(x8[q]), bf16_hi(w8[q]), a);
                }
                acc[t] = a;
            }
        }
        __shared__ float part8[8][TT];
        const int lane = tid & 63, wv8 = tid >> 6;
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            const float sm = wave_sum(acc[t]);
            if (lane == 0) part8[wv8][t] = sm;
        }
        __syncthreads();
        if constexpr (KPL > 0) {   // scores out device-coherently, as at one token
            __shared__ int last8;
            if (tid < m) {
                float z = part8[0][tid];
                for (int w = 1; w < 8; ++w) z += part8[w][tid];
                float sv, kv;
                bool bad;
                score_of(z, 0.f, ro.gate_temp, sv, kv, bad);
                __hip_atomic_store(logits + (size_t)tid * E + e, sv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __builtin_amdgcn_s_waitcnt(0);
            }
            __syncthreads();
            if (tid == 0) last8 = count_arrival(ro, e, E);
            __syncthreads();
            if (last8)
                select_small<KPL, 512, true>(logits, ro.bias, m, E, ro.k, ro.gate_temp, ro.norm, ro.route_scale, ro.idx,
                                             ro.gw, ro.err, ro.shared_chunks, ro.offsets, ro.active, ro.n_active,
                                             ro.perm, ro.inv, ro.chunks, ro.n_chunks, ro.slot_table);
            return;
        }
        if (tid < TT && tid < m) {
            float z = part8[0][tid];
            for (int w = 1; w < 8; ++w) z += part8[w][tid];
            logits[(size_t)tid * E + e] = z;
        }
        return;
    }
    // one token, 256 threads: thread i takes 16-byte units i, i + 256, i + 512 of the
    // expert's row and of x per round (768 units: rows of up to 6144 values in one
    // round), every load of a round requested at once in straight-line code (units
    // past the row read the last one and are not added)
    const int e = blockIdx.x % E;
    float pb[M1_PREFETCH];
    int psl[M1_PREFETCH];
    if constexpr (KPL > 0) {
#pragma unroll
        for (int i = 0; i < M1_PREFETCH; ++i) {
            const int ee = min((int)threadIdx.x + 256 * i, E - 1);
            pb[i] = ro.bias[ee];
            psl[i] = ro.slot_table[ee];
        }
    }
    const uint4* w4 = reinterpret_cast<const uint4*>(wr + (size_t)e * D);
    const uint4* x4 = reinterpret_cast<const uint4*>(x);
    constexpr int U1 = 3;
    const int nu = D / 8;
    float acc[TT] = {0.f};
    for (int base = 0; base < nu; base += 256 * U1) {
        uint4 xv[U1], wv[U1];
#pragma unroll
        for (int i = 0; i < U1; ++i) xv[i] = x4[min(base + (int)threadIdx.x + 256 * i, nu - 1)];
#pragma unroll
        for (int i = 0; i < U1; ++i) wv[i] = w4[min(base + (int)threadIdx.x + 256 * i, nu - 1)];
#pragma unroll
        for (int i = 0; i < U1; ++i) {
            if (base + (int)threadIdx.x + 256 * i >= nu) break;
            const uint32_t w8[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
            const uint32_t x8[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
            float a = acc[0];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                a = fmaf(bf16_lo(x8[q]), bf16_lo(w8[q]), a);
                a = fmaf(bf16_hi(x8[q]), bf16_hi(w8[q]), a);
            }
            acc[0] = a;
        }
    }
    const int t0 = 0;
    __shared__ float part[4][TT];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const float s = wave_sum(acc[t]);
        if (lane == 0) part[wv][t] = s;
    }
    __syncthreads();
    if constexpr (KPL > 0) {
        // The logit goes out as a device-coherent store (it passes every cache that
        // another XCD does not share) and the thread waits for it to complete before
        // counting its workgroup's arrival; the last workgroup reads the logits the
        // same way. (A release fence would write the whole L2 back in each of the E
        // workgroups, which costs more than the selection saves.)
        // What goes out is the expert's score sqrt(softplus(z / gate_temp)) rather than
        // its logit z: the last workgroup then adds only the bias.
        __shared__ int last;
        if (threadIdx.x == 0) {
            const float z = ((part[0][0] + part[1][0]) + part[2][0]) + part[3][0];
            float sv, kv;
            bool bad;
            score_of(z, 0.f, ro.gate_temp, sv, kv, bad);
            __hip_atomic_store(logits + e, sv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0);
            last = count_arrival(ro, e, E);
        }
        __syncthreads();
        if (last) select_tail_m1<KPL>(logits, ro, pb, psl);
        return;
    }
    if (threadIdx.x < TT && t0 + (int)threadIdx.x < m) {
        const int t = threadIdx.x;
        logits[(size_t)(t0 + t) * E + e] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
    }
}

// ---------------------------------------------------------------- q8_1 of rows
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ x, int nblocks,
                                                            int8_t* __restrict__ xq, float* __restrict__ xd,
                                                            int32_t* __restrict__ xs16, float* __restrict__ xs16f,
                                                            uint16_t* __restrict__ xs16b) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b < nblocks) quantize_block_bf16(x, b, xq, xd, xs16, xs16f, xs16b);
}

// ---------------------------------------------------------------- top-k
// The logit of expert e (< E) from `splits` (<= 8) partial arrays `stride` floats
// apart: all eight loads in flight at once (past `splits` they repeat the last
// one), then added in split order.
MOE_DEV float split_logit(const float* __restrict__ row, size_t stride, int splits, int e) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = row[(size_t)min(i, splits - 1) * stride + e];
    float z = p[0];
#pragma unroll
    for (int i = 1; i < 8; ++i)
        if (i < splits) z += p[i];
    return z;
}

// One wavefront per token (four per workgroup): its keys into LDS, then the
// one-wavefront top-k (no block barriers). `splits` partial logit arrays [m, E]
// one after another (the split-K router product); their sum is the logits.
template <int KPL>
__global__ __launch_bounds__(256) void topk_wave_kernel(const float* __restrict__ logits, int splits,
                                                        const float* __restrict__ bias, int m, int E, int k,
                                                        float gate_temp, int norm, float route_scale,
                                                        int32_t* __restrict__ idx, float* __restrict__ gw,
                                                        int32_t* __restrict__ err) {
    __shared__ float keys[4][64 * KPL], scores[4][64 * KPL];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= m) return;   // a whole wavefront; nothing below waits for the others
    bool bad_any = false;
    float z[KPL], b[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) {   // experts past E repeat the last one (their keys are -inf)
        const int ec = min(lane + 64 * i, E - 1);
        b[i] = bias[ec];
        z[i] = split_logit(logits + (size_t)t * E, (size_t)m * E, splits, ec);
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
        float s, key;
        bool bad;
        score_of(z[i], b[i], gate_temp, s, key, bad);
        const bool in = lane + 64 * i < E;
        keys[wv][lane + 64 * i] = in ? key : -INFINITY;
        scores[wv][lane + 64 * i] = s;
        bad_any |= bad && in;
    }
    if (__any(bad_any) && lane == 0) atomicOr(err, ERR_NONFINITE);
    __builtin_amdgcn_wave_barrier();   // the wavefront's LDS stores come before its reads of them
    int my_e;
    float my_s;
    bool near;
    wave_topk<KPL>(keys[wv], scores[wv], E, k, my_e, my_s, near);
    const float w = wave_pick_weight(my_s, k, norm, route_scale);
    if (lane < k) {
        idx[(size_t)t * k + lane] = my_e;
        gw[(size_t)t * k + lane] = w;
    }
    if (near && lane == 0) atomicAdd(reinterpret_cast<unsigned*>(err + ERR_NEAR_TIES), 1u);
}

// ---------------------------------------------------------------- bucketing
MOE_DEV int block_exclusive_scan(int v, int* lds, int& total) {
    // any block size up to 1024 (16 wavefronts); lds holds 16 ints
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int nw = (blockDim.x + 63) >> 6;
    const int incl = wave_inclusive_scan(v);
    if (lane == 63) lds[wv] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
        const int s = lds[w];
        if (w < wv) base += s;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return base + incl - v;
}

// Counts per expert, the exclusive scan into offsets, the ascending list of
// experts with work, and the chunk list(s); the K-quant shared expert's chunks
// follow the routed ones of their list. classes == 0: one list of
// GEMV_ROWS-row chunks. classes == 1: the three MMQ size classes (a group of
// <= 16 rows, of 17..32 rows, or 64-row chunks of a larger group), class c at
// chunks + base_c. classes == 2: as 1, but a group of at most GEMV_ROWS rows is
// one chunk of the GEMV list (list 3). One workgroup.
__global__ __launch_bounds__(1024) void bucket_count_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                            int m, int shared_chunks, int classes, int base1,
                                                            int base2, int base3, int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ active,
                                                            int32_t* __restrict__ n_active,
                                                            Chunk* __restrict__ chunks,
                                                            int32_t* __restrict__ n_chunks) {
    __shared__ int cnt[1024];
    __shared__ int scan_lds[16];
    const int tid = threadIdx.x;
    cnt[tid] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += 1024) atomicAdd(&cnt[idx[p]], 1);
    __syncthreads();
    const int v = tid < E ? cnt[tid] : 0;
    int total;
    const int excl = block_exclusive_scan(v, scan_lds, total);
    if (tid < E) offsets[tid] = excl;
    if (tid == 0) offsets[E] = total;
    int nact;
    const int aexcl = block_exclusive_scan((tid < E && v > 0) ? 1 : 0, scan_lds, nact);
    if (tid < E && v > 0) active[aexcl] = tid;
    if (tid == 0) *n_active = nact;
    // a group of n rows: class and chunk height
    auto cls_of = [&](int n) {
        return classes == 0                       ? 0
               : classes == 2 && n <= GEMV_ROWS   ? GEMV_LIST
               : n <= MMQ_CLASS_MAX[0]            ? 0
               : n <= MMQ_CLASS_MAX[1]            ? 1
                                                  : 2;
    };
    auto rows_of = [&](int c) { return classes == 0 || c == GEMV_LIST ? GEMV_ROWS : MMQ_CLASS_MAX[c]; };
    const int base[PLAN_LISTS] = {0, base1, base2, base3};
    const int ncls = classes == 0 ? 1 : classes == 1 ? MMQ_CLASSES : PLAN_LISTS;
    const int my_cls = cls_of(v);
    const int my_rows = rows_of(my_cls);
    const int nc = (tid < E && v > 0) ? (v + my_rows - 1) / my_rows : 0;
    const int sh_cls = cls_of(m), sh_rows = rows_of(sh_cls);
    const int nsh = shared_chunks ? (m + sh_rows - 1) / sh_rows : 0;
    for (int c = 0; c < ncls; ++c) {
        int ntot;
        const int cexcl = block_exclusive_scan(my_cls == c ? nc : 0, scan_lds, ntot);
        if (my_cls == c) {
            for (int q = 0; q < nc; ++q) {
                Chunk ch;
                ch.expert = tid;
                ch.row0 = excl + q * my_rows;
                ch.nrows = min(my_rows, v - q * my_rows);
                ch.slot = -1;
                ch.token = -1;
                ch.weight = 0.f;
                ch.pad0 = ch.pad1 = 0;
                chunks[base[c] + cexcl + q] = ch;
            }
        }
        const int nsh_c = sh_cls == c ? nsh : 0;
        for (int q = tid; q < nsh_c; q += 1024) {
            Chunk ch;
            ch.expert = -1;
            ch.row0 = q * sh_rows;
            ch.nrows = min(sh_rows, m - q * sh_rows);
            ch.slot = -1;
            ch.token = -1;
            ch.weight = 0.f;
            ch.pad0 = ch.pad1 = 0;
            chunks[base[c] + ntot + q] = ch;
        }
        if (tid == 0) n_chunks[c] = ntot + nsh_c;
    }
}

// Stable placement: workgroup e lists the pairs that picked expert e in pair
// order (token-major), so positions inside a group follow token order. The
// picks are read PLACE_STEPS steps of 256 at a time, every load of a batch
// requested at once; one barrier per batch publishes each wavefront's match
// count of every step.
constexpr int PLACE_STEPS = 16;
__global__ __launch_bounds__(256) void bucket_place_kernel(const int32_t* __restrict__ idx, int P,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv) {
    const int e = blockIdx.x;
    const int base = offsets[e];
    const int cnt = offsets[e + 1] - base;
    if (cnt == 0) return;
    __shared__ int wtot[PLACE_STEPS][4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const unsigned long long below = (1ull << lane) - 1ull;
    int running = 0;
    for (int p0 = 0; p0 < P && running < cnt; p0 += 256 * PLACE_STEPS) {
        int v[PLACE_STEPS];
#pragma unroll
        for (int j = 0; j < PLACE_STEPS; ++j) v[j] = idx[min(p0 + 256 * j + tid, P - 1)];
        unsigned match = 0u;
        int pre[PLACE_STEPS];
#pragma unroll
        for (int j = 0; j < PLACE_STEPS; ++j) {
            const bool mt = p0 + 256 * j + tid < P && v[j] == e;
            const unsigned long long bal = __ballot(mt);
            pre[j] = __popcll(bal & below);
            if (lane == 0) wtot[j][wv] = __popcll(bal);
            match |= mt ? 1u << j : 0u;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < PLACE_STEPS; ++j) {
            int woff = 0, all = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                woff += w < wv ? wtot[j][w] : 0;
                all += wtot[j][w];
            }
            if (match >> j & 1u) {
                const int p = p0 + 256 * j + tid;
                const int pos = base + running + woff + pre[j];
                perm[pos] = p;
                inv[p] = pos;
            }
            running += all;
        }
        __syncthreads();   // wtot is rewritten by the next batch
    }
}

// ---------------------------------------------------------------- small batches: top-k + bucketing
// One workgroup of NT threads (E <= NT) for m <= 8 tokens: every (token, expert)
// key is formed with all of a thread's loads requested at once (thread e takes
// expert e, e + NT, ... of each token; with the experts' slots), then wavefront t
// takes token t's top-k (the one-wavefront selection, no block barriers), then
// the bucketing of the m * k picks (counts, offsets, active experts, stable
// placement, and one single-row chunk per pick, then one per token for a
// K-quant shared expert) without leaving the workgroup. FROM_SCORES: src holds
// the scores (the router launch's own workgroups wrote them device-coherently);
// else the logits.
template <int KPL, int NT, bool FROM_SCORES>
MOE_DEV void select_small(const float* __restrict__ src, const float* __restrict__ bias, int m, int E, int k,
                          float gate_temp, int norm, float route_scale, int32_t* __restrict__ idx,
                          float* __restrict__ gw, int32_t* __restrict__ err, int shared_chunks,
                          int32_t* __restrict__ offsets, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                          int32_t* __restrict__ perm, int32_t* __restrict__ inv, Chunk* __restrict__ chunks,
                          int32_t* __restrict__ n_chunks, const int32_t* __restrict__ slot_table) {
    constexpr int MT = ROUTE_SMALL_MAX_M;
    __shared__ float keys[MT][64 * KPL], scores[MT][64 * KPL];
    __shared__ float pick_w[ROUTE_SMALL_MAX_PAIRS];
    __shared__ int pick_e[ROUTE_SMALL_MAX_PAIRS];
    __shared__ int cnt[NT];
    __shared__ int offs[NT + 1];
    __shared__ int slots[NT];
    __shared__ int scan_lds[16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    bool bad_any = false;
    for (int e = tid; e < 64 * KPL; e += NT) {
        // tokens past m and experts past E repeat the last ones (in bounds, not kept)
        const int ec = min(e, E - 1);
        const float b = bias[ec];
        const int sl = slot_table[ec];
        float z[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const float* q = src + (size_t)min(t, m - 1) * E + ec;
            z[t] = FROM_SCORES ? __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : *q;
        }
        if (e < E) slots[e] = sl;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            float sv, kv;
            bool bad;
            if (FROM_SCORES) {   // the key as score_of forms it: score + bias, NaN -> -inf
                sv = z[t];
                kv = sv + b;
                bad = kv != kv;
                if (bad) kv = -INFINITY;
            } else {
                score_of(z[t], b, gate_temp, sv, kv, bad);
            }
            keys[t][e] = e < E ? kv : -INFINITY;
            scores[t][e] = sv;
            bad_any |= bad && t < m && e < E;
        }
    }
    __syncthreads();
    if (wv < m) {   // wavefront t: token t's picks, in order, and their weights
        int my_e;
        float my_s;
        bool near;
        wave_topk<KPL>(keys[wv], scores[wv], E, k, my_e, my_s, near);
        const float w = wave_pick_weight(my_s, k, norm, route_scale);
        if (lane < k) {
            pick_e[wv * k + lane] = my_e;
            pick_w[wv * k + lane] = w;
            idx[wv * k + lane] = my_e;
            gw[wv * k + lane] = w;
        }
        if (near && lane == 0) atomicAdd(reinterpret_cast<unsigned*>(err + ERR_NEAR_TIES), 1u);
    }
    if (__any(bad_any) && (tid & 63) == 0) atomicOr(err, ERR_NONFINITE);
    const int P = m * k;
    cnt[tid] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += NT) atomicAdd(&cnt[pick_e[p]], 1);
    __syncthreads();
    const int v = tid < E ? cnt[tid] : 0;
    int total;
    const int excl = block_exclusive_scan(v, scan_lds, total);
    if (tid < E) {
        offsets[tid] = excl;
        offs[tid] = excl;
    }
    if (tid == 0) {
        offsets[E] = total;
        offs[E] = total;
    }
    int nact;
    const int aexcl = block_exclusive_scan((tid < E && v > 0) ? 1 : 0, scan_lds, nact);
    if (tid < E && v > 0) active[aexcl] = tid;
    if (tid == 0) *n_active = nact;
    if (tid == 0) *n_chunks = total + (shared_chunks ? m : 0);
    __syncthreads();
    // stable placement: position = offset of the expert + earlier pairs that picked
    // it; one chunk per position (a single row), carrying what the decode kernels
    // need without further lookups: the expert's slot, the token and the weight
    for (int p = tid; p < P; p += NT) {
        const int pe = pick_e[p];
        int before = 0;
        for (int q = 0; q < p; ++q) before += pick_e[q] == pe ? 1 : 0;
        const int pos = offs[pe] + before;
        perm[pos] = p;
        inv[p] = pos;
        Chunk c;
        c.expert = pe;
        c.row0 = pos;
        c.nrows = 1;
        c.slot = slots[pe];
        c.token = p / k;
        c.weight = pick_w[p];
        c.pad0 = c.pad1 = 0;
        chunks[pos] = c;
    }
    if (shared_chunks && tid < m) {
        Chunk c;
        c.expert = -1;
        c.row0 = tid;
        c.nrows = 1;
        c.slot = 0;
        c.token = tid;
        c.weight = 1.f;
        c.pad0 = c.pad1 = 0;
        chunks[total + tid] = c;
    }
}

template <int KPL>
__global__ __launch_bounds__(1024) void route_small_kernel(const float* __restrict__ logits,
                                                           const float* __restrict__ bias, int m, int E, int k,
                                                           float gate_temp, int norm, float route_scale,
                                                           int32_t* __restrict__ idx, float* __restrict__ gw,
                                                           int32_t* __restrict__ err, int shared_chunks,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ active,
                                                           int32_t* __restrict__ n_active,
                                                           int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                                                           Chunk* __restrict__ chunks,
                                                           int32_t* __restrict__ n_chunks,
                                                           const int32_t* __restrict__ slot_table, SharedRows sr) {
    if (blockIdx.x > 0) {   // the shared expert's rows
        shared_down_block<SR_DOWN_PIECES>(sr, blockIdx.x - 1);
        return;
    }
    select_small<KPL, 1024, false>(logits, bias, m, E, k, gate_temp, norm, route_scale, idx, gw, err, shared_chunks,
                                   offsets, active, n_active, perm, inv, chunks, n_chunks, slot_table);
}

// One token (decode): every thread scores one expert, then the first
// wavefront selects (wave_topk: ties to the lower expert id, NaN keys last as
// on the general path), weighs and lists the picks without further barriers.
constexpr int M1_MAX_KEYS = 16;   // keys per lane: E <= 1024

// The selection by the first wavefront, from all E keys and scores in LDS.
template <int KPL>
MOE_DEV void select_m1(const float* keys, const float* scores, int E, int k, int norm, float route_scale,
                       int32_t* __restrict__ idx, float* __restrict__ gw, int shared_chunks,
                       int32_t* __restrict__ offsets, int32_t* __restrict__ active, int32_t* __restrict__ n_active,
                       int32_t* __restrict__ perm, int32_t* __restrict__ inv, Chunk* __restrict__ chunks,
                       int32_t* __restrict__ n_chunks, const int32_t* __restrict__ slot_table,
                       int32_t* __restrict__ err) {
    const int lane = threadIdx.x;
    int my_e;
    float my_s;
    bool near;
    wave_topk<KPL>(keys, scores, E, k, my_e, my_s, near);
    if (near && lane == 0) atomicAdd(reinterpret_cast<unsigned*>(err + ERR_NEAR_TIES), 1u);
    // up to M1_FAST_K picks: every pick's id and score in scalar registers once (entries
    // past k: id INT_MAX, score 0, which leave the counts and the in-order sum as they are)
    constexpr int M1_FAST_K = 8;
    const bool fast = k <= M1_FAST_K;
    int pe[M1_FAST_K];
    float wgt;
    int pos = 0;
    if (fast) {
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < M1_FAST_K; ++q) {
            pe[q] = q < k ? __builtin_amdgcn_readlane(my_e, q) : INT_MAX;
            sum += q < k ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), q)) : 0.f;
        }
        wgt = (norm && k > 1 ? my_s / (sum + 1e-20f) : my_s) * route_scale;
#pragma unroll
        for (int q = 0; q < M1_FAST_K; ++q) pos += pe[q] < my_e ? 1 : 0;
    } else {
        wgt = wave_pick_weight(my_s, k, norm, route_scale);
        for (int q = 0; q < k; ++q) pos += __builtin_amdgcn_readlane(my_e, q) < my_e ? 1 : 0;
    }
    // the picks sorted by expert id (all distinct): position = rank of the id
    if (lane < k) {
        idx[lane] = my_e;
        gw[lane] = wgt;
        perm[pos] = lane;
        inv[lane] = pos;
        active[pos] = my_e;
        Chunk c;
        c.expert = my_e;
        c.row0 = pos;
        c.nrows = 1;
        c.slot = slot_table[my_e];
        c.token = 0;
        c.weight = wgt;
        c.pad0 = c.pad1 = 0;
        chunks[pos] = c;
    }
    if (shared_chunks && lane == 0) {
        Chunk c;
        c.expert = -1;
        c.row0 = 0;
        c.nrows = 1;
        c.slot = 0;
        c.token = 0;
        c.weight = 1.f;
        c.pad0 = c.pad1 = 0;
        chunks[k] = c;
    }
    if (lane == 0) {
        *n_active = k;
        *n_chunks = k + (shared_chunks ? 1 : 0);
    }
    // offsets[e] = picks with a smaller id
    for (int e = lane; e <= E; e += 64) {
        int cnt = 0;
        if (fast) {
#pragma unroll
            for (int q = 0; q < M1_FAST_K; ++q) cnt += pe[q] < e ? 1 : 0;
        } else {
            for (int q = 0; q < k; ++q) cnt += __builtin_amdgcn_readlane(my_e, q) < e ? 1 : 0;
        }
        offsets[e] = cnt;
    }
}

// The last router workgroup (256 threads): every thread forms the keys of experts
// tid, tid + 256, ... from their scores (read device-coherently) and prefetched
// biases into LDS, then the first wavefront selects.
template <int KPL>
MOE_DEV void select_tail_m1(const float* scores_in, const RouteSel& ro, const float (&b)[M1_PREFETCH],
                            const int (&sl)[M1_PREFETCH]) {
    static_assert(64 * KPL <= 256 * M1_PREFETCH, "one key per prefetched entry");
    __shared__ float keys[64 * KPL], scores[64 * KPL];
    __shared__ int slots[64 * KPL];
    float sc[M1_PREFETCH];
#pragma unroll
    for (int i = 0; i < M1_PREFETCH; ++i) {   // every score requested at once
        const int e = threadIdx.x + 256 * i;
        sc[i] = e < ro.E ? __hip_atomic_load(scores_in + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
    }
    bool bad_any = false;
#pragma unroll
    for (int i = 0; i < M1_PREFETCH; ++i) {
        const int e = threadIdx.x + 256 * i;
        if (e >= 64 * KPL) break;
        float kv = -INFINITY;
        bool bad = false;
        if (e < ro.E) {   // the key as score_of forms it: score + bias, NaN -> -inf
            kv = sc[i] + b[i];
            bad = kv != kv;
            if (bad) kv = -INFINITY;
        }
        keys[e] = kv;
        scores[e] = e < ro.E ? sc[i] : 0.f;
        slots[e] = sl[i];
        bad_any |= bad;
    }
    if (__any(bad_any) && (threadIdx.x & 63) == 0) atomicOr(ro.err, ERR_NONFINITE);
    __syncthreads();
    if (threadIdx.x >= 64) return;
    select_m1<KPL>(keys, scores, ro.E, ro.k, ro.norm, ro.route_scale, ro.idx, ro.gw, ro.shared_chunks, ro.offsets,
                   ro.active, ro.n_active, ro.perm, ro.inv, ro.chunks, ro.n_chunks, slots, ro.err);
}

template <int KPL>
__global__ __launch_bounds__(1024) void route_m1_kernel(const float* __restrict__ logits, const float* __restrict__ bias,
                                                        int E, int k, float gate_temp, int norm, float route_scale,
                                                        int32_t* __restrict__ idx, float* __restrict__ gw,
                                                        int32_t* __restrict__ err, int shared_chunks,
                                                        int32_t* __restrict__ offsets, int32_t* __restrict__ active,
                                                        int32_t* __restrict__ n_active, int32_t* __restrict__ perm,
                                                        int32_t* __restrict__ inv, Chunk* __restrict__ chunks,
                                                        int32_t* __restrict__ n_chunks,
                                                        const int32_t* __restrict__ slot_table, SharedRows sr) {
    if (blockIdx.x > 0) {   // the shared expert's rows
        shared_down_block<SR_DOWN_PIECES>(sr, blockIdx.x - 1);
        return;
    }
    __shared__ float keys[64 * M1_MAX_KEYS], scores[64 * M1_MAX_KEYS];
    const int tid = threadIdx.x;
    {
        float sv, kv;
        bool bad;
        score_key(logits, bias, tid, E, gate_temp, sv, kv, bad);
        keys[tid] = kv;
        scores[tid] = sv;
        if (__any(bad) && (tid & 63) == 0) atomicOr(err, ERR_NONFINITE);
    }
    __syncthreads();
    if (tid >= 64) return;
    select_m1<KPL>(keys, scores, E, k, norm, route_scale, idx, gw, shared_chunks, offsets, active, n_active, perm, inv,
              chunks, n_chunks, slot_table, err);
}

// After experts were streamed into slots: the single-row chunks of the small-batch
// routing take their experts' slots again from the table.
__global__ __launch_bounds__(256) void refresh_slots_kernel(Chunk* __restrict__ chunks,
                                                            const int32_t* __restrict__ n_chunks,
                                                            const int32_t* __restrict__ slot_table) {
    const int n = *n_chunks;
    for (int c = threadIdx.x; c < n; c += 256) {
        const int e = chunks[c].expert;
        if (e >= 0) chunks[c].slot = slot_table[e];
    }
}

// ---------------------------------------------------------------- one slot wave's chunks
// The chunks a slot wave computes, so that its launches spread them over the XCDs
// (the experts of a wave are mostly neighbours in the chunk order, which the tile
// order would otherwise place on one or two XCDs): for each list c of the plan,
// the chunks whose expert the wave's slot table does not mark SLOT_SKIP, in their
// order, at the list's base, and their count; a K-quant shared expert's chunks
// (expert -1) in the first wave only. One workgroup per list.
__global__ __launch_bounds__(256) void compact_wave_kernel(const Chunk* __restrict__ in, const int32_t* __restrict__ n_in,
                                                           const int32_t* __restrict__ slot_table, int first_wave,
                                                           ChunkPlan plan, Chunk* __restrict__ out,
                                                           int32_t* __restrict__ n_out) {
    __shared__ int wsum[4];
    __shared__ int kept;
    const int c = blockIdx.x, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int base = plan.base[c], n = min(n_in[c], plan.cap[c]);
    if (threadIdx.x == 0) kept = 0;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += 256) {
        const int i = i0 + threadIdx.x;
        Chunk ch{};
        bool keep = false;
        if (i < n) {
            ch = in[base + i];
            keep = ch.expert < 0 ? first_wave != 0 : slot_table[ch.expert] != SLOT_SKIP;
        }
        const unsigned long long bal = __ballot(keep);
        if (lane == 0) wsum[wv] = __popcll(bal);
        __syncthreads();
        int off = kept + __popcll(bal & ((1ull << lane) - 1));
        for (int w = 0; w < wv; ++w) off += wsum[w];
        if (keep) out[base + off] = ch;
        __syncthreads();
        if (threadIdx.x == 0) kept += wsum[0] + wsum[1] + wsum[2] + wsum[3];
        __syncthreads();
    }
    if (threadIdx.x == 0) n_out[c] = kept;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_compact_wave(const Chunk* chunks, const int32_t* n_chunks, const int32_t* slot_table, bool first_wave,
                               const ChunkPlan& plan, Chunk* out, int32_t* n_out, hipStream_t st) {
    return launch_kernel(compact_wave_kernel, PLAN_LISTS, 256, 0, st, chunks, n_chunks, slot_table,
                         first_wave ? 1 : 0, plan, out, n_out);
}

hipError_t launch_refresh_slots(Chunk* chunks, const int32_t* n_chunks, const int32_t* slot_table, hipStream_t st) {
    return launch_kernel(refresh_slots_kernel, 1, 256, 0, st, chunks, n_chunks, slot_table);
}

hipError_t launch_router_quant(const uint16_t* x, int m, const uint16_t* wr, int D, int E, float* logits,
                               int8_t* xq, float* xd, int32_t* xs16, float* xs16f, hipStream_t st,
                               const SharedRows* sr) {
    SharedRows none{};
    const SharedRows& s = sr ? *sr : none;
    // m = 1: 256 threads per workgroup, the router row strided over them; m = 2..8:
    // 512 threads, every load of a row hoisted (the workgroups of one launch share
    // their size: the q8_1 and shared-row workgroups follow it)
    const int th = m == 1 ? 256 : 512;
    const int nq = xq == nullptr ? 0 : (m * (D / QB) + th - 1) / th;
    const int nsh = sr ? shared_rows_blocks(*sr, th) : 0;
    const int grid = E + nq + nsh;
    const RouteSel no{};
    if (m == 1) return launch_kernel(router_quant_kernel<1>, grid, th, 0, st, x, m, wr, D, E, 1, logits, xq, xd, xs16, xs16f, s, no);
    if (m == 2) return launch_kernel(router_quant_kernel<2>, grid, th, 0, st, x, m, wr, D, E, 1, logits, xq, xd, xs16, xs16f, s, no);
    if (m <= 4) return launch_kernel(router_quant_kernel<4>, grid, th, 0, st, x, m, wr, D, E, 1, logits, xq, xd, xs16, xs16f, s, no);
    return launch_kernel(router_quant_kernel<8>, grid, th, 0, st, x, m, wr, D, E, 1, logits, xq, xd, xs16, xs16f, s, no);
}

bool router_select_ok(int E, int k, int m) {
    if (E < 1 || k < 1 || k > 64 || k > E || m < 1 || m > ROUTE_SMALL_MAX_M) return false;
    if (m == 1) return E <= 64 * M1_MAX_KEYS;
    return topk_kpl(E) <= 6 && m * k <= ROUTE_SMALL_MAX_PAIRS;   // E <= 384 (the selection's LDS in every workgroup)
}

hipError_t launch_router_select(const uint16_t* x, int m, const uint16_t* wr, int D, float* logits, int8_t* xq,
                                float* xd, int32_t* xs16, float* xs16f, const RouteSel& ro, hipStream_t st,
                                const SharedRows* sr) {
    if (!router_select_ok(ro.E, ro.k, m) || ro.arrive == nullptr) return hipErrorInvalidValue;
    SharedRows none{};
    const SharedRows& s = sr ? *sr : none;
    const int th = m == 1 ? 256 : 512;
    const int nq = xq == nullptr ? 0 : (m * (D / QB) + th - 1) / th;
    const int grid = ro.E + nq + (sr ? shared_rows_blocks(*sr, th) : 0);
    const int kpl = topk_kpl(ro.E);
#define RSEL(TT, KPL) launch_kernel(router_quant_kernel<TT, KPL>, grid, th, 0, st, x, m, wr, D, ro.E, 1, logits, xq, xd, \
                                    xs16, xs16f, s, ro)
    if (m == 1) return kpl == 2 ? RSEL(1, 2) : kpl == 6 ? RSEL(1, 6) : RSEL(1, 16);
    if (m == 2) return kpl == 2 ? RSEL(2, 2) : RSEL(2, 6);
    if (m <= 4) return kpl == 2 ? RSEL(4, 2) : RSEL(4, 6);
    return kpl == 2 ? RSEL(8, 2) : RSEL(8, 6);
#undef RSEL
}

hipError_t launch_quantize_rows(const uint16_t* x, int m, int D, int8_t* xq, float* xd, int32_t* xs16,
                                float* xs16f, uint16_t* xs16b, hipStream_t st) {
    const int nb = m * (D / QB);
    return launch_kernel(quantize_rows_kernel, (nb + 255) / 256, 256, 0, st, x, nb, xq, xd, xs16, xs16f, xs16b);
}

hipError_t launch_route_small(const float* logits, const float* bias, int m, int E, int k, float gate_temp,
                              int norm, float route_scale, int32_t* idx, float* gw, int32_t* err, int shared_chunks,
                              int32_t* offsets, int32_t* active, int32_t* n_active, int32_t* perm, int32_t* inv,
                              Chunk* chunks, int32_t* n_chunks, const int32_t* slot_table, hipStream_t st,
                              const SharedRows* sr) {
    SharedRows none{};
    const SharedRows& s = sr ? *sr : none;
    if (m == 1 && E <= 64 * M1_MAX_KEYS && k <= 64) {
        const int th = std::max(128, (E + 63) / 64 * 64);   // shared-expert rows take two wavefronts each
        const int grid = 1 + (sr ? shared_rows_blocks(*sr, th) : 0);
#define ROUTE_M1(KPL) launch_kernel(route_m1_kernel<KPL>, grid, th, 0, st, logits, bias, E, k, gate_temp, norm, \
                                    route_scale, idx, gw, err, shared_chunks, offsets, active, n_active, perm, inv, \
                                    chunks, n_chunks, slot_table, s)
        const int kpl = topk_kpl(E);
        const hipError_t e = kpl == 2 ? ROUTE_M1(2) : kpl == 6 ? ROUTE_M1(6) : ROUTE_M1(16);
#undef ROUTE_M1
        return e;
    }
    const int grid = 1 + (sr ? shared_rows_blocks(*sr, 1024) : 0);
#define ROUTE_SMALL(KPL) launch_kernel(route_small_kernel<KPL>, grid, 1024, 0, st, logits, bias, m, E, k, gate_temp, \
                                       norm, route_scale, idx, gw, err, shared_chunks, offsets, active, n_active, \
                                       perm, inv, chunks, n_chunks, slot_table, s)
    const int kpl = topk_kpl(E);
    const hipError_t e = kpl == 2 ? ROUTE_SMALL(2) : kpl == 6 ? ROUTE_SMALL(6) : ROUTE_SMALL(16);
#undef ROUTE_SMALL
    return e;
}

hipError_t launch_topk(const float* logits, int splits, const float* bias, int m, int E, int k, float gate_temp,
                       int norm, float route_scale, int32_t* idx, float* gw, int32_t* err, hipStream_t st) {
    // a wavefront per token (k <= 64 and E <= 1024, as the configuration checks ensure)
    const int grid = (m + 3) / 4, kpl = topk_kpl(E);
#define TOPK_WAVE(KPL) launch_kernel(topk_wave_kernel<KPL>, grid, 256, 0, st, logits, splits, bias, m, E, k, \
                                     gate_temp, norm, route_scale, idx, gw, err)
    const hipError_t e = kpl == 2 ? TOPK_WAVE(2) : kpl == 6 ? TOPK_WAVE(6) : TOPK_WAVE(16);
#undef TOPK_WAVE
    return e;
}

hipError_t launch_bucket(const int32_t* idx, int m, int k, int E, int shared_chunks, const ChunkPlan* plan,
                         int32_t* offsets, int32_t* active, int32_t* n_active, int32_t* perm, int32_t* inv,
                         Chunk* chunks, int32_t* n_chunks, hipStream_t st) {
    const int P = m * k;
    const int classes = plan == nullptr ? 0 : plan->mixed ? 2 : 1;
    hipError_t e = launch_kernel(bucket_count_kernel, 1, 1024, 0, st, idx, P, E, m, shared_chunks, classes,
                                 plan ? plan->base[1] : 0, plan ? plan->base[2] : 0, plan ? plan->base[GEMV_LIST] : 0,
                                 offsets, active, n_active, chunks, n_chunks);
    if (e != hipSuccess) return e;
    return launch_kernel(bucket_place_kernel, E, 256, 0, st, idx, P, offsets, perm, inv);
}

}  // namespace moe
