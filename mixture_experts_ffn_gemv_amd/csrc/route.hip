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
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- router logits
// z[t, e] = sum_d x[t, d] * W_R[e, d], f32 accumulation. One workgroup per
// (expert row, group of TT tokens); each thread walks 4-element chunks of the
// row, so a row's 10 KB are read once per token group with coalesced loads.
template <int TT>
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t* __restrict__ x, int m,
                                                          const uint16_t* __restrict__ wr, int D, int E,
                                                          float* __restrict__ logits) {
    const int e = blockIdx.x;
    const int t0 = blockIdx.y * TT;
    const uint2* w = reinterpret_cast<const uint2*>(wr + (size_t)e * D);
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.f;
    const int nc = D / 4;
    for (int c = threadIdx.x; c < nc; c += 256) {
        const uint2 wv = w[c];
        const float w0 = bf16_lo(wv.x), w1 = bf16_hi(wv.x), w2 = bf16_lo(wv.y), w3 = bf16_hi(wv.y);
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            if (t0 + t < m) {
                const uint2 xv = reinterpret_cast<const uint2*>(x + (size_t)(t0 + t) * D)[c];
                float a = acc[t];
                a = fmaf(bf16_lo(xv.x), w0, a);
                a = fmaf(bf16_hi(xv.x), w1, a);
                a = fmaf(bf16_lo(xv.y), w2, a);
                a = fmaf(bf16_hi(xv.y), w3, a);
                acc[t] = a;
            }
        }
    }
    __shared__ float part[4][TT];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
        const float s = wave_sum(acc[t]);
        if (lane == 0) part[wv][t] = s;
    }
    __syncthreads();
    if (threadIdx.x < TT && t0 + (int)threadIdx.x < m) {
        const int t = threadIdx.x;
        logits[(size_t)(t0 + t) * E + e] = ((part[0][t] + part[1][t]) + part[2][t]) + part[3][t];
    }
}

// ---------------------------------------------------------------- q8_1 of rows
// One lane per 32-value block of x [m, D] (bf16): int8 quants, fp16(d) as f32,
// and the two 16-value sums of the quants (used by the Q2_K min term).
__global__ __launch_bounds__(256) void quantize_rows_kernel(const uint16_t* __restrict__ x, int nblocks,
                                                            int8_t* __restrict__ xq, float* __restrict__ xd,
                                                            int32_t* __restrict__ xs16) {
    const int b = blockIdx.x * 256 + threadIdx.x;
    if (b >= nblocks) return;
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
}

// ---------------------------------------------------------------- top-k
// One wavefront per token. Each lane holds the keys of experts lane, lane+64,
// ... (at most 16 per lane, E <= 1024). k rounds of a wave-wide arg-max with the
// total order (key descending, id ascending); NaN keys raise the error bit and
// are ordered as -inf so a pick always exists.
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits,
                                                   const float* __restrict__ bias, int m, int E, int k,
                                                   float gate_temp, int norm, float route_scale,
                                                   int32_t* __restrict__ idx, float* __restrict__ gw,
                                                   int32_t* __restrict__ err) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= m) return;
    float key[16], sc[16];
    bool nan_seen = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = lane + 64 * i;
        key[i] = -INFINITY;
        sc[i] = 0.f;
        if (e < E) {
            const float v = logits[(size_t)t * E + e] / gate_temp;
            const float sp = v > 20.f ? v : log1pf(expf(v));
            const float s = sqrtf(sp);
            float kv = s + bias[e];
            if (kv != kv) {
                nan_seen = true;
                kv = -INFINITY;
            }
            key[i] = kv;
            sc[i] = s;
        }
    }
    if (__any(nan_seen) && lane == 0) atomicOr(err, ERR_NONFINITE);
    uint32_t taken = 0;
    float picked_s = 0.f;   // lane r keeps the score of pick r
    for (int r = 0; r < k; ++r) {
        float bk = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((taken >> i) & 1u)) {
                if (key[i] > bk || (key[i] == bk && e < bi)) {
                    bk = key[i];
                    bi = e;
                }
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ok = __shfl_xor(bk, off);
            const int oi = __shfl_xor(bi, off);
            if (ok > bk || (ok == bk && oi < bi)) {
                bk = ok;
                bi = oi;
            }
        }
        // bi is now uniform across the wave
        const int owner = bi & 63, slot = bi >> 6;
        float s_owner = 0.f;
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (i == slot) s_owner = sc[i];
            taken |= 1u << slot;
        }
        const float s_pick = __shfl(s_owner, owner);
        if (lane == r) picked_s = s_pick;
        if (lane == 0) idx[(size_t)t * k + r] = bi;
    }
    // weights: the unbiased scores in pick order, renormalised, scaled
    float denom = 1.f;
    if (norm && k > 1) {
        float sum = 0.f;
        for (int r = 0; r < k; ++r) sum += __shfl(picked_s, r);
        denom = sum + 1e-20f;
    }
    if (lane < k) {
        float wgt = (norm && k > 1) ? picked_s / denom : picked_s;
        gw[(size_t)t * k + lane] = wgt * route_scale;
    }
}

// ---------------------------------------------------------------- bucketing
MOE_DEV int block_exclusive_scan(int v, int* lds, int& total) {
    // 1024 threads = 16 waves; lds holds 16 ints
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
    }
    if (lane == 63) lds[wv] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int w = 0; w < 16; ++w) {
        const int s = lds[w];
        if (w < wv) base += s;
        tot += s;
    }
    __syncthreads();
    total = tot;
    return base + incl - v;
}

// Counts per expert, the exclusive scan into offsets, the ascending list of
// experts with work, and the chunk list (GEMV_ROWS rows per chunk; the
// K-quant shared expert's chunks follow the routed ones). One workgroup.
__global__ __launch_bounds__(1024) void bucket_count_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                            int m, int shared_chunks,
                                                            int32_t* __restrict__ offsets,
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
    const int nc = tid < E ? (v + GEMV_ROWS - 1) / GEMV_ROWS : 0;
    int ntot;
    const int cexcl = block_exclusive_scan(nc, scan_lds, ntot);
    for (int q = 0; q < nc; ++q) {
        Chunk c;
        c.expert = tid;
        c.row0 = excl + q * GEMV_ROWS;
        c.nrows = min(GEMV_ROWS, v - q * GEMV_ROWS);
        c.pad = 0;
        chunks[cexcl + q] = c;
    }
    const int nsh = shared_chunks ? (m + GEMV_ROWS - 1) / GEMV_ROWS : 0;
    for (int q = tid; q < nsh; q += 1024) {
        Chunk c;
        c.expert = -1;
        c.row0 = q * GEMV_ROWS;
        c.nrows = min(GEMV_ROWS, m - q * GEMV_ROWS);
        c.pad = 0;
        chunks[ntot + q] = c;
    }
    if (tid == 0) *n_chunks = ntot + nsh;
}

// Stable placement: workgroup e lists the pairs that picked expert e in pair
// order (token-major), so positions inside a group follow token order.
__global__ __launch_bounds__(256) void bucket_place_kernel(const int32_t* __restrict__ idx, int P,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ inv) {
    const int e = blockIdx.x;
    const int base = offsets[e];
    const int cnt = offsets[e + 1] - base;
    if (cnt == 0) return;
    __shared__ int wtot[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int running = 0;
    for (int p0 = 0; p0 < P && running < cnt; p0 += 256) {
        const int p = p0 + threadIdx.x;
        const bool match = p < P && idx[p] == e;
        const unsigned long long bal = __ballot(match);
        const int pre = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wtot[wv] = __popcll(bal);
        __syncthreads();
        int woff = 0, all = 0;
        for (int w = 0; w < 4; ++w) {
            if (w < wv) woff += wtot[w];
            all += wtot[w];
        }
        if (match) {
            const int pos = base + running + woff + pre;
            perm[pos] = p;
            inv[p] = pos;
        }
        running += all;
        __syncthreads();
    }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_router_gemv(const uint16_t* x, int m, const uint16_t* wr, int D, int E, float* logits,
                              hipStream_t st) {
    if (m == 1) {
        router_gemv_kernel<1><<<dim3(E, 1), 256, 0, st>>>(x, m, wr, D, E, logits);
    } else if (m <= 2) {
        router_gemv_kernel<2><<<dim3(E, 1), 256, 0, st>>>(x, m, wr, D, E, logits);
    } else if (m <= 4) {
        router_gemv_kernel<4><<<dim3(E, 1), 256, 0, st>>>(x, m, wr, D, E, logits);
    } else {
        router_gemv_kernel<8><<<dim3(E, (m + 7) / 8), 256, 0, st>>>(x, m, wr, D, E, logits);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const uint16_t* x, int m, int D, int8_t* xq, float* xd, int32_t* xs16,
                                hipStream_t st) {
    const int nb = m * (D / QB);
    quantize_rows_kernel<<<(nb + 255) / 256, 256, 0, st>>>(x, nb, xq, xd, xs16);
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const float* bias, int m, int E, int k, float gate_temp,
                       int norm, float route_scale, int32_t* idx, float* gw, int32_t* err, hipStream_t st) {
    topk_kernel<<<(m + 3) / 4, 256, 0, st>>>(logits, bias, m, E, k, gate_temp, norm, route_scale, idx, gw, err);
    return hipGetLastError();
}

hipError_t launch_bucket(const int32_t* idx, int m, int k, int E, int shared_chunks, int32_t* offsets,
                         int32_t* active, int32_t* n_active, int32_t* perm, int32_t* inv, Chunk* chunks,
                         int32_t* n_chunks, hipStream_t st) {
    const int P = m * k;
    bucket_count_kernel<<<1, 1024, 0, st>>>(idx, P, E, m, shared_chunks, offsets, active, n_active, chunks,
                                            n_chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    bucket_place_kernel<<<E, 256, 0, st>>>(idx, P, offsets, perm, inv);
    return hipGetLastError();
}

}  // namespace moe
