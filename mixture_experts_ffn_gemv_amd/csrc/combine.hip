// Weighted combine and finish: out[t] = bf16( sum_i G[t,i] E[pos(t,i)] + y_shared[t] ).
// The routed terms are added in pick order, then the shared expert (metrale's
// accumulate / finish kernels and `shared_side`: the shared output joins acc
// after the routed experts; Open Model Atlas: Delta_ffn = y_routed + y_shared).
// Fixed order and no atomics, so every run gives the same bits.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ e_rows,
                                                      const float* __restrict__ ys,
                                                      const float* __restrict__ gw,
                                                      const int32_t* __restrict__ inv, int k, int D,
                                                      uint16_t* __restrict__ out) {
    const int t = blockIdx.y;
    const int c4 = blockIdx.x * 256 + threadIdx.x;
    if (4 * c4 >= D) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int i = 0; i < k; ++i) {
        const int p = t * k + i;
        const float g = gw[p];
        const float4 v = reinterpret_cast<const float4*>(e_rows + (size_t)inv[p] * D)[c4];
        acc.x = fmaf(g, v.x, acc.x);
        acc.y = fmaf(g, v.y, acc.y);
        acc.z = fmaf(g, v.z, acc.z);
        acc.w = fmaf(g, v.w, acc.w);
    }
    if (ys != nullptr) {
        const float4 s = reinterpret_cast<const float4*>(ys + (size_t)t * D)[c4];
        acc.x += s.x;
        acc.y += s.y;
        acc.z += s.z;
        acc.w += s.w;
    }
    uint2 o;
    o.x = f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16);
    o.y = f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16);
    reinterpret_cast<uint2*>(out + (size_t)t * D)[c4] = o;
}

hipError_t launch_combine(const float* e_rows, const float* ys, const float* gw, const int32_t* inv, int m,
                          int k, int D, uint16_t* out, hipStream_t st) {
    const int n4 = D / 4;
    return launch_kernel(combine_kernel, dim3((n4 + 255) / 256, m), 256, 0, st, e_rows, ys, gw, inv, k, D, out);
}

}  // namespace moe
