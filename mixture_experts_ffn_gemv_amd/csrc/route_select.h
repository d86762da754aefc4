// Device pieces of the routing kernels: the score and key of an expert, and
// the top-k of up to 64 * KPL keys by a single wavefront.
//
// Semantics (metrale moe_v41.rs route_from_logits; Open Model Atlas router
// equations for DeepSeek V4.1): v = z / gate_temp; softplus(v) = v above 20,
// else ln(1 + e^v); s = sqrt(softplus(v)); key = s + bias; picks = the k
// largest keys, equal keys ordered by the lower expert id.
#pragma once

#include <climits>

#include "moe_common.h"

namespace moe {

// Score and key of logit z with bias b. A NaN key raises `bad` and is ordered
// as -inf, so k picks always exist.
MOE_DEV void score_of(float z, float b, float gate_temp, float& s, float& key, bool& bad) {
    const float v = z / gate_temp;
    const float sp = v > 20.f ? v : log1pf(expf(v));
    s = sqrtf(sp);
    key = s + b;
    bad = key != key;
    if (bad) key = -INFINITY;
}

// Expert e's score and key from a logits row (e >= E: key -inf). The logit is the
// sum of `splits` partial rows `split_stride` floats apart (a split-K router
// product), added in split order.
MOE_DEV void score_key(const float* __restrict__ logits_row, const float* __restrict__ bias, int e, int E,
                       float gate_temp, float& s, float& key, bool& bad, int splits = 1, size_t split_stride = 0) {
    key = -INFINITY;
    s = 0.f;
    bad = false;
    if (e < E) {
        const float b = bias[e];   // requested before the arithmetic
        float z = logits_row[e];
        for (int i = 1; i < splits; ++i) z += logits_row[i * split_stride + e];
        score_of(z, b, gate_temp, s, key, bad);
    }
}

// wavefront-wide max / min, the result in every lane: DPP inside each 16-lane
// row (quad swaps, then rotations by 4 and 8), then the four rows' values
template <int CTRL>
MOE_DEV int dpp_mov(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
MOE_DEV float wave_max_f32(float v) {
    v = fmaxf(v, __int_as_float(dpp_mov<0xB1>(__float_as_int(v))));    // quad_perm [1,0,3,2]
    v = fmaxf(v, __int_as_float(dpp_mov<0x4E>(__float_as_int(v))));    // quad_perm [2,3,0,1]
    v = fmaxf(v, __int_as_float(dpp_mov<0x124>(__float_as_int(v))));   // row_ror:4
    v = fmaxf(v, __int_as_float(dpp_mov<0x128>(__float_as_int(v))));   // row_ror:8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
MOE_DEV int wave_min_i32(int v) {
    v = min(v, dpp_mov<0xB1>(v));
    v = min(v, dpp_mov<0x4E>(v));
    v = min(v, dpp_mov<0x124>(v));
    v = min(v, dpp_mov<0x128>(v));
    const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return min(min(r0, r1), min(r2, r3));
}
MOE_DEV int wave_max_i32(int v) {
    v = max(v, dpp_mov<0xB1>(v));
    v = max(v, dpp_mov<0x4E>(v));
    v = max(v, dpp_mov<0x124>(v));
    v = max(v, dpp_mov<0x128>(v));
    const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// Order-preserving int32 image of a non-NaN float key (-0 taken as +0): a
// larger key gives a larger int, and INT_MIN lies below every key, -inf included.
MOE_DEV int ordered_key(float f) {
    const int b = __float_as_int(f + 0.0f);
    return b >= 0 ? b : b ^ 0x7FFFFFFF;
}

// Keys per lane for the one-wavefront top-k of E keys.
constexpr int topk_kpl(int E) { return E <= 128 ? 2 : E <= 384 ? 6 : 16; }

// The float key behind an ordered int (the inverse of ordered_key).
MOE_DEV float key_of_ordered(int o) { return __int_as_float(o >= 0 ? o : o ^ 0x7FFFFFFF); }

// Gap below which the k-th and (k+1)-th keys of a token count as a near tie
// (the selection there may differ from an exact one by rounding alone).
constexpr float NEAR_TIE_GAP = 1e-5f;

// The k (<= min(64, E)) largest of E <= 64 * KPL keys in LDS, by one whole
// wavefront, without branches. Lane l holds keys l, l + 64, ... as ordered
// ints; each of the k rounds takes the largest remaining key across the
// wavefront and the lowest id holding it (inside a lane the ids grow with the
// index, so a strict comparison keeps the lowest), then sets it to INT_MIN.
// The winner is wavefront-uniform, so lane r < k ends with pick r's expert and
// its score (from `scores`). `near` (wavefront-uniform) is set when k < E and
// the k-th key exceeds the largest key left out by less than NEAR_TIE_GAP.
template <int KPL>
MOE_DEV void wave_topk(const float* keys, const float* scores, int E, int k, int& my_e, float& my_s, bool& near) {
    const int lane = threadIdx.x & 63;
    int kk[KPL];
#pragma unroll
    for (int i = 0; i < KPL; ++i) kk[i] = lane + 64 * i < E ? ordered_key(keys[lane + 64 * i]) : INT_MIN;
    my_e = 0;
    int kth = INT_MIN;
    for (int r = 0; r < k; ++r) {
        int bk = kk[0], bi = lane;
#pragma unroll
        for (int i = 1; i < KPL; ++i) {
            const bool b = kk[i] > bk;
            bk = b ? kk[i] : bk;
            bi = b ? lane + 64 * i : bi;
        }
        const int kmax = wave_max_i32(bk);
        const int win = wave_min_i32(bk == kmax ? bi : INT_MAX);
#pragma unroll
        for (int i = 0; i < KPL; ++i) kk[i] = lane + 64 * i == win ? INT_MIN : kk[i];
        my_e = lane == r ? win : my_e;
        kth = kmax;
    }
    my_s = lane < k ? scores[my_e] : 0.f;
    near = false;
    if (k < E) {   // the largest key left out (a real key: E > k of them exist)
        int bk = kk[0];
#pragma unroll
        for (int i = 1; i < KPL; ++i) bk = max(bk, kk[i]);
        const int next = wave_max_i32(bk);
        near = key_of_ordered(kth) - key_of_ordered(next) < NEAR_TIE_GAP;
    }
}

// The routing weight of lane r's pick: the unbiased score, divided by (the sum
// of the k scores in pick order + 1e-20) when norm and k > 1, times route_scale.
// Called by the whole wavefront after wave_topk.
MOE_DEV float wave_pick_weight(float my_s, int k, int norm, float route_scale) {
    float sum = 0.f;
    for (int q = 0; q < k; ++q) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), q));
    return (norm && k > 1 ? my_s / (sum + 1e-20f) : my_s) * route_scale;
}

}  // namespace moe
