// topk.h -- one wavefront routes one token: logits (summed from split-K
// partials in a fixed order), k rounds of a wave-wide arg-max with ties to
// the lower expert index, and the softmax of the k selected logits.
//
// Page "CKE Zip: From Splitting Tokens To Splitting Qwen3.5 Weights", sections
// "What The First Prototype Split" (indices and routing weights travel with
// each row) and "What PR #382 Now Splits" (top eight of 256 experts).
#pragma once

#include "moe_internal.h"

namespace moe {

// (v, e) ranks above (bv, be): larger logit, ties to the lower expert index.
// A total order, so any reduction order selects the same winner.
__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
    return v > bv || (v == bv && e < be);
}

template <int CTRL>
__device__ __forceinline__ void dpp_pair(float& v, int& e) {
    const float ov = __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
    const int oe = __builtin_amdgcn_update_dpp(0, e, CTRL, 0xf, 0xf, false);
    if (better(ov, oe, v, e)) {
        v = ov;
        e = oe;
    }
}

// Wave-wide arg-max of (v, e), result in every lane.  Within each 16-lane row
// through DPP moves (xor 1, xor 2, half-row mirror, row mirror), then across
// the four rows through lane reads; no LDS traffic.
__device__ __forceinline__ void wave_argmax(float& v, int& e) {
    dpp_pair<0xB1>(v, e);    // quad_perm [1,0,3,2]
    dpp_pair<0x4E>(v, e);    // quad_perm [2,3,0,1]
    dpp_pair<0x141>(v, e);   // row_half_mirror
    dpp_pair<0x140>(v, e);   // row_mirror
    float bv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    int be = __builtin_amdgcn_readlane(e, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float rv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16 * r));
        const int re = __builtin_amdgcn_readlane(e, 16 * r);
        if (better(rv, re, bv, be)) {
            bv = rv;
            be = re;
        }
    }
    v = bv;
    e = be;
}

// part: [T][E][KS] partial logits.  Writes the k slots of token t to
// idx_row[0..k), w_row[0..k) (global or LDS).  Lane l holds experts l, l+64,
// ... (NE per lane: E <= 64*NE); every partial load is issued before any sum,
// and each expert's partials are added in ascending split order.
template <int NE, int KS>
__device__ __forceinline__ void wave_topk(const float* __restrict__ part, int E, int k, int t,
                                          int32_t* idx_row, float* w_row) {
    static_assert(KS == 1 || KS % 4 == 0, "partials per expert: 1 or a multiple of 4");
    const int lane = threadIdx.x & 63;
    float pv[NE][KS];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int e = min(lane + 64 * i, E - 1);   // clamped; masked below
        const float* p = part + ((size_t)t * E + e) * KS;
        if (KS == 1) {
            pv[i][0] = p[0];
        } else {
#pragma unroll
            for (int q = 0; q < KS / 4; ++q) {
                const float4 f = reinterpret_cast<const float4*>(p)[q];
                pv[i][4 * q] = f.x;
                pv[i][4 * q + 1] = f.y;
                pv[i][4 * q + 2] = f.z;
                pv[i][4 * q + 3] = f.w;
            }
        }
    }
    float l[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        float s = pv[i][0];
#pragma unroll
        for (int q = 1; q < KS; ++q) s += pv[i][q];
        if (s != s) s = -INFINITY;   // a NaN logit is never preferred
        l[i] = lane + 64 * i < E ? s : -INFINITY;
    }
    uint32_t taken = 0;
    float my_l = -INFINITY;   // lane j keeps slot j
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((taken >> i) & 1u) && better(l[i], e, bv, be)) {
                bv = l[i];
                be = e;
            }
        }
        wave_argmax(bv, be);
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (lane == j) {
            my_l = bv;
            my_e = be;
        }
    }
    // softmax of the selected logits (= the full softmax renormalised over
    // them); the butterfly gives every lane the same sum
    const float mx = __shfl(my_l, 0, 64);
    const float ex = lane < k ? expf(my_l - mx) : 0.f;
    float z = ex;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off, 64);
    if (lane < k) {
        idx_row[lane] = my_e;
        w_row[lane] = ex / z;
    }
}

}  // namespace moe
