// topk.h -- one wavefront routes one token: logits (summed from split-K
// partials in a fixed order), k rounds of a wave-wide maximum with ties to
// the lower expert index, and the softmax of the k selected logits.
//
// Page "CKE Zip: From Splitting Tokens To Splitting Qwen3.5 Weights", sections
// "What The First Prototype Split" (indices and routing weights travel with
// each row) and "What PR #382 Now Splits" (top eight of 256 experts).
#pragma once

#include "moe_internal.h"

namespace moe {

// Wave-wide maximum of v (every lane gets it): within each 16-lane row by DPP
// moves (xor 1, xor 2, half-row mirror, row mirror), then across the four
// rows through lane reads.  fmaxf ignores NaN operands.
__device__ __forceinline__ float readlane_f(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_mov_f<0xB1>(v));    // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_mov_f<0x4E>(v));    // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_mov_f<0x141>(v));   // row_half_mirror
    v = fmaxf(v, dpp_mov_f<0x140>(v));   // row_mirror
    return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
                 fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

// Sum over lanes 0-15 (row 0), the same bits in each of them: each step adds
// two equal-sized groups that mirror each other, and a + b == b + a.
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_mov_f<0xB1>(v);
    v += dpp_mov_f<0x4E>(v);
    v += dpp_mov_f<0x141>(v);
    v += dpp_mov_f<0x140>(v);
    return v;
}

// part: [T][E][KS] partial logits.  Writes the k slots of token t to
// idx_row[0..k), w_row[0..k) (global or LDS).  Lane l holds experts l, l+64,
// ... (NE per lane: E <= 64*NE); every partial load is issued before any sum,
// and each expert's partials are added in ascending split order.
//
// Each of the k rounds takes the wave maximum m of the remaining logits, then
// the lowest expert index holding m (ballots of l == m, scanned from the
// lowest expert block), so ties go to the lower index; the winner's logit is
// replaced by NaN, which the maximum ignores and no compare matches.  A NaN
// logit counts as -inf: never preferred over a number.  Lane j keeps slot j.
template <int NE, int KS>
__device__ __forceinline__ void wave_topk(const float* __restrict__ part, int E, int k, int t,
                                          int32_t* idx_row, float* w_row) {
    static_assert(KS == 1 || KS % 4 == 0, "partials per expert: 1 or a multiple of 4");
    static_assert(NE <= 16, "at most 1024 experts");
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
    const float qnan = __builtin_nanf("");
    float l[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        float s = pv[i][0];
#pragma unroll
        for (int q = 1; q < KS; ++q) s += pv[i][q];
        if (s != s) s = -INFINITY;
        l[i] = lane + 64 * i < E ? s : qnan;
    }
    float my_l = -INFINITY, top = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float m = l[0];
#pragma unroll
        for (int i = 1; i < NE; ++i) m = fmaxf(m, l[i]);
        m = wave_max(m);
        if (j == 0) top = m;
        int wi = 0;
        uint64_t wb = 0;
#pragma unroll
        for (int i = NE - 1; i >= 0; --i) {
            const uint64_t b = __builtin_amdgcn_ballot_w64(l[i] == m);
            if (b) {
                wi = i;
                wb = b;
            }
        }
        const int wl = wb ? (int)__builtin_ctzll(wb) : 0;
#pragma unroll
        for (int i = 0; i < NE; ++i)
            if (i == wi && lane == wl) l[i] = qnan;
        if (lane == j) {
            my_l = m;
            my_e = wl + 64 * wi;
        }
    }
    // softmax of the selected logits (= the full softmax renormalised over
    // them); k <= 16, so the slots sit in row 0
    const float ex = lane < k ? expf(my_l - top) : 0.f;
    const float z = row_sum(ex);
    if (lane < k) {
        idx_row[lane] = my_e;
        w_row[lane] = ex / z;
    }
}

}  // namespace moe
