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

// Logits are ranked as int32 keys with the same order as the floats: the
// bits of a non-negative float, and for a negative one the bits with the
// magnitude field flipped.  -0 is first made +0 (they compare equal), a NaN
// logit ranks as -inf, and INT32_MIN (below -inf's key) marks an expert that
// is taken or does not exist.
__device__ __forceinline__ int logit_key(float f) {
    if (f != f) f = -INFINITY;
    const int i = __builtin_bit_cast(int, f + 0.0f);
    return i < 0 ? i ^ 0x7fffffff : i;
}
__device__ __forceinline__ float key_logit(int k) {
    return __builtin_bit_cast(float, k < 0 ? k ^ 0x7fffffff : k);
}
constexpr int kKeyNone = (int)0x80000000;
constexpr int kFastK = 8;   // slots the branch-free selection pass covers

// Wave-wide maximum of int keys, returned wave-uniform: within each 16-lane
// row by DPP moves (xor 1, xor 2, half-row mirror, row mirror), then row 0
// into row 1 and row 2 into row 3 (row_bcast:15), rows 0-1 into rows 2-3
// (row_bcast:31), and lane 63 read out.
// Lanes that a step's row mask leaves out read INT32_MIN, the identity of max.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_max_step(int v) {
    return max(v, __builtin_amdgcn_update_dpp(kKeyNone, v, CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ int wave_max_key(int v) {
    v = dpp_max_step<0xB1, 0xf>(v);    // quad_perm [1,0,3,2]
    v = dpp_max_step<0x4E, 0xf>(v);    // quad_perm [2,3,0,1]
    v = dpp_max_step<0x141, 0xf>(v);   // row_half_mirror
    v = dpp_max_step<0x140, 0xf>(v);   // row_mirror
    v = dpp_max_step<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
    v = dpp_max_step<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
    return __builtin_amdgcn_readlane(v, 63);
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

// part: [T][E][KS] partial logits.  Fills the first k slots of token t (a
// caller that needs only slot j passes k = j + 1: the rounds are greedy, so
// the first slots do not depend on how many follow).  Lane l holds experts l, l+64,
// ... (NE per lane: E <= 64*NE); every partial load is issued before any sum,
// and each expert's partials are added in ascending split order.
//
// Each round takes the wave maximum m of the remaining keys and gives the
// next slot to the lowest-indexed expert holding m (ballots of key == m in
// scalar registers), so tied experts fill consecutive slots in ascending
// index and a tie group larger than the slots left is cut at the lowest
// indices.  The selected expert's key becomes INT32_MIN.  For k <= kFastK a
// branch-free pass runs first and the exact rounds run only after a tie.  A NaN logit counts as
// -inf: never preferred over a number.  Lane j keeps slot j (its logit in
// my_l, its expert in my_e); top is the largest logit.
template <int NE, int KS>
__device__ __forceinline__ void wave_topk_select(const float* __restrict__ part, int E, int k,
                                                 int t, float& my_l, int& my_e, float& top) {
    static_assert(KS == 1 || KS == 2 || KS % 4 == 0, "partials per expert: 1, 2 or a multiple of 4");
    static_assert(NE <= 16, "at most 1024 experts");
    const int lane = threadIdx.x & 63;
    float pv[NE][KS];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int e = min(lane + 64 * i, E - 1);   // clamped; masked below
        const float* p = part + ((size_t)t * E + e) * KS;
        if (KS == 1) {
            pv[i][0] = p[0];
        } else if (KS == 2) {
            const float2 f = *reinterpret_cast<const float2*>(p);
            pv[i][0] = f.x;
            pv[i][KS - 1] = f.y;
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
    int key[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        float s = pv[i][0];
#pragma unroll
        for (int q = 1; q < KS; ++q) s += pv[i][q];
        key[i] = lane + 64 * i < E ? logit_key(s) : kKeyNone;
    }
    my_l = -INFINITY;
    top = 0.f;
    my_e = 0;
    if (k <= kFastK) {
        // fast pass: unrolled rounds without data-dependent branches.  A
        // round clears every holder of the maximum by value, so the next
        // round's maximum waits only for the compare and the clear; the slot
        // bookkeeping (the holder's index from the ballots, in scalar
        // registers) runs beside it.  A round with more than one holder is a
        // tie: the exact pass below then reruns the selection.
        int kept[NE];
#pragma unroll
        for (int i = 0; i < NE; ++i) kept[i] = key[i];
        bool tie = false;
        int m = key[0];
#pragma unroll
        for (int i = 1; i < NE; ++i) m = max(m, key[i]);
        m = wave_max_key(m);
        top = key_logit(m);
#pragma unroll
        for (int j = 0; j < kFastK; ++j) {
            int e = 0, hits = 0;
#pragma unroll
            for (int i = NE - 1; i >= 0; --i) {
                const bool hit = key[i] == m;
                const uint64_t bl = __builtin_amdgcn_ballot_w64(hit);
                if (hit) key[i] = kKeyNone;
                hits += __builtin_popcountll(bl);
                if (bl != 0) e = (int)__builtin_ctzll(bl) + 64 * i;
            }
            // the next round's maximum comes before this round's exit test,
            // so the scalar bookkeeping below shares its straight-line block
            int mn = key[0];
#pragma unroll
            for (int i = 1; i < NE; ++i) mn = max(mn, key[i]);
            mn = wave_max_key(mn);
            asm volatile("" ::"s"(mn));   // keeps it above the exit test (no sinking)
            tie |= hits != 1;
            const bool mine = lane == j;   // selects, not a branch: nothing waits for e
            my_l = mine ? key_logit(m) : my_l;
            my_e = mine ? e : my_e;
            if (j + 1 == k) break;
            m = mn;
        }
        if (!tie) return;
#pragma unroll
        for (int i = 0; i < NE; ++i) key[i] = kept[i];
        my_l = -INFINITY;
        my_e = 0;
    }
    // exact pass: one expert per round, the lowest index holding the maximum
    for (int j = 0; j < k; ++j) {   // j: slots filled (wave-uniform)
        int m = key[0];
#pragma unroll
        for (int i = 1; i < NE; ++i) m = max(m, key[i]);
        m = wave_max_key(m);
        if (m == kKeyNone) break;   // nothing left (cannot happen for k <= E)
        const float ml = key_logit(m);
        if (j == 0) top = ml;
        int e = 0;
#pragma unroll
        for (int i = NE - 1; i >= 0; --i) {
            const uint64_t bl = __builtin_amdgcn_ballot_w64(key[i] == m);
            if (bl != 0) e = (int)__builtin_ctzll(bl) + 64 * i;
        }
#pragma unroll
        for (int i = 0; i < NE; ++i)
            if (lane + 64 * i == e) key[i] = kKeyNone;
        if (lane == j) {
            my_l = ml;
            my_e = e;
        }
    }
}

// The selection plus the routing weights: the softmax of the selected logits
// (= the full softmax renormalised over them); k <= 16, so the slots sit in
// row 0.
// Returns, in lane j, slot j's expert.
template <int NE, int KS>
__device__ __forceinline__ int wave_topk(const float* __restrict__ part, int E, int k, int t,
                                         int32_t* idx_row, float* w_row) {
    const int lane = threadIdx.x & 63;
    float my_l, top;
    int my_e;
    wave_topk_select<NE, KS>(part, E, k, t, my_l, my_e, top);
    const float ex = lane < k ? expf(my_l - top) : 0.f;
    const float z = row_sum(ex);
    if (lane < k) {
        idx_row[lane] = my_e;
        w_row[lane] = ex / z;
    }
    return my_e;
}

}  // namespace moe
