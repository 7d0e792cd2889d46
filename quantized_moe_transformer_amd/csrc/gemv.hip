// gemv.hip -- decode path: fused K-quant dequant-GEMV, fp32 accumulation.
//
// At one (or a few) token rows the layer is a stream of packed weight bytes:
// each byte is read once and used once, so the work is bound by HBM
// bandwidth (page "Distributed CPU: Zip Fusion Beyond Tensor Parallelism",
// section "Decode vs Prefill: Same Weights, Different Bottlenecks").  The
// kernels stream the superblocks of the selected experts with 16-byte loads,
// unpack the 6-bit scales/mins and the codes in registers and reduce across
// lanes of the wavefront.
//
// Work unit of a lane: a 16-byte piece of a superblock's codes -- 32 weights,
// 16 from sub-block 2c and 16 from sub-block 2c+1 -- plus the superblock's
// 16-byte head (and, at 5 bits, the matching 16 bytes of high bits).  Eight
// lanes cover one superblock, so the lanes of a wave read one contiguous run
// of a row.  The per-sub-block scale factors out of the dot product:
//   sum_i w_i x_i = d*sc_a*sum(q x)_a + d*sc_b*sum(q x)_b - dmin*(m_a sum x_a + m_b sum x_b)
//
//   gateup_gemv  h[p][r] = silu(Wg[r] . x) * (Wu[r] . x) for every selected
//                expert instance p = (token, slot) and the shared expert
//   down_gemv    out[t][o] = sum_j w_j (Wd_j[o] . h_j) + sw (Wd_sh[o] . h_sh),
//                slots in selected-slot order, shared expert last (page "CKE
//                Zip ...", section "A Separate Decode Result Shows Why Axis
//                Choice Matters": routes merged in the original slot order)
#include "moe_internal.h"

namespace moe {

// Partial dot product of one lane's piece.  xl/xh: the 16 activations under
// the low / high nibbles; sl/sh their sums.  qh: the 16 high-bit bytes of the
// piece (5-bit format) or nullptr-equivalent (HIGH = false).
template <bool HIGH>
__device__ __forceinline__ float piece_dot(const SbHead& h, const uint4& qs, const uint4& qh, int c,
                                           const float* xl, const float* xh, float sl, float sh) {
    float sca, ma, scb, mb;
    sub_scale_min(h, 2 * c, sca, ma);
    sub_scale_min(h, 2 * c + 1, scb, mb);
    float dl = 0.f, dh = 0.f;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
        const uint32_t byte = piece_byte(qs, b);
        uint32_t ql = byte & 15u, qq = byte >> 4;
        if (HIGH) {
            const uint32_t hb = piece_byte(qh, b);
            ql |= ((hb >> (2 * c)) & 1u) << 4;
            qq |= ((hb >> (2 * c + 1)) & 1u) << 4;
        }
        dl = __builtin_fmaf((float)ql, xl[b], dl);
        dh = __builtin_fmaf((float)qq, xh[b], dh);
    }
    return h.d * (sca * dl + scb * dh) - h.dmin * (ma * sl + mb * sh);
}

__device__ __forceinline__ void load16(const float* p, float* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 f = reinterpret_cast<const float4*>(p)[i];
        v[4 * i + 0] = f.x;
        v[4 * i + 1] = f.y;
        v[4 * i + 2] = f.z;
        v[4 * i + 3] = f.w;
    }
}

// LPR: lanes per row (8 * superblocks per row, capped at 64); NSBL:
// superblocks per lane per row (H / 2048 when LPR = 64, else 1).
template <int LPR, int NSBL>
__global__ void __launch_bounds__(256)
gateup_gemv_kernel(const uint8_t* __restrict__ gate, const uint8_t* __restrict__ up,
                   const uint8_t* __restrict__ sh_gate, const uint8_t* __restrict__ sh_up,
                   const float* __restrict__ x, const int32_t* __restrict__ idx, int H, int E,
                   int k, int I, int Is, int shard, int nshards, int nslot,
                   float* __restrict__ hbuf, int hstride) {
    constexpr int RS = 64 / LPR;   // rows side by side in a wave
    constexpr int RPW = 2;         // row steps per wave
    const int p = blockIdx.y;
    const int t = p / nslot, j = p % nslot;
    const uint8_t *G, *U;
    int Iexp;
    if (j < k) {
        const int e = idx[(size_t)t * k + j];
        if ((unsigned)e >= (unsigned)E) return;
        const size_t mat = (size_t)I * H / kSbWeights * kQ4Bytes;
        G = gate + (size_t)e * mat;
        U = up + (size_t)e * mat;
        Iexp = I;
    } else {
        G = sh_gate;
        U = sh_up;
        Iexp = Is;
    }
    const int Iloc = Iexp / nshards, i0 = shard * Iloc;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rslot = lane / LPR, task = lane % LPR;
    const int sbi = task >> 3, piece = task & 7, c = piece >> 1, hh = piece & 1;
    const int nsb_row = H / kSbWeights;

    const float* xt = x + (size_t)t * H;
    float xl[NSBL][16], xh[NSBL][16], sl[NSBL], sh[NSBL];
#pragma unroll
    for (int it = 0; it < NSBL; ++it) {
        const int sb = sbi + (LPR / 8) * it;
        const float* xp = xt + sb * kSbWeights + 64 * c + 16 * hh;
        load16(xp, xl[it]);
        load16(xp + 32, xh[it]);
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            a += xl[it][q];
            b += xh[it][q];
        }
        sl[it] = a;
        sh[it] = b;
    }

    const int rbase = (blockIdx.x * 4 + wave) * RPW * RS;
    float g[RPW], u[RPW];
#pragma unroll
    for (int st = 0; st < RPW; ++st) {
        const int r = rbase + st * RS + rslot;
        float pg = 0.f, pu = 0.f;
        if (r < Iloc) {
            const size_t row = (size_t)(i0 + r) * nsb_row;
#pragma unroll
            for (int it = 0; it < NSBL; ++it) {
                const int sb = sbi + (LPR / 8) * it;
                const uint8_t* gs = G + (row + sb) * kQ4Bytes;
                const uint8_t* us = U + (row + sb) * kQ4Bytes;
                const SbHead hg = load_head(gs);
                const SbHead hu = load_head(us);
                const uint4 qg = *reinterpret_cast<const uint4*>(gs + 16 + 32 * c + 16 * hh);
                const uint4 qu = *reinterpret_cast<const uint4*>(us + 16 + 32 * c + 16 * hh);
                pg += piece_dot<false>(hg, qg, qg, c, xl[it], xh[it], sl[it], sh[it]);
                pu += piece_dot<false>(hu, qu, qu, c, xl[it], xh[it], sl[it], sh[it]);
            }
        }
        g[st] = pg;
        u[st] = pu;
    }
#pragma unroll
    for (int st = 0; st < RPW; ++st) {
        const float gs = wave_sum_group(g[st], LPR);
        const float us = wave_sum_group(u[st], LPR);
        const int r = rbase + st * RS + rslot;
        if (task == 0 && r < Iloc) hbuf[(size_t)p * hstride + r] = silu_f(gs) * us;
    }
}

// One wave per RSd = 64 / LPRd output rows of one token; LPRd = I_loc / 32.
__global__ void __launch_bounds__(64)
down_gemv_kernel(const uint8_t* __restrict__ down, const uint8_t* __restrict__ sh_down,
                 const float* __restrict__ hbuf, int hstride, const int32_t* __restrict__ idx,
                 const float* __restrict__ w, float sw, int H, int E, int k, int I, int Is,
                 int shard, int nshards, int nslot, int lprd, float* __restrict__ out) {
    const int t = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int rslot = lane / lprd, task = lane % lprd;
    const int cg = task >> 1, hh = task & 1;
    const int o = blockIdx.x * (64 / lprd) + rslot;
    float acc = 0.f;
    for (int j = 0; j < nslot; ++j) {
        const uint8_t* D;
        float wj;
        int Iexp;
        if (j < k) {
            const int e = idx[(size_t)t * k + j];
            if ((unsigned)e >= (unsigned)E) continue;
            D = down + (size_t)e * ((size_t)H * I / kSbWeights * kQ5Bytes);
            wj = w[(size_t)t * k + j];
            Iexp = I;
        } else {
            D = sh_down;
            wj = sw;
            Iexp = Is;
        }
        const int Iloc = Iexp / nshards, i0 = shard * Iloc;
        float part = 0.f;
        if (o < H) {
            const size_t base = (size_t)o * Iexp + i0 + 64 * cg;
            const int c = (int)((base & 255) >> 6);
            const uint8_t* sb = D + (base >> 8) * kQ5Bytes;
            const SbHead hd = load_head(sb);
            const uint4 qh = *reinterpret_cast<const uint4*>(sb + 16 + 16 * hh);
            const uint4 qs = *reinterpret_cast<const uint4*>(sb + 48 + 32 * c + 16 * hh);
            const float* hp = hbuf + (size_t)(t * nslot + j) * hstride + 64 * cg + 16 * hh;
            float hl[16], hu[16];
            load16(hp, hl);
            load16(hp + 32, hu);
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                a += hl[q];
                b += hu[q];
            }
            part = piece_dot<true>(hd, qs, qh, c, hl, hu, a, b);
        }
        const float y = wave_sum_group(part, lprd);
        acc = __builtin_fmaf(wj, y, acc);
    }
    if (task == 0 && o < H) out[(size_t)t * H + o] = acc;
}

template <int LPR, int NSBL>
static void launch_gateup(const moe_layer_desc& d, const float* x, int T, const int32_t* idx,
                          int shard, int nshards, int nslot, float* hbuf, int hstride,
                          hipStream_t s) {
    constexpr int rows_per_block = 4 * 2 * (64 / LPR);
    const int Imax = (d.inter > d.shared_inter ? d.inter : d.shared_inter) / nshards;
    dim3 grid((Imax + rows_per_block - 1) / rows_per_block, T * nslot);
    gateup_gemv_kernel<LPR, NSBL><<<grid, 256, 0, s>>>(
        d.gate_q, d.up_q, d.sh_gate_q, d.sh_up_q, x, idx, d.hidden, d.n_experts, d.top_k,
        d.inter, d.shared_inter, shard, nshards, nslot, hbuf, hstride);
}

hipError_t launch_gemv(const moe_layer_desc& d, const float* x, int T, const int32_t* idx,
                       const float* w, int shard, int nshards, float* out, char* ws,
                       const WsLayout& L, hipStream_t s, const PhaseMarks& pm) {
    const int nslot = d.top_k + (d.shared_inter > 0 ? 1 : 0);
    const int Iloc = d.inter / nshards;
    float* hbuf = reinterpret_cast<float*>(ws + L.hbuf);
    const int nsb_row = d.hidden / kSbWeights;
    switch (nsb_row) {
        case 1: launch_gateup<8, 1>(d, x, T, idx, shard, nshards, nslot, hbuf, Iloc, s); break;
        case 2: launch_gateup<16, 1>(d, x, T, idx, shard, nshards, nslot, hbuf, Iloc, s); break;
        case 4: launch_gateup<32, 1>(d, x, T, idx, shard, nshards, nslot, hbuf, Iloc, s); break;
        case 8: launch_gateup<64, 1>(d, x, T, idx, shard, nshards, nslot, hbuf, Iloc, s); break;
        case 16: launch_gateup<64, 2>(d, x, T, idx, shard, nshards, nslot, hbuf, Iloc, s); break;
        default: return hipErrorInvalidValue;
    }
    pm.mark(2);
    const int lprd = Iloc / 32;
    dim3 grid2((d.hidden + (64 / lprd) - 1) / (64 / lprd), T);
    down_gemv_kernel<<<grid2, 64, 0, s>>>(d.down_q, d.sh_down_q, hbuf, Iloc, idx, w,
                                          d.shared_weight, d.hidden, d.n_experts, d.top_k,
                                          d.inter, d.shared_inter, shard, nshards, nslot, lprd,
                                          out);
    pm.mark(3);
    return hipGetLastError();
}

}  // namespace moe
