// router.hip -- fp32 router logits, top-k and renormalised routing weights.
//
// Page "CKE Zip: From Splitting Tokens To Splitting Qwen3.5 Weights", sections
// "What The First Prototype Split" (the selected top-k expert indices and
// their routing weights travel with each hidden row) and "What PR #382 Now
// Splits" (eight of 256 experts per token; one synchronised router decision
// feeds every shard).
//
// Logits stay fp32 throughout (the top-k must be exact up to near-ties).
// Few token rows (<= 32): split-K partial logits from the decode front
// kernel (gemv.hip), then router_topk.  Many rows use:
//   router_mfma     a dense [T x H] x [H x E] product on the fp32 matrix cores
//                   (v_mfma_f32_16x16x4_f32);
//   router_topk     one wave per token (topk.h).
#include "moe_internal.h"
#include "topk.h"

namespace moe {

int router_splits(int T, int H) { return T <= kGemvMaxT ? kRouterSplits : 1; }

// grid (ceil(T/16), ceil(E/256)); block 512 threads = 8 waves; the block owns
// 16 tokens x 256 experts, wave w the experts [32w, 32w+32) as two 16x16 tiles.
// K advances 32 at a time; the next step's operands are fetched into
// registers while the current step runs on the matrix cores.
constexpr int kRmT = 16, kRmE = 256, kRmK = 32;

__global__ void __launch_bounds__(512)
router_mfma_kernel(const float* __restrict__ x, const float* __restrict__ wr, int T, int H, int E,
                   float* __restrict__ logits) {
    __shared__ float xs[kRmT][kRmK + 1];
    __shared__ float ws[kRmK][kRmE + 4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * kRmT, e0 = blockIdx.y * kRmE;
    // loaders: x one float per thread; Wr four float4 per thread
    const int xt = tid >> 5, xk = tid & 31;
    const bool xok = t0 + xt < T;
    float xr;
    float4 wv[4];
    auto fetch = [&](int k0) {
        xr = xok ? x[(size_t)(t0 + xt) * H + k0 + xk] : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int f = tid + 512 * q;
            const int r = f >> 6, c4 = (f & 63) * 4;
            const int e = e0 + c4;
            const float* row = wr + (size_t)(k0 + r) * E;
            if ((E & 3) == 0 && e + 3 < E) {
                wv[q] = *reinterpret_cast<const float4*>(row + e);
            } else {
                wv[q].x = e < E ? row[e] : 0.f;
                wv[q].y = e + 1 < E ? row[e + 1] : 0.f;
                wv[q].z = e + 2 < E ? row[e + 2] : 0.f;
                wv[q].w = e + 3 < E ? row[e + 3] : 0.f;
            }
        }
    };
    fetch(0);
    float4v acc[2] = {};
    for (int k0 = 0; k0 < H; k0 += kRmK) {
        __syncthreads();
        xs[xt][xk] = xr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int f = tid + 512 * q;
            *reinterpret_cast<float4*>(&ws[f >> 6][(f & 63) * 4]) = wv[q];
        }
        __syncthreads();
        if (k0 + kRmK < H) fetch(k0 + kRmK);
#pragma unroll
        for (int ks = 0; ks < kRmK / 4; ++ks) {
            const float a = xs[lane & 15][ks * 4 + (lane >> 4)];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const float bv = ws[ks * 4 + (lane >> 4)][wave * 32 + b * 16 + (lane & 15)];
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv, acc[b], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int e = e0 + wave * 32 + b * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 4 * (lane >> 4) + i;
            if (t < T && e < E) logits[(size_t)t * E + e] = acc[b][i];
        }
    }
}

// Four tokens per workgroup, one wave each.
__global__ void __launch_bounds__(256)
router_topk_kernel(const float* __restrict__ part, int ks_n, int T, int E, int k,
                   int32_t* __restrict__ idx, float* __restrict__ w) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int32_t* ir = idx + (size_t)t * k;
    float* wr = w + (size_t)t * k;
    if (ks_n == 1) {
        if (E <= 256) wave_topk<4, 1>(part, E, k, t, ir, wr);
        else wave_topk<16, 1>(part, E, k, t, ir, wr);
    } else {
        if (E <= 256) wave_topk<4, kRouterSplits>(part, E, k, t, ir, wr);
        else wave_topk<16, kRouterSplits>(part, E, k, t, ir, wr);
    }
}

hipError_t launch_router_small(const moe_layer_desc& d, const float* x, int T, char* ws,
                               const WsLayout& L, const Ctx& c);   // gemv.hip: partials only

hipError_t launch_router(const moe_layer_desc& d, const float* x, int T, int32_t* idx, float* w,
                         char* ws, const WsLayout& L, const Ctx& c) {
    const int H = d.hidden, E = d.n_experts;
    float* part = reinterpret_cast<float*>(ws + L.router_part);
    if (T <= kGemvMaxT) {
        hipError_t e = launch_router_small(d, x, T, ws, L, c);
        if (e != hipSuccess) return e;
        launch_k(c, MOE_K_ROUTER_TOPK, router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, part,
                 L.router_ks, T, E, d.top_k, idx, w);
        return hipGetLastError();
    }
    dim3 g((T + kRmT - 1) / kRmT, (E + kRmE - 1) / kRmE);
    launch_k(c, MOE_K_ROUTER_MFMA, router_mfma_kernel, g, dim3(512), 0, x, d.router_w, T, H, E,
             part);
    launch_k(c, MOE_K_ROUTER_TOPK, router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, part, 1,
             T, E, d.top_k, idx, w);
    return hipGetLastError();
}

}  // namespace moe
