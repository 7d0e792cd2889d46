// router.hip -- fp32 router GEMM, top-k and renormalised routing weights.
//
// Page "CKE Zip: From Splitting Tokens To Splitting Qwen3.5 Weights", sections
// "What The First Prototype Split" (the selected top-k expert indices and
// their routing weights travel with each hidden row) and "What PR #382 Now
// Splits" (eight of 256 experts per token; one synchronised router decision
// feeds every shard).
//
// Two kernels:
//   router_partial  logits partial sums over a slice of H for a tile of tokens
//                   (split-K across many workgroups so that a single decode
//                   token still spreads the 2 MiB router matrix over the chip);
//   router_topk     per token (one wave): sum the partials in ascending split
//                   order, k rounds of a wave-wide arg-max (ties to the lower
//                   expert index), softmax of the k selected logits.
#include "moe_internal.h"

namespace moe {

constexpr int kRouterTT = 16;      // tokens per workgroup
constexpr int kRouterChunk = 128;  // rows of H staged in LDS at a time

int router_splits(int T, int H) {
    // enough workgroups to cover the chip; each split handles >= 16 rows of H
    const int tblocks = (T + kRouterTT - 1) / kRouterTT;
    int ks = 512 / (tblocks > 0 ? tblocks : 1);
    const int kmax = H / 16;
    if (ks > kmax) ks = kmax;
    if (ks < 1) ks = 1;
    return ks;
}

__global__ void __launch_bounds__(256)
router_partial_kernel(const float* __restrict__ x, const float* __restrict__ wr, int T, int H,
                      int E, int rows_per_split, float* __restrict__ part) {
    __shared__ float xs[kRouterTT][kRouterChunk];
    const int t0 = blockIdx.x * kRouterTT;
    const int ks = blockIdx.y;
    const int h0 = ks * rows_per_split;
    const int h1 = min(H, h0 + rows_per_split);
    const int nt = min(kRouterTT, T - t0);

    for (int e0 = 0; e0 < E; e0 += blockDim.x) {
        const int e = e0 + threadIdx.x;
        float acc[kRouterTT];
#pragma unroll
        for (int i = 0; i < kRouterTT; ++i) acc[i] = 0.f;
        for (int hc = h0; hc < h1; hc += kRouterChunk) {
            const int hn = min(kRouterChunk, h1 - hc);
            __syncthreads();
            for (int i = threadIdx.x; i < kRouterTT * kRouterChunk; i += blockDim.x) {
                const int tt = i / kRouterChunk, hh = i % kRouterChunk;
                xs[tt][hh] = (tt < nt && hh < hn) ? x[(size_t)(t0 + tt) * H + hc + hh] : 0.f;
            }
            __syncthreads();
            if (e < E) {
                for (int hh = 0; hh < hn; ++hh) {
                    const float wv = wr[(size_t)(hc + hh) * E + e];
#pragma unroll
                    for (int i = 0; i < kRouterTT; ++i) acc[i] = __builtin_fmaf(xs[i][hh], wv, acc[i]);
                }
            }
        }
        if (e < E) {
            for (int i = 0; i < nt; ++i) part[((size_t)ks * T + t0 + i) * E + e] = acc[i];
        }
    }
}

// One wave per token.  Lane l holds experts l, l+64, ... (E <= 1024).
__global__ void __launch_bounds__(256)
router_topk_kernel(const float* __restrict__ part, int ks_n, int T, int E, int k,
                   int32_t* __restrict__ idx, float* __restrict__ w) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (t >= T) return;
    float l[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = lane + 64 * i;
        float s = -INFINITY;
        if (e < E) {
            s = 0.f;
            for (int ks = 0; ks < ks_n; ++ks) s += part[((size_t)ks * T + t) * E + e];
            if (s != s) s = -INFINITY;  // a NaN logit is never preferred
        }
        l[i] = s;
    }
    uint32_t taken = 0;
    float sel_l[16];
    int sel_e[16];
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((taken >> i) & 1u) && (l[i] > bv || (l[i] == bv && e < be))) {
                bv = l[i];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oe = __shfl_xor(be, off, 64);
            if (ov > bv || (ov == bv && oe < be)) {
                bv = ov;
                be = oe;
            }
        }
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        sel_l[j] = bv;
        sel_e[j] = be;
    }
    if (lane == 0) {
        const float mx = sel_l[0];
        float ex[16];
        float z = 0.f;
        for (int j = 0; j < k; ++j) {
            ex[j] = expf(sel_l[j] - mx);
            z += ex[j];
        }
        const float inv = 1.0f / z;
        for (int j = 0; j < k; ++j) {
            idx[(size_t)t * k + j] = sel_e[j];
            w[(size_t)t * k + j] = ex[j] * inv;
        }
    }
}

hipError_t launch_router(const moe_layer_desc& d, const float* x, int T, int32_t* idx, float* w,
                         char* ws, const WsLayout& L, hipStream_t s) {
    const int H = d.hidden, E = d.n_experts;
    const int ks = L.router_ks;
    const int rows = (H + ks - 1) / ks;
    float* part = reinterpret_cast<float*>(ws + L.router_part);
    dim3 g1((T + kRouterTT - 1) / kRouterTT, ks);
    const int threads = E < 256 ? ((E + 63) / 64) * 64 : 256;
    router_partial_kernel<<<g1, threads, 0, s>>>(x, d.router_w, T, H, E, rows, part);
    router_topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(part, ks, T, E, d.top_k, idx, w);
    return hipGetLastError();
}

}  // namespace moe
