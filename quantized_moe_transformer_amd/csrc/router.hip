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
//   x_split, w_split, router_gemm  a dense [T x H] x [H x E] product on the
//                   fp16 matrix cores with split operands (fp32 accuracy);
//   router_topk     one wave per token (topk.h).
#include "moe_internal.h"
#include "topk.h"

namespace moe {

int router_splits(int T, int H) { return T <= kGemvMaxT ? kRouterSplits : 1; }

// ---------------------------------------------------------------------------
// Many rows: logits on the fp16 matrix cores with fp32 accuracy.  Each fp32
// operand v is split into two fp16 parts, hi = fp16(v) and
// lo = fp16((v - hi) * 2^11): v - hi is exact in fp32 and at most 2^-11 |v|, so
// the scaled remainder sits in fp16's normal range whenever hi does, and
// v = hi + 2^-11 lo to within 2^-22 |v|.  Then
//   x . w = x_hi . w_hi + 2^-11 (x_hi . w_lo + x_lo . w_hi)  (+ 2^-22 x_lo . w_lo, dropped)
// with exact fp16 products accumulated in two fp32 accumulators.  The router
// matrix is scaled by 2^10 before the split (exact) so that its small entries
// keep normal fp16 high parts, and the logits by 2^-10 after.  Requires
// |x| < 65504 and |w| < 64.
// ---------------------------------------------------------------------------
constexpr float kWrScale = 1024.0f, kLoScale = 2048.0f;
constexpr int kRgT = 32, kRgE = 128, kRgK = 64, kRgRow = kRgK + 8;

// x fp32 [T][H] -> hi (x16, also the grouped GEMM's operand) and lo parts
__global__ void __launch_bounds__(256)
x_split_kernel(const float* __restrict__ x, _Float16* __restrict__ xh, _Float16* __restrict__ xl,
               size_t n4) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const float4 v = reinterpret_cast<const float4*>(x)[i];
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    half4 h, l;
    const float f[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        h[j] = (_Float16)f[j];
        l[j] = (_Float16)((f[j] - (float)h[j]) * kLoScale);
    }
    reinterpret_cast<half4*>(xh)[i] = h;
    if (xl) reinterpret_cast<half4*>(xl)[i] = l;
}

// router matrix fp32 [H][E] -> 2^10 * (hi, lo) parts, transposed to [E][H]
__global__ void __launch_bounds__(256)
w_split_kernel(const float* __restrict__ wr, int H, int E, _Float16* __restrict__ wh,
               _Float16* __restrict__ wl) {
    __shared__ float tile[32][33];
    const int h0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
    for (int r = ty; r < 32; r += 8) {
        const int h = h0 + r, e = e0 + tx;
        tile[r][tx] = (h < H && e < E) ? wr[(size_t)h * E + e] * kWrScale : 0.f;
    }
    __syncthreads();
    for (int r = ty; r < 32; r += 8) {
        const int e = e0 + r, h = h0 + tx;
        if (e < E && h < H) {
            const float v = tile[tx][r];
            const _Float16 hi = (_Float16)v;
            wh[(size_t)e * H + h] = hi;
            wl[(size_t)e * H + h] = (_Float16)((v - (float)hi) * kLoScale);
        }
    }
}

// grid (ceil(T/32), ceil(E/128)); 4 waves, wave w owns experts [32w, 32w+32)
// of the block's 128.  K advances 64 at a time; the next step's operands are
// fetched into registers while the current one runs on the matrix cores.
__global__ void __launch_bounds__(256)
router_gemm_kernel(const _Float16* __restrict__ xh, const _Float16* __restrict__ xl,
                   const _Float16* __restrict__ wh, const _Float16* __restrict__ wl, int T, int H,
                   int E, float* __restrict__ logits) {
    __shared__ _Float16 as[2][kRgT][kRgRow];    // [hi/lo][token][k]
    __shared__ _Float16 bs[2][kRgE][kRgRow];    // [hi/lo][expert][k]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * kRgT, e0 = blockIdx.y * kRgE;
    // loaders: A: 2 parts x 32 rows x 8 chunks = 512 chunks (2 per thread);
    //          B: 2 parts x 128 rows x 8 chunks = 2048 chunks (8 per thread)
    uint4 ra[2], rb[8];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int f = tid + 256 * q;
            const int part = f >> 8, r = (f >> 3) & 31, c8 = f & 7;
            const int t = t0 + r;
            const _Float16* src = part ? xl : xh;
            ra[q] = t < T ? *reinterpret_cast<const uint4*>(src + (size_t)t * H + k0 + c8 * 8)
                          : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int f = tid + 256 * q;
            const int part = f >> 10, r = (f >> 3) & 127, c8 = f & 7;
            const int e = e0 + r;
            const _Float16* src = part ? wl : wh;
            rb[q] = e < E ? *reinterpret_cast<const uint4*>(src + (size_t)e * H + k0 + c8 * 8)
                          : make_uint4(0, 0, 0, 0);
        }
    };
    fetch(0);
    float16v acc = {}, acc_lo = {};
    for (int k0 = 0; k0 < H; k0 += kRgK) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int f = tid + 256 * q;
            *reinterpret_cast<uint4*>(&as[f >> 8][(f >> 3) & 31][(f & 7) * 8]) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int f = tid + 256 * q;
            *reinterpret_cast<uint4*>(&bs[f >> 10][(f >> 3) & 127][(f & 7) * 8]) = rb[q];
        }
        __syncthreads();
        if (k0 + kRgK < H) fetch(k0 + kRgK);
#pragma unroll
        for (int s = 0; s < kRgK / 16; ++s) {
            const int kof = s * 16 + 8 * (lane >> 5);
            const half8 ah = *reinterpret_cast<const half8*>(&as[0][lane & 31][kof]);
            const half8 al = *reinterpret_cast<const half8*>(&as[1][lane & 31][kof]);
            const half8 bh = *reinterpret_cast<const half8*>(&bs[0][32 * wave + (lane & 31)][kof]);
            const half8 bl = *reinterpret_cast<const half8*>(&bs[1][32 * wave + (lane & 31)][kof]);
            acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc, 0, 0, 0);
            acc_lo = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl, acc_lo, 0, 0, 0);
            acc_lo = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh, acc_lo, 0, 0, 0);
        }
    }
    const int e = e0 + 32 * wave + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int t = t0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (t < T && e < E)
            logits[(size_t)t * E + e] =
                __builtin_fmaf(acc_lo[v], 1.0f / kLoScale, acc[v]) * (1.0f / kWrScale);
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
    _Float16* xh = reinterpret_cast<_Float16*>(ws + L.x16);
    _Float16* xl = reinterpret_cast<_Float16*>(ws + L.x_lo);
    _Float16* wh = reinterpret_cast<_Float16*>(ws + L.w_hi);
    _Float16* wl = reinterpret_cast<_Float16*>(ws + L.w_lo);
    const size_t n4 = (size_t)T * H / 4;
    launch_k(c, MOE_K_X_F16, x_split_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, x,
             xh, xl, n4);
    launch_k(c, MOE_K_ROUTER_SPLIT, w_split_kernel, dim3((H + 31) / 32, (E + 31) / 32), dim3(256),
             0, d.router_w, H, E, wh, wl);
    launch_k(c, MOE_K_ROUTER_MFMA, router_gemm_kernel, dim3((T + kRgT - 1) / kRgT, (E + kRgE - 1) / kRgE),
             dim3(256), 0, xh, xl, wh, wl, T, H, E, part);
    launch_k(c, MOE_K_ROUTER_TOPK, router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, part, 1,
             T, E, d.top_k, idx, w);
    return hipGetLastError();
}

// fp16 tokens for the grouped GEMM when the router did not already make them
hipError_t launch_x16(const float* x, int T, int H, char* ws, const WsLayout& L, const Ctx& c) {
    const size_t n4 = (size_t)T * H / 4;
    launch_k(c, MOE_K_X_F16, x_split_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, x,
             reinterpret_cast<_Float16*>(ws + L.x16), (_Float16*)nullptr, n4);
    return hipGetLastError();
}

}  // namespace moe
