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
//   split, router_gemm  a dense [T x H] x [H x E] product on the fp16 matrix
//                   cores with split operands (fp32 accuracy);
//   router_topk     one wave per token (topk.h).
#include "launch.h"
#include "topk.h"

namespace moe {

constexpr int kRgSplit = 2;   // K splits of the matrix-core router (partials added by the top-k)

int router_splits(int T) { return T <= kRouterSmallMaxT ? kRouterSplits : kRgSplit; }

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
constexpr int kRgT = 64, kRgE = 128, kRgK = 64;

// One launch, two jobs.  Workgroups [0, nxb): x fp32 [T][H] -> hi (x16, also
// the grouped GEMM's operand) and lo parts, eight values (two 16-byte loads,
// one 16-byte store per part) per thread.
// Workgroups [nxb, nxb + nwb): the router matrix fp32 [H][E] -> 2^10 * (hi, lo)
// parts transposed to [E][H], one 32 x 32 tile each (LDS transpose).  xl and
// wr may be null (tokens only).
__global__ void __launch_bounds__(256)
split_kernel(const float* __restrict__ x, _Float16* __restrict__ xh, _Float16* __restrict__ xl,
             size_t n8, int nxb, const float* __restrict__ wr, int H, int E,
             _Float16* __restrict__ wh, _Float16* __restrict__ wl, int32_t* __restrict__ zero,
             size_t nzero) {
    __shared__ float tile[32][33];
    const int b = blockIdx.x;
    if (b < nxb) {
        const size_t i = (size_t)b * blockDim.x + threadIdx.x;
        // the top-k's slot counts start from zero (zero may be null)
        for (size_t z = i; z < nzero; z += (size_t)nxb * blockDim.x) zero[z] = 0;
        if (i >= n8) return;
        const float4 v0 = reinterpret_cast<const float4*>(x)[2 * i];
        const float4 v1 = reinterpret_cast<const float4*>(x)[2 * i + 1];
        half8 h, l;
        const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            h[j] = (_Float16)f[j];
            l[j] = (_Float16)((f[j] - (float)h[j]) * kLoScale);
        }
        reinterpret_cast<half8*>(xh)[i] = h;
        if (xl) reinterpret_cast<half8*>(xl)[i] = l;
        return;
    }
    const int wb = b - nxb, nhb = (H + 31) / 32;
    const int h0 = (wb % nhb) * 32, e0 = (wb / nhb) * 32;
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

// grid (ceil(T/64), ceil(E/128), kRgSplit); 4 waves, wave w owns experts
// [32w, 32w+32) of the block's 128 for all 64 token rows (two 32-row blocks,
// so each router fragment read from LDS feeds two token blocks).  The K range
// is split in kRgSplit parts (blockIdx.z), each written as a partial logit
// [T][E][kRgSplit] that the top-k adds in ascending order; the split keeps
// 256 workgroups at T = 4096.  K advances 64 at a time.  A step's operands --
// hi and lo parts of 64 token rows and of 128 router rows, 48 KB -- arrive by
// direct global-to-LDS loads two steps ahead into a three-stage ring (twelve
// 16-byte loads per thread per step).  Each row's eight 16-byte chunks sit
// XOR-swizzled by the row index (chunk c at position c ^ ((row >> 1) & 7)).  Rows
// past T or E re-read the last valid row; their results are not written.
constexpr int kRgStages = 3;
constexpr int kRgStageHalves = 2 * (kRgT + kRgE) * kRgK;   // 48 KB
constexpr int kRgDma = kRgStageHalves * 2 / 16 / 256;       // 12 loads per thread per step
constexpr int kRgAChunks = 2 * kRgT * 8;                    // A hi + lo chunks of a stage

__device__ __forceinline__ int rg_chunk(int row, int c) { return row * 8 + (c ^ ((row >> 1) & 7)); }

__global__ void __launch_bounds__(256)
router_gemm_kernel(const _Float16* __restrict__ xh, const _Float16* __restrict__ xl,
                   const _Float16* __restrict__ wh, const _Float16* __restrict__ wl, int T, int H,
                   int E, float* __restrict__ logits) {
    // per stage: A hi [64][64], A lo, B hi [128][64], B lo
    __shared__ __align__(16) _Float16 st[kRgStages][kRgStageHalves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t0 = blockIdx.x * kRgT, e0 = blockIdx.y * kRgE, z = blockIdx.z;
    const int nk = H / kRgK / kRgSplit;
    const size_t k0 = (size_t)z * nk * kRgK;   // first K of this split
    // chunk q = (12 wave + j) * 64 + lane of a stage: A parts first
    const _Float16* src[kRgDma];
#pragma unroll
    for (int j = 0; j < kRgDma; ++j) {
        const int q = (kRgDma * wave + j) * 64 + lane;
        if (q < kRgAChunks) {
            const int part = q / (kRgT * 8), row = (q >> 3) & (kRgT - 1), c = (q & 7) ^ ((row >> 1) & 7);
            const int t = min(t0 + row, T - 1);
            src[j] = (part ? xl : xh) + (size_t)t * H + k0 + c * 8;
        } else {
            const int qb = q - kRgAChunks;
            const int part = qb / (kRgE * 8), row = (qb >> 3) & (kRgE - 1), c = (qb & 7) ^ ((row >> 1) & 7);
            const int e = min(e0 + row, E - 1);
            src[j] = (part ? wl : wh) + (size_t)e * H + k0 + c * 8;
        }
    }
    auto issue = [&](int kk) {
        const uint32_t base = (uint32_t)(uintptr_t)&st[kk % kRgStages][0];
#pragma unroll
        for (int j = 0; j < kRgDma; ++j)
            lds_dma16(src[j] + (size_t)kk * kRgK,
                      __builtin_amdgcn_readfirstlane(base + (kRgDma * wave + j) * 1024));
    };
    issue(0);
    if (nk > 1) {
        issue(1);
        wait_vmcnt<kRgDma>();
    } else {
        wait_vmcnt<0>();
    }
    __syncthreads();
    float16v acc[2] = {}, acc_lo[2] = {};
    for (int kk = 0; kk < nk; ++kk) {
        // step kk + 2 into the stage step kk - 1 read (every wave passed the barrier)
        const bool more = kk + 2 < nk;
        if (more) issue(kk + 2);
        const _Float16* sa_h = &st[kk % kRgStages][0];
        const _Float16* sa_l = sa_h + kRgT * kRgK;
        const _Float16* sb_h = sa_h + 2 * kRgT * kRgK;
        const _Float16* sb_l = sb_h + kRgE * kRgK;
        const int ra = lane & 31, rb = 32 * wave + (lane & 31);
#pragma unroll
        for (int s = 0; s < kRgK / 16; ++s) {
            const int c = 2 * s + (lane >> 5);
            const half8 bh = *reinterpret_cast<const half8*>(sb_h + 8 * rg_chunk(rb, c));
            const half8 bl = *reinterpret_cast<const half8*>(sb_l + 8 * rg_chunk(rb, c));
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const half8 ah = *reinterpret_cast<const half8*>(sa_h + 8 * rg_chunk(32 * i + ra, c));
                const half8 al = *reinterpret_cast<const half8*>(sa_l + 8 * rg_chunk(32 * i + ra, c));
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc[i], 0, 0, 0);
                acc_lo[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bl, acc_lo[i], 0, 0, 0);
                acc_lo[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al, bh, acc_lo[i], 0, 0, 0);
            }
        }
        // step kk + 1's operands must have landed; step kk + 2's may be in flight
        if (more) wait_vmcnt<kRgDma>();
        else wait_vmcnt<0>();
        __syncthreads();
    }
    const int e = e0 + 32 * wave + (lane & 31);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int t = t0 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
            if (t < T && e < E)
                logits[((size_t)t * E + e) * kRgSplit + z] =
                    __builtin_fmaf(acc_lo[i][v], 1.0f / kLoScale, acc[i][v]) * (1.0f / kWrScale);
        }
}

// Four tokens per workgroup, one wave each.  With bhist (else null), lane j
// also adds slot t*k + j to its block's count of its expert: the bucketing's
// per-block histograms [T*k / kBucketSlots][E] (integer adds, in any order).
__global__ void __launch_bounds__(256)
router_topk_kernel(const float* __restrict__ part, int ks_n, int T, int E, int k,
                   int32_t* __restrict__ idx, float* __restrict__ w, int32_t* __restrict__ bhist) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    int32_t* ir = idx + (size_t)t * k;
    float* wr = w + (size_t)t * k;
    int e;
    if (ks_n == 1) {
        if (E <= 256) e = wave_topk<4, 1>(part, E, k, t, ir, wr);
        else e = wave_topk<16, 1>(part, E, k, t, ir, wr);
    } else if (ks_n == kRgSplit) {
        if (E <= 256) e = wave_topk<4, kRgSplit>(part, E, k, t, ir, wr);
        else e = wave_topk<16, kRgSplit>(part, E, k, t, ir, wr);
    } else {
        if (E <= 256) e = wave_topk<4, kRouterSplits>(part, E, k, t, ir, wr);
        else e = wave_topk<16, kRouterSplits>(part, E, k, t, ir, wr);
    }
    const int lane = threadIdx.x & 63;
    if (bhist != nullptr && lane < k && (unsigned)e < (unsigned)E) {
        const int s = t * k + lane;
        atomicAdd(&bhist[(size_t)(s / kBucketSlots) * E + e], 1);
    }
}

hipError_t launch_router_small(const moe_layer_desc& d, const float* x, int T, char* ws,
                               const WsLayout& L, const Ctx& c);   // gemv.hip: partials only

hipError_t launch_router(const moe_layer_desc& d, const float* x, int T, int32_t* idx, float* w,
                         char* ws, const WsLayout& L, const Ctx& c) {
    return launch_router_hist(d, x, T, idx, w, ws, L, c, nullptr);
}

hipError_t launch_router_hist(const moe_layer_desc& d, const float* x, int T, int32_t* idx,
                              float* w, char* ws, const WsLayout& L, const Ctx& c,
                              int32_t* bhist) {
    const int H = d.hidden, E = d.n_experts;
    float* part = reinterpret_cast<float*>(ws + L.router_part);
    if (T <= kRouterSmallMaxT) {
        hipError_t e = launch_router_small(d, x, T, ws, L, c);
        if (e != hipSuccess) return e;
        launch_k(c, MOE_K_ROUTER_TOPK, router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, part,
                 L.router_ks, T, E, d.top_k, idx, w, (int32_t*)nullptr);
        return hipGetLastError();
    }
    _Float16* xh = reinterpret_cast<_Float16*>(ws + L.x16);
    _Float16* xl = reinterpret_cast<_Float16*>(ws + L.x_lo);
    _Float16* wh = reinterpret_cast<_Float16*>(ws + L.w_hi);
    _Float16* wl = reinterpret_cast<_Float16*>(ws + L.w_lo);
    const size_t n8 = (size_t)T * H / 8;   // H is a multiple of 256
    const int nxb = (int)((n8 + 255) / 256), nwb = ((H + 31) / 32) * ((E + 31) / 32);
    const size_t nzero = bhist ? (size_t)bucket_blocks(T, d.top_k) * E : 0;
    launch_k(c, MOE_K_X_F16, split_kernel, dim3(nxb + nwb), dim3(256), 0, x, xh, xl, n8, nxb,
             d.router_w, H, E, wh, wl, bhist, nzero);
    launch_k(c, MOE_K_ROUTER_MFMA, router_gemm_kernel,
             dim3((T + kRgT - 1) / kRgT, (E + kRgE - 1) / kRgE, kRgSplit), dim3(256), 0, xh, xl, wh,
             wl, T, H, E, part);
    launch_k(c, MOE_K_ROUTER_TOPK, router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, part,
             kRgSplit, T, E, d.top_k, idx, w, bhist);
    return hipGetLastError();
}

// fp16 tokens for the grouped GEMM when the router did not already make them
hipError_t launch_x16(const float* x, int T, int H, char* ws, const WsLayout& L, const Ctx& c) {
    const size_t n8 = (size_t)T * H / 8;
    const int nxb = (int)((n8 + 255) / 256);
    launch_k(c, MOE_K_X_F16, split_kernel, dim3(nxb), dim3(256), 0, x,
             reinterpret_cast<_Float16*>(ws + L.x16), (_Float16*)nullptr, n8, nxb,
             (const float*)nullptr, H, 0, (_Float16*)nullptr, (_Float16*)nullptr,
             (int32_t*)nullptr, (size_t)0);
    return hipGetLastError();
}

}  // namespace moe
