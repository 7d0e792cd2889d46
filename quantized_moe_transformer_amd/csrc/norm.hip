// norm.hip -- the steps either side of the layer: RMSNorm of the layer's
// input rows, whole or one column shard at a time (page "Distributed CPU: Zip
// Fusion Beyond Tensor Parallelism", section "What Must Cross the Fabric: The
// Reduction Algebra": the norm's global dependency is one scalar per row, the
// sum of squares, which column shards form on their own columns and add in a
// declared order).  The residual after the layer is in api.hip (the shard
// reduce with a residual term).
//
//   y[c] = g[c] * x[c] / sqrt(S / H + eps),  S = sum of x^2 over the row's H columns.
//
// HBM-bound: one read of x (the second pass over a row hits the cache), one
// write of y, g once per workgroup.
#include "launch.h"

namespace moe {

constexpr int kNormThreads = 256;

struct SsqPtrs {
    const float* p[16];
};

// Sum of squares of one row's n4 float4 chunks in a fixed order: each thread
// its chunks in ascending order, then the 64-lane butterfly, then the four
// waves in order.  Every thread returns the same value.
__device__ __forceinline__ float row_sumsq(const float* __restrict__ x, int n4, float* red) {
    float s = 0.f;
    for (int i = threadIdx.x; i < n4; i += kNormThreads) {
        const float4 v = reinterpret_cast<const float4*>(x)[i];
        s = __builtin_fmaf(v.x, v.x, s);
        s = __builtin_fmaf(v.y, v.y, s);
        s = __builtin_fmaf(v.z, v.z, s);
        s = __builtin_fmaf(v.w, v.w, s);
    }
    s = wave_sum_group(s, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    const float tot = ((red[0] + red[1]) + red[2]) + red[3];
    __syncthreads();   // red is rewritten for the next row
    return tot;
}

// Partial sums of squares of T rows (n4 chunks each, row stride ldx floats).
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_sumsq_kernel(const float* __restrict__ x, int T, int n4, int64_t ldx,
                     float* __restrict__ ssq) {
    __shared__ float red[kNormThreads / 64];
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        const float s = row_sumsq(x + (int64_t)t * ldx, n4, red);
        if (threadIdx.x == 0) ssq[t] = s;
    }
}

// y = g * x * (1 / sqrt(S / h + eps)).  n_parts == 0: S is the row's own sum
// of squares; otherwise S = ((p_0 + p_1) + ...) of the shards' partial sums.
__global__ void __launch_bounds__(kNormThreads)
rmsnorm_kernel(const float* x, int T, int n4, int64_t ldx, SsqPtrs parts, int n_parts, float h,
               const float* __restrict__ g, float eps, float* y, int64_t ldy) {
    __shared__ float red[kNormThreads / 64];
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        const float* xr = x + (int64_t)t * ldx;
        float S;
        if (n_parts == 0) {
            S = row_sumsq(xr, n4, red);
        } else {
            S = parts.p[0][t];
            for (int s = 1; s < n_parts; ++s) S += parts.p[s][t];
        }
        const float inv = 1.0f / sqrtf(S / h + eps);
        float* yr = y + (int64_t)t * ldy;
        for (int i = threadIdx.x; i < n4; i += kNormThreads) {
            const float4 v = reinterpret_cast<const float4*>(xr)[i];
            const float4 w = reinterpret_cast<const float4*>(g)[i];
            float4 o;
            o.x = (v.x * inv) * w.x;
            o.y = (v.y * inv) * w.y;
            o.z = (v.z * inv) * w.z;
            o.w = (v.w * inv) * w.w;
            reinterpret_cast<float4*>(yr)[i] = o;
        }
    }
}

static unsigned norm_grid(int T) { return (unsigned)(T < 4096 ? T : 4096); }

hipError_t launch_rmsnorm_sumsq(const float* x, int T, int cols, int64_t ldx, float* ssq,
                                hipStream_t s) {
    rmsnorm_sumsq_kernel<<<norm_grid(T), kNormThreads, 0, s>>>(x, T, cols / 4, ldx, ssq);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(const float* x, int T, int cols, int64_t ldx,
                          const float* const* parts, int n_parts, int H, const float* g,
                          float eps, float* y, int64_t ldy, hipStream_t s) {
    SsqPtrs ps = {};
    for (int i = 0; i < n_parts; ++i) ps.p[i] = parts[i];
    rmsnorm_kernel<<<norm_grid(T), kNormThreads, 0, s>>>(x, T, cols / 4, ldx, ps, n_parts,
                                                         (float)H, g, eps, y, ldy);
    return hipGetLastError();
}

}  // namespace moe
