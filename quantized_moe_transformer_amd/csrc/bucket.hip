// bucket.hip -- token -> expert bucketing for the grouped-GEMM path.
//
// Rows are independent through the MoE region (page "CKE Zip: From Splitting
// Tokens To Splitting Qwen3.5 Weights", section "What The First Prototype
// Split"), so the slots (t, j) can be regrouped by expert and every expert's
// weights streamed once for all of its rows.  The regrouping is a stable
// counting sort of the slot ids s = t*k + j by expert:
//   bucket_hist     per 1024-slot block, per-expert counts (LDS integer adds);
//                   folded into bucket_scan when the blocks' table fits in LDS;
//   bucket_scan     one workgroup: counts, exclusive scan over experts
//                   (offsets), per-block bases, and the grouped-GEMM tile list
//                   (tiles of kTileM rows per expert, the shared expert last as
//                   group E with all T rows);
//   bucket_scatter  per block: per-wave histograms -> per-wave bases, the rank
//                   of a slot among equal experts inside its wave by a
//                   64-step lane scan, perm[base + rank] = s.
// Integer counts are order-independent and the ranks are positional, so the
// result is deterministic.
#include "launch.h"

namespace moe {

constexpr int kBucketBlock = 1024;   // slots (= threads) per block
constexpr int kBucketWaves = kBucketBlock / 64;

__global__ void __launch_bounds__(kBucketBlock)
bucket_hist_kernel(const int32_t* __restrict__ idx, int n, int E, int32_t* __restrict__ bhist) {
    extern __shared__ int32_t hist[];   // [E]
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int s = blockIdx.x * kBucketBlock + threadIdx.x;
    if (s < n) {
        const int e = idx[s];
        if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) bhist[(size_t)blockIdx.x * E + e] = hist[e];
}

// Single workgroup of 1024 threads; E <= 1024.  FUSED (few blocks,
// nblk * E <= kFusedHist): it first forms the per-block histograms itself in
// LDS (the same integer counts as bucket_hist_kernel), so that kernel is not
// launched; otherwise it reads them from bhist.
constexpr int kFusedHist = 8192;    // int32 entries of the LDS histogram (32 KB)
constexpr int kFusedMaxBlocks = 8;  // slot blocks (T*k <= 8192) up to which it fuses

template <bool FUSED>
__global__ void __launch_bounds__(1024)
bucket_scan_kernel(int nblk, int E, int T, int shared, const int32_t* __restrict__ idx, int n,
                   int32_t* __restrict__ bhist, int32_t* __restrict__ counts,
                   int32_t* __restrict__ offsets, int32_t* __restrict__ tile_off,
                   int4* __restrict__ tile_rec) {
    __shared__ int32_t sc[1024];
    __shared__ int32_t st[1024];
    extern __shared__ int32_t lh[];   // [nblk][E] when FUSED
    const int e = threadIdx.x;
    if (FUSED) {
        for (int i = threadIdx.x; i < nblk * E; i += blockDim.x) lh[i] = 0;
        __syncthreads();
        for (int s0 = 0; s0 < n; s0 += 4 * 1024) {
            int v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = s0 + j * 1024 + threadIdx.x;
                v[j] = s < n ? idx[s] : -1;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = s0 + j * 1024 + threadIdx.x;
                if ((unsigned)v[j] < (unsigned)E) atomicAdd(&lh[(s / kBucketBlock) * E + v[j]], 1);
            }
        }
        __syncthreads();
    }
    auto hist = [&](int b) -> int { return FUSED ? lh[b * E + e] : bhist[(size_t)b * E + e]; };
    constexpr int kBatch = 16;   // block counts in flight per thread
    int c = 0;
    if (e < E)
        for (int b0 = 0; b0 < nblk; b0 += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                v[j] = b0 + j < nblk ? hist(b0 + j) : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) c += v[j];
        }
    const int tiles = (c + kTileM - 1) / kTileM;
    // inclusive scans of counts and tiles: within each wave by lane shifts,
    // then plus the totals of the waves before (integers: exact)
    const int lane = e & 63, wv = e >> 6;
    int ic = e < E ? c : 0, it = e < E ? tiles : 0;
    for (int off = 1; off < 64; off <<= 1) {
        const int a = __shfl_up(ic, off, 64), b = __shfl_up(it, off, 64);
        if (lane >= off) {
            ic += a;
            it += b;
        }
    }
    __shared__ int32_t wc[16], wt[16];
    if (lane == 63) {
        wc[wv] = ic;
        wt[wv] = it;
    }
    __syncthreads();
    for (int w = 0; w < wv; ++w) {
        ic += wc[w];
        it += wt[w];
    }
    sc[e] = ic;
    st[e] = it;
    __syncthreads();
    if (e < E) {
        const int excl = sc[e] - c;
        counts[e] = c;
        offsets[e] = excl;
        tile_off[e] = st[e] - tiles;
        // the expert's row tiles: (group, first sorted row, rows, row offset)
        for (int j = 0; j < tiles; ++j)
            tile_rec[st[e] - tiles + j] = make_int4(e, excl + j * kTileM, min(kTileM, c - j * kTileM),
                                                    j * kTileM);
        // per-block bases for the scatter (in place when read from bhist)
        int base = excl;
        for (int b0 = 0; b0 < nblk; b0 += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                v[j] = b0 + j < nblk ? hist(b0 + j) : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (b0 + j < nblk) bhist[(size_t)(b0 + j) * E + e] = base;
                base += v[j];
            }
        }
    }
    if (shared) {
        // the shared expert (group E, all T rows in order) after the routed tiles
        const int nsh = (T + kTileM - 1) / kTileM;
        for (int j = threadIdx.x; j < nsh; j += blockDim.x)
            tile_rec[st[1023] + j] = make_int4(E, sc[1023] + j * kTileM, min(kTileM, T - j * kTileM),
                                               j * kTileM);
    }
    if (e == E - 1) {
        offsets[E] = sc[e];
        offsets[E + 1] = sc[e] + (shared ? T : 0);
        tile_off[E] = st[e];
        tile_off[E + 1] = st[e] + (shared ? (T + kTileM - 1) / kTileM : 0);
        counts[E] = shared ? T : 0;
    }
}

__global__ void __launch_bounds__(kBucketBlock)
bucket_scatter_kernel(const int32_t* __restrict__ idx, int n, int E,
                      const int32_t* __restrict__ bbase, int32_t* __restrict__ perm) {
    extern __shared__ int32_t wh[];   // [kBucketWaves][E]
    for (int i = threadIdx.x; i < kBucketWaves * E; i += blockDim.x) wh[i] = 0;
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int s = blockIdx.x * kBucketBlock + threadIdx.x;
    int e = -1;
    if (s < n) {
        e = idx[s];
        if ((unsigned)e >= (unsigned)E) e = -1;
    }
    if (e >= 0) atomicAdd(&wh[wave * E + e], 1);
    __syncthreads();
    // exclusive scan over waves, per expert
    for (int x = threadIdx.x; x < E; x += blockDim.x) {
        int run = bbase[(size_t)blockIdx.x * E + x];
        for (int w = 0; w < kBucketWaves; ++w) {
            const int h = wh[w * E + x];
            wh[w * E + x] = run;
            run += h;
        }
    }
    __syncthreads();
    // rank among earlier lanes of this wave with the same expert
    int rank = 0;
    for (int l = 0; l < 64; ++l) {
        const int el = __shfl(e, l, 64);
        rank += (l < lane && el == e) ? 1 : 0;
    }
    if (e >= 0) perm[wh[wave * E + e] + rank] = s;
}

hipError_t launch_bucket(const int32_t* idx, int T, int k, int E, bool shared, int32_t* counts,
                         int32_t* offsets, int32_t* tile_off, int4* tile_rec, int32_t* perm,
                         int32_t* bhist, const Ctx& c) {
    const int n = T * k;
    const int nblk = bucket_blocks(T, k);
    // few slots: the scan forms the per-block histograms itself (measured:
    // 5.0 us against 4.0 + 4.5 us for the two kernels at 32 rows; at 4096
    // rows, 32 blocks, one workgroup reading every slot is slower)
    const bool fused = nblk <= kFusedMaxBlocks && (int64_t)nblk * E <= kFusedHist;
    if (!fused)
        launch_k(c, MOE_K_BUCKET_HIST, bucket_hist_kernel, dim3(nblk), dim3(kBucketBlock),
                 (uint32_t)(E * sizeof(int32_t)), idx, n, E, bhist);
    if (fused)
        launch_k(c, MOE_K_BUCKET_SCAN, bucket_scan_kernel<true>, dim3(1), dim3(1024),
                 (uint32_t)(nblk * E * sizeof(int32_t)), nblk, E, T, shared ? 1 : 0, idx, n, bhist,
                 counts, offsets, tile_off, tile_rec);
    else
        launch_k(c, MOE_K_BUCKET_SCAN, bucket_scan_kernel<false>, dim3(1), dim3(1024), 0u, nblk, E,
                 T, shared ? 1 : 0, idx, n, bhist, counts, offsets, tile_off, tile_rec);
    launch_k(c, MOE_K_BUCKET_SCATTER, bucket_scatter_kernel, dim3(nblk), dim3(kBucketBlock),
             (uint32_t)(kBucketWaves * E * sizeof(int32_t)), idx, n, E, bhist, perm);
    return hipGetLastError();
}

}  // namespace moe
