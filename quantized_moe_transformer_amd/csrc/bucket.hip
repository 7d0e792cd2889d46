// bucket.hip -- token -> expert bucketing for the grouped-GEMM path.
//
// Rows are independent through the MoE region (page "CKE Zip: From Splitting
// Tokens To Splitting Qwen3.5 Weights", section "What The First Prototype
// Split"), so the slots (t, j) can be regrouped by expert and every expert's
// weights streamed once for all of its rows.  The regrouping is a stable
// counting sort of the slot ids s = t*k + j by expert:
//   bucket_hist     per 1024-slot block, per-expert counts (LDS integer adds);
//                   folded into bucket_sort when the blocks' table fits in LDS;
//   bucket_sort     per block: the exclusive scan over experts (offsets) and
//                   this block's bases, recomputed by every workgroup from the
//                   counts; workgroup 0 writes the grouped-GEMM tile list; then
//                   per-wave histograms -> per-wave bases, the rank of a slot
//                   among equal experts inside its wave by a 64-step lane scan,
//                   perm[base + rank] = s.
// Integer counts are order-independent and the ranks are positional, so the
// result is deterministic.
#include "launch.h"

namespace moe {

constexpr int kBucketBlock = kBucketSlots;   // slots (= threads) per block
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

// Per 1024-slot block b, 1024 threads; E <= 1024.  Every workgroup forms the
// expert totals and the counts of the blocks before its own, from the
// per-block histograms (SELF: it counts all blocks itself in LDS, the same
// integer counts as bucket_hist_kernel, so that kernel is not launched), and
// runs the exclusive scans over experts (integers: every workgroup gets the
// same offsets).  Workgroup 0 also writes counts, offsets, tile_off and the
// grouped GEMM's tile list (tiles of kTileM rows per expert, then the shared
// expert's as group E with all T rows, stored last tile first: the order in
// which the GEMM's workgroups take them).  Then each workgroup places its
// own slots: per-wave histograms -> per-wave bases, the rank of a slot among
// equal experts inside its wave by a 64-step lane scan, perm[base + rank] = s.
constexpr int kFusedHist = 8192;    // int32 entries of the LDS histogram (32 KB)
constexpr int kFusedMaxBlocks = 8;  // slot blocks (T*k <= 8192) up to which SELF is used

template <bool SELF>
__global__ void __launch_bounds__(kBucketBlock)
bucket_sort_kernel(const int32_t* __restrict__ idx, int n, int nblk, int E, int T, int shared,
                   const int32_t* __restrict__ bhist, int32_t* __restrict__ counts,
                   int32_t* __restrict__ offsets, int32_t* __restrict__ tile_off,
                   int4* __restrict__ tile_rec, int32_t* __restrict__ perm) {
    __shared__ int32_t sc[kBucketBlock];
    __shared__ int32_t st[kBucketBlock];
    __shared__ int32_t bbase[kBucketBlock];   // this block's first sorted row per expert
    __shared__ int32_t wc[kBucketWaves], wt[kBucketWaves];
    extern __shared__ int32_t dyn[];   // SELF: lh [nblk][E]; then wh [kBucketWaves][E]
    int32_t* lh = dyn;
    int32_t* wh = dyn + (SELF ? nblk * E : 0);
    const int b = blockIdx.x, tid = threadIdx.x, e = tid;
    const int wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < kBucketWaves * E; i += kBucketBlock) wh[i] = 0;
    if (SELF) {
        for (int i = tid; i < nblk * E; i += kBucketBlock) lh[i] = 0;
        __syncthreads();
        for (int s0 = 0; s0 < n; s0 += 4 * kBucketBlock) {
            int v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = s0 + j * kBucketBlock + tid;
                v[j] = s < n ? idx[s] : -1;
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s = s0 + j * kBucketBlock + tid;
                if ((unsigned)v[j] < (unsigned)E) atomicAdd(&lh[(s / kBucketBlock) * E + v[j]], 1);
            }
        }
    }
    // this block's slot and its expert (read before the barrier, used after)
    const int s = b * kBucketBlock + tid;
    int se = -1;
    if (s < n) {
        se = idx[s];
        if ((unsigned)se >= (unsigned)E) se = -1;
    }
    __syncthreads();
    // expert e: total over all blocks, and over the blocks before this one
    auto hist = [&](int bb) -> int { return SELF ? lh[bb * E + e] : bhist[(size_t)bb * E + e]; };
    constexpr int kBatch = 16;   // block counts in flight per thread
    int c = 0, pre = 0;
    if (e < E)
        for (int b0 = 0; b0 < nblk; b0 += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) v[j] = b0 + j < nblk ? hist(b0 + j) : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                c += v[j];
                pre += b0 + j < b ? v[j] : 0;
            }
        }
    const int tiles = (c + kTileM - 1) / kTileM;
    // inclusive scans of counts and tiles: within each wave by lane shifts,
    // then plus the totals of the waves before (integers: exact)
    int ic = e < E ? c : 0, it = e < E ? tiles : 0;
    for (int off = 1; off < 64; off <<= 1) {
        const int x = __shfl_up(ic, off, 64), y = __shfl_up(it, off, 64);
        if (lane >= off) {
            ic += x;
            it += y;
        }
    }
    if (lane == 63) {
        wc[wave] = ic;
        wt[wave] = it;
    }
    __syncthreads();
    for (int w = 0; w < wave; ++w) {
        ic += wc[w];
        it += wt[w];
    }
    sc[e] = ic;
    st[e] = it;
    __syncthreads();
    if (b == 0) {
        // row tile i (experts in order, then the shared expert) goes to record
        // ntot - 1 - i: the grouped GEMM's workgroups take the records in
        // order (the shared expert's, the largest, first) and read a record
        // without waiting for the tile count
        const int nsh = shared ? (T + kTileM - 1) / kTileM : 0;
        const int ntot = st[kBucketBlock - 1] + nsh;
        if (e < E) {
            const int excl = ic - c;
            counts[e] = c;
            offsets[e] = excl;
            tile_off[e] = it - tiles;
            // the expert's row tiles: (group, first sorted row, rows, row offset)
            for (int j = 0; j < tiles; ++j)
                tile_rec[ntot - 1 - (it - tiles + j)] =
                    make_int4(e, excl + j * kTileM, min(kTileM, c - j * kTileM), j * kTileM);
        }
        // the shared expert (group E, all T rows in order) after the routed tiles
        for (int j = tid; j < nsh; j += kBucketBlock)
            tile_rec[nsh - 1 - j] = make_int4(E, sc[kBucketBlock - 1] + j * kTileM,
                                              min(kTileM, T - j * kTileM), j * kTileM);
        if (e == E - 1) {
            offsets[E] = ic;
            offsets[E + 1] = ic + (shared ? T : 0);
            tile_off[E] = it;
            tile_off[E + 1] = it + (shared ? (T + kTileM - 1) / kTileM : 0);
            counts[E] = shared ? T : 0;
        }
    }
    // this block's base per expert: its exclusive offset plus the earlier blocks
    if (e < E) bbase[e] = ic - c + pre;
    if (se >= 0) atomicAdd(&wh[wave * E + se], 1);
    __syncthreads();
    // exclusive scan over waves, per expert
    for (int x = tid; x < E; x += kBucketBlock) {
        int run = bbase[x];
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
        const int el = __shfl(se, l, 64);
        rank += (l < lane && el == se) ? 1 : 0;
    }
    if (se >= 0) perm[wh[wave * E + se] + rank] = s;
}

bool bucket_self(int T, int k, int E) {
    const int nblk = bucket_blocks(T, k);
    return nblk <= kFusedMaxBlocks && (int64_t)nblk * E <= kFusedHist;
}

hipError_t launch_bucket(const int32_t* idx, int T, int k, int E, bool shared, int32_t* counts,
                         int32_t* offsets, int32_t* tile_off, int4* tile_rec, int32_t* perm,
                         int32_t* bhist, const Ctx& c) {
    const int n = T * k;
    const int nblk = bucket_blocks(T, k);
    // few slots: every workgroup counts all of them itself (one kernel); many:
    // per-block counts first, from bucket_hist_kernel unless the router's
    // top-k already made them
    const bool self = bucket_self(T, k, E);
    const uint32_t wh_bytes = (uint32_t)(kBucketWaves * E * sizeof(int32_t));
    if (self) {
        launch_k(c, MOE_K_BUCKET_SCATTER, bucket_sort_kernel<true>, dim3(nblk), dim3(kBucketBlock),
                 (uint32_t)(nblk * E * sizeof(int32_t)) + wh_bytes, idx, n, nblk, E, T,
                 shared ? 1 : 0, (const int32_t*)nullptr, counts, offsets, tile_off, tile_rec, perm);
    } else {
        if (!c.hist_ready)
            launch_k(c, MOE_K_BUCKET_HIST, bucket_hist_kernel, dim3(nblk), dim3(kBucketBlock),
                     (uint32_t)(E * sizeof(int32_t)), idx, n, E, bhist);
        launch_k(c, MOE_K_BUCKET_SCATTER, bucket_sort_kernel<false>, dim3(nblk), dim3(kBucketBlock),
                 wh_bytes, idx, n, nblk, E, T, shared ? 1 : 0, (const int32_t*)bhist, counts,
                 offsets, tile_off, tile_rec, perm);
    }
    return hipGetLastError();
}

}  // namespace moe
