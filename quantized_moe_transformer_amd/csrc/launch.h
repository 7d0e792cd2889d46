// launch.h -- host side of libmoe_hip.so: the workspace layout, the launch
// context and the kernel launchers (enqueue only; arguments already validated
// by api.hip).
#pragma once

#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------------------
// Workspace layout
// ---------------------------------------------------------------------------

struct WsLayout {
    // shared by both paths
    size_t router_part;   // float [T][E][ks]
    size_t x_lo;          // fp16 [T][H] low parts of x (router at large T)
    size_t w_hi, w_lo;    // fp16 [E][H] split router matrix (router at large T)
    size_t idx, w;        // int32 / float [T][k] (routing computed inside the forward call)
    // GEMV path
    size_t hbuf;          // float [T*(k+1)][I_loc]
    // grouped-GEMM path (overlays the GEMV region)
    size_t x16;           // fp16 [T][H]
    size_t bhist;         // int32 [nblk][E]
    size_t counts;        // int32 [E+1]
    size_t offsets;       // int32 [E+2]
    size_t tile_off;      // int32 [E+3]
    size_t tile_rec;      // int4 per row tile: group, first sorted row, rows, row offset in group
    size_t perm;          // int32 [T*k]
    size_t h16;           // fp16 [T*k + T][I_loc]
    size_t y;             // int16 [T*k][H]: per-slot expert rows (routing weight applied),
                          // 16-bit block floating point (store_rows_q16)
    size_t ysh;           // int16 [T][H]: shared-expert rows, shared weight applied
    size_t ysc;           // uint8 [T*k][H/8]: exponent byte of each 8 values of y
    size_t yshsc;         // uint8 [T][H/8]: the same for ysh
    // grouped GEMM on MXFP4 weights (block-scaled matrix cores): tokens and h
    // as kMxTerms MX-FP8 terms (in place of x16 and h16)
    size_t mx_xq;         // e4m3 [kMxTerms][T][H]
    size_t mx_xs;         // E8M0 [T][H/64][16]
    size_t mx_hq;         // e4m3 [kMxTerms][T*k + T][I_loc]
    size_t mx_hs;         // E8M0 [T*k + T][I_loc/64][16]
    size_t total;
    int router_ks;        // router K-splits
};

int router_splits(int T);
// iloc: the intermediate rows per expert that the call computes (I, or a shard's)
WsLayout ws_layout(const moe_layer_desc& d, int T, int iloc);
constexpr int kBucketSlots = 1024;   // slots per bucketing block
inline int bucket_blocks(int T, int k) { return (T * k + kBucketSlots - 1) / kBucketSlots; }
// whether the bucketing counts the slots itself (few blocks) rather than
// taking per-block counts from bucket_hist or the router's top-k
bool bucket_self(int T, int k, int E);
// upper bound on the grouped GEMM's row tiles: sum over experts of
// ceil(count / kTileM) <= T*k / kTileM + E, plus the shared expert's
inline int max_row_tiles(int T, int k, int E, bool shared) {
    return (T * k + kTileM - 1) / kTileM + E + (shared ? (T + kTileM - 1) / kTileM : 0);
}

// Launch context: the stream, and (optionally) caller-owned start/stop events
// per kernel id (moe_opts.kernel_events).  A timed kernel is launched with
// hipExtLaunchKernel, whose events carry the dispatch's own timestamps.
struct Ctx {
    hipStream_t s = nullptr;
    void** ev = nullptr;
    int n_ev = 0;
    bool hist_ready = false;   // the router's top-k counted the slots into the bucketing's bhist
    hipEvent_t start(int id) const { return (ev && 2 * id + 1 < n_ev) ? (hipEvent_t)ev[2 * id] : nullptr; }
    hipEvent_t stop(int id) const { return (ev && 2 * id + 1 < n_ev) ? (hipEvent_t)ev[2 * id + 1] : nullptr; }
};

template <typename... KArgs, typename... Args>
inline void launch_k(const Ctx& c, int id, void (*kern)(KArgs...), dim3 grid, dim3 block,
                     uint32_t shm, Args... args) {
    const hipEvent_t a = c.start(id), z = c.stop(id);
    if (a || z)
        hipExtLaunchKernelGGL(kern, grid, block, shm, c.s, a, z, 0, static_cast<KArgs>(args)...);
    else
        kern<<<grid, block, shm, c.s>>>(static_cast<KArgs>(args)...);
}

hipError_t launch_router(const moe_layer_desc& d, const float* x, int T, int32_t* idx, float* w,
                         char* ws, const WsLayout& L, const Ctx& c);
// the same; at T > kRouterSmallMaxT with bhist (else null) the top-k also
// counts the slots per 1024-slot block and expert into bhist (zeroed first),
// the bucketing's per-block histograms
hipError_t launch_router_hist(const moe_layer_desc& d, const float* x, int T, int32_t* idx,
                              float* w, char* ws, const WsLayout& L, const Ctx& c,
                              int32_t* bhist);
// route: run the router (and top-k) in the front kernel, writing L.idx / L.w
// i0, iloc: intermediate rows [i0, i0 + iloc) of every expert (the shard)
hipError_t launch_gemv(const moe_layer_desc& d, const float* x, int T, const int32_t* idx,
                       const float* w, int i0, int iloc, float* out, char* ws,
                       const WsLayout& L, const Ctx& c, bool route);
hipError_t launch_bucket(const int32_t* idx, int T, int k, int E, bool shared, int32_t* counts,
                         int32_t* offsets, int32_t* tile_off, int4* tile_rec, int32_t* perm,
                         int32_t* bhist,
                         const Ctx& c);
// x16_ready: the router already wrote the fp16 tokens (L.x16)
hipError_t launch_mfma(const moe_layer_desc& d, const float* x, int T, const int32_t* idx,
                       const float* w, int i0, int iloc, float* out, char* ws,
                       const WsLayout& L, const Ctx& c, bool x16_ready);
// the same for MXFP4 weights, on the block-scaled matrix cores (gemm_mx.hip)
hipError_t launch_mfma_mx(const moe_layer_desc& d, const float* x, int T, const int32_t* idx,
                          const float* w, int i0, int iloc, float* out, char* ws,
                          const WsLayout& L, const Ctx& c);
// out[t] = slot rows of y in slot order, then the shared rows (gemm.hip)
hipError_t launch_combine(const int16_t* y, const int16_t* ysh, const uint8_t* ysc,
                          const uint8_t* yshsc, const int32_t* idx, int T, int H, int E, int k,
                          bool shared, float* out, const Ctx& c);
hipError_t launch_x16(const float* x, int T, int H, char* ws, const WsLayout& L, const Ctx& c);
hipError_t launch_reduce(const float* const* partials, int n, int64_t count, const float* res,
                         float* out, hipStream_t s);
hipError_t launch_rmsnorm_sumsq(const float* x, int T, int cols, int64_t ldx, float* ssq,
                                hipStream_t s);
hipError_t launch_rmsnorm(const float* x, int T, int cols, int64_t ldx,
                          const float* const* parts, int n_parts, int H, const float* g,
                          float eps, float* y, int64_t ldy, hipStream_t s);
hipError_t launch_dequant(const uint8_t* sbs, int bits, int64_t n_sb, int out_dtype, void* out,
                          hipStream_t s);

}  // namespace moe
