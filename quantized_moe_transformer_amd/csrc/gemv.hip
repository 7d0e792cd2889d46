// gemv.hip -- decode path: fused K-quant dequant-GEMV, fp32 accumulation.
//
// At one (or a few) token rows the layer is a stream of packed weight bytes:
// each byte is read once and used once, so the work is bound by HBM
// bandwidth (page "Distributed CPU: Zip Fusion Beyond Tensor Parallelism",
// section "Decode vs Prefill: Same Weights, Different Bottlenecks").  On this
// chip every dependent kernel adds a fixed cost of a few us to a step, so the
// layer runs as three kernels, each streaming its share of the bytes:
//
//   front   the router's split-K partial logits (many small XCD-grouped
//           workgroups; not launched when the routing is given, as in the
//           shard calls: two kernels);
//   gateup  the first wave of every routed workgroup sums its token's
//           partial logits in a fixed order and runs the top-k up to the
//           workgroup's slot (the same selection in every workgroup of the
//           token), then all four waves compute gate/up + SwiGLU of the
//           routed expert's rows; the shared expert's workgroups, which need
//           no routing, stream its rows from the start;
//   down    down projections, one wave per slot, slot results added in the
//           selected-slot order with the shared expert last (page "CKE Zip:
//           From Splitting Tokens To Splitting Qwen3.5 Weights", section "A
//           Separate Decode Result Shows Why Axis Choice Matters").
//
// Both weight formats (K-quant and MXFP4) run through the same kernels,
// templated on the format; only the piece decode and the superblock size differ.
//
// Work unit of a lane: a 16-byte piece of a superblock's codes -- 32 weights,
// 16 from sub-block 2c and 16 from sub-block 2c+1 -- plus the superblock's
// 16-byte head (and, at 5 bits, the matching 16 bytes of high bits).  Eight
// lanes cover one superblock, so the lanes of a wave read one contiguous run
// of a row.  The per-sub-block scale factors out of the dot product:
//   sum_i w_i x_i = d*sc_a*sum(q x)_a + d*sc_b*sum(q x)_b - dmin*(m_a sum x_a + m_b sum x_b)
// Every weight load of a wave is issued before the first one is consumed.
#include "launch.h"
#include "topk.h"

namespace moe {

// ---------------------------------------------------------------------------
// lane-level pieces
// ---------------------------------------------------------------------------

// Partial dot product of one lane's piece.  xl/xh: the 16 activations under
// the low / high nibbles; sl/sh their sums.  qh: the 16 high-bit bytes of the
// piece (5-bit format only).  Codes are unpacked four at a time from masked
// words (one byte-convert per code).
template <bool HIGH>
__device__ __forceinline__ float piece_dot(const SbHead& h, const uint4& qs, const uint4& qh, int c,
                                           const float* xl, const float* xh, float sl, float sh) {
    float sca, ma, scb, mb;
    sub_scale_min(h, 2 * c, sca, ma);
    sub_scale_min(h, 2 * c + 1, scb, mb);
    const uint32_t qw[4] = {qs.x, qs.y, qs.z, qs.w};
    const uint32_t hw[4] = {qh.x, qh.y, qh.z, qh.w};
    float dl = 0.f, dh = 0.f;
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
        uint32_t lo = and_opaque(qw[wi], 0x0f0f0f0fu);
        uint32_t hi = and_opaque(qw[wi] >> 4, 0x0f0f0f0fu);
        if (HIGH) {
            lo |= ((hw[wi] >> (2 * c)) & 0x01010101u) << 4;
            hi |= ((hw[wi] >> (2 * c + 1)) & 0x01010101u) << 4;
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            dl = __builtin_fmaf((float)((lo >> (8 * b)) & 0xffu), xl[4 * wi + b], dl);
            dh = __builtin_fmaf((float)((hi >> (8 * b)) & 0xffu), xh[4 * wi + b], dh);
        }
    }
    return h.d * (sca * dl + scb * dh) - h.dmin * (ma * sl + mb * sh);
}

// E2M1 codes of a word's four bytes (bits 0..3 of each) -> the bytes
// u = 2 * value + 12 (0..24): a byte permute looks the positive and the
// negative values up in two 8-entry tables, and the sign bit picks one.
__device__ __forceinline__ uint32_t e2m1_offset_bytes(uint32_t w) {
    // u of codes 0..7: 12 + 2 * {0, 0.5, 1, 1.5, 2, 3, 4, 6}; of codes 8..15: 12 - the same
    const uint32_t n7 = w & 0x07070707u;
    const uint32_t pos = __builtin_amdgcn_perm(0x18141210u, 0x0F0E0D0Cu, n7);
    const uint32_t neg = __builtin_amdgcn_perm(0x00040608u, 0x090A0B0Cu, n7);
    const uint32_t neg_mask = ((w >> 3) & 0x01010101u) * 0xffu;
    return (neg & neg_mask) | (pos & ~neg_mask);
}

// The same for an MXFP4 piece: 16 codes of sub-block 2c (low nibbles, under
// xl, summing to sl) and 16 of sub-block 2c+1 (high nibbles, under xh, sh).
// Each sub-block's scale is a power of two and factors out of its sum, and
// with u = 2 value + 12 per code:
//   sum_i w_i x_i = X_2c (sum(u x)_lo / 2 - 6 sl) + X_2c+1 (sum(u x)_hi / 2 - 6 sh)
// (one byte-convert and one fma per code).  s0 / s1: the superblock's scale
// bytes 0..3 / 4..7.
__device__ __forceinline__ float piece_dot_mx(uint32_t s0, uint32_t s1, const uint4& qs, int c,
                                              const float* xl, const float* xh, float sl, float sh) {
    const uint32_t sw = c < 2 ? s0 : s1;
    const int sft = 16 * (c & 1);
    const float xa = e8m0_f32((sw >> sft) & 0xffu), xb = e8m0_f32((sw >> (sft + 8)) & 0xffu);
    const uint32_t qw[4] = {qs.x, qs.y, qs.z, qs.w};
    float dl = 0.f, dh = 0.f;
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
        const uint32_t ul = e2m1_offset_bytes(qw[wi]);
        const uint32_t uh = e2m1_offset_bytes(qw[wi] >> 4);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            dl = __builtin_fmaf((float)((ul >> (8 * b)) & 0xffu), xl[4 * wi + b], dl);
            dh = __builtin_fmaf((float)((uh >> (8 * b)) & 0xffu), xh[4 * wi + b], dh);
        }
    }
    return xa * __builtin_fmaf(0.5f, dl, -6.f * sl) + xb * __builtin_fmaf(0.5f, dh, -6.f * sh);
}

// A superblock's 16-byte head for either format: K-quant d, dmin and scale
// words; MXFP4 its eight scale bytes as s0, s1.
template <int FMT>
__device__ __forceinline__ SbHead load_head_f(const uint8_t* sb) {
    if constexpr (FMT == MOE_WFMT_MXFP4) {
        const uint4 v = *reinterpret_cast<const uint4*>(sb);
        SbHead h;
        h.d = h.dmin = 0.f;
        h.s0 = v.x;
        h.s1 = v.y;
        h.s2 = 0u;
        return h;
    } else {
        return load_head(sb);
    }
}

template <int FMT, bool HIGH>
__device__ __forceinline__ float piece_dot_f(const SbHead& h, const uint4& qs, const uint4& qh, int c,
                                             const float* xl, const float* xh, float sl, float sh) {
    if constexpr (FMT == MOE_WFMT_MXFP4)
        return piece_dot_mx(h.s0, h.s1, qs, c, xl, xh, sl, sh);
    else
        return piece_dot<HIGH>(h, qs, qh, c, xl, xh, sl, sh);
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

// A wave-uniform read through the scalar cache (constant address space): its
// wait is on the scalar counter, not behind the vector loads in flight.  Only
// for data no kernel of the same grid writes.
template <typename T>
__device__ __forceinline__ T scalar_read(const T* p) {
    return *(const __attribute__((address_space(4))) T*)p;
}

// 16-byte load of streamed-once weight bytes, marked non-temporal.
__device__ __forceinline__ uint4 stream_load(const uint8_t* p) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Sum of each of N values (N = 2, 4 or 8) over the 64 lanes of a wave, by
// exchanging halves: values 0..N/2-1 stay on lanes with bit 5 clear, the rest
// on the others, then bit 4, and so on (log2 N lane exchanges instead of
// N * 6), and the rest of the sum inside groups of 64/N lanes.  Lane l ends
// with the sum of value sum_s bit(5 - s, l) * N / 2^(s+1).  Fixed order:
// deterministic.
template <int N>
__device__ __forceinline__ float wave_sum_n(const float* v) {
    static_assert(N == 2 || N == 4 || N == 8, "2, 4 or 8 values");
    const int lane = threadIdx.x & 63;
    float cur[N];
#pragma unroll
    for (int i = 0; i < N; ++i) cur[i] = v[i];
#pragma unroll
    for (int n = N, off = 32; n > 1; n >>= 1, off >>= 1) {
        const bool up = lane & off;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            const float keep = up ? cur[n / 2 + i] : cur[i];
            const float give = up ? cur[i] : cur[n / 2 + i];
            cur[i] = keep + __shfl_xor(give, off, 64);
        }
    }
    return wave_sum_group(cur[0], 64 / N);
}

// ---------------------------------------------------------------------------
// gate/up + SwiGLU for a group of rows of one expert instance
// ---------------------------------------------------------------------------

constexpr int kGuWaves = 4;   // waves per routed gate/up workgroup
constexpr int kGuSteps = 2;   // row steps per wave (each step: gate row + up row)

// The activations under one lane's pieces (they do not depend on the expert).
template <int LPR, int NSBL>
struct XRegs {
    float xl[NSBL][16], xh[NSBL][16], sl[NSBL], sh[NSBL];

    __device__ __forceinline__ void load(const float* __restrict__ xt) {
        const int task = (threadIdx.x & 63) % LPR;
        const int sbi = task >> 3, piece = task & 7, c = piece >> 1, hh = piece & 1;
#pragma unroll
        for (int it = 0; it < NSBL; ++it) {
            const int sb = sbi + (LPR / 8) * it;
            const float* xp = xt + sb * kSbWeights + 64 * c + 16 * hh;
            load16(xp, xl[it]);
            load16(xp + 32, xh[it]);
        }
    }
    __device__ __forceinline__ void sums() {
#pragma unroll
        for (int it = 0; it < NSBL; ++it) {
            float a = 0.f, b = 0.f;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                a += xl[it][q];
                b += xh[it][q];
            }
            sl[it] = a;
            sh[it] = b;
        }
    }
};

// LPR: lanes per row (8 * superblocks per row, capped at 64); NSBL:
// superblocks per lane per row (H / 2048 when LPR = 64, else 1).
// Rows [rbase, rbase + STEPS * 64/LPR) of the instance, h written to hrow.
template <int FMT, int LPR, int NSBL, int STEPS>
__device__ __forceinline__ void gateup_rows(const uint8_t* __restrict__ G,
                                            const uint8_t* __restrict__ U, int H, int Iloc,
                                            int i0, XRegs<LPR, NSBL>& X, int rbase,
                                            float* __restrict__ hrow) {
    constexpr int RS = 64 / LPR;   // rows side by side in a wave
    const int lane = threadIdx.x & 63;
    const int rslot = lane / LPR, task = lane % LPR;
    const int sbi = task >> 3, piece = task & 7, c = piece >> 1, hh = piece & 1;
    const int nsb_row = H / kSbWeights;

    SbHead hg[STEPS][NSBL], hu[STEPS][NSBL];
    uint4 qg[STEPS][NSBL], qu[STEPS][NSBL];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        const int r = min(rbase + st * RS + rslot, Iloc - 1);   // tail rows clamped, discarded
        const size_t row = (size_t)(i0 + r) * nsb_row;
#pragma unroll
        for (int it = 0; it < NSBL; ++it) {
            const int sb = sbi + (LPR / 8) * it;
            const uint8_t* gs = G + (row + sb) * kQ4Bytes;
            const uint8_t* us = U + (row + sb) * kQ4Bytes;
            qg[st][it] = stream_load(gs + 16 + 32 * c + 16 * hh);
            qu[st][it] = stream_load(us + 16 + 32 * c + 16 * hh);
            hg[st][it] = load_head_f<FMT>(gs);
            hu[st][it] = load_head_f<FMT>(us);
        }
    }
    // every weight load goes out before the first wait: left free, the
    // scheduler interleaves waits and decoding with these loads (it did so
    // for the short MXFP4 decode), which serialises their round trips
    __builtin_amdgcn_sched_barrier(0);
    X.sums();
    float (&xl)[NSBL][16] = X.xl;
    float (&xh)[NSBL][16] = X.xh;
    float (&sl)[NSBL] = X.sl;
    float (&sh)[NSBL] = X.sh;
    float v[2 * STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        float pg = 0.f, pu = 0.f;
#pragma unroll
        for (int it = 0; it < NSBL; ++it) {
            pg += piece_dot_f<FMT, false>(hg[st][it], qg[st][it], qg[st][it], c, xl[it], xh[it], sl[it], sh[it]);
            pu += piece_dot_f<FMT, false>(hu[st][it], qu[st][it], qu[st][it], c, xl[it], xh[it], sl[it], sh[it]);
        }
        v[2 * st] = pg;
        v[2 * st + 1] = pu;
    }
    if (LPR == 64 && (STEPS == 1 || STEPS == 2 || STEPS == 4)) {
        // one row per step: value 2*st (+1 for up) ends on the lanes whose
        // top log2(2*STEPS) bits spell it; gate and up of a step sit G lanes
        // apart
        constexpr int G = 32 / STEPS;
        const float s = wave_sum_n<2 * STEPS>(v);
        const float other = __shfl_xor(s, G, 64);
        const int r = rbase + lane / (2 * G);
        if ((lane & (2 * G - 1)) == 0 && r < Iloc) hrow[r] = silu_f(s) * other;
    } else {
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const float gs = wave_sum_group(v[2 * st], LPR);
            const float us = wave_sum_group(v[2 * st + 1], LPR);
            const int r = rbase + st * RS + rslot;
            if (task == 0 && r < Iloc) hrow[r] = silu_f(gs) * us;
        }
    }
}

// ---------------------------------------------------------------------------
// kernel arguments
// ---------------------------------------------------------------------------

struct GemvArgs {
    const uint8_t *gate, *up, *down, *sh_gate, *sh_up, *sh_down;
    const float* router_w;
    const float* x;
    int T, H, E, k, I, Is, nslot;
    int fmt;              // MOE_WFMT_*
    int i0, iloc;         // intermediate rows [i0, i0 + iloc) of every expert
    float sw;
    const int32_t* idx;   // routing read by gateup (when given) and by down
    const float* w;
    float* hbuf;          // [T*nslot][Iloc]
    int hstride;
    float* part;          // [T][E][ks] router partial logits
    int route;            // gateup computes the top-k from `part` ...
    int32_t* idx_out;     // ... and its first workgroup per token writes it here
    float* w_out;
    float* out;
};

constexpr int kRtE = 8;        // experts per router workgroup (two groups of four)
constexpr int kRtLine = 32;    // experts in one 128-byte line of a router row
constexpr int kXcds = 8;       // workgroups go to the XCDs round-robin by index

// Router workgroups per token tile: the four 8-expert quarters of every
// 32-expert line group, for each of the kRouterSplits K splits.
__host__ __device__ inline int router_blocks_per_tile(int E) {
    return (kRtLine / kRtE) * ((E + kRtLine - 1) / kRtLine) * kRouterSplits;
}

// ---------------------------------------------------------------------------
// front: router partial logits and the shared expert's gate/up
// ---------------------------------------------------------------------------

// Partial logits of TT tokens x kRtE experts over the ROWS = H / kRouterSplits
// rows of one split (NSB = H / 256, so ROWS = 32 * NSB).  Spread over many
// small workgroups (8 KB of the router matrix each at H = 2048), the router
// reads in about one memory round trip.  The four workgroups that read the
// same 128-byte lines (one 32-expert group of a split) get indices congruent
// modulo kXcds: they run on one XCD, whose L2 fetches each line once.
//
// Thread (q, g), q = tid % 2: experts 4q..4q+3 of the workgroup (one 16-byte
// load per row when E % 4 == 0; a lane pair reads a row's 32 bytes);
// g = tid / 2: rows g, g + G, ... of the split.  Each wave sums its 32 row
// groups across its lanes, the four waves are added in LDS, in a fixed order.
template <int TT, int NSB>
__device__ __forceinline__ void router_role(float* __restrict__ part, int tb, int u,
                                            const float* router_w, const float* x, int E, int H,
                                            int T) {
    constexpr int KS = kRouterSplits;
    static_assert(KS == kXcds, "one K split per XCD slot in the workgroup mapping");
    constexpr int ROWS = 32 * NSB;
    constexpr int G = ROWS < 128 ? ROWS : 128;   // row groups per expert group
    constexpr int RPT = ROWS / G;                // rows per thread
    __shared__ float xs[TT][ROWS];
    __shared__ float red[4][TT][kRtE];
    // tb: the token tile; u: the workgroup within it (the tile's count of
    // workgroups is a multiple of kXcds, so u % kXcds is the XCD slot)
    const int w = u / kXcds;                     // index among the workgroups of its XCD
    const int quarter = w % (kRtLine / kRtE);
    const int pair = (w / (kRtLine / kRtE)) * kXcds + u % kXcds;   // (line group, split)
    const int ks = pair % KS;
    const int ec = (pair / KS) * (kRtLine / kRtE) + quarter;
    if (ec * kRtE >= E) return;                // a quarter past the last expert
    const int t0 = tb * TT;
    const int nt = min(TT, T - t0);
    const int h0 = ks * ROWS;
    const int tid = threadIdx.x;
    const int q = tid & 1, g = tid >> 1;
    const bool rows_on = g < G;
    const int e0 = ec * kRtE + 4 * q;
    float wv[RPT][4];
    if (!rows_on) {
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) wv[r][c] = 0.f;
    } else if ((E & 3) == 0 && e0 + 3 < E) {
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float4 f =
                *reinterpret_cast<const float4*>(router_w + (size_t)(h0 + g + G * r) * E + e0);
            wv[r][0] = f.x;
            wv[r][1] = f.y;
            wv[r][2] = f.z;
            wv[r][3] = f.w;
        }
    } else {
#pragma unroll
        for (int r = 0; r < RPT; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                wv[r][c] = router_w[(size_t)(h0 + g + G * r) * E + min(e0 + c, E - 1)];
    }
    for (int i = tid; i < TT * ROWS; i += 256) {   // the front kernel's 256 threads
        const int tt = i / ROWS, hh = i % ROWS;
        xs[tt][hh] = tt < nt ? x[(size_t)(t0 + tt) * H + h0 + hh] : 0.f;
    }
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        // values 0..3: this lane's experts if q = 0, 4..7 if q = 1; the
        // other four are exact zeros
        float acc[kRtE];
#pragma unroll
        for (int c = 0; c < kRtE; ++c) acc[c] = 0.f;
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            const float xv = rows_on ? xs[tt][g + G * r] : 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float p = __builtin_fmaf(xv, wv[r][c], q ? acc[4 + c] : acc[c]);
                acc[c] = q ? acc[c] : p;
                acc[4 + c] = q ? p : acc[4 + c];
            }
        }
        // expert ee's sum over the wave ends on lanes 8ee..8ee+7
        const float sum = wave_sum_n<kRtE>(acc);
        if ((lane & 7) == 0) red[wave][tt][lane >> 3] = sum;
    }
    __syncthreads();
    if (tid < TT * kRtE) {
        const int tt = tid / kRtE, ee = tid % kRtE;
        const int eg = ec * kRtE + ee;
        if (tt < nt && eg < E)
            part[((size_t)(t0 + tt) * E + eg) * KS + ks] =
                ((red[0][tt][ee] + red[1][tt][ee]) + red[2][tt][ee]) + red[3][tt][ee];
    }
}

// Router partial logits (T <= kRouterSmallMaxT).  Every argument is a
// scalar one that the hardware preloads into registers (8 dwords): no
// argument load, and so no wait for one, sits between the router's loads
// and its store (a wait for LDS before a barrier also waits for any scalar
// load in flight).
template <int LPR, int NSBL, int TT>
__global__ void __launch_bounds__(256)
gemv_front_kernel(const float* __restrict__ router_w, const float* __restrict__ x,
                  float* __restrict__ part, uint32_t e_h, int T) {
    router_role<TT, (LPR / 8) * NSBL>(part, blockIdx.y, blockIdx.x, router_w, x, lo16(e_h),
                                      hi16(e_h), T);
}

// grid (row blocks, k + SH, T): slot j of token t, the slot and the token
// read from the block index with no division; SH (the layer has a shared
// expert): slot k is the shared expert's, which needs no routing and starts
// streaming at once.  The pointers and
// counts a workgroup needs -- for its first
// loads (activations, partial logits or the given routing) and for its
// weights and h row -- come in as preloaded kernel arguments, so no load
// waits for a kernel-argument load.
template <int FMT, int LPR, int NSBL, bool ROUTE, bool SH>
__device__ __forceinline__ void gateup_body(const float* __restrict__ x,
                                            const float* __restrict__ part,
                                            const int32_t* __restrict__ idx,
                                            const uint8_t* __restrict__ gate,
                                            const uint8_t* __restrict__ up, float* __restrict__ hbuf,
                                            int k, int nslot, int E, int H, int I, int iloc, int i0,
                                            int T, const GemvArgs& a) {
    const int j = blockIdx.y, t = blockIdx.z;   // slot j of token t
    const int wave = threadIdx.x >> 6;
    constexpr int rows_per_wave = kGuSteps * (64 / LPR);
    const int rbase = (blockIdx.x * kGuWaves + wave) * rows_per_wave;
    if constexpr (SH) {
        if (j >= k) {
            if (rbase >= iloc) return;
            XRegs<LPR, NSBL> X;
            X.load(x + (size_t)t * H);
            // the activation loads go out first: left free, the scheduler
            // may wait for the weights and decode them before it issues
            // these read-only loads (a memory clobber does not hold them)
            __builtin_amdgcn_sched_barrier(0);
            // the shared expert has the routed width
            gateup_rows<FMT, LPR, NSBL, kGuSteps>(a.sh_gate, a.sh_up, H, iloc, i0, X, rbase,
                                                  hbuf + (size_t)(t * nslot + k) * iloc);
            return;
        }
    }
    XRegs<LPR, NSBL> X;
    X.load(x + (size_t)t * H);   // independent of the routing: in flight during the top-k
    int e;
    if constexpr (ROUTE) {
        // the first wave selects (stopping at slot j, whose expert lane j
        // holds) and hands the expert to the others through LDS; the first
        // wave of workgroup (0, 0, t) fills all k slots and writes the
        // token's routing
        __shared__ int s_e;
        if (threadIdx.x < 64) {
            if (blockIdx.x == 0 && j == 0) {
                const int my_e = wave_topk<4, kRouterSplits>(part, E, k, t,
                                                             a.idx_out + (size_t)t * k,
                                                             a.w_out + (size_t)t * k);   // E <= 256
                e = __builtin_amdgcn_readfirstlane(my_e);
            } else {
                float my_l, top;
                int my_e;
                wave_topk_select<4, kRouterSplits>(part, E, j + 1, t, my_l, my_e, top);
                e = __builtin_amdgcn_readlane(my_e, j);
            }
            if (threadIdx.x == 0) s_e = e;
        }
        __syncthreads();
        e = s_e;
    } else {
        e = idx[(size_t)t * k + j];
    }
    if ((unsigned)e >= (unsigned)E) return;
    if (rbase >= iloc) return;
    const size_t mat = (size_t)I * H / kSbWeights * kQ4Bytes;   // MXFP4: the same size
    gateup_rows<FMT, LPR, NSBL, kGuSteps>(gate + (size_t)e * mat, up + (size_t)e * mat, H, iloc,
                                          i0, X, rbase, hbuf + (size_t)(t * nslot + j) * iloc);
}

// The layer routes its own rows: the top-k from the front kernel's partial
// logits, for the whole layer (rows [0, I) of every expert).
template <int FMT, int LPR, int NSBL, bool SH>
__global__ void __launch_bounds__(64 * kGuWaves)
gemv_gateup_kernel(const float* __restrict__ x, const float* __restrict__ part,
                   const uint8_t* __restrict__ gate, const uint8_t* __restrict__ up,
                   float* __restrict__ hbuf, uint32_t k_nslot, uint32_t e_h, int I, int T,
                   GemvArgs a) {
    gateup_body<FMT, LPR, NSBL, true, SH>(x, part, nullptr, gate, up, hbuf, lo16(k_nslot),
                                          hi16(k_nslot), lo16(e_h), hi16(e_h), I, I, 0, T, a);
}

// The routing is given (shard and range calls, or the router ran first).
template <int FMT, int LPR, int NSBL, bool SH>
__global__ void __launch_bounds__(64 * kGuWaves)
gemv_gateup_given_kernel(const int32_t* __restrict__ idx, const uint8_t* __restrict__ gate,
                         const uint8_t* __restrict__ up, float* __restrict__ hbuf,
                         uint32_t k_nslot, uint32_t e_h, uint32_t iloc_i0, int I, int T,
                         GemvArgs a) {
    gateup_body<FMT, LPR, NSBL, false, SH>(a.x, nullptr, idx, gate, up, hbuf, lo16(k_nslot),
                                           hi16(k_nslot), lo16(e_h), hi16(e_h), I, lo16(iloc_i0),
                                           hi16(iloc_i0), T, a);
}

// ---------------------------------------------------------------------------
// down + slot-order combine
// ---------------------------------------------------------------------------

constexpr int kDnPasses = 2;   // row passes per wave in the down kernel

// Block: one wave per slot (nw = min(nslot, 16) waves, slot j on wave j % nw),
// kDnPasses * (64 / LPRD) output rows of one token.  A row's I_loc inputs are
// I_loc / 32 lane tasks of 32 (a 16-byte code piece each); LPRD, the lanes per
// row, is that count rounded up to a power of two, the extra lanes adding 0.
// The routing and h pointers and the counts their addresses need come first
// as scalar arguments, which the hardware preloads into registers: a wave's
// first loads (the slot's expert and weight, its h) then wait for no
// kernel-argument load.
template <int FMT, int LPRD>
__global__ void __launch_bounds__(1024)
gemv_down_kernel(const int32_t* __restrict__ idx, const float* __restrict__ wts,
                 const float* __restrict__ hbuf, int k, int nslot, int hstride, int iloc,
                 GemvArgs a) {
    constexpr int SBB = FMT == MOE_WFMT_MXFP4 ? kMxBytes : kQ5Bytes;
    constexpr int rs = 64 / LPRD;                 // rows per pass
    __shared__ float ys[17][kDnPasses * 64];
    __shared__ float s_wt[17];   // each slot's weight (0 for an invalid expert)
    const int t = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nw = nslot < 16 ? nslot : 16;       // the launch's waves (no argument load)
    const int rslot = lane / LPRD, task = lane % LPRD;
    const bool active = task < (iloc >> 5);
    const int cg = active ? task >> 1 : 0, hh = task & 1;
    const int obase = blockIdx.x * kDnPasses * rs;
    const int H = a.H;
    // the routing reads of the wave's first slot go out first of all, from
    // preloaded arguments only, so that they and the loads of the other
    // arguments take one round trip together
    const int jf = __builtin_amdgcn_readfirstlane(wave);
    int ef = 0;
    float wf = 0.f;
    if (jf < k) {
        ef = scalar_read(idx + (size_t)t * k + jf);
        wf = scalar_read(wts + (size_t)t * k + jf);
    }
    for (int jv = wave; jv < nslot; jv += nw) {
        const int j = __builtin_amdgcn_readfirstlane(jv);   // wave-uniform
        // the routing reads first, then h (it does not depend on the
        // routing): the wait for the expert index covers only the routing
        // reads, and the h sums wait only for h (vector loads complete in
        // issue order); the weight loads follow
        int e = 0;
        float wj = a.sw;
        if (j < k) {
            if (j == jf) {
                e = ef;
                wj = wf;
            } else {
                e = scalar_read(idx + (size_t)t * k + j);
                wj = scalar_read(wts + (size_t)t * k + j);
            }
        }
        const float* hp = hbuf + (size_t)(t * nslot + j) * hstride + 64 * cg + 16 * hh;
        float hl[16], hu[16];
        load16(hp, hl);
        load16(hp + 32, hu);
        const uint8_t* D;
        int Iexp;
        bool valid = true;
        if (j < k) {
            valid = (unsigned)e < (unsigned)a.E;
            D = a.down + (size_t)(valid ? e : 0) * ((size_t)H * a.I / kSbWeights * SBB);
            Iexp = a.I;
        } else {
            D = a.sh_down;
            Iexp = a.Is;
        }
        if (lane == 0) s_wt[j] = valid ? wj : 0.f;
        const int i0 = a.i0;
        SbHead hd[kDnPasses];
        uint4 qh[kDnPasses], qs[kDnPasses];
        int cc[kDnPasses];
#pragma unroll
        for (int ps = 0; ps < kDnPasses; ++ps) {
            const int o = min(obase + ps * rs + rslot, H - 1);
            const size_t base = (size_t)o * Iexp + i0 + 64 * cg;
            cc[ps] = (int)((base & 255) >> 6);
            const uint8_t* sb = D + (base >> 8) * SBB;
            if (FMT == MOE_WFMT_MXFP4) {
                qs[ps] = stream_load(sb + 16 + 32 * cc[ps] + 16 * hh);
                qh[ps] = qs[ps];
            } else {
                qs[ps] = stream_load(sb + 48 + 32 * cc[ps] + 16 * hh);
                qh[ps] = stream_load(sb + 16 + 16 * hh);
            }
            hd[ps] = load_head_f<FMT>(sb);
        }
        asm volatile("" ::: "memory");   // every load above is issued before the sums
        float sa = 0.f, sb2 = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            sa += hl[q];
            sb2 += hu[q];
        }
#pragma unroll
        for (int ps = 0; ps < kDnPasses; ++ps) {
            const float part =
                active ? piece_dot_f<FMT, true>(hd[ps], qs[ps], qh[ps], cc[ps], hl, hu, sa, sb2) : 0.f;
            const float y = wave_sum_group(part, LPRD);
            if (task == 0) ys[j][ps * rs + rslot] = valid ? y : 0.f;
        }
    }
    __syncthreads();
    if ((int)threadIdx.x < kDnPasses * rs) {
        const int r = threadIdx.x;
        const int o = obase + r;
        if (o < H) {
            float acc = 0.f;
            for (int j = 0; j < nslot; ++j) acc = __builtin_fmaf(s_wt[j], ys[j][r], acc);
            a.out[(size_t)t * H + o] = acc;
        }
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static GemvArgs base_args(const moe_layer_desc& d, const float* x, int T, int i0, int iloc) {
    GemvArgs a = {};
    a.gate = d.gate_q;
    a.up = d.up_q;
    a.down = d.down_q;
    a.sh_gate = d.sh_gate_q;
    a.sh_up = d.sh_up_q;
    a.sh_down = d.sh_down_q;
    a.router_w = d.router_w;
    a.x = x;
    a.T = T;
    a.H = d.hidden;
    a.E = d.n_experts;
    a.k = d.top_k;
    a.I = d.inter;
    a.Is = d.shared_inter;
    a.i0 = i0;
    a.iloc = iloc;
    a.nslot = d.top_k + (d.shared_inter > 0 ? 1 : 0);
    a.sw = d.shared_weight;
    a.fmt = d.weight_format;
    return a;
}

template <int LPR, int NSBL>
static void launch_front_t(const GemvArgs& a, const Ctx& c) {
    const int TT = a.T == 1 ? 1 : 4;   // tokens per workgroup
    const dim3 grid(router_blocks_per_tile(a.E), (a.T + TT - 1) / TT);
    const uint32_t e_h = pack16(a.E, a.H);
    if (a.T == 1)
        launch_k(c, MOE_K_GEMV_FRONT, gemv_front_kernel<LPR, NSBL, 1>, grid, dim3(256), 0,
                 a.router_w, a.x, a.part, e_h, a.T);
    else
        launch_k(c, MOE_K_GEMV_FRONT, gemv_front_kernel<LPR, NSBL, 4>, grid, dim3(256), 0,
                 a.router_w, a.x, a.part, e_h, a.T);
}

template <int LPR, int NSBL>
static hipError_t launch_gateup_t(const GemvArgs& a, const Ctx& c) {
    constexpr int rows_per_block = kGuWaves * kGuSteps * (64 / LPR);
    const int Iloc = a.iloc;
    const bool sh = a.nslot > a.k;   // a shared expert: slot k of each token
    const dim3 grid((Iloc + rows_per_block - 1) / rows_per_block, a.k + (sh ? 1 : 0), a.T);
    const dim3 block(64 * kGuWaves);
    if (a.k > 0xffff || a.nslot > 0xffff || a.E > 0xffff || a.H > 0xffff)
        return hipErrorInvalidValue;   // packed in 16 bits
    const uint32_t k_nslot = pack16(a.k, a.nslot), e_h = pack16(a.E, a.H);
    if (a.route) {
        // the whole layer: rows [0, I) of every expert
        if (a.i0 != 0 || a.iloc != a.I) return hipErrorInvalidValue;
#define MOE_GATEUP_R(F, S)                                                                       \
    launch_k(c, MOE_K_GATEUP_GEMV, gemv_gateup_kernel<F, LPR, NSBL, S>, grid, block, 0, a.x,     \
             (const float*)a.part, a.gate, a.up, a.hbuf, k_nslot, e_h, a.I, a.T, a)
        if (a.fmt == MOE_WFMT_MXFP4) {
            if (sh) MOE_GATEUP_R(MOE_WFMT_MXFP4, true);
            else MOE_GATEUP_R(MOE_WFMT_MXFP4, false);
        } else {
            if (sh) MOE_GATEUP_R(MOE_WFMT_KQUANT, true);
            else MOE_GATEUP_R(MOE_WFMT_KQUANT, false);
        }
#undef MOE_GATEUP_R
        return hipGetLastError();
    }
    if (a.i0 > 0xffff || a.iloc > 0xffff) return hipErrorInvalidValue;
    const uint32_t iloc_i0 = pack16(a.iloc, a.i0);
#define MOE_GATEUP(F, S)                                                                         \
    launch_k(c, MOE_K_GATEUP_GEMV, gemv_gateup_given_kernel<F, LPR, NSBL, S>, grid, block, 0,    \
             a.idx, a.gate, a.up, a.hbuf, k_nslot, e_h, iloc_i0, a.I, a.T, a)
    if (a.fmt == MOE_WFMT_MXFP4) {
        if (sh) MOE_GATEUP(MOE_WFMT_MXFP4, true);
        else MOE_GATEUP(MOE_WFMT_MXFP4, false);
    } else {
        if (sh) MOE_GATEUP(MOE_WFMT_KQUANT, true);
        else MOE_GATEUP(MOE_WFMT_KQUANT, false);
    }
#undef MOE_GATEUP
    return hipGetLastError();
}

#define MOE_DISPATCH_H(nsb, F, ...)                                  \
    switch (nsb) {                                                   \
        case 1: F<8, 1>(__VA_ARGS__); break;                         \
        case 2: F<16, 1>(__VA_ARGS__); break;                        \
        case 4: F<32, 1>(__VA_ARGS__); break;                        \
        case 8: F<64, 1>(__VA_ARGS__); break;                        \
        case 16: F<64, 2>(__VA_ARGS__); break;                       \
        default: return hipErrorInvalidValue;                        \
    }

// Front kernel: router partial logits (T <= kRouterSmallMaxT).
static hipError_t launch_front(GemvArgs& a, const WsLayout& L, char* ws, const Ctx& c) {
    const int nsb = a.H / kSbWeights;
    a.part = reinterpret_cast<float*>(ws + L.router_part);
    if (a.E > 0xffff || a.H > 0xffff) return hipErrorInvalidValue;   // packed in 16 bits
    MOE_DISPATCH_H(nsb, launch_front_t, a, c);
    return hipGetLastError();
}

// Router partial logits only (router_topk at T <= kRouterSmallMaxT).
hipError_t launch_router_small(const moe_layer_desc& d, const float* x, int T, char* ws,
                               const WsLayout& L, const Ctx& c) {
    GemvArgs a = base_args(d, x, T, 0, 1);
    return launch_front(a, L, ws, c);
}

hipError_t launch_router(const moe_layer_desc& d, const float* x, int T, int32_t* idx, float* w,
                         char* ws, const WsLayout& L, const Ctx& c);   // router.hip

template <int LPRD>
static hipError_t launch_down_t(const GemvArgs& a, int T, const Ctx& c) {
    constexpr int rows_per_block = kDnPasses * (64 / LPRD);
    const int nw = a.nslot < 16 ? a.nslot : 16;
    const dim3 grid2((a.H + rows_per_block - 1) / rows_per_block, T);
    if (a.fmt == MOE_WFMT_MXFP4)
        launch_k(c, MOE_K_DOWN_GEMV, gemv_down_kernel<MOE_WFMT_MXFP4, LPRD>, grid2, dim3(64 * nw),
                 0, a.idx, a.w, a.hbuf, a.k, a.nslot, a.hstride, a.iloc, a);
    else
        launch_k(c, MOE_K_DOWN_GEMV, gemv_down_kernel<MOE_WFMT_KQUANT, LPRD>, grid2, dim3(64 * nw),
                 0, a.idx, a.w, a.hbuf, a.k, a.nslot, a.hstride, a.iloc, a);
    return hipGetLastError();
}

hipError_t launch_gemv(const moe_layer_desc& d, const float* x, int T, const int32_t* idx,
                       const float* w, int i0, int iloc, float* out, char* ws,
                       const WsLayout& L, const Ctx& c, bool route) {
    GemvArgs a = base_args(d, x, T, i0, iloc);
    const int Iloc = iloc;
    a.hbuf = reinterpret_cast<float*>(ws + L.hbuf);
    a.hstride = Iloc;
    a.out = out;
    // small T: partials in the front kernel, top-k inside the gate/up kernel;
    // otherwise the matrix-core router runs first
    const bool fused_route = route && T <= kRouterSmallMaxT && d.n_experts <= 256;
    if (route) {
        a.idx_out = reinterpret_cast<int32_t*>(ws + L.idx);
        a.w_out = reinterpret_cast<float*>(ws + L.w);
        if (!fused_route) {
            hipError_t e = launch_router(d, x, T, a.idx_out, a.w_out, ws, L, c);
            if (e != hipSuccess) return e;
        }
        idx = a.idx_out;
        w = a.w_out;
    }
    // the front kernel: the router's partial logits, when this call routes
    // its own rows here (the gate/up kernel then runs the top-k)
    if (fused_route) {
        hipError_t e = launch_front(a, L, ws, c);
        if (e != hipSuccess) return e;
    } else {
        a.part = reinterpret_cast<float*>(ws + L.router_part);
    }
    a.route = fused_route ? 1 : 0;
    a.idx = idx;
    a.w = w;
    const int nsb = d.hidden / kSbWeights;
    hipError_t ge = hipSuccess;
    switch (nsb) {
        case 1: ge = launch_gateup_t<8, 1>(a, c); break;
        case 2: ge = launch_gateup_t<16, 1>(a, c); break;
        case 4: ge = launch_gateup_t<32, 1>(a, c); break;
        case 8: ge = launch_gateup_t<64, 1>(a, c); break;
        case 16: ge = launch_gateup_t<64, 2>(a, c); break;
        default: return hipErrorInvalidValue;
    }
    if (ge != hipSuccess) return ge;
    int lprd = 2;   // lanes per down row: Iloc / 32 rounded up to a power of two
    while (lprd < Iloc / 32) lprd *= 2;
    switch (lprd) {
        case 2: return launch_down_t<2>(a, T, c);
        case 4: return launch_down_t<4>(a, T, c);
        case 8: return launch_down_t<8>(a, T, c);
        case 16: return launch_down_t<16>(a, T, c);
        case 32: return launch_down_t<32>(a, T, c);
        case 64: return launch_down_t<64>(a, T, c);
        default: return hipErrorInvalidValue;   // Iloc > 2048 (not on this path)
    }
}

}  // namespace moe
