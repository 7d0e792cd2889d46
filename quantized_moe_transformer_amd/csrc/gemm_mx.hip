// gemm_mx.hip -- prefill path for MXFP4 expert weights: the grouped GEMM on
// gfx950's block-scaled matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// The page "Distributed CPU: Zip Fusion Beyond Tensor Parallelism", section
// "Decode vs Prefill: Same Weights, Different Bottlenecks", says the model
// class targeted ships an MXFP4-class format, and that with many rows the
// expert FFN is a dense contraction bound by matrix throughput.  gfx950's
// matrix cores take OCP MX operands directly: 4- or 8-bit codes with one E8M0
// power-of-two scale per 32 values along K, applied exactly in hardware.
//
// Weights (the B operand) go to the matrix cores as they are stored: FP4 E2M1
// codes and their E8M0 scale per 32 weights.  The only work on them is a
// repack from the superblock's nibble order (element 64c + l in the low
// nibble of code byte 32c + l, element 64c + 32 + l in its high nibble) into
// the operand's (element 32b + 2i in the low nibble of byte i, 2i + 1 in the
// high nibble).  There is no dequantisation and no 16-bit weight stage, so
// every E8M0 scale byte is honoured exactly (255, the format's NaN, gives NaN).
//
// Tokens (gate/up) and h (down) are the A operand, as the sum of NT MX-FP8
// terms: per 32 values, term t has an E8M0 scale s_t (the smallest that keeps
// the block's largest remainder within e4m3's 448) and e4m3 codes (rounded to
// nearest even) of what the terms before it left over.  The product is then
// NT block-scaled MFMAs into one fp32 accumulator.  Each term adds about four
// bits: the representation error of a value is at most 2^(-4 NT) times its
// block's largest magnitude (below e4m3's subnormal range it is absolute, at
// 2^-10 of the term's scale).
//
// Tile structure, bucketing and the block -> tile mapping are those of the
// fp16 grouped GEMM (gemm.hip): one tile is up to 160 rows of one expert's
// group times 256 weight rows, K in steps of 64 (one MFMA, two MX blocks).
//   4 consumer waves: the A stage by direct global-to-LDS loads one step
//     ahead; per step NT x MB x 2 block-scaled MFMAs;
//   4 producer waves: thread p owns weight row p; its codes and scales for
//     step k + 1 (loaded PD steps ahead into registers) are repacked into the
//     other B stage.
//   gateup (MODE 0): the epilogue forms h = silu(gate) * up in fp32, stages it
//     through LDS and writes it as NT-term MX-FP8 (the down GEMM's A operand).
//   down (MODE 1): the epilogue scales by the routing weight and writes the
//     slot's row of the per-slot buffer, as the fp16 kernel does.
#include "launch.h"

namespace moe {

constexpr int kMxK = 64;         // K per step (one MFMA)
constexpr int kMxScaleRow = 16;  // scale bytes per (row, step): byte 8b + t = term t of MX block b
constexpr int kMxPD = 2;         // producer prefetch distance (steps)
constexpr int kMxAStages = 3;    // A stages: the token / h rows of a step are requested two steps ahead
constexpr int kMxConsumers = 4;  // consumer waves
constexpr int kMxThreads = 512;  // 4 consumer + 4 producer waves
constexpr int kMxTN = 256;       // weight rows per tile

typedef int v8i __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// NT-term MX-FP8 coding of 32-value blocks
// ---------------------------------------------------------------------------

// E8M0 exponent for a block whose largest magnitude is m: the smallest s with
// m * 2^-s <= 448 (e4m3's largest finite value, 0.875 * 2^9), clamped to the
// format's range [-127, 127]; m = 0 gives -127.
__device__ __forceinline__ int mx_scale_exp(float m) {
    if (!(m > 0.f)) return -127;
    int e;
    const float f = __builtin_frexpf(m, &e);   // m = f 2^e, f in [0.5, 1)
    int s = e - 9 + (f > 0.875f ? 1 : 0);
    return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// The 8 values v of one lane, a quarter of a 32-value block held by 4
// consecutive lanes (lane % 4 = the quarter), as NT terms.  codes[t][w]
// packs the e4m3 codes of values 4w .. 4w+3 (the first in the low byte);
// scales packs the E8M0 bytes of the NT terms (term t in byte t), the same in
// the block's 4 lanes.  Every lane of the wave must take part (lane
// exchanges).
template <int NT>
__device__ __forceinline__ void mx_fp8_terms(const float (&v)[8], uint32_t (&codes)[NT][2],
                                             uint32_t& scales) {
    float r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = v[i];
    scales = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(r[i]));
        m = __builtin_fmaxf(m, __shfl_xor(m, 1, 64));
        m = __builtin_fmaxf(m, __shfl_xor(m, 2, 64));
        const int s = mx_scale_exp(m);
        scales |= (uint32_t)(s + 127) << (8 * t);
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            int c = 0;
            c = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(r[4 * w], -s),
                                                __builtin_ldexpf(r[4 * w + 1], -s), c, false);
            c = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_ldexpf(r[4 * w + 2], -s),
                                                __builtin_ldexpf(r[4 * w + 3], -s), c, true);
            codes[t][w] = (uint32_t)c;
            if (t + 1 < NT) {
                // what this term codes, exactly: code * 2^s (the difference
                // from r is exact in fp32)
                r[4 * w] -= __builtin_ldexpf(__builtin_amdgcn_cvt_f32_fp8(c, 0), s);
                r[4 * w + 1] -= __builtin_ldexpf(__builtin_amdgcn_cvt_f32_fp8(c, 1), s);
                r[4 * w + 2] -= __builtin_ldexpf(__builtin_amdgcn_cvt_f32_fp8(c, 2), s);
                r[4 * w + 3] -= __builtin_ldexpf(__builtin_amdgcn_cvt_f32_fp8(c, 3), s);
            }
        }
    }
}

// Store a lane's part of one block: codes of term t at rowq + t * term_stride
// (8 bytes, values [8 quarter, 8 quarter + 8) of the block), and the scales of
// block b of its 64-wide step at rows + 8 b (the block's quarter-0 lane).
template <int NT>
__device__ __forceinline__ void mx_store_block(uint8_t* rowq, size_t term_stride, uint8_t* rows,
                                               int b, int quarter, const uint32_t (&codes)[NT][2],
                                               uint32_t scales) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
        *reinterpret_cast<uint2*>(rowq + t * term_stride + 8 * quarter) =
            make_uint2(codes[t][0], codes[t][1]);
    if (quarter == 0) *reinterpret_cast<uint32_t*>(rows + 8 * b) = scales;
}

// Tokens x fp32 [T][H] -> NT-term MX-FP8: codes [NT][T][H], scales [T][H/64][16].
// One thread per quarter block.
template <int NT>
__global__ void __launch_bounds__(256)
mx_split_kernel(const float* __restrict__ x, int T, int H, uint8_t* __restrict__ q,
                uint8_t* __restrict__ s) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;   // quarter-block index
    const size_t nq = (size_t)T * H / 8;
    // the grid covers whole groups of 4 lanes; lanes past the end take part
    // in the exchanges with zeros and store nothing
    const bool live = i < nq;
    const size_t ii = live ? i : 0;
    const size_t row = ii / (H / 8);
    const int col = (int)(ii % (H / 8)) * 8;                          // first of the 8 values
    float v[8];
    if (live) {
        const float4 a = *reinterpret_cast<const float4*>(x + row * H + col);
        const float4 b = *reinterpret_cast<const float4*>(x + row * H + col + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = 0.f;
    }
    uint32_t codes[NT][2], scales;
    mx_fp8_terms<NT>(v, codes, scales);
    if (!live) return;
    const int blk = col / 32, quarter = (col / 8) & 3;
    mx_store_block<NT>(q + row * H + 32 * blk, (size_t)T * H,
                       s + (row * (H / kMxK) + blk / 2) * kMxScaleRow, blk & 1, quarter, codes,
                       scales);
}

// ---------------------------------------------------------------------------
// the block-scaled grouped GEMM
// ---------------------------------------------------------------------------

struct MxGemmArgs {
    const uint8_t* aq;              // A codes [NT][rows][K]
    const uint8_t* as;              // A scales [rows][K/64][16]
    size_t a_term;                  // bytes between A terms
    int K;                          // A row length (H for gate/up, the shard's width for down)
    const int32_t* perm;            // expert-sorted slot ids
    const int32_t* tile_off;        // [E+2]: group tile starts
    const int4* tile_rec;           // per row tile: group, first sorted row, rows, row offset
    int T, H, E, k, I, Is;
    int i0, iloc;                   // intermediate rows [i0, i0 + iloc) of every expert
    const uint8_t *w_routed, *w_routed2, *w_shared, *w_shared2;   // MODE 0: gate, up
    const float* route_w;           // [T*k] routing weights
    float sw;
    int n_ntiles;                   // weight-row tiles per group
    int nk;                         // K steps
    uint8_t* hq;                    // MODE 0: h codes [NT][T*k + T][iloc]
    uint8_t* hs;                    // MODE 0: h scales [T*k + T][iloc/64][16]
    size_t h_term;
    int16_t* y;                     // MODE 1: [T*k][H] (16-bit block floating point)
    int16_t* ysh;                   // MODE 1: [T][H]
    uint8_t* ysc;                   // MODE 1: [T*k][H/8] exponent bytes of y
    uint8_t* yshsc;                 // MODE 1: [T][H/8] those of ysh
};

// LDS banks as measured on gfx950 (SQ_LDS_BANK_CONFLICT of single access
// patterns): a 16-byte read serves 16 consecutive lanes per pass over 64
// four-byte banks, with address bit 7 XOR address bit 9 choosing the upper 32;
// a 16-byte write serves 8 lanes per pass over 32 banks (address bits 2..6); a
// 4-byte read serves 32 lanes per pass over 32 banks.  The code reads and
// writes below keep the accesses of one pass on distinct banks under those
// rules, assuming the MxLds object starts at LDS address 0 (it is the kernel's
// only LDS object).  The A-scale dword reads (one per row block and step) put
// 4 lanes on each bank through the 16-byte row stride; a 16-byte read of the
// whole chunk, which avoids that, measured no faster.
//
// A stage of MB 32-row blocks: term t's 64 code bytes of row r at 16-byte slot
// 4 (t R + r) + (c ^ sw(r)) (R = 32 MB rows, c the chunk), then row r's 16
// scale bytes at slot 4 NT R + r.  A fragment read pass takes 16 consecutive
// rows: row bits 0 and 1 ^ 3 pick the bank quarter and position, and the
// swizzle moves row bits 2 and 3 into the chunk position.
__device__ __forceinline__ int mx_swz(int r) { return (r >> 2) & 3; }
template <int NT, int MB>
struct MxStage {
    static constexpr int R = 32 * MB;
    static constexpr int kSlots = (4 * NT + 1) * R;           // 16-byte slots used
    static constexpr int kLoads = (kSlots + 255) / 256;        // loads per consumer thread
    static constexpr int kBytes = kLoads * 256 * 16;           // with the last load's tail
};

constexpr int kMxStageMax = MxStage<kMxTerms, 5>::kBytes;      // the largest A stage
constexpr int kMxRing = kMxPD + 1;                             // producer raw-chunk ring slots

// B stage row n: the 16 code bytes of MX block b at 16 (b ^ s(n)), s(n) = bit 2
// XOR bit 3 of n, so that both the 16 rows of a consumer's read pass and the 8
// rows of a producer's write pass fall on distinct banks.
__device__ __forceinline__ int mx_bswz(int n, int b) { return 16 * (b ^ (((n >> 2) ^ (n >> 3)) & 1)); }

struct __align__(16) MxLds {
    uint8_t a[kMxAStages][kMxStageMax];
    uint8_t bq[2][kMxTN][32];
    uint8_t bs[2][2][kMxTN];         // E8M0 byte of (weight row, MX block b)
    // producer ring: per step, weight row p's code bytes 32c .. 32c + 15,
    // 32c + 16 .. 32c + 31 and the scale word of its superblock holding bytes
    // 2c, 2c + 1
    uint4 rq[kMxRing][2][kMxTN];
    uint32_t rs[kMxRing][kMxTN];
    int32_t row_src[kTileM];         // MODE 1: slot id of each row
    float row_w[kTileM];             // MODE 1: routing weight of each row
};
// the bank layouts above hold for stages that start on 1 KiB boundaries; the
// epilogue's staging rows (at most 32 x (kMxTN + 4) floats) end before row_src
static_assert(kMxStageMax % 1024 == 0 && offsetof(MxLds, bq) % 1024 == 0, "stage alignment");
static_assert(32 * (kMxTN + 4) * sizeof(float) <= offsetof(MxLds, row_src), "epilogue staging");
static_assert(sizeof(MxLds) <= 160 * 1024, "LDS size");

// 32 code bytes (sub-block 2c: low nibbles, 2c + 1: high nibbles) -> the
// operand order of each sub-block: out0 (block 2c) and out1 (block 2c + 1),
// 16 bytes each, element 2i in the low nibble of byte i.
__device__ __forceinline__ void mx_repack(const uint4& lo, const uint4& hi, uint4& out0,
                                          uint4& out1) {
    const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t o0[4], o1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // bytes 8j .. 8j + 7: even and odd bytes side by side
        const uint32_t ev = __builtin_amdgcn_perm(w[2 * j + 1], w[2 * j], 0x06040200u);
        const uint32_t od = __builtin_amdgcn_perm(w[2 * j + 1], w[2 * j], 0x07050301u);
        o0[j] = (ev & 0x0f0f0f0fu) | ((od << 4) & 0xf0f0f0f0u);
        o1[j] = ((ev >> 4) & 0x0f0f0f0fu) | (od & 0xf0f0f0f0u);
    }
    out0 = make_uint4(o0[0], o0[1], o0[2], o0[3]);
    out1 = make_uint4(o1[0], o1[1], o1[2], o1[3]);
}

// The NT terms of one step, term T's MFMAs reading its scale from byte T of
// the A scale dword (the operand's scale byte select is an immediate).
template <int T, int NT, int MB>
struct MxTerms {
    __device__ __forceinline__ static void run(const uint8_t* sa, int nl, int hb, const v8i (&bf)[2],
                                               const uint32_t (&bsc)[2], const uint32_t (&asc)[MB],
                                               float16v (&acc)[MB][2]) {
        if constexpr (T < NT) {
            constexpr int R = MxStage<NT, MB>::R;
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                const int r = 32 * i + nl;
                const uint8_t* rowp = sa + 64 * (T * R + r);
                const uint4 p0 = *reinterpret_cast<const uint4*>(rowp + 16 * (hb ^ mx_swz(r)));
                const uint4 p1 = *reinterpret_cast<const uint4*>(rowp + 16 * ((2 + hb) ^ mx_swz(r)));
                const v8i af = v8i{(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w,
                                   (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
                acc[i][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    af, bf[0], acc[i][0], 0, 4, T, (int)asc[i], 0, (int)bsc[0]);
                acc[i][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    af, bf[1], acc[i][1], 0, 4, T, (int)asc[i], 0, (int)bsc[1]);
            }
            MxTerms<T + 1, NT, MB>::run(sa, nl, hb, bf, bsc, asc, acc);
        }
    }
};

struct MxTileInfo {
    int g, m0, mcount, grow0, Iexp, Iloc, i0, n0;
    bool is_sh;
};

// wait until at most 3 n of this wave's direct loads are in flight (n <= 2)
__device__ __forceinline__ void mx_wait_steps(int n) {
    if (n >= 2) wait_vmcnt<6>();
    else if (n == 1) wait_vmcnt<3>();
    else wait_vmcnt<0>();
}

// Producers: thread p owns weight row p of the tile.  Its three 16-byte
// chunks of step kk (the pair's 32 code bytes and the superblock's scale
// chunk) arrive by direct global-to-LDS loads kMxPD steps ahead into a ring
// of kMxRing slots, waited for with explicit counts; each step they are
// repacked into the B stage the consumers read next.
template <int MODE>
__device__ __forceinline__ void mx_produce(const MxGemmArgs& a, const MxTileInfo& ti, MxLds& lds) {
    static_assert(kMxPD <= 3, "mx_wait_steps covers two later steps");
    const int p = threadIdx.x - 64 * kMxConsumers;
    const int pw = p >> 6;
    // the weight row and the element offset of its K range in the flat matrix
    const uint8_t* mat;
    size_t e0;
    if (MODE == 0) {
        const int col = p & 127;
        const int colc = ti.n0 + col < ti.Iloc ? col : 0;   // ragged tile: discarded columns
        const size_t msz = (size_t)a.I * a.H / kSbWeights * kMxBytes;
        mat = ti.is_sh ? (p < 128 ? a.w_shared : a.w_shared2)
                       : (p < 128 ? a.w_routed : a.w_routed2) + (size_t)ti.g * msz;
        e0 = (size_t)(ti.i0 + ti.n0 + colc) * a.H;
    } else {
        const int o = ti.n0 + p < a.H ? ti.n0 + p : ti.n0;    // ragged tile: discarded rows
        mat = ti.is_sh ? a.w_shared
                       : a.w_routed + (size_t)ti.g * ((size_t)a.H * a.I / kSbWeights * kMxBytes);
        e0 = (size_t)o * ti.Iexp + ti.i0;
    }
    auto issue = [&](int kk) {
        const size_t e = e0 + (size_t)kk * kMxK;
        const uint8_t* sb = mat + (e >> 8) * kMxBytes;
        const int c = (int)((e & 255) >> 6);
        const int slot = kk % kMxRing;
#pragma unroll
        for (int j = 0; j < 2; ++j)
            lds_dma16(sb + 16 + 32 * c + 16 * j,
                      __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&lds.rq[slot][j][64 * pw]));
        lds_dma4(sb + 4 * (c >> 1),
                 __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&lds.rs[slot][64 * pw]));
    };
    auto produce = [&](int kk, int st) {
        const int slot = kk % kMxRing;
        const int c = (int)(((e0 + (size_t)kk * kMxK) & 255) >> 6);
        const uint4 lo = lds.rq[slot][0][p], hi = lds.rq[slot][1][p];
        const uint32_t sw = lds.rs[slot][p];                 // scale bytes 4(c>>1) .. +3
        uint4 b0, b1;
        mx_repack(lo, hi, b0, b1);
        *reinterpret_cast<uint4*>(&lds.bq[st][p][mx_bswz(p, 0)]) = b0;
        *reinterpret_cast<uint4*>(&lds.bq[st][p][mx_bswz(p, 1)]) = b1;
        const int sh = 16 * (c & 1);
        lds.bs[st][0][p] = (uint8_t)(sw >> sh);
        lds.bs[st][1][p] = (uint8_t)(sw >> (sh + 8));
    };
    for (int s = 0; s < kMxPD && s < a.nk; ++s) issue(s);
    mx_wait_steps(min(kMxPD - 1, a.nk - 1));
    produce(0, 0);
    if (kMxPD < a.nk) issue(kMxPD);
    __syncthreads();   // stage 0 ready
    for (int kk = 0; kk < a.nk; ++kk) {
        const int nxt = kk + 1;
        if (nxt < a.nk) {
            // step nxt landed; the steps after it already requested stay in flight
            mx_wait_steps(min(kMxPD - 1, a.nk - 1 - nxt));
            produce(nxt, nxt & 1);
            if (nxt + kMxPD < a.nk) issue(nxt + kMxPD);
        }
        __syncthreads();
    }
}

// Consumers: the A stage by direct loads, NT x MB x 2 block-scaled MFMAs per step.
template <int MODE, int MB, int NT>
__device__ __forceinline__ void mx_consume(const MxGemmArgs& a, const MxTileInfo& ti, MxLds& lds,
                                           float16v (&acc)[MB][2]) {
    using S = MxStage<NT, MB>;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    // load i of this thread fills slot q = tid + 256 i; slots past the stage's
    // end (the last load's tail) re-read a valid chunk into the tail bytes
    // load i's source (code chunks from aq, scale rows from as) and its advance per step
    const uint8_t* src[S::kLoads];
    int sstep[S::kLoads];
#pragma unroll
    for (int i = 0; i < S::kLoads; ++i) {
        int q = tid + 256 * i;
        if (q >= S::kSlots) q = 0;
        const bool is_code = q < 4 * NT * S::R;
        int r, t = 0, c = 0;
        if (is_code) {
            t = q / (4 * S::R);
            const int rem = q % (4 * S::R);
            r = rem >> 2;
            c = (rem & 3) ^ mx_swz(r);   // the chunk that this swizzled slot holds
        } else {
            r = q - 4 * NT * S::R;
        }
        const int rv = r < ti.mcount ? r : r % ti.mcount;
        const size_t row = MODE == 0 ? (size_t)(ti.is_sh ? ti.m0 + rv : a.perm[ti.grow0 + rv] / a.k)
                                     : (size_t)(ti.grow0 + rv);
        if (is_code) {
            src[i] = a.aq + (size_t)t * a.a_term + row * a.K + 16 * c;
            sstep[i] = kMxK;
        } else {
            src[i] = a.as + row * (size_t)(a.K / kMxK) * kMxScaleRow;
            sstep[i] = kMxScaleRow;
        }
    }
    auto issue = [&](int kk, int sidx) {
        const uint32_t stage = (uint32_t)(uintptr_t)&lds.a[sidx][0];
#pragma unroll
        for (int i = 0; i < S::kLoads; ++i)
            lds_dma16(src[i] + (size_t)kk * sstep[i],
                      __builtin_amdgcn_readfirstlane(stage + (64 * wave + 256 * i) * 16));
    };
    const int bc0 = MODE == 0 ? 32 * wave : 64 * wave;   // first B row of this wave's two blocks
    const int bstep = MODE == 0 ? 128 : 32;             // rows from block 0 to block 1
    const int nl = lane & 31, hb = lane >> 5;
    // the rows of step kk + L are requested at the start of step kk (L =
    // kMxAStages - 1 steps ahead); near the end the last step is requested
    // again into the free stage, never read, so that every step waits for
    // the same count
    constexpr int L = kMxAStages - 1;
#pragma unroll
    for (int j = 0; j < L; ++j) issue(min(j, a.nk - 1), j);
    wait_vmcnt<(L - 1) * S::kLoads>();   // step 0 landed, the next L - 1 may be in flight
    __syncthreads();   // stage 0 ready
    int sa_idx = 0;    // A stage of step kk (kk mod kMxAStages)
    for (int kk = 0; kk < a.nk; ++kk) {
        const int st = kk & 1;
        // into the stage that step kk - 1 read (every wave passed the barrier after it)
        const int s_prev = sa_idx == 0 ? kMxAStages - 1 : sa_idx - 1;
        issue(min(kk + L, a.nk - 1), s_prev);
        const uint8_t* sa = &lds.a[sa_idx][0];
        sa_idx = sa_idx == kMxAStages - 1 ? 0 : sa_idx + 1;
        // B fragments and scales of the wave's two blocks
        v8i bf[2];
        uint32_t bsc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = bc0 + j * bstep + nl;
            const uint4 v = *reinterpret_cast<const uint4*>(&lds.bq[st][n][mx_bswz(n, hb)]);
            bf[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            bsc[j] = lds.bs[st][hb][n];
        }
        // A scales of each row block: the dword of MX block hb (term t in byte t)
        uint32_t asc[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i)
            asc[i] = *reinterpret_cast<const uint32_t*>(sa + 16 * (4 * NT * S::R + 32 * i + nl) + 8 * hb);
        MxTerms<0, NT, MB>::run(sa, nl, hb, bf, bsc, asc, acc);
        wait_vmcnt<(L - 1) * S::kLoads>();   // step kk + 1's rows landed
        __syncthreads();
    }
    wait_vmcnt<0>();   // the last requests land before the epilogue reuses the LDS
}

// Epilogue, all 8 waves, one 32-row block at a time staged through LDS.
//   MODE 0: h = silu(gate) * up (fp32), then NT-term MX-FP8 codes and scales
//   of each (row, 32-column block), 4 threads per block.
//   MODE 1: the slot's row (the shared expert: its own buffer) times the
//   row's weight, as 16-bit block floating point (store_rows_q16).
template <int MODE, int MB, int NT>
__device__ __forceinline__ void mx_epilogue(const MxGemmArgs& a, const MxTileInfo& ti, MxLds& lds,
                                            const int32_t* row_src, const float* row_w,
                                            const float16v (&acc)[MB][2]) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const bool consumer = wave < kMxConsumers;
    constexpr int kPitch = MODE == 0 ? 128 + 4 : kMxTN + 4;   // LDS row pitch (floats)
    float* t = reinterpret_cast<float*>(&lds);                // [32][kPitch]
    __syncthreads();   // every wave is past its last operand read
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        if (consumer) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (MODE == 0) {
                    t[r * kPitch + 32 * wave + (lane & 31)] = silu_f(acc[i][0][v]) * acc[i][1][v];
                } else {
                    const float sc = row_w[32 * i + r];
                    t[r * kPitch + 64 * wave + (lane & 31)] = acc[i][0][v] * sc;
                    t[r * kPitch + 64 * wave + 32 + (lane & 31)] = acc[i][1][v] * sc;
                }
            }
        }
        __syncthreads();
        if (MODE == 0) {
            // thread: row r, 32-column block bb, quarter qt (8 values)
            const int r = tid >> 4, bb = (tid >> 2) & 3, qt = tid & 3;
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = t[r * kPitch + 32 * bb + 8 * qt + j];
            uint32_t codes[NT][2], scales;
            mx_fp8_terms<NT>(v, codes, scales);
            const int m = 32 * i + r, n = ti.n0 + 32 * bb;
            if (m < ti.mcount && n < ti.Iloc) {
                const size_t grow = (size_t)(ti.grow0 + m);
                mx_store_block<NT>(a.hq + grow * ti.Iloc + n, a.h_term,
                                   a.hs + (grow * (ti.Iloc / kMxK) + n / kMxK) * kMxScaleRow,
                                   (n / 32) & 1, qt, codes, scales);
            }
        } else {
            store_rows_q16<kMxThreads>(t, kPitch, ti.is_sh ? a.ysh : a.y,
                                       ti.is_sh ? a.yshsc : a.ysc, row_src, 32 * i, ti.mcount,
                                       ti.n0, a.H);
        }
        __syncthreads();   // the staging buffer is rewritten by the next block
    }
}

template <int MODE, int MB, int NT>
__device__ __forceinline__ void mx_tile(const MxGemmArgs& a, const MxTileInfo& ti, MxLds& lds,
                                        const int32_t* row_src, const float* row_w) {
    float16v acc[MB][2];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        acc[i][0] = float16v{};
        acc[i][1] = float16v{};
    }
    if (threadIdx.x >> 6 >= kMxConsumers)
        mx_produce<MODE>(a, ti, lds);
    else
        mx_consume<MODE, MB, NT>(a, ti, lds, acc);
    mx_epilogue<MODE, MB, NT>(a, ti, lds, row_src, row_w, acc);
}

// tile_off, tile_rec, the packed counts (experts | column tiles << 16) and the
// number of records come first as preloaded scalar arguments, as in the fp16
// grouped GEMM.
template <int MODE, int NT>
__global__ void __launch_bounds__(kMxThreads)
gemm_mx_kernel(const int32_t* __restrict__ tile_off, const int4* __restrict__ tile_rec,
               uint32_t e_nt, int max_tiles, MxGemmArgs a) {
    __shared__ MxLds lds;
    int32_t* row_src = lds.row_src;
    float* row_w = lds.row_w;

    // block -> (row tile, column tile) as in the fp16 grouped GEMM: the column
    // tiles of one row tile run on one XCD; records in the order taken
    const int b = blockIdx.x;
    const int nt = hi16(e_nt);
    const int tile_raw = (b / (8 * nt)) * 8 + (b & 7);
    const int ntile = (b >> 3) % nt;
    const int ntiles = tile_off[lo16(e_nt) + 1];
    const int4 rec = tile_rec[min(tile_raw, max_tiles - 1)];
    // both loads in flight together (the record in registers before the exit test)
    asm volatile("" ::"s"(rec.x), "s"(rec.y), "s"(rec.z), "s"(rec.w));
    if (tile_raw >= ntiles) return;
    MxTileInfo ti;
    ti.g = rec.x;
    ti.is_sh = ti.g == a.E;
    ti.grow0 = rec.y;
    ti.mcount = rec.z;
    ti.m0 = rec.w;
    ti.Iexp = ti.is_sh ? a.Is : a.I;
    ti.Iloc = a.iloc;
    ti.i0 = a.i0;
    ti.n0 = ntile * (MODE == 0 ? kMxTN / 2 : kMxTN);
    const int tid = threadIdx.x;
    if (MODE == 1 && tid < kTileM) {
        int src = -1;
        float rw = 0.f;
        if (tid < ti.mcount) {
            src = ti.is_sh ? (ti.m0 + tid) : a.perm[ti.grow0 + tid];
            rw = ti.is_sh ? a.sw : a.route_w[src];
        }
        row_src[tid] = src;
        row_w[tid] = rw;
    }
    switch ((ti.mcount + 31) >> 5) {
        case 1: mx_tile<MODE, 1, NT>(a, ti, lds, row_src, row_w); break;
        case 2: mx_tile<MODE, 2, NT>(a, ti, lds, row_src, row_w); break;
        case 3: mx_tile<MODE, 3, NT>(a, ti, lds, row_src, row_w); break;
        case 4: mx_tile<MODE, 4, NT>(a, ti, lds, row_src, row_w); break;
        default: mx_tile<MODE, 5, NT>(a, ti, lds, row_src, row_w); break;
    }
}

// Tokens to MX-FP8 terms, bucketing, the two block-scaled grouped GEMMs and
// the slot-order combine (gemm.hip's).  The tokens' fp16 copy is not needed.
hipError_t launch_mfma_mx(const moe_layer_desc& d, const float* x, int T, const int32_t* idx,
                          const float* w, int i0, int iloc, float* out, char* ws,
                          const WsLayout& L, const Ctx& c) {
    const int H = d.hidden, E = d.n_experts, k = d.top_k;
    const bool shared = d.shared_inter > 0;
    uint8_t* xq = reinterpret_cast<uint8_t*>(ws + L.mx_xq);
    uint8_t* xs = reinterpret_cast<uint8_t*>(ws + L.mx_xs);
    uint8_t* hq = reinterpret_cast<uint8_t*>(ws + L.mx_hq);
    uint8_t* hs = reinterpret_cast<uint8_t*>(ws + L.mx_hs);
    int32_t* bhist = reinterpret_cast<int32_t*>(ws + L.bhist);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* tile_off = reinterpret_cast<int32_t*>(ws + L.tile_off);
    int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
    int4* tile_rec = reinterpret_cast<int4*>(ws + L.tile_rec);
    int16_t* y = reinterpret_cast<int16_t*>(ws + L.y);
    int16_t* ysh = reinterpret_cast<int16_t*>(ws + L.ysh);
    uint8_t* ysc = reinterpret_cast<uint8_t*>(ws + L.ysc);
    uint8_t* yshsc = reinterpret_cast<uint8_t*>(ws + L.yshsc);

    const size_t nq = (size_t)T * H / 8;
    launch_k(c, MOE_K_X_MX, mx_split_kernel<kMxTerms>, dim3((unsigned)((nq + 255) / 256)),
             dim3(256), 0, x, T, H, xq, xs);
    hipError_t err =
        launch_bucket(idx, T, k, E, shared, counts, offsets, tile_off, tile_rec, perm, bhist, c);
    if (err != hipSuccess) return err;
    const int max_tiles = max_row_tiles(T, k, E, shared);
    const int max_tiles8 = (max_tiles + 7) / 8 * 8;
    const size_t hrows = (size_t)T * k + T;

    MxGemmArgs a = {};
    a.perm = perm;
    a.tile_off = tile_off;
    a.tile_rec = tile_rec;
    a.T = T;
    a.H = H;
    a.E = E;
    a.k = k;
    a.I = d.inter;
    a.Is = d.shared_inter;
    a.i0 = i0;
    a.iloc = iloc;
    a.route_w = w;
    a.sw = d.shared_weight;
    a.hq = hq;
    a.hs = hs;
    a.h_term = hrows * iloc;

    MxGemmArgs g1 = a;
    g1.aq = xq;
    g1.as = xs;
    g1.a_term = (size_t)T * H;
    g1.K = H;
    g1.w_routed = d.gate_q;
    g1.w_routed2 = d.up_q;
    g1.w_shared = d.sh_gate_q;
    g1.w_shared2 = d.sh_up_q;
    g1.n_ntiles = (iloc + kMxTN / 2 - 1) / (kMxTN / 2);
    g1.nk = H / kMxK;
    if (E > 0xffff || g1.n_ntiles > 0xffff) return hipErrorInvalidValue;   // packed in 16 bits
    launch_k(c, MOE_K_GEMM_GATEUP, gemm_mx_kernel<0, kMxTerms>, dim3(max_tiles8 * g1.n_ntiles),
             dim3(kMxThreads), 0, (const int32_t*)tile_off, (const int4*)tile_rec,
             pack16(E, g1.n_ntiles), max_tiles, g1);

    MxGemmArgs g2 = a;
    g2.aq = hq;
    g2.as = hs;
    g2.a_term = hrows * iloc;
    g2.K = iloc;
    g2.w_routed = d.down_q;
    g2.w_shared = d.sh_down_q;
    g2.n_ntiles = (H + kMxTN - 1) / kMxTN;
    g2.nk = iloc / kMxK;
    g2.y = y;
    g2.ysh = ysh;
    g2.ysc = ysc;
    g2.yshsc = yshsc;
    if (g2.n_ntiles > 0xffff) return hipErrorInvalidValue;
    launch_k(c, MOE_K_GEMM_DOWN, gemm_mx_kernel<1, kMxTerms>, dim3(max_tiles8 * g2.n_ntiles),
             dim3(kMxThreads), 0, (const int32_t*)tile_off, (const int4*)tile_rec,
             pack16(E, g2.n_ntiles), max_tiles, g2);
    return launch_combine(y, ysh, ysc, yshsc, idx, T, H, E, k, shared, out, c);
}

}  // namespace moe
