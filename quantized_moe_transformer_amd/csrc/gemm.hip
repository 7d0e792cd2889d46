// gemm.hip -- prefill path: grouped GEMM over experts on the MFMA cores.
//
// With many token rows each packed weight is reused by every row routed to
// its expert, and the expert FFN becomes a dense contraction bound by matrix
// throughput (page "Distributed CPU: Zip Fusion Beyond Tensor Parallelism",
// sections "Decode vs Prefill: Same Weights, Different Bottlenecks" and
// "Prefill First, Then One Matrix-Work Scheduler").
//
// Operands are fp16 with fp32 accumulation (v_mfma_f32_32x32x16_f16).  fp16
// rather than bf16: the synthetic Qwen3.5-shaped layer has strongly non-zero-
// mean weights and heavy-tailed outputs, and bf16 operand rounding alone
// exceeds a 1e-2 max-error/RMS bound while fp16 stays near 3e-3; gfx950 runs
// both at the same rate.
//
// One kernel template serves both projections.  A workgroup owns one tile:
// up to 160 rows of one expert's group (a whole routed expert at T = 4096, so
// its weights are dequantised once per column tile) times 256 weight rows, and
// walks K in steps of 64 (one pair of K-quant sub-blocks).  Its 8 waves are
//   4 consumer waves: MFMA only, from one LDS stage; wave w owns two 32-wide
//     column blocks times every 32-row block the tile has (up to 5), so each
//     fragment read from LDS feeds several MFMAs;
//   4 producer waves: dequantise the next step's packed weights into the
//     other LDS stage, with the weight loads issued ahead into a register
//     ring (whole superblocks per row where the layout allows);
//   the consumer waves also gather the next step's token rows (fp16) into the
//     other stage, so each group of waves waits only for its own loads;
// so dequantisation (VALU) and matrix work (MFMA) run side by side.
//
//   gateup (MODE 0): A = token rows of x16 gathered through the expert-sorted
//     slot list, B = 128 gate rows + the matching 128 up rows (4-bit); each
//     consumer wave holds a gate block and the matching up block, so the
//     epilogue writes h = silu(g) * u (fp16, scaled by 2^-4) straight from
//     registers, in sorted row order.
//   down (MODE 1): A = h rows (contiguous per expert), B = 256 down rows
//     (5-bit); the epilogue scales by the routing weight (and 2^4) and writes
//     the slot's row of the per-slot buffer (the shared expert: its own
//     buffer, times its weight).
//   combine: out[t] = sum over slots in selected-slot order, then the shared
//     expert (page "CKE Zip: From Splitting Tokens To Splitting Qwen3.5
//     Weights", section "A Separate Decode Result Shows Why Axis Choice
//     Matters").
#include "moe_internal.h"

namespace moe {

constexpr int kBK = 64;                 // K per step (one pair of sub-blocks)
constexpr int kLdsRow = kBK + 8;        // halves per LDS row (8 halves of padding)
constexpr int kTM = kTileM;             // rows per tile (up to 5 blocks of 32)
constexpr int kTN = 256;                // weight rows per tile
// weight-load prefetch distance (steps): 3 for the 4-bit gate/up stream, 2
// for the 5-bit down stream (its pieces carry high bits too: more registers)
template <int MODE> struct PrefetchDistance { static constexpr int v = MODE == 0 ? 3 : 2; };
constexpr int kConsumers = 4;           // consumer waves (two 32-column blocks each)
constexpr int kProducers = 4;           // producer waves
constexpr int kGemmThreads = 64 * (kConsumers + kProducers);
constexpr int kBTasks = kTN * 2 / (64 * kProducers);   // 16-byte code pieces per producer thread

// Dequantise one 16-byte code piece (32 weights: sub-block 2c low nibbles and
// sub-block 2c+1 high nibbles) to fp16 and store it into an LDS row at k
// offsets 16*hh + [0,16) and 32 + 16*hh + [0,16).
//
// The fp16 bit pattern 0x6400 | q is the number 1024 + q (q < 1024), so one
// and-or turns two code bytes of a word into two fp16 numbers, and
//   w = d*sc*q - dmin*m = (1024 + q) * (d*sc) - (1024*d*sc + dmin*m)
// is one mixed-precision fma per weight (fp16 operand, fp32 arithmetic,
// fp16 result).  The constant 1024*d*sc + dmin*m is rounded to fp32 once
// (relative 2^-24 of a value <= 1024 |d*sc| + |dmin*m|): far below the fp16
// rounding of w itself.
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// (x & m) | o in one v_and_or_b32 (the compiler splits it into an and and an
// or when the constants are literals).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(o));
    return r;
}

// bytes 0 and 2 of `bytes` (codes, masked by m) as the fp16 numbers 1024 + code
__device__ __forceinline__ half2v code_pair(uint32_t bytes, uint32_t m) {
    return __builtin_bit_cast(half2v, and_or(bytes, m, 0x64006400u));
}

__device__ __forceinline__ _Float16 mix_fma(_Float16 q1024, float ds, float c) {
    return (_Float16)__builtin_fmaf((float)q1024, ds, c);
}

template <bool HIGH>
__device__ __forceinline__ void dequant_piece_to_lds(const SbHead& hd, const uint4& qs,
                                                     const uint4& qh, int c, int hh,
                                                     _Float16* row) {
    float sca, ma, scb, mb;
    sub_scale_min(hd, 2 * c, sca, ma);
    sub_scale_min(hd, 2 * c + 1, scb, mb);
    const float dsa = hd.d * sca, dsb = hd.d * scb;
    const float ca = -__builtin_fmaf(1024.0f, dsa, hd.dmin * ma);
    const float cb = -__builtin_fmaf(1024.0f, dsb, hd.dmin * mb);
    const uint32_t qw[4] = {qs.x, qs.y, qs.z, qs.w};
    const uint32_t hw[4] = {qh.x, qh.y, qh.z, qh.w};
    half8 lo[2], hi[2];
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
        half2v la, lb, ha, hb;   // codes (0, 2) and (1, 3) of the low and high nibbles
        if (HIGH) {
            const uint32_t l5 = (qw[wi] & 0x0f0f0f0fu) | (((hw[wi] >> (2 * c)) & 0x01010101u) << 4);
            const uint32_t h5 =
                ((qw[wi] >> 4) & 0x0f0f0f0fu) | (((hw[wi] >> (2 * c + 1)) & 0x01010101u) << 4);
            la = code_pair(l5, 0x00ff00ffu);
            lb = code_pair(l5 >> 8, 0x00ff00ffu);
            ha = code_pair(h5, 0x00ff00ffu);
            hb = code_pair(h5 >> 8, 0x00ff00ffu);
        } else {
            la = code_pair(qw[wi], 0x000f000fu);
            lb = code_pair(qw[wi] >> 8, 0x000f000fu);
            ha = code_pair(qw[wi] >> 4, 0x000f000fu);
            hb = code_pair(qw[wi] >> 12, 0x000f000fu);
        }
        half8& L = lo[wi >> 1];
        half8& Hh = hi[wi >> 1];
        const int o = 4 * (wi & 1);
        L[o + 0] = mix_fma(la[0], dsa, ca);
        L[o + 1] = mix_fma(lb[0], dsa, ca);
        L[o + 2] = mix_fma(la[1], dsa, ca);
        L[o + 3] = mix_fma(lb[1], dsa, ca);
        Hh[o + 0] = mix_fma(ha[0], dsb, cb);
        Hh[o + 1] = mix_fma(hb[0], dsb, cb);
        Hh[o + 2] = mix_fma(ha[1], dsb, cb);
        Hh[o + 3] = mix_fma(hb[1], dsb, cb);
    }
    *reinterpret_cast<half8*>(row + 16 * hh) = lo[0];
    *reinterpret_cast<half8*>(row + 16 * hh + 8) = lo[1];
    *reinterpret_cast<half8*>(row + 32 + 16 * hh) = hi[0];
    *reinterpret_cast<half8*>(row + 32 + 16 * hh + 8) = hi[1];
}

struct GemmArgs {
    const _Float16* a_src;          // MODE 0: x16 [T][H]; MODE 1: h16 [T*k + T][Iloc]
    int a_stride;                   // halves per A row
    const int32_t* perm;            // expert-sorted slot ids
    const int32_t* offsets;         // [E+2]: group row starts (group E = shared expert)
    const int32_t* tile_off;        // [E+2]: group tile starts
    const int4* tile_rec;           // per row tile: group, first sorted row, rows, row offset
    int T, H, E, k, I, Is, shard, nshards;
    const uint8_t *w_routed, *w_routed2, *w_shared, *w_shared2;   // MODE 0: gate, up
    const float* route_w;           // [T*k] routing weights
    float sw;
    int n_ntiles;                   // weight-row tiles per group
    int nk;                         // K steps
    int sb_rows;                    // MODE 1: every row's K range is whole superblocks
    _Float16* h_out;                // MODE 0
    int h_stride;
    float* y;                       // MODE 1: [T*k][H]
    float* ysh;                     // MODE 1: [T][H]
};

// Packed weights of one producer task (weight row, 16-byte half) for one step.
struct BRegs {
    uint4 head, qs, qh;
};

// A stages hold kTM rows of kBK halves with no padding; the 16-byte chunk c
// of row r sits at chunk position c ^ (r & 7), so the 32 rows that one MFMA
// fragment read touches spread over all banks.
constexpr int kAStages = 3;
__device__ __forceinline__ int a_chunk(int r, int c) { return r * (kBK / 8) + (c ^ (r & 7)); }

struct __align__(16) GemmLds {
    _Float16 a[kAStages][kTM * kBK];
    _Float16 b[2][kTN][kLdsRow];
};


// Everything a workgroup knows about its tile.
struct TileInfo {
    int g, m0, mcount, grow0, Iexp, Iloc, i0, n0;
    bool is_sh;
};

// The tile's K loop and epilogue for exactly MB 32-row blocks, in three parts:
// producer waves, consumer waves, and an epilogue that all 8 waves run.
// Producers: (straight-line
// code: the fragment reads of a 16-wide K slice are issued before its MFMAs).
template <int MODE, int MB>
__device__ __forceinline__ void gemm_produce(const GemmArgs& a, const TileInfo& ti, GemmLds& lds,
                                          const int32_t* row_src, const float* row_w) {
    constexpr int kPD = PrefetchDistance<MODE>::v;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g = ti.g, m0 = ti.m0, mcount = ti.mcount, grow0 = ti.grow0;
    const int Iexp = ti.Iexp, Iloc = ti.Iloc, i0 = ti.i0, n0 = ti.n0;
    const bool is_sh = ti.is_sh;
    (void)m0;

    // ------------------------------- producers -------------------------------
    const int pt = tid - 64 * kConsumers;
    if constexpr (MODE == 0) {
        // Producer thread pt owns weight row pt of the tile (gate rows
        // 0-127, the matching up rows 128-255) and loads the row's whole
        // 144-byte superblock -- nine 16-byte loads, contiguous -- once per
        // four steps into a two-slot register ring, one superblock ahead;
        // each step dequantises its 64 weights of the current one.
        const int col = pt & (kTN / 2 - 1);
        const int colc = n0 + col < Iloc ? col : 0;   // ragged tile: discarded columns
        const size_t mat = (size_t)a.I * a.H / kSbWeights * kQ4Bytes;
        const uint8_t* m = is_sh ? (pt < kTN / 2 ? a.w_shared : a.w_shared2)
                                 : (pt < kTN / 2 ? a.w_routed : a.w_routed2) + (size_t)g * mat;
        const int nsb = a.H / kSbWeights;
        const uint8_t* rowp = m + (size_t)(i0 + n0 + colc) * nsb * kQ4Bytes;
        uint4 sbr[2][kQ4Bytes / 16];
        auto load_sb = [&](int p, uint4* r) {
            const uint4* src =
                reinterpret_cast<const uint4*>(rowp + (size_t)min(p, nsb - 1) * kQ4Bytes);
#pragma unroll
            for (int i = 0; i < kQ4Bytes / 16; ++i) r[i] = src[i];
        };
        auto deq_step = [&](const uint4* r, int c, int stage) {
            SbHead hd;
            hd.d = f16_bits_to_f32(r[0].x & 0xffffu);
            hd.dmin = f16_bits_to_f32(r[0].x >> 16);
            hd.s0 = r[0].y;
            hd.s1 = r[0].z;
            hd.s2 = r[0].w;
            _Float16* dst = &lds.b[stage][pt][0];
            dequant_piece_to_lds<false>(hd, r[1 + 2 * c], r[1 + 2 * c], c, 0, dst);
            dequant_piece_to_lds<false>(hd, r[2 + 2 * c], r[2 + 2 * c], c, 1, dst);
        };
        const int last = a.nk - 1;
        load_sb(0, sbr[0]);
        load_sb(1, sbr[1]);
        deq_step(sbr[0], 0, 0);
        __syncthreads();   // stage 0 ready
        // steps 4*p0 .. 4*p0+7 use superblocks p0 (slot 0) and p0+1 (slot 1)
        for (int p0 = 0; p0 < nsb; p0 += 2) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int kk = 4 * p0 + u;
                if (kk > last) break;
                const int nxt = kk + 1;
                if (nxt <= last) {
                    const int un = u + 1;   // step nxt: slot (un >> 2) & 1, sub-block pair un & 3
                    deq_step(sbr[(un >> 2) & 1], un & 3, nxt & 1);
                    if ((un & 3) == 3) load_sb(p0 + (un >> 2) + 2, sbr[(un >> 2) & 1]);
                }
                __syncthreads();
            }
        }
        return;
    }
    if (MODE == 1 && a.sb_rows) {
        // The down rows' K ranges are whole 5-bit superblocks: producer
        // thread pt owns output row n0 + pt and loads each 176-byte
        // superblock of it -- eleven 16-byte loads, contiguous -- once per
        // four steps, one superblock ahead, as the gate/up path does.
        const int o = n0 + pt < a.H ? n0 + pt : n0;   // ragged tile: discarded rows
        const uint8_t* m = is_sh ? a.w_shared
                                 : a.w_routed + (size_t)g * ((size_t)a.H * a.I / kSbWeights * kQ5Bytes);
        const int nsb = Iloc / kSbWeights;
        const uint8_t* rowp = m + (((size_t)o * Iexp + i0) >> 8) * kQ5Bytes;
        uint4 sbr[2][kQ5Bytes / 16];
        auto load_sb = [&](int p, uint4* r) {
            const uint4* src =
                reinterpret_cast<const uint4*>(rowp + (size_t)min(p, nsb - 1) * kQ5Bytes);
#pragma unroll
            for (int i = 0; i < kQ5Bytes / 16; ++i) r[i] = src[i];
        };
        auto deq_step = [&](const uint4* r, int c, int stage) {
            SbHead hd;
            hd.d = f16_bits_to_f32(r[0].x & 0xffffu);
            hd.dmin = f16_bits_to_f32(r[0].x >> 16);
            hd.s0 = r[0].y;
            hd.s1 = r[0].z;
            hd.s2 = r[0].w;
            _Float16* dst = &lds.b[stage][pt][0];
            dequant_piece_to_lds<true>(hd, r[3 + 2 * c], r[1], c, 0, dst);
            dequant_piece_to_lds<true>(hd, r[4 + 2 * c], r[2], c, 1, dst);
        };
        const int last = a.nk - 1;
        load_sb(0, sbr[0]);
        load_sb(1, sbr[1]);
        deq_step(sbr[0], 0, 0);
        __syncthreads();   // stage 0 ready
        for (int p0 = 0; p0 < nsb; p0 += 2) {
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int kk = 4 * p0 + u;
                if (kk > last) break;
                const int nxt = kk + 1;
                if (nxt <= last) {
                    const int un = u + 1;
                    deq_step(sbr[(un >> 2) & 1], un & 3, nxt & 1);
                    if ((un & 3) == 3) load_sb(p0 + (un >> 2) + 2, sbr[(un >> 2) & 1]);
                }
                __syncthreads();
            }
        }
        return;
    }
    const uint8_t* wsrc[kBTasks];   // MODE 0: the row's superblocks; MODE 1: matrix base
    size_t eoff[kBTasks];           // MODE 1: element offset of the row's range
    int bhh[kBTasks], brr[kBTasks];
    // weight rows past the matrix end (a ragged last column tile) read the
    // tile's first row instead: their LDS columns only feed outputs that
    // the epilogue discards
#pragma unroll
    for (int q = 0; q < kBTasks; ++q) {
        const int task = pt + 64 * kProducers * q;
        const int r = task >> 1;
        bhh[q] = task & 1;
        brr[q] = r;
        eoff[q] = 0;
        if (MODE == 0) {
            const int col = n0 + (r & (kTN / 2 - 1)) < Iloc ? (r & (kTN / 2 - 1)) : 0;
            const size_t mat = (size_t)a.I * a.H / kSbWeights * kQ4Bytes;
            const uint8_t* m = is_sh ? (r < kTN / 2 ? a.w_shared : a.w_shared2)
                                     : (r < kTN / 2 ? a.w_routed : a.w_routed2) + (size_t)g * mat;
            wsrc[q] = m + (size_t)(i0 + n0 + col) * (a.H / kSbWeights) * kQ4Bytes;
        } else {
            const int o = n0 + r < a.H ? n0 + r : n0;
            wsrc[q] = is_sh ? a.w_shared
                            : a.w_routed + (size_t)g * ((size_t)a.H * a.I / kSbWeights * kQ5Bytes);
            eoff[q] = (size_t)o * Iexp + i0;
        }
    }
    auto load_b = [&](int kk, BRegs* rg) {
#pragma unroll
        for (int q = 0; q < kBTasks; ++q) {
            if (MODE == 0) {
                const uint8_t* sb = wsrc[q] + (kk >> 2) * kQ4Bytes;
                rg[q].head = *reinterpret_cast<const uint4*>(sb);
                rg[q].qs = *reinterpret_cast<const uint4*>(sb + 16 + 32 * (kk & 3) + 16 * bhh[q]);
            } else {
                const size_t base = eoff[q] + (size_t)kk * kBK;
                const int c = (int)((base & 255) >> 6);
                const uint8_t* sb = wsrc[q] + (base >> 8) * kQ5Bytes;
                rg[q].head = *reinterpret_cast<const uint4*>(sb);
                rg[q].qh = *reinterpret_cast<const uint4*>(sb + 16 + 16 * bhh[q]);
                rg[q].qs = *reinterpret_cast<const uint4*>(sb + 48 + 32 * c + 16 * bhh[q]);
            }
        }
    };
    auto store_b = [&](int kk, const BRegs* rg, int stage) {
#pragma unroll
        for (int q = 0; q < kBTasks; ++q) {
            SbHead hd;
            hd.d = f16_bits_to_f32(rg[q].head.x & 0xffffu);
            hd.dmin = f16_bits_to_f32(rg[q].head.x >> 16);
            hd.s0 = rg[q].head.y;
            hd.s1 = rg[q].head.z;
            hd.s2 = rg[q].head.w;
            const int c = MODE == 0 ? (kk & 3)
                                    : (int)(((eoff[q] + (size_t)kk * kBK) & 255) >> 6);
            dequant_piece_to_lds<MODE == 1>(hd, rg[q].qs, rg[q].qh, c, bhh[q],
                                            &lds.b[stage][brr[q]][0]);
        }
    };
    BRegs ring[kPD][kBTasks];
#pragma unroll
    for (int s = 0; s < kPD; ++s)
        if (s < a.nk) load_b(s, ring[s]);
    store_b(0, ring[0], 0);
    if (kPD < a.nk) load_b(kPD, ring[0]);
    __syncthreads();   // stage 0 ready
    for (int kk0 = 0; kk0 < a.nk; kk0 += kPD) {
#pragma unroll
        for (int u = 0; u < kPD; ++u) {
            const int kk = kk0 + u;
            if (kk >= a.nk) break;
            // while the consumers work on step kk: step kk+1 into the other stage
            const int nxt = kk + 1;
            if (nxt < a.nk) {
                store_b(nxt, ring[(u + 1) % kPD], nxt & 1);
                if (nxt + kPD < a.nk) load_b(nxt + kPD, ring[(u + 1) % kPD]);
            }
            __syncthreads();
        }
    }
    return;
}

// Consumers: token rows into LDS, MFMAs into acc.
template <int MODE, int MB>
__device__ __forceinline__ void gemm_consume(const GemmArgs& a, const TileInfo& ti, GemmLds& lds,
                                          const int32_t* row_src, const float* row_w,
                                             float16v (&acc)[MB][2]) {
    constexpr int kPD = PrefetchDistance<MODE>::v;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g = ti.g, m0 = ti.m0, mcount = ti.mcount, grow0 = ti.grow0;
    const int Iexp = ti.Iexp, Iloc = ti.Iloc, i0 = ti.i0, n0 = ti.n0;
    const bool is_sh = ti.is_sh;
    (void)m0;

    // ------------------------------- consumers -------------------------------
    // The consumer waves move the token rows (A) into LDS themselves with direct
    // global-to-LDS loads (no registers), two steps ahead into a three-stage ring,
    // so their waits cover only these loads and the producers' waits only the
    // weight loads.  Thread tid's load i fills chunk slot q = tid + 256 i: row
    // q >> 3, chunk position q & 7, i.e. logical chunk (q & 7) ^ (row & 7).  Rows
    // past the tile's end re-read one of its rows (row r mod mcount): their
    // results are discarded, and every load is unconditional so each step
    // issues exactly MB of them per wave.
    size_t asrc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int q = tid + 256 * i;
        const int r = q >> 3, c = (q & 7) ^ (r & 7);
        const int rv = r < mcount ? r : r % mcount;
        // MODE 0: the row's token, read here rather than from row_src so that
        // no barrier stands between the tile record and the first loads
        const size_t row = MODE == 0 ? (size_t)(is_sh ? ti.m0 + rv : a.perm[grow0 + rv] / a.k)
                                     : (size_t)(grow0 + rv);
        asrc[i] = row * a.a_stride + c * 8;
    }
    auto issue_a = [&](int kk) {
        const uint32_t stage = (uint32_t)(uintptr_t)&lds.a[kk % kAStages][0];
#pragma unroll
        for (int i = 0; i < MB; ++i)
            lds_dma16(a.a_src + asrc[i] + (size_t)kk * kBK,
                      __builtin_amdgcn_readfirstlane(stage + (64 * wave + 256 * i) * 16));
    };

    // this wave's two 32-row blocks of B: gate block w and up block w (MODE 0),
    // or output blocks 2w and 2w+1 (MODE 1)
    const int bc0 = MODE == 0 ? 32 * wave : 64 * wave;
    const int bc1 = MODE == 0 ? kTN / 2 + 32 * wave : 64 * wave + 32;
    issue_a(0);
    if (a.nk > 1) {
        issue_a(1);
        wait_vmcnt<MB>();         // step 0's rows landed
    } else {
        wait_vmcnt<0>();
    }
    __syncthreads();              // stage 0 ready
    for (int kk = 0; kk < a.nk; ++kk) {
        const int st = kk & 1;
        const _Float16* sa = &lds.a[kk % kAStages][0];
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kof = ks * 16 + 8 * (lane >> 5);
            const half8 b0 = *reinterpret_cast<const half8*>(&lds.b[st][bc0 + (lane & 31)][kof]);
            const half8 b1 = *reinterpret_cast<const half8*>(&lds.b[st][bc1 + (lane & 31)][kof]);
            half8 av[MB];
#pragma unroll
            for (int i = 0; i < MB; ++i)
                av[i] = *reinterpret_cast<const half8*>(
                    sa + 8 * a_chunk(32 * i + (lane & 31), 2 * ks + (lane >> 5)));
#pragma unroll
            for (int i = 0; i < MB; ++i) {
                acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], b0, acc[i][0], 0, 0, 0);
                acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], b1, acc[i][1], 0, 0, 0);
            }
        }
        // the rows of step kk + 2 go to the stage that step kk - 1 read (all
        // waves left it at the last barrier); step kk + 1's must have landed
        // before the barrier
        if (kk + 2 < a.nk) {
            issue_a(kk + 2);
            wait_vmcnt<MB>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();
    }

}

// Epilogue, all 8 waves: each 32-row block of the tile is staged through LDS
// (the operand stages are no longer read) and written with 16-byte stores of
// whole row segments.
//   MODE 0: h = silu(gate) * up * 2^-4 as fp16, rows in sorted order.
//   MODE 1: the slot's row (the shared expert: its own buffer) times the
//   row's weight * 2^4, fp32.
template <int MODE, int MB>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, const TileInfo& ti, GemmLds& lds,
                                          const int32_t* row_src, const float* row_w,
                                              const float16v (&acc)[MB][2]) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const bool consumer = wave < kConsumers;
    constexpr int kPitch = MODE == 0 ? kTN / 2 + 8 : kTN + 4;   // LDS row pitch (elements)
    __syncthreads();   // every wave is past its last operand read
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        if (MODE == 0) {
            _Float16* t = reinterpret_cast<_Float16*>(&lds);   // [32][kPitch]
            if (consumer) {
                const int n = 32 * wave + (lane & 31);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    t[r * kPitch + n] = (_Float16)(silu_f(acc[i][0][v]) * acc[i][1][v] * kHScale);
                }
            }
            __syncthreads();
            // 32 rows x 128 halves = 512 chunks of 8 halves, one per thread
            const int r = tid >> 4, c8 = tid & 15;
            const int m = 32 * i + r, n = ti.n0 + 8 * c8;
            if (m < ti.mcount && n < ti.Iloc)
                *reinterpret_cast<uint4*>(a.h_out + (size_t)(ti.grow0 + m) * a.h_stride + n) =
                    *reinterpret_cast<const uint4*>(t + r * kPitch + 8 * c8);
        } else {
            float* t = reinterpret_cast<float*>(&lds);   // [32][kPitch]
            if (consumer) {
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int r = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                    const float sc = row_w[32 * i + r];
                    t[r * kPitch + 64 * wave + (lane & 31)] = acc[i][0][v] * sc;
                    t[r * kPitch + 64 * wave + 32 + (lane & 31)] = acc[i][1][v] * sc;
                }
            }
            __syncthreads();
            // 32 rows x 256 floats = 2048 chunks of 4 floats, four per thread
            float* dst = ti.is_sh ? a.ysh : a.y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int q = tid + 512 * j;
                const int r = q >> 6, c4 = q & 63;
                const int m = 32 * i + r, o = ti.n0 + 4 * c4;
                if (m < ti.mcount && o < a.H)
                    *reinterpret_cast<float4*>(dst + (size_t)row_src[m] * a.H + o) =
                        *reinterpret_cast<const float4*>(t + r * kPitch + 4 * c4);
            }
        }
        __syncthreads();   // the staging buffer is rewritten by the next block
    }
}

template <int MODE, int MB>
__device__ __forceinline__ void gemm_tile(const GemmArgs& a, const TileInfo& ti, GemmLds& lds,
                                          const int32_t* row_src, const float* row_w) {
    float16v acc[MB][2];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        acc[i][0] = float16v{};
        acc[i][1] = float16v{};
    }
    if (threadIdx.x >> 6 >= kConsumers)
        gemm_produce<MODE, MB>(a, ti, lds, row_src, row_w);
    else
        gemm_consume<MODE, MB>(a, ti, lds, row_src, row_w, acc);
    gemm_epilogue<MODE, MB>(a, ti, lds, row_src, row_w, acc);
}

template <int MODE>
__global__ void __launch_bounds__(kGemmThreads)
gemm_grouped_kernel(GemmArgs a) {
    __shared__ GemmLds lds;
    __shared__ int32_t row_src[kTM];     // MODE 0: token of each row; MODE 1: slot id
    __shared__ float row_w[kTM];         // MODE 1: routing weight * 2^4 of each row

    const int ngroups = a.E + 1;
    const int ntiles = a.tile_off[ngroups];
    // block -> (row tile, column tile): the column tiles of one row tile run
    // on one XCD (blocks 8 apart), so its gathered rows are reused in L2; row
    // tiles are taken in reverse (the shared expert's, the largest, first)
    const int b = blockIdx.x;
    const int nt = a.n_ntiles;
    const int tile_raw = (b / (8 * nt)) * 8 + (b & 7);
    const int ntile = (b >> 3) % nt;
    if (tile_raw >= ntiles) return;
    const int tile = ntiles - 1 - tile_raw;
    const int4 rec = a.tile_rec[tile];   // written by the bucketing scan
    TileInfo ti;
    ti.g = rec.x;
    ti.is_sh = ti.g == a.E;
    ti.grow0 = rec.y;                      // first row of the tile in sorted order
    ti.mcount = rec.z;
    ti.m0 = rec.w;
    ti.Iexp = ti.is_sh ? a.Is : a.I;
    ti.Iloc = ti.Iexp / a.nshards;
    ti.i0 = a.shard * ti.Iloc;
    ti.n0 = ntile * (MODE == 0 ? kTN / 2 : kTN);
    const int tid = threadIdx.x;
    if (tid < kTM) {
        int src = -1;
        float rw = 0.f;
        if (tid < ti.mcount) {
            if (MODE == 0) {
                src = ti.is_sh ? (ti.m0 + tid) : a.perm[ti.grow0 + tid] / a.k;
            } else {
                src = ti.is_sh ? (ti.m0 + tid) : a.perm[ti.grow0 + tid];
                rw = (ti.is_sh ? a.sw : a.route_w[src]) * kHUnscale;
            }
        }
        row_src[tid] = src;
        row_w[tid] = rw;
    }
    // row_src and row_w are read only in the epilogue, after the K loop's
    // barriers; the weight and token-row loads start without waiting for them
    switch ((ti.mcount + 31) >> 5) {
        case 1: gemm_tile<MODE, 1>(a, ti, lds, row_src, row_w); break;
        case 2: gemm_tile<MODE, 2>(a, ti, lds, row_src, row_w); break;
        case 3: gemm_tile<MODE, 3>(a, ti, lds, row_src, row_w); break;
        case 4: gemm_tile<MODE, 4>(a, ti, lds, row_src, row_w); break;
        default: gemm_tile<MODE, 5>(a, ti, lds, row_src, row_w); break;
    }
}

// out[t] = ((y[t,0] + y[t,1]) + ... + y[t,k-1]) + ysh[t]; y rows already carry
// their routing weight, ysh the shared weight.  Slots whose expert index is
// out of range contribute nothing.
// Every slot row of the token is requested before the first add (KMAX >= k
// rows, streamed once: non-temporal), then added in slot order.
__device__ __forceinline__ float4 ld_stream4(const float* p) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
}

template <int KMAX>
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ y, const float* __restrict__ ysh,
               const int32_t* __restrict__ idx, int T, int H, int E, int k, int has_shared,
               float* __restrict__ out) {
    const int h4 = H / 4;
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)T * h4) return;
    const int t = (int)(i / h4), o4 = (int)(i % h4);
    float4 v[KMAX];
    bool ok[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        ok[j] = false;
        if (j < k) {
            ok[j] = (unsigned)idx[(size_t)t * k + j] < (unsigned)E;
            v[j] = ld_stream4(y + ((size_t)t * k + j) * H + 4 * o4);
        }
    }
    const float4 sh = has_shared ? ld_stream4(ysh + (size_t)t * H + 4 * o4)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (ok[j]) {   // a slot whose expert index is out of range adds nothing
            acc.x += v[j].x;
            acc.y += v[j].y;
            acc.z += v[j].z;
            acc.w += v[j].w;
        }
    }
    if (has_shared) {
        acc.x += sh.x;
        acc.y += sh.y;
        acc.z += sh.z;
        acc.w += sh.w;
    }
    reinterpret_cast<float4*>(out + (size_t)t * H)[o4] = acc;
}

hipError_t launch_mfma(const moe_layer_desc& d, const float* x, int T, const int32_t* idx,
                       const float* w, int shard, int nshards, float* out, char* ws,
                       const WsLayout& L, const Ctx& c, bool x16_ready) {
    const int H = d.hidden, E = d.n_experts, k = d.top_k;
    const bool shared = d.shared_inter > 0;
    const int Iloc = d.inter / nshards;
    _Float16* x16 = reinterpret_cast<_Float16*>(ws + L.x16);
    int32_t* bhist = reinterpret_cast<int32_t*>(ws + L.bhist);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* tile_off = reinterpret_cast<int32_t*>(ws + L.tile_off);
    int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
    _Float16* h16 = reinterpret_cast<_Float16*>(ws + L.h16);
    float* y = reinterpret_cast<float*>(ws + L.y);
    float* ysh = reinterpret_cast<float*>(ws + L.ysh);

    if (!x16_ready) {
        hipError_t e = launch_x16(x, T, H, ws, L, c);
        if (e != hipSuccess) return e;
    }
    int4* tile_rec = reinterpret_cast<int4*>(ws + L.tile_rec);
    hipError_t err =
        launch_bucket(idx, T, k, E, shared, counts, offsets, tile_off, tile_rec, perm, bhist, c);
    if (err != hipSuccess) return err;
    // an upper bound on the number of row tiles; blocks past the real count exit
    const int max_tiles = max_row_tiles(T, k, E, shared);
    const int max_tiles8 = (max_tiles + 7) / 8 * 8;

    GemmArgs a = {};
    a.perm = perm;
    a.offsets = offsets;
    a.tile_off = tile_off;
    a.tile_rec = tile_rec;
    a.T = T;
    a.H = H;
    a.E = E;
    a.k = k;
    a.I = d.inter;
    a.Is = d.shared_inter;
    a.shard = shard;
    a.nshards = nshards;
    a.route_w = w;
    a.sw = d.shared_weight;

    GemmArgs g1 = a;
    g1.a_src = x16;
    g1.a_stride = H;
    g1.w_routed = d.gate_q;
    g1.w_routed2 = d.up_q;
    g1.w_shared = d.sh_gate_q;
    g1.w_shared2 = d.sh_up_q;
    g1.n_ntiles = (Iloc + kTN / 2 - 1) / (kTN / 2);
    g1.nk = H / kBK;
    g1.h_out = h16;
    g1.h_stride = Iloc;
    launch_k(c, MOE_K_GEMM_GATEUP, gemm_grouped_kernel<0>, dim3(max_tiles8 * g1.n_ntiles),
             dim3(kGemmThreads), 0, g1);

    GemmArgs g2 = a;
    g2.a_src = h16;
    g2.a_stride = Iloc;
    g2.w_routed = d.down_q;
    g2.w_shared = d.sh_down_q;
    g2.n_ntiles = (H + kTN - 1) / kTN;
    g2.nk = Iloc / kBK;
    g2.sb_rows = (d.inter % kSbWeights == 0 && Iloc % kSbWeights == 0) ? 1 : 0;
    g2.y = y;
    g2.ysh = ysh;
    launch_k(c, MOE_K_GEMM_DOWN, gemm_grouped_kernel<1>, dim3(max_tiles8 * g2.n_ntiles),
             dim3(kGemmThreads), 0, g2);

    const size_t nc = (size_t)T * H / 4;
    if (k <= 8)
        launch_k(c, MOE_K_COMBINE, combine_kernel<8>, dim3((unsigned)((nc + 255) / 256)), dim3(256),
                 0, y, ysh, idx, T, H, E, k, shared ? 1 : 0, out);
    else
        launch_k(c, MOE_K_COMBINE, combine_kernel<16>, dim3((unsigned)((nc + 255) / 256)), dim3(256),
                 0, y, ysh, idx, T, H, E, k, shared ? 1 : 0, out);
    return hipGetLastError();
}

}  // namespace moe
