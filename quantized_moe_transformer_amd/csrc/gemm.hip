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
// This kernel serves the K-quant weight format (MXFP4 weights take the
// block-scaled matrix cores, gemm_mx.hip).  One kernel template serves both
// projections.  A workgroup owns one tile:
// up to 160 rows of one expert's group (a whole routed expert at T = 4096, so
// its weights are dequantised once per column tile) times 256 weight rows, and
// walks K in steps of 64 (one pair of K-quant sub-blocks).  Its 8 waves are
//   4 consumer waves: MFMA only; wave w owns two 32-wide column blocks times
//     every 32-row block the tile has (up to 5), so each fragment read from
//     LDS feeds several MFMAs; the fragment reads of a 16-deep K slice are
//     issued two slices ahead of its MFMAs;
//   4 producer waves: dequantise the next step's packed weights into the
//     other fp16 weight stage.  Where every row's K range is whole
//     superblocks they fetch superblock p of all 256 rows together with
//     coalesced direct loads into LDS, one superblock ahead, and each copies
//     its own row into registers once per four steps;
//   the consumer waves also fetch the token rows (fp16) by direct loads, a
//     step ahead, so each group of waves waits only for its own loads.
// One producer and one consumer wave share each SIMD: the dequantisation
// (VALU) of one wave runs beside the MFMAs of the other, which measured far
// better than dequantising into MFMA operand registers in the MFMA wave
// itself, where the two serialise.  The cost is a barrier per K step: the
// consumers' fragment reads after each barrier, and the token rows, fetched
// one step ahead, bound a step at about twice its MFMA time.
//
//   gateup (MODE 0): A = token rows of x16 gathered through the expert-sorted
//     slot list, B = 128 gate rows + the matching 128 up rows (4-bit); each
//     consumer wave holds a gate block and the matching up block, so the
//     epilogue forms h = silu(g) * u (fp16, scaled by 2^-4) in registers and
//     writes it, staged through LDS, in sorted row order.
//   down (MODE 1): A = h rows (contiguous per expert), B = 256 down rows
//     (5-bit); the epilogue scales by the routing weight (and 2^4) and writes
//     the slot's row of the per-slot buffer (the shared expert: its own
//     buffer, times its weight).
//   combine: out[t] = sum over slots in selected-slot order, then the shared
//     expert (page "CKE Zip: From Splitting Tokens To Splitting Qwen3.5
//     Weights", section "A Separate Decode Result Shows Why Axis Choice
//     Matters").
#include "launch.h"

namespace moe {

constexpr int kBK = 64;                 // K per step (one pair of sub-blocks)
constexpr int kLdsRow = kBK + 8;        // halves per LDS row (8 halves of padding)
constexpr int kTM = kTileM;             // rows per tile (up to 5 blocks of 32)
constexpr int kTN = 256;                // weight rows per tile
// weight-load prefetch distance (steps) of the per-piece path (down rows whose
// K range is not whole superblocks): 2 steps for the 5-bit stream
template <int MODE> struct PrefetchDistance { static constexpr int v = MODE == 0 ? 3 : 2; };
constexpr int kConsumers = 4;           // consumer waves (two 32-column blocks each)
constexpr int kProducers = 4;           // producer waves
constexpr int kGemmThreads = 64 * (kConsumers + kProducers);
constexpr int kBTasks = kTN * 2 / (64 * kProducers);   // 16-byte code pieces per producer thread

// Dequantise one 16-byte K-quant code piece (32 weights: sub-block 2c low
// nibbles and sub-block 2c+1 high nibbles) to fp16 and store it into an LDS
// row at k offsets 16*hh + [0,16) and 32 + 16*hh + [0,16).  The operands are
// kq_piece_f16's: the round-to-nearest-even fp16 of the exact fp32 weight,
// the same function the dequantisation test hook runs.
template <bool HIGH>
__device__ __forceinline__ void dequant_piece_to_lds(const SbHead& hd, const uint4& qs,
                                                     const uint4& qh, int c, int hh,
                                                     _Float16* row) {
    uint32_t lo[8], hi[8];
    kq_piece_f16<HIGH>(hd, qs, qh, c, lo, hi);
    *reinterpret_cast<uint4*>(row + 16 * hh) = uint4{lo[0], lo[1], lo[2], lo[3]};
    *reinterpret_cast<uint4*>(row + 16 * hh + 8) = uint4{lo[4], lo[5], lo[6], lo[7]};
    *reinterpret_cast<uint4*>(row + 32 + 16 * hh) = uint4{hi[0], hi[1], hi[2], hi[3]};
    *reinterpret_cast<uint4*>(row + 32 + 16 * hh + 8) = uint4{hi[4], hi[5], hi[6], hi[7]};
}

// LDS operand fragments read as asm, so that the compiler keeps the reads
// where they stand (it otherwise sinks each read to its first MFMA and waits
// for it there); lds_wait_frags then waits for them.  LDS operations complete
// in order, so waiting until at most N are outstanding, N being the reads
// issued after the ones needed, is exact for this wave's own reads and only
// stricter when the compiler's own LDS or scalar loads are in flight too.
template <int OFF>
__device__ __forceinline__ void lds_read_frag(half8& dst, uint32_t addr) {
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(OFF));
}

// MB fragments at LDS byte addresses base + 4096 i (one per 32-row block)
template <int MB>
__device__ __forceinline__ void lds_read_rows(half8* dst, uint32_t base) {
    if constexpr (MB > 0) lds_read_frag<0>(dst[0], base);
    if constexpr (MB > 1) lds_read_frag<4096>(dst[1], base);
    if constexpr (MB > 2) lds_read_frag<8192>(dst[2], base);
    if constexpr (MB > 3) lds_read_frag<12288>(dst[3], base);
    if constexpr (MB > 4) lds_read_frag<16384>(dst[4], base);
}

// wait until at most N LDS operations are outstanding; each fragment is tied
// to the wait so that no use of it is scheduled above it
template <int N, int CNT>
__device__ __forceinline__ void lds_wait_frags(half8 (&f)[CNT]) {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)" : : "i"(N));
#pragma unroll
    for (int i = 0; i < CNT; ++i) asm volatile("" : "+v"(f[i]));
}

struct GemmArgs {
    const _Float16* a_src;          // MODE 0: x16 [T][H]; MODE 1: h16 [T*k + T][Iloc]
    int a_stride;                   // halves per A row
    const int32_t* perm;            // expert-sorted slot ids
    const int32_t* offsets;         // [E+2]: group row starts (group E = shared expert)
    const int32_t* tile_off;        // [E+2]: group tile starts
    const int4* tile_rec;           // per row tile: group, first sorted row, rows, row offset
    int T, H, E, k, I, Is;
    int i0, iloc;                   // intermediate rows [i0, i0 + iloc) of every expert
    const uint8_t *w_routed, *w_routed2, *w_shared, *w_shared2;   // MODE 0: gate, up
    const float* route_w;           // [T*k] routing weights
    float sw;
    int n_ntiles;                   // weight-row tiles per group
    int nk;                         // K steps
    int sb_rows;                    // MODE 1: every row's K range is whole superblocks
    _Float16* h_out;                // MODE 0
    int h_stride;
    int16_t* y;                     // MODE 1: [T*k][H] (16-bit block floating point)
    int16_t* ysh;                   // MODE 1: [T][H]
    uint8_t* ysc;                   // MODE 1: [T*k][H/8] exponent bytes of y
    uint8_t* yshsc;                 // MODE 1: [T][H/8] those of ysh
};

// Packed weights of one producer task (weight row, 16-byte half) for one step.
struct BRegs {
    uint4 head, qs, qh;
};

// A stages hold kTM rows of kBK halves with no padding; the 16-byte chunk c
// of row r sits at chunk position c ^ ((r >> 1) & 7), so the 32 rows that one MFMA
// fragment read touches spread over all banks.
// Token-row stages: the rows of step kk + kAStages - 1 are requested at the
// start of step kk, into the stage that step kk - 1 read.
constexpr int kAStages = 2;

// wait until at most n later steps' token-row loads (MB per step) are in flight
template <int MB>
__device__ __forceinline__ void wait_a_steps(int n) {
    static_assert(kAStages - 2 <= 2, "wait_a_steps covers up to two later steps");
    if (n >= 2) wait_vmcnt<2 * MB>();
    else if (n == 1) wait_vmcnt<MB>();
    else wait_vmcnt<0>();
}

// Packed superblocks of the tile's 256 weight rows, one superblock per row,
// row after row (the largest: 5-bit, 11 chunks of 16 bytes per row).
constexpr int kRawChunks = kTN * (kQ5Bytes / 16);

struct __align__(16) GemmLds {
    _Float16 a[kAStages][kTM * kBK];
    _Float16 b[2][kTN][kLdsRow];
    uint4 raw[kRawChunks];
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
__device__ __forceinline__ void gemm_produce(const GemmArgs& a, const TileInfo& ti, GemmLds& lds) {
    constexpr int DSB = kQ5Bytes;   // bytes of a down superblock
    constexpr int kPD = PrefetchDistance<MODE>::v;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int g = ti.g;
    const int Iexp = ti.Iexp, Iloc = ti.Iloc, i0 = ti.i0, n0 = ti.n0;
    const bool is_sh = ti.is_sh;

    // ------------------------------- producers -------------------------------
    const int pt = tid - 64 * kConsumers;
    if (MODE == 0 || a.sb_rows) {
        // Every weight row's K range is whole superblocks (gate/up always; the
        // down rows when the shard boundary falls on superblocks).  The
        // producer waves fetch superblock p of all 256 rows together -- chunk
        // q = 16-byte piece q % NCH of row q / NCH, consecutive lanes on
        // consecutive bytes of a row -- by direct loads into lds.raw, one
        // superblock ahead; producer thread pt owns row pt, copies its
        // superblock into registers once per four steps and dequantises one
        // sub-block pair of it per step.
        constexpr int SBB = MODE == 0 ? kQ4Bytes : DSB;
        constexpr int NCH = SBB / 16;
        const int nsb = a.nk / 4;
        auto row_base = [&](int r) -> const uint8_t* {
            if (MODE == 0) {
                const int col = r & (kTN / 2 - 1);
                const int colc = n0 + col < Iloc ? col : 0;   // ragged tile: discarded columns
                const size_t mat = (size_t)a.I * a.H / kSbWeights * kQ4Bytes;
                const uint8_t* m = is_sh ? (r < kTN / 2 ? a.w_shared : a.w_shared2)
                                         : (r < kTN / 2 ? a.w_routed : a.w_routed2) + (size_t)g * mat;
                return m + (size_t)(i0 + n0 + colc) * (a.H / kSbWeights) * kQ4Bytes;
            } else {
                const int o = n0 + r < a.H ? n0 + r : n0;     // ragged tile: discarded rows
                const uint8_t* m = is_sh ? a.w_shared
                                         : a.w_routed + (size_t)g * ((size_t)a.H * a.I / kSbWeights * DSB);
                return m + (((size_t)o * Iexp + i0) >> 8) * DSB;
            }
        };
        const uint8_t* gsrc[NCH];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const int q = pt + 64 * kProducers * i;
            gsrc[i] = row_base(q / NCH) + 16 * (q % NCH);
        }
        const uint32_t raw_lds = (uint32_t)(uintptr_t)&lds.raw[0];
        const int pw = wave - kConsumers;
        auto issue_raw = [&](int p) {
#pragma unroll
            for (int i = 0; i < NCH; ++i)
                lds_dma16(gsrc[i] + (size_t)p * SBB,
                          __builtin_amdgcn_readfirstlane(raw_lds + (64 * pw + 64 * kProducers * i) * 16));
        };
        uint4 R[NCH];
        auto read_raw = [&]() {
#pragma unroll
            for (int i = 0; i < NCH; ++i) R[i] = lds.raw[pt * NCH + i];
        };
        auto deq_step = [&](int c, int stage) {
            SbHead hd;
            hd.d = f16_bits_to_f32(R[0].x & 0xffffu);
            hd.dmin = f16_bits_to_f32(R[0].x >> 16);
            hd.s0 = R[0].y;
            hd.s1 = R[0].z;
            hd.s2 = R[0].w;
            _Float16* dst = &lds.b[stage][pt][0];
            if (MODE == 0) {
                dequant_piece_to_lds<false>(hd, R[1 + 2 * c], R[1 + 2 * c], c, 0, dst);
                dequant_piece_to_lds<false>(hd, R[2 + 2 * c], R[2 + 2 * c], c, 1, dst);
            } else {
                dequant_piece_to_lds<true>(hd, R[3 + 2 * c], R[1], c, 0, dst);
                dequant_piece_to_lds<true>(hd, R[4 + 2 * c], R[2], c, 1, dst);
            }
        };
        issue_raw(0);
        wait_vmcnt<0>();
        __syncthreads();   // superblock 0 of every row in lds.raw
        read_raw();
        deq_step(0, 0);
        __syncthreads();   // stage 0 ready; lds.raw free
        if (nsb > 1) issue_raw(1);
        // step kk = 4p + u: the consumers read stage kk & 1 while this
        // dequantises step kk + 1 into the other; superblock p + 1 is copied
        // from lds.raw in step 4p + 3, requested at the start of step 4p
        // and waited for at the end of step 4p + 2
        for (int p = 0; p < nsb; ++p) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int nxt = 4 * p + u + 1;
                if (u < 3) {
                    deq_step(u + 1, nxt & 1);
                } else if (p + 1 < nsb) {
                    read_raw();
                    deq_step(0, nxt & 1);
                }
                if (u == 2 && p + 1 < nsb) wait_vmcnt<0>();
                __syncthreads();
                if (u == 3 && p + 2 < nsb) issue_raw(p + 2);
            }
        }
        return;
    }
    __syncthreads();   // matches the superblock paths' first barrier
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
                            : a.w_routed + (size_t)g * ((size_t)a.H * a.I / kSbWeights * DSB);
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
                const uint8_t* sb = wsrc[q] + (base >> 8) * DSB;
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
                                             float16v (&acc)[MB][2]) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int mcount = ti.mcount, grow0 = ti.grow0;
    const bool is_sh = ti.is_sh;

    // ------------------------------- consumers -------------------------------
    // The consumer waves move the token rows (A) into LDS themselves with direct
    // global-to-LDS loads (no registers), into a ring of kAStages stages,
    // so their waits cover only these loads and the producers' waits only the
    // weight loads.  Thread tid's load i fills chunk slot q = tid + 256 i: row
    // q >> 3, chunk position q & 7, i.e. logical chunk (q & 7) ^ ((row >> 1) & 7).  Rows
    // past the tile's end re-read one of its rows (row r mod mcount): their
    // results are discarded, and every load is unconditional so each step
    // issues exactly MB of them per wave.
    size_t asrc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int q = tid + 256 * i;
        const int r = q >> 3, c = (q & 7) ^ ((r >> 1) & 7);
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

    // this wave's two 32-row blocks of B: gate block w and up block w (MODE 0,
    // rows 32w and 128 + 32w), or output blocks 2w and 2w+1 (MODE 1)
    const int bc0 = MODE == 0 ? 32 * wave : 64 * wave;
    for (int s = 0; s < kAStages - 1; ++s)
        if (s < a.nk) issue_a(s);
    __syncthreads();              // the producers' first superblock fetch
    wait_a_steps<MB>(min(kAStages - 1, a.nk) - 1);   // step 0's rows landed
    __syncthreads();              // stage 0 ready
    // The MFMAs of each step's last K slice run after the next barrier, from
    // fragments already in registers (the stage they came from may then be
    // overwritten): they cover the latency of the next step's first fragment
    // reads, which otherwise leave the matrix core idle from the barrier to
    // the first MFMA (several hundred cycles of a 2 500-cycle step in cycle
    // stamps).  Only slice 0's reads go out before them: with slice 1's as
    // well, the carried fragments no longer fit the 256 registers.
    const int nl = lane & 31, kh = lane >> 5;
    constexpr int kB1 = (MODE == 0 ? kTN / 2 : 32) * kLdsRow * 2;   // bytes from block bc0 to bc1
    half8 ft[MB + 2];   // the previous step's last slice
    auto mfma_slice = [&](const half8 (&g)[MB + 2]) {
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(g[i], g[MB], acc[i][0], 0, 0, 0);
            acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(g[i], g[MB + 1], acc[i][1], 0, 0, 0);
        }
    };
    for (int kk = 0; kk < a.nk; ++kk) {
        const int st = kk & 1;
        // fragments of K slice ks: f[ks][0..MB) token rows, f[ks][MB], f[ks][MB+1]
        // the two weight blocks; slice ks + 2's reads are issued before the
        // MFMAs of slice ks
        const uint32_t sa = (uint32_t)(uintptr_t)&lds.a[kk % kAStages][0] + 128 * nl;
        const uint32_t sb = (uint32_t)(uintptr_t)&lds.b[st][bc0 + nl][8 * kh];
        half8 f[4][MB + 2];
        auto read_slice = [&](int ks) {
            lds_read_rows<MB>(f[ks], sa + 16 * ((2 * ks + kh) ^ ((nl >> 1) & 7)));
            lds_read_frag<0>(f[ks][MB], sb + 32 * ks);
            lds_read_frag<kB1>(f[ks][MB + 1], sb + 32 * ks);
        };
        // the rows of step kk + kAStages - 1 go to the stage that step kk - 1
        // read (every wave left it at the last barrier)
        if (kk + kAStages - 1 < a.nk) issue_a(kk + kAStages - 1);
        read_slice(0);
        __builtin_amdgcn_sched_barrier(0);
        if (kk > 0) mfma_slice(ft);
        __builtin_amdgcn_sched_barrier(0);
        read_slice(1);
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            __builtin_amdgcn_sched_barrier(0x6);
            if (ks < 3) lds_wait_frags<MB + 2>(f[ks]);   // slice ks + 1 may still be in flight
            else lds_wait_frags<0>(f[ks]);
            if (ks < 2) read_slice(ks + 2);
            if (ks < 3) {
                mfma_slice(f[ks]);
            } else {
#pragma unroll
                for (int i = 0; i < MB + 2; ++i) ft[i] = f[3][i];
            }
        }
        // step kk + 1's rows must have landed before the barrier
        wait_a_steps<MB>(min(kAStages - 2, a.nk - kk - 2));
        __syncthreads();
    }
    mfma_slice(ft);   // the last step's last slice

}

// Epilogue, all 8 waves: each 32-row block of the tile is staged through LDS
// (the operand stages are no longer read) and written with 16-byte stores of
// whole row segments.
//   MODE 0: h = silu(gate) * up * 2^-4 as fp16, rows in sorted order.
//   MODE 1: the slot's row (the shared expert: its own buffer) times the
//   row's weight * 2^4, as 16-bit block floating point (store_rows_q16).
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
            store_rows_q16<kGemmThreads>(t, kPitch, ti.is_sh ? a.ysh : a.y,
                                         ti.is_sh ? a.yshsc : a.ysc, row_src, 32 * i, ti.mcount,
                                         ti.n0, a.H);
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
        gemm_produce<MODE, MB>(a, ti, lds);
    else
        gemm_consume<MODE, MB>(a, ti, lds, acc);
    gemm_epilogue<MODE, MB>(a, ti, lds, row_src, row_w, acc);
}

// tile_off, tile_rec, the packed counts (experts | column tiles << 16) and the
// number of records come first as scalar arguments, which the hardware
// preloads into registers: a workgroup reads the tile count and its record
// at once, with no kernel-argument load before them.
template <int MODE>
__global__ void __launch_bounds__(kGemmThreads)
gemm_grouped_kernel(const int32_t* __restrict__ tile_off, const int4* __restrict__ tile_rec,
                    uint32_t e_nt, int max_tiles, GemmArgs a) {
    __shared__ GemmLds lds;
    __shared__ int32_t row_src[kTM];     // MODE 0: token of each row; MODE 1: slot id
    __shared__ float row_w[kTM];         // MODE 1: routing weight * 2^4 of each row

    // block -> (row tile, column tile): the column tiles of one row tile run
    // on one XCD (blocks 8 apart), so its gathered rows are reused in L2; the
    // records are stored in the order the row tiles are taken (the shared
    // expert's, the largest, first)
    const int b = blockIdx.x;
    const int nt = hi16(e_nt);
    const int tile_raw = (b / (8 * nt)) * 8 + (b & 7);
    const int ntile = (b >> 3) % nt;
    const int ntiles = tile_off[lo16(e_nt) + 1];
    const int4 rec = tile_rec[min(tile_raw, max_tiles - 1)];   // written by the bucketing
    // both loads in flight together: the record is needed in registers
    // before the exit test (the compiler would otherwise load it after)
    asm volatile("" ::"s"(rec.x), "s"(rec.y), "s"(rec.z), "s"(rec.w));
    if (tile_raw >= ntiles) return;
    TileInfo ti;
    ti.g = rec.x;
    ti.is_sh = ti.g == a.E;
    ti.grow0 = rec.y;                      // first row of the tile in sorted order
    ti.mcount = rec.z;
    ti.m0 = rec.w;
    ti.Iexp = ti.is_sh ? a.Is : a.I;
    ti.Iloc = a.iloc;   // the shared expert has the routed width
    ti.i0 = a.i0;
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

// out[t] = ((y[t,0] + y[t,1]) + ... + y[t,k-1]) + ysh[t] in fp32, each row
// value its int16 mantissa times its block's factor (store_rows_q16); y rows
// already carry their routing weight, ysh the shared weight.
// Slots whose expert index is out of range contribute nothing.  One thread per
// 8 outputs: every slot row's 16 bytes of the token are requested before the
// first add (KMAX >= k rows, streamed once: non-temporal), then added in slot
// order.
__device__ __forceinline__ void ld_stream8q(const int16_t* p, float (&f)[8]) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t w = v[j];
        f[2 * j] = (float)(int)(int16_t)(w & 0xffffu);
        f[2 * j + 1] = (float)((int)w >> 16);
    }
}

// a block's exponent byte -> the factor of its int16 mantissas
__device__ __forceinline__ float yq_scale(int eb) {
    return eb == kYNanByte ? __builtin_nanf("") : __builtin_ldexpf(kYInvQ, eb - 126);
}

template <int KMAX>
__global__ void __launch_bounds__(256)
combine_kernel(const int16_t* __restrict__ y, const int16_t* __restrict__ ysh,
               const uint8_t* __restrict__ ysc, const uint8_t* __restrict__ yshsc,
               const int32_t* __restrict__ idx, int T, int H, int E, int k, int has_shared,
               float* __restrict__ out) {
    const int h8 = H / 8;
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)T * h8) return;
    const int t = (int)(i / h8), o8 = (int)(i % h8);
    float v[KMAX][8], sc[KMAX];
    bool ok[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        ok[j] = false;
        sc[j] = 0.f;
        if (j < k) {
            const size_t s = (size_t)t * k + j;
            ok[j] = (unsigned)idx[s] < (unsigned)E;
            ld_stream8q(y + s * H + 8 * o8, v[j]);
            sc[j] = yq_scale(ysc[s * h8 + o8]);
        }
    }
    float sh[8], shs = 0.f;
    if (has_shared) {
        ld_stream8q(ysh + (size_t)t * H + 8 * o8, sh);
        shs = yq_scale(yshsc[(size_t)t * h8 + o8]);
    } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) sh[c] = 0.f;
    }
    float acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = 0.f;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
        if (ok[j]) {   // a slot whose expert index is out of range adds nothing
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[c] += v[j][c] * sc[j];
        }
    }
    if (has_shared) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[c] += sh[c] * shs;
    }
    float4* o = reinterpret_cast<float4*>(out + (size_t)t * H + 8 * o8);
    o[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    o[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

hipError_t launch_mfma(const moe_layer_desc& d, const float* x, int T, const int32_t* idx,
                       const float* w, int i0, int iloc, float* out, char* ws,
                       const WsLayout& L, const Ctx& c, bool x16_ready) {
    const int H = d.hidden, E = d.n_experts, k = d.top_k;
    const bool shared = d.shared_inter > 0;
    const int Iloc = iloc;
    _Float16* x16 = reinterpret_cast<_Float16*>(ws + L.x16);
    int32_t* bhist = reinterpret_cast<int32_t*>(ws + L.bhist);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* tile_off = reinterpret_cast<int32_t*>(ws + L.tile_off);
    int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
    _Float16* h16 = reinterpret_cast<_Float16*>(ws + L.h16);
    int16_t* y = reinterpret_cast<int16_t*>(ws + L.y);
    int16_t* ysh = reinterpret_cast<int16_t*>(ws + L.ysh);
    uint8_t* ysc = reinterpret_cast<uint8_t*>(ws + L.ysc);
    uint8_t* yshsc = reinterpret_cast<uint8_t*>(ws + L.yshsc);

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
    a.i0 = i0;
    a.iloc = iloc;
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
    if (E > 0xffff || g1.n_ntiles > 0xffff) return hipErrorInvalidValue;   // packed in 16 bits
    launch_k(c, MOE_K_GEMM_GATEUP, gemm_grouped_kernel<0>, dim3(max_tiles8 * g1.n_ntiles),
             dim3(kGemmThreads), 0, (const int32_t*)tile_off, (const int4*)tile_rec,
             pack16(E, g1.n_ntiles), max_tiles, g1);

    GemmArgs g2 = a;
    g2.a_src = h16;
    g2.a_stride = Iloc;
    g2.w_routed = d.down_q;
    g2.w_shared = d.sh_down_q;
    g2.n_ntiles = (H + kTN - 1) / kTN;
    g2.nk = Iloc / kBK;
    g2.sb_rows = (d.inter % kSbWeights == 0 && Iloc % kSbWeights == 0 && i0 % kSbWeights == 0) ? 1 : 0;
    g2.y = y;
    g2.ysh = ysh;
    g2.ysc = ysc;
    g2.yshsc = yshsc;
    if (g2.n_ntiles > 0xffff) return hipErrorInvalidValue;
    launch_k(c, MOE_K_GEMM_DOWN, gemm_grouped_kernel<1>, dim3(max_tiles8 * g2.n_ntiles),
             dim3(kGemmThreads), 0, (const int32_t*)tile_off, (const int4*)tile_rec,
             pack16(E, g2.n_ntiles), max_tiles, g2);

    return launch_combine(y, ysh, ysc, yshsc, idx, T, H, E, k, shared, out, c);
}

hipError_t launch_combine(const int16_t* y, const int16_t* ysh, const uint8_t* ysc,
                          const uint8_t* yshsc, const int32_t* idx, int T, int H, int E, int k,
                          bool shared, float* out, const Ctx& c) {
    const size_t nc = (size_t)T * H / 8;
    if (k <= 8)
        launch_k(c, MOE_K_COMBINE, combine_kernel<8>, dim3((unsigned)((nc + 255) / 256)), dim3(256),
                 0, y, ysh, ysc, yshsc, idx, T, H, E, k, shared ? 1 : 0, out);
    else
        launch_k(c, MOE_K_COMBINE, combine_kernel<16>, dim3((unsigned)((nc + 255) / 256)), dim3(256),
                 0, y, ysh, ysc, yshsc, idx, T, H, E, k, shared ? 1 : 0, out);
    return hipGetLastError();
}

}  // namespace moe
