// moe_internal.h -- device helpers and constants of libmoe_hip.so
//
// Everything here is gfx950 (CDNA4) code: 64-lane wavefronts, MFMA matrix
// cores, 160 KB of LDS per CU.  Nothing in this directory is shared with the
// CPU oracle.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;
constexpr int kQ4Bytes = 144;   // 4-bit K-quant superblock
constexpr int kQ5Bytes = 176;   // 5-bit K-quant superblock
constexpr int kMxBytes = 144;   // MXFP4 superblock (8 scale bytes, 8 reserved, 128 code bytes)
constexpr int kSbWeights = 256;
// router: split-K fp32 partials on the vector units up to this many rows (the
// GEMV path folds them into its first kernel), the matrix-core router beyond
constexpr int kRouterSmallMaxT = 32;
constexpr int kTileM = 160;     // grouped-GEMM rows (slots) per tile (5 blocks of 32)
constexpr int kRouterSplits = 8;   // split-K partial logits per expert at small T
// h is carried into the down projection as fp16 scaled by 2^-4: the SwiGLU
// output of the Qwen3.5-shaped layer reaches ~2e4, the scale keeps a 50x
// margin to fp16's 65504 at no cost in relative precision.
constexpr float kHScale = 0.0625f;
constexpr float kHUnscale = 16.0f;
// MXFP4 prefill: tokens and h enter the block-scaled matrix cores as the sum
// of this many MX-FP8 terms (e4m3 codes, an E8M0 scale per 32 values)
constexpr int kMxTerms = 3;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// K-quant field decoding (device)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float f16_bits_to_f32(uint32_t bits16) {
    union { uint16_t u; _Float16 h; } cv;
    cv.u = (uint16_t)bits16;
    return (float)cv.h;
}

// The 16-byte head of a superblock: d, dmin and the 12 scale bytes as words.
struct SbHead {
    float d, dmin;
    uint32_t s0, s1, s2;
};

__device__ __forceinline__ SbHead load_head(const uint8_t* sb) {
    uint4 v = *reinterpret_cast<const uint4*>(sb);
    SbHead h;
    h.d = f16_bits_to_f32(v.x & 0xffffu);
    h.dmin = f16_bits_to_f32(v.x >> 16);
    h.s0 = v.y;
    h.s1 = v.z;
    h.s2 = v.w;
    return h;
}

// 6-bit scale and min of sub-block j.  Bytes 0..3 (word s0) carry the scales
// of sub-blocks 0..3 in their low six bits and the top two bits of the scales
// of sub-blocks 4..7; bytes 4..7 (s1) do the same for the mins; bytes 8..11
// (s2) carry the low nibbles of scale (low half) and min (high half) of
// sub-blocks 4..7.
__device__ __forceinline__ void sub_scale_min(const SbHead& h, int j, float& sc, float& m) {
    uint32_t isc, im;
    if (j < 4) {
        isc = (h.s0 >> (8 * j)) & 63u;
        im = (h.s1 >> (8 * j)) & 63u;
    } else {
        const int jj = j - 4;
        isc = ((h.s2 >> (8 * jj)) & 15u) | (((h.s0 >> (8 * jj + 6)) & 3u) << 4);
        im = ((h.s2 >> (8 * jj + 4)) & 15u) | (((h.s1 >> (8 * jj + 6)) & 3u) << 4);
    }
    sc = (float)isc;
    m = (float)im;
}

// One weight: w = d*sc*q - dmin*m.  d*sc (<= 17 significant bits) and dmin*m
// are exact in fp32, and the fused multiply-add rounds the exact value once,
// so the result is the round-to-nearest-even fp32 of the real weight.
__device__ __forceinline__ float kq_weight(float dsc, float dmm, float q) {
    return __builtin_fmaf(q, dsc, -dmm);
}

// x & m computed where the compiler cannot see the mask: with the mask in
// view it folds it into each later byte extraction (a bit-field extract per
// code before the convert); opaque, each byte converts in one
// v_cvt_f32_ubyteN.
__device__ __forceinline__ uint32_t and_opaque(uint32_t x, uint32_t m) {
    uint32_t r;
    asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(x), "v"(m));
    return r;
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

// Two fp32 values to a packed pair of fp16, each rounded to nearest even
// (v_cvt_pk_f16_f32; fp16 subnormals kept, overflow to inf).
__device__ __forceinline__ uint32_t pack_f16_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){a, b}, half2v));
}

// Per-slot expert rows between the grouped down GEMM and the combine: 16-bit
// block floating point.  Each 8 consecutive values of a row share one byte
// eb, the biased fp32 exponent of their largest magnitude m (at least 1), and
// each value v is the int16 q = snorm16(v 2^(126 - eb)) (v_cvt_pknorm_i16_f32:
// v 2^(126 - eb) lies in (-1, 1), times 32767, rounded to an integer), read
// back as q 2^(eb - 126) / 32767.  m is at least half of 2^(eb - 126), so the
// block's largest values keep 14 to 15 bits (absolute error about 2^-16 of
// 2^(eb - 126), against fp16's 11 bits), with no range limit: only blocks
// below fp32's normal range (eb = 0, taken as 1) lose bits, as fp32 itself
// does.  A block holding an inf or NaN has eb = 255, zero mantissas, and
// reads back as NaN.  m and eb come from an integer maximum of the values'
// magnitude bits, which also orders inf and NaN above every finite value.
constexpr int kYNanByte = 255;
constexpr float kYInvQ = 1.0f / 32767.0f;

// The grouped GEMMs' down epilogue: 32 staged fp32 rows of [32][pitch] floats
// (256 columns from n0) to 16-bit rows dst[row_src[m0 + r]][n0 ..] and their
// exponent bytes dse[row_src[m0 + r]][n0 / 8 ..] (H / 8 per row): 1024 chunks
// of 8 values over the NTHREADS threads, one 16-byte store each.
template <int NTHREADS>
__device__ __forceinline__ void store_rows_q16(const float* t, int pitch, int16_t* dst,
                                               uint8_t* dse, const int32_t* row_src, int m0,
                                               int mcount, int n0, int H) {
    static_assert(1024 % NTHREADS == 0, "whole chunks per thread");
#pragma unroll
    for (int j = 0; j < 1024 / NTHREADS; ++j) {
        const int q = (int)threadIdx.x + NTHREADS * j;
        const int r = q >> 5, c8 = q & 31;
        const int m = m0 + r, o = n0 + 8 * c8;
        if (m < mcount && o < H) {
            const float4 u = *reinterpret_cast<const float4*>(t + r * pitch + 8 * c8);
            const float4 v = *reinterpret_cast<const float4*>(t + r * pitch + 8 * c8 + 4);
            const float f[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
            uint32_t mb = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t b = __builtin_bit_cast(uint32_t, f[i]) & 0x7fffffffu;
                mb = mb > b ? mb : b;
            }
            int eb = (int)(mb >> 23);
            const bool bad = eb == kYNanByte;
            eb = eb < 1 ? 1 : eb;
            const int sh = 126 - eb;
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[i] = bad ? 0u
                           : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pknorm_i16(
                                                              __builtin_ldexpf(f[2 * i], sh),
                                                              __builtin_ldexpf(f[2 * i + 1], sh)));
            const size_t row = (size_t)row_src[m];
            *reinterpret_cast<uint4*>(dst + row * H + o) = make_uint4(w[0], w[1], w[2], w[3]);
            dse[row * (H / 8) + o / 8] = (uint8_t)eb;
        }
    }
}

// The 16-bit matrix-core operands of one 16-byte K-quant code piece: 16 codes
// of sub-block 2c (low nibbles, elements 64c + 16hh + [0,16)) and 16 of
// sub-block 2c+1 (high nibbles, elements 64c + 32 + 16hh + [0,16)), for the
// 5-bit format with their high bits from qh (bits 2c and 2c+1 of each byte).
// Each weight is formed exactly as kq_weight forms it (one fused multiply-add
// of the exact d*sc and dmin*m: the round-to-nearest-even fp32 weight), then
// rounded to the nearest-even fp16: lo[w] / hi[w] hold elements 2w, 2w+1 of
// the two runs of 16.
template <bool HIGH>
__device__ __forceinline__ void kq_piece_f16(const SbHead& hd, const uint4& qs, const uint4& qh,
                                             int c, uint32_t (&lo)[8], uint32_t (&hi)[8]) {
    float sca, ma, scb, mb;
    sub_scale_min(hd, 2 * c, sca, ma);
    sub_scale_min(hd, 2 * c + 1, scb, mb);
    const float dsa = hd.d * sca, dsb = hd.d * scb;      // exact in fp32
    const float dma = hd.dmin * ma, dmb = hd.dmin * mb;  // exact in fp32
    const uint32_t qw[4] = {qs.x, qs.y, qs.z, qs.w};
    const uint32_t hw[4] = {qh.x, qh.y, qh.z, qh.w};
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
        uint32_t l5 = and_opaque(qw[wi], 0x0f0f0f0fu);
        uint32_t h5 = and_opaque(qw[wi] >> 4, 0x0f0f0f0fu);
        if (HIGH) {
            l5 |= ((hw[wi] >> (2 * c)) & 0x01010101u) << 4;
            h5 |= ((hw[wi] >> (2 * c + 1)) & 0x01010101u) << 4;
        }
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            const float a0 = (float)((l5 >> (16 * pr)) & 0xffu);
            const float a1 = (float)((l5 >> (16 * pr + 8)) & 0xffu);
            const float b0 = (float)((h5 >> (16 * pr)) & 0xffu);
            const float b1 = (float)((h5 >> (16 * pr + 8)) & 0xffu);
            lo[2 * wi + pr] = pack_f16_rne(kq_weight(dsa, dma, a0), kq_weight(dsa, dma, a1));
            hi[2 * wi + pr] = pack_f16_rne(kq_weight(dsb, dmb, b0), kq_weight(dsb, dmb, b1));
        }
    }
}

// ---------------------------------------------------------------------------
// MXFP4 field decoding (device): OCP MX E8M0 block scales and E2M1 codes
// ---------------------------------------------------------------------------

// E8M0 scale byte s -> 2^(s-127), exact in fp32 (255: NaN; 0: 2^-127, a
// subnormal).
__device__ __forceinline__ float e8m0_f32(uint32_t s) {
    return s == 255u ? __builtin_nanf("")
                     : __uint_as_float(s == 0u ? 0x00400000u : (s << 23));
}

// E2M1 code (bits 0..3 of n) -> its value: magnitude m/2 for exponent 0,
// else 2^(e-1) * (1 + m/2), whose fp32 pattern is 0x3F000000 + (e,m) << 22;
// bit 3 is the sign.
__device__ __forceinline__ float e2m1_f32(uint32_t n) {
    const uint32_t em = n & 7u;
    const float mag = em >= 2u ? __uint_as_float(0x3F000000u + (em << 22)) : 0.5f * (float)em;
    return __uint_as_float(__float_as_uint(mag) | ((n & 8u) << 28));
}

// ---------------------------------------------------------------------------
// Wave reductions (64 lanes), fixed butterfly order: deterministic
// ---------------------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp_mov_f(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of `group` lanes (a power of two <= 64), the same
// bits in every lane of a group.  Up to 16 lanes by DPP moves inside a row
// (xor 1, xor 2, half-row mirror, row mirror: each step adds two equal
// groups that mirror each other, and a + b == b + a), beyond that by lane
// exchanges.
__device__ __forceinline__ float wave_sum_group(float v, int group) {
    if (group >= 2) v += dpp_mov_f<0xB1>(v);    // quad_perm [1,0,3,2]
    if (group >= 4) v += dpp_mov_f<0x4E>(v);    // quad_perm [2,3,0,1]
    if (group >= 8) v += dpp_mov_f<0x141>(v);   // row_half_mirror
    if (group >= 16) v += dpp_mov_f<0x140>(v);  // row_mirror
    if (group >= 32) v += __shfl_xor(v, 16, 64);
    if (group >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

__device__ __forceinline__ float silu_f(float z) {
    // z * sigmoid(z) with the hardware reciprocal (about 1 ulp); expf(-z)
    // overflows to +inf for very negative z, and rcp(inf) = 0 gives -0
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Small counts travel to kernels packed two to a 32-bit argument (16 bits
// each; the launchers check the ranges), so that the leading scalar
// arguments, which the hardware preloads into registers (at most 14 dwords),
// hold the pointers a workgroup needs on its critical path.
__host__ __device__ inline uint32_t pack16(int lo, int hi) {
    return (uint32_t)(lo & 0xffff) | ((uint32_t)hi << 16);
}
__device__ inline int lo16(uint32_t v) { return (int)(v & 0xffffu); }
__device__ inline int hi16(uint32_t v) { return (int)(v >> 16); }

// One 16-byte global-to-LDS load per lane: lane l's bytes land at LDS offset
// lds_off + 16 l.  Written as asm so that the compiler does not order it
// against LDS reads of other stages with waits of its own; the caller waits
// for these loads (wait_vmcnt) before any wave reads what they wrote.  Extra
// loads in the counter only make the compiler's own vmcnt waits stricter.
// The LDS address goes through m0, declared as an output of the asm (not a
// clobber of a reserved register), so that the compiler keeps any value of
// its own out of m0 across it.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_off) {
    uint32_t m0v;
    asm volatile("s_mov_b32 %0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 : "={m0}"(m0v)
                 : "v"(gptr), "s"(lds_off));
}

// The same with one dword per lane: lane l's 4 bytes land at lds_off + 4 l.
__device__ __forceinline__ void lds_dma4(const void* gptr, uint32_t lds_off) {
    uint32_t m0v;
    asm volatile("s_mov_b32 %0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                 : "={m0}"(m0v)
                 : "v"(gptr), "s"(lds_off));
}

// s_waitcnt with only the vector-memory count bounded (<= 63)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace moe
