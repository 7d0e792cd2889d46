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
//   gemm_gateup  per (expert, 64-row tile, 64 intermediate columns): the
//                rows' tokens gathered from x16, gate and up superblocks
//                dequantised into LDS as fp16, two accumulators; epilogue
//                h = silu(g) * u, stored fp16 (scaled by 2^-4) in expert-
//                sorted row order.
//   gemm_down    per (expert, 64-row tile, 128 outputs): h rows x dequantised
//                5-bit down weights; epilogue scales by the routing weight and
//                writes the row's slot of the per-slot output buffer (the
//                shared expert writes its own buffer, times its weight).
//   combine      out[t] = sum over slots in selected-slot order, then the
//                shared expert (page "CKE Zip ...", section "A Separate Decode
//                Result Shows Why Axis Choice Matters").
#include "moe_internal.h"

namespace moe {

constexpr int kBK = 64;           // K per LDS stage (one pair of sub-blocks)
constexpr int kLdsPad = 8;        // halves of padding per LDS row
constexpr int kLdsRow = kBK + kLdsPad;

__device__ __forceinline__ int find_group(const int32_t* __restrict__ tile_off, int ngroups,
                                          int tile) {
    // largest g with tile_off[g] <= tile (groups with no tiles are skipped)
    int lo = 0, hi = ngroups;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_off[mid] <= tile) lo = mid; else hi = mid;
    }
    return lo;
}

// Dequantise one 16-byte code piece (32 weights: sub-block 2c low nibbles and
// sub-block 2c+1 high nibbles) to fp16 and store it into an LDS row at k
// offsets 16*hh + [0,16) and 32 + 16*hh + [0,16).
template <bool HIGH>
__device__ __forceinline__ void dequant_piece_to_lds(const SbHead& hd, const uint4& qs,
                                                     const uint4& qh, int c, int hh,
                                                     _Float16* row) {
    float sca, ma, scb, mb;
    sub_scale_min(hd, 2 * c, sca, ma);
    sub_scale_min(hd, 2 * c + 1, scb, mb);
    const float dsa = hd.d * sca, dma = hd.dmin * ma;
    const float dsb = hd.d * scb, dmb = hd.dmin * mb;
    half8 lo[2], hi[2];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
        const uint32_t byte = piece_byte(qs, b);
        uint32_t ql = byte & 15u, qq = byte >> 4;
        if (HIGH) {
            const uint32_t hb = piece_byte(qh, b);
            ql |= ((hb >> (2 * c)) & 1u) << 4;
            qq |= ((hb >> (2 * c + 1)) & 1u) << 4;
        }
        lo[b >> 3][b & 7] = (_Float16)kq_weight(dsa, dma, (float)ql);
        hi[b >> 3][b & 7] = (_Float16)kq_weight(dsb, dmb, (float)qq);
    }
    *reinterpret_cast<half8*>(row + 16 * hh) = lo[0];
    *reinterpret_cast<half8*>(row + 16 * hh + 8) = lo[1];
    *reinterpret_cast<half8*>(row + 32 + 16 * hh) = hi[0];
    *reinterpret_cast<half8*>(row + 32 + 16 * hh + 8) = hi[1];
}

__global__ void __launch_bounds__(256)
gemm_gateup_kernel(const _Float16* __restrict__ x16, int T, int H,
                   const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
                   const int32_t* __restrict__ tile_off, int E, int k,
                   const uint8_t* __restrict__ gate, const uint8_t* __restrict__ up,
                   const uint8_t* __restrict__ sh_gate, const uint8_t* __restrict__ sh_up,
                   int I, int Is, int shard, int nshards, _Float16* __restrict__ h16,
                   int hstride) {
    __shared__ _Float16 As[kTileM][kLdsRow];
    __shared__ _Float16 Bs[128][kLdsRow];
    const int tile = blockIdx.x;
    const int ngroups = E + 1;
    if (tile >= tile_off[ngroups]) return;
    const int g = find_group(tile_off, ngroups, tile);
    const bool is_sh = g == E;
    const int m0 = (tile - tile_off[g]) * kTileM;
    const int rows = is_sh ? T : offsets[g + 1] - offsets[g];
    const int mcount = min(kTileM, rows - m0);
    const int hrow0 = offsets[g] + m0;
    const uint8_t *G, *U;
    int Iexp;
    if (!is_sh) {
        const size_t mat = (size_t)I * H / kSbWeights * kQ4Bytes;
        G = gate + (size_t)g * mat;
        U = up + (size_t)g * mat;
        Iexp = I;
    } else {
        G = sh_gate;
        U = sh_up;
        Iexp = Is;
    }
    const int Iloc = Iexp / nshards, i0 = shard * Iloc;
    const int n0 = blockIdx.y * 64;
    if (n0 >= Iloc) return;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // A loader: rows tid/8 and tid/8 + 32, 16-byte chunk tid%8
    const int ac = tid & 7;
    int tokA[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int m = (tid >> 3) + 32 * q;
        tokA[q] = -1;
        if (m < mcount) tokA[q] = is_sh ? (m0 + m) : perm[offsets[g] + m0 + m] / k;
    }
    // B loader: weight row tid/2 (first 64 gate, next 64 up), piece half tid%2
    const int br = tid >> 1, bhh = tid & 1;
    const int bcol = br & 63;
    const bool bvalid = n0 + bcol < Iloc;
    const int nsb_row = H / kSbWeights;
    const uint8_t* brow = (br < 64 ? G : U) + (size_t)(i0 + n0 + bcol) * nsb_row * kQ4Bytes;

    const int wm = wave & 1, wn = wave >> 1;
    float16v accG = {}, accU = {};
    const int nk = H / kBK;
    for (int kk = 0; kk < nk; ++kk) {
        uint4 av[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            av[q] = make_uint4(0, 0, 0, 0);
            if (tokA[q] >= 0)
                av[q] = *reinterpret_cast<const uint4*>(x16 + (size_t)tokA[q] * H + kk * kBK + ac * 8);
        }
        SbHead hd = {};
        uint4 qs = make_uint4(0, 0, 0, 0);
        const int c = kk & 3;
        if (bvalid) {
            const uint8_t* sb = brow + (kk >> 2) * kQ4Bytes;
            hd = load_head(sb);
            qs = *reinterpret_cast<const uint4*>(sb + 16 + 32 * c + 16 * bhh);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q)
            *reinterpret_cast<uint4*>(&As[(tid >> 3) + 32 * q][ac * 8]) = av[q];
        dequant_piece_to_lds<false>(hd, qs, qs, c, bhh, &Bs[br][0]);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kof = ks * 16 + 8 * (lane >> 5);
            const half8 a = *reinterpret_cast<const half8*>(&As[wm * 32 + (lane & 31)][kof]);
            const half8 bg = *reinterpret_cast<const half8*>(&Bs[wn * 32 + (lane & 31)][kof]);
            const half8 bu = *reinterpret_cast<const half8*>(&Bs[64 + wn * 32 + (lane & 31)][kof]);
            accG = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bg, accG, 0, 0, 0);
            accU = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bu, accU, 0, 0, 0);
        }
    }
    const int n = n0 + wn * 32 + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < mcount && n < Iloc) {
            const float h = silu_f(accG[v]) * accU[v] * kHScale;
            h16[(size_t)(hrow0 + m) * hstride + n] = (_Float16)h;
        }
    }
}

__global__ void __launch_bounds__(256)
gemm_down_kernel(const _Float16* __restrict__ h16, int hstride, int T, int H,
                 const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
                 const int32_t* __restrict__ tile_off, int E, int k,
                 const uint8_t* __restrict__ down, const uint8_t* __restrict__ sh_down, int I,
                 int Is, int shard, int nshards, const float* __restrict__ w, float sw,
                 float* __restrict__ y, float* __restrict__ ysh) {
    __shared__ _Float16 As[kTileM][kLdsRow];
    __shared__ _Float16 Bs[128][kLdsRow];
    __shared__ int32_t slot_s[kTileM];
    __shared__ float slot_w[kTileM];
    const int tile = blockIdx.x;
    const int ngroups = E + 1;
    if (tile >= tile_off[ngroups]) return;
    const int g = find_group(tile_off, ngroups, tile);
    const bool is_sh = g == E;
    const int m0 = (tile - tile_off[g]) * kTileM;
    const int rows = is_sh ? T : offsets[g + 1] - offsets[g];
    const int mcount = min(kTileM, rows - m0);
    const int hrow0 = offsets[g] + m0;
    const uint8_t* D;
    int Iexp;
    if (!is_sh) {
        D = down + (size_t)g * ((size_t)H * I / kSbWeights * kQ5Bytes);
        Iexp = I;
    } else {
        D = sh_down;
        Iexp = Is;
    }
    const int Iloc = Iexp / nshards, i0 = shard * Iloc;
    const int n0 = blockIdx.y * 128;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid < kTileM) {
        int s = -1;
        float ws = 0.f;
        if (tid < mcount) {
            if (is_sh) {
                s = m0 + tid;
                ws = sw * kHUnscale;
            } else {
                s = perm[hrow0 + tid];
                ws = w[s] * kHUnscale;
            }
        }
        slot_s[tid] = s;
        slot_w[tid] = ws;
    }
    const int ac = tid & 7;
    const int br = tid >> 1, bhh = tid & 1;
    const int o = n0 + br;
    const bool bvalid = o < H;
    const int wm = wave & 1, wn = wave >> 1;
    float16v acc0 = {}, acc1 = {};
    const int nk = Iloc / kBK;
    for (int kk = 0; kk < nk; ++kk) {
        uint4 av[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int m = (tid >> 3) + 32 * q;
            av[q] = make_uint4(0, 0, 0, 0);
            if (m < mcount)
                av[q] = *reinterpret_cast<const uint4*>(h16 + (size_t)(hrow0 + m) * hstride +
                                                        kk * kBK + ac * 8);
        }
        SbHead hd = {};
        uint4 qs = make_uint4(0, 0, 0, 0), qh = make_uint4(0, 0, 0, 0);
        int c = 0;
        if (bvalid) {
            const size_t base = (size_t)o * Iexp + i0 + kk * kBK;
            c = (int)((base & 255) >> 6);
            const uint8_t* sb = D + (base >> 8) * kQ5Bytes;
            hd = load_head(sb);
            qh = *reinterpret_cast<const uint4*>(sb + 16 + 16 * bhh);
            qs = *reinterpret_cast<const uint4*>(sb + 48 + 32 * c + 16 * bhh);
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 2; ++q)
            *reinterpret_cast<uint4*>(&As[(tid >> 3) + 32 * q][ac * 8]) = av[q];
        dequant_piece_to_lds<true>(hd, qs, qh, c, bhh, &Bs[br][0]);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            const int kof = ks * 16 + 8 * (lane >> 5);
            const half8 a = *reinterpret_cast<const half8*>(&As[wm * 32 + (lane & 31)][kof]);
            const half8 b0 = *reinterpret_cast<const half8*>(&Bs[wn * 64 + (lane & 31)][kof]);
            const half8 b1 = *reinterpret_cast<const half8*>(&Bs[wn * 64 + 32 + (lane & 31)][kof]);
            acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b0, acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b1, acc1, 0, 0, 0);
        }
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int m = wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < mcount) {
            const int s = slot_s[m];
            const float sc = slot_w[m];
            float* dst = is_sh ? ysh : y;
            const int oa = n0 + wn * 64 + (lane & 31);
            if (oa < H) dst[(size_t)s * H + oa] = acc0[v] * sc;
            if (oa + 32 < H) dst[(size_t)s * H + oa + 32] = acc1[v] * sc;
        }
    }
}

__global__ void __launch_bounds__(256)
x_to_f16_kernel(const float* __restrict__ x, _Float16* __restrict__ x16, size_t n4) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const float4 v = reinterpret_cast<const float4*>(x)[i];
    typedef _Float16 half4 __attribute__((ext_vector_type(4)));
    half4 h;
    h[0] = (_Float16)v.x;
    h[1] = (_Float16)v.y;
    h[2] = (_Float16)v.z;
    h[3] = (_Float16)v.w;
    reinterpret_cast<half4*>(x16)[i] = h;
}

// out[t] = ((y[t,0] + y[t,1]) + ... + y[t,k-1]) + ysh[t]; y rows already carry
// their routing weight, ysh the shared weight.  Slots whose expert index is
// out of range contribute nothing.
__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ y, const float* __restrict__ ysh,
               const int32_t* __restrict__ idx, int T, int H, int E, int k, int has_shared,
               float* __restrict__ out) {
    const int h4 = H / 4;
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (size_t)T * h4) return;
    const int t = (int)(i / h4), o4 = (int)(i % h4);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
        if ((unsigned)idx[(size_t)t * k + j] >= (unsigned)E) continue;
        const float4 v = reinterpret_cast<const float4*>(y + ((size_t)t * k + j) * H)[o4];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    if (has_shared) {
        const float4 v = reinterpret_cast<const float4*>(ysh + (size_t)t * H)[o4];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    reinterpret_cast<float4*>(out + (size_t)t * H)[o4] = acc;
}

hipError_t launch_mfma(const moe_layer_desc& d, const float* x, int T, const int32_t* idx,
                       const float* w, int shard, int nshards, float* out, char* ws,
                       const WsLayout& L, const Ctx& c) {
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

    const size_t n4 = (size_t)T * H / 4;
    launch_k(c, MOE_K_X_F16, x_to_f16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, x,
             x16, n4);
    hipError_t err = launch_bucket(idx, T, k, E, shared, counts, offsets, tile_off, perm, bhist, c);
    if (err != hipSuccess) return err;
    // an upper bound on the number of tiles; blocks past the real count exit
    const int max_tiles = (T * k + kTileM - 1) / kTileM + E + (shared ? (T + kTileM - 1) / kTileM : 0);
    const int Imax = (d.inter > d.shared_inter ? d.inter : d.shared_inter) / nshards;
    launch_k(c, MOE_K_GEMM_GATEUP, gemm_gateup_kernel, dim3(max_tiles, (Imax + 63) / 64), dim3(256),
             0, x16, T, H, perm, offsets, tile_off, E, k, d.gate_q, d.up_q, d.sh_gate_q, d.sh_up_q,
             d.inter, d.shared_inter, shard, nshards, h16, Iloc);
    launch_k(c, MOE_K_GEMM_DOWN, gemm_down_kernel, dim3(max_tiles, (H + 127) / 128), dim3(256), 0,
             h16, Iloc, T, H, perm, offsets, tile_off, E, k, d.down_q, d.sh_down_q, d.inter,
             d.shared_inter, shard, nshards, w, d.shared_weight, y, ysh);
    const size_t nc = (size_t)T * H / 4;
    launch_k(c, MOE_K_COMBINE, combine_kernel, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, y,
             ysh, idx, T, H, E, k, shared ? 1 : 0, out);
    return hipGetLastError();
}

}  // namespace moe
