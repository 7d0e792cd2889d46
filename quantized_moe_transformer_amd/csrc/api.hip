// api.hip -- the C ABI of libmoe_hip.so: argument checks, workspace layout,
// path choice and kernel launches.  The entry points are declared (with their
// contracts) in include/moe.h.
#include <string.h>

#include <atomic>
#include <mutex>

#include "launch.h"

namespace moe {

// ---------------------------------------------------------------------------
// small kernels: dequant test hook and shard-partial reduction
// ---------------------------------------------------------------------------

// One workgroup (256 threads) per superblock, thread i decodes element i:
// element 64c+l is the low nibble of qs[32c+l], 64c+32+l its high nibble;
// the 5-bit format adds 16 * bit (2c or 2c+1) of qh[l]; MXFP4 reads the code
// as E2M1 and scales it by its sub-block's E8M0 byte.
__global__ void __launch_bounds__(256)
dequant_kernel(const uint8_t* __restrict__ sbs, int bits, int64_t n_sb, int out_dtype,
               void* __restrict__ out) {
    const int i = threadIdx.x;
    const int c = i >> 6, r = i & 63, l = r & 31, upper = r >> 5;
    const int sbb = bits == 5 ? kQ5Bytes : kQ4Bytes;   // Q4_K and MXFP4: 144 bytes
    for (int64_t b = blockIdx.x; b < n_sb; b += gridDim.x) {
        const uint8_t* sb = sbs + b * sbb;
        const uint8_t* qs = sb + (bits == 5 ? 48 : 16);
        const uint32_t byte = qs[32 * c + l];
        uint32_t q = upper ? (byte >> 4) : (byte & 15u);
        float wv;
        if (bits == MOE_SB_MXFP4) {
            // MXFP4: the code's value times its sub-block's power of two
            wv = e2m1_f32(q) * e8m0_f32(sb[i >> 5]);
        } else {
            const SbHead hd = load_head(sb);
            float sc, m;
            sub_scale_min(hd, i >> 5, sc, m);
            if (bits == 5) q |= ((uint32_t)(sb[16 + l] >> (2 * c + upper)) & 1u) << 4;
            wv = kq_weight(hd.d * sc, hd.dmin * m, (float)q);
        }
        const int64_t o = b * kSbWeights + i;
        if (out_dtype == 0)
            reinterpret_cast<float*>(out)[o] = wv;
        else if (out_dtype == 1)
            reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_rne(wv);
        else
            reinterpret_cast<_Float16*>(out)[o] = (_Float16)wv;
    }
}

// fp16 output of the K-quant formats: one thread per 16-byte code piece
// (superblock b, sub-block pair c, half hh), through kq_piece_f16 -- the very
// function whose results the grouped GEMM's producer waves store as matrix-core
// operands -- written to elements 64c + 16hh + [0,16) and 64c + 32 + 16hh +
// [0,16) of the superblock.
template <bool HIGH>
__global__ void __launch_bounds__(256)
dequant_f16_kernel(const uint8_t* __restrict__ sbs, int64_t n_pieces,
                   _Float16* __restrict__ out) {
    constexpr int SBB = HIGH ? kQ5Bytes : kQ4Bytes;
    for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < n_pieces;
         p += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = p >> 3;
        const int c = (int)(p >> 1) & 3, hh = (int)p & 1;
        const uint8_t* sb = sbs + b * SBB;
        const SbHead hd = load_head(sb);
        const uint4 qs = *reinterpret_cast<const uint4*>(sb + (HIGH ? 48 : 16) + 32 * c + 16 * hh);
        const uint4 qh = HIGH ? *reinterpret_cast<const uint4*>(sb + 16 + 16 * hh) : qs;
        uint32_t lo[8], hi[8];
        kq_piece_f16<HIGH>(hd, qs, qh, c, lo, hi);
        _Float16* row = out + b * kSbWeights + 64 * c;
        uint4* d0 = reinterpret_cast<uint4*>(row + 16 * hh);
        uint4* d1 = reinterpret_cast<uint4*>(row + 32 + 16 * hh);
        d0[0] = uint4{lo[0], lo[1], lo[2], lo[3]};
        d0[1] = uint4{lo[4], lo[5], lo[6], lo[7]};
        d1[0] = uint4{hi[0], hi[1], hi[2], hi[3]};
        d1[1] = uint4{hi[4], hi[5], hi[6], hi[7]};
    }
}

struct PartialPtrs {
    const float* p[16];
};

// out = ((p0 + p1) + p2) + ... [+ residual]: ascending shard order, then the
// residual (page "CKE Zip: From Splitting Tokens To Splitting Qwen3.5
// Weights", section "What PR #382 Now Splits": the partials are reduced and
// the block completes its residual), fp32.
__global__ void __launch_bounds__(256)
reduce4_kernel(PartialPtrs ps, int n, size_t n4, const float* __restrict__ res,
               float* __restrict__ out) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    float4 acc = reinterpret_cast<const float4*>(ps.p[0])[i];
    for (int s = 1; s < n; ++s) {
        const float4 v = reinterpret_cast<const float4*>(ps.p[s])[i];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    if (res) {
        const float4 v = reinterpret_cast<const float4*>(res)[i];
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    reinterpret_cast<float4*>(out)[i] = acc;
}

__global__ void __launch_bounds__(256)
reduce1_kernel(PartialPtrs ps, int n, size_t count, const float* __restrict__ res,
               float* __restrict__ out) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    float acc = ps.p[0][i];
    for (int s = 1; s < n; ++s) acc += ps.p[s][i];
    if (res) acc += res[i];
    out[i] = acc;
}

hipError_t launch_reduce(const float* const* partials, int n, int64_t count, const float* res,
                         float* out, hipStream_t s) {
    PartialPtrs ps = {};
    bool vec = (count % 4) == 0 && ((uintptr_t)out & 15) == 0 && ((uintptr_t)res & 15) == 0;
    for (int i = 0; i < n; ++i) {
        ps.p[i] = partials[i];
        vec = vec && (((uintptr_t)partials[i] & 15) == 0);
    }
    if (vec) {
        const size_t n4 = (size_t)count / 4;
        reduce4_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(ps, n, n4, res, out);
    } else {
        reduce1_kernel<<<(unsigned)((count + 255) / 256), 256, 0, s>>>(ps, n, (size_t)count, res,
                                                                      out);
    }
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* sbs, int bits, int64_t n_sb, int out_dtype, void* out,
                          hipStream_t s) {
    if (out_dtype == 2 && bits != MOE_SB_MXFP4) {
        const int64_t n_pieces = n_sb * 8;
        const int64_t nb = (n_pieces + 255) / 256;
        const unsigned blocks = (unsigned)(nb < 65536 ? nb : 65536);
        if (bits == 5)
            dequant_f16_kernel<true><<<blocks, 256, 0, s>>>(sbs, n_pieces, (_Float16*)out);
        else
            dequant_f16_kernel<false><<<blocks, 256, 0, s>>>(sbs, n_pieces, (_Float16*)out);
        return hipGetLastError();
    }
    const int64_t blocks = n_sb < 65536 ? n_sb : 65536;
    dequant_kernel<<<(unsigned)blocks, 256, 0, s>>>(sbs, bits, n_sb, out_dtype, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// workspace layout
// ---------------------------------------------------------------------------

static inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(const moe_layer_desc& d, int T, int iloc) {
    WsLayout L = {};
    const size_t H = d.hidden, E = d.n_experts, k = d.top_k;
    const size_t Tz = T;
    const size_t Iloc = (size_t)iloc;
    const size_t nslot = k + (d.shared_inter > 0 ? 1 : 0);
    size_t off = 0;
    L.router_ks = router_splits(T);
    L.router_part = off;  off = align256(off + (size_t)L.router_ks * Tz * E * 4);
    const bool big = T > kRouterSmallMaxT;
    L.x_lo = off;         off = align256(off + (big ? Tz * H * 2 : 0));
    L.w_hi = off;         off = align256(off + (big ? E * H * 2 : 0));
    L.w_lo = off;         off = align256(off + (big ? E * H * 2 : 0));
    L.idx = off;          off = align256(off + Tz * k * 4);
    L.w = off;            off = align256(off + Tz * k * 4);
    const size_t base = off;
    L.hbuf = base;
    const size_t gemv_end = align256(base + Tz * nslot * Iloc * 4);
    off = base;
    L.x16 = off;          off = align256(off + Tz * H * 2);
    L.bhist = off;        off = align256(off + (size_t)bucket_blocks(T, (int)k) * E * 4);
    L.counts = off;       off = align256(off + (E + 1) * 4);
    L.offsets = off;      off = align256(off + (E + 2) * 4);
    L.tile_off = off;     off = align256(off + (E + 3) * 4);
    L.tile_rec = off;     off = align256(off + (size_t)max_row_tiles(T, (int)k, (int)E, d.shared_inter > 0) * 16);
    L.perm = off;         off = align256(off + Tz * k * 4);
    const size_t hrows = Tz * k + Tz;
    if (d.weight_format == MOE_WFMT_MXFP4) {
        L.mx_xq = off;    off = align256(off + (size_t)kMxTerms * Tz * H);
        L.mx_xs = off;    off = align256(off + Tz * (H / 64) * 16);
        L.mx_hq = off;    off = align256(off + (size_t)kMxTerms * hrows * Iloc);
        L.mx_hs = off;    off = align256(off + hrows * (Iloc / 64) * 16);
    } else {
        L.h16 = off;      off = align256(off + hrows * Iloc * 2);
    }
    L.y = off;            off = align256(off + Tz * k * H * 2);
    L.ysh = off;          off = align256(off + Tz * H * 2);
    L.ysc = off;          off = align256(off + Tz * k * (H / 8));
    L.yshsc = off;        off = align256(off + Tz * (H / 8));
    L.total = gemv_end > off ? gemv_end : off;
    return L;
}

// ---------------------------------------------------------------------------
// checks
// ---------------------------------------------------------------------------

static inline bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }

static int check_desc(const moe_layer_desc* d) {
    if (!d) return MOE_EINVAL;
    if (d->hidden <= 0 || d->n_experts <= 0 || d->top_k < 1 || d->inter <= 0 || d->shared_inter < 0)
        return MOE_EINVAL;
    if (d->n_experts > 1024) return MOE_EUNSUPPORTED;
    if (d->top_k > 16 || d->top_k > d->n_experts) return MOE_EINVAL;
    if (!d->router_w || !d->gate_q || !d->up_q || !d->down_q) return MOE_EINVAL;
    if (d->shared_inter > 0 && (!d->sh_gate_q || !d->sh_up_q || !d->sh_down_q)) return MOE_EINVAL;
    if (d->weight_format != MOE_WFMT_KQUANT && d->weight_format != MOE_WFMT_MXFP4) return MOE_EINVAL;
    const int nsb = d->hidden / kSbWeights;
    if (d->hidden % kSbWeights || !(nsb == 1 || nsb == 2 || nsb == 4 || nsb == 8 || nsb == 16))
        return MOE_EUNSUPPORTED;
    if (d->inter % 64) return MOE_EUNSUPPORTED;
    if (d->shared_inter != 0 && d->shared_inter != d->inter) return MOE_EUNSUPPORTED;
    if (!al16(d->router_w) || !al16(d->gate_q) || !al16(d->up_q) || !al16(d->down_q))
        return MOE_EUNSUPPORTED;
    if (d->shared_inter > 0 && (!al16(d->sh_gate_q) || !al16(d->sh_up_q) || !al16(d->sh_down_q)))
        return MOE_EUNSUPPORTED;
    return MOE_OK;
}

// Automatic path: the GEMV path up to this many token rows, the grouped GEMM
// beyond, per weight format.  Measured on the Qwen3.5-35B-A3B-shaped layer
// (uniform routing, HIP-graph replay, one MI355X): K-quant GEMV 122.9 us vs
// GEMM 135.0 us at 16 rows, 138.1 vs 137.2 at 18, 150.4 vs 139.0 at 20;
// MXFP4 159.0 vs 164.6 at 26 rows, 169.6 vs 165.5 at 28.  The GEMV cost grows
// by about 6 us per row (each row streams its own experts) while the GEMM
// reads each touched expert once per column tile.
constexpr int kGemvMaxT = 17;     // K-quant
constexpr int kGemvMaxTMx = 26;   // MXFP4

static bool gemv_supports(int iloc) { return iloc >= 64 && iloc <= 2048 && iloc % 64 == 0; }

static int choose_path(int T, int iloc, int fmt, const moe_opts* o, int* path) {
    const int req = o ? o->path : MOE_PATH_AUTO;
    if (req == MOE_PATH_GEMV) {
        if (!gemv_supports(iloc)) return MOE_EUNSUPPORTED;
        *path = MOE_PATH_GEMV;
    } else if (req == MOE_PATH_MFMA) {
        *path = MOE_PATH_MFMA;
    } else if (req == MOE_PATH_AUTO) {
        const int tmax = fmt == MOE_WFMT_MXFP4 ? kGemvMaxTMx : kGemvMaxT;
        *path = (T <= tmax && gemv_supports(iloc)) ? MOE_PATH_GEMV : MOE_PATH_MFMA;
    } else {
        return MOE_EINVAL;
    }
    return MOE_OK;
}

constexpr int kMaxDevices = 64;

// gfx950 check of the current device, remembered per device ordinal (0
// unknown, 1 gfx950, 2 not).  Two threads that race on a first check store
// the same value.
static std::atomic<int> g_device_kind[kMaxDevices];

static int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ENODEVICE;
    const bool slot = dev >= 0 && dev < kMaxDevices;
    const int known = slot ? g_device_kind[dev].load(std::memory_order_relaxed) : 0;
    if (known) return known == 1 ? MOE_OK : MOE_ENODEVICE;
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return MOE_ENODEVICE;
    const bool ok = strncmp(p.gcnArchName, "gfx950", 6) == 0;
    if (slot) g_device_kind[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? MOE_OK : MOE_ENODEVICE;
}

// ---------------------------------------------------------------------------
// The fixed scratch of moe_layer_forward_noalloc: a file-scope device array,
// one copy per device at that device's own address.  In host code `scratch`
// names only a host-side stand-in; the device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is ever handed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch keeps the workspace alignment");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::atomic<void*> g_scratch[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of the current device's scratch (set up on its first use).
static int scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ENODEVICE;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();   // clear the error it left
                return MOE_ELAUNCH;
            }
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MOE_OK;
}

static int launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ELAUNCH; }

}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_EUNSUPPORTED: return "unsupported shape or alignment";
        case MOE_EWORKSPACE: return "workspace too small";
        case MOE_ELAUNCH: return "kernel launch failed";
        case MOE_ENODEVICE: return "no gfx950 device";
        case MOE_ETOOBIG: return "input too large for the no-allocation scratch";
        default: return "unknown status";
    }
}

size_t moe_workspace_bytes(const moe_layer_desc* desc, int32_t T, int32_t num_shards) {
    if (check_desc(desc) != MOE_OK || T < 0 || num_shards < 1 || num_shards > 16) return 0;
    if (desc->inter % num_shards) return 0;
    return ws_layout(*desc, T, desc->inter / num_shards).total;
}

int router_topk(const moe_layer_desc* desc, const float* x, int32_t T, int32_t* topk_idx,
                float* topk_w, void* ws, size_t ws_bytes, void* stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (T < 0) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x || !topk_idx || !topk_w || !ws) return MOE_EINVAL;
    const WsLayout L = ws_layout(*desc, T, desc->inter);
    if (ws_bytes < L.total) return MOE_EWORKSPACE;
    if ((uintptr_t)ws & 255) return MOE_EUNSUPPORTED;
    if ((rc = check_device())) return rc;
    Ctx c;
    c.s = (hipStream_t)stream;
    return launched(launch_router(*desc, x, T, topk_idx, topk_w, (char*)ws, L, c));
}

// i0, iloc: intermediate rows [i0, i0 + iloc) of every expert, already
// checked against the descriptor (multiples of 64 inside [0, I))
static int forward_common(const moe_layer_desc* desc, const float* x, int32_t T,
                          const int32_t* idx, const float* w, int i0, int iloc, float* out,
                          const moe_opts* opts, void* ws, size_t ws_bytes, void* stream,
                          bool route) {
    int rc;
    if (T < 0) return MOE_EINVAL;
    int path = 0;
    if ((rc = choose_path(T, iloc, desc->weight_format, opts, &path))) return rc;
    if (opts && opts->path_used) *opts->path_used = path;
    if (T == 0) return MOE_OK;
    if (!x || !out || !ws || (!route && (!idx || !w))) return MOE_EINVAL;
    if (!al16(x) || !al16(out) || ((uintptr_t)ws & 255)) return MOE_EUNSUPPORTED;
    const WsLayout L = ws_layout(*desc, T, iloc);
    if (ws_bytes < L.total) return MOE_EWORKSPACE;
    if ((rc = check_device())) return rc;
    char* wsp = (char*)ws;
    Ctx c;
    c.s = (hipStream_t)stream;
    if (opts && opts->kernel_events && opts->n_kernel_events > 0) {
        c.ev = opts->kernel_events;
        c.n_ev = opts->n_kernel_events;
    }
    if (path == MOE_PATH_GEMV)
        return launched(launch_gemv(*desc, x, T, idx, w, i0, iloc, out, wsp, L, c, route));
    if (route) {
        int32_t* ridx = reinterpret_cast<int32_t*>(wsp + L.idx);
        float* rw = reinterpret_cast<float*>(wsp + L.w);
        // many slots: the top-k also makes the bucketing's per-block counts
        // (only the matrix-core router's top-k can; the few-row router never
        // meets this case, since T <= kRouterSmallMaxT slots bucket in one block)
        int32_t* hb = (T <= kRouterSmallMaxT || bucket_self(T, desc->top_k, desc->n_experts))
                          ? nullptr
                          : reinterpret_cast<int32_t*>(wsp + L.bhist);
        if (launch_router_hist(*desc, x, T, ridx, rw, wsp, L, c, hb) != hipSuccess)
            return MOE_ELAUNCH;
        c.hist_ready = hb != nullptr;
        idx = ridx;
        w = rw;
    }
    if (desc->weight_format == MOE_WFMT_MXFP4)
        return launched(launch_mfma_mx(*desc, x, T, idx, w, i0, iloc, out, wsp, L, c));
    return launched(launch_mfma(*desc, x, T, idx, w, i0, iloc, out, wsp, L, c,
                                route && T > kRouterSmallMaxT));
}

int moe_layer_forward(const moe_layer_desc* desc, const float* x, int32_t T, float* out,
                      const moe_opts* opts, void* ws, size_t ws_bytes, void* stream) {
    const int rc = check_desc(desc);
    if (rc) return rc;
    return forward_common(desc, x, T, nullptr, nullptr, 0, desc->inter, out, opts, ws, ws_bytes,
                          stream, true);
}

int moe_layer_forward_noalloc(const moe_layer_desc* desc, const float* x, int32_t T, float* out,
                              const moe_opts* opts, void* stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (T < 0) return MOE_EINVAL;
    if (T == 0)   // nothing to enqueue: the scratch is not touched
        return forward_common(desc, x, T, nullptr, nullptr, 0, desc->inter, out, opts, nullptr, 0,
                              stream, true);
    if (ws_layout(*desc, T, desc->inter).total > kScratchBytes) return MOE_ETOOBIG;
    if ((rc = check_device())) return rc;
    void* ws = nullptr;
    if ((rc = scratch_address(&ws))) return rc;
    return forward_common(desc, x, T, nullptr, nullptr, 0, desc->inter, out, opts, ws,
                          kScratchBytes, stream, true);
}

int moe_layer_forward_shard(const moe_layer_desc* desc, const float* x, int32_t T,
                            const int32_t* topk_idx, const float* topk_w, int32_t shard,
                            int32_t num_shards, float* partial, const moe_opts* opts, void* ws,
                            size_t ws_bytes, void* stream) {
    const int rc = check_desc(desc);
    if (rc) return rc;
    if (num_shards < 1 || num_shards > 16 || shard < 0 || shard >= num_shards) return MOE_EINVAL;
    if (desc->inter % num_shards || (desc->inter / num_shards) % 64) return MOE_EUNSUPPORTED;
    const int iloc = desc->inter / num_shards;
    return forward_common(desc, x, T, topk_idx, topk_w, shard * iloc, iloc, partial, opts, ws,
                          ws_bytes, stream, false);
}

int moe_layer_forward_range(const moe_layer_desc* desc, const float* x, int32_t T,
                            const int32_t* topk_idx, const float* topk_w, int32_t i_begin,
                            int32_t i_end, float* partial, const moe_opts* opts, void* ws,
                            size_t ws_bytes, void* stream) {
    const int rc = check_desc(desc);
    if (rc) return rc;
    if (i_begin < 0 || i_end <= i_begin || i_end > desc->inter) return MOE_EINVAL;
    if (i_begin % 64 || i_end % 64) return MOE_EUNSUPPORTED;
    return forward_common(desc, x, T, topk_idx, topk_w, i_begin, i_end - i_begin, partial, opts,
                          ws, ws_bytes, stream, false);
}

int moe_reduce_partials(const float* const* partials, int32_t num_shards, int64_t n_elems,
                        float* out, void* stream) {
    if (!partials || num_shards < 1 || num_shards > 16 || n_elems < 0) return MOE_EINVAL;
    if (n_elems == 0) return MOE_OK;
    if (!out) return MOE_EINVAL;
    for (int i = 0; i < num_shards; ++i)
        if (!partials[i]) return MOE_EINVAL;
    int rc = check_device();
    if (rc) return rc;
    return launched(launch_reduce(partials, num_shards, n_elems, nullptr, out, (hipStream_t)stream));
}

int moe_reduce_residual(const float* const* partials, int32_t num_shards, int64_t n_elems,
                        const float* residual, float* out, void* stream) {
    if (!partials || num_shards < 1 || num_shards > 16 || n_elems < 0) return MOE_EINVAL;
    if (n_elems == 0) return MOE_OK;
    if (!out || !residual) return MOE_EINVAL;
    for (int i = 0; i < num_shards; ++i)
        if (!partials[i]) return MOE_EINVAL;
    int rc = check_device();
    if (rc) return rc;
    return launched(launch_reduce(partials, num_shards, n_elems, residual, out, (hipStream_t)stream));
}

static bool norm_shape_ok(int cols, int64_t ld, const void* p) {
    return cols % 4 == 0 && ld % 4 == 0 && ld >= cols && al16(p);
}

int moe_rmsnorm(const float* x, int32_t T, int32_t H, const float* g, float eps, float* y,
                void* stream) {
    if (T < 0 || H < 1 || !(eps >= 0.f) || eps > 3.0e38f) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x || !g || !y) return MOE_EINVAL;
    if (!norm_shape_ok(H, H, x) || !al16(g) || !al16(y)) return MOE_EUNSUPPORTED;
    int rc = check_device();
    if (rc) return rc;
    return launched(launch_rmsnorm(x, T, H, H, nullptr, 0, H, g, eps, y, H, (hipStream_t)stream));
}

int moe_rmsnorm_sumsq(const float* x, int32_t T, int32_t cols, int64_t ldx, float* ssq,
                      void* stream) {
    if (T < 0 || cols < 1) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x || !ssq) return MOE_EINVAL;
    if (!norm_shape_ok(cols, ldx, x)) return MOE_EUNSUPPORTED;
    int rc = check_device();
    if (rc) return rc;
    return launched(launch_rmsnorm_sumsq(x, T, cols, ldx, ssq, (hipStream_t)stream));
}

int moe_rmsnorm_apply(const float* x, int32_t T, int32_t cols, int64_t ldx,
                      const float* const* ssq_parts, int32_t n_parts, int32_t H, const float* g,
                      float eps, float* y, int64_t ldy, void* stream) {
    if (T < 0 || cols < 1 || H < cols || n_parts < 1 || n_parts > 16 || !(eps >= 0.f) ||
        eps > 3.0e38f)
        return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!x || !g || !y || !ssq_parts) return MOE_EINVAL;
    for (int i = 0; i < n_parts; ++i)
        if (!ssq_parts[i]) return MOE_EINVAL;
    if (!norm_shape_ok(cols, ldx, x) || !norm_shape_ok(cols, ldy, y) || !al16(g))
        return MOE_EUNSUPPORTED;
    int rc = check_device();
    if (rc) return rc;
    return launched(launch_rmsnorm(x, T, cols, ldx, ssq_parts, n_parts, H, g, eps, y, ldy,
                                   (hipStream_t)stream));
}

int moe_dequant(const uint8_t* sbs, int32_t bits, int64_t n_sb, int32_t out_dtype, void* out,
                void* stream) {
    if ((bits != 4 && bits != 5 && bits != MOE_SB_MXFP4) || n_sb < 0 || out_dtype < 0 ||
        out_dtype > 2)
        return MOE_EINVAL;
    if (n_sb == 0) return MOE_OK;
    if (!sbs || !out) return MOE_EINVAL;
    if (!al16(sbs)) return MOE_EUNSUPPORTED;
    int rc = check_device();
    if (rc) return rc;
    return launched(launch_dequant(sbs, bits, n_sb, out_dtype, out, (hipStream_t)stream));
}

int moe_route_bucket(const moe_layer_desc* desc, const int32_t* topk_idx, int32_t T,
                     int32_t* counts, int32_t* offsets, int32_t* perm, void* ws, size_t ws_bytes,
                     void* stream) {
    int rc = check_desc(desc);
    if (rc) return rc;
    if (T < 0) return MOE_EINVAL;
    if (T == 0) return MOE_OK;
    if (!topk_idx || !counts || !offsets || !perm || !ws) return MOE_EINVAL;
    if ((uintptr_t)ws & 255) return MOE_EUNSUPPORTED;
    const WsLayout L = ws_layout(*desc, T, desc->inter);
    if (ws_bytes < L.total) return MOE_EWORKSPACE;
    if ((rc = check_device())) return rc;
    hipStream_t s = (hipStream_t)stream;
    Ctx c;
    c.s = s;
    char* wsp = (char*)ws;
    int32_t* wc = reinterpret_cast<int32_t*>(wsp + L.counts);
    int32_t* wo = reinterpret_cast<int32_t*>(wsp + L.offsets);
    int32_t* wt = reinterpret_cast<int32_t*>(wsp + L.tile_off);
    int4* wr = reinterpret_cast<int4*>(wsp + L.tile_rec);
    int32_t* bh = reinterpret_cast<int32_t*>(wsp + L.bhist);
    if (launch_bucket(topk_idx, T, desc->top_k, desc->n_experts, desc->shared_inter > 0, wc, wo,
                      wt, wr, perm, bh, c) != hipSuccess)
        return MOE_ELAUNCH;
    const size_t E = desc->n_experts;
    if (hipMemcpyAsync(counts, wc, E * 4, hipMemcpyDeviceToDevice, s) != hipSuccess ||
        hipMemcpyAsync(offsets, wo, (E + 1) * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
        return MOE_ELAUNCH;
    return MOE_OK;
}

}  // extern "C"
