/*
 * moe.h -- C ABI of the MI355X (gfx950) routed Mixture-of-Experts layer library
 *          (libmoe_hip.so).
 *
 * One routed MoE layer shaped like the Qwen3.5-35B-A3B layer of the page
 * "CKE Zip: From Splitting Tokens To Splitting Qwen3.5 Weights":
 *   - an fp32 router, softmax and top-k of E experts (section "What PR #382
 *     Now Splits": 256 routed experts, eight selected per token);
 *   - per selected expert a 4-bit K-quant (Q4_K) gate/up projection, SwiGLU
 *     and a 5-bit K-quant (Q5_K) down projection, scaled by the routing
 *     weight and merged in selected-slot order (section "A Separate Decode
 *     Result Shows Why Axis Choice Matters");
 *   - an always-on shared expert (section "What The First Prototype Split":
 *     the remote runs "the routed and shared SwiGLU branches");
 *   - a sharded mode in which the intermediate dimension of every routed and
 *     of the shared expert is split into shards, each yielding a hidden-sized
 *     partial; the partials add up to the whole (section "What PR #382 Now
 *     Splits"; page "Distributed CPU: Zip Fusion Beyond Tensor Parallelism",
 *     section "What Must Cross the Fabric: The Reduction Algebra").
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers unless stated otherwise; `stream`
 *     is a hipStream_t (NULL = the default stream).  All work is enqueued on
 *     `stream`; nothing synchronises the host.  Results are valid once the
 *     caller has synchronised the stream.
 *   - The caller owns every buffer, including the workspace
 *     (moe_layer_forward_noalloc uses the library's fixed scratch instead).
 *     The library allocates and frees nothing and keeps no pointer after
 *     returning.
 *   - Every argument is checked before anything is enqueued: on an error
 *     nothing runs and outputs are untouched.  Device faults surface at the
 *     caller's next synchronisation.  No exceptions cross the ABI.
 *   - T = 0 is valid and enqueues nothing.  Outputs are overwritten, never
 *     accumulated into.  Inputs must not alias outputs.
 *   - Identical inputs give bit-identical outputs (fixed reduction orders, no
 *     floating-point atomics).  Calls on different streams with different
 *     workspaces may overlap.  The library's only global state is a per-device
 *     record of its gfx950 check (set once, thread-safe) and the fixed scratch
 *     of moe_layer_forward_noalloc (one per device; see there).
 *
 * Weight format (a reading: the pages name Q4_K/Q5_K but print no layout)
 *   A superblock holds 256 weights, in 8 sub-blocks of 32:
 *     Q4_K, 144 bytes: fp16 d | fp16 dmin | 12 bytes scales | 128 bytes qs
 *     Q5_K, 176 bytes: fp16 d | fp16 dmin | 12 bytes scales | 32 bytes qh | 128 bytes qs
 *   Sub-block j has a 6-bit scale sc_j and min m_j: for j < 4 the low six
 *   bits of scales[j] and scales[j+4]; for j >= 4 the low/high nibble of
 *   scales[j+4] with the top two bits of scales[j-4] / scales[j] above them.
 *   Element 64c+l (c < 4, l < 32) is the low nibble of qs[32c+l], element
 *   64c+32+l its high nibble; Q5_K adds 16 * bit (2c) resp. (2c+1) of qh[l].
 *   w = d*sc_j*q - dmin*m_j.
 *   A matrix is stored one row per output feature with the reduction
 *   dimension K contiguous, its flat row-major array cut into superblocks
 *   (a superblock may hold several rows when K < 256).
 *
 * Second weight format, MXFP4 (moe_layer_desc.weight_format = MOE_WFMT_MXFP4;
 * the page "Distributed CPU: Zip Fusion Beyond Tensor Parallelism", section
 * "Decode vs Prefill: Same Weights, Different Bottlenecks", says the model
 * class targeted ships an MXFP4-class format; the encodings are those of the
 * OCP Microscaling formats v1.0, the byte layout is this library's):
 *     MXFP4, 144 bytes: 8 bytes E8M0 scales | 8 bytes reserved | 128 bytes qs
 *   Sub-block j (32 weights) has the scale X_j = 2^(scales[j] - 127); codes
 *   are FP4 E2M1 (bit 3 sign, bits 2..1 exponent e with bias 1, bit 0
 *   mantissa m: e = 0 gives m/2, else 2^(e-1) * (1 + m/2)) in the nibble
 *   order above; w = X_j * value(code).  Gate, up and down (and the shared
 *   expert) all use it; every matrix has I*H/256 superblocks of 144 bytes.
 *   The fp32 GEMV path decodes exactly for scale bytes 2..254 (smaller ones
 *   give fp32 subnormals, larger products overflow to inf).  The MFMA path
 *   hands codes and scales to gfx950's block-scaled matrix cores unchanged, so
 *   every scale byte 0..254 applies exactly (255, the format's NaN, gives
 *   NaN); its tokens and SwiGLU outputs enter as the sum of three MX-FP8
 *   (e4m3) terms with an E8M0 scale per 32 values, which represents each value
 *   to within 2^-12 of its 32-value block's largest magnitude.
 */
#ifndef MOE_HIP_H
#define MOE_HIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 6

/* Status codes returned by every entry point. */
#define MOE_OK 0
#define MOE_EINVAL (-1)        /* null pointer, negative size, k not in [1, min(E,16)], shard not in [0,n) */
#define MOE_EUNSUPPORTED (-2)  /* shape or alignment outside what the kernels handle (see below) */
#define MOE_EWORKSPACE (-3)    /* workspace smaller than moe_workspace_bytes() */
#define MOE_ELAUNCH (-4)       /* a kernel launch failed (hipGetLastError) */
#define MOE_ENODEVICE (-5)     /* no gfx950 device is current */
#define MOE_ETOOBIG (-6)       /* moe_layer_forward_noalloc: T rows need more than its fixed scratch */

/* Weight formats (moe_layer_desc.weight_format). */
#define MOE_WFMT_KQUANT 0      /* Q4_K gate/up, Q5_K down */
#define MOE_WFMT_MXFP4 1       /* MXFP4 gate, up and down */

/* Compute paths (moe_opts.path). */
#define MOE_PATH_AUTO 0        /* GEMV for T <= 17 (MXFP4: T <= 26), grouped MFMA GEMM above
                                  (measured crossovers) */
#define MOE_PATH_GEMV 1        /* fp32 dequant-GEMV, fp32 accumulation */
#define MOE_PATH_MFMA 2        /* grouped GEMM on the matrix cores, fp32 accumulation: fp16
                                  operands (K-quant), block-scaled MX operands (MXFP4) */
/*
 * The K-quant MFMA path rounds the tokens, the weights and h to fp16 once each.
 * Its error against an exact evaluation depends on the layer: 2.9e-3 and
 * 4.9e-3 of the output RMS on the Qwen3.5-shaped layer (T = 4096, and a Zipf
 * batch of 512), but about 2e-2 on a layer as small as H = 256 with I = 64,
 * where the tokens' rounding dominates.  MOE_PATH_GEMV keeps fp32 throughout.
 */
/*
 * The MFMA path hands each routed expert's weighted output row to the slot-order
 * combine as 16-bit block floating point: every 8 consecutive values share
 * their largest magnitude's fp32 exponent and keep 14 to 15 bits each, with
 * no range limit.  A group of 8 holding an inf or NaN reads back as 8 NaNs, so
 * a non-finite value in one expert's output turns the token's 8 outputs of
 * that column group to NaN (the GEMV path keeps fp32 rows throughout).
 */

/*
 * Layer description: plain values and device pointers, read during the call
 * only.
 *   hidden        H, a multiple of 256 with H/256 in {1, 2, 4} or H in {2048, 4096}
 *   n_experts     E, 1..1024
 *   top_k         k, 1..min(E, 16)
 *   inter         I, intermediate width of each routed expert, a multiple of 64
 *   shared_inter  Is, 0 (no shared expert) or equal to I
 *   shared_weight weight of the shared expert's output (1 in the Qwen3.5 layer)
 *   router_w      fp32 [H][E] row-major: logits = x . router_w
 *   gate_q, up_q  Q4_K, E consecutive matrices of [I rows][H] (I*H/256 superblocks each)
 *   down_q        Q5_K, E consecutive matrices of [H rows][I] (H*I/256 superblocks each)
 *   sh_gate_q, sh_up_q, sh_down_q  the shared expert, same formats, width Is
 *                 (may be NULL when Is = 0)
 *   weight_format MOE_WFMT_KQUANT (the formats above) or MOE_WFMT_MXFP4 (every
 *                 matrix in 144-byte MXFP4 superblocks); anything else: -1
 * Every weight pointer must be 16-byte aligned; router_w and token buffers
 * 16-byte aligned as well.
 */
typedef struct moe_layer_desc {
    int32_t hidden, n_experts, top_k, inter, shared_inter;
    float shared_weight;
    const float *router_w;
    const uint8_t *gate_q, *up_q, *down_q;
    const uint8_t *sh_gate_q, *sh_up_q, *sh_down_q;
    int32_t weight_format;
} moe_layer_desc;

/* Options.  `path` forces a compute path (MOE_PATH_*); `path_used`, a HOST
 * pointer that may be NULL, receives the path that ran.
 * `kernel_events` (HOST array of n_kernel_events hipEvent_t created by the
 * caller, may be NULL) times the kernels of a call: kernel id i (MOE_K_*) is
 * launched with hipExtLaunchKernel and events 2i / 2i+1 as its start / stop
 * events, so hipEventElapsedTime(ev[2i], ev[2i+1]) is that launch's own
 * duration.  Events of kernels the call does not launch are left untouched. */
typedef struct moe_opts {
    int32_t path;
    int32_t *path_used;
    void **kernel_events;
    int32_t n_kernel_events;
} moe_opts;

/* Kernel ids for moe_opts.kernel_events. */
#define MOE_K_GEMV_FRONT 0       /* T <= 32: router partial logits */
#define MOE_K_ROUTER_MFMA 1      /* T > 32: router logits on the matrix cores (split fp16, fp32-accurate) */
#define MOE_K_ROUTER_TOPK 2      /* top-k + weights */
#define MOE_K_GATEUP_GEMV 3      /* decode: top-k (when routing) + routed and shared gate/up
                                    + SwiGLU */
#define MOE_K_DOWN_GEMV 4        /* decode: down + slot-order combine */
#define MOE_K_X_F16 5            /* T > 32: tokens to fp16 hi/lo parts (and, when the router runs,
                                    the router matrix to fp16 hi/lo parts in the same launch) */
#define MOE_K_BUCKET_HIST 6      /* more than 8192 slots: per-1024-slot expert counts */
#define MOE_K_BUCKET_SCAN 7      /* not launched: the scan runs inside the sort (id kept) */
#define MOE_K_BUCKET_SCATTER 8   /* expert offsets, tile list and the slot order by expert */
#define MOE_K_GEMM_GATEUP 9      /* prefill: grouped GEMM gate/up + SwiGLU */
#define MOE_K_GEMM_DOWN 10       /* prefill: grouped GEMM down */
#define MOE_K_COMBINE 11         /* prefill: slot-order combine */
#define MOE_K_X_MX 12            /* prefill, MXFP4 weights: tokens to MX-FP8 terms */
#define MOE_K_COUNT 13

/* Bytes of device workspace that router_topk, moe_layer_forward and
 * moe_layer_forward_shard need for T token rows split into num_shards shards
 * (any path).  Host-only; needs no device.  Returns 0 for an invalid
 * description.  Its contents on entry do not matter (nothing is read before
 * the call writes it).  Calls that share one workspace must not overlap in
 * time. */
size_t moe_workspace_bytes(const moe_layer_desc *desc, int32_t T, int32_t num_shards);

/*
 * Router: logits[t][e] = sum_h x[t][h] * router_w[h][e] to fp32 accuracy (for
 * T > 32 on the matrix cores with each operand split into two fp16 parts,
 * which requires |x| < 65504 and |router_w| < 64: outside these limits the
 * affected logits, and so the routing of those rows, are wrong, and no status
 * says so, since the values are only on the device and no call synchronises;
 * the grouped GEMM of K-quant layers also takes x as fp16 and has the same
 * bound on |x|); the k largest
 * logits in descending order (ties to the lower expert index) become slots
 * 0..k-1 of topk_idx; topk_w[t][j] = softmax over all E logits of expert
 * topk_idx[t][j], renormalised over the k selected -- equal to the softmax of
 * the k selected logits alone.  (Page "CKE Zip ...", sections "What The First
 * Prototype Split" and "What PR #382 Now Splits": the top-k indices and their
 * routing weights are what the coordinator ships with each row, and the
 * synchronised router decision is what both shards consume.)
 *   x         fp32 [T][H]
 *   topk_idx  int32 [T][k] (output)
 *   topk_w    fp32 [T][k] (output)
 *   ws        device workspace of at least moe_workspace_bytes(desc, T, 1) bytes,
 *             256-byte aligned
 */
int router_topk(const moe_layer_desc *desc, const float *x, int32_t T,
                int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream);

/*
 * The whole layer: routing, then
 *   out[t] = sum_{j<k} topk_w[t][j] * FFN_{topk_idx[t][j]}(x[t]) + shared_weight * FFN_shared(x[t])
 * with FFN(x) = W_down (silu(W_gate x) * (W_up x)), summed in slot order and
 * the shared expert last.
 *   x    fp32 [T][H];  out fp32 [T][H]
 *   opts may be NULL (automatic path).
 */
int moe_layer_forward(const moe_layer_desc *desc, const float *x, int32_t T, float *out,
                      const moe_opts *opts, void *ws, size_t ws_bytes, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, kernels and results as moe_layer_forward, with no workspace
 * argument.  Its workspace is a fixed scratch array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes inside the library, one copy per device,
 * which each device that runs this call holds until the process ends.  The
 * call allocates and frees nothing; the caller still passes x and out.
 *   Returns MOE_ETOOBIG, enqueuing nothing, when T rows need more workspace
 *   than the scratch holds (moe_workspace_bytes(desc, T, 1) >
 *   MOE_NOALLOC_SCRATCH_BYTES: above 1106 rows of the Qwen3.5-shaped layer
 *   with K-quant weights, 913 with MXFP4; any T of the decode path fits).
 *   Other errors as moe_layer_forward.
 *   Every call on one device shares that device's scratch and leaves its last
 *   contents there (no call needs any particular contents on entry): calls
 *   that overlap in time on one device -- on different streams, or from
 *   different threads without ordering -- race and give undefined results.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_layer_forward_noalloc(const moe_layer_desc *desc, const float *x, int32_t T, float *out,
                              const moe_opts *opts, void *stream);

/*
 * Shard `shard` of `num_shards` of the layer, with the routing given (the
 * synchronised router decision, e.g. from router_topk): the same sum as
 * moe_layer_forward restricted to intermediate rows
 * [shard*I/num_shards, (shard+1)*I/num_shards) of every routed expert and
 * [shard*Is/num_shards, (shard+1)*Is/num_shards) of the shared one.  The
 * partials of all shards add up to the unsplit output (moe_reduce_partials).
 * Requires (I/num_shards) % 64 == 0.
 *   topk_idx int32 [T][k], topk_w fp32 [T][k] (device);  partial fp32 [T][H]
 */
int moe_layer_forward_shard(const moe_layer_desc *desc, const float *x, int32_t T,
                            const int32_t *topk_idx, const float *topk_w,
                            int32_t shard, int32_t num_shards, float *partial,
                            const moe_opts *opts, void *ws, size_t ws_bytes, void *stream);

/*
 * A shard of any width (page "Distributed CPU: Zip Fusion Beyond Tensor
 * Parallelism", section "Heterogeneous Topology": shards sized in proportion
 * to each lane's measured throughput, e.g. 30 % and 70 %, rather than equal):
 * the same sum as moe_layer_forward_shard restricted to intermediate rows
 * [i_begin, i_end) of every routed expert and of the shared expert (whose
 * width equals I).  Partials over any partition of [0, I) add up to the
 * unsplit output.  Requires i_begin and i_end to be multiples of 64 with
 * 0 <= i_begin < i_end <= I (else -1, or -2 for misaligned bounds).  The
 * workspace of moe_workspace_bytes(desc, T, 1) is enough for any range.
 */
int moe_layer_forward_range(const moe_layer_desc *desc, const float *x, int32_t T,
                            const int32_t *topk_idx, const float *topk_w,
                            int32_t i_begin, int32_t i_end, float *partial,
                            const moe_opts *opts, void *ws, size_t ws_bytes, void *stream);

/*
 * out[i] = sum over s = 0, 1, ..., num_shards-1 (ascending, fp32) of partials[s][i].
 * `partials` is a HOST array of num_shards (1..16) device pointers.  The hub's
 * sum of shard partials in a fixed, declared order (page "Distributed CPU
 * ...", sections "What Must Cross the Fabric: The Reduction Algebra" and
 * "Communication Must Be Measured").
 */
int moe_reduce_partials(const float *const *partials, int32_t num_shards, int64_t n_elems,
                        float *out, void *stream);

/*
 * The block's residual after the layer: out[i] = (partials[0][i] + ... +
 * partials[num_shards-1][i]) + residual[i], fp32, shards in ascending order,
 * then the residual (page "CKE Zip: From Splitting Tokens To Splitting
 * Qwen3.5 Weights", section "What PR #382 Now Splits": the MoE partials are
 * reduced and the block completes its residual).  num_shards = 1 adds the
 * residual to an unsplit layer output.  `partials` is a HOST array of
 * num_shards (1..16) device pointers; residual and out are device fp32
 * [n_elems].  out may alias residual or partials[0].  Errors: -1 for a null
 * pointer or num_shards outside 1..16; n_elems = 0 enqueues nothing.
 */
int moe_reduce_residual(const float *const *partials, int32_t num_shards, int64_t n_elems,
                        const float *residual, float *out, void *stream);

/*
 * RMSNorm of the layer's input rows (page "Distributed CPU: Zip Fusion Beyond
 * Tensor Parallelism", section "What Must Cross the Fabric: The Reduction
 * Algebra": the norm depends on the whole row only through its sum of
 * squares):
 *   y[t][c] = g[c] * x[t][c] / sqrt(S_t / H + eps),  S_t = sum_c x[t][c]^2.
 * The pages print no formula; this is the usual RMSNorm, with eps (>= 0) and
 * the per-column weight g [H] given by the caller.  x, y fp32 [T][H] (device,
 * 16-byte aligned, H % 4 == 0); y may alias x.  S_t is summed in fp32 in a
 * fixed order, so results are deterministic.  Errors: -1 for T < 0, a null
 * pointer or eps < 0 / NaN; -2 for H % 4 != 0 or misaligned pointers.
 */
int moe_rmsnorm(const float *x, int32_t T, int32_t H, const float *g, float eps, float *y,
                void *stream);

/*
 * RMSNorm over column shards (same section: each shard forms the sum of
 * squares of its own columns, and only those scalars meet):
 *   moe_rmsnorm_sumsq: ssq[t] = sum of x[t][c]^2 over the shard's `cols`
 *     columns, x pointing at the shard's first column, rows ldx floats apart
 *     (ldx = H for a view into the full rows, ldx = cols for a shard of its
 *     own);
 *   moe_rmsnorm_apply: S_t = ((ssq_parts[0][t] + ssq_parts[1][t]) + ...), the
 *     shards in ascending order, then y[t][c] = g[c] * x[t][c] / sqrt(S_t / H
 *     + eps) on the shard's columns, H being the full row width; g points at
 *     the shard's part of the weight, y rows are ldy floats apart.
 * `ssq_parts` is a HOST array of n_parts (1..16) device pointers to fp32 [T].
 * cols, ldx, ldy must be multiples of 4 and x, y, g 16-byte aligned (else
 * -2); y may alias x.
 */
int moe_rmsnorm_sumsq(const float *x, int32_t T, int32_t cols, int64_t ldx, float *ssq,
                      void *stream);
int moe_rmsnorm_apply(const float *x, int32_t T, int32_t cols, int64_t ldx,
                      const float *const *ssq_parts, int32_t n_parts, int32_t H, const float *g,
                      float eps, float *y, int64_t ldy, void *stream);

/*
 * Test hook: decode n_sb superblocks (bits = 4: Q4_K, 5: Q5_K,
 * MOE_SB_MXFP4: MXFP4) into n_sb*256 values in flat order.  out_dtype 0: fp32
 * (exactly the round-to-nearest-even fp32 value of d*sc*q - dmin*m, or of
 * X_j * value(code); MXFP4 scale byte 255 gives NaN); 1: bf16 and 2: fp16,
 * each the round-to-nearest-even conversion of that fp32 value.  For the
 * K-quant formats the fp16 output is produced by the same device function
 * that forms the grouped-GEMM path's fp16 matrix-core operands, so it shows
 * bit for bit the weights that path multiplies.
 */
#define MOE_SB_MXFP4 14
int moe_dequant(const uint8_t *sbs, int32_t bits, int64_t n_sb, int32_t out_dtype,
                void *out, void *stream);

/*
 * Test hook: the token->expert bucketing of the grouped-GEMM path.
 *   counts[e]   number of slots (t, j) with topk_idx[t][j] == e          (int32 [E])
 *   offsets[e]  exclusive prefix sum of counts, offsets[E] = T*k          (int32 [E+1])
 *   perm[p]     slot ids s = t*k + j sorted by expert, ascending s within
 *               an expert (a stable counting sort)                         (int32 [T*k])
 *   ws          workspace of at least moe_workspace_bytes(desc, T, 1) bytes
 * Entries of topk_idx outside [0, E) are a caller error (not checked on the device).
 */
int moe_route_bucket(const moe_layer_desc *desc, const int32_t *topk_idx, int32_t T,
                     int32_t *counts, int32_t *offsets, int32_t *perm,
                     void *ws, size_t ws_bytes, void *stream);

/* Text for a status code (static storage). */
const char *moe_status_str(int status);

/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_HIP_H */
