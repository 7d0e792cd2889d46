/*
 * moe_oracle.c -- plain, slow CPU oracle for one routed Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under quantized_moe_transformer_amd/) shares no code, header,
 * table or constant with this file, and never calls it.
 *
 * What it computes follows the page "CKE Zip: From Splitting Tokens To
 * Splitting Qwen3.5 Weights":
 *   - "What The First Prototype Split": an MoE region takes complete hidden
 *     rows X[T,H] plus, per row, the selected top-k expert indices and their
 *     routing weights, runs the routed and the shared SwiGLU branches and
 *     returns one completed output row per input row; rows are independent.
 *   - "What PR #382 Now Splits": 256 routed experts, eight selected per token,
 *     4-bit K-quant (Q4_K) gate/up and 5-bit K-quant (Q5_K) down; the
 *     intermediate dimension of every routed expert and of the shared expert
 *     is divided between shards, each shard runs gate, up, SwiGLU and down on
 *     its part and yields a hidden-sized partial; the partials add up to the
 *     whole.
 *   - "A Separate Decode Result Shows Why Axis Choice Matters": routed outputs
 *     are merged in the original selected-slot order.
 * and on the page "Distributed CPU: Zip Fusion Beyond Tensor Parallelism",
 * section "What Must Cross the Fabric: The Reduction Algebra": a weight split
 * into W = [W_1 .. W_N] lets each part run all of its local work and meet only
 * in a sum at the output projection, whose order is fixed.
 *
 * Precision: every product and sum is carried in double and rounded once to
 * fp32 at the end.  Weights are decoded exactly (see oracle_dequant).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - MXFP4 (section 1b): OCP MX element and scale encodings in a 144-byte
 *     superblock of this project's layout.
 *   - K-quant byte layout: the GGUF-shaped 144-byte Q4_K / 176-byte Q5_K
 *     superblock (fp16 d, fp16 dmin, 12 bytes of packed 6-bit scales/mins,
 *     [Q5_K: 32 bytes of high code bits], 128 bytes of code nibbles);
 *     w = d*sc*q - dmin*m.
 *   - Orientation: one row per output feature, reduction dimension contiguous,
 *     superblocks laid over the flat row-major array.
 *   - Top-k: experts ordered by their exact (double) logit, descending,
 *     ties to the lower index.  Slot j holds the j-th expert.
 *   - Routing weights: softmax over all E logits, then renormalised over the
 *     k selected ones.
 *   - SwiGLU: h = silu(gate) * up, silu(z) = z / (1 + exp(-z)).
 *   - Shared expert: always on, weight `shared_weight` (1 in every workload),
 *     added after the routed slots.
 *   - Shards: shard s of n owns intermediate rows [s*I/n, (s+1)*I/n) of every
 *     routed expert and [s*Is/n, (s+1)*Is/n) of the shared one.
 *   - RMSNorm (section 5): y = g * x / sqrt(mean(x^2) + eps) with eps and g
 *     from the caller; in shard mode the row's sum of squares is the sum of
 *     the shards' partial sums in ascending shard order.
 *   - Residual (section 5): out = (sum of the partials in ascending order)
 *     + residual.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-2)

/* ------------------------------------------------------------------------ */
/* 1. Decoding the K-quant superblocks                                       */
/* ------------------------------------------------------------------------ */

/* IEEE binary16 bits -> double, written out from the format's definition. */
double oracle_half_to_double(uint16_t h)
{
    int sign = h >> 15;
    int expo = (h >> 10) & 31;
    int frac = h & 1023;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);  /* (1 + frac/1024) * 2^(expo-15) */
    return sign ? -v : v;
}

/* 6-bit scale and min of sub-block j (0..7) from the 12 packed scale bytes.
 * Sub-blocks 0..3 keep their fields in the low six bits of bytes j and j+4;
 * sub-blocks 4..7 keep their low four bits in the nibbles of byte j+4 and
 * their top two bits in the top bits of bytes j-4 (scale) and j (min). */
static void scale_min(const uint8_t *s, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Code of element i (0..255).  The 128 code bytes hold four groups of 32; in
 * group c, byte l carries element 64c+l in its low nibble and element
 * 64c+32+l in its high nibble.  For 5 bits, bit (2c) (low-nibble element) or
 * bit (2c+1) (high-nibble element) of high-bit byte l adds 16. */
static int code_of(const uint8_t *qs, const uint8_t *qh, int i)
{
    int c = i / 64, r = i % 64, l = r % 32, upper = r / 32;
    int byte = qs[32 * c + l];
    int q = upper ? (byte >> 4) : (byte & 15);
    if (qh)
        q += 16 * ((qh[l] >> (2 * c + upper)) & 1);
    return q;
}

/* Decode one superblock (bits = 4: 144 bytes; bits = 5: 176 bytes) into 256
 * floats.  w_i = d*sc_j*q_i - dmin*m_j with j = i/32.  d*sc*q and dmin*m are
 * exact in double and so is their difference; the single rounding is the
 * final conversion to fp32 (round to nearest even). */
static void dequant_sb(const uint8_t *sb, int bits, float *out)
{
    double d = oracle_half_to_double((uint16_t)(sb[0] | (sb[1] << 8)));
    double dmin = oracle_half_to_double((uint16_t)(sb[2] | (sb[3] << 8)));
    const uint8_t *scales = sb + 4;
    const uint8_t *qh = bits == 5 ? sb + 16 : NULL;
    const uint8_t *qs = bits == 5 ? sb + 48 : sb + 16;
    for (int i = 0; i < 256; ++i) {
        int sc, m;
        scale_min(scales, i / 32, &sc, &m);
        int q = code_of(qs, qh, i);
        double w = d * sc * q - dmin * m;
        out[i] = (float)w;
    }
}

/* ------------------------------------------------------------------------ */
/* 1b. MXFP4 superblocks                                                      */
/* ------------------------------------------------------------------------ */

/* The page "Distributed CPU: Zip Fusion Beyond Tensor Parallelism" (section
 * "Decode vs Prefill: Same Weights, Different Bottlenecks") says the model
 * class targeted ships its packed weights in an MXFP4-class format, and names
 * nothing more.  The element and scale encodings are read as those of the OCP
 * Microscaling (MX) formats, v1.0: 32 elements share one E8M0 scale
 * X = 2^(s - 127) (s = 255 encodes NaN), each element is FP4 E2M1 (sign bit,
 * two exponent bits with bias 1, one mantissa bit; exponent 0 is subnormal),
 * and an element's value is X times the element's.  The byte layout is this
 * project's reading: a 144-byte superblock of 256 weights (8 MX blocks) --
 * bytes 0..7 the scales of blocks 0..7, bytes 8..15 reserved (zero), bytes
 * 16..143 the codes in the nibble order of the 4-bit K-quant superblock. */
#define ORC_SB_MXFP4 14

/* E2M1 code (0..15) -> its value. */
double oracle_e2m1(int code)
{
    int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = e == 0 ? 0.5 * m                      /* subnormal: 2^(1-1) * m/2 */
                      : ldexp(1.0 + 0.5 * m, e - 1); /* 2^(e-1) * (1 + m/2)      */
    return sign ? -v : v;
}

/* E8M0 scale byte -> 2^(s-127); 255 is NaN. */
double oracle_e8m0(int s) { return s == 255 ? NAN : ldexp(1.0, s - 127); }

/* One MXFP4 superblock into 256 floats: element value times its block's
 * scale, exact in double (a power of two times a 2-bit significand), rounded
 * once to fp32 (exact unless outside fp32's range). */
static void dequant_mx_sb(const uint8_t *sb, float *out)
{
    const uint8_t *qs = sb + 16;
    for (int i = 0; i < 256; ++i)
        out[i] = (float)(oracle_e2m1(code_of(qs, NULL, i)) * oracle_e8m0(sb[i / 32]));
}

int oracle_sb_bytes(int bits)
{
    return bits == 4 ? 144 : bits == 5 ? 176 : bits == ORC_SB_MXFP4 ? 144 : 0;
}

/* Decode n_sb consecutive superblocks into out[n_sb*256] (flat order);
 * bits = 4 (Q4_K), 5 (Q5_K) or 14 (MXFP4). */
int oracle_dequant(const uint8_t *blob, int bits, int64_t n_sb, float *out)
{
    int sbb = oracle_sb_bytes(bits);
    if (!sbb || n_sb < 0 || (n_sb && (!blob || !out)))
        return ORC_EINVAL;
    for (int64_t b = 0; b < n_sb; ++b) {
        if (bits == ORC_SB_MXFP4)
            dequant_mx_sb(blob + b * sbb, out + b * 256);
        else
            dequant_sb(blob + b * sbb, bits, out + b * 256);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 2. Router: logits, top-k, renormalised softmax weights                    */
/* ------------------------------------------------------------------------ */

/* Route one token: logits[e] = sum_h x[h]*Wr[h][e] (double, ascending h); the
 * k largest (compared exactly, in double; ties to the lower index) in
 * descending order;
 * p = softmax over all E; w_j = p[idx_j] / sum of the selected p. */
static void route_token(const float *x, int H, const float *Wr, int E, int k,
                        double *logits, int32_t *idx, double *w)
{
    for (int e = 0; e < E; ++e) {
        double l = 0.0;
        for (int h = 0; h < H; ++h)
            l += (double)x[h] * (double)Wr[(int64_t)h * E + e];
        logits[e] = l;
    }
    /* selection: repeatedly take the best remaining expert */
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            int taken = 0;
            for (int jj = 0; jj < j; ++jj)
                if (idx[jj] == e) taken = 1;
            if (taken) continue;
            if (best < 0 || logits[e] > logits[best])
                best = e;          /* strict '>' keeps the lower index on ties */
        }
        idx[j] = best;
    }
    double mx = logits[0];
    for (int e = 1; e < E; ++e)
        if (logits[e] > mx) mx = logits[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e)
        z += exp(logits[e] - mx);
    double sel = 0.0;
    for (int j = 0; j < k; ++j)
        sel += exp(logits[idx[j]] - mx) / z;
    for (int j = 0; j < k; ++j)
        w[j] = (exp(logits[idx[j]] - mx) / z) / sel;
}

/* Router for T rows.  logits (double [T][E]) may be NULL. */
int oracle_router(const float *x, int T, int H, const float *Wr, int E, int k,
                  double *logits, int32_t *idx, float *w, double *w_d)
{
    if (T < 0 || H <= 0 || E <= 0 || k < 1 || k > E || (T && (!x || !Wr || !idx)))
        return ORC_EINVAL;
    int fail = 0;
    /* token rows are independent: each is routed by the same code on any thread */
#pragma omp parallel reduction(|:fail)
    {
        double *l = malloc(sizeof(double) * E);
        double *wd = malloc(sizeof(double) * k);
        if (!l || !wd) fail = 1;
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            if (!l || !wd) continue;
            route_token(x + (int64_t)t * H, H, Wr, E, k, l, idx + (int64_t)t * k, wd);
            if (logits) memcpy(logits + (int64_t)t * E, l, sizeof(double) * E);
            for (int j = 0; j < k; ++j) {
                if (w) w[(int64_t)t * k + j] = (float)wd[j];
                if (w_d) w_d[(int64_t)t * k + j] = wd[j];
            }
        }
        free(l);
        free(wd);
    }
    return fail ? ORC_ENOMEM : ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 3. Token -> expert bucketing                                              */
/* ------------------------------------------------------------------------ */

/* counts[e] = number of slots (t, j) with idx[t][j] == e; offsets = exclusive
 * prefix sum of counts (offsets[E] = T*k); perm lists, expert by expert, the
 * slot ids s = t*k + j routed to that expert in ascending s; inv_pos[s] is the
 * position of s in perm.  The definition of a stable counting sort. */
int oracle_bucket(const int32_t *idx, int T, int k, int E,
                  int32_t *counts, int32_t *offsets, int32_t *perm, int32_t *inv_pos)
{
    if (T < 0 || k < 1 || E < 1)
        return ORC_EINVAL;
    int64_t n = (int64_t)T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t s = 0; s < n; ++s) {
        if (idx[s] < 0 || idx[s] >= E) return ORC_EINVAL;
        counts[idx[s]]++;
    }
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *fill = malloc(sizeof(int32_t) * (E > 0 ? E : 1));
    if (!fill) return ORC_ENOMEM;
    for (int e = 0; e < E; ++e) fill[e] = offsets[e];
    for (int64_t s = 0; s < n; ++s) {
        int32_t p = fill[idx[s]]++;
        perm[p] = (int32_t)s;
        if (inv_pos) inv_pos[s] = p;
    }
    free(fill);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 4. Expert FFN and the whole layer                                         */
/* ------------------------------------------------------------------------ */

typedef struct {
    int32_t H, E, k, I, Is;
    float shared_weight;
    const float *router_w;                           /* [H][E] */
    const uint8_t *gate, *up, *down;                 /* [E] blobs */
    const uint8_t *sh_gate, *sh_up, *sh_down;        /* shared expert blobs */
    int32_t fmt;       /* 0: Q4_K gate/up, Q5_K down; 1: MXFP4 all three */
} oracle_layer;

/* silu(z) = z * sigmoid(z), evaluated without overflow on either side. */
static double silu(double z)
{
    if (z >= 0.0)
        return z / (1.0 + exp(-z));
    double ez = exp(z);
    return z * ez / (1.0 + ez);
}

/* One expert on one token, intermediate rows [i0, i1):
 *   g_i = sum_h Wg[i][h] x_h,  u_i = sum_h Wu[i][h] x_h,  a_i = silu(g_i) u_i,
 *   y_o = sum_{i in [i0,i1)} Wd[o][i] a_i.
 * Wg, Wu are decoded [I][H]; Wd is decoded [H][I]. */
static void expert_ffn(const float *Wg, const float *Wu, const float *Wd,
                       int H, int I, int i0, int i1, const float *x,
                       double *a, double *y)
{
    for (int i = i0; i < i1; ++i) {
        double g = 0.0, u = 0.0;
        const float *rg = Wg + (int64_t)i * H, *ru = Wu + (int64_t)i * H;
        for (int h = 0; h < H; ++h) {
            g += (double)rg[h] * (double)x[h];
            u += (double)ru[h] * (double)x[h];
        }
        a[i - i0] = silu(g) * u;
    }
    for (int o = 0; o < H; ++o) {
        double acc = 0.0;
        const float *rd = Wd + (int64_t)o * I;
        for (int i = i0; i < i1; ++i)
            acc += (double)rd[i] * a[i - i0];
        y[o] = acc;
    }
}

typedef struct { float *g, *u, *d; } decoded_expert;

static int decode_expert(const uint8_t *g, const uint8_t *u, const uint8_t *d,
                         int H, int I, int fmt, decoded_expert *out)
{
    int64_t n = (int64_t)H * I;
    out->g = malloc(sizeof(float) * n);
    out->u = malloc(sizeof(float) * n);
    out->d = malloc(sizeof(float) * n);
    if (!out->g || !out->u || !out->d) return ORC_ENOMEM;
    oracle_dequant(g, fmt ? ORC_SB_MXFP4 : 4, n / 256, out->g);
    oracle_dequant(u, fmt ? ORC_SB_MXFP4 : 4, n / 256, out->u);
    oracle_dequant(d, fmt ? ORC_SB_MXFP4 : 5, n / 256, out->d);
    return ORC_OK;
}

static void free_expert(decoded_expert *e)
{
    free(e->g); free(e->u); free(e->d);
    e->g = e->u = e->d = NULL;
}

/*
 * The layer (or shard `shard` of `num_shards` of it) on T token rows.
 *   out[t] = sum_{j<k} w[t][j] * y(e_{t,j}, x_t) + shared_weight * y(shared, x_t)
 * summed in slot order, then the shared term, in double; written to out_d
 * (double, may be NULL) and out (fp32, may be NULL).
 * idx_in / w_in: given routing (the synchronised router decision); when NULL
 * the oracle routes itself.  nthreads <= 0: all available.
 * Decoded weights of the experts that are touched are held for the call; the
 * decode is exact, so holding it changes no arithmetic.
 */
static int forward_rows(const oracle_layer *L, const float *x, int T,
                        const int32_t *idx_in, const float *w_in, int i0, int i1, int s0,
                        int s1, float *out, double *out_d, int nthreads);

int oracle_forward(const oracle_layer *L, const float *x, int T,
                   const int32_t *idx_in, const float *w_in,
                   int shard, int num_shards, float *out, double *out_d, int nthreads)
{
    if (!L || T < 0 || num_shards < 1 || shard < 0 || shard >= num_shards)
        return ORC_EINVAL;
    if (L->I % num_shards || L->Is % num_shards)
        return ORC_EINVAL;
    const int I = L->I, Is = L->Is;
    return forward_rows(L, x, T, idx_in, w_in, shard * (I / num_shards),
                        (shard + 1) * (I / num_shards), shard * (Is / num_shards),
                        (shard + 1) * (Is / num_shards), out, out_d, nthreads);
}

/*
 * A shard of any size (page "Distributed CPU: Zip Fusion Beyond Tensor
 * Parallelism", section "Heterogeneous Topology": shards proportional to each
 * lane's measured throughput, e.g. 30 % and 70 %): intermediate rows
 * [i_begin, i_end) of every routed expert and of the shared expert (which then
 * has the routed width, or none).  Partials over any partition of [0, I) add
 * up to the layer.
 */
int oracle_forward_range(const oracle_layer *L, const float *x, int T,
                         const int32_t *idx_in, const float *w_in, int i_begin, int i_end,
                         float *out, double *out_d, int nthreads)
{
    if (!L || i_begin < 0 || i_end < i_begin || i_end > L->I) return ORC_EINVAL;
    if (L->Is != 0 && L->Is != L->I) return ORC_EINVAL;
    return forward_rows(L, x, T, idx_in, w_in, i_begin, i_end, i_begin, i_end, out, out_d,
                        nthreads);
}

/* The layer restricted to routed intermediate rows [i0, i1) and shared rows
 * [s0, s1). */
static int forward_rows(const oracle_layer *L, const float *x, int T,
                        const int32_t *idx_in, const float *w_in, int i0, int i1, int s0,
                        int s1, float *out, double *out_d, int nthreads)
{
    if (!L || T < 0 || L->k < 1 || L->k > L->E)
        return ORC_EINVAL;
    if ((L->H * L->I) % 256 || (L->H * L->Is) % 256 || L->fmt < 0 || L->fmt > 1)
        return ORC_EINVAL;
    if (T == 0)
        return ORC_OK;
    int H = L->H, E = L->E, k = L->k, I = L->I, Is = L->Is;
    int64_t nsb = (int64_t)I * H / 256;     /* superblocks per routed matrix */
    int nthr = nthreads > 0 ? nthreads : omp_get_max_threads();

    int32_t *idx = malloc(sizeof(int32_t) * (int64_t)T * k);
    double *w = malloc(sizeof(double) * (int64_t)T * k);
    decoded_expert *dec = calloc(E, sizeof(decoded_expert));
    decoded_expert sh = {0};
    int rc = ORC_OK;
    if (!idx || !w || !dec) { rc = ORC_ENOMEM; goto done; }

    if (idx_in) {
        for (int64_t s = 0; s < (int64_t)T * k; ++s) {
            if (idx_in[s] < 0 || idx_in[s] >= E) { rc = ORC_EINVAL; goto done; }
            idx[s] = idx_in[s];
            w[s] = (double)w_in[s];
        }
    } else {
        rc = oracle_router(x, T, H, L->router_w, E, k, NULL, idx, NULL, w);
        if (rc) goto done;
    }

    /* decode every touched expert once */
    char *used = calloc(E, 1);
    if (!used) { rc = ORC_ENOMEM; goto done; }
    for (int64_t s = 0; s < (int64_t)T * k; ++s) used[idx[s]] = 1;
    int fail = 0;
#pragma omp parallel for schedule(dynamic) num_threads(nthr) reduction(|:fail)
    for (int e = 0; e < E; ++e)
        if (used[e])
            fail |= decode_expert(L->gate + e * nsb * 144, L->up + e * nsb * 144,
                                  L->down + e * nsb * (L->fmt ? 144 : 176), H, I, L->fmt,
                                  &dec[e]) != ORC_OK;
    free(used);
    if (!fail && Is > 0)
        fail |= decode_expert(L->sh_gate, L->sh_up, L->sh_down, H, Is, L->fmt, &sh) != ORC_OK;
    if (fail) { rc = ORC_ENOMEM; goto done; }

    int amax = I > Is ? I : Is;
#pragma omp parallel num_threads(nthr)
    {
        double *a = malloc(sizeof(double) * (amax > 0 ? amax : 1));
        double *y = malloc(sizeof(double) * H);
        double *acc = malloc(sizeof(double) * H);
#pragma omp for schedule(dynamic)
        for (int t = 0; t < T; ++t) {
            const float *xt = x + (int64_t)t * H;
            for (int o = 0; o < H; ++o) acc[o] = 0.0;
            for (int j = 0; j < k; ++j) {            /* slot order */
                decoded_expert *ex = &dec[idx[(int64_t)t * k + j]];
                expert_ffn(ex->g, ex->u, ex->d, H, I, i0, i1, xt, a, y);
                double wj = w[(int64_t)t * k + j];
                for (int o = 0; o < H; ++o) acc[o] += wj * y[o];
            }
            if (Is > 0) {                             /* then the shared expert */
                expert_ffn(sh.g, sh.u, sh.d, H, Is, s0, s1, xt, a, y);
                for (int o = 0; o < H; ++o) acc[o] += (double)L->shared_weight * y[o];
            }
            for (int o = 0; o < H; ++o) {
                if (out) out[(int64_t)t * H + o] = (float)acc[o];
                if (out_d) out_d[(int64_t)t * H + o] = acc[o];
            }
        }
        free(a); free(y); free(acc);
    }

done:
    if (dec)
        for (int e = 0; e < E; ++e) free_expert(&dec[e]);
    free_expert(&sh);
    free(dec);
    free(idx);
    free(w);
    return rc;
}

/* Sum of shard partials in ascending shard order (fp32 inputs, double sum,
 * one rounding): the hub's z = sum_i z_i with a fixed, declared order. */
int oracle_reduce(const float *const *partials, int num_shards, int64_t n, float *out)
{
    if (num_shards < 1 || n < 0 || !partials || !out) return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int s = 0; s < num_shards; ++s) acc += (double)partials[s][i];
        out[i] = (float)acc;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* 5. The steps either side of the layer: RMSNorm before, residual after     */
/* ------------------------------------------------------------------------ */

/* Page "Distributed CPU: Zip Fusion Beyond Tensor Parallelism", section "What
 * Must Cross the Fabric: The Reduction Algebra": RMSNorm needs the whole
 * row, but only through one number, the row's sum of squares; split over
 * column shards, each shard forms the sum over its own columns and only those
 * scalars meet.  The pages print no formula; read as the usual RMSNorm,
 *   y[c] = g[c] * x[c] / sqrt(S / H + eps),  S = sum over the H columns of x^2,
 * with eps and the per-column weight g supplied by the caller. */

/* Sum of squares of columns [c0, c1) of each of T rows (row stride ld),
 * double, ascending column. */
int oracle_sumsq(const float *x, int T, int64_t ld, int c0, int c1, double *ssq)
{
    if (!x || !ssq || T < 0 || c0 < 0 || c1 < c0) return ORC_EINVAL;
    for (int t = 0; t < T; ++t) {
        double s = 0.0;
        for (int c = c0; c < c1; ++c) {
            const double v = (double)x[(int64_t)t * ld + c];
            s += v * v;
        }
        ssq[t] = s;
    }
    return ORC_OK;
}

/* RMSNorm of T rows of H columns (row stride H), rounded once to fp32. */
int oracle_rmsnorm(const float *x, int T, int H, const float *g, float eps, float *y)
{
    if (!x || !g || !y || T < 0 || H < 1) return ORC_EINVAL;
    double *ssq = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    if (!ssq) return ORC_ENOMEM;
    oracle_sumsq(x, T, H, 0, H, ssq);
    for (int t = 0; t < T; ++t) {
        const double r = sqrt(ssq[t] / (double)H + (double)eps);
        for (int c = 0; c < H; ++c) {
            const int64_t i = (int64_t)t * H + c;
            y[i] = (float)((double)g[c] * (double)x[i] / r);
        }
    }
    free(ssq);
    return ORC_OK;
}

/* The block's residual after the layer (page "CKE Zip: From Splitting Tokens
 * To Splitting Qwen3.5 Weights", section "What PR #382 Now Splits": the MoE
 * partials are reduced and the block completes its residual):
 *   out = (p_0 + p_1 + ... + p_{n-1}) + residual,
 * in double, rounded once. */
int oracle_reduce_residual(const float *const *partials, int num_shards, int64_t n,
                           const float *residual, float *out)
{
    if (num_shards < 1 || n < 0 || !partials || !residual || !out) return ORC_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int s = 0; s < num_shards; ++s) acc += (double)partials[s][i];
        out[i] = (float)(acc + (double)residual[i]);
    }
    return ORC_OK;
}

int oracle_max_threads(void) { return omp_get_max_threads(); }
