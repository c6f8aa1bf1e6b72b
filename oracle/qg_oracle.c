/*
 * qg_oracle.c -- CPU oracle for the quantized decode matrix-vector product.
 *
 * TEST INFRASTRUCTURE. This is the plain, slow, obviously correct definition
 * of what the GPU library computes, in double precision, written from the
 * pages that describe the method. Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load it. It shares no code, header,
 * table or helper with the GPU library, and the GPU library never calls it.
 *
 * Sources (page title, then the section used):
 *  [F]  "Booster la vitesse d'inference sur Apple Silicon -- avec le format
 *       .forge" (web research report): TL;DR (decode is bandwidth bound),
 *       section 1 "Le chemin de decodage rapide" (fused-dequant GEMV, the
 *       fusions: rmsnorm+QKV, residual+norm, gate.up SwiGLU, logits+top-k),
 *       section 3 item 4 (planar 4-bit codes packed in uint32 with separate
 *       scale and bias tensors, group 64; LUT type with 16 fp16 entries).
 *  [G]  GeekNews item on a C/Metal engine running a 397B MoE on a MacBook
 *       Pro: "Architecture du modele" (512 experts, K=4 active incl. one
 *       shared), "Noyau de dequantification optimise FMA" (the weight is
 *       nibble*scale+bias), "Shaders de calcul Metal" and "Deferred GPU
 *       Expert Compute" (MoE combine + residual + norm on the GPU).
 *  [B]  gist.science explainer of the BaseRT paper, "Methodologie": one
 *       matvec variant per quantization format from Q2 to FP16, each
 *       dequantizing inside its inner loop.
 *
 * Readings where the pages are silent:
 *  - code k of a row sits in word k/(32/bits) at bit offset bits*(k mod
 *    32/bits), least significant field first;
 *  - a group is 64 consecutive k of one row;
 *  - LUT format: one 16-entry fp16 table per output row, no scale/bias;
 *  - RMSNorm: x_k * g_k / sqrt(mean_j x_j^2 + eps);
 *  - SwiGLU: silu(gate) * up, silu(z) = z / (1 + exp(-z));
 *  - top-k order: larger value first, equal values by lower index; NaN is
 *    below every number;
 *  - routing weights: softmax over the selected logits only;
 *  - sampling after top-k: temperature and top-p over the k candidates, one
 *    uniform draw from the counter-based SplitMix64 generator (see og_sample);
 *  - the per-format matvec variants from Q2 to FP16 (BaseRT explainer,
 *    "Methodologie"): Q8 is the affine format with 8-bit codes, four to a
 *    word; FP16 is the dense format, where each 16-bit field of a word is the
 *    fp16 weight itself (two to a word, so a little-endian fp16 row is its
 *    own packing) and there is no scale, bias or table.
 *
 * Everything is computed in double. Dequantized weights q*s+b are exact in
 * double (q has at most 8 bits, s and b are fp16: q*s needs at most 19
 * significant bits and the sum spans 2^-24..2^9). Dot products run in k
 * order.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OG_AFFINE 0
#define OG_LUT 1
#define OG_DENSE 2

/* A planar quantized matrix as the oracle sees it ([F] section 3 item 4). */
typedef struct og_qmat {
    const uint32_t *q;      /* [N][K*bits/32] code words */
    const uint16_t *scales; /* [N][K/group] fp16 bits, affine only */
    const uint16_t *biases; /* [N][K/group] fp16 bits, affine only */
    const uint16_t *lut;    /* [N][2^bits] fp16 bits, LUT only */
    int N, K, group, bits, fmt; /* fmt: OG_AFFINE (bits 2, 4, 8), OG_LUT, OG_DENSE (bits 16) */
} og_qmat;

/* IEEE 754 binary16 -> double, from the format definition: 1 sign bit,
 * 5 exponent bits (bias 15), 10 fraction bits; exponent 0 encodes zero and
 * subnormals (fraction * 2^-24), exponent 31 encodes infinities and NaN. */
double og_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

static int valid_qmat(const og_qmat *W)
{
    if (!W || !W->q || W->N < 0 || W->K < 0)
        return 0;
    if (W->fmt == OG_DENSE)
        return W->bits == 16 && (W->K * 16) % 32 == 0;
    if (W->bits != 2 && W->bits != 4 && W->bits != 8)
        return 0;
    if (W->group <= 0 || W->K % W->group || (W->K * W->bits) % 32)
        return 0;
    if (W->fmt == OG_AFFINE)
        return W->scales && W->biases;
    if (W->fmt == OG_LUT)
        return W->lut != NULL && W->bits <= 4;
    return 0;
}

/* Code (quantized value) of element (n, k). */
static unsigned code_at(const og_qmat *W, int n, int k)
{
    int per_word = 32 / W->bits;
    size_t words_per_row = (size_t)W->K / per_word;
    uint32_t word = W->q[(size_t)n * words_per_row + k / per_word];
    unsigned shift = (unsigned)(W->bits * (k % per_word));
    return (word >> shift) & ((1u << W->bits) - 1u);
}

/* Dequantized weight W[n][k]: code*scale + bias for the affine format
 * ([G] FMA section writes the weight as nibble*scale + bias), the row's
 * table entry for the LUT format ([F] section 3 item 4), or the 16-bit field
 * read as an fp16 number for the dense format. */
static double weight_at(const og_qmat *W, int n, int k)
{
    unsigned c = code_at(W, n, k);
    if (W->fmt == OG_DENSE)
        return og_half_to_double((uint16_t)c);
    if (W->fmt == OG_LUT)
        return og_half_to_double(W->lut[(size_t)n * (1u << W->bits) + c]);
    size_t groups_per_row = (size_t)W->K / W->group;
    size_t gi = (size_t)n * groups_per_row + k / W->group;
    return (double)c * og_half_to_double(W->scales[gi]) + og_half_to_double(W->biases[gi]);
}

/* Codes of rows [0,N): codes[n*K + k]. */
int og_unpack(const og_qmat *W, uint8_t *codes)
{
    if (!valid_qmat(W) || !codes || W->bits > 8)
        return -1;
    for (int n = 0; n < W->N; ++n)
        for (int k = 0; k < W->K; ++k)
            codes[(size_t)n * W->K + k] = (uint8_t)code_at(W, n, k);
    return 0;
}

/* Dense dequantized matrix: out[n*K + k] = W[n][k]. */
int og_dequant(const og_qmat *W, double *out)
{
    if (!valid_qmat(W) || !out)
        return -1;
    for (int n = 0; n < W->N; ++n)
        for (int k = 0; k < W->K; ++k)
            out[(size_t)n * W->K + k] = weight_at(W, n, k);
    return 0;
}

/* ---- matrix-vector product ---------------------------------------------
 * y[m][n] = r[m][n] + sum_k W[n][k] * x[m][k]  ([F] section 1: the decode
 * matvec that dequantizes inside its loop; r is the optional residual). Rows
 * are independent, so splitting them over threads does not change any
 * result. */
typedef struct {
    const og_qmat *W;
    int M, n0, n1;
    const double *x, *residual;
    double *y;
} gemv_job;

static void *gemv_rows(void *arg)
{
    gemv_job *j = (gemv_job *)arg;
    const og_qmat *W = j->W;
    for (int m = 0; m < j->M; ++m) {
        const double *xm = j->x + (size_t)m * W->K;
        for (int n = j->n0; n < j->n1; ++n) {
            double acc = 0.0;
            for (int k = 0; k < W->K; ++k)
                acc += weight_at(W, n, k) * xm[k];
            size_t o = (size_t)m * W->N + n;
            j->y[o] = (j->residual ? j->residual[o] : 0.0) + acc;
        }
    }
    return NULL;
}

int og_gemv(const og_qmat *W, int M, const double *x, const double *residual, double *y,
            int nthreads)
{
    if (!valid_qmat(W) || M < 1 || !x || !y)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if (nthreads > W->N)
        nthreads = W->N > 0 ? W->N : 1;
    gemv_job jobs[256];
    pthread_t tids[256];
    for (int t = 0; t < nthreads; ++t) {
        jobs[t].W = W;
        jobs[t].M = M;
        jobs[t].n0 = (int)((long long)W->N * t / nthreads);
        jobs[t].n1 = (int)((long long)W->N * (t + 1) / nthreads);
        jobs[t].x = x;
        jobs[t].residual = residual;
        jobs[t].y = y;
    }
    if (nthreads == 1) {
        gemv_rows(&jobs[0]);
        return 0;
    }
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&tids[t], NULL, gemv_rows, &jobs[t]) != 0)
            break;
        ++started;
    }
    for (int t = started; t < nthreads; ++t) /* could not spawn: do it here */
        gemv_rows(&jobs[t]);
    for (int t = 0; t < started; ++t)
        pthread_join(tids[t], NULL);
    return 0;
}

/* ---- RMSNorm ([F] section 1, fused into the QKV matvec) -----------------
 * out_k = x_k * g_k / sqrt((1/K) sum_j x_j^2 + eps). */
int og_rmsnorm(const double *x, int K, const uint16_t *g, double eps, double *out)
{
    if (!x || !g || !out || K < 1)
        return -1;
    double ss = 0.0;
    for (int k = 0; k < K; ++k)
        ss += x[k] * x[k];
    double denom = sqrt(ss / K + eps);
    for (int k = 0; k < K; ++k)
        out[k] = x[k] * og_half_to_double(g[k]) / denom;
    return 0;
}

/* silu(z) = z / (1 + exp(-z)). */
double og_silu(double z) { return z / (1.0 + exp(-z)); }

/* ---- gate.up SwiGLU in one step ([F] section 1) --------------------------
 * u[m][j] = silu((Wg x_m)_j) * (Wu x_m)_j. */
int og_swiglu(const og_qmat *Wg, const og_qmat *Wu, int M, const double *x, double *u,
              int nthreads)
{
    if (!valid_qmat(Wg) || !valid_qmat(Wu) || Wg->N != Wu->N || Wg->K != Wu->K || !u)
        return -1;
    size_t n = (size_t)M * Wg->N;
    double *a = (double *)malloc(n * sizeof(double));
    double *c = (double *)malloc(n * sizeof(double));
    int rc = -1;
    if (a && c && og_gemv(Wg, M, x, NULL, a, nthreads) == 0 &&
        og_gemv(Wu, M, x, NULL, c, nthreads) == 0) {
        for (size_t i = 0; i < n; ++i)
            u[i] = og_silu(a[i]) * c[i];
        rc = 0;
    }
    free(a);
    free(c);
    return rc;
}

/* ---- top-k -------------------------------------------------------------
 * "a before b": a larger, or equal and with a lower index. NaN is below every
 * number (equal NaNs again by index). +0 and -0 are equal. */
static int before(double va, int ia, double vb, int ib)
{
    int na = isnan(va), nb = isnan(vb);
    if (na || nb) {
        if (na && nb)
            return ia < ib;
        return nb; /* a number is before NaN */
    }
    if (va != vb)
        return va > vb;
    return ia < ib;
}

/* The first k elements of z under the order above, by repeated selection of
 * the best element not yet taken ([F] section 1: logits matvec + top-k on
 * the GPU, returning only the chosen entries). */
int og_topk(const double *z, int V, int k, int32_t *idx, double *vals)
{
    if (!z || !idx || V < 1 || k < 1 || k > V)
        return -1;
    unsigned char *taken = (unsigned char *)calloc((size_t)V, 1);
    if (!taken)
        return -1;
    for (int r = 0; r < k; ++r) {
        int best = -1;
        for (int i = 0; i < V; ++i) {
            if (taken[i])
                continue;
            if (best < 0 || before(z[i], i, z[best], best))
                best = i;
        }
        taken[best] = 1;
        idx[r] = best;
        if (vals)
            vals[r] = z[best];
    }
    free(taken);
    return 0;
}

/* ---- MoE routing ([G] "Architecture du modele") ---------------------------
 * ids = top-k of the router logits; w_i = exp(l_i - l_max) / sum_{j in ids}
 * exp(l_j - l_max): softmax over the selected logits. */
int og_route(const double *logits, int E, int k, int32_t *ids, double *w)
{
    if (og_topk(logits, E, k, ids, NULL) != 0 || !w)
        return -1;
    double lmax = logits[ids[0]];
    double den = 0.0;
    for (int i = 0; i < k; ++i)
        den += exp(logits[ids[i]] - lmax);
    for (int i = 0; i < k; ++i)
        w[i] = exp(logits[ids[i]] - lmax) / den;
    return 0;
}

/* ---- Sampling from the top-k ([F] section 1: logits matvec + top-k
 * sampling on the GPU, only the token comes back) ---------------------------
 * The page names the step, not its rule; the plainest reading, used here:
 *   temperature == 0: the token is idx[0] (greedy);
 *   otherwise w_i = exp((vals_i - vals_0) / temperature) for the k candidates
 *   in their order (vals_0 is the largest); top_p keeps the shortest prefix
 *   0..m-1 whose weight sum reaches top_p times the total (m >= 1); with S the
 *   prefix sum, the token is idx[i] for the first i whose running sum
 *   w_0 + ... + w_i exceeds u * S (the last prefix entry if none does).
 * Sums run in index order. u is a uniform draw in [0, 1). */
int og_sample(const double *vals, const int32_t *idx, int k, double temperature, double top_p,
              double u, int32_t *token)
{
    if (!vals || !idx || !token || k < 1 || !(temperature >= 0.0) || !(top_p > 0.0) ||
        !(top_p <= 1.0) || !(u >= 0.0) || !(u < 1.0))
        return -1;
    if (temperature == 0.0) {
        *token = idx[0];
        return 0;
    }
    double *w = (double *)malloc((size_t)k * sizeof(double));
    if (!w)
        return -1;
    double total = 0.0;
    for (int i = 0; i < k; ++i) {
        w[i] = exp((vals[i] - vals[0]) / temperature);
        total += w[i];
    }
    int m = 0;
    double prefix = 0.0;
    while (m < k) {
        prefix += w[m];
        ++m;
        if (prefix >= top_p * total)
            break;
    }
    const double target = u * prefix;
    double run = 0.0;
    int pick = m - 1;
    for (int i = 0; i < m; ++i) {
        run += w[i];
        if (run > target) {
            pick = i;
            break;
        }
    }
    free(w);
    *token = idx[pick];
    return 0;
}

/* Counter-based SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014): output number `counter`
 * (0, 1, 2, ...) of the generator started from state `seed` is the mixing
 * function applied to seed + (counter + 1) * 0x9E3779B97F4A7C15. */
uint64_t og_splitmix64(uint64_t seed, uint64_t counter)
{
    uint64_t z = seed + (counter + 1u) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* The top 53 bits of the output as a double in [0, 1). */
double og_uniform(uint64_t seed, uint64_t counter)
{
    return (double)(og_splitmix64(seed, counter) >> 11) * 0x1.0p-53;
}

/* ---- Decode attention over a KV cache ([F] section 2 "KV cache") --------
 * The cache of one layer is [Hkv][T_max][d] fp16 per tensor (K and V), laid
 * out along the time axis per head; GQA: query head h reads kv head
 * h / (H / Hkv). One query per head (decode). For positions t = 0..n-1:
 *   s_t = scale * sum_j q[h][j] * K[g][t][j],
 *   out[h][j] = sum_t softmax(s)_t * V[g][t][j]   (softmax over t < n).
 * The page asks for split-K along the cache for long contexts; splitting
 * is an evaluation order, so the oracle is the plain definition. */
int og_attention(const double *q, const uint16_t *k_cache, const uint16_t *v_cache, int H, int Hkv,
                 int d, int T_max, int n, double scale, double *out)
{
    if (!q || !k_cache || !v_cache || !out || H < 1 || Hkv < 1 || H % Hkv || d < 1 || n < 1 ||
        n > T_max)
        return -1;
    double *s = (double *)malloc((size_t)n * sizeof(double));
    if (!s)
        return -1;
    const int G = H / Hkv;
    for (int h = 0; h < H; ++h) {
        const int g = h / G;
        const uint16_t *Kg = k_cache + (size_t)g * T_max * d;
        const uint16_t *Vg = v_cache + (size_t)g * T_max * d;
        double smax = -INFINITY;
        for (int t = 0; t < n; ++t) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j)
                acc += q[(size_t)h * d + j] * og_half_to_double(Kg[(size_t)t * d + j]);
            s[t] = scale * acc;
            if (s[t] > smax)
                smax = s[t];
        }
        double den = 0.0;
        for (int t = 0; t < n; ++t) {
            s[t] = exp(s[t] - smax);
            den += s[t];
        }
        for (int j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int t = 0; t < n; ++t)
                acc += s[t] * og_half_to_double(Vg[(size_t)t * d + j]);
            out[(size_t)h * d + j] = acc / den;
        }
    }
    free(s);
    return 0;
}
