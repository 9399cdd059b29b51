/*
 * oracle.c - TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * A plain fp64 CPU decode step. Loops are written in the order the
 * definitions read; OpenMP is used only across independent outputs (rows of a
 * matrix-vector product, heads of attention), never inside a sum.
 *
 * Readings where the pages are silent (each is repeated where it is used):
 *   - architecture: Llama-style pre-norm decoder, no biases, untied lm_head;
 *   - RMSNorm y_i = x_i / sqrt(mean(x^2) + eps) * g_i;
 *   - RoPE: rotate-half pairs (i, i + dh/2), theta_i = base^(-2i/dh), angle
 *     pos * theta_i, absolute position also in sliding layers;
 *   - cached K is post-RoPE; the new k, v are rounded to bf16, written to
 *     the pool and read back like every other position;
 *   - attention scale 1/sqrt(dh), GQA kv head = floor(h / (Hq/Hkv));
 *   - sliding window W: keys j with pos - W < j <= pos;
 *   - SwiGLU: silu(gate) * up, silu(z) = z / (1 + e^-z);
 *   - MoE: top-k by router logit (ties to the lower index), softmax over the
 *     k selected logits;
 *   - temperature sampling by Gumbel-max with a SplitMix64 counter noise.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ bf16 */

double orc_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* Round-to-nearest-even of an fp64 value to bf16 (8 significant bits),
 * done directly on the fp64 bit pattern so there is no double rounding. */
uint16_t orc_f64_to_bf16(double x)
{
    if (x != x) return 0x7FC0u;
    uint64_t u;
    memcpy(&u, &x, 8);
    const uint64_t drop = 45; /* 52 - 7 mantissa bits dropped */
    uint64_t exp = (u >> 52) & 0x7FFu;
    if (exp != 0 && exp != 0x7FFu) {
        u += ((1ULL << (drop - 1)) - 1) + ((u >> drop) & 1ULL);
        u &= ~((1ULL << drop) - 1);
    }
    double r;
    memcpy(&r, &u, 8);
    float f = (float)r; /* exact whenever r is in the normal bf16 range */
    uint32_t fu;
    memcpy(&fu, &f, 4);
    return (uint16_t)(fu >> 16);
}

/* --------------------------------------------------------------- SplitMix64
 * One output step of SplitMix64 (Steele, Lea and Flood, OOPSLA 2014):
 * add the golden gamma, then the two xor-shift-multiply rounds. The sampler's
 * noise is drawn from it (see orc_gumbel). */
uint64_t orc_splitmix64(uint64_t z)
{
    z += 0x9E3779B97F4A7C15ULL;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

/* ------------------------------------------------------------------ layers */

/* RMSNorm (reading: y_i = x_i * (1/sqrt(mean(x^2) + eps)) * g_i). */
void orc_rmsnorm(int32_t d, const double *x, const uint16_t *g, double eps, double *y)
{
    double ss = 0.0;
    for (int32_t i = 0; i < d; ++i) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / (double)d + eps);
    for (int32_t i = 0; i < d; ++i) y[i] = x[i] * r * orc_bf16_to_f64(g[i]);
}

/* y = W x with W row-major [rows][cols] (torch nn.Linear layout). Each row is
 * a sequential fp64 sum in column order. At batch 1 this product is the
 * matrix-vector work that the Kog AI page ("Bellek Bant Genişliği LLM Hızının
 * Temel Darboğazı") says bounds decode by memory bandwidth. */
void orc_matvec(int32_t rows, int32_t cols, const uint16_t *W, const double *x, double *y)
{
#pragma omp parallel for schedule(static) if ((int64_t)rows * cols > (1 << 16))
    for (int32_t r = 0; r < rows; ++r) {
        const uint16_t *w = W + (int64_t)r * cols;
        double acc = 0.0;
        for (int32_t c = 0; c < cols; ++c) acc += orc_bf16_to_f64(w[c]) * x[c];
        y[r] = acc;
    }
}

/* RoPE, rotate-half convention (reading): for every head and i < dh/2,
 * a = pos * base^(-2i/dh),
 * (v_i, v_{i+dh/2}) <- (v_i cos a - v_{i+dh/2} sin a, v_i sin a + v_{i+dh/2} cos a). */
void orc_rope(int32_t n_heads, int32_t head_dim, int32_t pos, double base, double *v)
{
    const int32_t half = head_dim / 2;
    for (int32_t h = 0; h < n_heads; ++h) {
        double *x = v + (int64_t)h * head_dim;
        for (int32_t i = 0; i < half; ++i) {
            double theta = pow(base, -2.0 * (double)i / (double)head_dim);
            double a = (double)pos * theta;
            double c = cos(a), s = sin(a);
            double x0 = x[i], x1 = x[i + half];
            x[i] = x0 * c - x1 * s;
            x[i + half] = x0 * s + x1 * c;
        }
    }
}

/* silu(z) = z * sigmoid(z) = z / (1 + e^-z). */
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* SwiGLU FFN: y = W_down (silu(W_gate n2) * (W_up n2)). */
void orc_swiglu_ffn(int32_t d, int32_t f, const uint16_t *w_gate, const uint16_t *w_up,
                    const uint16_t *w_down, const double *n2, double *y)
{
    double *g = (double *)malloc(sizeof(double) * (size_t)f);
    double *u = (double *)malloc(sizeof(double) * (size_t)f);
    orc_matvec(f, d, w_gate, n2, g);
    orc_matvec(f, d, w_up, n2, u);
    for (int32_t i = 0; i < f; ++i) g[i] = orc_silu(g[i]) * u[i];
    orc_matvec(d, f, w_down, g, y);
    free(g);
    free(u);
}

/* First key position a query at ``pos`` attends to. Reading of "kayan pencere
 * dikkati" (sliding-window attention, Cohere Megakernel page, "Sınırlar açıkça
 * yazılmış"): window W > 0 keeps the W most recent keys, the current one
 * included; W = 0 is full attention. */
int32_t orc_window_lo(int32_t pos, int32_t window)
{
    if (window <= 0) return 0;
    int32_t lo = pos - window + 1;
    return lo > 0 ? lo : 0;
}

/* One query head of decode attention over paged K/V ("sayfalı KV önbelleği",
 * paged KV cache, Cohere Megakernel page, "Sınırlar açıkça yazılmış").
 * Keys j in [lo, pos] are read through ``pages`` (the request's page-table
 * row): slot (pages[j / 16], j % 16). s_j = (q . K_j) / sqrt(dh); two-pass
 * softmax; o = sum_j p_j V_j. ``probs`` (optional) receives p_j, j = lo..pos.
 * Layout of a pool layer: [n_pages][n_kv_heads][16][head_dim]. */
void orc_attend(int32_t n_kv_heads, int32_t head_dim, int32_t n_pages,
                const uint16_t *kpool_layer, const uint16_t *vpool_layer,
                const int32_t *pages, int32_t lo, int32_t pos, int32_t kv_head,
                const double *q, double *o, double *probs)
{
    (void)n_pages;
    const int32_t n = pos - lo + 1;
    const double scale = 1.0 / sqrt((double)head_dim);
    double *s = (double *)malloc(sizeof(double) * (size_t)n);
    double m = -INFINITY;
    for (int32_t j = lo; j <= pos; ++j) {
        int64_t page = pages[j / ORC_PAGE];
        const uint16_t *k = kpool_layer +
            (((page * n_kv_heads + kv_head) * ORC_PAGE + (j % ORC_PAGE)) * (int64_t)head_dim);
        double dot = 0.0;
        for (int32_t i = 0; i < head_dim; ++i) dot += q[i] * orc_bf16_to_f64(k[i]);
        s[j - lo] = dot * scale;
        if (s[j - lo] > m) m = s[j - lo];
    }
    double z = 0.0;
    for (int32_t t = 0; t < n; ++t) {
        s[t] = exp(s[t] - m);
        z += s[t];
    }
    for (int32_t i = 0; i < head_dim; ++i) o[i] = 0.0;
    for (int32_t j = lo; j <= pos; ++j) {
        double p = s[j - lo] / z;
        if (probs) probs[j - lo] = p;
        int64_t page = pages[j / ORC_PAGE];
        const uint16_t *v = vpool_layer +
            (((page * n_kv_heads + kv_head) * ORC_PAGE + (j % ORC_PAGE)) * (int64_t)head_dim);
        for (int32_t i = 0; i < head_dim; ++i) o[i] += p * orc_bf16_to_f64(v[i]);
    }
    free(s);
}

/* Routing weights of a selection (reading of "top-8 softmax routing"): the
 * softmax over the selected experts' logits, taken from their largest. */
void orc_moe_weights(int32_t top_k, const double *logits, const int32_t *idx, double *w)
{
    double m = -INFINITY;
    for (int32_t k = 0; k < top_k; ++k)
        if (logits[idx[k]] > m) m = logits[idx[k]];
    double z = 0.0;
    for (int32_t k = 0; k < top_k; ++k) {
        w[k] = exp(logits[idx[k]] - m);
        z += w[k];
    }
    for (int32_t k = 0; k < top_k; ++k) w[k] /= z;
}

/* MoE routing (reading of "top-8 softmax routing"): the top_k experts by
 * router logit, ties to the lower expert index, listed in that order; weights
 * are the softmax over the selected logits. */
void orc_moe_route(int32_t n_experts, int32_t top_k, const double *logits, int32_t *idx,
                   double *w)
{
    char *taken = (char *)calloc((size_t)n_experts, 1);
    for (int32_t k = 0; k < top_k; ++k) {
        int32_t best = -1;
        for (int32_t e = 0; e < n_experts; ++e) {
            if (taken[e]) continue;
            if (best < 0 || logits[e] > logits[best]) best = e;
        }
        taken[best] = 1;
        idx[k] = best;
    }
    orc_moe_weights(top_k, logits, idx, w);
    free(taken);
}

/* How far a selection of top_k experts is from being a top-k set of the
 * logits: min over the selected logits minus max over the others (+inf when
 * every expert is selected). A top-k set has a margin >= 0; a set whose
 * margin is -t becomes a top-k set once no logit moves by more than t/2. */
double orc_moe_margin(int32_t n_experts, int32_t top_k, const double *logits, const int32_t *idx)
{
    double in_min = INFINITY, out_max = -INFINITY;
    for (int32_t e = 0; e < n_experts; ++e) {
        int taken = 0;
        for (int32_t k = 0; k < top_k; ++k) taken |= idx[k] == e;
        if (taken) {
            if (logits[e] < in_min) in_min = logits[e];
        } else if (logits[e] > out_max) {
            out_max = logits[e];
        }
    }
    return in_min - out_max;
}

/* Gumbel noise for vocabulary entry i of request b (reading of "sıcaklık",
 * temperature sampling, Cohere Megakernel page, "Sınırlar açıkça yazılmış";
 * the Kog AI page's list puts LM-head sampling on the GPU, so the noise is a
 * counter function both sides can evaluate):
 *   key = SM(SM(SM(seed) + step) + b),  h = SM(key + i),
 *   u = (2 (h >> 41) + 1) / 2^24  in (0, 1),   G = -ln(-ln u). */
double orc_gumbel(uint64_t seed, uint32_t step, int32_t b, int32_t i)
{
    uint64_t key = orc_splitmix64(orc_splitmix64(orc_splitmix64(seed) + step) + (uint64_t)b);
    uint64_t h = orc_splitmix64(key + (uint64_t)i);
    double u = (double)(2 * (h >> 41) + 1) * (1.0 / 16777216.0);
    return -log(-log(u));
}

/* Greedy (temperature 0): argmax of the logits. Temperature T > 0:
 * argmax_i (l_i / T + G_i), an exact draw from softmax(l / T) (Gumbel-max).
 * Exact ties go to the lowest index. */
int32_t orc_sample(int32_t vocab, const double *logits, double temperature, uint64_t seed,
                   uint32_t step, int32_t b, double *score_out)
{
    int32_t best = 0;
    double bs = -INFINITY;
    for (int32_t i = 0; i < vocab; ++i) {
        double s = logits[i];
        if (temperature > 0.0) s = s / temperature + orc_gumbel(seed, step, b, i);
        if (s > bs) {
            bs = s;
            best = i;
        }
    }
    if (score_out) *score_out = bs;
    return best;
}

/* Temperature sampling limited to the top_k largest logits (Cohere Megakernel
 * page, "Sınırlar açıkça yazılmış": greedy and temperature sampling, top-k
 * limited). Reading: the candidates are the top_k largest logits, equal
 * logits ordered by index; among them the Gumbel-max rule of orc_sample picks
 * the token (ties to the lower index). Greedy (T <= 0), top_k <= 0 and
 * top_k >= vocab are orc_sample. */
int32_t orc_sample_topk(int32_t vocab, const double *logits, double temperature, int32_t top_k,
                        uint64_t seed, uint32_t step, int32_t b, double *score_out)
{
    if (temperature <= 0.0 || top_k <= 0 || top_k >= vocab)
        return orc_sample(vocab, logits, temperature, seed, step, b, score_out);
    unsigned char *taken = (unsigned char *)calloc((size_t)vocab, 1);
    if (!taken) return -1;
    int32_t best = -1;
    double bs = -INFINITY;
    for (int32_t r = 0; r < top_k; ++r) {
        int32_t m = -1;  /* the largest logit not taken yet, lowest index first */
        for (int32_t i = 0; i < vocab; ++i)
            if (!taken[i] && (m < 0 || logits[i] > logits[m])) m = i;
        taken[m] = 1;
        const double s = logits[m] / temperature + orc_gumbel(seed, step, b, m);
        if (best < 0 || s > bs || (s == bs && m < best)) {
            bs = s;
            best = m;
        }
    }
    free(taken);
    if (score_out) *score_out = bs;
    return best;
}

/* ------------------------------------------------------------ FP8 weights
 * Reading of the pages' 8-bit weights (Kog AI page, "Büyük Üçüncü Taraf MoE
 * Modellerine Ölçeklendirme": FP8/FP4 weights; Cerebras catalogue page,
 * "Model Sıkıştırma Mimarisi ve Şeffaflık": selected 8-bit weights expanded
 * on the fly): OCP FP8 E4M3 (sign, 4-bit exponent of bias 7, 3-bit mantissa,
 * subnormals, largest finite 448; 0x7F/0xFF are NaN) with one fp32 scale per
 * output row: s = amax / 448 (fp32 division; 1 for an all-zero row), code =
 * E4M3 round-to-nearest-even of (w / s) (fp32 division), saturated to +-448.
 * The dequantized weight is code * s; a product applies s to the row's sum. */

double orc_fp8_value(uint8_t q)
{
    const int sgn = q >> 7, e = (q >> 3) & 15, m = q & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return sgn ? -mag : mag;
}

/* E4M3 code of x: nearest representable value, ties to the even mantissa,
 * magnitudes at or above 448 saturated to 448. Done in fp64: the grid step of
 * the binade of |x| is 2^(e-3) (2^-9 below 2^-6), and rint() rounds to even. */
uint8_t orc_fp8_encode(double x)
{
    const uint8_t sgn = (x < 0.0 || (x == 0.0 && signbit(x))) ? 0x80 : 0x00;
    double a = fabs(x);
    if (!(a < 448.0)) return (uint8_t)(sgn | 0x7E);  /* also NaN input: not produced from finite weights */
    if (a < ldexp(1.0, -6)) {
        const double m = rint(a * 512.0);              /* subnormal grid 2^-9; m = 8 is 2^-6 */
        return (uint8_t)(sgn | (uint8_t)m);            /* m <= 8: 8 encodes e = 1, mantissa 0 */
    }
    int e2;
    (void)frexp(a, &e2);                               /* a = f 2^e2, f in [0.5, 1) */
    const int e = e2 - 1;                              /* a in [2^e, 2^(e+1)) */
    double r = rint(ldexp(a, 3 - e));                  /* mantissa grid 8 .. 16 */
    int ee = e, mm;
    if (r >= 16.0) { ee += 1; r = 8.0; }
    mm = (int)r - 8;
    if (ee > 8 || (ee == 8 && mm > 6)) return (uint8_t)(sgn | 0x7E);
    return (uint8_t)(sgn | ((ee + 7) << 3) | mm);
}

void orc_fp8_quantize_rows(int32_t rows, int32_t cols, const uint16_t *W, uint8_t *q, float *scale)
{
    for (int32_t r = 0; r < rows; ++r) {
        const uint16_t *w = W + (int64_t)r * cols;
        float amax = 0.0f;
        for (int32_t c = 0; c < cols; ++c) {
            const float a = (float)fabs(orc_bf16_to_f64(w[c]));
            if (a > amax) amax = a;
        }
        const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
        scale[r] = s;
        for (int32_t c = 0; c < cols; ++c) {
            const float t = (float)orc_bf16_to_f64(w[c]) / s;  /* fp32 quotient */
            q[(int64_t)r * cols + c] = orc_fp8_encode((double)t);
        }
    }
}

/* y_r = scale_r * sum_c value(q[r][c]) x_c, the sum sequential in c (fp64). */
void orc_matvec_fp8(int32_t rows, int32_t cols, const uint8_t *q, const float *scale, const double *x, double *y)
{
#pragma omp parallel for schedule(static) if ((int64_t)rows * cols > (1 << 16))
    for (int32_t r = 0; r < rows; ++r) {
        const uint8_t *w = q + (int64_t)r * cols;
        double acc = 0.0;
        for (int32_t c = 0; c < cols; ++c) acc += orc_fp8_value(w[c]) * x[c];
        y[r] = (double)scale[r] * acc;
    }
}

/* One linear map of the decode step: bf16 weights, or their FP8 form. */
static void lin(int32_t rows, int32_t cols, const uint16_t *W, const orc_fp8_mat *m8, const double *x, double *y)
{
    if (m8) orc_matvec_fp8(rows, cols, m8->q, m8->scale, x, y);
    else orc_matvec(rows, cols, W, x, y);
}

/* ------------------------------------------------------------- decode step */

static void put_bf16(uint16_t *dst, const double *src, int32_t n)
{
    for (int32_t i = 0; i < n; ++i) dst[i] = orc_f64_to_bf16(src[i]);
}

/* One decode step (Cohere Megakernel page, "Megakernel ne demek": the whole
 * decode pass for one new token per request; batch 1-8 per "Sınırlar açıkça
 * yazılmış"). For each request b with p = seq_lens[b] tokens cached:
 *   x = E[tokens_in[b]]
 *   for each layer: n = RMSNorm(x); q, k, v = Wq n, Wk n, Wv n; RoPE(q, k, p);
 *     write bf16(k), bf16(v) at slot p; attention over [lo, p];
 *     h = x + Wo o; n2 = RMSNorm(h); x = h + FFN(n2)  (SwiGLU or MoE)
 *   logits = W_lm RMSNorm(x); token = sample(logits). */
int32_t orc_decode_step_ex(const orc_cfg *cfg, const orc_weights *w, const orc_fp8_weights *w8,
                           uint16_t *kpool, uint16_t *vpool, int32_t n, const int32_t *seq_lens,
                           const int32_t *page_table, const int32_t *tokens_in,
                           const double *temperature, uint64_t seed, uint32_t step,
                           int32_t *tokens_out, double *logits_out, double *layer_x_out,
                           const orc_route_io *route)
{
    const int32_t L = cfg->n_layers, d = cfg->d_model, Hq = cfg->n_q_heads;
    const int32_t Hkv = cfg->n_kv_heads, dh = cfg->head_dim, V = cfg->vocab;
    const int32_t G = Hq / Hkv;
    const int64_t layer_elems = (int64_t)cfg->n_pages * Hkv * ORC_PAGE * dh;
    const int moe = cfg->n_experts > 0;
    if (moe && w8) return -1; /* FP8 weights: dense models */

    /* validate everything before touching the pool */
    for (int32_t b = 0; b < n; ++b) {
        int32_t p = seq_lens[b];
        if (p < 0 || p / ORC_PAGE >= cfg->max_pages_per_seq) return -1;
        if (tokens_in[b] < 0 || tokens_in[b] >= V) return -1;
        for (int32_t pg = 0; pg <= p / ORC_PAGE; ++pg) {
            int32_t id = page_table[(int64_t)b * cfg->max_pages_per_seq + pg];
            if (id < 0 || id >= cfg->n_pages) return -1;
        }
    }
    /* a given selection must name top_k distinct experts in range */
    if (moe && route && route->sel_in) {
        const int32_t E = cfg->n_experts, K = cfg->top_k;
        for (int64_t i = 0; i < (int64_t)n * L; ++i)
            for (int32_t k = 0; k < K; ++k) {
                const int32_t e = route->sel_in[i * K + k];
                if (e < 0 || e >= E) return -1;
                for (int32_t k2 = 0; k2 < k; ++k2)
                    if (route->sel_in[i * K + k2] == e) return -1;
            }
    }

    double *x = (double *)malloc(sizeof(double) * (size_t)d);
    double *nrm = (double *)malloc(sizeof(double) * (size_t)d);
    double *hbuf = (double *)malloc(sizeof(double) * (size_t)d);
    double *q = (double *)malloc(sizeof(double) * (size_t)Hq * dh);
    double *k = (double *)malloc(sizeof(double) * (size_t)Hkv * dh);
    double *v = (double *)malloc(sizeof(double) * (size_t)Hkv * dh);
    double *o = (double *)malloc(sizeof(double) * (size_t)Hq * dh);
    double *y = (double *)malloc(sizeof(double) * (size_t)d);
    double *logits = (double *)malloc(sizeof(double) * (size_t)V);

    for (int32_t b = 0; b < n; ++b) {
        const int32_t p = seq_lens[b];
        const int32_t *pages = page_table + (int64_t)b * cfg->max_pages_per_seq;
        const uint16_t *e = w->embed + (int64_t)tokens_in[b] * d;
        for (int32_t i = 0; i < d; ++i) x[i] = orc_bf16_to_f64(e[i]);

        for (int32_t l = 0; l < L; ++l) {
            uint16_t *kl = kpool + l * layer_elems;
            uint16_t *vl = vpool + l * layer_elems;
            orc_rmsnorm(d, x, w->attn_norm[l], cfg->rms_eps, nrm);
            lin(Hq * dh, d, w->wq[l], w8 ? &w8->wq[l] : NULL, nrm, q);
            lin(Hkv * dh, d, w->wk[l], w8 ? &w8->wk[l] : NULL, nrm, k);
            lin(Hkv * dh, d, w->wv[l], w8 ? &w8->wv[l] : NULL, nrm, v);
            orc_rope(Hq, dh, p, cfg->rope_base, q);
            orc_rope(Hkv, dh, p, cfg->rope_base, k);
            {
                int64_t page = pages[p / ORC_PAGE];
                for (int32_t g = 0; g < Hkv; ++g) {
                    int64_t off = ((page * Hkv + g) * ORC_PAGE + (p % ORC_PAGE)) * (int64_t)dh;
                    put_bf16(kl + off, k + (int64_t)g * dh, dh);
                    put_bf16(vl + off, v + (int64_t)g * dh, dh);
                }
            }
            const int32_t lo = orc_window_lo(p, cfg->window ? cfg->window[l] : 0);
#pragma omp parallel for schedule(static)
            for (int32_t h = 0; h < Hq; ++h)
                orc_attend(Hkv, dh, cfg->n_pages, kl, vl, pages, lo, p, h / G,
                           q + (int64_t)h * dh, o + (int64_t)h * dh, NULL);
            lin(d, Hq * dh, w->wo[l], w8 ? &w8->wo[l] : NULL, o, y);
            for (int32_t i = 0; i < d; ++i) hbuf[i] = x[i] + y[i];
            orc_rmsnorm(d, hbuf, w->ffn_norm[l], cfg->rms_eps, nrm);
            if (!moe && w8) {
                /* SwiGLU on the FP8 matrices: y = W_down (silu(W_gate n2) * (W_up n2)) */
                const int32_t F = cfg->ffn_dim;
                double *g = (double *)malloc(sizeof(double) * (size_t)F);
                double *u = (double *)malloc(sizeof(double) * (size_t)F);
                lin(F, d, NULL, &w8->w_gate[l], nrm, g);
                lin(F, d, NULL, &w8->w_up[l], nrm, u);
                for (int32_t i = 0; i < F; ++i) g[i] = orc_silu(g[i]) * u[i];
                lin(d, F, NULL, &w8->w_down[l], g, y);
                free(g);
                free(u);
            } else if (!moe) {
                orc_swiglu_ffn(d, cfg->ffn_dim, w->w_gate[l], w->w_up[l], w->w_down[l], nrm, y);
            } else {
                const int32_t E = cfg->n_experts, K = cfg->top_k, fe = cfg->expert_ffn_dim;
                double *r = (double *)malloc(sizeof(double) * (size_t)E);
                int32_t *idx = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
                double *wt = (double *)malloc(sizeof(double) * (size_t)K);
                double *ye = (double *)malloc(sizeof(double) * (size_t)d);
                orc_matvec(E, d, w->router[l], nrm, r);
                orc_moe_route(E, K, r, idx, wt);
                const int64_t rl = (int64_t)b * L + l;
                if (route && route->sel_out) memcpy(route->sel_out + rl * K, idx, sizeof(int32_t) * (size_t)K);
                if (route && route->gap_out) {
                    /* own selection: the last one taken against the best left out */
                    route->gap_out[rl] = K < E ? orc_moe_margin(E, K, r, idx) : INFINITY;
                }
                if (route && route->sel_in) {
                    /* continue with the given selection (another valid choice at a
                     * near tie): its experts, weighted by the softmax of their logits */
                    memcpy(idx, route->sel_in + rl * K, sizeof(int32_t) * (size_t)K);
                    orc_moe_weights(K, r, idx, wt);
                }
                if (route && route->margin_out)
                    route->margin_out[rl] = K < E ? orc_moe_margin(E, K, r, idx) : INFINITY;
                for (int32_t i = 0; i < d; ++i) y[i] = 0.0;
                for (int32_t t = 0; t < K; ++t) {
                    int64_t eo = (int64_t)idx[t] * fe * d;
                    orc_swiglu_ffn(d, fe, w->w_gate[l] + eo, w->w_up[l] + eo,
                                   w->w_down[l] + eo, nrm, ye);
                    for (int32_t i = 0; i < d; ++i) y[i] += wt[t] * ye[i];
                }
                free(r);
                free(idx);
                free(wt);
                free(ye);
            }
            for (int32_t i = 0; i < d; ++i) x[i] = hbuf[i] + y[i];
            if (layer_x_out) memcpy(layer_x_out + ((int64_t)b * L + l) * d, x, sizeof(double) * (size_t)d);
        }
        orc_rmsnorm(d, x, w->final_norm, cfg->rms_eps, nrm);
        lin(V, d, w->lm_head, w8 ? &w8->lm_head : NULL, nrm, logits);
        if (logits_out) memcpy(logits_out + (int64_t)b * V, logits, sizeof(double) * (size_t)V);
        double T = temperature ? temperature[b] : 0.0;
        tokens_out[b] = orc_sample(V, logits, T, seed, step, b, NULL);
    }
    free(x);
    free(nrm);
    free(hbuf);
    free(q);
    free(k);
    free(v);
    free(o);
    free(y);
    free(logits);
    return 0;
}

int32_t orc_decode_step_routed(const orc_cfg *cfg, const orc_weights *w, uint16_t *kpool,
                               uint16_t *vpool, int32_t n, const int32_t *seq_lens,
                               const int32_t *page_table, const int32_t *tokens_in,
                               const double *temperature, uint64_t seed, uint32_t step,
                               int32_t *tokens_out, double *logits_out, double *layer_x_out,
                               const orc_route_io *route)
{
    return orc_decode_step_ex(cfg, w, NULL, kpool, vpool, n, seq_lens, page_table, tokens_in, temperature,
                              seed, step, tokens_out, logits_out, layer_x_out, route);
}

/* The decode step with the oracle's own routing, reporting per request the
 * smallest margin over the layers of that routing (+inf for dense models). */
int32_t orc_decode_step(const orc_cfg *cfg, const orc_weights *w, uint16_t *kpool,
                        uint16_t *vpool, int32_t n, const int32_t *seq_lens,
                        const int32_t *page_table, const int32_t *tokens_in,
                        const double *temperature, uint64_t seed, uint32_t step,
                        int32_t *tokens_out, double *logits_out, double *layer_x_out,
                        double *route_gap_out)
{
    const int32_t L = cfg->n_layers;
    double *gaps = NULL;
    orc_route_io io = {NULL, NULL, NULL, NULL};
    if (route_gap_out) {
        gaps = (double *)malloc(sizeof(double) * (size_t)n * (size_t)L);
        io.gap_out = gaps;
    }
    const int32_t rc = orc_decode_step_routed(cfg, w, kpool, vpool, n, seq_lens, page_table, tokens_in,
                                              temperature, seed, step, tokens_out, logits_out,
                                              layer_x_out, route_gap_out ? &io : NULL);
    if (route_gap_out && rc == 0) {
        for (int32_t b = 0; b < n; ++b) {
            double g = INFINITY;
            if (cfg->n_experts > 0)
                for (int32_t l = 0; l < L; ++l)
                    if (gaps[(int64_t)b * L + l] < g) g = gaps[(int64_t)b * L + l];
            route_gap_out[b] = g;
        }
    }
    free(gaps);
    return rc;
}
