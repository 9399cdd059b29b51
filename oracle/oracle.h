/*
 * oracle.h - TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU decode step for a Llama-style
 * pre-norm decoder with paged bf16 K/V. Only the tests, the smoke check and
 * the benchmark's CPU-baseline leg may load it; the product path never does.
 * It shares no code, header or table with the GPU library.
 *
 * Precision: weights and K/V are bf16 (the Cohere Megakernel page, section
 * "Sınırlar açıkça yazılmış", fixes BF16 as the datapath); every other value
 * and every sum is fp64. Dot products are accumulated sequentially in index
 * order.
 *
 * What the pages say the step is: one decode pass of the model per token,
 * batch 1-8, paged KV, ragged lengths, sliding window, greedy and temperature
 * sampling on the GPU (Cohere Megakernel page, "Megakernel ne demek" and
 * "Sınırlar açıkça yazılmış"; Kog page, list under "Standart Çıkarım
 * Yığınları Neden Mikro Saniyeleri Kaybediyor?"). The pages never give the
 * architecture; every reading taken here is listed beside the function that
 * takes it.
 */
#ifndef DPS_ORACLE_H
#define DPS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORC_PAGE 16

typedef struct {
    int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
    double rms_eps, rope_base;
    int32_t n_experts, top_k, expert_ffn_dim; /* 0,0,0 = dense FFN */
    const int32_t *window;                    /* [n_layers]; 0 = full attention */
    int32_t n_pages;                          /* pages in the oracle's own pool */
    int32_t max_pages_per_seq;                /* page-table row stride */
} orc_cfg;

/* bf16 bit patterns, row-major [out][in] like torch.nn.Linear.weight. Per-layer
 * entries are arrays of n_layers pointers. MoE expert tensors are
 * [n_experts][rows][cols] per layer. */
typedef struct {
    const uint16_t *embed;      /* [vocab][d] */
    const uint16_t *final_norm; /* [d] */
    const uint16_t *lm_head;    /* [vocab][d] */
    const uint16_t *const *attn_norm, *const *wq, *const *wk, *const *wv, *const *wo;
    const uint16_t *const *ffn_norm, *const *w_gate, *const *w_up, *const *w_down;
    const uint16_t *const *router; /* MoE only, [n_experts][d] */
} orc_weights;

/* Oracle pool layout (its own): [n_layers][n_pages][n_kv_heads][16][head_dim] bf16. */

double orc_bf16_to_f64(uint16_t h);
uint16_t orc_f64_to_bf16(double x);
uint64_t orc_splitmix64(uint64_t z);

void orc_rmsnorm(int32_t d, const double *x, const uint16_t *g, double eps, double *y);
void orc_matvec(int32_t rows, int32_t cols, const uint16_t *W, const double *x, double *y);
void orc_rope(int32_t n_heads, int32_t head_dim, int32_t pos, double base, double *v);
double orc_silu(double z);
void orc_swiglu_ffn(int32_t d, int32_t f, const uint16_t *w_gate, const uint16_t *w_up,
                    const uint16_t *w_down, const double *n2, double *y);
int32_t orc_window_lo(int32_t pos, int32_t window);
void orc_attend(int32_t n_kv_heads, int32_t head_dim, int32_t n_pages,
                const uint16_t *kpool_layer, const uint16_t *vpool_layer,
                const int32_t *pages, int32_t lo, int32_t pos, int32_t kv_head,
                const double *q, double *o, double *probs);
void orc_moe_route(int32_t n_experts, int32_t top_k, const double *logits, int32_t *idx,
                   double *w);
void orc_moe_weights(int32_t top_k, const double *logits, const int32_t *idx, double *w);
double orc_moe_margin(int32_t n_experts, int32_t top_k, const double *logits, const int32_t *idx);
double orc_gumbel(uint64_t seed, uint32_t step, int32_t b, int32_t i);
int32_t orc_sample(int32_t vocab, const double *logits, double temperature, uint64_t seed,
                   uint32_t step, int32_t b, double *score_out);
int32_t orc_sample_topk(int32_t vocab, const double *logits, double temperature, int32_t top_k,
                        uint64_t seed, uint32_t step, int32_t b, double *score_out);

/* One decode step for n requests. kpool/vpool are the oracle's own pools and
 * receive the new K/V. Returns 0, or -1 on an invalid page id / page table.
 * route_gap_out (optional, [n]): for MoE models, per request the smallest gap
 * over the layers between its top_k-th and (top_k+1)-th router logits (+inf
 * when top_k = n_experts or the model is dense), so a caller can tell a routing
 * decision that rounding could flip. */
int32_t orc_decode_step(const orc_cfg *cfg, const orc_weights *w, uint16_t *kpool,
                        uint16_t *vpool, int32_t n, const int32_t *seq_lens,
                        const int32_t *page_table, const int32_t *tokens_in,
                        const double *temperature, uint64_t seed, uint32_t step,
                        int32_t *tokens_out, double *logits_out, double *layer_x_out, double *route_gap_out);

/* MoE routing in and out of a decode step, per (request b, layer l) at index
 * b * n_layers + l; every member may be NULL.
 *   sel_in   [n][L][top_k]: experts to use instead of the oracle's own top-k
 *            (e.g. another implementation's choice at a near tie); each row
 *            must hold top_k distinct ids in range, else the step returns -1;
 *   sel_out  [n][L][top_k]: the oracle's own top-k, best first;
 *   gap_out  [n][L]: margin (orc_moe_margin) of the oracle's own top-k: the
 *            k-th largest logit minus the (k+1)-th (+inf if top_k = n_experts);
 *   margin_out [n][L]: margin of the selection actually used (sel_in if
 *            given, else the own one); a value below 0 means the used set is
 *            not a top-k set of the oracle's logits. */
typedef struct {
    const int32_t *sel_in;
    int32_t *sel_out;
    double *gap_out;
    double *margin_out;
} orc_route_io;

/* FP8 form of a matrix [rows][cols]: E4M3 codes row-major and one fp32 scale
 * per row (orc_fp8_quantize_rows). */
typedef struct {
    const uint8_t *q;
    const float *scale;
} orc_fp8_mat;
/* The FP8 forms of a dense model's linear maps ([n_layers] arrays, lm_head). */
typedef struct {
    const orc_fp8_mat *wq, *wk, *wv, *wo, *w_gate, *w_up, *w_down;
    orc_fp8_mat lm_head;
} orc_fp8_weights;

double orc_fp8_value(uint8_t q);
uint8_t orc_fp8_encode(double x);
void orc_fp8_quantize_rows(int32_t rows, int32_t cols, const uint16_t *W, uint8_t *q, float *scale);
void orc_matvec_fp8(int32_t rows, int32_t cols, const uint8_t *q, const float *scale, const double *x, double *y);

/* The decode step of orc_decode_step_routed; with w8 non-NULL (dense models
 * only, else -1) every linear map uses its FP8 form instead of w's bf16
 * matrix (embedding rows and norm gains stay bf16). */
int32_t orc_decode_step_ex(const orc_cfg *cfg, const orc_weights *w, const orc_fp8_weights *w8,
                           uint16_t *kpool, uint16_t *vpool, int32_t n, const int32_t *seq_lens,
                           const int32_t *page_table, const int32_t *tokens_in,
                           const double *temperature, uint64_t seed, uint32_t step,
                           int32_t *tokens_out, double *logits_out, double *layer_x_out,
                           const orc_route_io *route);

int32_t orc_decode_step_routed(const orc_cfg *cfg, const orc_weights *w, uint16_t *kpool,
                               uint16_t *vpool, int32_t n, const int32_t *seq_lens,
                               const int32_t *page_table, const int32_t *tokens_in,
                               const double *temperature, uint64_t seed, uint32_t step,
                               int32_t *tokens_out, double *logits_out, double *layer_x_out,
                               const orc_route_io *route);

#ifdef __cplusplus
}
#endif
#endif
