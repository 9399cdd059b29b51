/*
 * mk.h - C ABI of the MI355X (gfx950) small-batch decode step.
 *
 * One call, mk_decode_step, runs one autoregressive decode step of a
 * Llama-style decoder for 1..8 requests as ONE persistent HIP kernel launch:
 * RMSNorm, fused QKV projection with RoPE and paged K/V append, paged GQA
 * split-K attention (full or sliding window), O projection, SwiGLU or top-k
 * MoE FFN, lm_head and a greedy / temperature sampler, ordered on the device
 * by per-stage flags instead of kernel boundaries.
 *
 * What the method is comes from two pages: the Cohere Megakernel page
 * ("Cohere, Megakernel sunum sistemini açık kaynak yaptı", sections
 * "Megakernel ne demek" and "Sınırlar açıkça yazılmış": one persistent kernel
 * per decode step, a task graph instead of full-grid barriers, BF16, batch
 * 1-8, greedy and temperature sampling, continuous batching, ragged lengths,
 * paged KV cache, sliding-window attention) and the Kog AI page (linuxcum.com,
 * "Standart Çıkarım Yığınları Neden Mikro Saniyeleri Kaybediyor?": sampling
 * on the GPU, no kernel boundaries, prefetch across op sections, a weight
 * layout for small batches). The pages give no API: the calls below are this
 * library's own.
 *
 * Conventions for every call:
 *   - status codes only; no call aborts or throws;
 *   - host-checkable arguments are checked before anything is enqueued and a
 *     rejected call changes no state;
 *   - "device" pointers are HIP device memory; "host" pointers are ordinary
 *     host memory; the library never keeps a caller pointer after returning,
 *     except the stream;
 *   - all device work is enqueued on the stream given to mk_create and is
 *     ordered with the caller's other work on that stream; calls return
 *     without waiting unless stated;
 *   - a handle is used by one host thread at a time.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MK_OK = 0,
    MK_ERR_INVALID_ARG = 1,     /* a host-checkable argument is wrong */
    MK_ERR_UNSUPPORTED = 2,     /* a shape the kernels do not support */
    MK_ERR_OOM = 3,             /* device memory or KV pages exhausted */
    MK_ERR_HIP = 4,             /* a HIP runtime call failed */
    MK_ERR_BAD_PAGE = 5,        /* device-side: page id / length / token out of range */
    MK_ERR_DEVICE_TIMEOUT = 6   /* device-side: a bounded wait expired */
} mk_status;

typedef struct mk_handle mk_handle; /* opaque; owned by the library */

#define MK_PAGE_SIZE 16
#define MK_MAX_BATCH 8

/* Model shape. Readings where the pages are silent: pre-norm decoder, no
 * biases, untied lm_head, RMSNorm y = x / sqrt(mean(x^2) + eps) * g,
 * rotate-half RoPE with theta_i = rope_base^(-2i/head_dim) at the absolute
 * position, K cached after RoPE, GQA kv head = floor(h / (Hq / Hkv)),
 * attention scale 1/sqrt(head_dim), SwiGLU silu(gate) * up, MoE top_k by
 * router logit with softmax over the selected logits. */
typedef struct {
    int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn_dim, vocab;
    float rms_eps, rope_base;
    int32_t n_experts, top_k, expert_ffn_dim; /* 0, 0, 0 = dense SwiGLU FFN */
    const int32_t *window;     /* host [n_layers]; 0 = full attention, W > 0 keeps the last W keys; NULL = all full */
    int32_t max_batch;         /* 1..8 */
    int32_t page_size;         /* must be 16 */
    int32_t n_pages;           /* KV pool capacity in pages (each page: 16 tokens x all layers x K and V) */
    int32_t max_pages_per_seq; /* row stride of page tables */
    /* MK_WEIGHTS_BF16 (0): the bf16 weights are streamed as given.
     * MK_WEIGHTS_FP8 (1): mk_create quantizes every linear map (QKV, O,
     * gate/up, down, lm_head) to OCP FP8 E4M3 with one fp32 scale per output
     * row, scale = max |w| / 448 (1 for an all-zero row) and code = E4M3
     * round-to-nearest-even of w / scale (both correctly rounded fp32
     * divisions), saturated at 448; each product applies the scale to its
     * row's sum. Embedding rows, norm gains and K/V stay bf16. Dense models
     * with query groups of 2 only (Kog AI page, "Büyük Üçüncü Taraf MoE
     * Modellerine Ölçeklendirme": FP8/FP4 weights; Cerebras catalogue page,
     * "Model Sıkıştırma Mimarisi ve Şeffaflık": 8-bit weights expanded on the
     * fly). */
    int32_t weight_format;
} mk_model_cfg;

#define MK_WEIGHTS_BF16 0
#define MK_WEIGHTS_FP8 1

/* Weights: device pointers to bf16, row-major [out][in] (the layout of
 * torch.nn.Linear.weight). Per-layer entries are HOST arrays of n_layers
 * device pointers. Dense: w_gate/w_up [ffn_dim][d_model], w_down
 * [d_model][ffn_dim]. MoE: w_gate/w_up [n_experts][expert_ffn_dim][d_model],
 * w_down [n_experts][d_model][expert_ffn_dim], router [n_experts][d_model].
 * embed and lm_head are [vocab][d_model]; the norm gains are [d_model].
 * mk_create copies everything into its own packed buffers: the caller may
 * free these tensors once mk_create has returned and the stream has passed
 * the copy (mk_create synchronises its stream before returning). */
typedef struct {
    const void *embed, *final_norm, *lm_head;
    const void *const *attn_norm, *const *wq, *const *wk, *const *wv, *const *wo;
    const void *const *ffn_norm, *const *w_gate, *const *w_up, *const *w_down;
    const void *const *router; /* MoE only; NULL for dense models */
} mk_weights;

/* One decode step's batch. All arrays are DEVICE memory, read in stream
 * order; the library never writes them. Request b has seq_lens[b] tokens
 * cached (positions 0..seq_lens[b]-1); this step decodes the token at
 * position p = seq_lens[b], writes its K and V into slot p % 16 of page
 * page_table[b][p / 16], and attends over positions [lo, p]. Page-table
 * entries 0 .. p/16 must be valid page ids. The caller advances seq_lens and
 * step between calls and allocates pages ahead of growth. */
typedef struct {
    int32_t n;                  /* 1..max_batch */
    const int32_t *seq_lens;    /* [n] */
    const int32_t *page_table;  /* [n][max_pages_per_seq] */
    const int32_t *tokens_in;   /* [n] token ids in [0, vocab) */
    const float *temperature;   /* [n]; 0 = greedy, > 0 = temperature; NULL = all greedy */
    uint64_t seed;              /* sampler noise key (caller-owned) */
    uint32_t step;              /* sampler noise counter (caller-owned) */
    /* [n] or NULL: at temperature > 0, sample among the top_k largest logits
     * only (Cohere Megakernel page, "Sınırlar açıkça yazılmış": top-k is
     * limited). <= 0 or >= vocab: no limit; 1..MK_MAX_TOP_K: the candidates
     * are the top_k largest logits, equal logits ordered by index, and the
     * Gumbel-max rule below picks among them; values between MK_MAX_TOP_K and
     * vocab are taken as MK_MAX_TOP_K. Greedy requests ignore it.
     * MK_ERR_INVALID_ARG if top_k is given and a workgroup's share of the
     * lm_head rows exceeds what its selection holds (vocabularies above 64 K
     * rows per 128 workgroups). */
    const int32_t *top_k;
} mk_batch;

/* Largest limited top_k (mk_batch.top_k). */
#define MK_MAX_TOP_K 16

/* Create a handle on the current HIP device. Validates cfg, allocates the
 * packed-weight buffer, the K/V pool, the flag arrays and scratch, packs the
 * weights (device to device, once) and builds the RoPE table (fp64 on the
 * host, rounded to fp32). stream: a hipStream_t (NULL = the default stream).
 * Errors: MK_ERR_INVALID_ARG (NULL or inconsistent cfg/weights, unknown
 * weight_format), MK_ERR_UNSUPPORTED (FP8 weights for an MoE model or query
 * groups other than 2, FP8 GEMV widths not multiples of 256; shape outside
 * the kernels' limits: head_dim 64 or
 * 128, group size n_q_heads / n_kv_heads of 2, or 8 with head_dim 128,
 * n_kv_heads <= 8, d_model, n_q_heads * head_dim and ffn_dim (MoE:
 * expert_ffn_dim) multiples of 128, at most one distinct sliding-window size,
 * MoE with at most 128 experts, top_k <= 8 and one layer's packed weights
 * under 2 GiB), MK_ERR_OOM, MK_ERR_HIP. On error *out is NULL. Host-checkable
 * rejections happen before any HIP call.
 * MoE layers (the routing the Kog AI page counts among a decode step's
 * non-GEMM work, "GEMM Disi Isler"): router logits r = W_r n2; per token the
 * top_k experts by logit, exact ties to the lower index; weights = softmax of
 * the selected logits; x' = h + sum_k w_k W_d^k(silu(W_g^k n2) * W_u^k n2).
 * The expert outputs are summed with fp32 atomic adds, so the last bits of a
 * MoE step can vary between runs. */
mk_status mk_create(const mk_model_cfg *cfg, const mk_weights *w, void *stream, mk_handle **out);

/* Static text saying why the calling thread's last mk_create or
 * mk_check_plan failed ("" after a success). */
const char *mk_create_error(void);

/* Host only (no HIP call, no weights, nothing allocated): the planning
 * mk_create does for a device of compute_units CUs (at most 256 are used)
 * and lds_bytes of LDS per workgroup: GEMV partitions, kernel variants and
 * their LDS layouts, the exchange-buffer layout, then a bounds check of every
 * index the kernels form from them (exchange buffers per layer copy and
 * split, 32-bit buffer offsets of tagged words and weight chunks, each
 * workgroup's partition of each matrix, the LDS regions). mk_create runs the
 * same check before it allocates and refuses a plan that fails it.
 * Returns MK_OK, or mk_create's status for the configuration (the reason in
 * mk_create_error). Errors: MK_ERR_INVALID_ARG also for compute_units or
 * lds_bytes < 1. */
mk_status mk_check_plan(const mk_model_cfg *cfg, int32_t compute_units, int32_t lds_bytes);

/* Release every resource of the handle after its stream has drained. NULL is a no-op. */
void mk_destroy(mk_handle *h);

/* Pop n page ids from the pool's free list into pages_out (host [n]). The
 * free list starts as 0..n_pages-1 and hands out the lowest free ids first.
 * All-or-nothing: MK_ERR_OOM leaves the pool unchanged. */
mk_status mk_kv_alloc(mk_handle *h, int32_t n, int32_t *pages_out);

/* Drop one reference to each of n page ids (host [n]); a page whose last
 * reference goes returns to the free list. For a page that was never shared
 * this is the inverse of mk_kv_alloc. MK_ERR_INVALID_ARG (and no change) if
 * any id is out of range, not allocated, or repeated. Same as mk_kv_unref. */
mk_status mk_kv_free(mk_handle *h, int32_t n, const int32_t *pages);

/* Prefix cache (Cohere Megakernel page, "Sınırlar açıkça yazılmış": the
 * engine keeps a prefix cache; Magnitude page, "Bellek ve eşzamanlılık için
 * ne anlama geliyor?": concurrent sessions share prefix caches). Requests
 * that start with the same tokens can hold the same K/V pages: each holder
 * takes a reference. A decode step only appends to the page that holds its
 * position, so pages before it are never written again and sharing them is
 * safe; a shared page that a request will append to must first be made
 * private with mk_kv_cow.
 *
 * mk_kv_ref: take one more reference to each of n allocated, distinct page
 * ids (host [n]). MK_ERR_INVALID_ARG (and no change) if any id is out of
 * range, free, or repeated.
 * mk_kv_unref: drop one reference to each (see mk_kv_free). */
mk_status mk_kv_ref(mk_handle *h, int32_t n, const int32_t *pages);
mk_status mk_kv_unref(mk_handle *h, int32_t n, const int32_t *pages);

/* References held on a page (0: free; -1: id out of range or h NULL). */
int32_t mk_kv_refcount(const mk_handle *h, int32_t page);

/* Copy-on-write of one page for a request about to append to it. If the
 * caller holds the only reference, *page_out = page and nothing happens.
 * Otherwise a free page (the lowest id) is allocated, every layer's K and V
 * blocks of the page are copied into it on the handle's stream (ordered with
 * the decode steps there), the caller's reference moves from page to the new
 * page, and *page_out is the new id for the caller's page table.
 * MK_ERR_INVALID_ARG if page is out of range or free; MK_ERR_OOM (no change)
 * if no page is free; MK_ERR_HIP if the copy cannot be enqueued. */
mk_status mk_kv_cow(mk_handle *h, int32_t page, int32_t *page_out);

/* Number of free pages. */
int32_t mk_kv_available(const mk_handle *h);

/* Device pointers to the K and V pools and their strides in elements
 * (bf16). The block of (layer, page, kv_head) starts at
 * layer*strides[0] + page*strides[1] + kv_head*strides[2] and holds
 * 16 * head_dim elements in the attention kernel's matrix-core order, which
 * is not affine in (slot, dim), so strides[3] = strides[4] = 0. Element
 * (slot s, dim i) of the block is at
 *   K: (i / 32) * 512 + (16 * ((i % 32) / 8) + s) * 8 + i % 8,
 *   V: (i / 16) * 256 + (16 * (s / 4) + i % 16) * 4 + s % 4.
 * mk_kv_write / mk_kv_read do this scatter and gather. Writing K/V for
 * prefilled positions through these pointers is allowed while no decode step
 * is in flight. */
mk_status mk_kv_layout(mk_handle *h, void **k_pool, void **v_pool, int64_t strides[5]);

/* Scatter (mk_kv_write) or gather (mk_kv_read) n token rows of one layer's
 * K (kv = 0) or V (kv = 1): slots is a DEVICE int32 [n] of pool slots
 * (page * 16 + offset), rows is DEVICE bf16 [n][n_kv_heads][head_dim].
 * Bit-exact copies. MK_ERR_BAD_PAGE is latched if a slot is out of range
 * (that row is skipped). */
mk_status mk_kv_write(mk_handle *h, int32_t layer, int32_t kv, int32_t n, const int32_t *slots,
                      const void *rows);
mk_status mk_kv_read(mk_handle *h, int32_t layer, int32_t kv, int32_t n, const int32_t *slots,
                     void *rows);

/* Enqueue one decode step (one persistent kernel launch). tokens_out: DEVICE
 * int32 [batch->n] receives the sampled tokens; logits_out: DEVICE fp32
 * [batch->n][vocab] or NULL. Greedy takes the lowest index among exact
 * maxima; temperature T > 0 takes argmax_i(l_i / T + G_i) with Gumbel noise
 * G_i = -ln(-ln u_i), u_i = (2 (h_i >> 41) + 1) / 2^24,
 * h_i = SM(SM(SM(SM(seed) + step) + b) + i), SM = one SplitMix64 output step.
 * Host-side errors: MK_ERR_INVALID_ARG (NULL pointers, n outside
 * 1..max_batch). Device-side errors are latched: a request whose seq_len,
 * token, temperature or touched page id is out of range gets
 * tokens_out[b] = -1, writes nothing to the pool, and MK_ERR_BAD_PAGE is
 * reported by mk_last_error; an expired bounded wait latches
 * MK_ERR_DEVICE_TIMEOUT and ends the launch. */
mk_status mk_decode_step(mk_handle *h, const mk_batch *batch, int32_t *tokens_out,
                         float *logits_out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode step as mk_decode_step, with the same arguments, results, errors
 * and K/V writes, but its exchange buffers and flags live in a static device
 * array of MK_STATIC_SCRATCH_BYTES per device (the library's own, held by
 * each device it runs on until the process ends) instead of the handle's
 * buffers. The call allocates nothing: no hipMalloc, hipFree or allocating
 * library routine. The first call on a device looks up that device's copy of
 * the array and enqueues a kernel clearing it on the handle's stream; no
 * later call clears anything (flags and exchanged words carry values unique
 * to each call). Every call on a device shares that device's array, so calls
 * that overlap on one device (any handles, any streams) race: serialise
 * them. Errors: as mk_decode_step; MK_ERR_INVALID_ARG also if the current
 * device is not the handle's; MK_ERR_UNSUPPORTED if the model's exchange
 * buffers need more than MK_STATIC_SCRATCH_BYTES (e.g. MoE models with many
 * layers); MK_ERR_HIP if the array cannot be located. Device-side errors are
 * latched in the handle, as for mk_decode_step. */
#define MK_STATIC_SCRATCH_BYTES (96u << 20)
mk_status mk_decode_step_noalloc(mk_handle *h, const mk_batch *batch, int32_t *tokens_out,
                                 float *logits_out);

/* Paged prefill: run one request's prompt tokens through the model, write
 * their K and V into its pages, and sample the token after the last one, so
 * that decode steps continue from position pos0 + n_tokens (Cohere Megakernel
 * page, "Sınırlar açıkça yazılmış": prefill beside the decode kernel;
 * Cerebras disaggregation page, "Ön Doldurma ve Çözümleme Donanım Üzerinde
 * Farklı Talepler Oluşturur": prefill is compute-bound). Computes exactly what
 * n_tokens decode steps at positions pos0, pos0 + 1, ... fed these tokens
 * compute (same readings, causal attention over each position's window),
 * with matrix-core kernels over chunks of up to 1024 tokens. With FP8
 * weights it reads the same E4M3 tiles and row scales as the decode step. */
typedef struct {
    int32_t n_tokens;          /* >= 1 */
    int32_t pos0;              /* tokens already cached before the prompt (their K/V in the pages) */
    const int32_t *tokens;     /* DEVICE [n_tokens] token ids in [0, vocab) */
    const int32_t *page_table; /* DEVICE [max_pages_per_seq]: entries 0 .. (pos0 + n_tokens - 1) / 16 valid;
                                  the pages of positions pos0 .. pos0 + n_tokens - 1 are written, so one
                                  that other requests share (mk_kv_ref) needs a private copy first
                                  (mk_kv_cow), as before a decode step appends to it */
    float temperature;         /* 0 = greedy, > 0 = temperature (as mk_decode_step) */
    uint64_t seed;             /* sampler noise key of the token after the last position: */
    uint32_t step;             /*   as mk_decode_step's (seed, step) with request index */
    int32_t request;           /*   request (0 .. 7) */
} mk_prefill_req;

/* Enqueue a prefill. token_out: DEVICE int32 [1]; logits_out: DEVICE fp32
 * [vocab] or NULL (the last position's logits). The first call allocates the
 * handle's prefill workspace: 1024 x (36 d_model + 4 n_q_heads head_dim +
 * 4 max(d_model, n_q_heads head_dim) + 4 ffn_dim) bytes (120 MiB for d_model
 * 2048, 16 x 128 heads, ffn_dim 8192). Errors: MK_ERR_INVALID_ARG (NULL
 * pointers, n_tokens < 1, pos0 < 0, pos0 + n_tokens beyond max_pages_per_seq
 * x 16, a temperature < 0 or not finite, request outside 0..7),
 * MK_ERR_UNSUPPORTED (MoE models), MK_ERR_OOM (workspace),
 * MK_ERR_HIP. Device-side: an out-of-range token or page id latches
 * MK_ERR_BAD_PAGE (reported by mk_last_error); nothing is written through an
 * out-of-range page id. */
mk_status mk_prefill(mk_handle *h, const mk_prefill_req *req, int32_t *token_out, float *logits_out);

/* Synchronise the handle's stream, then return and clear the latched device
 * error. *where_out (may be NULL) receives the stage id of a timeout or the
 * request index of a bad request, else -1. */
mk_status mk_last_error(mk_handle *h, int32_t *where_out);

/* Per-stage timeline of the decode kernel, for profiling: buf is DEVICE
 * uint64 [workgroups][S * n_layers + 1][8], S = 5 stages per layer (6 for MoE
 * models: QKV, attention, O, router, expert gate/up, expert down), or NULL to
 * stop. Each decode step
 * overwrites it with 100 MHz clock stamps: slot 0 stage start, 1 compute done,
 * 2 own outputs published, 3 producers of the next stage done, 4 next inputs
 * loaded, 5 compute wave 0 finished streaming, 6 attention merge done. */
mk_status mk_set_trace(mk_handle *h, uint64_t *buf);

/* MoE models, for checking the routing: buf is DEVICE int32
 * [n_layers][8][8] or NULL to stop. Each decode step then writes, for every
 * layer l and request b < n, the top_k experts the step selected for it,
 * best first, at buf[(l * 8 + b) * 8 + k], k < top_k (other entries are left
 * as they are). MK_ERR_INVALID_ARG for a NULL or dense handle. */
mk_status mk_set_route_debug(mk_handle *h, int32_t *buf);

/* MoE models, for profiling: *total receives the sum, over the decode steps
 * since the previous call and over their layers, of the number of distinct
 * experts the batch's routing selected (the experts whose weights the step
 * streamed), and the count restarts from 0. Synchronises the stream. 0 for
 * dense models. MK_ERR_INVALID_ARG for NULL arguments. */
mk_status mk_moe_experts_used(mk_handle *h, int64_t *total);

/* Bound on every device-side wait, in microseconds (default 2,000,000). */
mk_status mk_set_wait_limit(mk_handle *h, uint32_t usec);

/* How mk_decode_step launches its kernel. on = 1 (default): a cooperative
 * launch, which guarantees that every workgroup is resident at once, as the
 * flag waits between workgroups require. on = 0: an ordinary launch of the same
 * grid, for tools that cannot follow cooperative launches (rocprofv3's kernel
 * trace). Residency then rests on the grid having at most one workgroup per
 * compute unit and the device running nothing else; if that fails the waits
 * expire and the step reports MK_ERR_DEVICE_TIMEOUT instead of hanging.
 * MK_ERR_INVALID_ARG for other values. */
mk_status mk_set_cooperative(mk_handle *h, int32_t on);

/* Launch shape of the decode kernel: workgroups, threads per workgroup,
 * LDS bytes per workgroup, and the compute path (0 = vector ALU, 1 = MFMA). */
mk_status mk_launch_info(const mk_handle *h, int32_t *workgroups, int32_t *threads,
                         int32_t *lds_bytes, int32_t *path);

/* The kernel variant a step of `batch` requests runs (1 <= batch <= max_batch):
 * its compute waves per workgroup (8, or 4 where 8 do not fit the LDS or the
 * GEMV widths), its DMA ring slots per compute wave, its LDS bytes per
 * workgroup and its compute path (0 = vector ALU, 1 = MFMA). Any output pointer
 * may be NULL. MK_ERR_INVALID_ARG for a NULL handle or a batch out of range. */
mk_status mk_variant_info(const mk_handle *h, int32_t batch, int32_t *compute_waves, int32_t *ring_slots,
                          int32_t *lds_bytes, int32_t *path);

/* Static text for a status code. */
const char *mk_status_str(mk_status s);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
