// mk_params.h - launch parameters shared by the host runtime and the kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace mk {

constexpr int kPage = 16;           // tokens per KV page
constexpr int kMaxBatch = 8;
constexpr int kMaxSampleTopK = 16;   // largest limited top-k of the sampler
constexpr int kTopKLane = 8;         // logits per lane of a workgroup's top-k selection (lm_head rows per WG <= 64x)
constexpr int kMaxNW = 256;          // workgroups, at most
constexpr int kMaxComputeWaves = 8; // waves that stream weights / K/V, at most
// Compute waves of a decode kernel variant (plus one I/O wave per workgroup).
// Eight keep more of the DMA stream and the compute in flight per CU and let
// two waves per SIMD overlap their waits. Four where eight do not fit: 8-head
// attention groups (their attention needs more registers than nine waves per
// CU leave) and MoE models (expert widths that are not multiples of 8 x 32).
constexpr int compute_waves(int G, bool moe, bool mfma) { return (G == 8 || moe) ? 4 : 8; }
// LDS ring slots (1 KB chunks) per compute wave: 8 x 16 (vector ALU), 8 x 8
// (batch 3..8 matrix-core variant: its operand takes 64 KB of the LDS), 4 x 32,
// or 4 x 16 (batch 3..8 or group size 8).
constexpr int ring_slots(int W, bool mfma, int G) { return W == 8 ? (mfma ? 8 : 16) : ((mfma || G == 8) ? 16 : 32); }
constexpr int kMaxSplit = 4;        // most K-splits of a GEMV stage
constexpr int kChunk = 1024;        // bytes per streamed chunk: 64 lanes x 16 B
constexpr int kCtrlBytes = 2048;   // LDS control block of the decode kernel
constexpr int kMaxExperts = 128;    // MoE: experts per layer (two router logits per lane)
constexpr int kMaxTopK = 8;         // MoE: experts per token
constexpr int kMaxUnion = kMaxBatch * kMaxTopK;  // distinct experts one step can touch
constexpr int kMaxSpan = 4;         // MoE down-projection: experts one workgroup's tiles span
constexpr int kRouteBytes = 1024;   // LDS routing block of the MoE stages
constexpr int kFlagStride = 256;    // flags per flag array are padded to a multiple of this
// Exchange buffers and flags of the allocation-free decode entry point: one
// static device array of this many bytes per device (96 MiB).
constexpr size_t kStaticScratchBytes = (size_t)96 << 20;

// Attention workgroup partials: header words (m_h, l_h) per head, padded to a
// multiple of 4 words, then G x dh values.
constexpr int att_hdr_words(int G) { return (2 * G + 3) / 4 * 4; }
// Segment merge: items (value pairs, header pairs) per lane of the I/O wave;
// the host checks that no slice needs more than 64 * att_merge_pu of either.
constexpr int att_merge_pu(int G, int dh) { return G * dh / 4 <= 128 ? 4 : 8; }

// FP8 weights (E4M3, one fp32 scale per row) use the same tiles with chunks of
// 16 rows x 64 K: lane l holds row(t, l % 16) at k = 64 kb + 8 (l / 16) + e
// (bytes 0..7) and 64 kb + 32 + 8 (l / 16) + e (bytes 8..15), e = 0..7.
// Packed tile layout: a matrix of N rows (N % 16 == 0) and K columns (K % 32 == 0) is
// stored as N/16 tiles; tile t holds K/32 chunks of 1 KB; in chunk (t, kb) the 16 bytes
// of lane l are W[row(t, l % 16)][32 kb + 8 (l / 16) + e], e = 0..7 (the A-operand
// order of the 16x16x32 bf16 MFMA). row() is the identity except for the fused QKV
// matrix (RoPE partners i and i + dh/2 of a head sit at tile rows r and r + 8) and the
// gate/up matrix (tile t: rows 0..7 = gate features 8t..8t+7, rows 8..15 = up features).
struct GemvStage {
    int64_t off;      // byte offset of the matrix inside a layer's packed weights (absolute for lm_head)
    int32_t T;        // tiles
    int32_t nkb;      // chunks per tile (K / 32)
    int32_t S;        // K-splits: WG w handles split s = w * S / NW only
    int32_t ncw;      // chunks per wave per task = nkb / S / W (the W compute waves split each task's K)
    int32_t max_tasks;// most tiles any WG handles
    int32_t K;        // input width
    int32_t tpw;      // 1: each compute wave takes whole tiles (ncw = nkb) instead of a K-slice of every tile
    int32_t te;       // MoE expert stages: tiles per expert (T is then a bound: experts touched x te)
    uint32_t ebytes;  // MoE expert stages: packed bytes per expert
    int64_t soff;     // FP8 weights: offset (floats) of the matrix's row scales in a layer's scales (absolute for lm_head)
};

// flag kinds (per layer), plus two global arrays after the per-layer ones
enum FlagKind { FK_QKV = 0, FK_ATTP = 1, FK_ATT = 2, FK_O = 3, FK_GU = 4, FK_DN = 5, FK_RT = 6, FK_PER_LAYER = 7 };

// Stages of a layer, in order: dense QKV, ATT, O, GU, DN (kinds 0..4); MoE QKV,
// ATT, O, RT (router, kind 6), GU and DN over the selected experts (kinds 3, 4).
// Kind 5 is the final norm + lm_head + sampler stage after the last layer.
enum StageKind { SK_QKV = 0, SK_ATT = 1, SK_O = 2, SK_GU = 3, SK_DN = 4, SK_LM = 5, SK_RT = 6, SK_KINDS = 7 };

struct Params {
    // model
    int32_t L, d, Hq, Hkv, dh, F, V, G;
    float eps;
    int32_t spl;                 // stages per layer: 5 dense, 6 MoE
    int32_t moe, E, topk, fe;    // MoE: experts, experts per token, expert FFN width (moe = 0: dense)
    // packed weights
    const uint8_t* wpack;
    int64_t layer_bytes;
    GemvStage qkv, o, gu, dn, lm, rt;  // gu, dn: one expert's matrices in MoE models; rt: MoE router
    int32_t fp8;                 // weights are FP8 (E4M3 tiles + row scales)
    const float* wscale;         // FP8: row scales, per layer scale_lb floats (QKV, O, GU, DN in packed row order), then lm_head
    int64_t scale_lb;
    const uint16_t* embed;       // [V][d] bf16
    const uint16_t* attn_norm;   // [L][d]
    const uint16_t* ffn_norm;    // [L][d]
    const uint16_t* final_norm;  // [d]
    const float* rope_cs;        // [max_pos][dh/2][2] (cos, sin), fp64 on host rounded to fp32
    int32_t max_pos;
    // K/V pool: [L][n_pages][Hkv][16 * dh] bf16 each, in the attention kernel's page layouts
    uint16_t* kpool;
    uint16_t* vpool;
    int64_t kv_layer_elems;
    int32_t n_pages, mpps;
    const int32_t* window;       // device [L]; 0 = full
    int32_t win_sliding;         // the one nonzero window value (0 if every layer is full)
    // batch
    int32_t n;
    const int32_t* seq_lens;
    const int32_t* page_table;
    const int32_t* tokens_in;
    const float* temperature;    // may be null
    uint64_t seed;
    uint32_t step;
    const int32_t* top_k;        // may be null
    int32_t* tokens_out;
    float* logits_out;           // may be null
    // device scratch exchanged between workgroups: tagged 64-bit words (value, tag)
    uint64_t* q;                 // [8][Hq*dh] fp32
    uint64_t* kvcur;             // [8][Hkv][2][dh] bf16 (in the low 16 bits)
    uint64_t* attp;              // [8*Hkv][NW][hdr + G*dh] fp32 workgroup partials (m, l, o)
    // GEMV operands: plain fp32 read once their producers' flags are up, or (dense
    // vector-ALU variants) tagged 64-bit words polled directly; sized for the latter
    float* atto;                 // [8][Hq*dh] merged attention output
    float* hparts;               // [o.S][8][d] (S <= kMaxSplit)
    float* act;                  // dense [8][F]; MoE [kMaxUnion][8][fe] per selected expert
    float* xparts;               // dense: [dn.S][8][d] (S <= kMaxSplit); MoE: [1][8][d], h + sum of expert outputs
    int32_t xn;                  // parts of x: dn.S dense, 1 MoE
    // Each layer has its own copy of the operand buffers (x: one per layer
    // input, 1..L), so within a launch every address is written once and then
    // only read: readers behind a flag may take it through the L2 they share
    // with the other workgroups of their XCD. Byte strides between copies:
    int64_t atto_lb, h_lb, act_lb, x_lb, rlog_lb;
    float* rlog;                 // MoE router logits [8][E]
    unsigned long long* moe_used;// MoE: running sum over launches and layers of the experts selected
    float* lmpart;               // [NW][8][2]
    float* lmtopk;               // [NW][8][kMaxSampleTopK][2]: each WG's top-k (logit, index) per request
    uint32_t* flags;             // [(L * FK_PER_LAYER + 2) * NWpad + 256]
    uint32_t* err;               // [0] status, [1] where, [2 + lcount % 2] bad-request mask of a launch
    uint32_t epoch;              // value of this launch's flags: above every flag value already in `flags`
    uint32_t tag_base;           // tag of stage sid's exchanged words: tag_base + sid (never 0)
    uint32_t lcount;             // launches of the handle so far (parity picks the bad-request word)
    int32_t* route_dbg;          // optional [L][8][kMaxTopK]: MoE selection of each layer and request (null = off)
    uint64_t wait_ticks;         // 100 MHz ticks
    int32_t NW, NWpad;
    // LDS layout (bytes)
    int32_t lds_units, lds_op, lds_total, maxu;
    int32_t lds_ring;            // the compute waves' DMA rings (R KB each)
    int32_t lds_gain;            // bf16 norm gains of the current / next normalised stage [d]
    int32_t lds_res;             // I/O-wave prefetch: residual rows or RoPE factors [tasks][8][16] fp32
    int32_t lds_part[SK_KINDS];  // per stage kind: partials after that stage's operand
    int32_t lds_route;           // MoE routing block (kRouteBytes)
    int32_t lds_scale;           // FP8: row scales of the current stage's tiles [tasks][16] fp32
    uint64_t* trace;             // optional [NW][spl*L+1][8] timestamps (100 MHz clock), null = off
};

// The host runtime fills Params and passes it by value as the kernel argument;
// the device code reads it at the offsets its own compilation computes. Both
// compilations (hipcc's device and host passes, and the host-only runtime)
// check the same layout here, so a field added on one side only, or a type
// that differs between them, fails to build instead of shifting every later
// field (which would turn pointers into wild addresses on the GPU).
static_assert(sizeof(GemvStage) == 56 && alignof(GemvStage) == 8, "GemvStage layout");
static_assert(sizeof(Params) == 864 && alignof(Params) == 8, "Params size");
static_assert(offsetof(Params, wpack) == 56 && offsetof(Params, qkv) == 72 && offsetof(Params, rt) == 352 &&
                  offsetof(Params, fp8) == 408 && offsetof(Params, wscale) == 416 && offsetof(Params, kpool) == 480,
              "Params layout: model and weights");
static_assert(offsetof(Params, n) == 524 && offsetof(Params, seed) == 560 && offsetof(Params, step) == 568 &&
                  offsetof(Params, q) == 600 && offsetof(Params, atto) == 624 && offsetof(Params, xn) == 656,
              "Params layout: batch and exchange buffers");
static_assert(offsetof(Params, atto_lb) == 664 && offsetof(Params, rlog_lb) == 696 && offsetof(Params, flags) == 736 &&
                  offsetof(Params, epoch) == 752 && offsetof(Params, tag_base) == 756 && offsetof(Params, lcount) == 760,
              "Params layout: copy strides, flags and tags");
static_assert(offsetof(Params, route_dbg) == 768 && offsetof(Params, wait_ticks) == 776 && offsetof(Params, NW) == 784 &&
                  offsetof(Params, lds_part) == 820 && offsetof(Params, lds_scale) == 852 && offsetof(Params, trace) == 856,
              "Params layout: launch shape and LDS offsets");

}  // namespace mk
