// mk_api.cpp - host runtime behind the C ABI of include/mk.h: argument checks,
// weight packing, the paged-KV page allocator, work partitions, LDS layout and
// the one-launch-per-step decode call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <cstdio>
#include <set>
#include <vector>

#include "../../include/mk.h"
#include "mk_params.h"
#include "mk_prefill.h"

static_assert(mk::kStaticScratchBytes == (size_t)MK_STATIC_SCRATCH_BYTES, "static scratch size");

namespace mk {
const void* select_kernel(int nb, bool mfma, int dh, int G, int ring, bool moe, int waves, bool fp8);
hipError_t launch_rowscale(const uint16_t* W, int rows, int K, float* out, hipStream_t stream);
hipError_t launch_pack8(uint8_t* dst, int T, int nkb8, int K, int mode, const uint16_t* s0, const uint16_t* s1,
                        const uint16_t* s2, int n0, int n1, int dh, const float* c0, const float* c1, const float* c2,
                        float* sdst, hipStream_t stream);
hipError_t launch_decode(const void* fn, const Params& P, int threads, hipStream_t stream, bool cooperative);
hipError_t launch_pack(uint8_t* dst, int T, int nkb, int K, int mode, const uint16_t* s0, const uint16_t* s1,
                       const uint16_t* s2, int n0, int n1, int dh, hipStream_t stream);
hipError_t launch_kv_copy(uint16_t* pool_layer, const int32_t* slots, uint16_t* rows, int n, int Hkv, int dh, int isv,
                          int64_t n_slots, int dir, uint32_t* err, hipStream_t stream);
// This device's copy of the allocation-free entry point's static scratch (its
// device address, cleared at the first call on the device) and the flag value
// and tag base of one more launch on it.
struct StaticScratch { uint8_t* base; uint32_t epoch, tag_base; };
hipError_t static_scratch_acquire(int device, hipStream_t stream, uint32_t stages, StaticScratch* out);
}  // namespace mk

using namespace mk;

namespace {

struct Variant {  // one compiled kernel, its GEMV partitions and its LDS layout
    const void* fn = nullptr;
    int nb = 1;
    bool mfma = false;
    int ring = 0;  // DMA ring slots (1 KB) per compute wave
    int W = 4;     // compute waves per workgroup
    GemvStage qkv{}, o{}, gu{}, dn{}, lm{}, rt{};
    int lds_units = 0, lds_gain = 0, lds_res = 0, lds_op = 0, lds_ring = 0, lds_total = 0, lds_route = 0, lds_scale = 0;
    int lds_part[SK_KINDS] = {0, 0, 0, 0, 0, 0, 0};
};

// The exchange buffers and flags of one launch: byte offsets inside one block
// (each 256-byte aligned) and the per-layer copy strides. Sized for any batch
// up to kMaxBatch (the kernels index them with kMaxBatch strides).
struct Scratch {
    size_t q = 0, kvcur = 0, attp = 0, atto = 0, hparts = 0, act = 0, xparts = 0, rlog = 0, lmpart = 0,
           lmtopk = 0, flags = 0, total = 0;
    size_t q_bytes = 0, kvcur_bytes = 0, attp_bytes = 0, flags_bytes = 0;
    int64_t atto_lb = 0, h_lb = 0, act_lb = 0, x_lb = 0, rlog_lb = 0;
};

}  // namespace

struct mk_handle {
    mk_model_cfg cfg{};
    std::vector<int32_t> window;
    int win_sliding = 0;
    hipStream_t stream = nullptr;
    int device = 0;
    int NW = 0, NWpad = 0, maxu = 0, upg = 0;
    GemvStage qkv{}, o{}, gu{}, dn{}, lm{}, rt{};
    bool moe = false;
    bool fp8 = false;            // FP8 weights (E4M3 tiles + row scales)
    float* wscale = nullptr;     // FP8 row scales: per layer scale_lb floats, then lm_head's
    int64_t scale_lb = 0;
    int span_max = 1;  // MoE: most experts one WG's down-projection tiles span
    int64_t layer_bytes = 0;
    // device memory
    uint8_t* wpack = nullptr;
    uint16_t *embed = nullptr, *attn_norm = nullptr, *ffn_norm = nullptr, *final_norm = nullptr;
    float* rope = nullptr;
    int max_pos = 0;
    uint16_t *kpool = nullptr, *vpool = nullptr;
    int64_t kv_layer_elems = 0;
    int32_t* window_dev = nullptr;
    uint64_t *q = nullptr, *attp = nullptr;
    float *atto = nullptr, *hparts = nullptr, *act = nullptr, *xparts = nullptr, *rlog = nullptr;
    unsigned long long* moe_used = nullptr;
    float* lmpart = nullptr;
    float* lmtopk = nullptr;
    uint64_t* kvcur = nullptr;
    uint32_t *flags = nullptr, *err = nullptr;
    uint8_t* scratch = nullptr;   // the exchange buffers and flags (layout `sl`)
    Scratch sl;
    uint32_t epoch = 0;           // flag value of the last launch on the handle's own buffers
    uint32_t launches = 0;        // launches of either entry point (bad-request word parity)
    int32_t* route_dbg = nullptr;
    // paged prefill workspace (allocated by the first mk_prefill): one chunk's
    // residual stream, norm scales, q, the residual GEMMs' partial sums, the
    // operand blocks (of x, h and the attention output; of the SwiGLU
    // activations), and the last position's logits
    float *pf_x = nullptr, *pf_rs = nullptr, *pf_q = nullptr, *pf_part = nullptr, *pf_logits = nullptr;
    uint8_t *pf_blk = nullptr, *pf_blk_act = nullptr;
    uint32_t wait_usec = 2000000;
    bool cooperative = true;
    uint64_t* trace = nullptr;
    Variant var[3];  // [0] VALU batch 1, [1] VALU batch 2, [2] MFMA batch <= 8
    // page allocator
    std::set<int32_t> free_pages;
    std::vector<int32_t> refs;  // references held on each page (0: free)
    std::vector<void*> allocs;
};

namespace {

bool hip_ok(hipError_t e) { return e == hipSuccess; }

template <class T>
mk_status dalloc(mk_handle* h, T** p, size_t bytes) {
    void* q = nullptr;
    if (bytes == 0) bytes = 16;
    if (hipMalloc(&q, bytes) != hipSuccess) {
        (void)hipGetLastError();
        return MK_ERR_OOM;
    }
    h->allocs.push_back(q);
    *p = static_cast<T*>(q);
    return MK_OK;
}

void free_all(mk_handle* h) {
    if (h->stream || true) (void)hipStreamSynchronize(h->stream);
    for (void* p : h->allocs) (void)hipFree(p);
    h->allocs.clear();
}

// WG w -> split s and tiles [t0, t1); identical to the device function.
void part_of(const GemvStage& g, int w, int NW, int* s, int* t0, int* t1) {
    *s = (int)(((long)w * g.S) / NW);
    int f0 = (int)(((long)*s * NW + g.S - 1) / g.S);
    int f1 = (int)(((long)(*s + 1) * NW + g.S - 1) / g.S);
    int nw = f1 - f0, wi = w - f0;
    *t0 = (int)(((long)wi * g.T) / nw);
    *t1 = (int)(((long)(wi + 1) * g.T) / nw);
}

// Partition of a GEMV with `rows` outputs and K inputs. Linear stages (no
// nonlinear epilogue) may split K across workgroups: while there are fewer
// tiles than workgroups, and up to min_split splits to bound the operand each
// workgroup holds in LDS. The W compute waves split each task's K.
GemvStage make_stage(int64_t off, int rows, int K, int NW, int W, bool may_split, int min_split, int kw) {
    GemvStage g{};
    g.off = off;
    g.T = (rows + 15) / 16;
    g.nkb = K / kw;  // chunks per tile: 32 K of bf16, or 64 K of FP8
    g.K = K;
    g.S = 1;
    if (may_split) {
        while (g.S < kMaxSplit && g.nkb % (W * g.S * 2) == 0 && (g.T * g.S * 2 <= NW || g.S < min_split)) g.S *= 2;
    }
    g.ncw = g.nkb / g.S / W;
    g.max_tasks = 0;
    for (int w = 0; w < NW; ++w) {
        int s, t0, t1;
        part_of(g, w, NW, &s, &t0, &t1);
        g.max_tasks = std::max(g.max_tasks, t1 - t0);
    }
    return g;
}

int64_t stage_bytes(const GemvStage& g) { return (int64_t)g.T * g.nkb * kChunk; }

// An MoE expert stage: per selected expert a matrix of `rows` x K, tiles taken
// in (expert, tile) order and split evenly over the workgroups, each compute
// wave taking whole tiles. T is the bound for nu_max selected experts.
GemvStage make_expert_stage(int64_t off, int rows, int K, int NW, int nu_max) {
    GemvStage g{};
    g.off = off;
    g.te = rows / 16;
    g.nkb = K / 32;
    g.K = K;
    g.S = 1;
    g.tpw = 1;
    g.ncw = g.nkb;
    g.T = nu_max * g.te;
    g.ebytes = (uint32_t)((int64_t)g.te * g.nkb * kChunk);
    g.max_tasks = (g.T + NW - 1) / NW;
    return g;
}

// LDS layout of one kernel variant: control block, attention unit tables,
// then per stage the operand (inputs) followed by that stage's partials, then
// the compute waves' DMA rings.
bool layout(mk_handle* h, Variant& v, int lds_limit) {
    const mk_model_cfg& c = h->cfg;
    const int NBo = v.mfma ? 8 : v.nb;
    const int G = c.n_q_heads / c.n_kv_heads, dh = c.head_dim;
    auto align = [](int x) { return (x + 255) & ~255; };
    const int W = v.W;
    const int units = 2 * W * h->maxu * h->upg * 4;
    v.lds_units = kCtrlBytes;  // after the control block
    v.lds_gain = align(v.lds_units + units);
    v.lds_route = align(v.lds_gain + c.d_model * 2);
    v.lds_scale = align(v.lds_route + (h->moe ? kRouteBytes : 0));
    int scale_tasks = 0;  // FP8: row scales of the largest stage partition
    if (h->fp8)
        for (const GemvStage* g : {&v.qkv, &v.o, &v.gu, &v.dn, &v.lm}) scale_tasks = std::max(scale_tasks, g->max_tasks);
    v.lds_res = align(v.lds_scale + scale_tasks * 16 * 4);
    // residual rows prefetched per tile: QKV (RoPE factors), O, and the dense down-projection
    const int res_tasks = std::max(v.qkv.max_tasks, std::max(v.o.max_tasks, h->moe ? 0 : v.dn.max_tasks));
    v.lds_op = align(v.lds_res + res_tasks * kMaxBatch * 16 * 4);
    const int pb = v.mfma ? 512 : v.nb * 16 * 4;
    const GemvStage* st[SK_KINDS] = {&v.qkv, nullptr, &v.o, &v.gu, &v.dn, &v.lm, h->moe ? &v.rt : nullptr};
    int total = 0;
    for (int k = 0; k < SK_KINDS; ++k) {
        int op, part;
        if (k == SK_RT && !h->moe) continue;
        if (h->moe && k == SK_DN) {
            // the activations of each expert slot the WG's tiles span; one partial per tile
            op = h->span_max * st[k]->K * NBo * 4;
            part = st[k]->max_tasks * pb;
        } else if (k == 1) {
            // q and k~/v~ of each compute wave; the segment merge's weights, headers and products
            const int pu = att_merge_pu(G, dh);
            op = std::max(W * G * dh * 4 + W * 2 * dh * 2, G * 256 * 4 + 2 * 64 * pu * 4 + 64 * pu * 16);
            part = W * (16 + G * dh) * 4;
        } else {
            // (MoE gate/up has the router's operand: same K, same place)
            const int Ks = st[k]->K / st[k]->S;
            op = Ks * NBo * 4;
            part = st[k]->max_tasks * (st[k]->tpw ? 1 : W) * pb;
        }
        v.lds_part[k] = align(v.lds_op + op);
        total = std::max(total, align(v.lds_part[k] + part));
    }
    v.lds_ring = (total + 1023) & ~1023;
    v.lds_total = v.lds_ring + W * v.ring * kChunk;
    return v.lds_total <= lds_limit;
}

Scratch scratch_layout(const mk_model_cfg& c, bool moe, int NW, int NWpad) {
    const int L = c.n_layers, d = c.d_model, Hq = c.n_q_heads, Hkv = c.n_kv_heads, dh = c.head_dim;
    const int G = Hq / Hkv;
    const int GR = att_hdr_words(G) + G * dh;
    // q, k~/v~ and attention partials are tagged 64-bit words; GEMV operands are
    // fp32 or tagged words (dense vector-ALU variants), sized for the latter, one
    // copy per layer (x: one per layer input 1..L, index 0 unused)
    const size_t xq = (size_t)kMaxBatch * Hq * dh, xkv = (size_t)kMaxBatch * Hkv * 2 * dh,
                 xattp = (size_t)kMaxBatch * Hkv * NW * GR, xparts = (size_t)kMaxSplit * kMaxBatch * d,
                 xact = moe ? (size_t)kMaxUnion * kMaxBatch * c.expert_ffn_dim : (size_t)kMaxBatch * c.ffn_dim,
                 xrlog = (size_t)kMaxBatch * std::max(1, (int)c.n_experts);
    Scratch S;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = (off + std::max<size_t>(bytes, 16) + 255) & ~(size_t)255;
        return at;
    };
    S.q_bytes = xq * 8;
    S.kvcur_bytes = xkv * 8;
    S.attp_bytes = xattp * 8;
    S.q = take(S.q_bytes);
    S.kvcur = take(S.kvcur_bytes);
    S.attp = take(S.attp_bytes);
    S.atto = take(xq * 8 * L);
    S.hparts = take(xparts * 8 * L);
    S.act = take(xact * 8 * L);
    S.xparts = take(xparts * 8 * (L + 1));
    S.rlog = take(xrlog * 4 * L);
    S.lmpart = take((size_t)NW * kMaxBatch * 2 * 4);
    S.lmtopk = take((size_t)NW * kMaxBatch * kMaxSampleTopK * 2 * 4);
    S.flags_bytes = ((size_t)(L * FK_PER_LAYER + 2) * NWpad + 256) * 4;
    S.flags = take(S.flags_bytes);
    S.total = off;
    S.atto_lb = (int64_t)xq * 8;
    S.h_lb = (int64_t)xparts * 8;
    S.act_lb = (int64_t)xact * 8;
    S.x_lb = (int64_t)xparts * 8;
    S.rlog_lb = (int64_t)xrlog * 4;
    return S;
}

// Host-side bounds check of everything a launch indexes, for every variant the
// handle may run and every workgroup, layer and stage: the exchange buffers
// (the largest index each kernel formula forms against the buffer's size, per
// layer copy and split), the byte offsets of tagged words and weight chunks
// (32-bit buffer offsets), the GEMV partitions, and the LDS regions. Run by
// mk_create before anything is allocated and by mk_check_plan on the host
// alone. Returns nullptr or the first violation found.
const char* check_extents(const mk_handle* h) {
    const mk_model_cfg& c = h->cfg;
    const Scratch& S = h->sl;
    const int64_t L = c.n_layers, d = c.d_model, Hq = c.n_q_heads, Hkv = c.n_kv_heads, dh = c.head_dim;
    const int64_t G = Hq / Hkv, NW = h->NW, B = kMaxBatch;
    const int64_t GR = att_hdr_words((int)G) + G * dh;
    const int64_t act_row = h->moe ? c.expert_ffn_dim : c.ffn_dim;
    const int64_t E = std::max(1, (int)c.n_experts);
    static thread_local char msg[160];
    auto bad = [&](const char* what, int64_t need, int64_t have) {
        snprintf(msg, sizeof msg, "%s: needs %lld bytes, has %lld", what, (long long)need, (long long)have);
        return msg;
    };
    // region sizes in the scratch block (next offset minus this one)
    const int64_t q_sz = (int64_t)(S.kvcur - S.q), kv_sz = (int64_t)(S.attp - S.kvcur), attp_sz = (int64_t)(S.atto - S.attp),
                  atto_sz = (int64_t)(S.hparts - S.atto), h_sz = (int64_t)(S.act - S.hparts),
                  act_sz = (int64_t)(S.xparts - S.act), x_sz = (int64_t)(S.rlog - S.xparts),
                  rlog_sz = (int64_t)(S.lmpart - S.rlog), lmp_sz = (int64_t)(S.lmtopk - S.lmpart),
                  lmt_sz = (int64_t)(S.flags - S.lmtopk), fl_sz = (int64_t)(S.total - S.flags);
    // QKV epilogue: q words b Hq dh + head dh + i (+ dh/2); k~/v~ words ((b Hkv + g) 2 + isv) dh + i (+ dh/2)
    if ((B * Hq * dh) * 8 > q_sz) return bad("q", B * Hq * dh * 8, q_sz);
    if ((((B - 1) * Hkv + Hkv - 1) * 2 + 1) * dh * 8 + dh * 8 > kv_sz) return bad("k~/v~", B * Hkv * 2 * dh * 8, kv_sz);
    // attention partials: record (seg NW + slice) GR + GR words, seg < max_batch Hkv, slice < NW
    if (((c.max_batch * Hkv - 1) * NW + NW) * GR * 8 > attp_sz) return bad("attention partials", (c.max_batch * Hkv * NW) * GR * 8, attp_sz);
    // merged attention output of layer l: word b Hq dh + ... (+4), copy stride atto_lb
    if ((L - 1) * S.atto_lb + B * Hq * dh * 8 > atto_sz) return bad("attention output copies", L * B * Hq * dh * 8, atto_sz);
    if (S.atto_lb < B * Hq * dh * 8) return bad("attention output stride", B * Hq * dh * 8, S.atto_lb);
    // O / DN parts: word (s B + b) d + 16 t + r with s < S, t < T; x has L + 1 copies
    int smax_o = 1, smax_dn = 1;
    for (const Variant& v : h->var) {
        if (!v.fn) continue;
        smax_o = std::max(smax_o, v.o.S);
        if (!h->moe) smax_dn = std::max(smax_dn, v.dn.S);
    }
    if (smax_o > kMaxSplit || smax_dn > kMaxSplit) return "a split count exceeds kMaxSplit";
    const int64_t h_need = (int64_t)smax_o * B * d * 8, x_need = (int64_t)smax_dn * B * d * 8;
    if ((L - 1) * S.h_lb + h_need > h_sz || S.h_lb < h_need) return bad("h parts copies", L * h_need, h_sz);
    if (L * S.x_lb + x_need > x_sz || S.x_lb < x_need) return bad("x parts copies", (L + 1) * x_need, x_sz);
    // activations: dense word b F + 8 t + r; MoE fp32 (u B + b) fe + ..., u < selected experts
    const int64_t nu_max = h->moe ? std::min<int64_t>(c.n_experts, (int64_t)c.max_batch * c.top_k) : 1;
    if (nu_max > kMaxUnion) return "more selected experts per step than kMaxUnion";
    const int64_t act_need = h->moe ? nu_max * B * act_row * 4 : B * act_row * 8;
    if ((L - 1) * S.act_lb + act_need > act_sz || S.act_lb < act_need) return bad("activation copies", L * act_need, act_sz);
    // router logits b E + e (e < E), sampler partials, flags
    if (h->moe && ((L - 1) * S.rlog_lb + B * E * 4 > rlog_sz || S.rlog_lb < B * E * 4)) return bad("router logits", L * B * E * 4, rlog_sz);
    if (NW * B * 2 * 4 > lmp_sz) return bad("sampler partials", NW * B * 2 * 4, lmp_sz);
    if (NW * B * kMaxSampleTopK * 2 * 4 > lmt_sz) return bad("sampler top-k partials", NW * B * kMaxSampleTopK * 2 * 4, lmt_sz);
    if (NW > h->NWpad) return "more workgroups than the flag arrays' stride";
    if (((L * FK_PER_LAYER + 1) * h->NWpad + NW) * 4 > fl_sz) return bad("flags", ((L * FK_PER_LAYER + 2) * h->NWpad) * 4, fl_sz);
    // tagged words and parts are addressed with 32-bit buffer offsets from each region's base
    for (int64_t sz : {q_sz, kv_sz, attp_sz, atto_sz, h_sz, act_sz, x_sz})
        if (sz >= (1ll << 31)) return "an exchange buffer exceeds 2 GiB (32-bit buffer offsets)";
    // per variant: GEMV partitions, weight chunk offsets, LDS regions
    for (const Variant& v : h->var) {
        if (!v.fn) continue;
        for (const GemvStage* g : {&v.qkv, &v.o, &v.gu, &v.dn, &v.lm, &v.rt}) {
            if (g == &v.rt && !h->moe) continue;
            if (h->moe && (g == &v.gu || g == &v.dn)) {
                if ((int64_t)c.n_experts * g->ebytes >= (1ll << 31)) return "an expert stage exceeds 2 GiB";
                continue;
            }
            if ((int64_t)g->T * g->nkb * kChunk >= (1ll << 31)) return "a weight matrix exceeds 2 GiB (32-bit chunk offsets)";
            if (g->tpw ? (g->S != 1 || g->ncw != g->nkb)
                       : (g->S < 1 || g->nkb % g->S != 0 || g->ncw * g->S * v.W != g->nkb))
                return "a GEMV split does not tile K";
            for (int w = 0; w < NW; ++w) {
                int sp, t0, t1;
                part_of(*g, w, NW, &sp, &t0, &t1);
                if (sp < 0 || sp >= g->S || t0 < 0 || t1 > g->T || t1 - t0 > g->max_tasks)
                    return "a workgroup's GEMV partition leaves the matrix";
                // last chunk a wave streams: split mode ((t1 - 1) nkb + s nkb / S + (W - 1) ncw + ncw - 1) KB,
                // whole-tile mode ((t1 - 1) nkb + nkb - 1) KB
                const int64_t end = g->tpw ? (int64_t)t1 * g->nkb
                                           : (int64_t)(t1 - 1) * g->nkb + (int64_t)sp * (g->nkb / g->S) + (int64_t)v.W * g->ncw;
                if (t1 > t0 && end * kChunk > (int64_t)g->T * g->nkb * kChunk)
                    return "a wave's weight chunks leave the matrix";
            }
        }
        // LDS: control block, unit tables, gains, routing, scales, residual rows,
        // operand, each kind's partials, rings: in order and inside the total
        const int regions[] = {kCtrlBytes, v.lds_units, v.lds_gain, v.lds_route, v.lds_scale, v.lds_res, v.lds_op};
        for (size_t i = 1; i < sizeof regions / sizeof regions[0]; ++i)
            if (regions[i] < regions[i - 1]) return "LDS regions out of order";
        for (int k = 0; k < SK_KINDS; ++k)
            if (v.lds_part[k] && (v.lds_part[k] < v.lds_op || v.lds_part[k] > v.lds_ring)) return "LDS partials outside their region";
        if (v.lds_ring + v.W * v.ring * kChunk != v.lds_total || v.lds_ring % 1024 != 0) return "LDS rings misplaced";
    }
    return nullptr;
}

}  // namespace

extern "C" {

const char* mk_status_str(mk_status s) {
    switch (s) {
        case MK_OK: return "ok";
        case MK_ERR_INVALID_ARG: return "invalid argument";
        case MK_ERR_UNSUPPORTED: return "unsupported shape";
        case MK_ERR_OOM: return "out of memory or KV pages";
        case MK_ERR_HIP: return "HIP runtime error";
        case MK_ERR_BAD_PAGE: return "page id, length, token or temperature out of range";
        case MK_ERR_DEVICE_TIMEOUT: return "device wait timed out";
    }
    return "unknown status";
}

namespace {
thread_local const char* g_create_error = "";
mk_status why(mk_status s, const char* reason) {
    g_create_error = reason;
    return s;
}
}  // namespace

const char* mk_create_error(void) { return g_create_error; }

namespace {
// mk_create, or with dry_cus > 0 its planning alone on the host: partitions,
// kernel variants and layouts for a device of dry_cus compute units and
// dry_lds bytes of LDS per workgroup, then check_extents; no HIP call, no
// weights read, nothing allocated.
mk_status create_impl(const mk_model_cfg* cfg, const mk_weights* w, void* stream, mk_handle** out, int dry_cus,
                      int dry_lds) {
    const bool dry = dry_cus > 0;
    g_create_error = "";
    if (!out) return why(MK_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!cfg || (!w && !dry)) return why(MK_ERR_INVALID_ARG, "cfg or weights is NULL");
    const mk_model_cfg& c = *cfg;
    if (c.n_layers < 1 || c.d_model < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.head_dim < 1 || c.vocab < 1 ||
        c.max_batch < 1 || c.max_batch > MK_MAX_BATCH || c.page_size != MK_PAGE_SIZE || c.n_pages < 1 ||
        c.max_pages_per_seq < 1 || !(c.rms_eps >= 0.f) || !(c.rope_base > 0.f) || c.n_q_heads % c.n_kv_heads != 0)
        return why(MK_ERR_INVALID_ARG, "a model or pool size is out of range");
    const bool moe = c.n_experts != 0 || c.top_k != 0 || c.expert_ffn_dim != 0;
    if (moe) {
        if (c.n_experts < 1 || c.top_k < 1 || c.top_k > c.n_experts || c.expert_ffn_dim < 1)
            return why(MK_ERR_INVALID_ARG, "inconsistent MoE sizes");
    } else if (c.ffn_dim < 1) {
        return why(MK_ERR_INVALID_ARG, "ffn_dim < 1");
    }
    if (!dry && (!w->embed || !w->final_norm || !w->lm_head || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
                 !w->ffn_norm || !w->w_gate || !w->w_up || !w->w_down || (moe && !w->router)))
        return why(MK_ERR_INVALID_ARG, "a weight pointer is NULL");
    for (int l = 0; l < c.n_layers && !dry; ++l)
        if (!w->attn_norm[l] || !w->wq[l] || !w->wk[l] || !w->wv[l] || !w->wo[l] || !w->ffn_norm[l] || !w->w_gate[l] ||
            !w->w_up[l] || !w->w_down[l] || (moe && !w->router[l]))
            return why(MK_ERR_INVALID_ARG, "a per-layer weight pointer is NULL");
    const int G = c.n_q_heads / c.n_kv_heads;
    const int dh = c.head_dim;
    if ((dh != 64 && dh != 128) || (G != 2 && G != 8) || (G == 8 && dh != 128) || c.n_kv_heads > 8 || c.d_model % 128 != 0 ||
        (c.n_q_heads * dh) % 128 != 0 || (moe ? c.expert_ffn_dim : c.ffn_dim) % 128 != 0)
        return why(MK_ERR_UNSUPPORTED, "shape outside the kernels' limits (head_dim, group size, multiples of 128)");
    if (moe && (c.n_experts > kMaxExperts || c.top_k > kMaxTopK))
        return why(MK_ERR_UNSUPPORTED, "more than 128 experts or top_k above 8");
    if (c.weight_format != MK_WEIGHTS_BF16 && c.weight_format != MK_WEIGHTS_FP8)
        return why(MK_ERR_INVALID_ARG, "unknown weight_format");
    if (c.weight_format == MK_WEIGHTS_FP8 && (moe || G != 2))
        return why(MK_ERR_UNSUPPORTED, "FP8 weights need a dense model with query groups of 2");
    int win_sliding = 0;
    std::vector<int32_t> window(c.n_layers, 0);
    if (c.window) {
        for (int l = 0; l < c.n_layers; ++l) {
            if (c.window[l] < 0) return why(MK_ERR_INVALID_ARG, "negative window");
            window[l] = c.window[l];
            if (c.window[l] > 0) {
                if (win_sliding && win_sliding != c.window[l])
                    return why(MK_ERR_UNSUPPORTED, "more than one sliding-window size");
                win_sliding = c.window[l];
            }
        }
    }

    if (win_sliding && c.n_layers > 64)
        return why(MK_ERR_UNSUPPORTED, "sliding windows with more than 64 layers");

    mk_handle* h = new (std::nothrow) mk_handle();
    if (!h) return MK_ERR_OOM;
    h->cfg = c;
    h->cfg.window = nullptr;
    h->window = window;
    h->win_sliding = win_sliding;
    h->stream = static_cast<hipStream_t>(stream);
    mk_status st = MK_OK;
    auto fail = [&](mk_status s) {
        if (!dry) free_all(h);
        delete h;
        return s;
    };
    int cus = dry_cus, lds_limit = dry_lds;
    if (!dry && (!hip_ok(hipGetDevice(&h->device)) ||
                 !hip_ok(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device)) ||
                 !hip_ok(hipDeviceGetAttribute(&lds_limit, hipDeviceAttributeMaxSharedMemoryPerBlock, h->device))))
        return fail(MK_ERR_HIP);
    if (cus > 256) cus = 256;  // the attention merge handles at most 256 workgroup partials per segment
    h->NW = cus;
    h->NWpad = (cus + kFlagStride - 1) / kFlagStride * kFlagStride;
    const int L = c.n_layers, d = c.d_model, Hq = c.n_q_heads, Hkv = c.n_kv_heads, F = c.ffn_dim, V = c.vocab;
    const int NW = h->NW;

    const bool fp8 = c.weight_format == MK_WEIGHTS_FP8;
    const int kw = fp8 ? 64 : 32;  // K per 1 KB chunk
    // partitions and packed layout: per layer QKV, O, then the dense gate/up and
    // down, or the MoE router and every expert's gate/up and down
    int64_t off = 0;
    h->moe = moe;
    h->fp8 = fp8;
    // the packed layout and the handle's checks use four compute waves (the
    // fewest a variant has); variants with eight re-partition below
    const int W = 4;
    h->qkv = make_stage(off, (Hq + 2 * Hkv) * dh, d, NW, W, false, 1, kw);
    off += stage_bytes(h->qkv);
    h->o = make_stage(off, d, Hq * dh, NW, W, true, 1, kw);
    off += stage_bytes(h->o);
    if (moe) {
        const int E = c.n_experts, fe = c.expert_ffn_dim;
        const int nu_max = std::min(E, c.max_batch * c.top_k);
        h->rt = make_stage(off, E, d, NW, W, false, 1, kw);
        off += stage_bytes(h->rt);
        h->gu = make_expert_stage(off, 2 * fe, d, NW, nu_max);
        off += (int64_t)E * h->gu.ebytes;
        h->dn = make_expert_stage(off, d, fe, NW, nu_max);
        off += (int64_t)E * h->dn.ebytes;
        if (off >= (1ll << 31)) return fail(why(MK_ERR_UNSUPPORTED, "one layer's packed weights would exceed 2 GiB"));
        // experts spanned by one WG's down-projection tiles, for every union size
        h->span_max = 1;
        for (int nu = 1; nu <= nu_max; ++nu)
            for (int w2 = 0; w2 < NW; ++w2) {
                const long T4 = (long)nu * h->dn.te;
                const long d0 = (long)w2 * T4 / NW, d1 = (long)(w2 + 1) * T4 / NW;
                if (d1 > d0) h->span_max = std::max(h->span_max, (int)((d1 - 1) / h->dn.te - d0 / h->dn.te + 1));
            }
        if (h->span_max > kMaxSpan)
            return fail(why(MK_ERR_UNSUPPORTED, "expert down-projection tiles span too many experts per workgroup"));
    } else {
        h->gu = make_stage(off, 2 * F, d, NW, W, false, 1, kw);
        off += stage_bytes(h->gu);
        h->dn = make_stage(off, d, F, NW, W, true, 1, kw);
        off += stage_bytes(h->dn);
    }
    h->layer_bytes = off;
    h->lm = make_stage((int64_t)L * off, V, d, NW, W, false, 1, kw);
    for (const GemvStage* g : {&h->qkv, &h->o, &h->gu, &h->dn, &h->lm})
        if (g->ncw < 1 || g->nkb % (W * g->S) != 0)
            return fail(why(MK_ERR_UNSUPPORTED, fp8 ? "a GEMV width is not a multiple of 64 x the compute waves (FP8)"
                                                    : "a GEMV width is not a multiple of 32 x the compute waves"));
    if (fp8) {
        // row scales: per layer QKV, O, gate/up, down (packed row order), then lm_head
        h->qkv.soff = 0;
        h->o.soff = h->qkv.soff + (int64_t)h->qkv.T * 16;
        h->gu.soff = h->o.soff + (int64_t)h->o.T * 16;
        h->dn.soff = h->gu.soff + (int64_t)h->gu.T * 16;
        h->scale_lb = h->dn.soff + (int64_t)h->dn.T * 16;
        h->lm.soff = (int64_t)L * h->scale_lb;
    }
    if (moe && (h->rt.ncw < 1 || h->rt.nkb % W != 0))
        return fail(why(MK_ERR_UNSUPPORTED, "a GEMV width is not a multiple of 32 x the compute waves"));

    // The segment merge gives each (partial, 4-value quad) pair and each (head,
    // partial) header one item of the I/O wave, at most 64 * att_merge_pu each.
    // A segment has at most NW / Hkv + 2 workgroup partials (the Hkv segments of a
    // request share its pages equally); it is merged by nm of its ns workgroups
    // (ns - 1 when its first workgroup starts with another segment, else ns), and
    // slice me of nm holds quads [me QD / nm, (me + 1) QD / nm), QD = G dh / 4.
    {
        const int QD = G * dh / 4, cap = 64 * att_merge_pu(G, dh);
        const int ns_max = std::min(NW, NW / Hkv + 2);
        for (int ns = 1; ns <= ns_max; ++ns)
            for (int nm = std::max(1, ns - 1); nm <= ns; ++nm)
                for (int me = 0; me < nm; ++me) {
                    const int q0 = me * QD / nm, q1 = (me + 1) * QD / nm;
                    if (q1 <= q0) continue;
                    const int nh = (4 * q1 - 1) / dh - 4 * q0 / dh + 1;
                    if (ns * (q1 - q0) > cap || nh * ns > cap)
                        return fail(why(MK_ERR_UNSUPPORTED, "attention merge slices exceed the I/O wave's items"));
                }
    }

    // attention geometry and unit-table size
    h->upg = 1;  // attention is split at page granularity
    const int max_seg = c.max_batch * Hkv;
    if (W * NW - max_seg < 1) return fail(why(MK_ERR_UNSUPPORTED, "more attention segments than waves"));
    const long max_units = (long)max_seg * c.max_pages_per_seq;
    h->maxu = (int)((max_units + (W * NW - max_seg) - 1) / (W * NW - max_seg)) + 1;
    h->max_pos = c.max_pages_per_seq * kPage;

    // kernel variants
    const int nbs[3] = {1, 2, 8};
    for (int i = 0; i < 3; ++i) {
        if (c.max_batch < nbs[i] && !(i == 2 && c.max_batch > 2)) continue;  // only the variants max_batch needs
        Variant& v = h->var[i];
        v.nb = nbs[i];
        v.mfma = i == 2;
        // the variant's preferred compute-wave count first, four if eight do not
        // fit (LDS) or do not divide the GEMV widths; the linear stages split K
        // further when the operand would not fit beside the rings
        bool fits = false;
        const int Wpref = compute_waves(G, moe, v.mfma);
        for (int W2 = Wpref; W2 >= 4 && !fits; W2 /= 2) {
            v.W = W2;
            v.ring = ring_slots(v.W, v.mfma, G);
            v.fn = select_kernel(v.nb, v.mfma, dh, G, v.ring, moe, v.W, fp8);
            if (!v.fn) return fail(why(MK_ERR_UNSUPPORTED, "no kernel instantiated for this head_dim / group size"));
            for (int ms = 1; ms <= kMaxSplit && !fits; ms *= 2) {
                v.qkv = make_stage(h->qkv.off, (Hq + 2 * Hkv) * dh, d, NW, v.W, false, 1, kw);
                v.gu = moe ? h->gu : make_stage(h->gu.off, 2 * F, d, NW, v.W, false, 1, kw);
                v.lm = make_stage(h->lm.off, V, d, NW, v.W, false, 1, kw);
                if (v.mfma && v.W == 8) {
                    // lm_head in whole-tile mode: each wave takes whole tiles, so the
                    // partials are one per tile (not per wave): 8 tiles x 8 waves of
                    // [16][8] floats would not fit beside the 64 KB operand
                    v.lm.tpw = 1;
                    v.lm.ncw = v.lm.nkb;
                }
                v.rt = moe ? make_stage(h->rt.off, c.n_experts, d, NW, v.W, false, 1, kw) : h->rt;
                // The matrix-core variant keeps O unsplit when its operand is no wider
                // than gate/up's (which is never split): half the workgroups stream O, but
                // the next stage reads one part of h instead of up to four (dense2b_b8
                // 2.338 -> 2.318 ms). The LDS-driven splits (ms) are down's.
                const bool o_unsplit = v.mfma && (int64_t)Hq * dh <= d;
                v.o = make_stage(h->o.off, d, Hq * dh, NW, v.W, !o_unsplit, o_unsplit ? 1 : ms, kw);
                v.dn = moe ? h->dn : make_stage(h->dn.off, d, F, NW, v.W, true, ms, kw);
                v.qkv.soff = h->qkv.soff;
                v.o.soff = h->o.soff;
                v.gu.soff = h->gu.soff;
                v.dn.soff = h->dn.soff;
                v.lm.soff = h->lm.soff;
                bool widths = true;
                for (const GemvStage* g : {&v.qkv, &v.o, &v.gu, &v.dn, &v.lm, &v.rt}) {
                    if ((g == &v.gu || g == &v.dn) && moe) continue;  // expert stages: whole tiles per wave
                    if (g == &v.rt && !moe) continue;
                    widths = widths && g->ncw >= 1 && g->nkb % (v.W * g->S) == 0;
                }
                if (!widths) {
                    if (v.W == 4)
                        return fail(why(MK_ERR_UNSUPPORTED, fp8 ? "a GEMV width is not a multiple of 256 (FP8)"
                                                                : "a GEMV width is not a multiple of 128"));
                    break;  // try four waves
                }
                fits = layout(h, v, lds_limit);
            }
        }
        if (!fits) {
            static thread_local char msg[128];
            snprintf(msg, sizeof msg, "the kernel's LDS layout needs %d bytes, the limit is %d", v.lds_total, lds_limit);
            return fail(why(MK_ERR_UNSUPPORTED, msg));
        }
        if (dry) continue;
        if (!hip_ok(hipFuncSetAttribute(v.fn, hipFuncAttributeMaxDynamicSharedMemorySize, v.lds_total)))
            return fail(MK_ERR_HIP);
        int occ = 0;
        if (!hip_ok(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, v.fn, (v.W + 1) * 64, v.lds_total)) || occ < 1)
            return fail(why(MK_ERR_UNSUPPORTED, "the kernel cannot be resident (registers or LDS)"));
    }
    h->sl = scratch_layout(c, moe, NW, h->NWpad);
    if (const char* e = check_extents(h)) return fail(why(MK_ERR_UNSUPPORTED, e));

    // device memory
    const int64_t wbytes = (int64_t)L * h->layer_bytes + stage_bytes(h->lm);
    h->kv_layer_elems = (int64_t)c.n_pages * Hkv * kPage * dh;
    if (c.n_pages > 0 && (int64_t)c.n_pages * Hkv * kPage * dh * 2 >= (1ll << 31))
        return fail(why(MK_ERR_UNSUPPORTED, "one layer's K or V pool would exceed 2 GiB"));
    if (dry) {
        delete h;
        return MK_OK;
    }
    if ((st = dalloc(h, &h->wpack, wbytes)) != MK_OK) return fail(st);
    float* rowscale = nullptr;  // FP8: one source matrix's row scales at a time (stream-ordered reuse)
    if (fp8) {
        const int64_t nsc = (int64_t)L * h->scale_lb + (int64_t)h->lm.T * 16;
        const int64_t nrow = std::max<int64_t>({(int64_t)Hq * dh, (int64_t)F, (int64_t)d, (int64_t)V});
        if ((st = dalloc(h, &h->wscale, (size_t)nsc * 4)) != MK_OK) return fail(st);
        if ((st = dalloc(h, &rowscale, (size_t)nrow * 3 * 4)) != MK_OK) return fail(st);
    }
    if ((st = dalloc(h, &h->embed, (size_t)V * d * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->attn_norm, (size_t)L * d * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->ffn_norm, (size_t)L * d * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->final_norm, (size_t)d * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->rope, (size_t)h->max_pos * (dh / 2) * 2 * 4)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->kpool, (size_t)L * h->kv_layer_elems * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->vpool, (size_t)L * h->kv_layer_elems * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->window_dev, (size_t)L * 4)) != MK_OK) return fail(st);
    // exchange buffers and flags in one block (layout h->sl), zeroed at creation
    // (no word holds a valid tag, no flag is raised)
    if ((st = dalloc(h, &h->scratch, h->sl.total)) != MK_OK) return fail(st);
    {
        uint8_t* b = h->scratch;
        h->q = reinterpret_cast<uint64_t*>(b + h->sl.q);
        h->kvcur = reinterpret_cast<uint64_t*>(b + h->sl.kvcur);
        h->attp = reinterpret_cast<uint64_t*>(b + h->sl.attp);
        h->atto = reinterpret_cast<float*>(b + h->sl.atto);
        h->hparts = reinterpret_cast<float*>(b + h->sl.hparts);
        h->act = reinterpret_cast<float*>(b + h->sl.act);
        h->xparts = reinterpret_cast<float*>(b + h->sl.xparts);
        h->rlog = reinterpret_cast<float*>(b + h->sl.rlog);
        h->lmpart = reinterpret_cast<float*>(b + h->sl.lmpart);
        h->lmtopk = reinterpret_cast<float*>(b + h->sl.lmtopk);
        h->flags = reinterpret_cast<uint32_t*>(b + h->sl.flags);
    }
    if ((st = dalloc(h, &h->moe_used, 8)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->err, 64)) != MK_OK) return fail(st);
    hipStream_t s = h->stream;
    if (!hip_ok(hipMemsetAsync(h->scratch, 0, h->sl.total, s)) || !hip_ok(hipMemsetAsync(h->err, 0, 64, s)) ||
        !hip_ok(hipMemsetAsync(h->kpool, 0, (size_t)L * h->kv_layer_elems * 2, s)) ||
        !hip_ok(hipMemsetAsync(h->vpool, 0, (size_t)L * h->kv_layer_elems * 2, s)) ||
        !hip_ok(hipMemsetAsync(h->moe_used, 0, 8, s)))
        return fail(MK_ERR_HIP);

    // RoPE table: fp64 on the host, rounded to fp32; [pos][dh/2][cos, sin]
    {
        std::vector<float> tab((size_t)h->max_pos * (dh / 2) * 2);
        for (int p = 0; p < h->max_pos; ++p)
            for (int i = 0; i < dh / 2; ++i) {
                const double theta = std::pow((double)c.rope_base, -2.0 * i / dh);
                const double a = (double)p * theta;
                tab[((size_t)p * (dh / 2) + i) * 2] = (float)std::cos(a);
                tab[((size_t)p * (dh / 2) + i) * 2 + 1] = (float)std::sin(a);
            }
        if (!hip_ok(hipMemcpyAsync(h->rope, tab.data(), tab.size() * 4, hipMemcpyHostToDevice, s)) ||
            !hip_ok(hipMemcpyAsync(h->window_dev, window.data(), (size_t)L * 4, hipMemcpyHostToDevice, s)) ||
            !hip_ok(hipStreamSynchronize(s)))
            return fail(MK_ERR_HIP);
    }
    // copies of the small tensors
    if (!hip_ok(hipMemcpyAsync(h->embed, w->embed, (size_t)V * d * 2, hipMemcpyDeviceToDevice, s)) ||
        !hip_ok(hipMemcpyAsync(h->final_norm, w->final_norm, (size_t)d * 2, hipMemcpyDeviceToDevice, s)))
        return fail(MK_ERR_HIP);
    for (int l = 0; l < L; ++l)
        if (!hip_ok(hipMemcpyAsync(h->attn_norm + (size_t)l * d, w->attn_norm[l], (size_t)d * 2, hipMemcpyDeviceToDevice, s)) ||
            !hip_ok(hipMemcpyAsync(h->ffn_norm + (size_t)l * d, w->ffn_norm[l], (size_t)d * 2, hipMemcpyDeviceToDevice, s)))
            return fail(MK_ERR_HIP);
    // packing (device to device)
    auto U = [](const void* p) { return static_cast<const uint16_t*>(p); };
    if (fp8) {
        // FP8: each source matrix's row scales (c0, c1, c2 in rowscale), then its
        // quantized tiles and the scales in packed row order
        const int64_t nrow = std::max<int64_t>({(int64_t)Hq * dh, (int64_t)F, (int64_t)d, (int64_t)V});
        float* c0 = rowscale;
        float* c1 = rowscale + nrow;
        float* c2 = rowscale + 2 * nrow;
        for (int l = 0; l < L; ++l) {
            uint8_t* lb = h->wpack + (int64_t)l * h->layer_bytes;
            float* sl = h->wscale + (int64_t)l * h->scale_lb;
            if (!hip_ok(launch_rowscale(U(w->wq[l]), Hq * dh, d, c0, s)) || !hip_ok(launch_rowscale(U(w->wk[l]), Hkv * dh, d, c1, s)) ||
                !hip_ok(launch_rowscale(U(w->wv[l]), Hkv * dh, d, c2, s)) ||
                !hip_ok(launch_pack8(lb + h->qkv.off, h->qkv.T, h->qkv.nkb, d, 1, U(w->wq[l]), U(w->wk[l]), U(w->wv[l]), Hq * dh,
                                     Hkv * dh, dh, c0, c1, c2, sl + h->qkv.soff, s)) ||
                !hip_ok(launch_rowscale(U(w->wo[l]), d, Hq * dh, c0, s)) ||
                !hip_ok(launch_pack8(lb + h->o.off, h->o.T, h->o.nkb, Hq * dh, 0, U(w->wo[l]), nullptr, nullptr, d, 0, dh, c0,
                                     nullptr, nullptr, sl + h->o.soff, s)) ||
                !hip_ok(launch_rowscale(U(w->w_gate[l]), F, d, c0, s)) || !hip_ok(launch_rowscale(U(w->w_up[l]), F, d, c1, s)) ||
                !hip_ok(launch_pack8(lb + h->gu.off, h->gu.T, h->gu.nkb, d, 2, U(w->w_gate[l]), U(w->w_up[l]), nullptr, F, F, dh,
                                     c0, c1, nullptr, sl + h->gu.soff, s)) ||
                !hip_ok(launch_rowscale(U(w->w_down[l]), d, F, c0, s)) ||
                !hip_ok(launch_pack8(lb + h->dn.off, h->dn.T, h->dn.nkb, F, 0, U(w->w_down[l]), nullptr, nullptr, d, 0, dh, c0,
                                     nullptr, nullptr, sl + h->dn.soff, s)))
                return fail(MK_ERR_HIP);
        }
        if (!hip_ok(launch_rowscale(U(w->lm_head), V, d, c0, s)) ||
            !hip_ok(launch_pack8(h->wpack + h->lm.off, h->lm.T, h->lm.nkb, d, 0, U(w->lm_head), nullptr, nullptr, V, 0, dh, c0,
                                 nullptr, nullptr, h->wscale + h->lm.soff, s)))
            return fail(MK_ERR_HIP);
    } else {
    for (int l = 0; l < L; ++l) {
        uint8_t* lb = h->wpack + (int64_t)l * h->layer_bytes;
        if (!hip_ok(launch_pack(lb + h->qkv.off, h->qkv.T, h->qkv.nkb, d, 1, U(w->wq[l]), U(w->wk[l]), U(w->wv[l]),
                                Hq * dh, Hkv * dh, dh, s)) ||
            !hip_ok(launch_pack(lb + h->o.off, h->o.T, h->o.nkb, Hq * dh, 0, U(w->wo[l]), nullptr, nullptr, d, 0, dh, s)))
            return fail(MK_ERR_HIP);
        if (moe) {
            const int E = c.n_experts, fe = c.expert_ffn_dim;
            if (!hip_ok(launch_pack(lb + h->rt.off, h->rt.T, h->rt.nkb, d, 0, U(w->router[l]), nullptr, nullptr, E, 0, dh, s)))
                return fail(MK_ERR_HIP);
            for (int e = 0; e < E; ++e) {
                const size_t eo = (size_t)e * fe * d;  // [E][fe][d] and [E][d][fe] alike
                if (!hip_ok(launch_pack(lb + h->gu.off + (int64_t)e * h->gu.ebytes, h->gu.te, h->gu.nkb, d, 2,
                                        U(w->w_gate[l]) + eo, U(w->w_up[l]) + eo, nullptr, fe, fe, dh, s)) ||
                    !hip_ok(launch_pack(lb + h->dn.off + (int64_t)e * h->dn.ebytes, h->dn.te, h->dn.nkb, fe, 0,
                                        U(w->w_down[l]) + eo, nullptr, nullptr, d, 0, dh, s)))
                    return fail(MK_ERR_HIP);
            }
        } else if (!hip_ok(launch_pack(lb + h->gu.off, h->gu.T, h->gu.nkb, d, 2, U(w->w_gate[l]), U(w->w_up[l]), nullptr,
                                       F, F, dh, s)) ||
                   !hip_ok(launch_pack(lb + h->dn.off, h->dn.T, h->dn.nkb, F, 0, U(w->w_down[l]), nullptr, nullptr, d, 0,
                                       dh, s))) {
            return fail(MK_ERR_HIP);
        }
    }
    if (!hip_ok(launch_pack(h->wpack + h->lm.off, h->lm.T, h->lm.nkb, d, 0, static_cast<const uint16_t*>(w->lm_head),
                            nullptr, nullptr, V, 0, dh, s)))
        return fail(MK_ERR_HIP);
    }
    if (!hip_ok(hipStreamSynchronize(s))) return fail(MK_ERR_HIP);

    // page allocator: 0..n_pages-1 free, lowest first
    h->refs.assign(c.n_pages, 0);
    for (int i = 0; i < c.n_pages; ++i) h->free_pages.insert(h->free_pages.end(), i);
    *out = h;
    return MK_OK;
}
}  // namespace

mk_status mk_create(const mk_model_cfg* cfg, const mk_weights* w, void* stream, mk_handle** out) {
    return create_impl(cfg, w, stream, out, 0, 0);
}

mk_status mk_check_plan(const mk_model_cfg* cfg, int32_t compute_units, int32_t lds_bytes) {
    if (compute_units < 1 || lds_bytes < 1) return why(MK_ERR_INVALID_ARG, "compute_units and lds_bytes must be >= 1");
    mk_handle* h = nullptr;
    return create_impl(cfg, nullptr, nullptr, &h, compute_units, lds_bytes);
}

void mk_destroy(mk_handle* h) {
    if (!h) return;
    free_all(h);
    delete h;
}

mk_status mk_kv_alloc(mk_handle* h, int32_t n, int32_t* pages_out) {
    if (!h || n < 0 || (n > 0 && !pages_out)) return MK_ERR_INVALID_ARG;
    if ((size_t)n > h->free_pages.size()) return MK_ERR_OOM;
    for (int32_t i = 0; i < n; ++i) {
        auto it = h->free_pages.begin();
        pages_out[i] = *it;
        h->refs[*it] = 1;
        h->free_pages.erase(it);
    }
    return MK_OK;
}

// n held, distinct page ids (the checks of mk_kv_ref / mk_kv_unref)
static bool held_distinct(const mk_handle* h, int32_t n, const int32_t* pages) {
    std::set<int32_t> seen;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t p = pages[i];
        if (p < 0 || p >= h->cfg.n_pages || h->refs[p] <= 0 || !seen.insert(p).second) return false;
    }
    return true;
}

mk_status mk_kv_ref(mk_handle* h, int32_t n, const int32_t* pages) {
    if (!h || n < 0 || (n > 0 && !pages) || !held_distinct(h, n, pages)) return MK_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i)
        if (h->refs[pages[i]] == INT32_MAX) return MK_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) ++h->refs[pages[i]];
    return MK_OK;
}

mk_status mk_kv_unref(mk_handle* h, int32_t n, const int32_t* pages) {
    if (!h || n < 0 || (n > 0 && !pages) || !held_distinct(h, n, pages)) return MK_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i)
        if (--h->refs[pages[i]] == 0) h->free_pages.insert(pages[i]);
    return MK_OK;
}

mk_status mk_kv_free(mk_handle* h, int32_t n, const int32_t* pages) { return mk_kv_unref(h, n, pages); }

int32_t mk_kv_refcount(const mk_handle* h, int32_t page) {
    if (!h || page < 0 || page >= h->cfg.n_pages) return -1;
    return h->refs[page];
}

mk_status mk_kv_cow(mk_handle* h, int32_t page, int32_t* page_out) {
    if (!h || !page_out || page < 0 || page >= h->cfg.n_pages || h->refs[page] <= 0) return MK_ERR_INVALID_ARG;
    if (h->refs[page] == 1) {
        *page_out = page;
        return MK_OK;
    }
    if (h->free_pages.empty()) return MK_ERR_OOM;
    const int32_t np = *h->free_pages.begin();
    // the page's blocks of every layer, K and V: one strided copy per pool
    // (rows = layers, each row the page's n_kv_heads x 16 x head_dim elements)
    const size_t blk = (size_t)h->cfg.n_kv_heads * kPage * h->cfg.head_dim * sizeof(uint16_t);
    const size_t pitch = (size_t)h->kv_layer_elems * sizeof(uint16_t);
    for (uint16_t* pool : {h->kpool, h->vpool}) {
        uint8_t* base = reinterpret_cast<uint8_t*>(pool);
        if (!hip_ok(hipMemcpy2DAsync(base + (size_t)np * blk, pitch, base + (size_t)page * blk, pitch, blk,
                                     (size_t)h->cfg.n_layers, hipMemcpyDeviceToDevice, h->stream)))
            return MK_ERR_HIP;
    }
    h->free_pages.erase(h->free_pages.begin());
    h->refs[np] = 1;
    --h->refs[page];
    *page_out = np;
    return MK_OK;
}

int32_t mk_kv_available(const mk_handle* h) { return h ? (int32_t)h->free_pages.size() : 0; }

mk_status mk_kv_layout(mk_handle* h, void** k_pool, void** v_pool, int64_t strides[5]) {
    if (!h || !k_pool || !v_pool || !strides) return MK_ERR_INVALID_ARG;
    *k_pool = h->kpool;
    *v_pool = h->vpool;
    const int64_t dh = h->cfg.head_dim;
    strides[4] = 0;  // the (slot, dim) order inside a block is not affine
    strides[3] = 0;
    strides[2] = kPage * dh;
    strides[1] = (int64_t)h->cfg.n_kv_heads * kPage * dh;
    strides[0] = h->kv_layer_elems;
    return MK_OK;
}

static mk_status kv_copy(mk_handle* h, int32_t layer, int32_t kv, int32_t n, const int32_t* slots, void* rows, int dir) {
    if (!h || layer < 0 || layer >= h->cfg.n_layers || (kv != 0 && kv != 1) || n < 0 || (n > 0 && (!slots || !rows)))
        return MK_ERR_INVALID_ARG;
    uint16_t* pool = (kv ? h->vpool : h->kpool) + (int64_t)layer * h->kv_layer_elems;
    const hipError_t e = launch_kv_copy(pool, slots, static_cast<uint16_t*>(rows), n, h->cfg.n_kv_heads, h->cfg.head_dim, kv,
                                        (int64_t)h->cfg.n_pages * kPage, dir, h->err, h->stream);
    return e == hipSuccess ? MK_OK : MK_ERR_HIP;
}

mk_status mk_kv_write(mk_handle* h, int32_t layer, int32_t kv, int32_t n, const int32_t* slots, const void* rows) {
    return kv_copy(h, layer, kv, n, slots, const_cast<void*>(rows), 0);
}

mk_status mk_kv_read(mk_handle* h, int32_t layer, int32_t kv, int32_t n, const int32_t* slots, void* rows) {
    return kv_copy(h, layer, kv, n, slots, rows, 1);
}

}  // extern "C"

namespace {

// Host-side checks of a decode call and the variant it runs (null: rejected).
const Variant* check_step(const mk_handle* h, const mk_batch* b, const int32_t* tokens_out) {
    if (!h || !b || !tokens_out || !b->seq_lens || !b->page_table || !b->tokens_in) return nullptr;
    if (b->n < 1 || b->n > h->cfg.max_batch) return nullptr;
    const Variant& v = b->n == 1 ? h->var[0] : b->n == 2 ? h->var[1] : h->var[2];
    if (!v.fn) return nullptr;
    if (b->top_k && v.lm.max_tasks * 16 > 64 * kTopKLane) return nullptr;  // vocabulary too wide per WG
    return &v;
}

// Launch parameters of one step on the exchange buffers and flags at `base`
// (layout h->sl); epoch, tag_base and lcount are the caller's.
Params step_params(const mk_handle* h, const Variant& v, const mk_batch* b, int32_t* tokens_out, float* logits_out,
                   uint8_t* base) {
    static_assert(kMaxSampleTopK == MK_MAX_TOP_K, "top-k bound");
    const mk_model_cfg& c = h->cfg;
    const Scratch& sl = h->sl;
    Params P{};
    P.L = c.n_layers;
    P.d = c.d_model;
    P.Hq = c.n_q_heads;
    P.Hkv = c.n_kv_heads;
    P.dh = c.head_dim;
    P.F = c.ffn_dim;
    P.V = c.vocab;
    P.G = c.n_q_heads / c.n_kv_heads;
    P.eps = c.rms_eps;
    P.moe = h->moe ? 1 : 0;
    P.spl = h->moe ? 6 : 5;
    P.E = c.n_experts;
    P.topk = c.top_k;
    P.fe = c.expert_ffn_dim;
    P.rt = v.rt;
    P.moe_used = h->moe_used;
    P.wpack = h->wpack;
    P.layer_bytes = h->layer_bytes;
    P.qkv = v.qkv;
    P.o = v.o;
    P.gu = v.gu;
    P.dn = v.dn;
    P.lm = v.lm;
    P.embed = h->embed;
    P.attn_norm = h->attn_norm;
    P.ffn_norm = h->ffn_norm;
    P.final_norm = h->final_norm;
    P.rope_cs = h->rope;
    P.max_pos = h->max_pos;
    P.kpool = h->kpool;
    P.vpool = h->vpool;
    P.kv_layer_elems = h->kv_layer_elems;
    P.n_pages = c.n_pages;
    P.mpps = c.max_pages_per_seq;
    P.window = h->window_dev;
    P.win_sliding = h->win_sliding;
    P.n = b->n;
    P.seq_lens = b->seq_lens;
    P.page_table = b->page_table;
    P.tokens_in = b->tokens_in;
    P.temperature = b->temperature;
    P.top_k = b->top_k;
    P.seed = b->seed;
    P.step = b->step;
    P.tokens_out = tokens_out;
    P.logits_out = logits_out;
    P.q = reinterpret_cast<uint64_t*>(base + sl.q);
    P.kvcur = reinterpret_cast<uint64_t*>(base + sl.kvcur);
    P.attp = reinterpret_cast<uint64_t*>(base + sl.attp);
    P.atto = reinterpret_cast<float*>(base + sl.atto);
    P.hparts = reinterpret_cast<float*>(base + sl.hparts);
    P.act = reinterpret_cast<float*>(base + sl.act);
    P.xparts = reinterpret_cast<float*>(base + sl.xparts);
    P.rlog = reinterpret_cast<float*>(base + sl.rlog);
    P.lmpart = reinterpret_cast<float*>(base + sl.lmpart);
    P.lmtopk = reinterpret_cast<float*>(base + sl.lmtopk);
    P.flags = reinterpret_cast<uint32_t*>(base + sl.flags);
    P.xn = h->moe ? 1 : v.dn.S;
    P.atto_lb = sl.atto_lb;
    P.h_lb = sl.h_lb;
    P.act_lb = sl.act_lb;
    P.x_lb = sl.x_lb;
    P.rlog_lb = sl.rlog_lb;
    P.err = h->err;
    P.wait_ticks = (uint64_t)h->wait_usec * 100u;  // 100 MHz constant clock
    P.NW = h->NW;
    P.NWpad = h->NWpad;
    P.lds_units = v.lds_units;
    P.lds_op = v.lds_op;
    for (int k = 0; k < SK_KINDS; ++k) P.lds_part[k] = v.lds_part[k];
    P.lds_route = v.lds_route;
    P.lds_scale = v.lds_scale;
    P.fp8 = h->fp8 ? 1 : 0;
    P.wscale = h->wscale;
    P.scale_lb = h->scale_lb;
    P.lds_total = v.lds_total;
    P.lds_ring = v.lds_ring;
    P.lds_gain = v.lds_gain;
    P.lds_res = v.lds_res;
    P.maxu = h->maxu;
    P.trace = h->trace;
    P.route_dbg = h->route_dbg;
    return P;
}

}  // namespace

extern "C" {

mk_status mk_decode_step(mk_handle* h, const mk_batch* b, int32_t* tokens_out, float* logits_out) {
    const Variant* v = check_step(h, b, tokens_out);
    if (!v) return MK_ERR_INVALID_ARG;
    Params P = step_params(h, *v, b, tokens_out, logits_out, h->scratch);
    P.epoch = h->epoch + 1;
    P.tag_base = P.epoch * (uint32_t)(P.spl * P.L + 1);
    P.lcount = h->launches + 1;
    const hipError_t e = launch_decode(v->fn, P, (v->W + 1) * 64, h->stream, h->cooperative);
    if (e != hipSuccess) return MK_ERR_HIP;
    ++h->epoch;
    ++h->launches;
    return MK_OK;
}

mk_status mk_decode_step_noalloc(mk_handle* h, const mk_batch* b, int32_t* tokens_out, float* logits_out) {
    const Variant* v = check_step(h, b, tokens_out);
    if (!v) return MK_ERR_INVALID_ARG;
    int dev = -1;
    if (!hip_ok(hipGetDevice(&dev))) return MK_ERR_HIP;
    if (dev != h->device) return MK_ERR_INVALID_ARG;
    if (h->sl.total > kStaticScratchBytes) return MK_ERR_UNSUPPORTED;
    StaticScratch ss{};
    if (!hip_ok(static_scratch_acquire(dev, h->stream, (uint32_t)(h->moe ? 6 : 5) * h->cfg.n_layers + 1, &ss)))
        return MK_ERR_HIP;
    Params P = step_params(h, *v, b, tokens_out, logits_out, ss.base);
    P.epoch = ss.epoch;
    P.tag_base = ss.tag_base;
    P.lcount = h->launches + 1;
    const hipError_t e = launch_decode(v->fn, P, (v->W + 1) * 64, h->stream, h->cooperative);
    if (e != hipSuccess) return MK_ERR_HIP;
    ++h->launches;
    return MK_OK;
}

mk_status mk_prefill(mk_handle* h, const mk_prefill_req* r, int32_t* token_out, float* logits_out) {
    if (!h || !r || !token_out || !r->tokens || !r->page_table || r->n_tokens < 1 || r->pos0 < 0 ||
        (int64_t)r->pos0 + r->n_tokens > h->max_pos || !(r->temperature >= 0.f) || !(r->temperature < 3.0e38f) ||
        r->request < 0 || r->request >= MK_MAX_BATCH)
        return MK_ERR_INVALID_ARG;
    if (h->moe) return MK_ERR_UNSUPPORTED;
    const mk_model_cfg& c = h->cfg;
    const int L = c.n_layers, d = c.d_model, Hq = c.n_q_heads, Hkv = c.n_kv_heads, dh = c.head_dim, F = c.ffn_dim,
              V = c.vocab;
    const int C = kPfChunk, HD = Hq * dh;
    if (!h->pf_x) {
        mk_status st;
        if ((st = dalloc(h, &h->pf_x, (size_t)C * d * 4)) != MK_OK || (st = dalloc(h, &h->pf_rs, (size_t)C * 4)) != MK_OK ||
            (st = dalloc(h, &h->pf_q, (size_t)C * HD * 4)) != MK_OK ||
            (st = dalloc(h, &h->pf_part, (size_t)kPfSplitMax * C * d * 4)) != MK_OK ||
            (st = dalloc(h, &h->pf_logits, (size_t)V * 4)) != MK_OK ||
            (st = dalloc(h, &h->pf_blk, (size_t)C * std::max(d, HD) * 4)) != MK_OK ||
            (st = dalloc(h, &h->pf_blk_act, (size_t)C * F * 4)) != MK_OK)
            return st;
    }
    hipStream_t s = h->stream;
    bool ok = true;
    auto chk = [&](hipError_t e) { ok = ok && e == hipSuccess; };
    int nc = 0;
    for (int c0 = 0; c0 < r->n_tokens && ok; c0 += C) {
        nc = std::min(C, r->n_tokens - c0);
        const int pos = r->pos0 + c0, groups = (nc + 15) / 16;
        // the residual stream, its attention-norm scale and operand blocks from the embeddings
        PfRows rw{};
        rw.embed = h->embed; rw.V = V; rw.part = h->pf_part; rw.y = h->pf_x; rw.rs = h->pf_rs; rw.blk = h->pf_blk;
        rw.n = nc; rw.n_groups = groups; rw.d = d; rw.eps = c.rms_eps; rw.err = h->err;
        rw.tokens = r->tokens + c0; rw.S = 0; rw.gains = h->attn_norm;
        chk(pf_launch_rows(rw, s));
        rw.tokens = nullptr;
        for (int l = 0; l < L && ok; ++l) {
            const uint8_t* lb = h->wpack + (int64_t)l * h->layer_bytes;
            uint16_t* kp = h->kpool + (int64_t)l * h->kv_layer_elems;
            uint16_t* vp = h->vpool + (int64_t)l * h->kv_layer_elems;
            const float* sl = h->fp8 ? h->wscale + (int64_t)l * h->scale_lb : nullptr;  // FP8 row scales
            auto scales = [&](const GemvStage& m) { return sl ? sl + m.soff : nullptr; };
            PfGemm g{};
            g.x = h->pf_blk;
            g.n = nc;
            g.n_groups = groups;
            g.err = h->err;
            // attention block: QKV with RoPE and the K/V writes, attention, O into partial sums
            g.w = lb + h->qkv.off; g.wscale = scales(h->qkv); g.T = h->qkv.T; g.nkb = h->qkv.nkb; g.rs = h->pf_rs;
            g.rope = h->rope; g.pos0 = pos; g.Hq = Hq; g.Hkv = Hkv; g.dh = dh; g.q = h->pf_q;
            g.kpool = kp; g.vpool = vp; g.pages = r->page_table; g.n_pages = c.n_pages;
            chk(pf_launch_gemm(PF_QKV, g, 1, s));
            PfAttn at{};
            at.q = h->pf_q; at.o_blk = h->pf_blk; at.kpool = kp; at.vpool = vp; at.pages = r->page_table;
            at.pos0 = pos; at.n = nc; at.Hq = Hq; at.Hkv = Hkv; at.win = h->window[l]; at.n_pages = c.n_pages; at.err = h->err;
            chk(pf_launch_attn(dh, at, s));
            g.w = lb + h->o.off; g.wscale = scales(h->o); g.T = h->o.T; g.nkb = h->o.nkb; g.out = h->pf_part; g.ldo = d; g.rs = nullptr;
            int S = pf_splits(PF_PART, g);
            chk(pf_launch_gemm(PF_PART, g, S, s));
            // h = x + O; the FFN norm's scale and operand blocks
            rw.S = S; rw.gains = h->ffn_norm + (int64_t)l * d;
            chk(pf_launch_rows(rw, s));
            // FFN block: gate/up with SwiGLU into the down projection's operand blocks, down into partial sums
            g.w = lb + h->gu.off; g.wscale = scales(h->gu); g.T = h->gu.T; g.nkb = h->gu.nkb; g.rs = h->pf_rs; g.act_blk = h->pf_blk_act; g.F = F;
            chk(pf_launch_gemm(PF_GU, g, 1, s));
            g.x = h->pf_blk_act;
            g.w = lb + h->dn.off; g.wscale = scales(h->dn); g.T = h->dn.T; g.nkb = h->dn.nkb; g.out = h->pf_part; g.ldo = d; g.rs = nullptr;
            S = pf_splits(PF_PART, g);
            chk(pf_launch_gemm(PF_PART, g, S, s));
            // x = h + down; the next layer's attention norm (or the final norm) and its operand blocks
            rw.S = S; rw.gains = l + 1 < L ? h->attn_norm + (int64_t)(l + 1) * d : h->final_norm;
            chk(pf_launch_rows(rw, s));
        }
    }
    // the last position: lm_head over its token group's final-norm operand block, then the sampler
    const int lg = (nc - 1) / 16;
    PfGemm g{};
    g.w = h->wpack + h->lm.off; g.wscale = h->fp8 ? h->wscale + h->lm.soff : nullptr; g.T = h->lm.T; g.nkb = h->lm.nkb;
    g.x = h->pf_blk + (int64_t)lg * (d / 32) * 2048; g.n = nc - 16 * lg; g.n_groups = 1; g.rs = h->pf_rs + 16 * lg;
    g.out = h->pf_logits; g.ldo = V;
    chk(pf_launch_gemm(PF_LM, g, 1, s));
    chk(pf_launch_sample(h->pf_logits, V, r->temperature, r->seed, r->step, r->request, token_out, logits_out, s));
    return ok ? MK_OK : MK_ERR_HIP;
}

mk_status mk_set_route_debug(mk_handle* h, int32_t* buf) {
    if (!h || !h->moe) return MK_ERR_INVALID_ARG;
    h->route_dbg = buf;
    return MK_OK;
}

mk_status mk_last_error(mk_handle* h, int32_t* where_out) {
    if (!h) return MK_ERR_INVALID_ARG;
    if (where_out) *where_out = -1;
    uint32_t e[4] = {0, 0, 0, 0};
    if (!hip_ok(hipStreamSynchronize(h->stream)) ||
        !hip_ok(hipMemcpy(e, h->err, sizeof(e), hipMemcpyDeviceToHost)) ||
        !hip_ok(hipMemset(h->err, 0, 64)))
        return MK_ERR_HIP;
    if (e[0] == 0) return MK_OK;
    if (where_out) *where_out = (int32_t)e[1];
    return (mk_status)e[0];
}

mk_status mk_set_trace(mk_handle* h, uint64_t* buf) {
    if (!h) return MK_ERR_INVALID_ARG;
    h->trace = buf;
    return MK_OK;
}

mk_status mk_set_wait_limit(mk_handle* h, uint32_t usec) {
    if (!h || usec == 0) return MK_ERR_INVALID_ARG;
    h->wait_usec = usec;
    return MK_OK;
}

mk_status mk_moe_experts_used(mk_handle* h, int64_t* total) {
    if (!h || !total) return MK_ERR_INVALID_ARG;
    unsigned long long v = 0;
    if (!hip_ok(hipStreamSynchronize(h->stream)) ||
        !hip_ok(hipMemcpy(&v, h->moe_used, 8, hipMemcpyDeviceToHost)) || !hip_ok(hipMemset(h->moe_used, 0, 8)))
        return MK_ERR_HIP;
    *total = (int64_t)v;
    return MK_OK;
}

mk_status mk_set_cooperative(mk_handle* h, int32_t on) {
    if (!h || (on != 0 && on != 1)) return MK_ERR_INVALID_ARG;
    h->cooperative = on != 0;
    return MK_OK;
}

mk_status mk_variant_info(const mk_handle* h, int32_t batch, int32_t* compute_waves, int32_t* ring_slots,
                          int32_t* lds_bytes, int32_t* path) {
    if (!h || batch < 1 || batch > h->cfg.max_batch) return MK_ERR_INVALID_ARG;
    const Variant& v = batch == 1 ? h->var[0] : batch == 2 ? h->var[1] : h->var[2];
    if (compute_waves) *compute_waves = v.W;
    if (ring_slots) *ring_slots = v.ring;
    if (lds_bytes) *lds_bytes = v.lds_total;
    if (path) *path = v.mfma ? 1 : 0;
    return MK_OK;
}

mk_status mk_launch_info(const mk_handle* h, int32_t* workgroups, int32_t* threads, int32_t* lds_bytes, int32_t* path) {
    if (!h) return MK_ERR_INVALID_ARG;
    if (workgroups) *workgroups = h->NW;
    if (threads) *threads = (h->var[0].W + 1) * 64;
    if (lds_bytes) *lds_bytes = h->var[0].lds_total;
    if (path) *path = 0;
    return MK_OK;
}

}  // extern "C"
