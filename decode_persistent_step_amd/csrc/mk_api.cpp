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

namespace mk {
const void* select_kernel(int nb, bool mfma, int dh, int G, int ring, bool moe, int waves);
hipError_t launch_decode(const void* fn, const Params& P, int threads, hipStream_t stream, bool cooperative);
hipError_t launch_pack(uint8_t* dst, int T, int nkb, int K, int mode, const uint16_t* s0, const uint16_t* s1,
                       const uint16_t* s2, int n0, int n1, int dh, hipStream_t stream);
hipError_t launch_kv_copy(uint16_t* pool_layer, const int32_t* slots, uint16_t* rows, int n, int Hkv, int dh, int isv,
                          int64_t n_slots, int dir, uint32_t* err, hipStream_t stream);
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
    int lds_units = 0, lds_gain = 0, lds_res = 0, lds_op = 0, lds_ring = 0, lds_total = 0, lds_route = 0;
    int lds_part[SK_KINDS] = {0, 0, 0, 0, 0, 0, 0};
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
    int span_max = 1;  // MoE: most experts one WG's down-projection tiles span
    int64_t layer_bytes = 0;
    int64_t atto_lb = 0, h_lb = 0, act_lb = 0, x_lb = 0, rlog_lb = 0;  // operand buffers: bytes per layer copy
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
    uint32_t epoch = 0;
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
GemvStage make_stage(int64_t off, int rows, int K, int NW, int W, bool may_split, int min_split = 1) {
    GemvStage g{};
    g.off = off;
    g.T = (rows + 15) / 16;
    g.nkb = K / 32;
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
    v.lds_res = align(v.lds_route + (h->moe ? kRouteBytes : 0));
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

mk_status mk_create(const mk_model_cfg* cfg, const mk_weights* w, void* stream, mk_handle** out) {
    g_create_error = "";
    if (!out) return why(MK_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!cfg || !w) return why(MK_ERR_INVALID_ARG, "cfg or weights is NULL");
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
    if (!w->embed || !w->final_norm || !w->lm_head || !w->attn_norm || !w->wq || !w->wk || !w->wv || !w->wo ||
        !w->ffn_norm || !w->w_gate || !w->w_up || !w->w_down || (moe && !w->router))
        return why(MK_ERR_INVALID_ARG, "a weight pointer is NULL");
    for (int l = 0; l < c.n_layers; ++l)
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
        free_all(h);
        delete h;
        return s;
    };
    if (!hip_ok(hipGetDevice(&h->device))) return fail(MK_ERR_HIP);
    int cus = 0, lds_limit = 0;
    if (!hip_ok(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, h->device)) ||
        !hip_ok(hipDeviceGetAttribute(&lds_limit, hipDeviceAttributeMaxSharedMemoryPerBlock, h->device)))
        return fail(MK_ERR_HIP);
    if (cus > 256) cus = 256;  // the attention merge handles at most 256 workgroup partials per segment
    h->NW = cus;
    h->NWpad = (cus + kFlagStride - 1) / kFlagStride * kFlagStride;
    const int L = c.n_layers, d = c.d_model, Hq = c.n_q_heads, Hkv = c.n_kv_heads, F = c.ffn_dim, V = c.vocab;
    const int NW = h->NW;

    // partitions and packed layout: per layer QKV, O, then the dense gate/up and
    // down, or the MoE router and every expert's gate/up and down
    int64_t off = 0;
    h->moe = moe;
    // the packed layout and the handle's checks use four compute waves (the
    // fewest a variant has); variants with eight re-partition below
    const int W = 4;
    h->qkv = make_stage(off, (Hq + 2 * Hkv) * dh, d, NW, W, false);
    off += stage_bytes(h->qkv);
    h->o = make_stage(off, d, Hq * dh, NW, W, true);
    off += stage_bytes(h->o);
    if (moe) {
        const int E = c.n_experts, fe = c.expert_ffn_dim;
        const int nu_max = std::min(E, c.max_batch * c.top_k);
        h->rt = make_stage(off, E, d, NW, W, false);
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
        h->gu = make_stage(off, 2 * F, d, NW, W, false);
        off += stage_bytes(h->gu);
        h->dn = make_stage(off, d, F, NW, W, true);
        off += stage_bytes(h->dn);
    }
    h->layer_bytes = off;
    h->lm = make_stage((int64_t)L * off, V, d, NW, W, false);
    for (const GemvStage* g : {&h->qkv, &h->o, &h->gu, &h->dn, &h->lm})
        if (g->ncw < 1 || g->nkb % (W * g->S) != 0)
            return fail(why(MK_ERR_UNSUPPORTED, "a GEMV width is not a multiple of 32 x the compute waves"));
    if (moe && (h->rt.ncw < 1 || h->rt.nkb % W != 0))
        return fail(why(MK_ERR_UNSUPPORTED, "a GEMV width is not a multiple of 32 x the compute waves"));

    // The segment merge gives each (partial, 4-value quad) pair and each (head,
    // partial) header one item of the I/O wave, at most 64 * att_merge_pu each.
    // A segment has at most NW / Hkv + 2 workgroup partials (the Hkv segments of a
    // request share its pages equally); slice me of ns holds quads
    // [me QD / ns, (me + 1) QD / ns), QD = G dh / 4.
    {
        const int QD = G * dh / 4, cap = 64 * att_merge_pu(G, dh);
        const int ns_max = std::min(NW, NW / Hkv + 2);
        for (int ns = 1; ns <= ns_max; ++ns)
            for (int me = 0; me < ns; ++me) {
                const int q0 = me * QD / ns, q1 = (me + 1) * QD / ns;
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
            v.fn = select_kernel(v.nb, v.mfma, dh, G, v.ring, moe, v.W);
            if (!v.fn) return fail(why(MK_ERR_UNSUPPORTED, "no kernel instantiated for this head_dim / group size"));
            for (int ms = 1; ms <= kMaxSplit && !fits; ms *= 2) {
                v.qkv = make_stage(h->qkv.off, (Hq + 2 * Hkv) * dh, d, NW, v.W, false);
                v.gu = moe ? h->gu : make_stage(h->gu.off, 2 * F, d, NW, v.W, false);
                v.lm = make_stage(h->lm.off, V, d, NW, v.W, false);
                v.rt = moe ? make_stage(h->rt.off, c.n_experts, d, NW, v.W, false) : h->rt;
                v.o = make_stage(h->o.off, d, Hq * dh, NW, v.W, true, ms);
                v.dn = moe ? h->dn : make_stage(h->dn.off, d, F, NW, v.W, true, ms);
                bool widths = true;
                for (const GemvStage* g : {&v.qkv, &v.o, &v.gu, &v.dn, &v.lm, &v.rt}) {
                    if ((g == &v.gu || g == &v.dn) && moe) continue;  // expert stages: whole tiles per wave
                    if (g == &v.rt && !moe) continue;
                    widths = widths && g->ncw >= 1 && g->nkb % (v.W * g->S) == 0;
                }
                if (!widths) {
                    if (v.W == 4) return fail(why(MK_ERR_UNSUPPORTED, "a GEMV width is not a multiple of 128"));
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
        if (!hip_ok(hipFuncSetAttribute(v.fn, hipFuncAttributeMaxDynamicSharedMemorySize, v.lds_total)))
            return fail(MK_ERR_HIP);
        int occ = 0;
        if (!hip_ok(hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, v.fn, (v.W + 1) * 64, v.lds_total)) || occ < 1)
            return fail(why(MK_ERR_UNSUPPORTED, "the kernel cannot be resident (registers or LDS)"));
    }

    // device memory
    const int64_t wbytes = (int64_t)L * h->layer_bytes + stage_bytes(h->lm);
    h->kv_layer_elems = (int64_t)c.n_pages * Hkv * kPage * dh;
    if (c.n_pages > 0 && (int64_t)c.n_pages * Hkv * kPage * dh * 2 >= (1ll << 31))
        return fail(why(MK_ERR_UNSUPPORTED, "one layer's K or V pool would exceed 2 GiB"));
    const int GR = att_hdr_words(G) + G * dh;
    if ((st = dalloc(h, &h->wpack, wbytes)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->embed, (size_t)V * d * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->attn_norm, (size_t)L * d * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->ffn_norm, (size_t)L * d * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->final_norm, (size_t)d * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->rope, (size_t)h->max_pos * (dh / 2) * 2 * 4)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->kpool, (size_t)L * h->kv_layer_elems * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->vpool, (size_t)L * h->kv_layer_elems * 2)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->window_dev, (size_t)L * 4)) != MK_OK) return fail(st);
    // exchange buffers: q, k~/v~ and attention partials are tagged 64-bit words,
    // zeroed (no valid tag) at creation; GEMV operands are plain fp32
    const size_t xq = (size_t)kMaxBatch * Hq * dh, xkv = (size_t)kMaxBatch * Hkv * 2 * dh,
                 xattp = (size_t)kMaxBatch * Hkv * NW * GR, xparts = (size_t)kMaxSplit * kMaxBatch * d,
                 xact = moe ? (size_t)kMaxUnion * kMaxBatch * c.expert_ffn_dim : (size_t)kMaxBatch * F,
                 xrlog = (size_t)kMaxBatch * std::max(1, (int)c.n_experts);
    if ((st = dalloc(h, &h->q, xq * 8)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->kvcur, xkv * 8)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->attp, xattp * 8)) != MK_OK) return fail(st);
    // GEMV operand buffers: fp32, or tagged 64-bit words in the dense vector-ALU variants
    // (one copy per layer; x one per layer input 1..L, index 0 unused)
    if ((st = dalloc(h, &h->atto, xq * 8 * L)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->hparts, xparts * 8 * L)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->act, xact * 8 * L)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->xparts, xparts * 8 * (L + 1))) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->rlog, xrlog * 4 * L)) != MK_OK) return fail(st);
    h->atto_lb = (int64_t)xq * 8;
    h->h_lb = (int64_t)xparts * 8;
    h->act_lb = (int64_t)xact * 8;
    h->x_lb = (int64_t)xparts * 8;
    h->rlog_lb = (int64_t)xrlog * 4;
    if ((st = dalloc(h, &h->moe_used, 8)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->lmpart, (size_t)NW * kMaxBatch * 2 * 4)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->lmtopk, (size_t)NW * kMaxBatch * kMaxSampleTopK * 2 * 4)) != MK_OK) return fail(st);
    const size_t nflags = (size_t)(L * FK_PER_LAYER + 2) * h->NWpad + 256;
    if ((st = dalloc(h, &h->flags, nflags * 4)) != MK_OK) return fail(st);
    if ((st = dalloc(h, &h->err, 64)) != MK_OK) return fail(st);
    hipStream_t s = h->stream;
    if (!hip_ok(hipMemsetAsync(h->flags, 0, nflags * 4, s)) || !hip_ok(hipMemsetAsync(h->err, 0, 64, s)) ||
        !hip_ok(hipMemsetAsync(h->kpool, 0, (size_t)L * h->kv_layer_elems * 2, s)) ||
        !hip_ok(hipMemsetAsync(h->vpool, 0, (size_t)L * h->kv_layer_elems * 2, s)) ||
        !hip_ok(hipMemsetAsync(h->q, 0, xq * 8, s)) || !hip_ok(hipMemsetAsync(h->kvcur, 0, xkv * 8, s)) ||
        !hip_ok(hipMemsetAsync(h->attp, 0, xattp * 8, s)) || !hip_ok(hipMemsetAsync(h->atto, 0, xq * 8 * L, s)) ||
        !hip_ok(hipMemsetAsync(h->hparts, 0, xparts * 8 * L, s)) || !hip_ok(hipMemsetAsync(h->act, 0, xact * 8 * L, s)) ||
        !hip_ok(hipMemsetAsync(h->xparts, 0, xparts * 8 * (L + 1), s)) ||
        !hip_ok(hipMemsetAsync(h->rlog, 0, xrlog * 4 * L, s)) ||
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
    for (int l = 0; l < L; ++l) {
        uint8_t* lb = h->wpack + (int64_t)l * h->layer_bytes;
        auto U = [](const void* p) { return static_cast<const uint16_t*>(p); };
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
    if (!hip_ok(hipStreamSynchronize(s))) return fail(MK_ERR_HIP);

    // page allocator: 0..n_pages-1 free, lowest first
    h->refs.assign(c.n_pages, 0);
    for (int i = 0; i < c.n_pages; ++i) h->free_pages.insert(h->free_pages.end(), i);
    *out = h;
    return MK_OK;
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

mk_status mk_decode_step(mk_handle* h, const mk_batch* b, int32_t* tokens_out, float* logits_out) {
    if (!h || !b || !tokens_out || !b->seq_lens || !b->page_table || !b->tokens_in) return MK_ERR_INVALID_ARG;
    if (b->n < 1 || b->n > h->cfg.max_batch) return MK_ERR_INVALID_ARG;
    const Variant& v = b->n == 1 ? h->var[0] : b->n == 2 ? h->var[1] : h->var[2];
    if (!v.fn) return MK_ERR_INVALID_ARG;
    if (b->top_k && v.lm.max_tasks * 16 > 64 * kTopKLane) return MK_ERR_INVALID_ARG;  // vocabulary too wide per WG
    static_assert(kMaxSampleTopK == MK_MAX_TOP_K, "top-k bound");
    const mk_model_cfg& c = h->cfg;
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
    P.rlog = h->rlog;
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
    P.q = h->q;
    P.kvcur = h->kvcur;
    P.attp = h->attp;
    P.atto = h->atto;
    P.hparts = h->hparts;
    P.act = h->act;
    P.xparts = h->xparts;
    P.xn = h->moe ? 1 : v.dn.S;
    P.atto_lb = h->atto_lb;
    P.h_lb = h->h_lb;
    P.act_lb = h->act_lb;
    P.x_lb = h->x_lb;
    P.rlog_lb = h->rlog_lb;
    P.lmpart = h->lmpart;
    P.lmtopk = h->lmtopk;
    P.flags = h->flags;
    P.err = h->err;
    P.epoch = ++h->epoch;
    P.wait_ticks = (uint64_t)h->wait_usec * 100u;  // 100 MHz constant clock
    P.NW = h->NW;
    P.NWpad = h->NWpad;
    P.lds_units = v.lds_units;
    P.lds_op = v.lds_op;
    for (int k = 0; k < SK_KINDS; ++k) P.lds_part[k] = v.lds_part[k];
    P.lds_route = v.lds_route;
    P.lds_total = v.lds_total;
    P.lds_ring = v.lds_ring;
    P.lds_gain = v.lds_gain;
    P.lds_res = v.lds_res;
    P.maxu = h->maxu;
    P.trace = h->trace;
    const hipError_t e = launch_decode(v.fn, P, (v.W + 1) * 64, h->stream, h->cooperative);
    if (e != hipSuccess) {
        --h->epoch;
        return MK_ERR_HIP;
    }
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
