// mk_kernel.hip - the persistent decode-step kernel for gfx950 (MI355X), plus the
// weight-packing and K/V copy kernels.
//
// Method (Cohere Megakernel page, "Megakernel ne demek"): the whole decode pass
// runs in ONE kernel launch whose work is split into GEMM pieces and attention
// partitions, with no full-grid barrier between ops. Here every workgroup (one
// per CU) owns a fixed slice of every stage; a stage's consumers wait on
// per-workgroup flags raised by its producers (epoch-valued, never reset).
// Following the Kog AI page ("GEMM Dışı İşler": prefetch overlapped across op
// sections; "Ağırlık Yeniden Yüklemeleri": a weight layout for small batches),
// four or eight compute waves per workgroup stream packed weights and K/V pages
// through an LDS ring filled by DMA that runs ahead ACROSS stage boundaries, so the
// loads of the next ops are in flight while the workgroup waits for an op's
// activations. One more wave does all cross-workgroup I/O (flags, activations,
// epilogues, outputs), so the compute waves issue nothing but the stream.
#include "mk_device.h"
#include "mk_params.h"

namespace mk {

#define MK_AI __attribute__((always_inline))

// --------------------------------------------------------------- LDS control
struct Ctrl {
    int32_t abort;
    int32_t n;
    int32_t valid;   // bit b: request b has in-range scalars
    int32_t bad;     // bit b: request b touched an out-of-range page (after validation)
    int32_t seq[kMaxBatch];
    int32_t tok[kMaxBatch];
    float temp[kMaxBatch];
    float rsc[kMaxBatch];  // RMSNorm scale of the current stage's input
    int32_t wseg[2][kMaxComputeWaves];  // segment of each compute wave in table t (-1: none)
    int32_t wu0[2][kMaxComputeWaves];   // first unit of the wave inside its segment
    int32_t wnu[2][kMaxComputeWaves];   // number of units of the wave
    int32_t nseg[2];
    int32_t segu[2][kMaxBatch * 8 + 1];  // unit prefix sums per segment (segment = b * Hkv + g)
    int32_t segw[2][kMaxBatch * 8 + 1];  // first compute wave of each segment (prefix sums of its wave counts)
    uint32_t sliding[2];             // bit l: layer l uses the sliding window (l < 64)
    uint64_t tdata[6];               // trace: compute wave 0 timestamps inside a stage
    int32_t part[SK_KINDS][3];       // this WG's GEMV partition per stage kind: split, first tile, end tile
    int32_t route_layer;             // MoE: layer whose routing the LDS routing block holds (-1: none)
    int32_t opsync;                  // compute-wave arrivals at operand hand-overs (LDS counter)
    int32_t pubs;                    // stages whose outputs the I/O wave has published (flag raised)
    int32_t topk[kMaxBatch];         // limited top-k per request (0: none)
    int32_t apid[kMaxBatch];         // page receiving each request's new K/V row
    float ssw[kMaxComputeWaves][kMaxBatch];  // per-wave sums of squares of the operand rows
};
static_assert(sizeof(Ctrl) <= kCtrlBytes, "ctrl block");

__device__ __forceinline__ Ctrl& ctrl(uint8_t* lds) { return *reinterpret_cast<Ctrl*>(lds); }

// MoE routing block in LDS, written by the I/O wave once a layer's router
// logits are final and read by both roles until the next layer's routing.
struct Route {
    int32_t eu[kMaxUnion];             // the step's selected experts, ascending (nU of them)
    int32_t sel[kMaxBatch][kMaxTopK];  // per request: its experts, best first
    float selw[kMaxBatch][kMaxTopK];   // per request: their softmax weights
    float wu[kMaxSpan][kMaxBatch];     // down-projection: weight of request b for this WG's expert slot i (0: not selected)
    uint32_t umask[4];                 // union of the selections (bit e of word e / 32), built by LDS atomics
    int32_t nU;                        // experts selected by any request
    int32_t uf;                        // index in eu of the expert of this WG's first down-projection tile
};
static_assert(sizeof(Route) <= kRouteBytes, "routing block");

// An opaque copy of a pointer: values loaded through it are not hoisted out of
// the enclosing loop, which keeps per-stage parameters from pinning registers
// for the whole kernel.
// Kernel parameters are read in place from the kernarg segment (constant
// address space, scalar loads); taking the address of the by-value argument
// would force a private copy.
typedef const Params __attribute__((address_space(4)))* KParams;
__device__ __forceinline__ KParams kparams() {
    return (KParams)__builtin_amdgcn_kernarg_segment_ptr();
}
__device__ __forceinline__ KParams launder(KParams p) {
    asm volatile("" : "+s"(p));
    return p;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// A value every lane holds alike (LDS control fields), as a scalar.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint32_t uni(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ uint32_t* flag_array(const Params& P, int layer, int kind) {
    return P.flags + (size_t)(layer * FK_PER_LAYER + kind) * P.NWpad;
}
__device__ __forceinline__ uint32_t* flag_val(const Params& P) { return P.flags + (size_t)(P.L * FK_PER_LAYER) * P.NWpad; }
__device__ __forceinline__ uint32_t* flag_lm(const Params& P) { return P.flags + (size_t)(P.L * FK_PER_LAYER + 1) * P.NWpad; }

// Quotient of non-negative ints whose products stay below 2^31 (unsigned
// 32-bit division: far less code than the signed or 64-bit forms).
__device__ __forceinline__ int udiv(int a, int b) { return (int)((uint32_t)a / (uint32_t)b); }

// GEMV partition: WG w -> K split s and tiles [t0, t1)
struct GemvPart { int s, t0, t1; };
__device__ __forceinline__ GemvPart gemv_part(const GemvStage& g, int w, int NW) {
    GemvPart p;
    p.s = udiv(w * g.S, NW);
    const int f0 = udiv(p.s * NW + g.S - 1, g.S);        // first WG of split s
    const int f1 = udiv((p.s + 1) * NW + g.S - 1, g.S);  // first WG of split s+1
    const int nw = f1 - f0, wi = w - f0;
    p.t0 = udiv(wi * g.T, nw);
    p.t1 = udiv((wi + 1) * g.T, nw);
    return p;
}

// This WG's partition of GEMV stage `kind` (0 qkv, 2 o, 3 gu, 4 dn, 5 lm), as
// computed once by the prologue.
__device__ __forceinline__ GemvPart wg_part(uint8_t* lds, int kind) {
    const Ctrl& C = ctrl(lds);
    GemvPart p;
    p.s = uni(C.part[kind][0]);
    p.t0 = uni(C.part[kind][1]);
    p.t1 = uni(C.part[kind][2]);
    return p;
}

// Bad-request mask of this launch (offset 0) or of the next one (offset 1):
// a handle's launches alternate between err[2] and err[3] by the parity of
// its launch count, and each launch clears the next one's word in its
// prologue, so a launch that ends early leaves nothing behind.
__device__ __forceinline__ uint32_t* bad_mask(const Params& P, int next) {
    return P.err + 2 + ((P.lcount + (uint32_t)next) & 1u);
}

// ------------------------------------------------------------ error latching
__device__ void latch_error(const Params& P, uint32_t code, uint32_t where) {
    // first error wins
    if (atomicCAS(P.err, 0u, code) == 0u) __hip_atomic_store(P.err + 1, where, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (I/O wave) until flags[first .. first+count) all reached the epoch.
__device__ bool wait_flags(const Params& P, const uint32_t* f, int first, int count, uint32_t where) {
    if (count <= 0) return true;
    const int lane = lane_id();
    const uint64_t deadline = rt_clock() + P.wait_ticks;
    const int a0 = first & ~3;
    for (int base = a0; base < first + count; base += 256) {
        const int i0 = base + lane * 4;
        while (true) {
            v4u v = ld_sc1_v4(f, (uint32_t)i0 * 4u);
            bool ok = true;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                int idx = i0 + e;
                if (idx >= first && idx < first + count) ok = ok && ((int32_t)(v[e] - P.epoch) >= 0);
            }
            if (__all(ok)) break;
            if (rt_clock() > deadline) {
                if (lane == 0) latch_error(P, 6u, where);
                return false;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    return true;
}

// Coherent (sc1) loads the compiler may schedule freely; `base` must be
// wave-uniform, idx is a per-lane element index (< 2^29).
__device__ __forceinline__ float ldc_f(const float* base, int64_t idx) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(base), (uint32_t)idx * 4u, 0, kCachePolicySC1));
}
__device__ __forceinline__ int32_t ldc_i(const int32_t* base, int64_t idx) {
    return __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(rsrc(base), (uint32_t)idx * 4u, 0, kCachePolicySC1));
}
__device__ __forceinline__ v4f ldc_v4f(const float* base, int64_t idx) {
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), (uint32_t)idx * 4u, 0, kCachePolicySC1));
}
// Loads through L1 and L2, for operand data that is written once per launch
// (write-through stores) and read only after its producers' flags: no cache
// can hold an older copy of the line (each layer has its own copy of the
// buffer, and the launch boundary invalidates the L2), and the workgroups of
// an XCD share the line in their L2 instead of each fetching it from memory.
__device__ __forceinline__ float ldk_f(const float* base, int64_t idx) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc(base), (uint32_t)idx * 4u, 0, 0));
}
__device__ __forceinline__ v4f ldk_v4f(const float* base, int64_t idx) {
    return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), (uint32_t)idx * 4u, 0, 0));
}
// Layer `layer`'s copy of an operand buffer (copies lb bytes apart).
template <class T>
__device__ __forceinline__ T* layer_copy(T* base, int64_t lb, int layer) {
    return reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(base) + (uint64_t)((int64_t)layer * lb));
}

// Optional timeline: slot k of stage sid of this WG (lane 0 only).
__device__ __forceinline__ void trace_mark(const Params& P, int sid, int k) {
    if (P.trace && lane_id() == 0) P.trace[((size_t)blockIdx.x * (P.spl * P.L + 1) + sid) * 8 + k] = rt_clock();
}

// Raise this WG's flag (I/O wave): all its prior stores must be complete.
__device__ __forceinline__ void raise_flag(const Params& P, uint32_t* f) {
    wait_vm_all();
    if (lane_id() == 0) st_sc1_u(f + blockIdx.x, P.epoch);
}
// Raise this WG's flag without waiting for its data stores: the data are
// tagged words, so the flag only tells readers when to start looking.
__device__ __forceinline__ void raise_flag_now(const Params& P, uint32_t* f) {
    if (lane_id() == 0) st_sc1_u(f + blockIdx.x, P.epoch);
}

// Tag of the words written by stage sid of this launch: the launch's base plus
// the stage, unique across the launches that share the exchange buffers until
// the 32-bit counter wraps (each launch advances the base by its stage count).
__device__ __forceinline__ uint32_t stage_tag(const Params& P, int sid) {
    return P.tag_base + (uint32_t)sid;
}

// Store four consecutive tagged fp32 words at word index idx (idx even).
__device__ __forceinline__ void st_tag4(uint64_t* base, uint32_t idx, v4f v, uint32_t tag) {
    st_sc1_v4(base, idx * 8u, (v4u){__float_as_uint(v[0]), tag, __float_as_uint(v[1]), tag});
    st_sc1_v4(base, (idx + 2u) * 8u, (v4u){__float_as_uint(v[2]), tag, __float_as_uint(v[3]), tag});
}

// Bounded retry of a tagged read: returns false (and latches a timeout) once
// the deadline passes.
__device__ __forceinline__ bool retry_or_fail(const Params& P, uint64_t deadline, uint32_t where) {
    if (rt_clock() > deadline) {
        if (lane_id() == 0) latch_error(P, 6u, where);
        return false;
    }
    __builtin_amdgcn_s_sleep(1);
    return true;
}

// ================================================================ streaming
// Every compute wave consumes ONE flat sequence of 1 KB chunks: per layer its
// share of the QKV tiles, of the attention pages (the K chunks, then the V
// chunks of each page), of O, gate/up and down; after the last layer its share
// of lm_head. Chunks move global -> LDS by DMA (buffer loads with the LDS bit,
// 16 B per lane: lane l later reads back exactly the 16 B it fetched) into a
// ring of R slots per wave. The issue cursor runs up to R - 1 chunks ahead of
// consumption and crosses stage boundaries, so while the workgroup waits for a
// stage's activations the weights of that stage and of the next ones keep
// arriving. A wave's loads complete in order and compute waves issue no other
// vector-memory instruction, so "chunk c has landed" is "no more loads
// outstanding than were issued after c" (vmcnt).
template <int V_>
struct IC { static constexpr int value = V_; };
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(IC<I>{});
        static_for<I + 1, N>(f);
    }
}

constexpr uint32_t KB = kChunk;

// Stages per layer: 5 dense, 6 MoE (a compile-time choice of the kernel).
template <bool MOE>
constexpr int kSPL = MOE ? 6 : 5;
template <bool MOE>
__device__ __forceinline__ int stage_layer(const Params& P, int sid) { return (int)((uint32_t)sid / (uint32_t)kSPL<MOE>); }
template <bool MOE>
__device__ __forceinline__ int stage_kind(const Params& P, int sid) {
    if (sid == kSPL<MOE> * P.L) return SK_LM;
    const int pos = sid - stage_layer<MOE>(P, sid) * kSPL<MOE>;
    if constexpr (!MOE) return pos;
    else return pos < 3 ? pos : pos == 3 ? SK_RT : pos - 1;  // MoE: QKV ATT O RT GU DN
}
__device__ __forceinline__ const GemvStage& stage_of(const Params& P, int kind) {
    return kind == 0 ? P.qkv : kind == 2 ? P.o : kind == 3 ? P.gu : kind == 4 ? P.dn : kind == 6 ? P.rt : P.lm;
}
// MoE expert stages: GU and DN of an MoE model
template <bool MOE>
__device__ __forceinline__ bool expert_stage(int kind) { return MOE && (kind == 3 || kind == 4); }
// Dense vector-ALU variants publish the GEMV operands (attention output, h
// parts, activations, x parts) as tagged words that the consuming compute waves
// poll directly: no flag, no store acknowledgement, one round trip per hop.
// The MFMA (batch 3..8) and MoE variants move 2-8x more operand bytes and keep
// plain fp32 behind flags.
template <bool MFMA, bool MOE>
constexpr bool kTagOps = !MFMA && !MOE;
__device__ __forceinline__ const uint8_t* layer_w(const Params& P, int layer) { return P.wpack + (int64_t)layer * P.layer_bytes; }
// Attention table of a layer: 0 full, 1 sliding window (from the LDS control
// block, so compute waves never read global memory outside the stream).
__device__ __forceinline__ int att_table(uint8_t* lds, int layer) {
    return (int)((uni(ctrl(lds).sliding[layer >> 5]) >> (layer & 31)) & 1u);
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) const int32_t lds_i32c;
typedef __attribute__((address_space(3))) const volatile v4u lds_v4u_cv;

template <int R>
struct Stream {
    lds_u8* ring;            // this wave's R KB of LDS
    int issued, consumed;    // chunks issued / consumed so far
    int att_ok;              // the attention tables in LDS are final
    // issue cursor
    int isid;                // stage being issued
    int ic, in;              // chunks of that stage issued / to issue
    int ikind;               // 0 GEMV, 1 attention
    int ncw, kb, page;       // GEMV: chunks per task, position in the task; attention: chunk in page, page
    __amdgpu_buffer_rsrc_t rs0, rs1;  // weights, or the layer's K and V pools at the wave's kv head
    uint32_t cur;            // GEMV: byte offset of the next chunk; attention: offset of the current page
    uint32_t tskip;          // GEMV: bytes from the end of a task's run to the start of the next
    uint32_t pstride;        // attention: bytes per page
    lds_i32c* pids;          // attention: the wave's page ids
    GemvPart qp;             // this WG's QKV partition, for the stream's start
    // MoE expert stages: the cursor's expert (index into the routing block's
    // list) and tile inside it; te = 0 elsewhere
    int te, eu_i, eu_t;
    uint32_t ebytes;
    lds_i32c* eul;
};

// Point the issue cursor at stage sid (the wave's share of it).
template <int R, int DH, bool MOE, int W>
__device__ __forceinline__ void stream_enter(Stream<R>& S, const Params& P, uint8_t* lds, int sid, int v) {
    constexpr int CPP = DH * kPage * 2 / kChunk;
    const int kind = stage_kind<MOE>(P, sid), layer = stage_layer<MOE>(P, sid);
    S.isid = sid;
    S.ic = 0;
    S.kb = 0;
    S.page = 0;
    if (kind == 1) {
        Ctrl& C = ctrl(lds);
        const int tab = att_table(lds, layer);
        const int seg = uni(C.wseg[tab][v]);
        const int npg = seg < 0 ? 0 : uni(C.wnu[tab][v]);
        const int g = seg < 0 ? 0 : seg % P.Hkv;
        S.ikind = 1;
        S.in = npg * 2 * CPP;
        S.pids = (lds_i32c*)(lds + P.lds_units) + (tab * W + v) * P.maxu;
        S.pstride = (uint32_t)(P.Hkv * kPage * DH * 2);
        const uint32_t head_off = (uint32_t)g * kPage * DH * 2;
        const uint32_t layer_bytes = (uint32_t)(P.kv_layer_elems * 2);
        S.rs0 = rsrc_n(reinterpret_cast<const uint8_t*>(P.kpool + (int64_t)layer * P.kv_layer_elems) + head_off, layer_bytes - head_off);
        S.rs1 = rsrc_n(reinterpret_cast<const uint8_t*>(P.vpool + (int64_t)layer * P.kv_layer_elems) + head_off, layer_bytes - head_off);
    } else {
        const GemvStage& st = stage_of(P, kind);
        const uint8_t* mat = (kind == 5 ? P.wpack : layer_w(P, layer)) + st.off;
        const GemvPart gp = S.att_ok ? wg_part(lds, kind) : S.qp;  // before the prologue: layer 0 QKV
        S.ikind = 0;
        S.te = 0;
        S.ncw = st.ncw;
        if (st.tpw) {
            // whole tiles per wave: wave v takes its W-th of the WG's tiles
            const int nt = gp.t1 - gp.t0;
            const int a = gp.t0 + udiv(v * nt, W), b = gp.t0 + udiv((v + 1) * nt, W);
            S.in = uni((b - a) * st.nkb);
            S.tskip = 0;
            if (expert_stage<MOE>(kind)) {
                S.eul = (lds_i32c*)(lds + P.lds_route);  // Route::eu
                S.te = st.te;
                S.ebytes = st.ebytes;
                S.eu_i = udiv(a, st.te);
                S.eu_t = a - S.eu_i * st.te;
                S.rs0 = rsrc_n(mat, (uint32_t)P.E * st.ebytes);
                S.cur = b > a ? uni((uint32_t)S.eul[S.eu_i] * st.ebytes + (uint32_t)S.eu_t * st.nkb * KB) : 0u;
            } else {
                S.rs0 = rsrc_n(mat, (uint32_t)((int64_t)st.T * st.nkb * KB));
                S.cur = uni((uint32_t)a * st.nkb * KB);
            }
        } else {
            S.in = uni((gp.t1 - gp.t0) * st.ncw);
            S.rs0 = rsrc_n(mat, (uint32_t)((int64_t)st.T * st.nkb * KB));
            S.cur = uni((uint32_t)(((int64_t)gp.t0 * st.nkb + (int64_t)gp.s * (st.nkb / st.S) + (int64_t)v * st.ncw) * KB));
            S.tskip = (uint32_t)(st.nkb - st.ncw) * KB;
        }
    }
}

// Issue the cursor's next k chunks (all inside the current stage) into ring
// slots issued mod R.
template <int R, int DH, bool MOE>
__device__ __forceinline__ void stream_issue(Stream<R>& S, int k, uint32_t lane16) {
    constexpr int CPP = DH * kPage * 2 / kChunk;
    if (S.ikind == 0) {
        for (; k > 0; --k) {
            dma_chunk(S.rs0, S.ring + (S.issued & (R - 1)) * KB, S.cur + lane16);
            ++S.issued;
            ++S.ic;
            S.cur += KB;
            if (++S.kb == S.ncw) {
                S.kb = 0;
                S.cur += S.tskip;
                if (MOE && S.te && ++S.eu_t == S.te) {  // next selected expert
                    S.eu_t = 0;
                    ++S.eu_i;
                    if (S.ic < S.in) S.cur = (uint32_t)uni(S.eul[S.eu_i]) * S.ebytes;
                }
            }
        }
    } else {
        for (; k > 0; --k) {
            if (S.kb == 0) S.cur = (uint32_t)uni(S.pids[S.page]) * S.pstride;
            const uint32_t off = S.cur + (uint32_t)(S.kb % CPP) * KB;
            dma_chunk(S.kb < CPP ? S.rs0 : S.rs1, S.ring + (S.issued & (R - 1)) * KB, off + lane16);
            ++S.issued;
            ++S.ic;
            if (++S.kb == 2 * CPP) {
                S.kb = 0;
                ++S.page;
            }
        }
    }
}

// Keep the ring full: R chunks in flight from the next one consumed on (fewer
// at the end of the kernel, or before the attention tables are final). The
// slot refilled last belongs to the chunk consumed last, whose LDS read has
// completed (its value was used).
template <int R, int DH, bool MOE, int W>
__device__ __forceinline__ void stream_refill(Stream<R>& S, KParams PK, uint8_t* lds, int v) {
    const uint32_t lane16 = (uint32_t)lane_id() * 16u;
    int room = S.consumed + R - S.issued;
    while (room > 0) {
        const int k = min(room, S.in - S.ic);
        if (k > 0) {
            stream_issue<R, DH, MOE>(S, k, lane16);
            room -= k;
        } else {
            const Params& P = *(const Params*)launder(PK);
            const int nsid = S.isid + 1;
            if (nsid > kSPL<MOE> * P.L) break;
            if (stage_kind<MOE>(P, nsid) == 1 && !S.att_ok) break;
            // MoE: the expert tiles of a layer are known once its routing is in LDS
            if (MOE && stage_kind<MOE>(P, nsid) == SK_GU && uni(ctrl(lds).route_layer) != stage_layer<MOE>(P, nsid)) break;
            stream_enter<R, DH, MOE, W>(S, P, lds, nsid, v);
        }
    }
}

// Wait until the next U chunks of the sequence have landed (conservatively, at
// one of a few vmcnt levels), then read them (this lane's 16 bytes of each).
template <int R, int U>
__device__ __forceinline__ void stream_wait(const Stream<R>& S) {
    const int m = S.issued - S.consumed - U;  // loads issued after the last of the U chunks
    if (m >= R - U) wait_vm<R - U>();
    else if (m >= R / 2 - U && R / 2 > U) wait_vm<(R / 2 > U ? R / 2 - U : 0)>();
    else if (m >= R / 4 - U && R / 4 > U) wait_vm<(R / 4 > U ? R / 4 - U : 0)>();
    else wait_vm<0>();
}
template <int R>
__device__ __forceinline__ v4u stream_read(const Stream<R>& S, int i) {
    return *(lds_v4u_cv*)(S.ring + ((S.consumed + i) & (R - 1)) * KB + lane_id() * 16);
}

// ============================================================ GEMV compute
// Operand in LDS, kb-major. It arrives as fp32 [kb][NBo][32]; the waves turn it
// in place into the hi/lo bf16 split x = hi + lo (about 16 significant bits,
// the same for both paths):
//   VALU: per (kb, b) a 128-byte block: hi[32] bf16 then lo[32] bf16;
//   MFMA: per kb the 16x16x32 B operand (1 KB, [lane][8]): column = lane % 16
//         (0..7 hi part of batch column b, 8..15 lo part), k = 8 (lane / 16) + e.


// Store 8 consecutive operand values x[k], k = 32 kb + 8 kg + e, of batch row b
// (already times the gains) in the final layout: their hi/lo bf16 split.
// (Hardware round-to-nearest-even conversions, no branches: this runs for every
// operand element of every stage.)
template <int NB, bool MFMA>
__device__ __forceinline__ void store_operand8(uint8_t* op, int kb, int b, int kg, const float (&x)[8]) {
    uint32_t h2[4], l2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h2[e] = cvt_bf16x2(x[2 * e], x[2 * e + 1]);
        const float lo0 = x[2 * e] - __uint_as_float(h2[e] << 16);
        const float lo1 = x[2 * e + 1] - __uint_as_float(h2[e] & 0xffff0000u);
        l2[e] = cvt_bf16x2(lo0, lo1);
    }
    const v4u ph = {h2[0], h2[1], h2[2], h2[3]};
    const v4u pl = {l2[0], l2[1], l2[2], l2[3]};
    if constexpr (MFMA) {
        *reinterpret_cast<v4u*>(op + kb * 1024 + (b + 16 * kg) * 16) = ph;
        *reinterpret_cast<v4u*>(op + kb * 1024 + (b + 8 + 16 * kg) * 16) = pl;
    } else {
        *reinterpret_cast<v4u*>(op + (kb * NB + b) * 128 + kg * 16) = ph;
        *reinterpret_cast<v4u*>(op + (kb * NB + b) * 128 + 64 + kg * 16) = pl;
    }
}

// Partials in LDS, per task and wave: VALU [NB][16] floats (batch-major);
// MFMA [16 rows][8 batch] floats (the hi and lo columns already added).
template <int NB, bool MFMA>
__device__ __forceinline__ constexpr int part_bytes() { return MFMA ? 512 : NB * 16 * 4; }

// One GEMV stage for one compute wave: its tasks (tiles) in order, per task its
// ncw chunks (operand blocks kb0 .. kb0 + ncw - 1) in groups of U, the partial
// written to LDS. Each chunk of a group has its own accumulator (short FMA chains).
// FP8 chunks (1 KB = 16 rows x 64 K of E4M3 codes): lane l's 16 bytes are
// row l % 16 at k = 8 (l / 16) + e (bytes 0..7, operand block 2c) and
// 32 + 8 (l / 16) + e (bytes 8..15, block 2c + 1), e = 0..7. Decoded to bf16
// in registers, exactly (E4M3 values need 4 significant bits): two codes per
// v_cvt_pk_f32_fp8 (OCP E4M3 on gfx950), two floats per bf16 pair.

template <int NB, bool MFMA, int U, bool FP8>
__device__ __forceinline__ void gemv_group(const uint8_t* op, const v4u (&w)[U], int kb, int kg, int lane,
                                           float (&acc)[U][MFMA ? 4 : NB]) {
    if constexpr (FP8) {
        // kb: operand block of the group's first chunk; chunk u covers blocks kb + 2u, kb + 2u + 1
        if constexpr (MFMA) {
            v4u bop[U][2];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h) bop[u][h] = reinterpret_cast<const v4u*>(op + (size_t)(kb + 2 * u + h) * 1024)[lane];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const v4u a0 = fp8x8_to_bf16x8(w[u].x, w[u].y), a1 = fp8x8_to_bf16x8(w[u].z, w[u].w);
                v4f c = {acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
                c = mfma16x16x32(a0, bop[u][0], c);
                c = mfma16x16x32(a1, bop[u][1], c);
                acc[u][0] = c[0]; acc[u][1] = c[1]; acc[u][2] = c[2]; acc[u][3] = c[3];
            }
        } else {
            v4u xh[U][2][NB], xl[U][2][NB];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint8_t* xb = op + (size_t)(kb + 2 * u + h) * NB * 128 + kg * 16;
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        xh[u][h][b] = *reinterpret_cast<const v4u*>(xb + b * 128);
                        xl[u][h][b] = *reinterpret_cast<const v4u*>(xb + b * 128 + 64);
                    }
                }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const v4u wa = fp8x8_to_bf16x8(w[u].x, w[u].y), wb = fp8x8_to_bf16x8(w[u].z, w[u].w);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    float sacc = acc[u][b];
                    sacc = dot2_bf16(wa.x, xh[u][0][b].x, sacc);
                    sacc = dot2_bf16(wa.y, xh[u][0][b].y, sacc);
                    sacc = dot2_bf16(wa.z, xh[u][0][b].z, sacc);
                    sacc = dot2_bf16(wa.w, xh[u][0][b].w, sacc);
                    sacc = dot2_bf16(wa.x, xl[u][0][b].x, sacc);
                    sacc = dot2_bf16(wa.y, xl[u][0][b].y, sacc);
                    sacc = dot2_bf16(wa.z, xl[u][0][b].z, sacc);
                    sacc = dot2_bf16(wa.w, xl[u][0][b].w, sacc);
                    sacc = dot2_bf16(wb.x, xh[u][1][b].x, sacc);
                    sacc = dot2_bf16(wb.y, xh[u][1][b].y, sacc);
                    sacc = dot2_bf16(wb.z, xh[u][1][b].z, sacc);
                    sacc = dot2_bf16(wb.w, xh[u][1][b].w, sacc);
                    sacc = dot2_bf16(wb.x, xl[u][1][b].x, sacc);
                    sacc = dot2_bf16(wb.y, xl[u][1][b].y, sacc);
                    sacc = dot2_bf16(wb.z, xl[u][1][b].z, sacc);
                    sacc = dot2_bf16(wb.w, xl[u][1][b].w, sacc);
                    acc[u][b] = sacc;
                }
            }
        }
    } else if constexpr (MFMA) {
        v4u bop[U];
#pragma unroll
        for (int u = 0; u < U; ++u) bop[u] = reinterpret_cast<const v4u*>(op + (size_t)(kb + u) * 1024)[lane];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v4f c = {acc[u][0], acc[u][1], acc[u][2], acc[u][3]};
            c = mfma16x16x32(w[u], bop[u], c);
            acc[u][0] = c[0]; acc[u][1] = c[1]; acc[u][2] = c[2]; acc[u][3] = c[3];
        }
    } else {
        // all operand reads of the group first, then bf16 dot2 against hi and lo
        v4u xh[U][NB], xl[U][NB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint8_t* xb = op + (size_t)(kb + u) * NB * 128 + kg * 16;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                xh[u][b] = *reinterpret_cast<const v4u*>(xb + b * 128);
                xl[u][b] = *reinterpret_cast<const v4u*>(xb + b * 128 + 64);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float sacc = acc[u][b];
                sacc = dot2_bf16(w[u].x, xh[u][b].x, sacc);
                sacc = dot2_bf16(w[u].y, xh[u][b].y, sacc);
                sacc = dot2_bf16(w[u].z, xh[u][b].z, sacc);
                sacc = dot2_bf16(w[u].w, xh[u][b].w, sacc);
                sacc = dot2_bf16(w[u].x, xl[u][b].x, sacc);
                sacc = dot2_bf16(w[u].y, xl[u][b].y, sacc);
                sacc = dot2_bf16(w[u].z, xl[u][b].z, sacc);
                sacc = dot2_bf16(w[u].w, xl[u][b].w, sacc);
                acc[u][b] = sacc;
            }
        }
    }
}

template <int NB, bool MFMA, int R, int DH, int U, bool MOE, int W, bool FP8>
__device__ __forceinline__ void gemv_consume_u(const Params& P, KParams PK, uint8_t* lds, Stream<R>& S,
                                               const GemvStage& st, int kind, int v, int part_off) {
    const int lane = lane_id();
    const int kg = lane >> 4;
    const GemvPart gp = wg_part(lds, kind);
    // split mode: every wave a K-slice (1/W of K) of each of the WG's tiles;
    // whole-tile mode (tpw): wave v its W-th of the tiles, all of K
    int ta = gp.t0, tb = gp.t1;
    if (st.tpw) {
        const int nt = gp.t1 - gp.t0;
        ta = gp.t0 + udiv(v * nt, W);
        tb = gp.t0 + udiv((v + 1) * nt, W);
    }
    const int ntask = uni(tb - ta);
    const int ncw = st.ncw;
    const int kb0 = st.tpw ? 0 : v * ncw;  // wave's first block inside the operand
    // MoE down-projection: tile t belongs to expert slot t / te - uf, whose
    // operand sits at block slot * nkb
    const int uf = (MOE && kind == SK_DN) ? uni(reinterpret_cast<const Route*>(lds + P.lds_route)->uf) : 0;
    const uint8_t* op = lds + P.lds_op;
    uint8_t* part = lds + part_off;
    constexpr int NA = MFMA ? 4 : NB;
    for (int task = 0; task < ntask; ++task) {
        const int kbt = (MOE && kind == SK_DN) ? kb0 + (udiv(ta + task, st.te) - uf) * st.nkb : kb0;
        float acc[U][NA];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < NA; ++i) acc[u][i] = 0.f;
        for (int k = 0; k < ncw; k += U) {
            if (P.trace && v == 0 && lane == 0 && task == 0 && k == 0) ctrl(lds).tdata[2] = rt_clock();
            stream_refill<R, DH, MOE, W>(S, PK, lds, v);
            if (P.trace && v == 0 && lane == 0 && task == 0 && k == 0) ctrl(lds).tdata[3] = rt_clock();
            stream_wait<R, U>(S);
            if (P.trace && v == 0 && lane == 0 && task == 0 && k == 0) ctrl(lds).tdata[4] = rt_clock();
            v4u w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = stream_read<R>(S, u);
            S.consumed += U;
            gemv_group<NB, MFMA, U, FP8>(op, w, FP8 ? 2 * (kbt + k) : kbt + k, kg, lane, acc);
        }
#pragma unroll
        for (int u = 1; u < U; ++u)
#pragma unroll
            for (int i = 0; i < NA; ++i) acc[0][i] += acc[u][i];
        const int slot = st.tpw ? ta + task - gp.t0 : task * W + v;
        float* dst = reinterpret_cast<float*>(part + (size_t)slot * part_bytes<NB, MFMA>());
        if constexpr (MFMA) {
            // C[row][col] sits at lane col + 16 (row / 4), element row % 4; column b + 8
            // holds the lo part of batch column b
            const int col = lane & 15;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float s = acc[0][i] + xor8(acc[0][i]);
                if (col < 8) dst[(4 * (lane >> 4) + i) * 8 + col] = s;
            }
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float sum = acc[0][b];
                sum = sum_xor32(sum_xor16(sum));
                if (lane < 16) dst[b * 16 + lane] = sum;
            }
        }
    }
}

template <int NB, bool MFMA, int R, int DH, bool MOE, int W, bool FP8>
__device__ __forceinline__ void gemv_consume(const Params& P, KParams PK, uint8_t* lds, Stream<R>& S,
                                             const GemvStage& st, int kind, int v, int part_off) {
    if (st.ncw % 4 == 0) gemv_consume_u<NB, MFMA, R, DH, 4, MOE, W, FP8>(P, PK, lds, S, st, kind, v, part_off);
    else gemv_consume_u<NB, MFMA, R, DH, 1, MOE, W, FP8>(P, PK, lds, S, st, kind, v, part_off);
}

// I/O wave: sum of the partials of task `task` (relative to the WG's first
// tile) for row r (0..15), batch b: the nw compute waves' K-slices, or the one
// wave's partial in whole-tile mode (nw = 1).
template <int NB, bool MFMA>
__device__ __forceinline__ float part_sum(const uint8_t* lds, int part_off, int task, int r, int b, int nw) {
    const uint8_t* base = lds + part_off + (size_t)task * nw * part_bytes<NB, MFMA>();
    float s = 0.f;
    for (int v = 0; v < nw; ++v) {
        const float* p = reinterpret_cast<const float*>(base + v * part_bytes<NB, MFMA>());
        s += MFMA ? p[r * 8 + b] : p[b * 16 + r];
    }
    return s;
}

// Scale of row r of the WG's task-th tile of the current stage (FP8 weights:
// the I/O wave prefetched the stage's row scales into LDS; bf16: 1).
template <bool FP8>
__device__ __forceinline__ float row_scale(const Params& P, const uint8_t* lds, int task, int r) {
    if constexpr (FP8) return reinterpret_cast<const float*>(lds + P.lds_scale)[task * 16 + r];
    else return 1.0f;
}

// ============================================================ attention compute
// K/V page layouts. A page holds 16 positions x DH dims of one kv head (bf16),
// ordered so that each 1 KB chunk is already an MFMA A operand when the DMA
// leaves it in LDS (lane l reads back the 16 bytes it fetched):
//   K: chunk j covers dims 32j..32j+31; lane 16 ((dim % 32) / 8) + pos holds
//      8 dims of one position: the 16x16x32 A operand of S^T = K Q^T
//      (rows = positions, k = dims).
//   V: block jb (512 B, two per chunk) covers dims 16jb..16jb+15; lane
//      16 (pos / 4) + dim % 16 holds 4 positions of one dim: the 16x16x16
//      A operand of O^T = V^T P^T (rows = dims, k = positions).

typedef __attribute__((address_space(3))) const volatile v2u lds_v2u_cv;
// 8 bytes of chunk i of the sequence at byte `off` inside it (lane l: off + 8 l).
template <int R>
__device__ __forceinline__ v2u stream_read8(const Stream<R>& S, int i, int off) {
    return *(lds_v2u_cv*)(S.ring + ((S.consumed + i) & (R - 1)) * KB + off + lane_id() * 8);
}

// One compute wave's pages of one (request, kv head) segment, split-K with an
// online softmax (running max m, sum l, unnormalised o per head, one rescale
// per page), on the matrix cores:
//   S^T[pos][c] = K[pos][:] . B[:][c]: column c = head c % 8, the bf16 hi part
//     of q for c < 8 and the lo part (q - hi) for c >= 8, so that summing
//     columns c and c + 8 gives K . q with q to about 16 significant bits;
//   O^T[dim][c] += V^T[dim][:] . P^T[:][c], P split into hi and lo columns alike.
// Scores are kept in log2 units (q carries log2 e). Lane l ends holding, for
// head l % 8, the scores of positions 4 (l / 16) .. +3 of the page; columns of
// heads >= G are zero and are never written out.
template <int DH, int G, int R, bool MOE, int W>
__device__ __forceinline__ void att_consume(const Params& P, KParams PK, uint8_t* lds, Stream<R>& S, int layer, int v) {
    constexpr int CPP = DH * kPage * 2 / kChunk;  // chunks per page of K (k-steps), and of V
    constexpr int NJB = DH / 16;                  // V dim blocks
    static_assert(G >= 1 && G <= 8, "group size");
    Ctrl& C = ctrl(lds);
    const int lane = lane_id();
    const int tab = att_table(lds, layer);
    const int seg = uni(C.wseg[tab][v]);
    const int npg = seg < 0 ? 0 : uni(C.wnu[tab][v]);
    if (npg == 0) return;
    const int b = seg / P.Hkv;
    const int p = uni(C.seq[b]);
    const int win = tab ? P.win_sliding : 0;
    const int lo = win > 0 ? max(0, p - win + 1) : 0;
    const int lp_first = lo / kPage + uni(C.wu0[tab][v]);  // first logical page of this wave
    const int col = lane & 15, hd = col & 7, rg = lane >> 4;
    const bool hi_col = col < 8;
    // q of the segment as [head][hi, lo][dh] bf16 (the I/O wave split it): lane l's
    // B operand is 8 consecutive values of one head's hi or lo row
    const uint16_t* qh = reinterpret_cast<const uint16_t*>(lds + P.lds_op) + (size_t)v * G * DH * 2;
    const uint16_t* kvs = reinterpret_cast<const uint16_t*>(lds + P.lds_op + W * G * DH * 4) + (size_t)v * 2 * DH;
    v4u qb[CPP];
#pragma unroll
    for (int j = 0; j < CPP; ++j)
        qb[j] = hd < G ? *reinterpret_cast<const v4u*>(qh + (2 * hd + (hi_col ? 0 : 1)) * DH + 32 * j + 8 * rg)
                       : (v4u){0u, 0u, 0u, 0u};

    float m = -INFINITY, lsum = 0.f;
    v4f o[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) o[jb] = (v4f){0.f, 0.f, 0.f, 0.f};

    for (int pg = 0; pg < npg; ++pg) {
        stream_refill<R, DH, MOE, W>(S, PK, lds, v);
        if (P.trace && v == 0 && lane == 0 && pg == 0) ctrl(lds).tdata[2] = rt_clock();
        stream_wait<R, 2 * CPP>(S);
        if (P.trace && v == 0 && lane == 0 && pg == 0) ctrl(lds).tdata[4] = rt_clock();
        v4u kw[CPP];
        v2u vw[NJB];
#pragma unroll
        for (int j = 0; j < CPP; ++j) kw[j] = stream_read<R>(S, j);
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) vw[jb] = stream_read8<R>(S, CPP + jb / 2, (jb & 1) * 512);
        S.consumed += 2 * CPP;
        const int pos0 = (lp_first + pg) * kPage;
        if (pos0 < lo || p - pos0 < kPage) {  // a page with positions outside [lo, p] (uniform)
            // V entries outside the range are zeroed (their weights are 0, their
            // bits need not be finite); the current token's K and V come from the
            // exchange, since its pool slot is being written concurrently.
            uint32_t mk[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int q0 = pos0 + 4 * rg + 2 * h2;
                mk[h2] = ((q0 >= lo && q0 <= p) ? 0x0000FFFFu : 0u) | ((q0 + 1 >= lo && q0 + 1 <= p) ? 0xFFFF0000u : 0u);
            }
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) vw[jb] = (v2u){vw[jb].x & mk[0], vw[jb].y & mk[1]};
            if (p - pos0 < kPage) {
                if (pos0 + col == p) {
#pragma unroll
                    for (int j = 0; j < CPP; ++j) kw[j] = *reinterpret_cast<const v4u*>(kvs + 32 * j + 8 * rg);
                }
                const int e = p - pos0 - 4 * rg;
                if (e >= 0 && e < 4) {
                    const uint32_t sh = (e & 1) * 16, keep = ~(0xFFFFu << sh);
#pragma unroll
                    for (int jb = 0; jb < NJB; ++jb) {
                        const uint32_t vc = (uint32_t)kvs[DH + 16 * jb + col] << sh;
                        if (e < 2) vw[jb].x = (vw[jb].x & keep) | vc;
                        else vw[jb].y = (vw[jb].y & keep) | vc;
                    }
                }
            }
        }
        // scores: hi and lo columns summed, positions outside [lo, p] masked
        v4f sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < CPP; ++j) sc = mfma16x16x32(kw[j], qb[j], sc);
        float s[4], pm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pos = pos0 + 4 * rg + i;
            const float t = sc[i] + dpp_xor8(sc[i]);
            s[i] = (pos >= lo && pos <= p) ? t : -INFINITY;
            pm = fmaxf(pm, s[i]);
        }
        pm = max_xor32(max_xor16(pm));  // page max of head hd
        const float mn = fmaxf(m, pm);  // finite: every page holds a position in [lo, p]
        const float alpha = fast_exp2(m - mn);
        float pr[4], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[i] = fast_exp2(s[i] - mn);
            ps += pr[i];
        }
        lsum = lsum * alpha + ps;
        m = mn;
        if (!__all(alpha == 1.0f)) {
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) o[jb] *= alpha;
        }
        uint32_t pw[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const uint32_t ph = cvt_bf16x2(pr[2 * h2], pr[2 * h2 + 1]);
            const uint32_t pl = cvt_bf16x2(pr[2 * h2] - bf_lo(ph), pr[2 * h2 + 1] - bf_hi(ph));
            pw[h2] = hi_col ? ph : pl;
        }
        const v2u pb = {pw[0], pw[1]};
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) o[jb] = mfma16x16x16(vw[jb], pb, o[jb]);
    }
    // hi + lo columns of O; l over the four row groups; the wave partial to LDS
    // (m in natural-log units)
    constexpr float kLog2e = 1.4426950408889634f;
    const float lt = sum_xor32(sum_xor16(lsum));
    float* rec = reinterpret_cast<float*>(lds + P.lds_part[1]) + (size_t)v * (16 + G * DH);
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
        v4f t = o[jb];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] += dpp_xor8(t[i]);
        if (col < G) *reinterpret_cast<v4f*>(rec + 16 + col * DH + 16 * jb + 4 * rg) = t;
    }
    if (lane < G) {
        rec[lane] = m * (1.0f / kLog2e);
        rec[8 + lane] = lt;
    }
}

// ============================================================ I/O wave helpers
// bf16 gains [K] -> LDS (kept bf16, widened on use); all loads issued before any is used.
__device__ __forceinline__ void io_load_gains(const uint16_t* g, uint16_t* dst, int K) {
    const int lane = lane_id();
    const v4u* src = reinterpret_cast<const v4u*>(g);
    for (int base = 0; base < K / 8; base += 64 * 8) {
        v4u t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = base + u * 64 + lane;
            t[u] = i < K / 8 ? __builtin_nontemporal_load(src + i) : (v4u){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = base + u * 64 + lane;
            if (i < K / 8) reinterpret_cast<v4u*>(dst)[i] = t[u];
        }
    }
}

// Embedding rows as the layer-0 input, times the layer-0 attention-norm gains,
// in the final operand layout; their sums of squares (for the RMSNorm scale)
// go to the control block as wave 0's share.
template <int NB, bool MFMA>
__device__ __forceinline__ void io_load_embed(const Params& P, uint8_t* lds, int n) {
    Ctrl& C = ctrl(lds);
    const int lane = lane_id();
    constexpr int NBo = MFMA ? 8 : NB;
    const int K = P.d;
    uint8_t* op = lds + P.lds_op;
    uint16_t* gains = reinterpret_cast<uint16_t*>(lds + P.lds_gain);
    // Rows in groups of BG, each group's loads in flight together (the first
    // group's also with the gains' loads): one round trip per group, not per row.
    constexpr int BG = NBo < 4 ? NBo : 4;
    bool have_gains = false;
#pragma unroll
    for (int b0 = 0; b0 < NBo; b0 += BG) {
        float ss[BG];
#pragma unroll
        for (int bb = 0; bb < BG; ++bb) ss[bb] = 0.f;
        for (int k0 = lane * 8; k0 < K; k0 += 512 * 4) {
            v4u t[BG][4];
#pragma unroll
            for (int bb = 0; bb < BG; ++bb) {
                const int b = b0 + bb;
                const int tok = (b < n && ((C.valid >> b) & 1)) ? C.tok[b] : 0;
                const uint16_t* e = P.embed + (int64_t)tok * K;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int k = k0 + u * 512;
                    t[bb][u] = (v4u){0u, 0u, 0u, 0u};
                    if (k < K && b < n) t[bb][u] = *reinterpret_cast<const v4u*>(e + k);
                }
            }
            if (!have_gains) {
                io_load_gains(P.attn_norm, gains, K);
                __builtin_amdgcn_s_waitcnt(0xc07f);  // the gains are in LDS
                have_gains = true;
            }
#pragma unroll
            for (int bb = 0; bb < BG; ++bb) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int k = k0 + u * 512;
                    if (k < K) {
                        float x[8] = {bf_lo(t[bb][u].x), bf_hi(t[bb][u].x), bf_lo(t[bb][u].y), bf_hi(t[bb][u].y),
                                      bf_lo(t[bb][u].z), bf_hi(t[bb][u].z), bf_lo(t[bb][u].w), bf_hi(t[bb][u].w)};
                        const v4u g = *reinterpret_cast<const v4u*>(gains + k);
                        const float gf[8] = {bf_lo(g.x), bf_hi(g.x), bf_lo(g.y), bf_hi(g.y),
                                             bf_lo(g.z), bf_hi(g.z), bf_lo(g.w), bf_hi(g.w)};
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            ss[bb] += x[j] * x[j];
                            x[j] *= gf[j];
                        }
                        store_operand8<NB, MFMA>(op, k / 32, b0 + bb, (k % 32) / 8, x);
                    }
                }
            }
        }
#pragma unroll
        for (int bb = 0; bb < BG; ++bb) {
            const float t = wave_sum_f(ss[bb]);
            if (lane == 0) {
                C.ssw[0][b0 + bb] = t;
                for (int x = 1; x < kMaxComputeWaves; ++x) C.ssw[x][b0 + bb] = 0.f;
            }
        }
    }
}

// Integer sum over the 64 lanes (every lane gets it).
__device__ __forceinline__ int wave_sum_i(int x) {
    x += __builtin_amdgcn_mov_dpp(x, 0xB1, 0xf, 0xf, false);   // lane ^ 1
    x += __builtin_amdgcn_mov_dpp(x, 0x4E, 0xf, 0xf, false);   // lane ^ 2
    x += __builtin_amdgcn_mov_dpp(x, 0x141, 0xf, 0xf, false);  // 8-lane half-row mirror
    x += __builtin_amdgcn_mov_dpp(x, 0x140, 0xf, 0xf, false);  // 16-lane row mirror
    auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    x = (int)(r[0] + r[1]);
    r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    return (int)(r[0] + r[1]);
}

// MoE routing of one layer (I/O wave; the router logits are final). Per
// request: the top_k experts by router logit, exact ties to the lower expert
// index (a logit that is NaN ranks below every number), and the softmax of
// their logits. Then the step's expert list (ascending), this WG's tiles of the
// expert gate/up and down stages, and its down-projection weights per expert
// slot. Lane l holds experts l and l + 64.
__device__ void io_route(const Params& P, uint8_t* lds, int layer) {
    Ctrl& C = ctrl(lds);
    Route& RT = *reinterpret_cast<Route*>(lds + P.lds_route);
    const int lane = lane_id();
    const int n = P.n, E = P.E, K = P.topk;
    const float* rlg = layer_copy(P.rlog, P.rlog_lb, layer);
    // Top-k of every request at once: lane l serves request g = l / 8 and holds
    // experts [q EPL, (q + 1) EPL), q = l % 8, EPL = ceil(E / 8) <= 16. Each lane
    // keeps its best 8 in order (higher logit first, ties to the lower expert);
    // the 8 lanes of a request then take their heads' maximum 8 times (ties to the
    // lower lane, whose experts are the lower ones). NaN logits count as -inf.
    const int g = lane >> 3, q = lane & 7;
    const int EPL = (E + 7) >> 3;
    float lv[kMaxTopK];
    int li[kMaxTopK];
    {
        // unconditional loads of clamped in-range indices (all 16 in flight
        // together), masked afterwards
        float av[16];
        int ai[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) av[i] = rlg[min(g * E + q * EPL + i, kMaxBatch * E - 1)];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int e = q * EPL + i;
            const bool real = g < n && i < EPL && e < E;
            av[i] = (real && av[i] == av[i]) ? av[i] : -INFINITY;
            ai[i] = real ? e : 0x7fffffff;
        }
        // bitonic sort of the 16 (logit, expert) keys, best first: key a beats b
        // if its logit is higher, or equal with the lower expert (keys are unique)
#pragma unroll
        for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
            for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int l = i ^ j;
                    if (l <= i) continue;
                    const bool l_beats_i = av[l] > av[i] || (av[l] == av[i] && ai[l] < ai[i]);
                    const bool sw = (i & k) == 0 ? l_beats_i : !l_beats_i;
                    const float tv = sw ? av[l] : av[i];
                    const int ti = sw ? ai[l] : ai[i];
                    av[l] = sw ? av[i] : av[l];
                    ai[l] = sw ? ai[i] : ai[l];
                    av[i] = tv;
                    ai[i] = ti;
                }
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j) {
            lv[j] = av[j];
            li[j] = ai[j];
        }
    }
    float top[kMaxTopK];
    int sel[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        top[k] = -INFINITY;
        sel[k] = 0;
        if (k >= K) continue;
        float M = lv[0];
        M = fmaxf(M, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(M), 0x041F)));  // lane ^ 1
        M = fmaxf(M, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(M), 0x081F)));  // lane ^ 2
        M = fmaxf(M, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(M), 0x101F)));  // lane ^ 4
        const uint64_t hit = __ballot(lv[0] == M);
        const uint32_t mine = (uint32_t)(hit >> (8 * g)) & 0xFFu;  // lanes of this request at the maximum
        const int wl = __builtin_ctz(mine | 0x100u);
        const int e = __shfl(li[0], 8 * g + (wl & 7), 64);
        if (q == wl) {  // the winning lane pops its head
#pragma unroll
            for (int j = 0; j + 1 < kMaxTopK; ++j) {
                lv[j] = lv[j + 1];
                li[j] = li[j + 1];
            }
            lv[kMaxTopK - 1] = -INFINITY;
            li[kMaxTopK - 1] = 0x7fffffff;
        }
        top[k] = M;
        sel[k] = e;
    }
    if (lane < 4) RT.umask[lane] = 0u;
    if (g < n) {
        float z = 0.f, ex[kMaxTopK];
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
            ex[k] = (k < K && top[0] > -INFINITY) ? __expf(top[k] - top[0]) : (k < K ? 1.f : 0.f);
            z += ex[k];
        }
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k)
            if (q == k && k < K) {
                RT.sel[g][k] = sel[k];
                RT.selw[g][k] = ex[k] / z;
                // optional export of the selection (workgroup 0), for checking
                if (P.route_dbg && blockIdx.x == 0) P.route_dbg[(layer * kMaxBatch + g) * kMaxTopK + k] = sel[k];
            }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the selections and the cleared mask are in LDS
    __builtin_amdgcn_wave_barrier();
    // union of the selections: lane 8 g + k ORs in its request's k-th expert
    if (g < n && q < K)
        __hip_atomic_fetch_or(&RT.umask[sel[q] >> 5], 1u << (sel[q] & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    const uint64_t m0 = (uint64_t)uni(RT.umask[0]) | ((uint64_t)uni(RT.umask[1]) << 32);
    const uint64_t m1 = (uint64_t)uni(RT.umask[2]) | ((uint64_t)uni(RT.umask[3]) << 32);
    const int n0 = __builtin_popcountll(m0), nU = n0 + __builtin_popcountll(m1);
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;  // bits of the lanes below this one
    if ((m0 >> lane) & 1ull) RT.eu[__builtin_popcountll(m0 & below)] = lane;
    if ((m1 >> lane) & 1ull) RT.eu[n0 + __builtin_popcountll(m1 & below)] = 64 + lane;
    const int w = blockIdx.x, NW = P.NW;
    const int T3 = nU * P.gu.te, T4 = nU * P.dn.te;
    const int d0 = udiv(w * T4, NW), d1 = udiv((w + 1) * T4, NW);
    const int uf = udiv(d0, P.dn.te);
    if (lane == 0) {
        if (w == 0) __hip_atomic_fetch_add(P.moe_used, (unsigned long long)nU, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        C.part[SK_GU][0] = 0;
        C.part[SK_GU][1] = udiv(w * T3, NW);
        C.part[SK_GU][2] = udiv((w + 1) * T3, NW);
        C.part[SK_DN][0] = 0;
        C.part[SK_DN][1] = d0;
        C.part[SK_DN][2] = d1;
        RT.nU = nU;
        RT.uf = uf;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the lists are in LDS
    __builtin_amdgcn_wave_barrier();
    // down-projection weights of request b for expert slot i (expert eu[uf + i])
    if (lane < kMaxSpan * kMaxBatch) {
        const int i = lane >> 3, b = lane & 7;
        float wv = 0.f;
        if (b < n && uf + i < nU) {
            const int e = RT.eu[uf + i];
            for (int k = 0; k < K; ++k)
                if (RT.sel[b][k] == e) wv = RT.selw[b][k];
        }
        RT.wu[i][b] = wv;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) C.route_layer = layer;
}

// SplitMix64 output step (Steele, Lea, Flood 2014)
__device__ __forceinline__ uint64_t splitmix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// ============================================================ the kernel
// I/O role (wave 0 of each workgroup, between stages): prologue (request
// checks, page-table validation, attention partitions, layer-0 input); after
// each stage: epilogue, publish, wait for the producers of the next stage,
// load its inputs into LDS.
template <int NB, bool MFMA, int DH, int G, bool MOE, int W>
__device__ __forceinline__ void io_prologue(KParams PK, uint8_t* lds) {
    const Params& P = *(const Params*)launder(PK);
    Ctrl& C = ctrl(lds);
    const int lane = lane_id();
    const int w = blockIdx.x;
    const int NW = P.NW;
    const int n = P.n;
    // Every lane loads its own layer's window and its own request's scalars, so
    // these loads are in flight together (one round trip, not one per layer or
    // request).
    {
        const int win_l = (P.win_sliding > 0 && lane < P.L) ? P.window[lane] : 0;
        int p = 0, t = 0, k = 0;
        float T = 0.f;
        if (lane < n) {
            p = P.seq_lens[lane];
            t = P.tokens_in[lane];
            T = P.temperature ? P.temperature[lane] : 0.f;
            k = P.top_k ? P.top_k[lane] : 0;
        }
        const uint64_t slide = __ballot(win_l > 0);
        const bool ok = lane < n && p >= 0 && p < P.max_pos && (p / kPage) < P.mpps && t >= 0 && t < P.V && T >= 0.f &&
                        T == T && T < 3.0e38f;
        const int valid = (int)(uint32_t)__ballot(ok);
        if (lane < n) {
            C.seq[lane] = p;
            C.tok[lane] = t;
            C.temp[lane] = T;
            C.topk[lane] = (k <= 0 || k >= P.V) ? 0 : min(k, kMaxSampleTopK);  // 0: no limit
        }
        if (lane == 0) {
            C.abort = 0;
            C.n = n;
            C.sliding[0] = (uint32_t)slide;
            C.sliding[1] = (uint32_t)(slide >> 32);
            C.route_layer = -1;
            C.opsync = 0;
            C.pubs = 0;
            for (int kk = 0; kk < SK_KINDS; ++kk) {
                if (kk == 1 || (kk == SK_RT && !MOE)) continue;
                const GemvPart gp = gemv_part(stage_of(P, kk), w, NW);
                C.part[kk][0] = gp.s;
                C.part[kk][1] = gp.t0;
                C.part[kk][2] = gp.t1;
            }
            C.valid = valid;
            C.bad = 0;
            if (w == 0) st_sc1_u(bad_mask(P, 1), 0u);
        }
    }
    __builtin_amdgcn_wave_barrier();
    // validate this WG's share of the page-table entries 0 .. p/16 of every request
    {
        int tot = 0, off[kMaxBatch + 1];
        for (int b = 0; b < n; ++b) { off[b] = tot; tot += ((C.valid >> b) & 1) ? C.seq[b] / kPage + 1 : 0; }
        off[n] = tot;
        const int e0 = udiv(w * tot, NW), e1 = udiv((w + 1) * tot, NW);
        int badm = 0;
        for (int e = e0 + lane; e < e1; e += 64) {
            int b = 0;
            while (e >= off[b + 1]) ++b;
            int pid = P.page_table[(int64_t)b * P.mpps + (e - off[b])];
            if (pid < 0 || pid >= P.n_pages) badm |= 1 << b;
        }
        for (int msk = 1; msk < 64; msk <<= 1) badm |= __shfl_xor(badm, msk, 64);
        if (lane == 0 && badm) {
            __hip_atomic_fetch_or(bad_mask(P, 0), (uint32_t)badm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            latch_error(P, 5u, 0xFFFFu);
        }
        raise_flag(P, flag_val(P));
    }
    // attention partitions for the full (table 0) and sliding (table 1) layers:
    // segment s = b * Hkv + g has U_s pages covering [lo, p]. It is served by
    // n_s consecutive compute waves from Wf(s) = sum of n_s' over s' < s, with
    // n_s proportional to U_s over all W NW waves (so every workgroup gets about
    // the same number of pages, whatever the mix of lengths): n_s =
    // max(least_s, floor(U_s W NW / U)); then the waves left over (or missing)
    // go to (or come from) the segments with the most (fewest) pages per wave,
    // at most one per segment and round (ties to the lower segment). Wave j of
    // n_s gets pages [ceil(j U_s / n_s), ceil((j+1) U_s / n_s)). Lane s holds
    // segment s throughout (nseg <= 64): no serial scans, and every page id the
    // workgroup's waves need is loaded in one go.
    for (int tab = 0; tab < (P.win_sliding > 0 ? 2 : 1); ++tab) {
        const int win = tab ? P.win_sliding : 0;
        const int nseg = n * P.Hkv;
        const bool segl = lane < nseg;
        int us = 0;
        if (segl) {
            const int b = lane / P.Hkv;
            if ((C.valid >> b) & 1) {
                const int p = C.seq[b], lo = win > 0 ? max(0, p - win + 1) : 0;
                us = p / kPage - lo / kPage + 1;
            }
        }
        int uincl = us;  // inclusive prefix sum of the pages over the segments
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(uincl, d, 64);
            if (lane >= d) uincl += t;
        }
        const int U = __builtin_amdgcn_readlane(uincl, 63);
        if (segl) C.segu[tab][lane] = uincl - us;
        if (lane == 0) {
            C.segu[tab][nseg] = U;
            C.nseg[tab] = nseg;
        }
        const int WT = W * NW;
        // fewest waves a segment may have: its pages must fit the page-id table
        // (P.maxu per wave); the host sized it so that these minima always fit
        // within the W NW waves
        const int least = segl ? max(1, udiv(us + P.maxu - 1, P.maxu)) : 0;
        int need = segl ? max(least, U > 0 ? (int)(((uint64_t)us * (uint64_t)WT) / (uint64_t)U) : 1) : 0;
        int spare = WT - wave_sum_i(need);
        while (spare != 0) {
            // pages per wave x 1024 ranks the segments; -1 where no change applies
            const bool give = spare > 0;
            int key = -1;
            if (segl) {
                const int ppw = (int)((uint32_t)us * 1024u / (uint32_t)need);
                if (give && us > need) key = ppw;                   // most pages per wave gain one
                if (!give && need > least) key = 0x7fffffff - ppw;  // fewest pages per wave lose one
            }
            const int cnt = __builtin_popcountll(__ballot(key >= 0));
            if (cnt == 0) break;  // giving: no segment gains from another wave
            const int k = min(give ? spare : -spare, cnt);
            int rank = 0;  // eligible segments ahead of this one
            for (int t = 0; t < nseg; ++t) {
                const int kt = __builtin_amdgcn_readlane(key, t);
                rank += (kt > key || (kt == key && t < lane)) ? 1 : 0;
            }
            if (key >= 0 && rank < k) need += give ? 1 : -1;
            spare += give ? -k : k;
        }
        int incl = need;  // inclusive prefix sum over lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int t = __shfl_up(incl, d, 64);
            if (lane >= d) incl += t;
        }
        const int excl = incl - need;
        if (segl) C.segw[tab][lane] = excl;
        if (lane == nseg - 1) C.segw[tab][nseg] = incl;
        // this workgroup's waves: segment, first page and page count
        const uint64_t starts = __ballot(segl);  // (need >= 1: the starts increase)
        int wsg[W], wu0[W], wnu[W];
#pragma unroll
        for (int vv = 0; vv < W; ++vv) {
            const int om = W * w + vv;
            const int sn = __builtin_popcountll(__ballot(segl && excl <= om) & starts);  // segments starting at or before om
            int seg = -1, u0 = 0, nu = 0;
            if (U > 0 && sn > 0) {
                const int s0 = sn - 1;
                const int wf1 = __builtin_amdgcn_readlane(incl, s0);
                const int uss = __builtin_amdgcn_readlane(us, s0);
                if (om < wf1 && uss > 0) {
                    const int wf0 = __builtin_amdgcn_readlane(excl, s0);
                    const int nwv = __builtin_amdgcn_readlane(need, s0), j = om - wf0;
                    u0 = udiv(j * uss + nwv - 1, nwv);
                    nu = udiv((j + 1) * uss + nwv - 1, nwv) - u0;
                    seg = s0;
                }
            }
            wsg[vv] = seg;
            wu0[vv] = u0;
            wnu[vv] = nu;
            if (lane == 0) {
                C.wseg[tab][vv] = seg;
                C.wu0[tab][vv] = u0;
                C.wnu[tab][vv] = nu;
            }
        }
        // page ids of the waves' pages: item i of the W waves' pages in order,
        // four per lane per round, all loads of a round in flight together
        int tot = 0;
#pragma unroll
        for (int vv = 0; vv < W; ++vv) tot += wnu[vv];
        int32_t* pids0 = reinterpret_cast<int32_t*>(lds + P.lds_units) + tab * W * P.maxu;
        for (int r0 = 0; r0 < tot; r0 += 256) {
            int pid[4], dst[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int it = r0 + 64 * q + lane;
                int vv = 0, base = 0, acc = 0, sg = -1, u0 = 0;
#pragma unroll
                for (int x = 0; x < W; ++x) {
                    if (it >= acc && it < acc + wnu[x]) {
                        vv = x;
                        base = acc;
                        sg = wsg[x];
                        u0 = wu0[x];
                    }
                    acc += wnu[x];
                }
                const int k = it - base;
                dst[q] = it < tot ? vv * P.maxu + k : -1;
                pid[q] = 0;
                if (it < tot && sg >= 0) {
                    const int b = sg / P.Hkv;
                    const int p = C.seq[b], lo = win > 0 ? max(0, p - win + 1) : 0;
                    pid[q] = P.page_table[(int64_t)b * P.mpps + lo / kPage + u0 + k];
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (dst[q] >= 0) pids0[dst[q]] = (pid[q] < 0 || pid[q] >= P.n_pages) ? 0 : pid[q];  // (a bad id: the request is already marked bad)
        }
    }
    io_load_embed<NB, MFMA>(P, lds, n);

}

// I/O wave, while the compute waves stream stage sid: fetch what this stage's
// epilogue and the next stage's prologue need that is already final, so that
// after B_out only the producer-dependent work remains. Results go to LDS
// regions the compute waves do not touch during this stage:
//   QKV: RoPE (cos, sin) per (task, request, pair) and the page of each new K/V row;
//   ATT: the FFN-norm gains (for the gate/up or router operand, two stages on);
//   O:   the residual x rows of this WG's tiles;
//   DN:  the residual h rows of this WG's tiles; the next attention-norm (or final-norm) gains.
template <int NB, bool MFMA, int DH, int G, bool MOE, bool FP8>
__device__ __forceinline__ void io_prefetch(KParams PK, uint8_t* lds, int sid) {
    const Params& P = *(const Params*)launder(PK);
    Ctrl& C = ctrl(lds);
    const int lane = lane_id();
    const int n = P.n;
    const int layer = stage_layer<MOE>(P, sid), kind = stage_kind<MOE>(P, sid);
    float* res = reinterpret_cast<float*>(lds + P.lds_res);  // [task][b][16]
    if (FP8 && kind != 1) {
        // FP8 weights: the row scales of this WG's tiles, in packed row order
        const GemvStage& st = stage_of(P, kind);
        const GemvPart gp = wg_part(lds, kind);
        const float* sc = P.wscale + (kind == 5 ? 0 : (int64_t)layer * P.scale_lb) + st.soff;
        float* dst = reinterpret_cast<float*>(lds + P.lds_scale);
        for (int i = lane; i < (gp.t1 - gp.t0) * 16; i += 64) dst[i] = sc[(int64_t)gp.t0 * 16 + i];
    }
    if (kind == 0) {
        const GemvPart gp = wg_part(lds, 0);
        const int tpl = DH / 16;
        const int ntask = gp.t1 - gp.t0;
        for (int idx = lane; idx < ntask * kMaxBatch * 8; idx += 64) {
            const int r = idx & 7, b = (idx >> 3) & 7, task = idx >> 6;
            const int i = 8 * ((gp.t0 + task) % tpl) + r;  // pair index < dh/2
            float cs = 1.f, sn = 0.f;
            if (b < n && ((C.valid >> b) & 1)) {
                const float2 v = reinterpret_cast<const float2*>(P.rope_cs)[(int64_t)C.seq[b] * (DH / 2) + i];
                cs = v.x;
                sn = v.y;
            }
            res[(task * kMaxBatch + b) * 16 + 2 * r] = cs;
            res[(task * kMaxBatch + b) * 16 + 2 * r + 1] = sn;
        }
        if (lane < n) {
            const int b = lane;
            C.apid[b] = ((C.valid >> b) & 1) ? P.page_table[(int64_t)b * P.mpps + C.seq[b] / kPage] : 0;
        }
    } else if (MOE && kind == 6) {
        // MoE: x of the next layer starts as h (the expert outputs are added to
        // it atomically); this WG's slice of the [n][d] rows. The previous x is
        // dead: every WG has read it before raising its O flag.
        const int tot = n * P.d;
        const int e0 = udiv(blockIdx.x * tot, P.NW), e1 = udiv((blockIdx.x + 1) * tot, P.NW);
        const float* hl = layer_copy(P.hparts, P.h_lb, layer);
        float* xn1 = layer_copy(P.xparts, P.x_lb, layer + 1);
        for (int e = e0 + lane; e < e1; e += 64) {
            const int b = udiv(e, P.d), row = e - b * P.d;
            float h = 0.f;
            for (int sp = 0; sp < P.o.S; ++sp) h += ldk_f(hl, (int64_t)(sp * kMaxBatch + b) * P.d + row);
            st_sc1_f(xn1 + b * P.d + row, h);
        }
    } else if (kind == 2 || kind == 4) {
        const GemvStage& st = kind == 2 ? P.o : P.dn;
        const GemvPart gp = wg_part(lds, kind);
        if (gp.s == 0 && !(MOE && kind == 4)) {
            // residual rows: x_l (embedding at layer 0, else the sum of the x parts) or h
            const int ntask = gp.t1 - gp.t0;
            const bool emb = kind == 2 && layer == 0;
            const float* src = kind == 2 ? layer_copy(P.xparts, P.x_lb, layer) : layer_copy(P.hparts, P.h_lb, layer);
            const int nparts = kind == 2 ? P.xn : P.o.S;
            for (int idx0 = 0; idx0 < ntask * kMaxBatch * 16; idx0 += 64 * 8) {
                float v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int idx = idx0 + u * 64 + lane;
                    const int r = idx & 15, b = (idx >> 4) & 7, task = idx >> 7;
                    const int row = 16 * (gp.t0 + task) + r;
                    v[u] = 0.f;
                    if (idx < ntask * kMaxBatch * 16 && b < n) {
                        if (emb) {
                            const int tok = ((C.valid >> b) & 1) ? C.tok[b] : 0;
                            v[u] = bf16_to_f(P.embed[(int64_t)tok * P.d + row]);
                        } else {
#pragma unroll
                            for (int sp = 0; sp < kMaxSplit; ++sp)
                                if (sp < nparts) {
                                    const int64_t wi = (int64_t)(sp * kMaxBatch + b) * P.d + row;
                                    // (already seen current by this WG's operand loads)
                                    if constexpr (kTagOps<MFMA, MOE>) v[u] += ld_tag_value(reinterpret_cast<const uint64_t*>(src), (uint32_t)wi);
                                    else if (MOE && kind == 2) v[u] += ldc_f(src, wi);  // MoE x: summed by atomics
                                    else v[u] += ldk_f(src, wi);
                                }
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int idx = idx0 + u * 64 + lane;
                    if (idx < ntask * kMaxBatch * 16) res[idx] = v[u];
                }
            }
        }
        (void)st;
        // the next attention-norm (or final-norm) gains; the FFN-norm gains were
        // fetched during the attention stage
        if (kind == 4)
            io_load_gains(layer + 1 < P.L ? P.attn_norm + (int64_t)(layer + 1) * P.d : P.final_norm,
                          reinterpret_cast<uint16_t*>(lds + P.lds_gain), P.d);
    } else if (kind == 1) {
        // FFN-norm gains (the gate/up or router operand's): the attention stage is
        // long and its inputs are the I/O wave's, while the O stage is short and
        // its I/O wave fetches the residual rows; no compute wave reads the gains
        // between the QKV operand load and the gate/up (router) one
        io_load_gains(P.ffn_norm + (int64_t)layer * P.d, reinterpret_cast<uint16_t*>(lds + P.lds_gain), P.d);
    }
}

template <int NB, bool MFMA, int DH, int G, bool MOE, int W, bool FP8>
__device__ __forceinline__ void io_stage(KParams PK, uint8_t* lds, int sid) {
    const Params& P = *(const Params*)launder(PK);
    Ctrl& C = ctrl(lds);
    const int lane = lane_id();
    const int w = blockIdx.x;
    const int NW = P.NW;
    const int n = P.n;
    const int layer = stage_layer<MOE>(P, sid), kind = stage_kind<MOE>(P, sid);
    const float* res = reinterpret_cast<const float*>(lds + P.lds_res);
    const uint32_t tag = stage_tag(P, sid);
    trace_mark(P, sid, 1);
    // RMSNorm scale of each input row, 1/sqrt(mean of squares + eps), from the
    // compute waves' sums of squares (hardware reciprocal and reciprocal square
    // root, a few ulp). At batch 1 every lane keeps it in a register (this
    // epilogue is on the step's critical path); otherwise lane b stores request b's.
    float rsc1 = 0.f;
    if (kind == 0 || kind == 3 || kind == 5 || kind == 6) {
        if constexpr (NB == 1) {
            float t = 0.f;
#pragma unroll
            for (int x = 0; x < W; ++x) t += C.ssw[x][0];
            rsc1 = __builtin_amdgcn_rsqf(t * __builtin_amdgcn_rcpf((float)P.d) + P.eps);
        } else {
            if (lane < kMaxBatch) {
                float t = 0.f;
#pragma unroll
                for (int x = 0; x < W; ++x) t += C.ssw[x][lane];
                C.rsc[lane] = __builtin_amdgcn_rsqf(t * __builtin_amdgcn_rcpf((float)P.d) + P.eps);
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
        }
    }
    auto rscale = [&](int b) -> float {
        if constexpr (NB == 1) return rsc1;
        else return C.rsc[b];
    };
    // ============================ epilogue of this stage
    bool ok = true;
    if (kind == 0) {
        // ---- QKV epilogue: RoPE, q out, k/v append + current-token copy
        if (layer == 0) {
            ok = wait_flags(P, flag_val(P), 0, NW, 0xFFFE);  // page-table validation complete
            if (ok && lane == 0) C.bad = (int32_t)ld_sc1_u(bad_mask(P, 0));
            __builtin_amdgcn_wave_barrier();
        }
        const GemvPart gp = wg_part(lds, 0);
        const int tpl = DH / 16;  // tiles per head
        const int valid = uni(C.valid), bad = uni(C.bad);
        for (int t = gp.t0; ok && t < gp.t1; ++t) {
            const int task = t - gp.t0;
            const int head = t / tpl, j = t % tpl;
            for (int idx = lane; idx < 8 * kMaxBatch; idx += 64) {
                const int r = idx & 7, b = idx >> 3;
                if (b >= n || !((valid >> b) & 1)) continue;
                float y0 = part_sum<NB, MFMA>(lds, P.lds_part[kind], task, r, b, W) * row_scale<FP8>(P, lds, task, r) * rscale(b);
                float y1 = part_sum<NB, MFMA>(lds, P.lds_part[kind], task, r + 8, b, W) * row_scale<FP8>(P, lds, task, r + 8) *
                           rscale(b);
                const int i = 8 * j + r;          // pair index < dh/2
                const int p = C.seq[b];
                if (head < P.Hq + P.Hkv) {
                    const float cs = res[(task * kMaxBatch + b) * 16 + 2 * r], sn = res[(task * kMaxBatch + b) * 16 + 2 * r + 1];
                    const float a = y0, c2 = y1;
                    y0 = a * cs - c2 * sn;
                    y1 = a * sn + c2 * cs;
                }
                if (head < P.Hq) {
                    st_tag_f(P.q, (uint32_t)(b * P.Hq * DH + head * DH + i), y0, tag);
                    st_tag_f(P.q, (uint32_t)(b * P.Hq * DH + head * DH + i + DH / 2), y1, tag);
                } else {
                    const int kvh = head - P.Hq;
                    const int isv = kvh >= P.Hkv;
                    const int g = isv ? kvh - P.Hkv : kvh;
                    const uint16_t h0 = f_to_bf16(y0), h1 = f_to_bf16(y1);
                    const uint32_t cb = (uint32_t)(((b * P.Hkv + g) * 2 + isv) * DH);
                    st_tag(P.kvcur, cb + i, h0, tag);
                    st_tag(P.kvcur, cb + i + DH / 2, h1, tag);
                    if (!((bad >> b) & 1)) {
                        const int pid = C.apid[b];
                        uint16_t* blk = (isv ? P.vpool : P.kpool) + (int64_t)layer * P.kv_layer_elems +
                                        ((int64_t)pid * P.Hkv + g) * kPage * DH;
                        const int sl = p % kPage;
                        blk[isv ? kv_elem_v<DH>(sl, i) : kv_elem_k<DH>(sl, i)] = h0;
                        blk[isv ? kv_elem_v<DH>(sl, i + DH / 2) : kv_elem_k<DH>(sl, i + DH / 2)] = h1;
                    }
                }
            }
        }
    } else if (kind == 1) {
        // ---- ATT epilogue. (1) the compute waves merged their wave partials
        // into this WG's partial of each segment it serves (att_wg_merge).
        // (2) every WG of a segment merges a slice of the segment's outputs.
        const int tab = att_table(lds, layer);
        constexpr int hdr = att_hdr_words(G);
        const int GR = hdr + G * DH;                   // global record (words)
        constexpr float kL2e = 1.4426950408889634f;
        trace_mark(P, sid, 2);
        // (2) every WG of a segment merges a slice (quads [q0, q1) of the G x DH / 4)
        // of the segment's outputs from all its ns WG partials: one lane per
        // (partial, quad) value pair and per (head of the slice, partial) header,
        // all loaded together and polled until every tag is current.
        constexpr int PU = att_merge_pu(G, DH);             // items per lane (at most 64 PU of each kind)
        float* cbuf = reinterpret_cast<float*>(lds + P.lds_op);             // weights [head - h0][256]
        float* mlb = cbuf + G * 256;                                        // headers [item][m, l]
        v4f* red = reinterpret_cast<v4f*>(mlb + 2 * 64 * PU);               // products [pair]
        const uint64_t deadline = rt_clock() + P.wait_ticks;
        for (int vv = 0; vv < W && ok;) {
            const int s = C.wseg[tab][vv];
            int ve = vv + 1;
            if (s < 0) { vv = ve; continue; }
            while (ve < W && C.wseg[tab][ve] == s) ++ve;
            vv = ve;
            const int wf0 = C.segw[tab][s], wf1 = C.segw[tab][s + 1];
            const int g0 = wf0 / W, g1 = (wf1 - 1) / W;
            const int ns = g1 - g0 + 1;        // WG partials of this segment (<= 256)
            // The merging WGs are those whose first wave serves the segment, so that
            // a WG serving the end of one segment and the start of the next merges
            // only the first (every WG then polls and merges one slice, not two in a
            // row); a segment inside one WG that does not start there is merged by it.
            const int m0 = (wf0 % W == 0 || g0 == g1) ? g0 : g0 + 1;
            if (w < m0) continue;
            const int nm = g1 - m0 + 1;        // merging WGs
            const int me = w - m0;             // my slice index
            constexpr int QD = G * DH / 4;
            const int q0 = udiv(me * QD, nm), q1 = udiv((me + 1) * QD, nm);
            if (q1 <= q0) continue;
            const int nq = q1 - q0, npair = ns * nq;
            const int h0 = 4 * q0 / DH, nh = (4 * q1 - 1) / DH - h0 + 1;
            const int nhdr = nh * ns;
            const int b = s / P.Hkv, g = s % P.Hkv;
            const uint64_t* src = P.attp + (int64_t)s * NW * GR;
            // Register path: partial j of the segment at lane j of a group of
            // NSP = 2^lg >= ns lanes; headers (head h0 + hh, partial j) at lane
            // hh NSP + j of the first row, values (quad q, partial j) at item
            // q NSP + j (64 per register row). Weights and each quad's sum over
            // the partials are reductions inside the aligned NSP-lane groups
            // (DPP moves and lane swaps), without LDS.
            const int lg = uni(ns) <= 1 ? 0 : 32 - __builtin_clz((uint32_t)uni(ns) - 1u);
            if (uni(ns) <= 64 && (uni(nh) << lg) <= 64 && (uni(nq) << lg) <= 64 * PU) {
                const int NSP = 1 << lg;
                auto gsum = [&](float x) {
                    if (lg > 0) x += dpp_f<0xB1>(x);   // lane ^ 1
                    if (lg > 1) x += dpp_f<0x4E>(x);   // lane ^ 2
                    if (lg > 2) x += dpp_f<0x141>(x);  // 8-lane half-row mirror
                    if (lg > 3) x += dpp_f<0x140>(x);  // 16-lane row mirror
                    if (lg > 4) x = sum_xor16(x);
                    if (lg > 5) x = sum_xor32(x);
                    return x;
                };
                auto gmax = [&](float x) {
                    if (lg > 0) x = fmaxf(x, dpp_f<0xB1>(x));
                    if (lg > 1) x = fmaxf(x, dpp_f<0x4E>(x));
                    if (lg > 2) x = fmaxf(x, dpp_f<0x141>(x));
                    if (lg > 3) x = fmaxf(x, dpp_f<0x140>(x));
                    if (lg > 4) x = max_xor16(x);
                    if (lg > 5) x = max_xor32(x);
                    return x;
                };
                const int jl = lane & (NSP - 1), hl = lane >> lg;
                const bool hv = hl < nh && jl < ns;
                v4u rh, rv[PU][2];
                while (true) {
                    rh = hv ? ld_tag2(src, (uint32_t)(jl * GR + 2 * (h0 + hl))) : (v4u){0u, tag, 0u, tag};
                    bool good = tags_ok(rh, tag);
#pragma unroll
                    for (int u = 0; u < PU; ++u) {
                        const int q = (lane + 64 * u) >> lg;
                        const uint32_t wi = (uint32_t)(jl * GR + hdr + 4 * (q0 + q));
                        const bool use = q < nq && jl < ns;
                        rv[u][0] = use ? ld_tag2(src, wi) : (v4u){0u, tag, 0u, tag};
                        rv[u][1] = use ? ld_tag2(src, wi + 2) : (v4u){0u, tag, 0u, tag};
                        good = good && tags_ok(rv[u][0], tag) && tags_ok(rv[u][1], tag);
                    }
                    if (__all(good)) break;
                    if (!(ok = retry_or_fail(P, deadline, sid))) break;
                }
                if (!ok) break;
                const float mj = hv ? __uint_as_float(rh.x) : -INFINITY;
                const float lj = hv ? __uint_as_float(rh.z) : 0.f;
                const float M = gmax(mj);
                const float ej = mj == -INFINITY ? 0.f : fast_exp2((mj - M) * kL2e);
                const float cj = ej * __builtin_amdgcn_rcpf(gsum(lj * ej));  // the sum is >= 1
                float* atl = layer_copy(P.atto, P.atto_lb, layer);
#pragma unroll
                for (int u = 0; u < PU; ++u) {
                    if (64 * u >= (uni(nq) << lg)) break;
                    const int q = (lane + 64 * u) >> lg;
                    const int hh = min(4 * (q0 + q) / DH - h0, nh - 1);
                    const float c = __shfl(cj, (hh << lg) + jl, 64);
                    v4f acc = {__uint_as_float(rv[u][0].x), __uint_as_float(rv[u][0].z), __uint_as_float(rv[u][1].x),
                               __uint_as_float(rv[u][1].z)};
                    acc = (q < nq && jl < ns) ? acc * c : (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] = gsum(acc[e]);
                    if (jl == 0 && q < nq) {
                        const int f = 4 * (q0 + q), h = f / DH, e = f % DH;
                        const uint32_t wi = (uint32_t)(b * P.Hq * DH + (g * G + h) * DH + e);
                        if constexpr (kTagOps<MFMA, MOE>) st_tag4(reinterpret_cast<uint64_t*>(atl), wi, acc, tag);
                        else st_sc1_v4(atl, wi * 4u, __builtin_bit_cast(v4u, acc));
                    }
                }
                continue;
            }
            v4u th[PU], to[PU][2];
            while (true) {
                bool good = true;
#pragma unroll
                for (int u = 0; u < PU; ++u) {
                    const int i = lane + 64 * u;
                    const int hh = udiv(i, ns), j = i - hh * ns;
                    th[u] = i < nhdr ? ld_tag2(src, (uint32_t)(j * GR + 2 * (h0 + hh))) : (v4u){0u, tag, 0u, tag};
                    good = good && tags_ok(th[u], tag);
                }
#pragma unroll
                for (int u = 0; u < PU; ++u) {
                    const int pr = lane + 64 * u;
                    const int j = udiv(pr, nq), q = pr - j * nq;
                    const uint32_t wi = (uint32_t)(j * GR + hdr + 4 * (q0 + q));
                    to[u][0] = pr < npair ? ld_tag2(src, wi) : (v4u){0u, tag, 0u, tag};
                    to[u][1] = pr < npair ? ld_tag2(src, wi + 2) : (v4u){0u, tag, 0u, tag};
                    good = good && tags_ok(to[u][0], tag) && tags_ok(to[u][1], tag);
                }
                if (__all(good)) break;
                if (!(ok = retry_or_fail(P, deadline, sid))) break;
            }
            if (!ok) break;
#pragma unroll
            for (int u = 0; u < PU; ++u) {
                const int i = lane + 64 * u;
                if (i < nhdr) {
                    mlb[2 * i] = __uint_as_float(th[u].x);
                    mlb[2 * i + 1] = __uint_as_float(th[u].z);
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            // weights c_j[h] = e^{m_j[h] - M_h} / L_h, lanes over partials j
            for (int hh = 0; hh < nh; ++hh) {
                float mj[4], lj[4];
                float M = -INFINITY;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int j = lane + 64 * u;
                    mj[u] = j < ns ? mlb[2 * (hh * ns + j)] : -INFINITY;
                    lj[u] = j < ns ? mlb[2 * (hh * ns + j) + 1] : 0.f;
                    M = fmaxf(M, mj[u]);
                }
                M = wave_max_f(M);
                float Ls = 0.f;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    mj[u] = (mj[u] == -INFINITY) ? 0.f : fast_exp2((mj[u] - M) * kL2e);
                    Ls += lj[u] * mj[u];
                }
                Ls = wave_sum_f(Ls);
                const float inv = __builtin_amdgcn_rcpf(Ls);  // Ls >= 1: the partial holding the maximum adds at least 1
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int j = lane + 64 * u;
                    if (j < ns) cbuf[hh * 256 + j] = mj[u] * inv;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): weights visible to the wave
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int u = 0; u < PU; ++u) {
                const int pr = lane + 64 * u;
                if (pr < npair) {
                    const int j = udiv(pr, nq), q = pr - j * nq;
                    const int hh = 4 * (q0 + q) / DH - h0;
                    const float c = cbuf[hh * 256 + j];
                    const v4f o = {__uint_as_float(to[u][0].x), __uint_as_float(to[u][0].z),
                                   __uint_as_float(to[u][1].x), __uint_as_float(to[u][1].z)};
                    red[pr] = o * c;
                }
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
            for (int q = lane; q < nq; q += 64) {
                v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
                for (int j = 0; j < ns; ++j) acc += red[j * nq + q];  // 8 LDS reads in flight
                const int f = 4 * (q0 + q), h = f / DH, e = f % DH;
                const uint32_t wi = (uint32_t)(b * P.Hq * DH + (g * G + h) * DH + e);
                float* atl = layer_copy(P.atto, P.atto_lb, layer);
                if constexpr (kTagOps<MFMA, MOE>) st_tag4(reinterpret_cast<uint64_t*>(atl), wi, acc, tag);
                else st_sc1_v4(atl, wi * 4u, __builtin_bit_cast(v4u, acc));
            }
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
        }
        if constexpr (!kTagOps<MFMA, MOE>) raise_flag(P, flag_array(P, layer, FK_ATT));
        trace_mark(P, sid, 6);
    } else if (MOE && kind == 6) {
        // ---- router epilogue: logits of this WG's experts
        const GemvPart gp = wg_part(lds, 6);
        for (int t = gp.t0; t < gp.t1; ++t) {
            const int task = t - gp.t0;
            for (int idx = lane; idx < 16 * kMaxBatch; idx += 64) {
                const int r = idx & 15, b = idx >> 4;
                if (b >= n || 16 * t + r >= P.E) continue;
                st_sc1_f(layer_copy(P.rlog, P.rlog_lb, layer) + b * P.E + 16 * t + r, part_sum<NB, MFMA>(lds, P.lds_part[kind], task, r, b, W) * rscale(b));
            }
        }
        raise_flag(P, flag_array(P, layer, FK_RT));
    } else if (MOE && kind == 3) {
        // ---- expert gate/up epilogue: a_u = silu(gate) * up for expert slot u
        // (every request's row; the down-projection weights unselected ones by 0)
        const GemvPart gp = wg_part(lds, 3);
        const int te = P.gu.te;
        for (int t = gp.t0; t < gp.t1; ++t) {
            const int task = t - gp.t0;
            const int u = udiv(t, te), tt = t - u * te;
            for (int idx = lane; idx < 8 * kMaxBatch; idx += 64) {
                const int r = idx & 7, b = idx >> 3;
                if (b >= n) continue;
                const float gt = part_sum<NB, MFMA>(lds, P.lds_part[kind], task, r, b, 1) * rscale(b);
                const float up = part_sum<NB, MFMA>(lds, P.lds_part[kind], task, r + 8, b, 1) * rscale(b);
                const float a = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
                st_sc1_f(layer_copy(P.act, P.act_lb, layer) + ((size_t)u * kMaxBatch + b) * P.fe + 8 * tt + r, a);
            }
        }
        raise_flag(P, flag_array(P, layer, FK_GU));
    } else if (MOE && kind == 4) {
        // ---- expert down epilogue: x[b] += w_b,u W_d^u a_u (the weight is already
        // in the operand), for the requests that selected the tile's expert
        const GemvPart gp = wg_part(lds, 4);
        const Route& RT = *reinterpret_cast<const Route*>(lds + P.lds_route);
        const int te = P.dn.te, uf = RT.uf;
        for (int t = gp.t0; t < gp.t1; ++t) {
            const int task = t - gp.t0;
            const int u = udiv(t, te), tt = t - u * te;
            for (int idx = lane; idx < 16 * kMaxBatch; idx += 64) {
                const int r = idx & 15, b = idx >> 4;
                if (b >= n || RT.wu[u - uf][b] == 0.f) continue;
                const float y = part_sum<NB, MFMA>(lds, P.lds_part[kind], task, r, b, 1);
                __hip_atomic_fetch_add(layer_copy(P.xparts, P.x_lb, layer + 1) + b * P.d + 16 * tt + r, y, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        raise_flag(P, flag_array(P, layer, FK_DN));
    } else if (kind == 2 || kind == 4) {
        // ---- O / DN epilogue: part s = W[:, Ks] a (+ the residual for s = 0)
        const GemvPart gp = wg_part(lds, kind);
        float* dst = kind == 2 ? layer_copy(P.hparts, P.h_lb, layer) : layer_copy(P.xparts, P.x_lb, layer + 1);
        for (int t = gp.t0; t < gp.t1; ++t) {
            const int task = t - gp.t0;
            for (int idx = lane; idx < 16 * kMaxBatch; idx += 64) {
                const int r = idx & 15, b = idx >> 4;
                if (b >= n) continue;
                float y = part_sum<NB, MFMA>(lds, P.lds_part[kind], task, r, b, W) * row_scale<FP8>(P, lds, task, r);
                if (gp.s == 0) y += res[(task * kMaxBatch + b) * 16 + r];
                const uint32_t wi = (uint32_t)((gp.s * kMaxBatch + b) * P.d + 16 * t + r);
                if constexpr (kTagOps<MFMA, MOE>) st_tag_f(reinterpret_cast<uint64_t*>(dst), wi, y, tag);
                else st_sc1_f(dst + wi, y);
            }
        }
        if constexpr (!kTagOps<MFMA, MOE>) raise_flag(P, flag_array(P, layer, kind == 2 ? FK_O : FK_DN));
    } else if (kind == 3) {
        // ---- GU epilogue: a = silu(gate) * up, one lane per (tile, row pair, request)
        const GemvPart gp = wg_part(lds, 3);
        const int items = (gp.t1 - gp.t0) * 8 * n;
        {
            for (int idx = lane; idx < items; idx += 64) {
                const int r = idx & 7, q = idx >> 3;
                const int task = udiv(q, n), b = q - task * n, t = gp.t0 + task;
                const float gt = part_sum<NB, MFMA>(lds, P.lds_part[kind], task, r, b, W) * row_scale<FP8>(P, lds, task, r) * rscale(b);
                const float up = part_sum<NB, MFMA>(lds, P.lds_part[kind], task, r + 8, b, W) *
                                 row_scale<FP8>(P, lds, task, r + 8) * rscale(b);
                const float a = gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up;
                const uint32_t wi = (uint32_t)(b * P.F + 8 * t + r);
                float* acl = layer_copy(P.act, P.act_lb, layer);
                if constexpr (kTagOps<MFMA, MOE>) st_tag_f(reinterpret_cast<uint64_t*>(acl), wi, a, tag);
                else st_sc1_f(acl + wi, a);
            }
        }
        if constexpr (!kTagOps<MFMA, MOE>) raise_flag(P, flag_array(P, layer, FK_GU));
    } else {
        // ---- LM epilogue: logits, per-WG sampler partial, then WG 0 reduces.
        // lane = row (lane & 15) and batches (lane >> 4) + 4k; at batch 1 the four
        // 16-lane groups take four tiles at a time instead.
        GemvPart gp = wg_part(lds, 5);
        const int r = lane & 15;
        constexpr int TPP = NB == 1 ? 4 : 1;  // tiles per pass
        constexpr int KB = NB == 1 ? 1 : 2;   // batch groups per lane
        float best[2] = {-INFINITY, -INFINITY};
        int bidx[2] = {0x7fffffff, 0x7fffffff};
        uint64_t gkey[KB];  // the Gumbel noise key of each batch group's request (fixed per lane)
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int b = NB == 1 ? 0 : (lane >> 4) + 4 * k;
            gkey[k] = splitmix64(splitmix64(splitmix64(P.seed) + P.step) + (uint64_t)b);
        }
        for (int tp = gp.t0; tp < gp.t1; tp += TPP) {
            const int t = tp + (TPP > 1 ? (lane >> 4) : 0);
            const int task = t - gp.t0;
            const int row = 16 * t + r;
#pragma unroll
            for (int k = 0; k < KB; ++k) {
                const int b = NB == 1 ? 0 : (lane >> 4) + 4 * k;
                if (t >= gp.t1 || b >= n || row >= P.V) continue;
                const float y = part_sum<NB, MFMA>(lds, P.lds_part[kind], task, r, b, P.lm.tpw ? 1 : W) *
                                row_scale<FP8>(P, lds, task, r) * rscale(b);
                if (P.logits_out) P.logits_out[(int64_t)b * P.V + row] = y;
                float sc = y;
                const float T = C.temp[b];
                if (T > 0.f) {
                    const uint64_t hh = splitmix64(gkey[k] + (uint64_t)row);
                    const float u = (float)(2u * (uint32_t)(hh >> 41) + 1u) * (1.0f / 16777216.0f);
                    sc = y / T - __logf(-__logf(u));
                }
                if (sc > best[k] || (sc == best[k] && row < bidx[k])) { best[k] = sc; bidx[k] = row; }
            }
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            float sc = best[k];
            int ix = bidx[k];
            for (int msk = 1; msk < 16 * TPP; msk <<= 1) {  // within the lanes of one batch
                const float s2 = __shfl_xor(sc, msk, 64);
                const int i2 = __shfl_xor(ix, msk, 64);
                if (s2 > sc || (s2 == sc && i2 < ix)) { sc = s2; ix = i2; }
            }
            const int b = NB == 1 ? 0 : (lane >> 4) + 4 * k;
            if ((NB == 1 ? lane == 0 : r == 0) && b < n) {
                st_sc1_f(P.lmpart + ((int64_t)w * kMaxBatch + b) * 2, sc);
                st_sc1_i(reinterpret_cast<int32_t*>(P.lmpart) + ((int64_t)w * kMaxBatch + b) * 2 + 1, ix);
            }
        }
        // Requests sampling among their top-k logits: this WG's k largest logits
        // (equal logits by index), largest first, for workgroup 0 to merge.
        for (int b = 0; b < n; ++b) {
            const int k = C.topk[b];
            if (k == 0 || !(C.temp[b] > 0.f)) continue;
            const int nv = (gp.t1 - gp.t0) * 16;  // this WG's rows (at most 64 kTopKLane, checked on the host)
            float val[kTopKLane];
#pragma unroll
            for (int u = 0; u < kTopKLane; ++u) {
                const int j = lane + 64 * u;
                val[u] = (j < nv && 16 * gp.t0 + j < P.V)
                             ? part_sum<NB, MFMA>(lds, P.lds_part[kind], j >> 4, j & 15, b, P.lm.tpw ? 1 : W) *
                                   row_scale<FP8>(P, lds, j >> 4, j & 15) * rscale(b)
                             : -INFINITY;
            }
            for (int r = 0; r < k; ++r) {
                float bv = -INFINITY;
                int bj = 0x7fffffff;
#pragma unroll
                for (int u = 0; u < kTopKLane; ++u)
                    if (val[u] > bv) { bv = val[u]; bj = lane + 64 * u; }
                for (int msk = 1; msk < 64; msk <<= 1) {
                    const float v2 = __shfl_xor(bv, msk, 64);
                    const int j2 = __shfl_xor(bj, msk, 64);
                    if (v2 > bv || (v2 == bv && j2 < bj)) { bv = v2; bj = j2; }
                }
#pragma unroll
                for (int u = 0; u < kTopKLane; ++u)
                    if (lane + 64 * u == bj) val[u] = -INFINITY;
                if (lane == 0) {
                    float* o = P.lmtopk + (((int64_t)w * kMaxBatch + b) * kMaxSampleTopK + r) * 2;
                    st_sc1_f(o, bv);
                    st_sc1_i(reinterpret_cast<int32_t*>(o) + 1, bj == 0x7fffffff ? -1 : 16 * gp.t0 + bj);
                }
            }
        }
        raise_flag(P, flag_lm(P));
        trace_mark(P, sid, 2);
        if (w == 0) {
            ok = wait_flags(P, flag_lm(P), 0, NW, sid);
            const uint32_t badm = ld_sc1_u(bad_mask(P, 0));
            for (int b = 0; b < n; ++b) {
                float sc = -INFINITY;
                int ix = 0x7fffffff;
                const int k = C.topk[b];
                if (k > 0 && C.temp[b] > 0.f) {
                    // k-way merge of the NW lists (each largest first): the global k
                    // largest logits, then the Gumbel-max among them. The lists go
                    // to LDS first (the DMA rings are idle once the streams ended);
                    // lane l owns lists l, l + 64, ...
                    float* scr = reinterpret_cast<float*>(lds + P.lds_ring);
                    const int tot = NW * k;
                    for (int e0 = 0; e0 < tot; e0 += 64 * 8) {
                        float tv[8];
                        int ti[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const int e = e0 + 64 * u + lane;
                            const int list = e / k, ent = e - list * k;
                            const int64_t o = (((int64_t)list * kMaxBatch + b) * kMaxSampleTopK + ent) * 2;
                            tv[u] = e < tot ? ldc_f(P.lmtopk, o) : -INFINITY;
                            ti[u] = e < tot ? ldc_i(reinterpret_cast<const int32_t*>(P.lmtopk), o + 1) : -1;
                        }
#pragma unroll
                        for (int u = 0; u < 8; ++u) {
                            const int e = e0 + 64 * u + lane;
                            if (e < tot) {
                                scr[2 * e] = tv[u];
                                scr[2 * e + 1] = __int_as_float(ti[u]);
                            }
                        }
                    }
                    __builtin_amdgcn_s_waitcnt(0xc07f);
                    __builtin_amdgcn_wave_barrier();
                    int pos[kMaxNW / 64];
#pragma unroll
                    for (int q = 0; q < kMaxNW / 64; ++q) pos[q] = 0;
                    const float T = C.temp[b];
                    const uint64_t key = splitmix64(splitmix64(splitmix64(P.seed) + P.step) + (uint64_t)b);
                    for (int r = 0; r < k; ++r) {
                        float hv = -INFINITY;
                        int hi = 0x7fffffff, hq = -1;
#pragma unroll
                        for (int q = 0; q < kMaxNW / 64; ++q) {
                            const int list = lane + 64 * q;
                            if (list < NW && pos[q] < k) {
                                const float v = scr[2 * (list * k + pos[q])];
                                const int i = __float_as_int(scr[2 * (list * k + pos[q]) + 1]);
                                if (i >= 0 && (v > hv || (v == hv && i < hi))) { hv = v; hi = i; hq = q; }
                            }
                        }
                        float gv = hv;
                        int gi = hi;
                        for (int msk = 1; msk < 64; msk <<= 1) {
                            const float v2 = __shfl_xor(gv, msk, 64);
                            const int i2 = __shfl_xor(gi, msk, 64);
                            if (v2 > gv || (v2 == gv && i2 < gi)) { gv = v2; gi = i2; }
                        }
                        if (gi == 0x7fffffff) break;  // fewer than k rows in all
#pragma unroll
                        for (int q = 0; q < kMaxNW / 64; ++q)
                            if (q == hq && hi == gi) ++pos[q];  // indices are unique: one lane advances
                        const uint64_t hh = splitmix64(key + (uint64_t)gi);
                        const float uu = (float)(2u * (uint32_t)(hh >> 41) + 1u) * (1.0f / 16777216.0f);
                        const float g = gv / T - __logf(-__logf(uu));
                        if (g > sc || (g == sc && gi < ix)) { sc = g; ix = gi; }
                    }
                } else {
                for (int w0 = 0; w0 < NW; w0 += 64) {
                    const int ww = w0 + lane;
                    if (ww < NW) {
                        const float s2 = ldc_f(P.lmpart, ((int64_t)ww * kMaxBatch + b) * 2);
                        const int i2 = ldc_i(reinterpret_cast<const int32_t*>(P.lmpart), ((int64_t)ww * kMaxBatch + b) * 2 + 1);
                        if (s2 > sc || (s2 == sc && i2 < ix)) { sc = s2; ix = i2; }
                    }
                }
                for (int msk = 1; msk < 64; msk <<= 1) {
                    const float s2 = __shfl_xor(sc, msk, 64);
                    const int i2 = __shfl_xor(ix, msk, 64);
                    if (s2 > sc || (s2 == sc && i2 < ix)) { sc = s2; ix = i2; }
                }
                }
                if (lane == 0) {
                    const bool good = ok && ((C.valid >> b) & 1) && !((badm >> b) & 1) && ix >= 0 && ix < P.V;
                    P.tokens_out[b] = good ? ix : -1;
                    if (!((C.valid >> b) & 1)) latch_error(P, 5u, (uint32_t)b);
                }
            }
        }
    }
    // the stage's outputs are published (their flag store issued): see compute_role
    if constexpr (!kTagOps<MFMA, MOE>)
        if (lane == 0) *(volatile int32_t*)&C.pubs = sid + 1;
    if (kind != 1) trace_mark(P, sid, 2);
    // ============================ inputs of the next stage
    if (kind != 5) {
        if (ok && kind != 0 && !kTagOps<MFMA, MOE>) {
            // GEMV operands: the compute waves load them once the producers' flags are up
            const int wk = kind == 1 ? FK_ATT : kind == 2 ? FK_O : kind == 3 ? FK_GU : kind == 6 ? FK_RT : FK_DN;
            ok = wait_flags(P, flag_array(P, layer, wk), 0, NW, sid);
            if (MOE && ok && kind == 6) io_route(P, lds, layer);  // the expert stages' tiles
        }
        trace_mark(P, sid, 3);
        if (ok && kind == 0) {
            // q and k~/v~ of each compute wave's segment, polled until current (once
            // per distinct segment: consecutive waves often share one)
            const int tab = att_table(lds, layer);
            const float scale = 1.4426950408889634f / sqrtf((float)DH);  // log2 e / sqrt(dh)
            constexpr int QL = (G * DH + 127) / 128;  // 16-byte loads per lane for q (2 words each)
            constexpr int KL = (2 * DH + 127) / 128;  // ... for k~ and v~
            const uint64_t deadline = rt_clock() + P.wait_ticks;
            for (int vv = 0; vv < W && ok;) {
                const int seg = C.wseg[tab][vv];
                int ve = vv + 1;
                while (ve < W && C.wseg[tab][ve] == seg) ++ve;
                if (seg < 0) {
                    vv = ve;
                    continue;
                }
                const int b = seg / P.Hkv, g = seg % P.Hkv;
                v4u tq[QL], tk[KL];
                while (true) {
                    bool good = true;
#pragma unroll
                    for (int u = 0; u < QL; ++u) {
                        const int e = lane * 2 + u * 128;
                        tq[u] = e < G * DH ? ld_tag2(P.q, (uint32_t)(b * P.Hq * DH + g * G * DH + e)) : (v4u){0u, tag, 0u, tag};
                        good = good && tags_ok(tq[u], tag);
                    }
#pragma unroll
                    for (int u = 0; u < KL; ++u) {
                        const int e = lane * 2 + u * 128;
                        tk[u] = e < 2 * DH ? ld_tag2(P.kvcur, (uint32_t)((b * P.Hkv + g) * 2 * DH + e)) : (v4u){0u, tag, 0u, tag};
                        good = good && tags_ok(tk[u], tag);
                    }
                    if (__all(good)) break;
                    if (!(ok = retry_or_fail(P, deadline, sid))) break;
                }
                if (!ok) break;
                // q times log2 e / sqrt(dh) as the hi and lo bf16 halves of each
                // value, [head][hi, lo][dh]: the attention's matrix-core operand
                // rows as they are read, split once here instead of in every wave
                uint32_t qhp[QL], qlp[QL];
#pragma unroll
                for (int u = 0; u < QL; ++u) {
                    const float x0 = __uint_as_float(tq[u].x) * scale, x1 = __uint_as_float(tq[u].z) * scale;
                    qhp[u] = cvt_bf16x2(x0, x1);
                    qlp[u] = cvt_bf16x2(x0 - bf_lo(qhp[u]), x1 - bf_hi(qhp[u]));
                }
                for (int w2 = vv; w2 < ve; ++w2) {
                    uint16_t* qh = reinterpret_cast<uint16_t*>(lds + P.lds_op) + (size_t)w2 * G * DH * 2;
                    uint16_t* kvs = reinterpret_cast<uint16_t*>(lds + P.lds_op + W * G * DH * 4) + (size_t)w2 * 2 * DH;
#pragma unroll
                    for (int u = 0; u < QL; ++u) {
                        const int e = lane * 2 + u * 128;
                        if (e < G * DH) {
                            const int h = e / DH, d = e - h * DH;
                            *reinterpret_cast<uint32_t*>(qh + (2 * h) * DH + d) = qhp[u];
                            *reinterpret_cast<uint32_t*>(qh + (2 * h + 1) * DH + d) = qlp[u];
                        }
                    }
#pragma unroll
                    for (int u = 0; u < KL; ++u) {
                        const int e = lane * 2 + u * 128;
                        if (e < 2 * DH) *reinterpret_cast<uint32_t*>(kvs + e) = (tk[u].x & 0xFFFFu) | (tk[u].z << 16);
                    }
                }
                vv = ve;
            }
        }
    }
    trace_mark(P, sid, 4);
    if (!ok && lane == 0) C.abort = 1;
}

// Compute wave v of W: its slice (k in [v Kop/W, (v+1) Kop/W)) of the GEMV
// operand of a stage, x[b][k] = sum over `nparts` parts of src[part][b][k0 + k]
// (zero rows for b >= n), times the gains when `gains` is set, written straight
// into the final LDS layout (store_operand8). Returns this wave's per-row sum of
// squares of x (before the gains) for the RMSNorm scale. Plain loads: the
// producers' flags were seen before B_in. They are vector-memory loads issued
// after the wave's ring DMAs, so waiting for them never leaves a DMA unaccounted.
template <int NB, bool MFMA, int NP, int W, bool CACHED>
__device__ __forceinline__ void load_operand_slice_np(const Params& P, uint8_t* lds, const float* src, int pstride,
                                                        int rstride, int k0, int Kop, int v, int n,
                                                        const uint16_t* gains, float (&ss)[MFMA ? 8 : NB],
                                                        const float* rowscale, int kb_out0) {
    constexpr int NBo = MFMA ? 8 : NB;
    // items per lane per round trip: 16-32 loads in flight (half with eight
    // waves, each of which loads half as much)
    constexpr int U = (NP == 1 ? 8 : 4) / (W == 8 ? 2 : 1);
    const int lane = lane_id();
    uint8_t* op = lds + P.lds_op;
    const int G8 = Kop / (8 * W);    // 8-value groups per row in this wave's slice
    const int kq0 = v * (Kop / W);
    const int total = NBo * G8;
#pragma unroll
    for (int b = 0; b < NBo; ++b) ss[b] = 0.f;
    for (int base = 0; base < total; base += 64 * U) {
        v4f t[NP][U][2];
        int bb[U], kk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * 64 + lane;
            const int b = udiv(j, G8), k = kq0 + 8 * (j - b * G8);
            const bool live = j < total && b < n;
            bb[u] = j < total ? b : -1;
            kk[u] = k;
#pragma unroll
            for (int sp = 0; sp < NP; ++sp) {
                const int64_t off = (int64_t)sp * pstride + (int64_t)b * rstride + k0 + k;
                t[sp][u][0] = live ? (CACHED ? ldk_v4f(src, off) : ldc_v4f(src, off)) : (v4f){0.f, 0.f, 0.f, 0.f};
                t[sp][u][1] = live ? (CACHED ? ldk_v4f(src, off + 4) : ldc_v4f(src, off + 4)) : (v4f){0.f, 0.f, 0.f, 0.f};
            }
        }
        // branch-free per item (selects, not branches; only the LDS store is
        // masked): items past the end (bb < 0) carry zeros
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v4f x0 = t[0][u][0], x1 = t[0][u][1];
#pragma unroll
            for (int sp = 1; sp < NP; ++sp) {
                x0 += t[sp][u][0];
                x1 += t[sp][u][1];
            }
            float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            float q = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) q += x[e] * x[e];
#pragma unroll
            for (int b = 0; b < NBo; ++b) ss[b] += b == bb[u] ? q : 0.f;
            if (gains) {
                const v4u g = *reinterpret_cast<const v4u*>(gains + kk[u]);
                const float gf[8] = {bf_lo(g.x), bf_hi(g.x), bf_lo(g.y), bf_hi(g.y),
                                     bf_lo(g.z), bf_hi(g.z), bf_lo(g.w), bf_hi(g.w)};
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] *= gf[e];
            }
            if (rowscale) {
                const float rsb = rowscale[max(bb[u], 0)];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] *= rsb;
            }
            if (bb[u] >= 0) store_operand8<NB, MFMA>(op, kb_out0 + kk[u] / 32, bb[u], (kk[u] % 32) / 8, x);
        }
    }
#pragma unroll
    for (int b = 0; b < NBo; ++b) ss[b] = wave_sum_f(ss[b]);
}

// Dispatch on the number of parts: 1, 2 or 4 (K-splits double from 1 up to kMaxSplit).
// CACHED: loads through L1/L2 (ldk_*), else agent-coherent loads (ldc_*).
template <int NB, bool MFMA, int W, bool CACHED>
__device__ __forceinline__ void load_operand_slice(const Params& P, uint8_t* lds, const float* src, int nparts,
                                                     int pstride, int rstride, int k0, int Kop, int v, int n,
                                                     const uint16_t* gains, float (&ss)[MFMA ? 8 : NB],
                                                     const float* rowscale = nullptr, int kb_out0 = 0) {
    if (nparts == 1)
        load_operand_slice_np<NB, MFMA, 1, W, CACHED>(P, lds, src, pstride, rstride, k0, Kop, v, n, gains, ss, rowscale, kb_out0);
    else if (nparts == 2)
        load_operand_slice_np<NB, MFMA, 2, W, CACHED>(P, lds, src, pstride, rstride, k0, Kop, v, n, gains, ss, rowscale, kb_out0);
    else
        load_operand_slice_np<NB, MFMA, 4, W, CACHED>(P, lds, src, pstride, rstride, k0, Kop, v, n, gains, ss, rowscale, kb_out0);
}

// As load_operand_slice, from tagged words (value, tag) that the producers
// publish without a flag: the wave's loads are reissued until every word it
// needs carries the producing stage's tag. Returns false (and latches a
// timeout) once the wait limit passes. Lanes hold U items of 8 values.
template <int NB, bool MFMA, int W>
__device__ __forceinline__ bool load_operand_slice_tagged(const Params& P, uint8_t* lds, const uint64_t* src,
                                                            int nparts, int pstride, int rstride, int k0, int Kop,
                                                            int v, int n, const uint16_t* gains,
                                                            float (&ss)[MFMA ? 8 : NB], uint32_t tag, uint32_t where) {
    constexpr int NBo = MFMA ? 8 : NB;
    constexpr int U = W == 8 ? 1 : 2;
    const int lane = lane_id();
    uint8_t* op = lds + P.lds_op;
    const int G8 = Kop / (8 * W);    // 8-value groups per row in this wave's slice
    const int kq0 = v * (Kop / W);
    const int total = NBo * G8;
    // rows of invalid requests are not polled: no producer publishes all of them
    // (their attention outputs are never merged); they load as zeros
    const int valid = uni(ctrl(lds).valid);
    const uint64_t deadline = rt_clock() + P.wait_ticks;
#pragma unroll
    for (int b = 0; b < NBo; ++b) ss[b] = 0.f;
    for (int base = 0; base < total; base += 64 * U) {
        int bb[U], kk[U];
        bool live[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * 64 + lane;
            const int b = udiv(j, G8);
            kk[u] = kq0 + 8 * (j - b * G8);
            bb[u] = j < total ? b : -1;
            live[u] = j < total && b < n && ((valid >> b) & 1);
        }
        v4u t[kMaxSplit][U][4];
        while (true) {
            bool good = true;
#pragma unroll
            for (int sp = 0; sp < kMaxSplit; ++sp)
#pragma unroll
                for (int u = 0; u < U; ++u)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const bool use = live[u] && sp < nparts;
                        const uint32_t wi = (uint32_t)(sp * pstride + bb[u] * rstride + k0 + kk[u] + 2 * q);
                        t[sp][u][q] = use ? ld_tag2(src, wi) : (v4u){0u, tag, 0u, tag};
                        good = good && tags_ok(t[sp][u][q], tag);
                    }
            if (__all(good)) break;
            if (rt_clock() > deadline) {
                if (lane == 0) latch_error(P, 6u, where);
                return false;
            }
            __builtin_amdgcn_s_sleep(1);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float a = 0.f, c = 0.f;
#pragma unroll
                for (int sp = 0; sp < kMaxSplit; ++sp) {
                    a += __uint_as_float(t[sp][u][q].x);
                    c += __uint_as_float(t[sp][u][q].z);
                }
                x[2 * q] = a;
                x[2 * q + 1] = c;
            }
            float qq = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) qq += x[e] * x[e];
#pragma unroll
            for (int b = 0; b < NBo; ++b) ss[b] += b == bb[u] ? qq : 0.f;
            if (gains) {
                const v4u g = *reinterpret_cast<const v4u*>(gains + kk[u]);
                const float gf[8] = {bf_lo(g.x), bf_hi(g.x), bf_lo(g.y), bf_hi(g.y),
                                     bf_lo(g.z), bf_hi(g.z), bf_lo(g.w), bf_hi(g.w)};
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] *= gf[e];
            }
            if (bb[u] >= 0) store_operand8<NB, MFMA>(op, kk[u] / 32, bb[u], (kk[u] % 32) / 8, x);
        }
    }
#pragma unroll
    for (int b = 0; b < NBo; ++b) ss[b] = wave_sum_f(ss[b]);
    return true;
}

// Compute wave v, after the attention stage: its slice of this WG's partial of
// each segment the WG serves, from the wave records in LDS (the waves of the
// segment that had pages; a WG whose waves are all empty writes a null partial,
// m = -inf and l = 0). Global record: header words 2h, 2h + 1 = (m_h, l_h), then
// G x DH values unnormalised against m_h. Wave v writes value quads
// [v QW, (v + 1) QW) and the headers of heads v, v + W, ... The segment merge
// polls the tags, so no local hand-over to the I/O wave is needed.
template <int DH, int G, int W>
__device__ __forceinline__ void att_wg_merge(const Params& P, uint8_t* lds, int layer, uint32_t tag, int v) {
    const Ctrl& C = ctrl(lds);
    const int lane = lane_id();
    const int w = blockIdx.x, NW = P.NW;
    const int tab = att_table(lds, layer);
    const int RS = 16 + G * DH;                    // LDS wave record (floats)
    constexpr int hdr = att_hdr_words(G);
    const int GR = hdr + G * DH;                   // global record (words)
    constexpr int QW = G * DH / (4 * W);           // value quads per wave
    static_assert(QW >= 1 && QW <= 64 && G * DH % (4 * W) == 0, "merge slices");
    const float* rec = reinterpret_cast<const float*>(lds + P.lds_part[1]);
    constexpr float kL2e = 1.4426950408889634f;
    int wsg[W], wn[W];
#pragma unroll
    for (int x = 0; x < W; ++x) {
        wsg[x] = uni(C.wseg[tab][x]);
        wn[x] = uni(C.wnu[tab][x]);
    }
    for (int vv = 0; vv < W;) {
        const int seg = wsg[vv];
        int ve = vv + 1;
        while (ve < W && wsg[ve] == seg) ++ve;
        if (seg >= 0) {
            const int wf0 = uni(C.segw[tab][seg]);
            uint64_t* dst = P.attp + ((int64_t)seg * NW + (w - wf0 / W)) * GR;
            bool inw[W];
#pragma unroll
            for (int x = 0; x < W; ++x) inw[x] = x >= vv && x < ve && wn[x] > 0;
            // head h's running max M over the segment's waves, their weights
            // 2^((m_x - M) log2 e) and the weighted sum of their l
            auto weights = [&](int h, float (&cw)[W], float& M, float& Ls) {
                float mv[W], lv[W];
#pragma unroll
                for (int x = 0; x < W; ++x) {
                    mv[x] = rec[x * RS + h];
                    lv[x] = rec[x * RS + 8 + h];
                }
                M = -INFINITY;
#pragma unroll
                for (int x = 0; x < W; ++x)
                    if (inw[x]) M = fmaxf(M, mv[x]);
                Ls = 0.f;
#pragma unroll
                for (int x = 0; x < W; ++x) {
                    const bool use = inw[x] && mv[x] != -INFINITY;
                    cw[x] = use ? fast_exp2((mv[x] - M) * kL2e) : 0.f;
                    Ls += use ? lv[x] * cw[x] : 0.f;
                }
            };
            if (lane < QW) {
                const int e0 = 4 * (v * QW + lane);  // value index in [0, G DH)
                float cw[W], M, Ls;
                weights(e0 / DH, cw, M, Ls);
                v4f ov[W];
#pragma unroll
                for (int x = 0; x < W; ++x) ov[x] = *reinterpret_cast<const v4f*>(rec + x * RS + 16 + e0);
                v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int x = 0; x < W; ++x)
                    if (cw[x] != 0.f) acc += ov[x] * cw[x];
                st_tag4(dst, (uint32_t)(hdr + e0), acc, tag);
            }
            for (int h = v; h < G; h += W) {
                float cw[W], M, Ls;
                weights(h, cw, M, Ls);
                if (lane == 0) st_sc1_v4(dst, (uint32_t)(2 * h) * 8u, (v4u){__float_as_uint(M), tag, __float_as_uint(Ls), tag});
            }
        }
        vv = ve;
    }
}

// Compute waves (0 .. W-1): stream their share of every stage through the LDS ring.
template <int NB, bool MFMA, int DH, int G, int R, bool MOE, int W, bool FP8>
__device__ __forceinline__ void compute_role(KParams PK, uint8_t* lds, int v) {
    Ctrl& C = ctrl(lds);
    Stream<R> S;
    int n_stages;
    {
        const Params& P = *(const Params*)launder(PK);
        S.ring = (lds_u8*)(lds + P.lds_ring + (size_t)v * R * KB);
        S.issued = S.consumed = 0;
        S.att_ok = 0;
        S.isid = -1;
        S.ic = S.in = 0;
        S.ikind = 0;
        S.qp = gemv_part(P.qkv, blockIdx.x, P.NW);
        n_stages = kSPL<MOE> * P.L + 1;
    }
    stream_refill<R, DH, MOE, W>(S, PK, lds, v);  // the attention tables are not final yet: stops there
    int opsyncs = 0;  // operand hand-overs this wave took part in
    for (int sid = 0; sid < n_stages; ++sid) {
        const Params& P = *(const Params*)launder(PK);
        const int layer = stage_layer<MOE>(P, sid), kind = stage_kind<MOE>(P, sid);
        lds_barrier();  // B_in: inputs of this stage are in LDS
        if (uni(C.abort)) {
            wait_vm<0>();  // no DMA may still be writing this workgroup's LDS
            return;
        }
        S.att_ok = 1;
        // Advance the issue cursor at every stage, also in waves with no tiles
        // here: it must enter a layer's expert stages while that layer's routing
        // and partitions are in LDS (the next router stage replaces them), and it
        // starts the prefetch of later stages early.
        if (MOE) stream_refill<R, DH, MOE, W>(S, PK, lds, v);
        if (P.trace && v == 0 && lane_id() == 0) C.tdata[0] = rt_clock();
        const bool normed = kind == 0 || kind == 3 || kind == 5 || kind == 6;
        constexpr int NBo = MFMA ? 8 : NB;
        float ss[NBo];
        if (kind == 1 || sid == 0 || (MOE && kind == SK_GU)) {
            // attention (its inputs come from the I/O wave), layer 0 QKV (the
            // embedding rows, prologue), MoE expert gate/up (the router's
            // operand, the same normalised h, is still in LDS)
        } else if (MOE && kind == SK_DN) {
            // expert down-projection: per expert slot of this WG's tiles, the
            // expert's activations times each request's routing weight
            const Route& RT = *reinterpret_cast<const Route*>(lds + P.lds_route);
            const GemvPart gp = wg_part(lds, SK_DN);
            if (gp.t1 > gp.t0) {
                const int uf = uni(RT.uf), ul = udiv(gp.t1 - 1, P.dn.te);
                for (int u = uf; u <= ul; ++u)
                    load_operand_slice<NB, MFMA, W, true>(P, lds, layer_copy(P.act, P.act_lb, layer) + (size_t)u * kMaxBatch * P.fe,
                                                          1, 0, P.fe, 0, P.fe, v, P.n, nullptr, ss, RT.wu[u - uf],
                                                          (u - uf) * (P.fe / 32));
                // Each wave wrote a K-slice, but whole-tile mode reads all of K:
                // wait until every compute wave's slice is in LDS (the I/O wave
                // takes no part, so no s_barrier).
                __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done
                ++opsyncs;
                if (lane_id() == 0)
                    __hip_atomic_fetch_add(&C.opsync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                while (*(volatile int32_t*)&C.opsync < opsyncs * W) __builtin_amdgcn_s_sleep(0);
            }
        } else {
            // this wave's slice of the operand, then the norm scales from all W
            const GemvStage& st = stage_of(P, kind);
            const float* src;
            int nparts = 1, pstride = 0, rstride = P.d, k0 = 0;
            if (kind == 2) {
                src = layer_copy(P.atto, P.atto_lb, layer);
                rstride = P.Hq * P.dh;
                k0 = wg_part(lds, 2).s * (st.K / st.S);
            } else if (kind == 4) {
                src = layer_copy(P.act, P.act_lb, layer);
                rstride = P.F;
                k0 = wg_part(lds, 4).s * (st.K / st.S);
            } else {
                const bool from_h = kind == 3 || kind == 6;  // FFN / router input: h, else x
                src = from_h ? layer_copy(P.hparts, P.h_lb, layer) : layer_copy(P.xparts, P.x_lb, layer);
                nparts = from_h ? P.o.S : P.xn;
                pstride = kMaxBatch * P.d;
            }
            const uint16_t* gains = normed ? reinterpret_cast<const uint16_t*>(lds + P.lds_gain) : nullptr;
            if constexpr (kTagOps<MFMA, MOE>) {
                // the producing stage is the one before (tags of its words)
                if (!load_operand_slice_tagged<NB, MFMA, W>(P, lds, reinterpret_cast<const uint64_t*>(src), nparts, pstride,
                                                           rstride, k0, st.K / st.S, v, P.n, gains, ss,
                                                           stage_tag(P, sid - 1), (uint32_t)sid))
                    C.abort = 1;  // seen by every wave at the next stage boundary
            } else {
                if (MOE && (kind == 0 || kind == 5))  // MoE x: summed by atomics, read coherently
                    load_operand_slice<NB, MFMA, W, false>(P, lds, src, nparts, pstride, rstride, k0, st.K / st.S, v, P.n, gains, ss);
                else
                    load_operand_slice<NB, MFMA, W, true>(P, lds, src, nparts, pstride, rstride, k0, st.K / st.S, v, P.n, gains, ss);
            }
            if (normed && lane_id() == 0) {
#pragma unroll
                for (int b = 0; b < NBo; ++b) C.ssw[v][b] = ss[b];  // the epilogue forms the RMSNorm scale
            }
            if (st.tpw) {
                // whole-tile mode reads all of K: wait until every compute wave's
                // slice of the operand is in LDS (LDS arrival counter; the I/O wave
                // takes no part, so no s_barrier)
                __builtin_amdgcn_s_waitcnt(0xC07F);
                ++opsyncs;
                if (lane_id() == 0)
                    __hip_atomic_fetch_add(&C.opsync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                while (*(volatile int32_t*)&C.opsync < opsyncs * W) __builtin_amdgcn_s_sleep(0);
            }
        }
        if (P.trace && v == 0 && lane_id() == 0) C.tdata[5] = rt_clock();
        if (kind == 1) {
            att_consume<DH, G, R, MOE, W>(P, PK, lds, S, layer, v);
        } else {
            const GemvStage& st = stage_of(P, kind);
            gemv_consume<NB, MFMA, R, DH, MOE, W, FP8>(P, PK, lds, S, st, kind, v, P.lds_part[kind]);
        }
        lds_barrier();  // B_out: partials of this stage are in LDS
        if (kind == 1) {
            att_wg_merge<DH, G, W>(P, lds, layer, stage_tag(P, sid), v);
        } else if constexpr (!kTagOps<MFMA, MOE>) {
            // Flag-published GEMV outputs: the I/O wave's stores, the wait for their
            // completion and the flag store go ahead of this workgroup's refill burst
            // in the CU's vector-memory queue (behind it they reach the consumers
            // later); where outputs are tagged words polled directly, refilling at
            // once was faster.
            while (*(volatile int32_t*)&C.pubs <= sid) __builtin_amdgcn_s_sleep(1);
        }
        // Refill the slots of the stage's last chunks now, while the I/O wave runs
        // the epilogue and the next operand is in transit: a DMA burst blocks the
        // issuing wave for a while, which at the next stage's first group would
        // delay the compute that follows the operand.
        stream_refill<R, DH, MOE, W>(S, PK, lds, v);
    }
}

// I/O wave (W): prologue, then after each stage its epilogue and the next
// stage's inputs.
template <int NB, bool MFMA, int DH, int G, bool MOE, int W, bool FP8>
__device__ __forceinline__ void io_role(KParams PK, uint8_t* lds) {
    Ctrl& C = ctrl(lds);
    io_prologue<NB, MFMA, DH, G, MOE, W>(PK, lds);
    const int n_stages = kSPL<MOE> * ((const Params*)launder(PK))->L + 1;
    for (int sid = 0; sid < n_stages; ++sid) {
        const Params& P = *(const Params*)launder(PK);
        __syncthreads();  // B_in
        if (C.abort) return;
        const uint64_t t0 = P.trace ? rt_clock() : 0;  // (kept: reading the trace word back could race its store)
        if (P.trace && lane_id() == 0) P.trace[((size_t)blockIdx.x * (P.spl * P.L + 1) + sid) * 8] = t0;
        io_prefetch<NB, MFMA, DH, G, MOE, FP8>(PK, lds, sid);
        __syncthreads();  // B_out
        trace_mark(P, sid, 5);
        if (P.trace && lane_id() == 0) {
            uint64_t* tr = P.trace + ((size_t)blockIdx.x * (P.spl * P.L + 1) + sid) * 8;
            uint64_t packed = 0;
            const int slot[4] = {0, 5, 2, 3};  // checked, operand loaded, refill start, refill done
            for (int k = 0; k < 4; ++k) packed |= ((C.tdata[slot[k]] - t0) & 0xFFFFull) << (16 * k);
            tr[6] = packed;
            tr[7] = C.tdata[4];
        }
        io_stage<NB, MFMA, DH, G, MOE, W, FP8>(PK, lds, sid);
    }
}

template <int NB, bool MFMA, int DH, int G, int R, bool MOE, int W, bool FP8>
__global__ void __launch_bounds__((W + 1) * 64, 1) mk_decode_kernel(const Params P) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    (void)P;
    const int v = wave_id();
    if (v < W) compute_role<NB, MFMA, DH, G, R, MOE, W, FP8>(kparams(), lds, v);
    else io_role<NB, MFMA, DH, G, MOE, W, FP8>(kparams(), lds);
}

// ============================================================ packing & K/V copies
// mode 0: identity rows of s0 (rows >= n0 are zero); mode 1: RoPE-pair rows over the
// concatenation [s0 (n0 rows); s1 (n1); s2 (n2)] in heads of dh; mode 2: gate/up tiles.
__global__ void mk_pack_kernel(uint8_t* dst, int64_t n_lanes16, int nkb, int K, int mode, const uint16_t* s0,
                               const uint16_t* s1, const uint16_t* s2, int n0, int n1, int dh) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_lanes16) return;
    const int lane = (int)(i % 64);
    const int64_t rest = i / 64;
    const int kb = (int)(rest % nkb);
    const int64_t t = rest / nkb;
    const int r = lane & 15;
    const int k0 = 32 * kb + 8 * (lane >> 4);
    const int64_t R = 16 * t + r;
    const uint16_t* src = nullptr;
    if (mode == 0) {
        if (R < n0) src = s0 + R * K;
    } else if (mode == 1) {
        const int64_t head = R / dh;
        const int within = (int)(R % dh), jj = within / 16, rr = within % 16;
        const int dim = rr < 8 ? 8 * jj + rr : dh / 2 + 8 * jj + rr - 8;
        const int64_t row = head * dh + dim;
        if (row < n0) src = s0 + row * K;
        else if (row < n0 + n1) src = s1 + (row - n0) * K;
        else src = s2 + (row - n0 - n1) * K;
    } else {
        const int64_t f = 8 * t + (r & 7);
        src = (r < 8 ? s0 : s1) + f * K;
    }
    v4u val = {0u, 0u, 0u, 0u};
    if (src) val = *reinterpret_cast<const v4u*>(src + k0);
    reinterpret_cast<v4u*>(dst)[i] = val;
}

// ------------------------------------------------------------ FP8 weights
// Each output row's scale is its largest magnitude / 448 (1 for an all-zero
// row); its codes are the OCP E4M3 round-to-nearest-even of (w / scale), both
// divisions correctly rounded fp32, magnitudes at or above 448 saturated (the
// reading of the pages' 8-bit weights: Kog AI page, "Büyük Üçüncü Taraf MoE
// Modellerine Ölçeklendirme"; Cerebras catalogue page, "Model Sıkıştırma
// Mimarisi ve Şeffaflık").
__device__ __forceinline__ uint32_t e4m3_rne(float t) {
    const uint32_t u = __float_as_uint(t);
    const uint32_t sgn = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t code;
    if (a >= 0x43E00000u) {
        code = 0x7Eu;  // >= 448: saturate
    } else if (a < 0x3C800000u) {
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);  // below 2^-6: grid 2^-9; 8 is 2^-6
    } else {
        const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;  // exponent and 3 mantissa bits, rounded
        code = min(r - (120u << 3), 0x7Eu);                          // rebias 127 -> 7
    }
    return sgn | code;
}

// One wave per row of W [rows][K] (bf16): scale = max |w| / 448, or 1.
__global__ void mk_rowscale_kernel(const uint16_t* W, int rows, int K, float* out) {
    const int row = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int lane = threadIdx.x & 63;
    float m = 0.f;
    for (int k = lane; k < K; k += 64) m = fmaxf(m, fabsf(bf16_to_f(W[(int64_t)row * K + k])));
    for (int msk = 1; msk < 64; msk <<= 1) m = fmaxf(m, __shfl_xor(m, msk, 64));
    if (lane == 0) out[row] = m > 0.f ? __fdiv_rn(m, 448.0f) : 1.0f;
}

// FP8 tiles: the row order of mk_pack_kernel (modes 0, 1, 2), chunks of 64 K
// (see gemv_group), and the scales of the tile rows in the same order
// (sdst[16 t + r]); c0..c2 are the source matrices' row scales.
__global__ void mk_pack8_kernel(uint8_t* dst, int64_t n_lanes16, int nkb8, int K, int mode, const uint16_t* s0,
                                const uint16_t* s1, const uint16_t* s2, int n0, int n1, int dh, const float* c0,
                                const float* c1, const float* c2, float* sdst) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n_lanes16) return;
    const int lane = (int)(i % 64);
    const int64_t rest = i / 64;
    const int c = (int)(rest % nkb8);
    const int64_t t = rest / nkb8;
    const int r = lane & 15, kg = lane >> 4;
    const int64_t R = 16 * t + r;
    const uint16_t* src = nullptr;
    float sc = 1.0f;
    if (mode == 0) {
        if (R < n0) { src = s0 + R * K; sc = c0[R]; }
    } else if (mode == 1) {
        const int64_t head = R / dh;
        const int within = (int)(R % dh), jj = within / 16, rr = within % 16;
        const int dim = rr < 8 ? 8 * jj + rr : dh / 2 + 8 * jj + rr - 8;
        const int64_t row = head * dh + dim;
        if (row < n0) { src = s0 + row * K; sc = c0[row]; }
        else if (row < n0 + n1) { src = s1 + (row - n0) * K; sc = c1[row - n0]; }
        else { src = s2 + (row - n0 - n1) * K; sc = c2[row - n0 - n1]; }
    } else {
        const int64_t f = 8 * t + (r & 7);
        src = (r < 8 ? s0 : s1) + f * K;
        sc = (r < 8 ? c0 : c1)[f];
    }
    uint32_t wd[4] = {0u, 0u, 0u, 0u};
    if (src) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const v4u v = *reinterpret_cast<const v4u*>(src + 64 * c + 32 * h + 8 * kg);
            const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = e4m3_rne(__fdiv_rn(bf_lo(x[e]), sc)), hi = e4m3_rne(__fdiv_rn(bf_hi(x[e]), sc));
                wd[2 * h + e / 2] |= (lo | (hi << 8)) << (16 * (e & 1));
            }
        }
    }
    reinterpret_cast<v4u*>(dst)[i] = (v4u){wd[0], wd[1], wd[2], wd[3]};
    if (c == 0 && kg == 0) sdst[R] = sc;
}

// rows [n][Hkv][dh] <-> pool slots of one layer of the K (isv = 0) or V pool, in
// the page layouts of the attention kernel; dir 0: write pool, 1: read pool
template <int DH>
__device__ void kv_copy_rows(uint16_t* blk, uint16_t* rr, int off, int isv, int dir) {
    for (int e = threadIdx.x; e < DH; e += blockDim.x) {
        const int idx = isv ? kv_elem_v<DH>(off, e) : kv_elem_k<DH>(off, e);
        if (dir == 0) blk[idx] = rr[e];
        else rr[e] = blk[idx];
    }
}
__global__ void mk_kv_copy_kernel(uint16_t* pool, const int32_t* slots, uint16_t* rows, int n, int dh, int isv,
                                  int64_t n_slots, int dir, uint32_t* err) {
    const int r = blockIdx.x;
    if (r >= n) return;
    const int32_t s = slots[r];
    if (s < 0 || (int64_t)s >= n_slots) {
        if (threadIdx.x == 0) {
            if (atomicCAS(err, 0u, 5u) == 0u) err[1] = (uint32_t)r;
        }
        return;
    }
    const int page = s / kPage, off = s % kPage;
    const int head = blockIdx.y;  // one block per (row, kv head)
    uint16_t* blk = pool + ((int64_t)page * gridDim.y + head) * kPage * dh;
    uint16_t* rr = rows + ((int64_t)r * gridDim.y + head) * dh;
    if (dh == 128) kv_copy_rows<128>(blk, rr, off, isv, dir);
    else kv_copy_rows<64>(blk, rr, off, isv, dir);
}

// Zero n words from p (grid-stride).
__global__ void mk_zero_kernel(uint32_t* p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// The exchange buffers and flags of the allocation-free decode entry point:
// one copy per device, held until the process ends, shared by every such call
// on the device (calls that overlap on one device race).
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

}  // namespace mk

// ================================================================ host launchers
#include <hip/hip_runtime.h>

#include <mutex>

namespace mk {

// Per device: the device address of `scratch` (from hipGetSymbolAddress with
// that device current; host code never passes the array's name), the flag
// value of the last launch on it and the next tag base.
struct StaticScratch { uint8_t* base; uint32_t epoch, tag_base; };
namespace {
constexpr int kMaxDevices = 64;
struct DevScratch { uint8_t* ptr = nullptr; uint32_t epoch = 0; uint32_t tag_next = 1; };
DevScratch g_dev_scratch[kMaxDevices];
std::mutex g_dev_scratch_mu;
}  // namespace

hipError_t static_scratch_acquire(int device, hipStream_t stream, uint32_t stages, StaticScratch* out) {
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_dev_scratch_mu);
    DevScratch& ds = g_dev_scratch[device];
    if (!ds.ptr) {
        // set-up, once per device, with the device current (the caller checked):
        // the symbol's address on this device, then a clear so that no flag is
        // raised and no exchanged word carries a tag
        void* ptr = nullptr;
        hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
        hipLaunchKernelGGL(mk_zero_kernel, dim3(1024), dim3(256), 0, stream, static_cast<uint32_t*>(ptr),
                           kStaticScratchBytes / 4);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        ds.ptr = static_cast<uint8_t*>(ptr);
    }
    // flags compare against a value above every flag already raised in the
    // array; tags are unique across the calls sharing it (tag_base + stage)
    out->base = ds.ptr;
    out->epoch = ++ds.epoch;
    out->tag_base = ds.tag_next;
    ds.tag_next += stages;
    if (ds.tag_next < stages) ds.tag_next = 1;  // (wrapped: tags restart above 0)
    return hipSuccess;
}

typedef void (*KernelFn)(const Params);

template <int NB, bool MFMA, int DH, int G, bool MOE, int W, bool FP8>
static const void* kernel_ptr_w(int ring) {
    constexpr int RING = ring_slots(W, MFMA, G);
    return ring == RING ? (const void*)mk_decode_kernel<NB, MFMA, DH, G, RING, MOE, W, FP8> : nullptr;
}
// The variant's preferred compute-wave count, and four where that is eight (the
// host falls back to four when eight do not fit).
template <int NB, bool MFMA, int DH, int G, bool MOE, bool FP8 = false>
static const void* kernel_ptr(int ring, int waves) {
    constexpr int WP = compute_waves(G, MOE, MFMA);
    if (waves == WP) return kernel_ptr_w<NB, MFMA, DH, G, MOE, WP, FP8>(ring);
    if constexpr (WP != 4)
        if (waves == 4) return kernel_ptr_w<NB, MFMA, DH, G, MOE, 4, FP8>(ring);
    return nullptr;
}

// Returns the kernel for (nb class, mfma, dh, G, ring slots, MoE, compute waves,
// FP8 weights) or null if not instantiated (FP8: dense models with groups of 2).
const void* select_kernel(int nb, bool mfma, int dh, int G, int ring, bool moe, int waves, bool fp8) {
    if (fp8) {
#define MK_CASE8(NB_, MF_, DH_) \
        if (nb == NB_ && mfma == MF_ && dh == DH_ && G == 2 && !moe) return kernel_ptr<NB_, MF_, DH_, 2, false, true>(ring, waves);
        MK_CASE8(1, false, 128)
        MK_CASE8(2, false, 128)
        MK_CASE8(8, true, 128)
        MK_CASE8(1, false, 64)
        MK_CASE8(2, false, 64)
        MK_CASE8(8, true, 64)
#undef MK_CASE8
        return nullptr;
    }
#define MK_CASE(NB_, MF_, DH_, G_, MOE_) \
    if (nb == NB_ && mfma == MF_ && dh == DH_ && G == G_ && moe == MOE_) return kernel_ptr<NB_, MF_, DH_, G_, MOE_>(ring, waves);
    MK_CASE(1, false, 128, 2, false)
    MK_CASE(2, false, 128, 2, false)
    MK_CASE(8, true, 128, 2, false)
    MK_CASE(1, false, 64, 2, false)
    MK_CASE(2, false, 64, 2, false)
    MK_CASE(8, true, 64, 2, false)
    MK_CASE(1, false, 128, 8, false)
    MK_CASE(2, false, 128, 8, false)
    MK_CASE(8, true, 128, 8, false)
    MK_CASE(1, false, 64, 2, true)
    MK_CASE(2, false, 64, 2, true)
    MK_CASE(8, true, 64, 2, true)
    MK_CASE(1, false, 128, 8, true)
    MK_CASE(2, false, 128, 8, true)
    MK_CASE(8, true, 128, 8, true)
#undef MK_CASE
    return nullptr;
}

hipError_t launch_decode(const void* fn, const Params& P, int threads, hipStream_t stream, bool cooperative) {
    void* args[] = {const_cast<Params*>(&P)};
    if (!cooperative) return hipLaunchKernel(fn, dim3(P.NW), dim3(threads), args, (unsigned)P.lds_total, stream);
    return hipLaunchCooperativeKernel(fn, dim3(P.NW), dim3(threads), args, (unsigned)P.lds_total, stream);
}

hipError_t launch_pack(uint8_t* dst, int T, int nkb, int K, int mode, const uint16_t* s0, const uint16_t* s1,
                       const uint16_t* s2, int n0, int n1, int dh, hipStream_t stream) {
    const int64_t n = (int64_t)T * nkb * 64;
    if (n == 0) return hipSuccess;
    const int threads = 256;
    const int64_t blocks = (n + threads - 1) / threads;
    hipLaunchKernelGGL(mk_pack_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, dst, n, nkb, K, mode, s0, s1,
                       s2, n0, n1, dh);
    return hipGetLastError();
}

hipError_t launch_rowscale(const uint16_t* W, int rows, int K, float* out, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(mk_rowscale_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, W, rows, K, out);
    return hipGetLastError();
}

hipError_t launch_pack8(uint8_t* dst, int T, int nkb8, int K, int mode, const uint16_t* s0, const uint16_t* s1,
                        const uint16_t* s2, int n0, int n1, int dh, const float* c0, const float* c1, const float* c2,
                        float* sdst, hipStream_t stream) {
    const int64_t n = (int64_t)T * nkb8 * 64;
    if (n == 0) return hipSuccess;
    const int threads = 256;
    const int64_t blocks = (n + threads - 1) / threads;
    hipLaunchKernelGGL(mk_pack8_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, dst, n, nkb8, K, mode, s0,
                       s1, s2, n0, n1, dh, c0, c1, c2, sdst);
    return hipGetLastError();
}

hipError_t launch_kv_copy(uint16_t* pool_layer, const int32_t* slots, uint16_t* rows, int n, int Hkv, int dh, int isv,
                          int64_t n_slots, int dir, uint32_t* err, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(mk_kv_copy_kernel, dim3(n, Hkv), dim3(64), 0, stream, pool_layer, slots, rows, n, dh, isv,
                       n_slots, dir, err);
    return hipGetLastError();
}

}  // namespace mk
