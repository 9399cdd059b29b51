// mk_prefill.hip - paged prefill for gfx950: a prompt's tokens run through the
// model in chunks, their K and V written into the request's 16-token pages, and
// the last position's logits and token produced, so that decode steps can take
// over from there. The pages place prefill beside the decode path (Cohere
// Megakernel page, "Sınırlar açıkça yazılmış": prefill runs outside the decode
// kernel; Cerebras disaggregation page, "Ön Doldurma ve Çözümleme Donanım
// Üzerinde Farklı Talepler Oluşturur": prefill is compute-bound), so it is
// built from matrix-core kernels rather than the bandwidth-bound decode path:
//   - GEMMs read the decode path's packed 1 KB weight tiles directly as the
//     16x16x32 MFMA A operand (rows = output features; the same lane order
//     serves A and B), so the RoPE-pair and gate/up row orders of the tiles
//     carry over to the epilogues; activations enter as 16-token "operand
//     blocks" in the B-operand lane order, split into bf16 hi and lo parts
//     (x = hi + lo, about 16 significant bits, as in the decode path). The
//     blocks stream through an eight-deep LDS ring by DMA and the weight chunks
//     through registers, seven k-steps ahead of the matrix cores; GEMMs with
//     few output tiles split K over workgroups into partial sums;
//   - every producer writes its consumer's operand blocks directly: the row
//     pass after a residual GEMM (residual add, the next RMSNorm's scale and
//     gains), the gate/up epilogue (SwiGLU) and the attention merge;
//   - attention: one workgroup per (16-token group, query head), its eight
//     waves taking interleaved K/V pages (in their matrix-core page order:
//     K . Q^T on 16x16x32, V^T . P^T on 16x16x16, whose B operand is the
//     score accumulator's own lane layout) with an online softmax each, merged
//     through LDS; causal and windowed by position; the workgroups of one kv
//     head are dispatched to one XCD so that its L2 holds that head's pages;
//   - chunks of up to kPfChunk tokens are independent except through the
//     pool: a chunk's attention reads the keys and values earlier chunks (and
//     earlier prompts or decode steps) wrote.
#include <type_traits>

#include "mk_device.h"
#include "mk_params.h"
#include "mk_prefill.h"

namespace mk {

// One 2 KB operand block per (16-token group g, 32-k block kb): bytes
// [0, 1024) the hi parts, [1024, 2048) the lo parts; lane l's 16 bytes hold
// token 16 g + l % 16 at k = 32 kb + 8 (l / 16) + e, e = 0..7.
constexpr int kBlk = 2048;
constexpr int kPfStages = 8;   // operand ring depth of the GEMMs (k-steps in flight + 1)

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), in order
template <int N, int J = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (J < N) {
        f(std::integral_constant<int, J>{});
        static_for<N, J + 1>(f);
    }
}

// Byte offset of (token i, k .. k + 3 or k + 7) inside the operand blocks of a
// K = 32 nkb matrix: the hi parts there, the lo parts 1024 bytes further.
__device__ __forceinline__ int64_t blk_off(int i, int k, int nkb) {
    return ((int64_t)(i >> 4) * nkb + (k >> 5)) * kBlk + ((i & 15) + 16 * ((k & 31) >> 3)) * 16 + (k & 7) * 2;
}
// Four values as hi and lo bf16 pairs (hi = RNE(x), lo = RNE(x - hi)).
__device__ __forceinline__ void split4(const float* x, v2u* hi, v2u* lo) {
    uint32_t h[2], l[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        h[e] = cvt_bf16x2(x[2 * e], x[2 * e + 1]);
        l[e] = cvt_bf16x2(x[2 * e] - bf_lo(h[e]), x[2 * e + 1] - bf_hi(h[e]));
    }
    *hi = (v2u){h[0], h[1]};
    *lo = (v2u){l[0], l[1]};
}

__device__ __forceinline__ void latch(uint32_t* err, uint32_t code, uint32_t where) {
    if (atomicCAS(err, 0u, code) == 0u) __hip_atomic_store(err + 1, where, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup per row i < 16 n_groups of a chunk (rows >= n: zero blocks).
// Each thread owns 8 consecutive columns: y = E[token] (an out-of-range token
// gives a zero row and latches MK_ERR_BAD_PAGE) or res + the splits' partial
// sums in split order; y is stored, rs = 1/sqrt(mean(y^2) + eps), and y * gains
// goes to the operand blocks. (The GEMMs take the RMSNorm scale in their
// epilogue: x * gains of an embedding row needs at most 16 significant bits,
// so its hi/lo split is exact.)
__global__ void __launch_bounds__(256) pf_rows_kernel(const PfRows a) {
    __shared__ float red[4];
    const int i = blockIdx.x;
    const bool live = i < a.n;
    const int d8 = a.d / 8;
    int tok = 0;
    bool tok_ok = true;
    if (a.tokens && live) {
        tok = a.tokens[i];
        tok_ok = tok >= 0 && tok < a.V;
        if (!tok_ok && threadIdx.x == 0) latch(a.err, 5u, (uint32_t)i);
    }
    float ss = 0.f;
    for (int c = threadIdx.x; c < d8; c += blockDim.x) {
        const int k = 8 * c;
        float y[8];
        if (!live) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = 0.f;
        } else if (a.tokens) {
            const v4u u = tok_ok ? *reinterpret_cast<const v4u*>(a.embed + (int64_t)tok * a.d + k) : (v4u){0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y[2 * e] = bf_lo(u[e]);
                y[2 * e + 1] = bf_hi(u[e]);
            }
        } else {
            const float* r = a.y + (int64_t)i * a.d + k;
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = 0.f;
            for (int z = 0; z < a.S; ++z) {
                const float* p = a.part + ((int64_t)z * kPfChunk + i) * a.d + k;
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] += p[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = r[e] + y[e];
        }
        if (live) {
            float* o = a.y + (int64_t)i * a.d + k;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o[e] = y[e];
                ss += y[e] * y[e];
            }
        }
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = y[e] * bf16_to_f(a.gains[k + e]);
        v2u h0, l0, h1, l1;
        split4(x, &h0, &l0);
        split4(x + 4, &h1, &l1);
        uint8_t* b = a.blk + blk_off(i, k, a.d / 32);
        *reinterpret_cast<v4u*>(b) = (v4u){h0.x, h0.y, h1.x, h1.y};
        *reinterpret_cast<v4u*>(b + 1024) = (v4u){l0.x, l0.y, l1.x, l1.y};
    }
    if (!live) return;
    for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.f;
        for (int w = 0; w < (int)(blockDim.x / 64); ++w) t += red[w];
        a.rs[i] = 1.0f / sqrtf(t / (float)a.d + a.eps);
    }
}

// Output tiles TPW (WV blockIdx.x + wave) .. + TPW - 1 x token groups
// [NG blockIdx.y, + NG) over the k-blocks of split blockIdx.z. Per k-step
// the workgroup's NG operand blocks go global -> LDS by DMA into a ring of
// kPfStages slots and each wave's weight chunks into registers, seven steps
// ahead; each wave runs two MFMAs (hi and lo parts) per (tile, token group).
// Every wave issues the same number of vector-memory operations per step, so
// one vmcnt bound serves every step.
template <int EPI, int TPW, int NG, int WV, int KPC>
__global__ void __launch_bounds__(64 * WV, 1) pf_gemm_kernel(const PfGemm a) {
    static_assert((NG == 4 || NG == 8) && (WV == 4 || WV == 8) && 2 * NG >= WV && (KPC == 1 || KPC == 2),
                  "workgroup shape");
    // KPC operand k-blocks per weight chunk: 1 (bf16, 32 K per chunk) or 2 (FP8, 64 K)
    constexpr int NST = KPC == 1 ? kPfStages : kPfStages / 2;   // ring slots (the LDS holds NST x NG x KPC blocks)
    __shared__ __attribute__((aligned(16))) uint8_t stage[NST][NG * KPC][kBlk];
    constexpr int DPW = 2 * NG * KPC / WV;   // 1 KB halves of operand blocks each wave moves per step
    constexpr int OPS = DPW + TPW;           // vector-memory operations per wave per step
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t0 = TPW * (WV * blockIdx.x + w);
    const int g0 = NG * blockIdx.y;
    const int z = blockIdx.z, S = gridDim.z;
    const int kb0 = (int)(((int64_t)a.nkb * z) / S);   // weight chunks of this split
    const int nk = (int)(((int64_t)a.nkb * (z + 1)) / S) - kb0;
    const int nkx = KPC * a.nkb;                         // operand blocks per token group
    const uint32_t lane16 = (uint32_t)lane * 16u;
    const __amdgpu_buffer_rsrc_t rx = rsrc_n(a.x, (uint32_t)((int64_t)a.n_groups * nkx * kBlk));
    const __amdgpu_buffer_rsrc_t rw = rsrc_n(a.w, (uint32_t)((int64_t)a.T * a.nkb * 1024));
    // Steps past the split's end, tiles past T and token groups past n_groups
    // load (clamped) data that is never used: no branches around the loads,
    // so the compiler keeps them in flight across the steps.
    auto issue = [&](int i, int slot) {
        const int kb = kb0 + min(i, nk - 1);
#pragma unroll
        for (int q = 0; q < DPW; ++q) {
            const int j = DPW * w + q, bi = j >> 1, h = j & 1;   // block bi = (group bi / KPC, k-block bi % KPC)
            const int g = min(g0 + bi / KPC, a.n_groups - 1);
            const uint32_t off = (uint32_t)(((int64_t)g * nkx + KPC * kb + bi % KPC) * kBlk) + (uint32_t)h * 1024u + lane16;
            dma_chunk(rx, (__attribute__((address_space(3))) uint8_t*)&stage[slot][bi][h * 1024], off);
        }
    };
    v4u wr[NST][TPW];
    auto wload = [&](int i, v4u* dst) {
        const int kb = kb0 + min(i, nk - 1);
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int t = min(t0 + j, a.T - 1);
            dst[j] = ld_chunk(rw, (uint32_t)(((int64_t)t * a.nkb + kb) * 1024), lane16);
        }
    };
    v4f acc[TPW][NG];
#pragma unroll
    for (int j = 0; j < TPW; ++j)
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) acc[j][gi] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NST - 1; ++s) {
        issue(s, s);
        wload(s, wr[s]);
    }
    auto step = [&](int i, auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
        wait_vm<OPS * (NST - 2)>();         // step i's DMAs and weights (this wave's)
        lds_barrier();                      // every wave's; and step i - 1 is done with its slot
        issue(i + NST - 1, (slot + NST - 1) % NST);
        wload(i + NST - 1, wr[(slot + NST - 1) % NST]);
        if (i < nk) {
            // the weight chunk as KPC 16x16x32 A operands (FP8: decoded to bf16, exactly)
            v4u wa[KPC][TPW];
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                if constexpr (KPC == 1) {
                    wa[0][j] = wr[slot][j];
                } else {
                    wa[0][j] = fp8x8_to_bf16x8(wr[slot][j].x, wr[slot][j].y);
                    wa[KPC - 1][j] = fp8x8_to_bf16x8(wr[slot][j].z, wr[slot][j].w);
                }
            }
#pragma unroll
            for (int kk = 0; kk < KPC; ++kk) {
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    const v4u bh = *reinterpret_cast<const v4u*>(&stage[slot][gi * KPC + kk][lane16]);
#pragma unroll
                    for (int j = 0; j < TPW; ++j) acc[j][gi] = mfma16x16x32(wa[kk][j], bh, acc[j][gi]);
                }
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    const v4u bl = *reinterpret_cast<const v4u*>(&stage[slot][gi * KPC + kk][1024 + lane16]);
#pragma unroll
                    for (int j = 0; j < TPW; ++j) acc[j][gi] = mfma16x16x32(wa[kk][j], bl, acc[j][gi]);
                }
            }
        }
    };
    for (int i = 0; i < nk; i += NST)
        static_for<NST>([&](auto J) { step(i + decltype(J)::value, J); });
    wait_vm<0>();   // the DMAs past the end land before the workgroup exits
    // D: lane l holds token 16 g + l % 16, rows 4 (l / 16) + j of the tile
    const int r0 = 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < TPW; ++j) {
        const int t = t0 + j;
        if (t >= a.T) continue;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            if (g0 + gi >= a.n_groups) continue;
            const int tok = 16 * (g0 + gi) + (lane & 15);
            const bool live = tok < a.n;
            v4f y = acc[j][gi];
            if (a.rs && live) y *= a.rs[tok];  // RMSNorm scale after the product (operand x * gains)
            if constexpr (KPC == 2) {
                // FP8: each row's scale (rows 16 t + r0 .. + 3, packed row order)
                const v4f sc4 = *reinterpret_cast<const v4f*>(a.wscale + 16 * t + r0);
                y *= sc4;
            }
            if constexpr (EPI == PF_PART) {
                const int row = 16 * t + r0;
                if (live && row < a.ldo)
                    *reinterpret_cast<v4f*>(a.out + ((int64_t)z * kPfChunk + tok) * a.ldo + row) = y;
            } else if constexpr (EPI == PF_LM) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int row = 16 * t + r0 + jj;
                    if (tok == a.n - 1 && row < a.ldo) a.out[row] = y[jj];
                }
            } else {
                // rows r and r + 8 of a tile pair up (RoPE halves, or gate and up):
                // lanes 0..31 hold rows 0..7, lanes 32..63 rows 8..15 of the same tokens
                float part[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) part[jj] = __shfl_xor(y[jj], 32, 64);
                if (lane >= 32) continue;
                if constexpr (EPI == PF_GU) {
                    // features 8 t + r0 .. + 3: four consecutive k of the down projection's operand
                    float v[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) v[jj] = live ? y[jj] / (1.0f + __expf(-y[jj])) * part[jj] : 0.f;
                    v2u hi, lo;
                    split4(v, &hi, &lo);
                    uint8_t* b = a.act_blk + blk_off(tok, 8 * t + r0, a.F / 32);
                    *reinterpret_cast<v2u*>(b) = hi;
                    *reinterpret_cast<v2u*>(b + 1024) = lo;
                } else {
                    if (!live) continue;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int r = r0 + jj;  // 0..7
                        const float y0 = y[jj], y1 = part[jj];
                        const int head = 16 * t / a.dh, ii = 8 * ((16 * t % a.dh) / 16) + r;  // pair (ii, ii + dh/2)
                        const int p = a.pos0 + tok;
                        float v0 = y0, v1 = y1;
                        if (head < a.Hq + a.Hkv) {
                            const float2 cs = reinterpret_cast<const float2*>(a.rope)[(int64_t)p * (a.dh / 2) + ii];
                            v0 = y0 * cs.x - y1 * cs.y;
                            v1 = y0 * cs.y + y1 * cs.x;
                        }
                        if (head < a.Hq) {
                            a.q[(int64_t)tok * a.Hq * a.dh + head * a.dh + ii] = v0;
                            a.q[(int64_t)tok * a.Hq * a.dh + head * a.dh + ii + a.dh / 2] = v1;
                        } else {
                            const int kvh = head - a.Hq, isv = kvh >= a.Hkv, g = isv ? kvh - a.Hkv : kvh;
                            const int pid = a.pages[p / kPage];
                            if (pid < 0 || pid >= a.n_pages) {
                                latch(a.err, 5u, (uint32_t)tok);
                            } else {
                                uint16_t* blk = (isv ? a.vpool : a.kpool) + ((int64_t)pid * a.Hkv + g) * kPage * a.dh;
                                const int sl = p % kPage;
                                const uint16_t h0 = f_to_bf16(v0), h1 = f_to_bf16(v1);
                                if (a.dh == 128) {
                                    blk[isv ? kv_elem_v<128>(sl, ii) : kv_elem_k<128>(sl, ii)] = h0;
                                    blk[isv ? kv_elem_v<128>(sl, ii + 64) : kv_elem_k<128>(sl, ii + 64)] = h1;
                                } else {
                                    blk[isv ? kv_elem_v<64>(sl, ii) : kv_elem_k<64>(sl, ii)] = h0;
                                    blk[isv ? kv_elem_v<64>(sl, ii + 32) : kv_elem_k<64>(sl, ii + 32)] = h1;
                                }
                            }
                        }
                    }
                }
            }
        }
    }
}

// One workgroup per (token group g, query head h): causal (and windowed)
// attention of the group's 16 tokens over the pool pages. Token column
// c = lane % 16 is position pos0 + 16 g + c; it attends to keys [lo, that
// position] (lo = max(0, position - win + 1) for a window, else 0). Wave w
// takes pages first + w, first + w + 8, ... with its own online softmax
// (m, l, o) and the next page's K and V loaded while it computes one; the
// eight partials merge through LDS and the result is written as the output
// projection's operand blocks. Workgroup id -> (kv head = id % Hkv, query head
// in the group, token group): the hardware deals consecutive ids to the XCDs
// in turn, so with Hkv dividing 8 each XCD serves whole kv heads.
template <int DH>
__global__ void __launch_bounds__(512, 1) pf_attn_kernel(const PfAttn a) {
    constexpr int CPP = DH / 32;   // K chunks per page
    constexpr int NJB = DH / 16;   // V dim blocks
    constexpr int NW = 8;
    __shared__ float s_m[NW][16], s_l[NW][16];
    __shared__ __attribute__((aligned(16))) v4f s_o[NW][NJB][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int G = a.Hq / a.Hkv;
    const int id = blockIdx.x;
    const int kvh = id % a.Hkv, rest = id / a.Hkv;
    const int h = kvh * G + rest % G, g = rest / G;
    const int col = lane & 15, rg = lane >> 4;
    const int ti = 16 * g + col;
    const bool tok_ok = ti < a.n;
    const int p_tok = a.pos0 + ti;
    const int lo_tok = a.win > 0 ? max(0, p_tok - a.win + 1) : 0;
    const int pmin = a.pos0 + 16 * g, pmax = a.pos0 + min(16 * g + 15, a.n - 1);
    const int lo_min = a.win > 0 ? max(0, pmin - a.win + 1) : 0;
    // q of this column's token, times log2 e / sqrt(dh), as hi and lo B operands
    // (columns past the chunk read the last token's row and use zeros)
    const float scale = 1.4426950408889634f / sqrtf((float)DH);
    const float* qrow = a.q + (int64_t)min(ti, a.n - 1) * a.Hq * DH + h * DH + 8 * rg;
    v4u qh[CPP], ql[CPP];
#pragma unroll
    for (int j = 0; j < CPP; ++j) {
        const v4f x0 = *reinterpret_cast<const v4f*>(qrow + 32 * j);
        const v4f x1 = *reinterpret_cast<const v4f*>(qrow + 32 * j + 4);
        const float sc = tok_ok ? scale : 0.f;
        float x[8] = {x0[0] * sc, x0[1] * sc, x0[2] * sc, x0[3] * sc, x1[0] * sc, x1[1] * sc, x1[2] * sc, x1[3] * sc};
        uint32_t hh[4], ll[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            hh[e] = cvt_bf16x2(x[2 * e], x[2 * e + 1]);
            ll[e] = cvt_bf16x2(x[2 * e] - bf_lo(hh[e]), x[2 * e + 1] - bf_hi(hh[e]));
        }
        qh[j] = (v4u){hh[0], hh[1], hh[2], hh[3]};
        ql[j] = (v4u){ll[0], ll[1], ll[2], ll[3]};
    }
    float m = -INFINITY, lsum = 0.f;
    v4f o[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) o[jb] = (v4f){0.f, 0.f, 0.f, 0.f};
    const int P_last = pmax / kPage;
    // Pages P0, P0 + 8, ... of this wave, two in flight while one is computed.
    // Loads past P_last re-read page P_last and are not used; an id outside
    // the pool reads page 0's slot and is skipped (and latched) when computed.
    const int P0 = lo_min / kPage + __builtin_amdgcn_readfirstlane(w);
    // page ids through the scalar cache (the table is not written during the
    // launch), so that reading one waits on no K/V load in flight
    const __attribute__((address_space(4))) int32_t* ptab = (const __attribute__((address_space(4))) int32_t*)a.pages;
    auto pid_of = [&](int P) { return ptab[min(P, P_last)]; };
    auto load = [&](int pid, v4u* kk, v2u* vv) {
        const bool ok = pid >= 0 && pid < a.n_pages;
        const int64_t blk = ok ? ((int64_t)pid * a.Hkv + kvh) * kPage * DH : 0;
#pragma unroll
        for (int j = 0; j < CPP; ++j) kk[j] = *reinterpret_cast<const v4u*>(a.kpool + blk + j * 512 + lane * 8);
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) vv[jb] = *reinterpret_cast<const v2u*>(a.vpool + blk + jb * 256 + lane * 4);
    };
    auto process = [&](int P, int pid, const v4u* kw, const v2u* vw) {
        if (P > P_last) return;
        if (pid < 0 || pid >= a.n_pages) {
            if (lane == 0) latch(a.err, 5u, (uint32_t)P);
            return;
        }
        // V rows outside [lo_min, pmax] were not written for these tokens: zero them
        // (their weights are 0, their bits need not be finite)
        uint32_t mk2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int q0 = P * kPage + 4 * rg + 2 * hh;
            mk2[hh] = ((q0 >= lo_min && q0 <= pmax) ? 0x0000FFFFu : 0u) |
                      ((q0 + 1 >= lo_min && q0 + 1 <= pmax) ? 0xFFFF0000u : 0u);
        }
        // S^T[pos][token] = K Q^T: lane holds token col, positions 4 rg + i of the page
        v4f sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < CPP; ++j) {
            sc = mfma16x16x32(kw[j], qh[j], sc);
            sc = mfma16x16x32(kw[j], ql[j], sc);
        }
        float s[4], pm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pos = P * kPage + 4 * rg + i;
            const bool ok = tok_ok && pos >= lo_tok && pos <= p_tok;
            s[i] = ok ? sc[i] : -INFINITY;
            pm = fmaxf(pm, s[i]);
        }
        pm = max_xor32(max_xor16(pm));  // page max of this token
        const float mn = fmaxf(m, pm);
        const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mn);
        float pr[4], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[i] = s[i] == -INFINITY ? 0.f : fast_exp2(s[i] - mn);
            ps += pr[i];
        }
        lsum = lsum * alpha + ps;
        if (mn != -INFINITY) m = mn;
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) o[jb] *= alpha;
        uint32_t ph[2], pl[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            ph[hh] = cvt_bf16x2(pr[2 * hh], pr[2 * hh + 1]);
            pl[hh] = cvt_bf16x2(pr[2 * hh] - bf_lo(ph[hh]), pr[2 * hh + 1] - bf_hi(ph[hh]));
        }
        const v2u bh = {ph[0], ph[1]}, bl = {pl[0], pl[1]};
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            const v2u vm = {vw[jb].x & mk2[0], vw[jb].y & mk2[1]};
            o[jb] = mfma16x16x16(vm, bh, o[jb]);
            o[jb] = mfma16x16x16(vm, bl, o[jb]);
        }
    };
    v4u kA[CPP], kB[CPP], kC[CPP];
    v2u vA[NJB], vB[NJB], vC[NJB];
    int pA = pid_of(P0), pB = pid_of(P0 + NW), pC;
    load(pA, kA, vA);
    load(pB, kB, vB);
    for (int P = P0; P <= P_last; P += 3 * NW) {
        pC = pid_of(P + 2 * NW);
        load(pC, kC, vC);
        process(P, pA, kA, vA);
        pA = pid_of(P + 3 * NW);
        load(pA, kA, vA);
        process(P + NW, pB, kB, vB);
        pB = pid_of(P + 4 * NW);
        load(pB, kB, vB);
        process(P + 2 * NW, pC, kC, vC);
    }
    // this wave's partial: m per column, l summed over the column's four lanes
    const float lt = sum_xor32(sum_xor16(lsum));
    if (rg == 0) {
        s_m[w][col] = m;
        s_l[w][col] = lt;
    }
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) s_o[w][jb][lane] = o[jb];
    __syncthreads();
    // merge: thread -> (column c, dims 4 d4 .. + 3), in wave order
    const int c = threadIdx.x & 15, d4 = threadIdx.x >> 4;
    if (d4 >= DH / 4) return;
    const int jb = d4 >> 2, r = d4 & 3;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, s_m[v][c]);
    float L = 0.f;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const float f = s_m[v][c] == -INFINITY ? 0.f : fast_exp2(s_m[v][c] - M);
            L += s_l[v][c] * f;
            acc += s_o[v][jb][c + 16 * r] * f;
        }
    }
    const int tok = 16 * g + c;
    float y[4];
    const float inv = (tok < a.n && L > 0.f) ? 1.0f / L : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = acc[i] * inv;
    v2u hi, lo;
    split4(y, &hi, &lo);
    uint8_t* b = a.o_blk + blk_off(tok, h * DH + 16 * jb + 4 * r, a.Hq * DH / 32);
    *reinterpret_cast<v2u*>(b) = hi;
    *reinterpret_cast<v2u*>(b + 1024) = lo;
}

// SplitMix64 output step (Steele, Lea, Flood 2014)
__device__ __forceinline__ uint64_t pf_splitmix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Token of the last position: greedy (lowest index among equal maxima) or the
// Gumbel-max rule of the decode sampler with request index b; one block.
__global__ void __launch_bounds__(1024) pf_sample_kernel(const float* logits, int V, float T, uint64_t seed, uint32_t step,
                                                         int b, int32_t* token_out, float* logits_out) {
    __shared__ float bs[16];
    __shared__ int bi[16];
    const int tid = threadIdx.x;
    float best = -INFINITY;
    int idx = 0x7fffffff;
    const uint64_t key = pf_splitmix64(pf_splitmix64(pf_splitmix64(seed) + step) + (uint64_t)b);
    for (int i = tid; i < V; i += blockDim.x) {
        const float y = logits[i];
        if (logits_out) logits_out[i] = y;
        float sc = y;
        if (T > 0.f) {
            const uint64_t hh = pf_splitmix64(key + (uint64_t)i);
            const float u = (float)(2u * (uint32_t)(hh >> 41) + 1u) * (1.0f / 16777216.0f);
            sc = y / T - __logf(-__logf(u));
        }
        if (sc > best || (sc == best && i < idx)) { best = sc; idx = i; }
    }
    for (int m = 1; m < 64; m <<= 1) {
        const float s2 = __shfl_xor(best, m, 64);
        const int i2 = __shfl_xor(idx, m, 64);
        if (s2 > best || (s2 == best && i2 < idx)) { best = s2; idx = i2; }
    }
    if ((tid & 63) == 0) { bs[tid >> 6] = best; bi[tid >> 6] = idx; }
    __syncthreads();
    if (tid == 0) {
        for (int k = 1; k < (int)(blockDim.x / 64); ++k)
            if (bs[k] > best || (bs[k] == best && bi[k] < idx)) { best = bs[k]; idx = bi[k]; }
        token_out[0] = idx;
    }
}

}  // namespace mk

// ================================================================ host launchers
namespace mk {

namespace {
// Workgroup shape of each epilogue's GEMM: waves, tiles per wave, token groups.
struct GemmShape { int wv, tpw, ng; };
// (8 waves: each operand block read from LDS feeds more tiles; an 8192-token
// prompt of the 2B model took 114 ms with 4-wave workgroups everywhere,
// 104 ms with this gate/up shape alone.)
constexpr GemmShape kGemmShape[4] = {
    {8, 1, 8},   // PF_PART: 128 rows x 128 tokens
    {8, 2, 4},   // PF_QKV: 256 rows x 64 tokens (few tiles: more workgroups over the tokens)
    {8, 2, 8},   // PF_GU: 256 rows x 128 tokens
    {4, 2, 4},   // PF_LM: one token group
};
}  // namespace

// K splits of a GEMM: residual GEMMs (PF_PART) split K while there are fewer
// than 256 workgroups, keeping at least 8 k-blocks per split; the others 1.
int pf_splits(int epi, const PfGemm& a) {
    if (epi != PF_PART) return 1;
    const GemmShape g = kGemmShape[epi];
    const int wgs = ((a.T + g.wv * g.tpw - 1) / (g.wv * g.tpw)) * ((a.n_groups + g.ng - 1) / g.ng);
    int S = 1;
    while (wgs * S < 256 && 2 * S <= kPfSplitMax && a.nkb / (2 * S) >= 8) S *= 2;
    return S;
}

template <int EPI, int TPW, int NG, int WV>
hipError_t launch_gemm_shape(const PfGemm& a, int splits, hipStream_t s) {
    const dim3 grid((a.T + WV * TPW - 1) / (WV * TPW), (a.n_groups + NG - 1) / NG, splits);
    if (a.wscale) hipLaunchKernelGGL((pf_gemm_kernel<EPI, TPW, NG, WV, 2>), grid, dim3(64 * WV), 0, s, a);
    else hipLaunchKernelGGL((pf_gemm_kernel<EPI, TPW, NG, WV, 1>), grid, dim3(64 * WV), 0, s, a);
    return hipGetLastError();
}

hipError_t pf_launch_gemm(int epi, const PfGemm& a, int splits, hipStream_t s) {
    if (splits < 1 || splits > kPfSplitMax || splits > a.nkb || (epi != PF_PART && splits != 1) ||
        (epi == PF_PART && a.n > kPfChunk))
        return hipErrorInvalidValue;
#define MK_PF_SHAPE(E) kGemmShape[E].tpw, kGemmShape[E].ng, kGemmShape[E].wv
    switch (epi) {
        case PF_PART: return launch_gemm_shape<PF_PART, MK_PF_SHAPE(PF_PART)>(a, splits, s);
        case PF_QKV: return launch_gemm_shape<PF_QKV, MK_PF_SHAPE(PF_QKV)>(a, splits, s);
        case PF_GU: return launch_gemm_shape<PF_GU, MK_PF_SHAPE(PF_GU)>(a, splits, s);
        default: return launch_gemm_shape<PF_LM, MK_PF_SHAPE(PF_LM)>(a, splits, s);
    }
#undef MK_PF_SHAPE
}

hipError_t pf_launch_rows(const PfRows& a, hipStream_t s) {
    if (a.d % 32 != 0 || a.n > 16 * a.n_groups || a.S < 0 || a.S > kPfSplitMax || !a.gains) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pf_rows_kernel, dim3(16 * a.n_groups), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t pf_launch_attn(int dh, const PfAttn& a, hipStream_t s) {
    const dim3 grid(((a.n + 15) / 16) * a.Hq);
    if (dh == 128) hipLaunchKernelGGL(pf_attn_kernel<128>, grid, dim3(512), 0, s, a);
    else hipLaunchKernelGGL(pf_attn_kernel<64>, grid, dim3(512), 0, s, a);
    return hipGetLastError();
}

hipError_t pf_launch_sample(const float* logits, int V, float T, uint64_t seed, uint32_t step, int b, int32_t* token_out,
                            float* logits_out, hipStream_t s) {
    hipLaunchKernelGGL(pf_sample_kernel, dim3(1), dim3(1024), 0, s, logits, V, T, seed, step, b, token_out, logits_out);
    return hipGetLastError();
}

}  // namespace mk
