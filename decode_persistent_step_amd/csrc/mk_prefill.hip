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
//     (x = hi + lo, about 16 significant bits, as in the decode path);
//   - attention: one wave per (16-token tile, query head), an online softmax
//     over the K/V pages in their matrix-core page order (K . Q^T on
//     16x16x32, V^T . P^T on 16x16x16, whose B operand is the score
//     accumulator's own lane layout), causal and windowed by position;
//   - chunks of up to kPfChunk tokens are independent except through the
//     pool: a chunk's attention reads the keys and values earlier chunks (and
//     earlier prompts or decode steps) wrote.
#include "mk_device.h"
#include "mk_params.h"
#include "mk_prefill.h"

namespace mk {

// One 2 KB operand block per (16-token group g, 32-k block kb): bytes
// [0, 1024) the hi parts, [1024, 2048) the lo parts; lane l's 16 bytes hold
// token 16 g + l % 16 at k = 32 kb + 8 (l / 16) + e, e = 0..7.
constexpr int kBlk = 2048;

__device__ __forceinline__ void latch(uint32_t* err, uint32_t code, uint32_t where) {
    if (atomicCAS(err, 0u, code) == 0u) __hip_atomic_store(err + 1, where, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// X[i][:] = fp32(E[tokens[i]]); an out-of-range token gives a zero row and latches MK_ERR_BAD_PAGE.
__global__ void pf_embed_kernel(const int32_t* tokens, int n, const uint16_t* embed, int d, int V, float* X,
                                uint32_t* err) {
    const int i = blockIdx.x;
    if (i >= n) return;
    int tok = tokens[i];
    const bool ok = tok >= 0 && tok < V;
    if (!ok && threadIdx.x == 0) latch(err, 5u, (uint32_t)i);
    for (int k = threadIdx.x; k < d; k += blockDim.x) X[(int64_t)i * d + k] = ok ? bf16_to_f(embed[(int64_t)tok * d + k]) : 0.f;
}

// rs[i] = 1 / sqrt(mean(X[i]^2) + eps), one wave per row.
__global__ void pf_rms_kernel(const float* X, int n, int K, int ldx, float eps, float* rs) {
    const int i = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
    if (i >= n) return;
    const int lane = threadIdx.x & 63;
    float ss = 0.f;
    for (int k = lane; k < K; k += 64) {
        const float x = X[(int64_t)i * ldx + k];
        ss += x * x;
    }
    for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m, 64);
    if (lane == 0) rs[i] = 1.0f / sqrtf(ss / (float)K + eps);
}

// Operand blocks of rows [0, n) of X [*][ldx] (K columns), each value times
// rs[row] and gains[k] when given; rows n .. 16 n_groups - 1 are zero. (The
// GEMMs take the RMSNorm scale in their epilogue instead: x * gains of an
// embedding row needs at most 16 significant bits, so its hi/lo split is exact.)
__global__ void pf_blocks_kernel(const float* X, int n, int K, int ldx, const float* rs, const uint16_t* gains,
                                 uint8_t* out, int n_groups) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int nkb = K / 32;
    if (idx >= (int64_t)n_groups * nkb * 64) return;
    const int lane = (int)(idx % 64);
    const int64_t gk = idx / 64;
    const int kb = (int)(gk % nkb), g = (int)(gk / nkb);
    const int tok = 16 * g + (lane & 15), k0 = 32 * kb + 8 * (lane >> 4);
    float x[8];
    const float r = (rs && tok < n) ? rs[tok] : 1.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float v = tok < n ? X[(int64_t)tok * ldx + k0 + e] * r : 0.f;
        if (gains) v *= bf16_to_f(gains[k0 + e]);
        x[e] = v;
    }
    uint32_t h2[4], l2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h2[e] = cvt_bf16x2(x[2 * e], x[2 * e + 1]);
        l2[e] = cvt_bf16x2(x[2 * e] - bf_lo(h2[e]), x[2 * e + 1] - bf_hi(h2[e]));
    }
    uint8_t* blk = out + gk * kBlk;
    *reinterpret_cast<v4u*>(blk + lane * 16) = (v4u){h2[0], h2[1], h2[2], h2[3]};
    *reinterpret_cast<v4u*>(blk + 1024 + lane * 16) = (v4u){l2[0], l2[1], l2[2], l2[3]};
}

// out tiles [4 bx, 4 bx + 4) (one per wave) x token groups [8 by, 8 by + 8):
// per 32-k step the workgroup's eight operand blocks go global -> LDS by DMA
// (double buffered); each wave keeps its tile's weight chunk in registers and
// runs two MFMAs (hi and lo parts) per token group.
template <int EPI>
__global__ void __launch_bounds__(256, 1) pf_gemm_kernel(const PfGemm a) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[2][8][kBlk];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t = 4 * blockIdx.x + w;          // this wave's tile
    const int g0 = 8 * blockIdx.y;             // first token group
    const uint32_t lane16 = (uint32_t)lane * 16u;
    const __amdgpu_buffer_rsrc_t rx = rsrc_n(a.x, (uint32_t)((int64_t)a.n_groups * a.nkb * kBlk));
    const __amdgpu_buffer_rsrc_t rw = rsrc_n(a.w, (uint32_t)((int64_t)a.T * a.nkb * 1024));
    // wave w moves groups 2w, 2w + 1 (hi and lo) of each step
    auto issue = [&](int kb, int s) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int gi = 2 * w + q, g = g0 + gi;
            const uint32_t off = g < a.n_groups ? (uint32_t)((int64_t)(g * a.nkb + kb) * kBlk) : kOOB;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                dma_chunk(rx, (__attribute__((address_space(3))) uint8_t*)&stage[s][gi][h * 1024],
                          off == kOOB ? kOOB : off + h * 1024u + lane16);
        }
    };
    v4f acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = (v4f){0.f, 0.f, 0.f, 0.f};
    issue(0, 0);
    v4u wc = ld_chunk(rw, t < a.T ? (uint32_t)t * a.nkb * 1024u : kOOB, lane16);
    for (int kb = 0; kb < a.nkb; ++kb) {
        const int s = kb & 1;
        wait_vm<0>();                          // this wave's DMAs of step kb and its weight chunk
        __syncthreads();                       // every wave's; and step kb - 1 is done with the other buffer
        const v4u wk = wc;
        if (kb + 1 < a.nkb) {
            issue(kb + 1, s ^ 1);
            wc = ld_chunk(rw, t < a.T ? (uint32_t)(t * a.nkb + kb + 1) * 1024u : kOOB, lane16);
        }
        if (t < a.T) {
#pragma unroll
            for (int gi = 0; gi < 8; ++gi) {
                const v4u bh = *reinterpret_cast<const v4u*>(&stage[s][gi][lane16]);
                const v4u bl = *reinterpret_cast<const v4u*>(&stage[s][gi][1024 + lane16]);
                acc[gi] = mfma16x16x32(wk, bh, acc[gi]);
                acc[gi] = mfma16x16x32(wk, bl, acc[gi]);
            }
        }
    }
    if (t >= a.T) return;
    // D: lane l holds token 16 g + l % 16, rows 4 (l / 16) + j of the tile
    const int r0 = 4 * (lane >> 4);
#pragma unroll
    for (int gi = 0; gi < 8; ++gi) {
        const int tok = 16 * (g0 + gi) + (lane & 15);
        const bool live = tok < a.n;
        if (a.rs && live) acc[gi] *= a.rs[tok];  // RMSNorm scale after the product (operand x * gains)
        if constexpr (EPI == PF_RES) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * t + r0 + j;
                if (live && row < a.ldo) a.out[(int64_t)tok * a.ldo + row] = a.res[(int64_t)tok * a.ldo + row] + acc[gi][j];
            }
        } else if constexpr (EPI == PF_LM) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = 16 * t + r0 + j;
                if (tok == a.n - 1 && row < a.ldo) a.out[row] = acc[gi][j];
            }
        } else {
            // rows r and r + 8 of a tile pair up (RoPE halves, or gate and up):
            // lanes 0..31 hold rows 0..7, lanes 32..63 rows 8..15 of the same tokens
            float part[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) part[j] = __shfl_xor(acc[gi][j], 32, 64);
            if (lane < 32 && live) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = r0 + j;  // 0..7
                    const float y0 = acc[gi][j], y1 = part[j];
                    if constexpr (EPI == PF_GU) {
                        const int f = 8 * t + r;
                        a.act[(int64_t)tok * a.F + f] = y0 / (1.0f + __expf(-y0)) * y1;
                    } else {
                        const int head = 16 * t / a.dh, i = 8 * ((16 * t % a.dh) / 16) + r;  // pair (i, i + dh/2)
                        const int p = a.pos0 + tok;
                        float v0 = y0, v1 = y1;
                        if (head < a.Hq + a.Hkv) {
                            const float2 cs = reinterpret_cast<const float2*>(a.rope)[(int64_t)p * (a.dh / 2) + i];
                            v0 = y0 * cs.x - y1 * cs.y;
                            v1 = y0 * cs.y + y1 * cs.x;
                        }
                        if (head < a.Hq) {
                            a.q[(int64_t)tok * a.Hq * a.dh + head * a.dh + i] = v0;
                            a.q[(int64_t)tok * a.Hq * a.dh + head * a.dh + i + a.dh / 2] = v1;
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
                                    blk[isv ? kv_elem_v<128>(sl, i) : kv_elem_k<128>(sl, i)] = h0;
                                    blk[isv ? kv_elem_v<128>(sl, i + 64) : kv_elem_k<128>(sl, i + 64)] = h1;
                                } else {
                                    blk[isv ? kv_elem_v<64>(sl, i) : kv_elem_k<64>(sl, i)] = h0;
                                    blk[isv ? kv_elem_v<64>(sl, i + 32) : kv_elem_k<64>(sl, i + 32)] = h1;
                                }
                            }
                        }
                    }
                }
            }
        }
    }
}

// One wave per (16-token group blockIdx.x, query head 4 blockIdx.y + wave):
// causal (and windowed) attention of the group's tokens over the pool pages.
// Token column c = lane % 16 is position pos0 + 16 g + c; it attends to keys
// [lo, that position] (lo = max(0, position - win + 1) for a window, else 0).
template <int DH>
__global__ void __launch_bounds__(256, 1) pf_attn_kernel(const PfAttn a) {
    constexpr int CPP = DH / 32;   // K chunks per page
    constexpr int NJB = DH / 16;   // V dim blocks
    const int lane = threadIdx.x & 63;
    const int h = 4 * blockIdx.y + (threadIdx.x >> 6);
    if (h >= a.Hq) return;
    const int G = a.Hq / a.Hkv, kvh = h / G, g = blockIdx.x;
    const int col = lane & 15, rg = lane >> 4;
    const int ti = 16 * g + col;
    const bool tok_ok = ti < a.n;
    const int p_tok = a.pos0 + ti;
    const int lo_tok = a.win > 0 ? max(0, p_tok - a.win + 1) : 0;
    const int pmin = a.pos0 + 16 * g, pmax = a.pos0 + min(16 * g + 15, a.n - 1);
    const int lo_min = a.win > 0 ? max(0, pmin - a.win + 1) : 0;
    // q of this column's token, times log2 e / sqrt(dh), as hi and lo B operands
    const float scale = 1.4426950408889634f / sqrtf((float)DH);
    v4u qh[CPP], ql[CPP];
#pragma unroll
    for (int j = 0; j < CPP; ++j) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = tok_ok ? a.q[(int64_t)ti * a.Hq * DH + h * DH + 32 * j + 8 * rg + e] * scale : 0.f;
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
    for (int P = lo_min / kPage; P <= pmax / kPage; ++P) {
        const int pid = a.pages[P];
        if (pid < 0 || pid >= a.n_pages) {
            if (lane == 0) latch(a.err, 5u, (uint32_t)P);
            continue;
        }
        const int64_t blk = ((int64_t)pid * a.Hkv + kvh) * kPage * DH;
        v4u kw[CPP];
        v2u vw[NJB];
#pragma unroll
        for (int j = 0; j < CPP; ++j) kw[j] = *reinterpret_cast<const v4u*>(a.kpool + blk + j * 512 + lane * 8);
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) vw[jb] = *reinterpret_cast<const v2u*>(a.vpool + blk + jb * 256 + lane * 4);
        // V rows outside [lo_min, pmax] were not written for these tokens: zero them
        // (their weights are 0, their bits need not be finite)
        uint32_t mk2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const int q0 = P * kPage + 4 * rg + 2 * hh;
            mk2[hh] = ((q0 >= lo_min && q0 <= pmax) ? 0x0000FFFFu : 0u) | ((q0 + 1 >= lo_min && q0 + 1 <= pmax) ? 0xFFFF0000u : 0u);
        }
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) vw[jb] = (v2u){vw[jb].x & mk2[0], vw[jb].y & mk2[1]};
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
            o[jb] = mfma16x16x16(vw[jb], bh, o[jb]);
            o[jb] = mfma16x16x16(vw[jb], bl, o[jb]);
        }
    }
    const float lt = sum_xor32(sum_xor16(lsum));
    if (!tok_ok || !(lt > 0.f)) return;
    const float inv = 1.0f / lt;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
        for (int i = 0; i < 4; ++i) a.o[(int64_t)ti * a.Hq * DH + h * DH + 16 * jb + 4 * rg + i] = o[jb][i] * inv;
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
#include <hip/hip_runtime.h>

namespace mk {

hipError_t pf_launch_embed(const int32_t* tokens, int n, const uint16_t* embed, int d, int V, float* X, uint32_t* err,
                           hipStream_t s) {
    hipLaunchKernelGGL(pf_embed_kernel, dim3(n), dim3(256), 0, s, tokens, n, embed, d, V, X, err);
    return hipGetLastError();
}

hipError_t pf_launch_rms(const float* X, int n, int K, int ldx, float eps, float* rs, hipStream_t s) {
    hipLaunchKernelGGL(pf_rms_kernel, dim3((n + 3) / 4), dim3(256), 0, s, X, n, K, ldx, eps, rs);
    return hipGetLastError();
}

hipError_t pf_launch_blocks(const float* X, int n, int K, int ldx, const float* rs, const uint16_t* gains, uint8_t* out,
                            hipStream_t s) {
    const int n_groups = (n + 15) / 16;
    const int64_t total = (int64_t)n_groups * (K / 32) * 64;
    hipLaunchKernelGGL(pf_blocks_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, X, n, K, ldx, rs, gains,
                       out, n_groups);
    return hipGetLastError();
}

hipError_t pf_launch_gemm(int epi, const PfGemm& a, hipStream_t s) {
    const dim3 grid((a.T + 3) / 4, (a.n_groups + 7) / 8);
    switch (epi) {
        case PF_RES: hipLaunchKernelGGL(pf_gemm_kernel<PF_RES>, grid, dim3(256), 0, s, a); break;
        case PF_QKV: hipLaunchKernelGGL(pf_gemm_kernel<PF_QKV>, grid, dim3(256), 0, s, a); break;
        case PF_GU: hipLaunchKernelGGL(pf_gemm_kernel<PF_GU>, grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL(pf_gemm_kernel<PF_LM>, grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t pf_launch_attn(int dh, const PfAttn& a, hipStream_t s) {
    const dim3 grid((a.n + 15) / 16, (a.Hq + 3) / 4);
    if (dh == 128) hipLaunchKernelGGL(pf_attn_kernel<128>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(pf_attn_kernel<64>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t pf_launch_sample(const float* logits, int V, float T, uint64_t seed, uint32_t step, int b, int32_t* token_out,
                            float* logits_out, hipStream_t s) {
    hipLaunchKernelGGL(pf_sample_kernel, dim3(1), dim3(1024), 0, s, logits, V, T, seed, step, b, token_out, logits_out);
    return hipGetLastError();
}

}  // namespace mk
