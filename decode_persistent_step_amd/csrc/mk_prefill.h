// mk_prefill.h - arguments of the paged-prefill kernels (mk_prefill.hip),
// shared by the kernels and the host runtime.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

constexpr int kPfChunk = 1024;   // tokens per prefill chunk (64 token groups)
constexpr int kPfSplitMax = 8;   // most K splits of a residual GEMM (partial sums [split][kPfChunk][ldo])

// GEMM epilogues: PF_PART writes the split's partial sums (the residual and
// the next norm are applied by pf_launch_rows), PF_QKV applies RoPE and writes
// q and the K/V pages, PF_GU applies SwiGLU and writes the down projection's
// operand blocks, PF_LM writes the last position's logits.
enum PfEpi { PF_PART = 0, PF_QKV = 1, PF_GU = 2, PF_LM = 3 };

struct PfGemm {
    const uint8_t* w;  // packed tiles: T tiles of nkb 1 KB chunks (bf16: 32 K per chunk; FP8: 64 K)
    const float* wscale;  // FP8 weights: the matrix's row scales in packed row order (null: bf16)
    int T, nkb;
    const uint8_t* x;  // operand blocks [n_groups][nkb]
    int n, n_groups;
    float* out;        // PF_PART: out[split][i][row] (i < kPfChunk); PF_LM: out[row] = y of row n - 1
    int ldo;
    const float* rs;    // per-token RMSNorm scale applied to every output (null: none)
    // PF_QKV
    const float* rope;  // [max_pos][dh / 2][cos, sin]
    int pos0, Hq, Hkv, dh;
    float* q;           // [n][Hq dh]
    uint16_t *kpool, *vpool;  // this layer's pools
    const int32_t* pages;
    int n_pages;
    uint32_t* err;
    // PF_GU
    uint8_t* act_blk;   // operand blocks [n_groups][F / 32] of SwiGLU(gate, up)
    int F;
};

struct PfAttn {
    const float* q;  // [n][Hq dh] (after RoPE)
    uint8_t* o_blk;  // operand blocks [n_groups][Hq dh / 32] of the attention output
    const uint16_t *kpool, *vpool;  // this layer's pools
    const int32_t* pages;
    int pos0, n, Hq, Hkv, win, n_pages;
    uint32_t* err;
};

// One residual-stream row per token of a chunk: y = E[tokens[i]] (tokens
// given) or res[i] + sum over splits of part[split][i]; then rs[i] =
// 1/sqrt(mean(y^2) + eps) and the row's operand-block entries of y * gains.
struct PfRows {
    const int32_t* tokens;
    const uint16_t* embed;
    int V;
    const float* part;
    int S;
    float* y;           // [n][d], in place over res
    float* rs;
    const uint16_t* gains;
    uint8_t* blk;       // [n_groups][d / 32]
    int n, n_groups, d;
    float eps;
    uint32_t* err;
};

int pf_splits(int epi, const PfGemm& a);
hipError_t pf_launch_gemm(int epi, const PfGemm& a, int splits, hipStream_t s);
hipError_t pf_launch_rows(const PfRows& a, hipStream_t s);
hipError_t pf_launch_attn(int dh, const PfAttn& a, hipStream_t s);
hipError_t pf_launch_sample(const float* logits, int V, float T, uint64_t seed, uint32_t step, int b, int32_t* token_out,
                            float* logits_out, hipStream_t s);

}  // namespace mk
