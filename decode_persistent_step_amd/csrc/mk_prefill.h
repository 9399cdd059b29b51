// mk_prefill.h - arguments of the paged-prefill kernels (mk_prefill.hip),
// shared by the kernels and the host runtime.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

constexpr int kPfChunk = 256;  // tokens per prefill chunk (16 token groups)

enum PfEpi { PF_RES = 0, PF_QKV = 1, PF_GU = 2, PF_LM = 3 };

struct PfGemm {
    const uint8_t* w;  // packed tiles: T tiles of nkb 1 KB chunks
    int T, nkb;
    const uint8_t* x;  // operand blocks [n_groups][nkb]
    int n, n_groups;
    float* out;        // PF_RES: out[i][row] = res[i][row] + y; PF_LM: out[row] = y of row n - 1
    int ldo;
    const float* res;
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
    float* act;         // [n][F]
    int F;
};

struct PfAttn {
    const float* q;  // [n][Hq dh] (after RoPE)
    float* o;        // [n][Hq dh]
    const uint16_t *kpool, *vpool;  // this layer's pools
    const int32_t* pages;
    int pos0, n, Hq, Hkv, win, n_pages;
    uint32_t* err;
};

hipError_t pf_launch_embed(const int32_t* tokens, int n, const uint16_t* embed, int d, int V, float* X, uint32_t* err,
                           hipStream_t s);
hipError_t pf_launch_rms(const float* X, int n, int K, int ldx, float eps, float* rs, hipStream_t s);
hipError_t pf_launch_blocks(const float* X, int n, int K, int ldx, const float* rs, const uint16_t* gains, uint8_t* out,
                            hipStream_t s);
hipError_t pf_launch_gemm(int epi, const PfGemm& a, hipStream_t s);
hipError_t pf_launch_attn(int dh, const PfAttn& a, hipStream_t s);
hipError_t pf_launch_sample(const float* logits, int V, float T, uint64_t seed, uint32_t step, int b, int32_t* token_out,
                            float* logits_out, hipStream_t s);

}  // namespace mk
