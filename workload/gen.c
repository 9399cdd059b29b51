/*
 * Seeded synthetic inputs for the small-batch decode step: weights, prefilled
 * K/V, context lengths, page shuffles and initial tokens.
 *
 * This module holds none of the decode arithmetic. It only draws numbers from
 * a counter-based generator so that any tensor, or any slice of one, can be
 * regenerated bit-identically from (seed, tensor id, flat index). Both the
 * oracle and the GPU path receive what it produces as plain inputs.
 *
 * Generator:
 *   SM(z)  = one SplitMix64 output step (Steele, Lea, Flood, "Fast splittable
 *            pseudorandom number generators", OOPSLA 2014; constants as in
 *            Vigna's public-domain splitmix64.c):
 *              z += 0x9E3779B97F4A7C15
 *              z  = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
 *              z  = (z ^ (z >> 27)) * 0x94D049BB133111EB
 *              return z ^ (z >> 31)
 *   h      = SM(SM(seed ^ tensor_id) + index)
 *   s      = sum_{j<4} ((h >> 16 j) & 0xFFFF) - 131070      (Irwin-Hall(4), exact mean 0)
 *   value  = bf16_rne(mean + fp32(s) * c_sigma),   c_sigma = fp32(sigma / sqrt(4 (65536^2 - 1) / 12))
 * with every product and sum rounded to fp32 in that order.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define WL_GOLDEN 0x9E3779B97F4A7C15ULL

uint64_t wl_splitmix64(uint64_t z)
{
    z += WL_GOLDEN;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint16_t wl_f32_to_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    /* inputs here are always finite */
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float wl_sigma_scale(double sigma)
{
    return (float)(sigma / sqrt(4.0 * (65536.0 * 65536.0 - 1.0) / 12.0));
}

/* Irwin-Hall(4) integer draw for (seed, tensor_id, index). */
int32_t wl_draw_ih4(uint64_t seed, uint64_t tensor_id, uint64_t index)
{
    uint64_t h = wl_splitmix64(wl_splitmix64(seed ^ tensor_id) + index);
    int32_t s = 0;
    for (int j = 0; j < 4; ++j) s += (int32_t)((h >> (16 * j)) & 0xFFFFu);
    return s - 131070;
}

/* out[i] = bf16(mean + fp32(s_{index0+i}) * c_sigma) for i < n. */
void wl_fill_normal_bf16(uint16_t *out, int64_t n, uint64_t seed, uint64_t tensor_id,
                         uint64_t index0, double sigma, float mean)
{
    const float c = wl_sigma_scale(sigma);
    const uint64_t key = wl_splitmix64(seed ^ tensor_id);
#pragma omp parallel for schedule(static, 65536)
    for (int64_t i = 0; i < n; ++i) {
        uint64_t h = wl_splitmix64(key + index0 + (uint64_t)i);
        int32_t s = -131070;
        s += (int32_t)(h & 0xFFFFu);
        s += (int32_t)((h >> 16) & 0xFFFFu);
        s += (int32_t)((h >> 32) & 0xFFFFu);
        s += (int32_t)((h >> 48) & 0xFFFFu);
        float v = (float)s * c;
        if (mean != 0.0f) v = mean + v;
        out[i] = wl_f32_to_bf16_rne(v);
    }
}

/* Uniform integer in [0, m): SM(seed + i) mod m. */
uint64_t wl_draw_mod(uint64_t seed, uint64_t i, uint64_t m)
{
    return wl_splitmix64(seed + i) % m;
}

/* In-place Fisher-Yates: for i = n-1 .. 1, j = SM(seed + i) mod (i + 1), swap(a[i], a[j]). */
void wl_shuffle_i32(int32_t *a, int64_t n, uint64_t seed)
{
    for (int64_t i = n - 1; i > 0; --i) {
        int64_t j = (int64_t)(wl_splitmix64(seed + (uint64_t)i) % (uint64_t)(i + 1));
        int32_t t = a[i];
        a[i] = a[j];
        a[j] = t;
    }
}
