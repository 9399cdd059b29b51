// mk_device.h - device helpers for the gfx950 decode kernel.
//
// Cross-workgroup data on MI355X: each XCD has its own L2, so data that one
// workgroup publishes for another is written and read with the "sc1" cache
// policy (coherent at agent scope, no L2 writeback/invalidate needed). The
// data are tagged words (below); flags, where used, only tell a reader when to
// start looking. Weight and K/V streams use non-temporal loads (they are read
// once per step).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kCachePolicySC1 = 16;  // buffer cache-policy bits: sc1 (agent-coherent)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
    // raw buffer: stride 0, num_records = 2^31-1 bytes from base, default data format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}

// ---------------------------------------------------------------- coherent I/O
__device__ __forceinline__ v4u ld_sc1_v4(const void* base, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), byte_off, 0, kCachePolicySC1);
}
__device__ __forceinline__ void st_sc1_v4(void* base, uint32_t byte_off, v4u v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(base), byte_off, 0, kCachePolicySC1);
}
__device__ __forceinline__ float ld_sc1_f(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc1_f(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_sc1_u(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_sc1_i(const int32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc1_u(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_sc1_i(int32_t* p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every vector memory operation this wave issued has completed
// (its stores are visible at agent scope).
// s_waitcnt encoding (gfx9): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14].
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// ---------------------------------------------------------------- tagged words
// Activations exchanged between workgroups travel as 64-bit words: the value's
// 32 bits in the low half, a tag unique to (launch, stage) in the high half.
// An aligned 8-byte store is seen whole or not at all, so a reader that checks
// the tag knows the value is current without any ordering between the data
// and a separate flag.
typedef unsigned v2u __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_tag(uint64_t* base, uint32_t idx, uint32_t bits, uint32_t tag) {
    const v2u w = {bits, tag};
    __builtin_amdgcn_raw_buffer_store_b64(w, rsrc(base), idx * 8u, 0, kCachePolicySC1);
}
__device__ __forceinline__ void st_tag_f(uint64_t* base, uint32_t idx, float v, uint32_t tag) {
    st_tag(base, idx, __float_as_uint(v), tag);
}
// Words idx and idx + 1 (idx even): (value0, tag0, value1, tag1).
__device__ __forceinline__ v4u ld_tag2(const uint64_t* base, uint32_t idx) {
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc(base), idx * 8u, 0, kCachePolicySC1);
}
__device__ __forceinline__ bool tags_ok(v4u w, uint32_t tag) { return w.y == tag && w.w == tag; }
// The value half of word idx, for a reader that has already seen it current.
__device__ __forceinline__ float ld_tag_value(const uint64_t* base, uint32_t idx) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(base), idx * 8u, 0, kCachePolicySC1));
}

// Streamed (read-once) 16-byte load.
__device__ __forceinline__ v4u ld_stream(const v4u* p) { return __builtin_nontemporal_load(p); }

// ----------------------------------------------------------------------- bf16
__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// Round-to-nearest-even fp32 -> bf16 (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ------------------------------------------------------------ lane exchanges
// x from lane l ^ 16 (within each half-wave), through the LDS crossbar.
__device__ __forceinline__ float xor16(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));  // SWAP,16
}
// x_l + x_{l^8}: ds_swizzle SWAP,8
__device__ __forceinline__ float xor8(float x) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x201F));
}
// x from lane l ^ 8 inside each 16-lane row (DPP row_ror:8, no LDS).
__device__ __forceinline__ float dpp_xor8(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xf, 0xf, false));
}
// Sums and maxima of x_l and x_{l^16} / x_{l^32} with the gfx950 VALU lane swaps
// (v_permlane16_swap, v_permlane32_swap): with both operands x, lane l receives
// the pair (x[l & ~m], x[l | m]) for m = 16 (inside each half-wave) or m = 32.
__device__ __forceinline__ float sum_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor_shfl(float x, int m) { return __shfl_xor(x, m, 64); }
// x from lane l ^ 1, l ^ 2 (DPP quad permutations), from lane 7 - l within each
// 8-lane half row and from lane 15 - l within each 16-lane row (DPP mirrors):
// register-to-register moves, without the LDS crossbar round trip of a
// ds_bpermute-based shuffle.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum and maximum over the 64 lanes, every lane getting the same bits: inside
// each 16-lane row the partners are paired symmetrically (xor 1, xor 2, half
// mirror, mirror), so both lanes of a pair add the same two values; then the
// lane swaps across rows.
__device__ __forceinline__ float wave_sum_f(float x) {
    x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_f<0x141>(x);  // row_half_mirror
    x += dpp_f<0x140>(x);  // row_mirror
    return sum_xor32(sum_xor16(x));
}
__device__ __forceinline__ float wave_max_f(float x) {
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x141>(x));
    x = fmaxf(x, dpp_f<0x140>(x));
    return max_xor32(max_xor16(x));
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// acc + a.lo * b.lo + a.hi * b.hi over two packed bf16 pairs (v_dot2c_f32_bf16).
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, a), __builtin_bit_cast(v2bf, b), acc, false);
}

constexpr int kCachePolicyNT = 2;    // buffer cache-policy bits: nt (streaming)
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past every range: reads return 0, touch no memory
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_n(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier after this wave's LDS accesses have completed. Unlike
// __syncthreads it does not wait for outstanding global loads: a wave's DMA
// and load stream stays in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
}

// DMA of 16 bytes per lane from buffer `rs` at byte offset `off` (per lane) into
// LDS at `lds_dst` + 16 * lane, streaming cache policy. Completion is tracked by
// vmcnt like any load.
__device__ __forceinline__ void dma_chunk(__amdgpu_buffer_rsrc_t rs, __attribute__((address_space(3))) uint8_t* lds_dst,
                                          uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_dst, 16, off, 0, 0,
                                             kCachePolicyNT);
}

// 16-byte streamed load of lane `lane` of the 1 KB chunk at byte offset `off` (kOOB: zeros).
__device__ __forceinline__ v4u ld_chunk(__amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t lane16) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off + lane16, 0, kCachePolicyNT);
}

// ----------------------------------------------------------------------- MFMA

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16). Lane l holds A row l%16,
// k = 8(l/16)..+7; B column l%16, same k; D column l%16, rows 4(l/16)..+3.
__device__ __forceinline__ v4f mfma16x16x32(v4u a, v4u b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}
// D(16x16 fp32) += A(16x16 bf16) * B(16x16 bf16). Lane l holds A row l%16,
// k = 4(l/16)..+3; B column l%16, same k; D column l%16, rows 4(l/16)..+3.
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4f mfma16x16x16(v2u a, v2u b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(v4s, a), __builtin_bit_cast(v4s, b), c, 0, 0, 0);
}
// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {
    const v2bf r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}

// ------------------------------------------------------------- K/V page order
// Element (position pos, dim) of a (page, kv head) block of 16 positions x DH
// dims, so that each 1 KB chunk is an MFMA operand as it lands:
//   K: chunk j = dims 32j..32j+31; lane 16 ((dim % 32) / 8) + pos holds 8 dims
//      of one position (the 16x16x32 A operand of K . Q^T, rows = positions);
//   V: block jb (512 B) = dims 16jb..16jb+15; lane 16 (pos / 4) + dim % 16 holds
//      4 positions of one dim (the 16x16x16 A operand of V^T . P^T).
template <int DH>
__device__ __forceinline__ int kv_elem_k(int pos, int dim) {
    return (dim >> 5) * 512 + ((((dim & 31) >> 3) << 4) + pos) * 8 + (dim & 7);
}
template <int DH>
__device__ __forceinline__ int kv_elem_v(int pos, int dim) {
    return (dim >> 4) * 256 + (((pos >> 2) << 4) + (dim & 15)) * 4 + (pos & 3);
}

// ----------------------------------------------------------------- timeouts
__device__ __forceinline__ uint64_t rt_clock() { return __builtin_amdgcn_s_memrealtime(); }  // 100 MHz

// Two E4M3 codes (bytes 2 HI, 2 HI + 1 of w4) -> a packed bf16 pair, exactly (an
// E4M3 value has 4 significant bits): v_cvt_pk_f32_fp8 (OCP E4M3 on gfx950).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w4) {
    const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w4, HI);
    return cvt_bf16x2(f[0], f[1]);
}
// Eight codes (two dwords) -> the eight bf16 values of one 16x16x32 operand lane.
__device__ __forceinline__ v4u fp8x8_to_bf16x8(uint32_t a, uint32_t b) {
    return (v4u){fp8x2_to_bf16x2<false>(a), fp8x2_to_bf16x2<true>(a), fp8x2_to_bf16x2<false>(b),
                 fp8x2_to_bf16x2<true>(b)};
}

}  // namespace mk
