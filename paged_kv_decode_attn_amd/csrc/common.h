// Device and host helpers shared by the libpkd kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pkd.h"

namespace pkd {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

constexpr int kWave = 64;
constexpr int kPage = 32;

// ------------------------------------------------------------------ formats
// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
// f32 -> bf16, round to nearest even, NaN kept quiet, overflow to infinity
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned f32_to_bf16_bits(float f) {
  const bf16x2_t v = {(__bf16)f, (__bf16)0.0f};
  return __builtin_bit_cast(unsigned, v) & 0xffffu;
}
__device__ __forceinline__ float bf16_bits_to_f32(unsigned b) { return __uint_as_float(b << 16); }
// Two bf16 packed in one dword: low half element 0, high half element 1.
__device__ __forceinline__ float bf16lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ unsigned pack_bf16(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
}

// Two E4M3 codes (bytes 0/1 of `w` when hi = false, bytes 2/3 when true) -> floats.
__device__ __forceinline__ f32x2_t fp8x2_to_f32(unsigned w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true) : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}
// Four E4M3 codes -> two dwords of bf16 (exact: every E4M3 value is a bf16 value).
// One gfx950 scaled conversion per pair, scale 1; over all 65,536 code pairs
// in both halves of a dword it gives the same bits, NaN payloads included, as
// widening to f32 and keeping the upper halves (checked on the card).
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(unsigned w) {
  u32x2 r;
  r.x = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  r.y = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
  return r;
}
// Clamps to the E4M3 range, keeping NaN (the hardware conversion does not saturate).
__device__ __forceinline__ float sat448(float x) {
  return (x != x) ? x : fminf(fmaxf(x, -448.0f), 448.0f);
}
// Two floats -> two E4M3 codes (RNE, saturating) in the low 16 bits.
__device__ __forceinline__ unsigned f32x2_to_fp8x2(float a, float b) {
  return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false) & 0xffffu;
}

// ------------------------------------------------------------------ wave ops
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Exchanges across 16 and 32 lanes in registers (gfx950 lane swaps): with
// both operands x, the two results hold x of this lane and of lane l ^ 16
// (l ^ 32), in an order that depends on the lane, so a max or a sum of the
// two equals the same operation on (x[l], x[l ^ d]) bit for bit.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Butterfly sum over the 64 lanes: every lane ends with the same value, formed by
// the same fixed tree for every call (pairs at distance 32, 16, ..., 1).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

// ------------------------------------------------------------------ LDS staging
// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left unconstrained).
#define PKD_VMCNT(n) (0x0F70 | ((n) & 0xF) | (((n) & 0x30) << 10))

// Raw buffer view of `bytes` bytes at `base`: loads past num_records bytes
// (checked per dword, SGPR offset included) return zeros instead of touching
// memory (the GEMM tiles that overhang the last weight or activation row are
// filled this way).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_view(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// One 16-byte-per-lane load from a buffer view straight into LDS: lane l's
// 16 bytes (at voff + soff) land at lds + 16 l (lds is wave-uniform).  The
// host compilation pass never sees the device builtin.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint8_t* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, (int)voff, (int)soff, 0, 0);
#else
  (void)r;
  (void)voff;
  (void)soff;
  (void)lds;
#endif
}

// Workgroup barrier that no memory access may cross in either direction (the
// compiler cannot see the LDS writes of the direct loads, so an intrinsic
// barrier alone would let it hoist LDS reads above it).  It waits for nothing
// by itself: the vmcnt / lgkmcnt waits around it are explicit.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------------ sticky errors
enum : unsigned { kErrSeq = 1u, kErrPos = 2u, kErrPage = 4u };

}  // namespace pkd

// ------------------------------------------------------------------ host side
struct pkd_pool {
  pkd_pool_desc desc;
  uint8_t* base;
  size_t bytes;
  pkd_pool_info info;
  int device;
  int32_t* page_refs;    // host: sequences whose block table lists each physical page
  int64_t shared_pages;  // pages listed by two or more sequences
  int32_t* host_table;   // host copy of the block tables [max_seqs][max_pages_per_seq] (-1 unset)
  int32_t* host_counts;  // host copy of the page counts [max_seqs]
};

namespace pkd {

size_t align256(size_t x);
pkd_status fail(pkd_error* err, pkd_status code, int64_t needed, int64_t available, const char* fmt, ...);
pkd_status ok(pkd_error* err);
pkd_status check_launch(pkd_error* err, const char* what);
int elem_size(int dtype);

// Attention launch used by paged_attn_decode and decode_step.
struct AttnArgs {
  const pkd_pool* pool;
  const int32_t* seq;
  const int32_t* pos;
  int32_t n_rows;
  int32_t n_q_heads;
  const void* q;
  int64_t q_stride;  // elements between rows
  const void* k_new;
  const void* v_new;
  int64_t kv_new_stride;
  void* out;
  int32_t out_dtype;
  int64_t out_stride;
  int32_t distinct;  // no sequence has two rows: the append may run inside attention
};
size_t attn_workspace_bytes(const pkd_pool* pool, int32_t n_q_heads, int32_t max_rows);
pkd_status attn_launch(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t stream, pkd_error* err);

// The tiled matrix-core families (large batches, K splits, workspace).
inline bool tiled_family(int f) { return f == PKD_FAMILY_MFMA || f == PKD_FAMILY_MFMA_FP8; }

// Projection launch used by gemv_rows and decode_step.
// Projection input code used inside the library only (next to PKD_F32 and
// PKD_BF16): f32 storage, each value rounded to bf16 (RNE) as the vector GEMV
// loads it, which gives the same products as rounding it in a pass of its own.
constexpr int32_t kXF32AsBf16 = 3;

struct ProjArgs {
  const pkd_matrix* W;
  const void* x;
  int32_t x_dtype;
  int32_t n_rows;
  void* y;
  int32_t out_dtype;
  const float* residual;
  int32_t silu_pair;
  void* y_bf16;
  const float* row_scale;  // [n_rows] factor on every output of the row, or null
  const float* rope_cs;    // [n_rows][rope_hd / 2] (cos, sin), or null
  int32_t rope_cols;       // outputs [0, rope_cols) are rotated in consecutive pairs
  int32_t rope_hd;
};
size_t proj_workspace_bytes(const pkd_matrix* W, int32_t max_rows);
int suggest_k_splits(int rows, int cols, int family, int typical_rows);
pkd_status proj_validate(const ProjArgs& a, pkd_error* err);
pkd_status proj_launch(const ProjArgs& a, void* ws, size_t ws_bytes, hipStream_t stream, pkd_error* err);
pkd_status gemv_gather_launch(const pkd_matrix& W, const void* x, int32_t x_dtype, int32_t n_rows,
                              const int32_t* cand, const int32_t* n_cand, int32_t max_cand, float* y,
                              hipStream_t stream, pkd_error* err);

// Elementwise f32 -> bf16 rounding of n values (projection inputs).
pkd_status cast_bf16_launch(const float* x, void* y, int64_t n, hipStream_t stream, pkd_error* err);

// Per-row RMSNorm factor 1 / sqrt(mean(x^2) + eps) (and optionally the bf16
// rounding of the row), and the rotary-position table of a set of rows.
pkd_status rms_factor_launch(const float* x, int32_t n_rows, int32_t cols, float eps, float* inv_rms,
                             void* x_bf16, hipStream_t stream, pkd_error* err);
pkd_status rope_table_launch(const int32_t* pos, int32_t n_rows, int32_t head_dim, float base, float* cs,
                             hipStream_t stream, pkd_error* err);

// Rotary positions on the consecutive output pair (v0, v1) at column n (even)
// of activation row m, from the row's (cos, sin) table.  Written with explicit
// fused multiply-adds so that every kernel that calls it rounds alike.
__device__ __forceinline__ void rope_pair(const float* cs, int hd, int m, int n, float& v0, float& v1) {
  const float* t = cs + ((int64_t)m * (hd / 2) + (n % hd) / 2) * 2;
  const float c = t[0], sn = t[1], a = v0, b = v1;
  v0 = fmaf(a, c, -(b * sn));
  v1 = fmaf(a, sn, b * c);
}

}  // namespace pkd
