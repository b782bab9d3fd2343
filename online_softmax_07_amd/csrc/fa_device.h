// Device-side building blocks shared by the gfx950 kernels: vector types, MFMA
// wrappers, base-2 transcendentals and lane exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;   // log2(e): e^x = 2^(x * log2 e)
constexpr float kLn2 = 0.6931471805599453f;     // ln(2):   ln x = log2(x) * ln 2
constexpr float kNegInf = -__builtin_inff();

// 2^x and log2(x) on the hardware transcendental unit (v_exp_f32 / v_log_f32).
// exp2(-inf) = 0, which the masked scores rely on.
__device__ __forceinline__ float exp2f_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2f_hw(float x) { return __builtin_amdgcn_logf(x); }

// D(32x32 f32) += A(32x16 bf16) * B(16x32 bf16).  Lane l holds A row (l % 32) and B
// column (l % 32), each with 8 consecutive k of the k-group (l / 32); D element
// (i, j) sits in lane j + 32 * ((i / 4) % 2), register (i % 4) + 4 * (i / 8).
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16 f32) += A(16x32 bf16) * B(32x16 bf16).  Lane l holds A row (l % 16) and B
// column (l % 16) with 8 k of the k-group (l / 16); D element (i, j) sits in lane
// j + 16 * (i / 4), register i % 4.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Value held by lane (l ^ mask) of the 64-lane wave.
__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

// max(x, x of lane l ^ 32): the two halves of the wave swapped by one v_permlane32_swap.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Pack halves: result = (hi16 of b or lo16 of b) << 16 | (same half of a).
// Used to transpose 4x(8 bf16) row chunks into 8x(4 bf16) column chunks.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ bf16x8 to_bf16x8(f32x8 v) {
  return __builtin_convertvector(v, bf16x8);
}


typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane j
// supplies the address of 4 consecutive 16-bit values; result lane i receives, in slot
// s, value (i % 4) of lane (4 s + i / 4)'s four.  Two such reads fill one 8-element
// MFMA operand whose k index runs across the rows the source lanes point at.
__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<__bf16*>(p)));
}

__device__ __forceinline__ bf16x8 join_bf16x8(s16x4 lo, s16x4 hi) {
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// True in every lane if `pred` holds in any active lane (wave-uniform).
__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Sum of the eight bf16 values of an MFMA operand, accumulated in fp32 (v_dot2c_f32_bf16
// against (1, 1)).  Summing the rounded values the PV product uses keeps numerator and
// denominator of O = sum p V / sum p consistent.
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
  return acc;
}

// Raw buffer access (gfx9 family descriptor).  Loads at byte offsets >= `bytes` return
// zero, which is how tiles running past the end of a sequence are zero-filled without
// any per-element test.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voffset) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voffset, 0, 0));
}

// 16 bytes per lane from a buffer straight into LDS: lane L of the wave writes
// lds_wave_base + 16 L bytes (lds_wave_base must be wave-uniform); lanes whose offset is
// out of the descriptor's range write zeros.  Completion is counted by vmcnt.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t voffset,
                                                  __bf16* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_wave_base, 16,
                                           (int)voffset, 0, 0, 0);
}

// 16 bytes per lane from a global address straight into LDS: lane L of the wave writes
// lds_wave_base + 16 L bytes (lds_wave_base must be wave-uniform); no range check.
__device__ __forceinline__ void global_load16_lds(const void* src, __bf16* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)const_cast<void*>(src),
                                   (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}

// s_waitcnt vmcnt(0): every vector-memory load of this wave (LDS DMAs included) has landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Bytes from element `start` to the end of a range of `n` rows of `row_bytes`, clamped to
// the 32-bit descriptor range.
__device__ __forceinline__ uint32_t range_bytes(long long rows_left, int row_bytes) {
  const long long b = rows_left <= 0 ? 0 : rows_left * (long long)row_bytes;
  return b > 0xffffffffLL ? 0xffffffffu : (uint32_t)b;
}

}  // namespace fa
