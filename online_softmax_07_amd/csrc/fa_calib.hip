// Calibration kernels (include/fa_calib.h): the matrix-core ceiling, the one-pass HBM
// read ceiling in the decode kernel's access pattern, and the shader clock.  Each kernel
// touches only the buffers it is given, with every index bounded by the sizes passed in.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_calib.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaWaves = 8;      // two waves per SIMD, as the prefill kernels run
constexpr int kStreamThreads = 256;

__global__ __launch_bounds__(64 * kMfmaWaves, 1) void mfma_loop_kernel(float* sink, uint64_t* cycles, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)((float)(threadIdx.x & 63) * 0.001f);
    b[i] = (__bf16)((float)i * 0.01f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  // The two waves of a SIMD do not share the matrix core evenly (the older one issues
  // first and finishes early), so the loop is timed from the workgroup's common start to
  // the end of its last wave.
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    cycles[2 * blockIdx.x] = t1 - t0;
    cycles[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// The matrix core and the vector unit sharing a SIMD: the MFMA loop above with `fmas` fp32
// FMAs after each round's four MFMAs, in eight independent chains (FMAS = 0: MFMAs only;
// MFMA = false: the FMAs only).  Comparing the three times shows how much of the vector work
// hides under the matrix work when both come from the same waves, as in the attention loops.
template <bool MFMA, int FMAS>
__global__ __launch_bounds__(64 * kMfmaWaves, 1) void mix_loop_kernel(float* sink, uint64_t* cycles, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)((float)(threadIdx.x & 63) * 0.001f);
    b[i] = (__bf16)((float)i * 0.01f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)threadIdx.x * 0.01f + (float)i;
  const float fa = 0.999f, fb = 0.001f * (float)(blockIdx.x & 7);
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (MFMA) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
#pragma unroll
    for (int f = 0; f < FMAS; ++f) x[f & 7] = __builtin_fmaf(x[f & 7], fa, fb);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  __syncthreads();
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    cycles[2 * blockIdx.x] = t1 - t0;
    cycles[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// Every thread reads items gid, gid + stride, ... < n16 (16 bytes each), two in flight.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ in, size_t n16,
                                                                     float* sink) {
  const size_t stride = (size_t)gridDim.x * kStreamThreads;
  size_t i = (size_t)blockIdx.x * kStreamThreads + threadIdx.x;
  u32x4 acc0 = {0u, 0u, 0u, 0u}, acc1 = acc0;
  for (; i + stride < n16; i += 2 * stride) {
    acc0 ^= __builtin_nontemporal_load(in + i);
    acc1 ^= __builtin_nontemporal_load(in + i + stride);
  }
  if (i < n16) acc0 ^= __builtin_nontemporal_load(in + i);
  acc0 ^= acc1;
  sink[(size_t)blockIdx.x * kStreamThreads + threadIdx.x] = (float)(acc0[0] ^ acc0[1] ^ acc0[2] ^ acc0[3]);
}

__global__ __launch_bounds__(64) void clock_kernel(uint64_t* out, uint64_t spin_ticks) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint64_t r = r0;
  for (int it = 0; it < (1 << 24) && r - r0 < spin_ticks; ++it) r = __builtin_amdgcn_s_memrealtime();
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : 6; }

}  // namespace

extern "C" {

int fa_calib_mfma(float* sink, uint64_t* cycles, int blocks, int iters, void* stream) {
  if (sink == nullptr || cycles == nullptr) return 1;
  if (blocks < 1 || iters < 1) return 2;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(64 * kMfmaWaves), 0, (hipStream_t)stream, sink, cycles,
                     iters);
  return launched();
}

int fa_calib_mfma_valu(float* sink, uint64_t* cycles, int blocks, int iters, int mfma, int fmas, void* stream) {
  if (sink == nullptr || cycles == nullptr) return 1;
  if (blocks < 1 || iters < 1 || (mfma != 0 && mfma != 1) || (fmas != 0 && fmas != 24 && fmas != 48) ||
      (mfma == 0 && fmas == 0))
    return 2;
  auto k = mix_loop_kernel<true, 24>;
  if (mfma && fmas == 0) k = mix_loop_kernel<true, 0>;
  else if (mfma && fmas == 48) k = mix_loop_kernel<true, 48>;
  else if (!mfma && fmas == 24) k = mix_loop_kernel<false, 24>;
  else if (!mfma && fmas == 48) k = mix_loop_kernel<false, 48>;
  hipLaunchKernelGGL(k, dim3(blocks), dim3(64 * kMfmaWaves), 0, (hipStream_t)stream, sink, cycles, iters);
  return launched();
}

int fa_calib_stream_read(const void* buf, size_t bytes, float* sink, int blocks, void* stream) {
  if (buf == nullptr || sink == nullptr) return 1;
  if (bytes < 16 || bytes % 16 != 0 || blocks < 1 || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0) return 2;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kStreamThreads), 0, (hipStream_t)stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return launched();
}

int fa_calib_clock(uint64_t* out, int spin_ticks, void* stream) {
  if (out == nullptr) return 1;
  if (spin_ticks < 1 || spin_ticks > 10000000) return 2;
  hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, out, (uint64_t)spin_ticks);
  return launched();
}

}  // extern "C"
