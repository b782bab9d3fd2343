// LSE merge of normalized partial results (page "Attention kernel chains", chain "The
// log-sum-exp merge"): lse = ln sum_s e^{lse_s}, O = sum_s e^{lse_s - lse} O_s, evaluated
// against m* = max_s lse_s.
//
// One workgroup per output row.  Wave 0 reduces the row's partial lse values; then the
// four waves take every fourth partial each (lanes stride over the head dimension, so
// every partial row is one coalesced read and all of a wave's reads are independent and
// in flight together) and their sums are combined through LDS.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kMergeWaves = 4;
constexpr int kMergeMaxPerLane = 8;  // d <= 512

template <typename OutT>
__global__ __launch_bounds__(64 * kMergeWaves) void lse_merge_kernel(
    const float* __restrict__ O_part, const float* __restrict__ LSE_part, OutT* __restrict__ O,
    float* __restrict__ LSE, int ns, int rows, int d) {
  __shared__ float red[kMergeWaves][64 * kMergeMaxPerLane];
  __shared__ float stat[2];  // m*, lse
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  if (wave == 0) {
    float mx = kNegInf;
    for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, LSE_part[(size_t)s * rows + row]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
    float sum = 0.f;
    if (mx != kNegInf)
      for (int s = lane; s < ns; s += 64) sum += exp2f_hw((LSE_part[(size_t)s * rows + row] - mx) * kLog2e);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += shfl_xor_f(sum, off);
    if (lane == 0) {
      stat[0] = mx;
      stat[1] = mx == kNegInf ? kNegInf : mx + log2f_hw(sum) * kLn2;
    }
  }
  __syncthreads();
  const float lse = stat[1];

  float acc[kMergeMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMergeMaxPerLane; ++i) acc[i] = 0.f;
  if (lse != kNegInf) {
#pragma unroll 4
    for (int s = wave; s < ns; s += kMergeWaves) {
      const float w = exp2f_hw((LSE_part[(size_t)s * rows + row] - lse) * kLog2e);  // e^{lse_s - lse}
      const float* Op = O_part + ((size_t)s * rows + row) * d;
#pragma unroll
      for (int i = 0; i < kMergeMaxPerLane; ++i) {
        const int c = lane + 64 * i;
        if (c < d) acc[i] = __builtin_fmaf(w, Op[c], acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kMergeMaxPerLane; ++i) red[wave][lane + 64 * i] = acc[i];
  __syncthreads();
  OutT* Orow = O + (size_t)row * d;
  for (int c = threadIdx.x; c < d; c += 64 * kMergeWaves) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) v += red[w][c];
    Orow[c] = (OutT)v;   // a row no partial saw stays 0
  }
  if (LSE != nullptr && threadIdx.x == 0) LSE[row] = lse;
}

hipError_t launch_lse_merge(const float* O_part, const float* LSE_part, void* O, float* LSE,
                            int num_splits, int rows, int d, bool out_f32, void* stream) {
  dim3 grid(rows);
  if (out_f32) {
    hipLaunchKernelGGL(lse_merge_kernel<float>, grid, dim3(64 * kMergeWaves), 0, (hipStream_t)stream,
                       O_part, LSE_part, (float*)O, LSE, num_splits, rows, d);
  } else {
    hipLaunchKernelGGL(lse_merge_kernel<__bf16>, grid, dim3(64 * kMergeWaves), 0, (hipStream_t)stream,
                       O_part, LSE_part, (__bf16*)O, LSE, num_splits, rows, d);
  }
  return hipGetLastError();
}

}  // namespace fa
