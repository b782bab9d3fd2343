// LSE merge of normalized partial results (page "Attention kernel chains", chain "The
// log-sum-exp merge"): lse = ln sum_s e^{lse_s}, O = sum_s e^{lse_s - lse} O_s, evaluated
// against m* = max_s lse_s.  One wave per output row; lanes stride over the head
// dimension, so each partial row is read with coalesced loads.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kMergeRowsPerWG = 4;
constexpr int kMergeMaxPerLane = 8;  // d <= 512

template <typename OutT>
__global__ __launch_bounds__(64 * kMergeRowsPerWG) void lse_merge_kernel(
    const float* __restrict__ O_part, const float* __restrict__ LSE_part, OutT* __restrict__ O,
    float* __restrict__ LSE, int ns, int rows, int d) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMergeRowsPerWG + (threadIdx.x >> 6);
  if (row >= rows) return;

  // m* = max_s lse_s
  float mx = kNegInf;
  for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, LSE_part[(size_t)s * rows + row]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));

  OutT* Orow = O + (size_t)row * d;
  if (mx == kNegInf) {  // no partial saw a key
    for (int c = lane; c < d; c += 64) Orow[c] = (OutT)0.f;
    if (LSE != nullptr && lane == 0) LSE[row] = kNegInf;
    return;
  }
  // sum_s e^{lse_s - m*}
  float sum = 0.f;
  for (int s = lane; s < ns; s += 64) sum += exp2f_hw((LSE_part[(size_t)s * rows + row] - mx) * kLog2e);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += shfl_xor_f(sum, off);
  const float lse = mx + log2f_hw(sum) * kLn2;

  float acc[kMergeMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMergeMaxPerLane; ++i) acc[i] = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = exp2f_hw((LSE_part[(size_t)s * rows + row] - lse) * kLog2e);  // e^{lse_s - lse}
    const float* Op = O_part + ((size_t)s * rows + row) * d;
#pragma unroll
    for (int i = 0; i < kMergeMaxPerLane; ++i) {
      const int c = lane + 64 * i;
      if (c < d) acc[i] = __builtin_fmaf(w, Op[c], acc[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < kMergeMaxPerLane; ++i) {
    const int c = lane + 64 * i;
    if (c < d) Orow[c] = (OutT)acc[i];
  }
  if (LSE != nullptr && lane == 0) LSE[row] = lse;
}

hipError_t launch_lse_merge(const float* O_part, const float* LSE_part, void* O, float* LSE,
                            int num_splits, int rows, int d, bool out_f32, void* stream) {
  dim3 grid((rows + kMergeRowsPerWG - 1) / kMergeRowsPerWG);
  if (out_f32) {
    hipLaunchKernelGGL(lse_merge_kernel<float>, grid, dim3(64 * kMergeRowsPerWG), 0, (hipStream_t)stream,
                       O_part, LSE_part, (float*)O, LSE, num_splits, rows, d);
  } else {
    hipLaunchKernelGGL(lse_merge_kernel<__bf16>, grid, dim3(64 * kMergeRowsPerWG), 0, (hipStream_t)stream,
                       O_part, LSE_part, (__bf16*)O, LSE, num_splits, rows, d);
  }
  return hipGetLastError();
}

}  // namespace fa
