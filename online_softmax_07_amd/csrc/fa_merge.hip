// LSE merge of normalized partial results (page "Attention kernel chains", chain "The
// log-sum-exp merge"): lse = ln sum_s e^{lse_s}, O = sum_s e^{lse_s - lse} O_s, evaluated
// against m* = max_s lse_s.
//
// One workgroup (4 waves) per output row.  The merge is tiny and latency-bound, so it is
// arranged as a single round trip to memory: each wave issues the loads of its partial
// rows (every fourth split, lanes across the head dimension) together with the lse values
// (one per lane), then every wave reduces m* and sum_s e^{lse_s - m*} in registers, weighs
// its partial rows, and the four sums meet in LDS.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kMergeWaves = 4;
constexpr int kMergeMaxPerLane = 8;  // d <= 512
constexpr int kMergeBatch = 8;       // partial rows per wave per round of loads

template <typename OutT>
__global__ __launch_bounds__(64 * kMergeWaves) void lse_merge_kernel(
    const float* __restrict__ O_part, const float* __restrict__ LSE_part, OutT* __restrict__ O,
    float* __restrict__ LSE, int ns, int rows, int d) {
  __shared__ float red[kMergeWaves][64 * kMergeMaxPerLane];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nper = (d + 63) / 64;   // columns per lane

  // this wave's first batch of partial rows (independent of the lse values)
  float v[kMergeBatch][kMergeMaxPerLane];
  float ls[kMergeBatch];
#pragma unroll
  for (int u = 0; u < kMergeBatch; ++u) {
    const int s = wave + kMergeWaves * u;
    const bool ok = s < ns;
    const int sc = ok ? s : 0;
    ls[u] = ok ? LSE_part[(size_t)sc * rows + row] : kNegInf;
    const float* Op = O_part + ((size_t)sc * rows + row) * d;
#pragma unroll
    for (int i = 0; i < kMergeMaxPerLane; ++i) {
      const int c = lane + 64 * i;
      v[u][i] = (ok && i < nper && c < d) ? Op[c] : 0.f;
    }
  }

  // m* and sum_s e^{lse_s - m*} over all splits (each lane holds every 64th lse; the first
  // one stays in a register, so up to 64 splits need a single load per lane)
  const float ls0 = lane < ns ? LSE_part[(size_t)lane * rows + row] : kNegInf;
  float mx = ls0;
  for (int s = lane + 64; s < ns; s += 64) mx = fmaxf(mx, LSE_part[(size_t)s * rows + row]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, shfl_xor_f(mx, off));
  float sum = 0.f;
  if (mx != kNegInf) {
    sum = exp2f_hw((ls0 - mx) * kLog2e);
    for (int s = lane + 64; s < ns; s += 64) sum += exp2f_hw((LSE_part[(size_t)s * rows + row] - mx) * kLog2e);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += shfl_xor_f(sum, off);
  const float lse = mx == kNegInf ? kNegInf : mx + log2f_hw(sum) * kLn2;

  float acc[kMergeMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMergeMaxPerLane; ++i) acc[i] = 0.f;
  if (lse != kNegInf) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float w = exp2f_hw((ls[u] - lse) * kLog2e);  // e^{lse_s - lse}; 0 for -inf or absent
#pragma unroll
      for (int i = 0; i < kMergeMaxPerLane; ++i) acc[i] = __builtin_fmaf(w, v[u][i], acc[i]);
    }
    // further batches (more than kMergeWaves * kMergeBatch splits), each again issued as
    // one round of loads before its weights are applied
    for (int s0 = wave + kMergeWaves * kMergeBatch; s0 < ns; s0 += kMergeWaves * kMergeBatch) {
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const int s = s0 + kMergeWaves * u;
        const bool ok = s < ns;
        const int sc = ok ? s : 0;
        ls[u] = ok ? LSE_part[(size_t)sc * rows + row] : kNegInf;
        const float* Op = O_part + ((size_t)sc * rows + row) * d;
#pragma unroll
        for (int i = 0; i < kMergeMaxPerLane; ++i) {
          const int c = lane + 64 * i;
          v[u][i] = (ok && i < nper && c < d) ? Op[c] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < kMergeBatch; ++u) {
        const float w = exp2f_hw((ls[u] - lse) * kLog2e);
#pragma unroll
        for (int i = 0; i < kMergeMaxPerLane; ++i) acc[i] = __builtin_fmaf(w, v[u][i], acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kMergeMaxPerLane; ++i) red[wave][lane + 64 * i] = acc[i];
  __syncthreads();
  OutT* Orow = O + (size_t)row * d;
  for (int c = threadIdx.x; c < d; c += 64 * kMergeWaves) {
    float val = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) val += red[w][c];
    Orow[c] = (OutT)val;   // a row no partial saw stays 0
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
