// FlashAttention forward in fp32 on the vector ALUs (the fp32 path: fp32 Q/K/V/O).
//
// Same FlashAttention-2 loop order and online-softmax carries as the bf16 MFMA kernel
// (page "Softmax and FlashAttention", "Concept"; page "Kernel visualization: Flash
// Attention 1", "The tiled version"), with a plain schedule: one thread per query row,
// 64 rows per workgroup, K/V tiles of 16 keys staged in LDS and read by every thread
// (broadcast), the row's output accumulated unnormalized in registers and divided once.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kRows32 = 64;   // query rows (= threads) per workgroup
constexpr int kKeys32 = 16;   // keys per K/V tile (keeps LDS under 64 KiB at d = 128)

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kRows32) void fwd_fp32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_k,
    float scale_log2, int n_rblocks) {
  __shared__ float Qs[kRows32][D + 1];
  __shared__ __attribute__((aligned(16))) float Ks[kKeys32][D];
  __shared__ __attribute__((aligned(16))) float Vs[kKeys32][D];

  // one-dimensional grid: (batch, head) major, then the 64-row block
  const int bh = blockIdx.x / n_rblocks;
  const int b = bh / H_q;
  const int h = bh - b * H_q;
  const int hk = h / (H_q / H_kv);
  const int tid = threadIdx.x;
  const int q0 = (blockIdx.x - bh * n_rblocks) * kRows32;
  const int row = q0 + tid;
  const int shift = N_k - N_q;
  const float* Qp = Q + (size_t)bh * N_q * D;
  const float* Kp = K + ((size_t)b * H_kv + hk) * N_k * D;
  const float* Vp = V + ((size_t)b * H_kv + hk) * N_k * D;

  for (int x = tid; x < kRows32 * D; x += kRows32) {
    const int r = x / D, c = x % D;
    Qs[r][c] = (q0 + r < N_q) ? Qp[(size_t)(q0 + r) * D + c] : 0.f;
  }

  int n_tiles = (N_k + kKeys32 - 1) / kKeys32;
  if (CAUSAL) {
    const int max_key = min(q0 + kRows32 - 1, N_q - 1) + shift;
    n_tiles = max_key < 0 ? 0 : min(n_tiles, max_key / kKeys32 + 1);
  }
  const int lim = CAUSAL ? min(N_k - 1, row + shift) : N_k - 1;  // last key this row sees

  float m_run = kNegInf, l_run = 0.f;
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;

  for (int j = 0; j < n_tiles; ++j) {
    const int kbase = j * kKeys32;
    __syncthreads();
    for (int x = tid; x < kKeys32 * D / 4; x += kRows32) {
      const int r = x / (D / 4), c4 = x % (D / 4);
      const bool ok = kbase + r < N_k;
      const f32x4 kz = ok ? *reinterpret_cast<const f32x4*>(Kp + (size_t)(kbase + r) * D + 4 * c4) : f32x4{};
      const f32x4 vz = ok ? *reinterpret_cast<const f32x4*>(Vp + (size_t)(kbase + r) * D + 4 * c4) : f32x4{};
      *reinterpret_cast<f32x4*>(&Ks[r][4 * c4]) = kz;
      *reinterpret_cast<f32x4*>(&Vs[r][4 * c4]) = vz;
    }
    __syncthreads();

    float s[kKeys32];
    float mx = kNegInf;
#pragma unroll
    for (int k = 0; k < kKeys32; ++k) {
      float dot = 0.f;
#pragma unroll 16
      for (int c = 0; c < D; ++c) dot = __builtin_fmaf(Qs[tid][c], Ks[k][c], dot);
      s[k] = (kbase + k <= lim) ? dot : kNegInf;
      mx = fmaxf(mx, s[k]);
    }
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f_hw(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < kKeys32; ++k) {
      s[k] = exp2f_hw(__builtin_fmaf(s[k], scale_log2, -m_use));
      psum += s[k];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int c = 0; c < D; ++c) {
      float a = acc[c] * alpha;
#pragma unroll
      for (int k = 0; k < kKeys32; ++k) a = __builtin_fmaf(s[k], Vs[k][c], a);
      acc[c] = a;
    }
  }

  if (row >= N_q) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* Orow = O + ((size_t)bh * N_q + row) * D;
#pragma unroll
  for (int c = 0; c < D; c += 4)
    *reinterpret_cast<f32x4*>(Orow + c) = f32x4{acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
  if (LSE != nullptr)
    LSE[(size_t)bh * N_q + row] = l_run > 0.f ? (m_run + log2f_hw(l_run)) * kLn2 : kNegInf;
}

template <int D, bool CAUSAL>
static hipError_t launch32(const FwdArgs& a) {
  const int n_rb = (a.N_q + kRows32 - 1) / kRows32;
  const long long total = (long long)a.B * a.H_q * n_rb;  // <= B*H_q*N_q < 2^31 (checked by the caller)
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_fp32_kernel<D, CAUSAL>), dim3((unsigned)total), dim3(kRows32), 0, (hipStream_t)a.stream,
                     (const float*)a.Q, (const float*)a.K, (const float*)a.V, (float*)a.O, a.LSE,
                     a.H_q, a.H_kv, a.N_q, a.N_k, a.scale * kLog2e, n_rb);
  return hipGetLastError();
}

hipError_t launch_fwd_fp32(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch32<128, true>(a) : launch32<128, false>(a);
  return a.causal ? launch32<64, true>(a) : launch32<64, false>(a);
}

}  // namespace fa
