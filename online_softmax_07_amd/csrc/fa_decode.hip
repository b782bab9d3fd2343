// Split-KV decode ("flash decoding") on gfx950 MFMA, contiguous or paged KV cache.
//
// Page "Attention kernel chains":
//   * "How many splits for decode": the key axis of each (batch, KV head) is cut into
//     num_splits contiguous ranges, one workgroup each, so that batch x KV heads x splits
//     fills the GPU;
//   * "GQA loads KV once per group": the g = H_q / H_kv query heads of a group, times the
//     T new tokens, are stacked as the rows of one MFMA tile, so each K/V element is read
//     once per group and feeds g*T rows;
//   * "The block-table cost of paged attention": with a block table, token j of sequence b
//     is slot j % page_size of pool page block_table[b][j / page_size];
//   * "The causal mask for a decode step": query t of the T new ones sits at position
//     N_k - T + t and sees keys j <= N_k - T + t;
//   * "The log-sum-exp merge": each split writes its normalized partial output and lse.
//
// Per workgroup: 4 waves, 16 MFMA rows (stacked heads x tokens; a second row chunk goes
// to blockIdx.z).  Each wave streams its own 64-key chunks of the split (chunks w, w+4,
// ...), loads K straight into MFMA A fragments (16-byte loads), computes S^T = K Q^T
// with the 16x16x32 bf16 MFMA (each lane then holds one row and 16 keys), runs the
// online-softmax update, stages the chunk's V through a wave-private LDS area, transposed
// while written, and accumulates O^T += V^T P^T.  At the end the four waves' carries
// are merged in LDS by the same LSE rule.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kDecThreads = 256;
constexpr int kDecRows = 16;

// Position of key k (0 <= k < 64) inside a V^T row: key 32u + 16a + 4g + b goes to
// 32u + 8g + 4a + b, making the 8 keys of one P^T k-group contiguous.
__device__ __forceinline__ int dec_vt_pos(int k) {
  return (k & 32) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

template <int D, bool PAGED, typename OutT>
__global__ __launch_bounds__(kDecThreads, 2) void decode_split_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    OutT* __restrict__ O, float* __restrict__ LSE, float* __restrict__ O_part,
    float* __restrict__ LSE_part, const int32_t* __restrict__ block_table, int page_size,
    int pages_per_seq, int H_q, int H_kv, int T, int N_k, int causal, int ns, int split_len,
    float scale_log2) {
  constexpr int VPITCH = kDecodeChunk + 8;  // bf16 per V^T row (16-byte pad)
  constexpr int CH = D / 8;                 // 16-byte chunks per K/V row
  constexpr int VUNITS = (kDecodeChunk / 4) * CH / 64;  // 4-key x 8-col units per lane
  constexpr int VT_BYTES = D * VPITCH * 2;
  constexpr int MERGE_BYTES = (4 * kDecRows * 2 + 4 * kDecRows * D) * 4;
  constexpr int SMEM = 4 * VT_BYTES > MERGE_BYTES ? 4 * VT_BYTES : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  const int split = blockIdx.x;
  const int bk = blockIdx.y;  // b * H_kv + hk
  const int b = bk / H_kv;
  const int hk = bk - b * H_kv;
  const int g = H_q / H_kv;
  const int R = g * T;                      // stacked rows of this (b, hk)
  const int rows_total = gridDim.y * R;     // B * H_q * T
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // ---- this lane's MFMA row: (query head within the group, new token) ----
  const int rho = blockIdx.z * kDecRows + l16;
  const bool row_ok = rho < R;
  const int hg = row_ok ? rho / T : 0;
  const int tq = row_ok ? rho - hg * T : 0;
  const int hq = hk * g + hg;
  const int lim = causal ? N_k - T + tq : N_k - 1;  // last key this row sees (bottom-right)

  bf16x8 qf[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    qf[t] = row_ok ? *reinterpret_cast<const bf16x8*>(Q + (((size_t)b * H_q + hq) * T + tq) * D + 32 * t + 8 * g4)
                   : bf16x8{};
  }

  const int k0 = split * split_len;
  const int k1 = min(k0 + split_len, N_k);
  const int nchunks = k0 < k1 ? (k1 - k0 + kDecodeChunk - 1) / kDecodeChunk : 0;
  const int min_lim = causal ? N_k - T : N_k - 1;  // smallest per-row limit

  auto key_row = [&](const __bf16* base, int key) -> const __bf16* {
    if constexpr (PAGED) {
      const int page = block_table[(size_t)b * pages_per_seq + key / page_size];
      return base + (((size_t)page * page_size + key % page_size) * H_kv + hk) * D;
    } else {
      return base + ((size_t)bk * N_k + key) * D;
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) o[cb] = f32x4{};

  __bf16* Vt = reinterpret_cast<__bf16*>(smem) + wave * D * VPITCH;

  for (int ci = wave; ci < nchunks; ci += 4) {
    const int cbase = k0 + ci * kDecodeChunk;

    // ---- loads: K as MFMA A fragments, V as 4-row x 8-column units ----
    bf16x8 kf[4][D / 32];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = cbase + kb * 16 + l16;
      if (key < k1) {
        const __bf16* kr = key_row(K, key);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) kf[kb][t] = *reinterpret_cast<const bf16x8*>(kr + 32 * t + 8 * g4);
      } else {
#pragma unroll
        for (int t = 0; t < D / 32; ++t) kf[kb][t] = bf16x8{};
      }
    }
    u32x4 vreg[VUNITS][4];
#pragma unroll
    for (int i = 0; i < VUNITS; ++i) {
      const int u = i * 64 + lane;
      const int quad = u / CH;
      const int chunk = u % CH;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = cbase + quad * 4 + r;
        vreg[i][r] = key < k1 ? *reinterpret_cast<const u32x4*>(key_row(V, key) + chunk * 8) : u32x4{};
      }
    }

    // ---- S^T = K Q^T: lane holds row l16, keys 16 kb + 4 g4 + r ----
    f32x4 s[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int t = 0; t < D / 32; ++t) s[kb] = mfma16x16x32(kf[kb][t], qf[t], s[kb]);
    }
    if (cbase + kDecodeChunk > k1 || cbase + kDecodeChunk - 1 > min_lim) {
      const int last = min(k1 - 1, lim);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (cbase + kb * 16 + 4 * g4 + r > last) s[kb][r] = kNegInf;
    }

    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f_hw(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[kb][r] = exp2f_hw(__builtin_fmaf(s[kb][r], scale_log2, -m_use));
        psum += s[kb][r];
      }
    l_run = l_run * alpha + psum;
    // P^T operands (bf16, RNE) for the two 32-key steps
    bf16x8 pf[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
      pf[u] = to_bf16x8(f32x8{s[2 * u][0], s[2 * u][1], s[2 * u][2], s[2 * u][3],
                              s[2 * u + 1][0], s[2 * u + 1][1], s[2 * u + 1][2], s[2 * u + 1][3]});
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) o[cb] *= alpha;

    // ---- V chunk -> wave-private LDS, transposed to V^T ----
#pragma unroll
    for (int i = 0; i < VUNITS; ++i) {
      const int u = i * 64 + lane;
      const int quad = u / CH;
      const int chunk = u % CH;
      const int pos = dec_vt_pos(quad * 4);
#pragma unroll
      for (int e0 = 0; e0 < 8; ++e0) {
        const int e = (e0 + chunk) & 7;
        const int m = e >> 1;
        uint32_t lo, hi;
        if (e & 1) {
          lo = pack_hi(vreg[i][0][m], vreg[i][1][m]);
          hi = pack_hi(vreg[i][2][m], vreg[i][3][m]);
        } else {
          lo = pack_lo(vreg[i][0][m], vreg[i][1][m]);
          hi = pack_lo(vreg[i][2][m], vreg[i][3][m]);
        }
        *reinterpret_cast<u32x2*>(Vt + (chunk * 8 + e) * VPITCH + pos) = u32x2{lo, hi};
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- O^T += V^T P^T (two k-steps of 32 keys) ----
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int cb = 0; cb < D / 16; ++cb) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vt + (cb * 16 + l16) * VPITCH + 32 * u + 8 * g4);
        o[cb] = mfma16x16x32(vf, pf[u], o[cb]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- merge the four waves (same LSE rule, in base 2) ----
  float l_row = l_run + shfl_xor_f(l_run, 16);
  l_row += shfl_xor_f(l_row, 32);
  __syncthreads();
  float* Mw = reinterpret_cast<float*>(smem);  // [4][16]
  float* Lw = Mw + 4 * kDecRows;               // [4][16]
  float* Ow = Lw + 4 * kDecRows;               // [4][16][D]
  if (g4 == 0) {
    Mw[wave * kDecRows + l16] = m_run;
    Lw[wave * kDecRows + l16] = l_row;
  }
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb)
    *reinterpret_cast<f32x4*>(Ow + (wave * kDecRows + l16) * D + cb * 16 + 4 * g4) = o[cb];
  __syncthreads();

  const int row = tid >> 4;        // 16 rows x 16 threads
  const int cpart = tid & 15;
  constexpr int CPT = D / 16;      // columns per thread
  const int rr = blockIdx.z * kDecRows + row;
  if (rr >= R) return;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, Mw[w * kDecRows + row]);
  float out[CPT];
  float lse;
  if (M == kNegInf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) out[i] = 0.f;
    lse = kNegInf;
  } else {
    float wsum = 0.f, wt[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wt[w] = exp2f_hw(Mw[w * kDecRows + row] - M);
      wsum += Lw[w * kDecRows + row] * wt[w];
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) a = __builtin_fmaf(Ow[(w * kDecRows + row) * D + cpart * CPT + i], wt[w], a);
      out[i] = a * inv;
    }
    lse = (M + log2f_hw(wsum)) * kLn2;
  }
  const int rhg = rr / T;
  const int rt = rr - rhg * T;
  const size_t grow = ((size_t)b * H_q + hk * g + rhg) * T + rt;  // row of [B, H_q, T]
  if (ns == 1) {
    OutT* Orow = O + grow * D + cpart * CPT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) Orow[i] = (OutT)out[i];
    if (LSE != nullptr && cpart == 0) LSE[grow] = lse;
  } else {
    float* Orow = O_part + ((size_t)split * rows_total + grow) * D + cpart * CPT;
#pragma unroll
    for (int i = 0; i < CPT; i += 4) *reinterpret_cast<f32x4*>(Orow + i) = f32x4{out[i], out[i + 1], out[i + 2], out[i + 3]};
    if (cpart == 0) LSE_part[(size_t)split * rows_total + grow] = lse;
  }
}

template <int D, bool PAGED, typename OutT>
static hipError_t launch_dec(const DecodeArgs& a) {
  const int R = (a.H_q / a.H_kv) * a.T;
  dim3 grid(a.num_splits, a.B * a.H_kv, (R + kDecRows - 1) / kDecRows);
  hipLaunchKernelGGL((decode_split_kernel<D, PAGED, OutT>), grid, dim3(kDecThreads), 0, (hipStream_t)a.stream,
                     (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (OutT*)a.O, a.LSE, a.O_part,
                     a.LSE_part, a.block_table, a.page_size, a.pages_per_seq, a.H_q, a.H_kv, a.T, a.N_k,
                     a.causal, a.num_splits, a.split_len, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_dec(const DecodeArgs& a, bool out_f32) {
  if (a.block_table != nullptr)
    return out_f32 ? launch_dec<D, true, float>(a) : launch_dec<D, true, __bf16>(a);
  return out_f32 ? launch_dec<D, false, float>(a) : launch_dec<D, false, __bf16>(a);
}

hipError_t launch_decode_split(const DecodeArgs& a, bool out_f32) {
  const int R = (a.H_q / a.H_kv) * a.T;
  if (a.B * (long long)a.H_kv > 65535 || (R + kDecRows - 1) / kDecRows > 65535) return hipErrorInvalidConfiguration;
  if (a.d == 128) return dispatch_dec<128>(a, out_f32);
  return dispatch_dec<64>(a, out_f32);
}

}  // namespace fa
