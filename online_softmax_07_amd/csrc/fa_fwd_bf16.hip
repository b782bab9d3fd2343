// FlashAttention forward, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// Loop order (page "Softmax and FlashAttention", "Concept", FlashAttention-2): one
// workgroup owns a block of BR = 128 query rows of one (batch, head) and streams the K/V
// tiles of BC keys past it; each BR x BC score tile lives only in registers and is folded
// into the running output with the online-softmax carries of page "Kernel visualization:
// Flash Attention 1" ("Derivation", "The tiled version"): running max m, running sum l,
// unnormalized accumulator; one division by l at the end (page "Attention kernel chains",
// chain "The online softmax on numbers"), and the per-row LSE written once.
//
// MI355X mapping:
//   * 4 waves x 32 query rows.  Scores are computed transposed, S^T = K Q^T, with the
//     32x32x16 bf16 MFMA: K (from LDS) is the A operand, the wave's Q rows (registers,
//     loaded once) the B operand.  In the accumulator layout each lane then owns ONE query
//     row (lane % 32) and 16 keys per 32-key block, so the row max is a register reduction
//     plus one exchange between the two wave halves, the row sum stays a per-lane partial
//     until the end, and the rescale factor alpha is a per-lane scalar.
//   * O^T = V^T P^T on the same MFMA: P^T comes straight from the score registers
//     (converted to bf16), V^T is read from an LDS copy of the V tile that was transposed
//     while it was staged (4 key rows x 8 columns per thread, regrouped with v_perm).
//   * K/V tiles: coalesced 16-byte global loads into registers one tile ahead, then into
//     padded (bank-conflict-free for the MFMA reads) LDS tiles.
//   * Workgroup order: heaviest causal query blocks first, and consecutive blocks of a
//     head kept on one XCD so the K/V re-reads of the FlashAttention-2 order hit its L2.
//   * Softmax in base 2: p = 2^(s * scale * log2 e - m), with m kept in the same units.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kBR = 128;      // query rows per workgroup
constexpr int kThreads = 256; // 4 waves

template <int D, int BC>
struct FwdTile {
  static constexpr int KPITCH = D + 8;   // bf16 elements per K row in LDS (16-byte pad)
  static constexpr int VPITCH = BC + 8;  // bf16 elements per V^T row in LDS
  static constexpr int CHUNKS = D / 8;   // 16-byte chunks per K/V row
  static constexpr int KLOADS = BC * CHUNKS / kThreads;  // K chunks per thread per tile
  static_assert(BC * CHUNKS % kThreads == 0, "K tile must split evenly");
  static_assert((BC / 4) * CHUNKS == kThreads, "V tile: one 4-row x 8-col unit per thread");
};

// Position of key k (0 <= k < BC) inside a V^T row in LDS.  Keys are grouped by 16; in a
// group, key 8a + 4h + b (a, h in {0,1}, b in 0..3) goes to 8h + 4a + b, so the eight keys
// that one MFMA k-group of P^T holds (see the S^T accumulator layout) are contiguous.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) | (((k >> 2) & 1) << 3) | (((k >> 3) & 1) << 2) | (k & 3);
}

template <int D, int BC, bool CAUSAL, typename OutT>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    OutT* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_k,
    float scale_log2, int n_qblocks, int total_wg) {
  using T = FwdTile<D, BC>;
  __shared__ __attribute__((aligned(16))) __bf16 Ks[BC * T::KPITCH];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[D * T::VPITCH];

  // ---- which (batch, head, query block) this workgroup owns ----
  int wg = blockIdx.x;
  int logical = wg;
  if ((total_wg & 7) == 0) logical = (wg & 7) * (total_wg >> 3) + (wg >> 3);  // XCD-contiguous
  const int bh = logical / n_qblocks;
  const int qb = n_qblocks - 1 - (logical % n_qblocks);  // heavy (late) blocks first
  const int b = bh / H_q;
  const int h = bh - b * H_q;
  const int hk = h / (H_q / H_kv);
  const __bf16* Qp = Q + (size_t)bh * N_q * D;
  const __bf16* Kp = K + ((size_t)b * H_kv + hk) * N_k * D;
  const __bf16* Vp = V + ((size_t)b * H_kv + hk) * N_k * D;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;  // k-group of the MFMA operands
  const int q0 = qb * kBR;
  const int wave_row0 = q0 + wave * 32;
  const int qrow = wave_row0 + l32;
  const int shift = N_k - N_q;  // bottom-right alignment: row i sees keys j <= i + shift

  // ---- Q block: read once, kept as MFMA B fragments ----
  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    if (qrow < N_q) {
      qf[t] = *reinterpret_cast<const bf16x8*>(Qp + (size_t)qrow * D + 16 * t + 8 * hh);
    } else {
      qf[t] = bf16x8{};
    }
  }

  // ---- which K/V tiles this block visits ----
  int n_tiles = (N_k + BC - 1) / BC;
  if (CAUSAL) {
    const int last_row = min(q0 + kBR - 1, N_q - 1);
    const int max_key = last_row + shift;
    n_tiles = max_key < 0 ? 0 : min(n_tiles, max_key / BC + 1);
  }
  const int wave_last_key = min(wave_row0 + 31, N_q - 1) + shift;  // causal reach of this wave

  // ---- carries (one query row per lane; l is this lane's partial over its keys) ----
  float m_run = kNegInf;
  float l_run = 0.f;
  f32x16 o[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) o[cb] = f32x16{};

  // ---- register staging of the next K/V tile ----
  u32x4 kreg[T::KLOADS];
  u32x4 vreg[4];
  const int v_quad = tid / T::CHUNKS;  // 4 consecutive keys
  const int v_chunk = tid % T::CHUNKS; // 8 consecutive columns

  auto load_tile = [&](int j) {
    const int kbase = j * BC;
#pragma unroll
    for (int i = 0; i < T::KLOADS; ++i) {
      const int c = i * kThreads + tid;
      const int row = c / T::CHUNKS;
      const int col = c % T::CHUNKS;
      const int key = kbase + row;
      kreg[i] = key < N_k ? *reinterpret_cast<const u32x4*>(Kp + (size_t)key * D + col * 8) : u32x4{};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kbase + v_quad * 4 + r;
      vreg[r] = key < N_k ? *reinterpret_cast<const u32x4*>(Vp + (size_t)key * D + v_chunk * 8) : u32x4{};
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < T::KLOADS; ++i) {
      const int c = i * kThreads + tid;
      const int row = c / T::CHUNKS;
      const int col = c % T::CHUNKS;
      *reinterpret_cast<u32x4*>(Ks + row * T::KPITCH + col * 8) = kreg[i];
    }
    // transpose 4 keys x 8 columns into 8 columns x 4 keys
    const int pos = vt_pos(v_quad * 4);
#pragma unroll
    for (int e0 = 0; e0 < 8; ++e0) {
      const int e = (e0 + v_chunk) & 7;  // rotate to spread LDS banks
      const int m = e >> 1;
      uint32_t lo, hi;
      if (e & 1) {
        lo = pack_hi(vreg[0][m], vreg[1][m]);
        hi = pack_hi(vreg[2][m], vreg[3][m]);
      } else {
        lo = pack_lo(vreg[0][m], vreg[1][m]);
        hi = pack_lo(vreg[2][m], vreg[3][m]);
      }
      *reinterpret_cast<u32x2*>(Vt + (v_chunk * 8 + e) * T::VPITCH + pos) = u32x2{lo, hi};
    }
  };

  if (n_tiles > 0) load_tile(0);

  for (int j = 0; j < n_tiles; ++j) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (j + 1 < n_tiles) load_tile(j + 1);  // in flight while this tile is computed

    const int kbase = j * BC;
    if (CAUSAL && kbase > wave_last_key) continue;  // no row of this wave sees this tile

    // ---- S^T = K_j Q^T for this wave's 32 rows ----
    f32x16 s[BC / 32];
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + l32) * T::KPITCH + 16 * t + 8 * hh);
        s[kb] = mfma32x32x16(kf, qf[t], s[kb]);
      }
    }

    // ---- mask: ragged tail and the bottom-right causal edge ----
    const bool need_mask = (kbase + BC > N_k) || (CAUSAL && kbase + BC - 1 > wave_row0 + shift);
    if (need_mask) {
      const int lim = CAUSAL ? min(N_k - 1, qrow + shift) : N_k - 1;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
          if (key > lim) s[kb][r] = kNegInf;
        }
    }

    // ---- online softmax update (base 2) ----
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f_hw(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f_hw(__builtin_fmaf(s[kb][r], scale_log2, -m_use));
        s[kb][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) o[cb] *= alpha;

    // ---- O^T += V_j^T P^T ----
#pragma unroll
    for (int u = 0; u < BC / 16; ++u) {
      const f32x16& sk = s[u >> 1];
      const int r0 = (u & 1) * 8;
      const bf16x8 pf = to_bf16x8(f32x8{sk[r0 + 0], sk[r0 + 1], sk[r0 + 2], sk[r0 + 3],
                                        sk[r0 + 4], sk[r0 + 5], sk[r0 + 6], sk[r0 + 7]});
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vt + (cb * 32 + l32) * T::VPITCH + 16 * u + 8 * hh);
        o[cb] = mfma32x32x16(vf, pf, o[cb]);
      }
    }
  }

  // ---- epilogue: one division, O and LSE written once ----
  const float l_tot = l_run + shfl_xor_f(l_run, 32);  // the two wave halves hold one row's keys
  if (qrow >= N_q) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  OutT* Orow = O + ((size_t)bh * N_q + qrow) * D;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = cb * 32 + 8 * g + 4 * hh;
      const f32x4 v = {o[cb][4 * g] * inv, o[cb][4 * g + 1] * inv, o[cb][4 * g + 2] * inv,
                       o[cb][4 * g + 3] * inv};
      if constexpr (sizeof(OutT) == 4) {
        *reinterpret_cast<f32x4*>(Orow + c) = v;
      } else {
        *reinterpret_cast<bf16x4*>(Orow + c) = __builtin_convertvector(v, bf16x4);
      }
    }
  if (LSE != nullptr && hh == 0) {
    LSE[(size_t)bh * N_q + qrow] = l_tot > 0.f ? (m_run + log2f_hw(l_tot)) * kLn2 : kNegInf;
  }
}

template <int D, int BC, bool CAUSAL, typename OutT>
static hipError_t launch(const FwdArgs& a) {
  const int n_qblocks = (a.N_q + kBR - 1) / kBR;
  const long long total = (long long)a.B * a.H_q * n_qblocks;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, CAUSAL, OutT>), dim3((unsigned)total), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V,
                     (OutT*)a.O, a.LSE, a.H_q, a.H_kv, a.N_q, a.N_k, a.scale * kLog2e, n_qblocks,
                     (int)total);
  return hipGetLastError();
}

template <int D, int BC>
static hipError_t dispatch_out(const FwdArgs& a, bool out_f32) {
  if (a.causal) return out_f32 ? launch<D, BC, true, float>(a) : launch<D, BC, true, __bf16>(a);
  return out_f32 ? launch<D, BC, false, float>(a) : launch<D, BC, false, __bf16>(a);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, bool out_f32) {
  if (a.d == 128) return dispatch_out<128, 64>(a, out_f32);
  return dispatch_out<64, 128>(a, out_f32);
}

}  // namespace fa
