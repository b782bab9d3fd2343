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
//   * "The log-sum-exp merge": a split stores its output divided by its own sum, and the
//     log of that sum, for the merge to weigh.
//
// Per workgroup: 4 waves, 16 MFMA rows (stacked heads x tokens; a further row chunk goes
// to blockIdx.z).  Decode is a bytes problem, so the kernel is built around keeping loads
// in flight: each wave streams its own 32-key chunks of the split (chunks w, w+4, ...),
// and the loads of the next chunk are issued before the current one is computed (two
// register sets).  K goes straight from memory into MFMA A fragments; V is written
// row-major into a wave-private LDS area and read back as V^T with the transposing LDS
// read.  S^T = K Q^T and O^T += V^T P^T run on the 16x16x32 bf16 MFMA (each lane holds
// one row and 8 keys of a chunk).  Rows of keys past the split are loaded from a clamped
// (valid) address and masked: their P is exactly 0, so no zero fill is needed.  With a
// block table, every lane fetches the page of one key two chunks ahead and the row
// addresses are exchanged with ds_bpermute, so the dependent table load never stalls the
// stream.  K and V are read exactly once per call, so their loads are nontemporal: the
// lines stream through the caches without displacing anything (on this chip that raises a
// streaming read from about 5.8 to 6.7 TB/s).  At the end the four waves' carries are
// merged in LDS by the LSE rule.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kDecThreads = 256;
constexpr int kDecRows = 16;
constexpr int kDecChunk = 32;  // keys per wave iteration
static_assert(kDecChunk * 2 == kDecodeChunk, "split lengths are multiples of two chunks");

template <int D>
struct DecChunk {
  static constexpr int KT = D / 32;                   // 16x16x32 k-steps over the head dimension
  static constexpr int VL = kDecChunk * D / 8 / 64;   // 16-byte V pieces per lane
  static constexpr int VROWS_PER_LOAD = 64 / (D / 8); // V rows covered by one load instruction
  bf16x8 k[2][KT];
  u32x4 v[VL];
};

template <int D, bool PAGED, typename OutT>
__global__ __launch_bounds__(kDecThreads, 2) void decode_split_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    OutT* __restrict__ O, float* __restrict__ LSE, float* __restrict__ O_part,
    float* __restrict__ LSE_part, const int32_t* __restrict__ block_table, int page_size,
    int pages_per_seq, int H_q, int H_kv, int T, int N_k, int causal, int ns, int split_len,
    float scale_log2) {
  using C = DecChunk<D>;
  constexpr int VP = D + 16;                          // V row pitch in LDS (32-byte pad)
  constexpr int VT_ELEMS = kDecChunk * VP;            // per wave
  constexpr int MERGE_BYTES = (4 * kDecRows * 2 + 4 * kDecRows * D) * 4;
  constexpr int SMEM = 4 * VT_ELEMS * 2 > MERGE_BYTES ? 4 * VT_ELEMS * 2 : MERGE_BYTES;
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

  bf16x8 qf[C::KT];
#pragma unroll
  for (int t = 0; t < C::KT; ++t) {
    qf[t] = *reinterpret_cast<const bf16x8*>(Q + (((size_t)b * H_q + hq) * T + tq) * D + 32 * t + 8 * g4);
    if (!row_ok) qf[t] = bf16x8{};
  }

  // 64-bit products: with many splits split * split_len passes 2^31 (such splits are empty)
  const int k0 = (int)min((long long)split * split_len, (long long)N_k);
  const int k1 = (int)min((long long)k0 + split_len, (long long)N_k);
  const int nchunks = k0 < k1 ? (k1 - k0 + kDecChunk - 1) / kDecChunk : 0;
  const int min_lim = causal ? N_k - T : N_k - 1;  // smallest per-row limit
  const int my_chunks = nchunks > wave ? (nchunks - wave + 3) / 4 : 0;  // chunks wave, wave+4, ...

  // Row index (in units of D elements) of key `key` of this (b, hk).
  auto row_of = [&](int key) -> int {
    if constexpr (PAGED) {
      const int page = block_table[(size_t)b * pages_per_seq + key / page_size];
      return (page * page_size + key % page_size) * H_kv + hk;
    } else {
      return bk * N_k + key;
    }
  };
  // Each lane's share of a chunk's row indices: lane l holds key (cbase + l % 32), clamped
  // into the split so every address is valid.
  auto chunk_rows = [&](int i) -> int {
    const int ci = wave + 4 * min(i, my_chunks - 1);
    const int key = min(k0 + ci * kDecChunk + (lane & 31), k1 - 1);
    return row_of(key);
  };
  auto load = [&](int rows, C& c) {
    // K: lane (key l16 of block kb, k-group g4) -> MFMA A fragments
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int r = __builtin_amdgcn_ds_bpermute(4 * (kb * 16 + l16), rows);
      const __bf16* kr = K + (size_t)r * D + 8 * g4;
#pragma unroll
      for (int t = 0; t < C::KT; ++t)
        c.k[kb][t] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + 32 * t)));
    }
    // V: load i covers VROWS_PER_LOAD whole rows, 16 bytes per lane
#pragma unroll
    for (int i = 0; i < C::VL; ++i) {
      const int row = i * C::VROWS_PER_LOAD + lane / (D / 8);
      const int r = __builtin_amdgcn_ds_bpermute(4 * row, rows);
      c.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(V + (size_t)r * D + (lane % (D / 8)) * 8));
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x4 o[D / 16];
#pragma unroll
  for (int cb = 0; cb < D / 16; ++cb) o[cb] = f32x4{};
  __bf16* Vt = reinterpret_cast<__bf16*>(smem) + wave * VT_ELEMS;

  auto compute = [&](int i, C& c) {
    const int cbase = k0 + (wave + 4 * i) * kDecChunk;
    // ---- S^T = K Q^T: lane holds row l16, keys 16 kb + 4 g4 + r ----
    f32x4 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int t = 0; t < C::KT; ++t) s[kb] = mfma16x16x32(c.k[kb][t], qf[t], s[kb]);
    }
    if (cbase + kDecChunk > k1 || cbase + kDecChunk - 1 > min_lim) {
      const int last = min(k1 - 1, lim);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (cbase + kb * 16 + 4 * g4 + r > last) s[kb][r] = kNegInf;
    }
    // ---- online softmax (exact running max) ----
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f_hw(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[kb][r] = exp2f_hw(__builtin_fmaf(s[kb][r], scale_log2, -m_use));
        psum += s[kb][r];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) o[cb] *= alpha;
    // P^T operand: slots 0-3 = keys 4 g4 + r, slots 4-7 = keys 16 + 4 g4 + r
    const bf16x8 pf = to_bf16x8(f32x8{s[0][0], s[0][1], s[0][2], s[0][3], s[1][0], s[1][1], s[1][2], s[1][3]});

    // ---- V chunk -> wave-private LDS, row-major ----
#pragma unroll
    for (int i2 = 0; i2 < C::VL; ++i2) {
      const int row = i2 * C::VROWS_PER_LOAD + lane / (D / 8);
      *reinterpret_cast<u32x4*>(Vt + row * VP + (lane % (D / 8)) * 8) = c.v[i2];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- O^T += V^T P^T: A fragment (cb) via two transposing reads.  Lane (16-group g4,
    // index l16) points at key 16 r + 4 g4 + l16/4, columns 16 cb + 4 (l16 % 4) .. +3.
    const __bf16* vb = Vt + (4 * g4 + (l16 >> 2)) * VP + 4 * (l16 & 3);
#pragma unroll
    for (int cb = 0; cb < D / 16; ++cb) {
      const bf16x8 vf = join_bf16x8(lds_read_tr16(vb + 16 * cb), lds_read_tr16(vb + 16 * VP + 16 * cb));
      o[cb] = mfma16x16x32(vf, pf, o[cb]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // ---- the stream: loads of chunk i+1 in flight while chunk i is computed; table rows
  // (paged) fetched one chunk earlier still ----
  if (my_chunks > 0) {
    C ca, cb_;
    int rows_next = chunk_rows(0);
    int rows_after = chunk_rows(1);
    load(rows_next, ca);
    rows_next = rows_after;
    rows_after = chunk_rows(2);
    int i = 0;
    for (; i + 1 < my_chunks; i += 2) {
      load(rows_next, cb_);
      rows_next = rows_after;
      rows_after = chunk_rows(i + 3);
      compute(i, ca);
      if (i + 2 < my_chunks) load(rows_next, ca);
      rows_next = rows_after;
      rows_after = chunk_rows(i + 4);
      compute(i + 1, cb_);
    }
    if (i < my_chunks) compute(i, ca);
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
