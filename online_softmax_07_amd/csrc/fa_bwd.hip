// FlashAttention backward, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// What is kept from the forward pass and how P comes back (page "Attention kernel chains",
// chain "What the backward pass saves"): the inputs, the output and a single fp32 LSE value for each query row;
// each probability tile is rebuilt on chip as P = exp(S - LSE), and the softmax gradient
// uses one extra row vector D = rowsum(dO * O), computed once before the main loops.  With
// dS = P * (dP - D), dP = dO V^T, the gradients are dV = P^T dO, dK = scale dS^T Q and
// dQ = scale dS K (the chain rule of the forward definition).
//
// Three kernels on the caller's stream:
//   * bwd_prep_kernel: per query row, D = rowsum(dO * O) and LSE in base 2, written to the
//     workspace as one 64-float record per 32-row block (32 log2-LSE values, then 32 D
//     values), rows padded to a multiple of 64.  Rows past N_q, and rows that see no key,
//     get LSE = +inf, so every P that refers to them is exactly 0 without a test.
//   * bwd_dq_kernel: the forward's layout.  4 waves x 32 query rows own a 128-row block;
//     K and V tiles of 64 keys stream through a double-buffered LDS ring (LDS-DMA loads).
//     S^T = K Q^T and dP^T = V dO^T on the 32x32x16 MFMA put one query row in each lane,
//     so LSE and D are per-lane scalars; dQ^T += K^T dS^T reads K^T with the transposing
//     LDS read.  dQ is written once.
//   * bwd_dkdv_kernel: the transposed roles.  4 waves x 32 keys own a 128-key block and
//     hold their K and V rows as MFMA operands in registers; Q and dO tiles of 64 rows
//     (of every query head of the GQA group in turn) stream through LDS and are taken in
//     two 32-row halves.  S = Q K^T and
//     dP = dO V^T put one key in each lane; dV^T += dO^T P and dK^T += Q^T dS read dO^T
//     and Q^T with the transposing LDS read.  The kernel runs one wave per SIMD, so each
//     64-row step is issued as one software-pipelined stream of MFMAs with the operand
//     reads and the softmax placed between them.  dK and dV (summed over the group) are
//     written once: no atomics, and the result does not depend on scheduling.
// Both main kernels walk only the tiles the bottom-right causal mask leaves visible, and a
// causal workgroup takes a heavy and a light block of one head so all cost the same.
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kRowBlk = 32;    // rows per LSE/D record
#ifndef FA_BWD_DKDV_ROWS
#define FA_BWD_DKDV_ROWS 64    // query rows per dK/dV step (64 or 128)
#endif
constexpr int kRecPerStep = FA_BWD_DKDV_ROWS / 32;  // records per dK/dV step

// LSE/D records per (batch, query head): whole steps of kRecPerStep records, so a step's
// records always exist (rows past N_q are padding with LSE = +inf, D = 0).
__host__ __device__ __forceinline__ int rec_blocks(int n_q) {
  return (n_q + kRowBlk * kRecPerStep - 1) / (kRowBlk * kRecPerStep) * kRecPerStep;
}
constexpr float kPosInf = __builtin_inff();

// Logical 16-byte chunk c of LDS row r sits at position c ^ swz(r); keeps the plain b128
// operand reads (16 rows, one chunk) and the transposing reads (4 rows x 4 chunks)
// conflict-free on unpadded rows.
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? ((r & 3) << 2) | ((r >> 2) & 3) : (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Workgroup -> (head, unit).  Workgroups are dispatched round-robin over the 8 XCDs; each
// XCD gets a contiguous range of heads, so the blocks of one head share that XCD's L2.
__device__ __forceinline__ void map_workgroup(int wg, int total_wg, int n_units, int& head, int& unit) {
  const int n_heads = total_wg / n_units;
  if ((n_heads & 7) == 0) {
    const int hpx = n_heads >> 3;
    const int x = wg & 7, idx = wg >> 3;
    head = x * hpx + idx / n_units;
    unit = idx % n_units;
  } else {
    int logical = wg;
    if ((total_wg & 7) == 0) logical = (wg & 7) * (total_wg >> 3) + (wg >> 3);
    head = logical / n_units;
    unit = logical % n_units;
  }
}

// Offsets (elements) of this lane's MFMA operand reads in a row-major swizzled LDS tile:
//   plain: A/B fragment of k-step t (16 columns), row l32, logical chunk 2t + hh;
//   transposing: column block cb, half r of a 16-row step: lane (g16, i16) points at row
//     8r + 4hh + i16/4, columns 32cb + 16(g16%2) + 4(i16%4) .. +3.
template <int D>
struct OperandOffsets {
  int plain[D / 16];
  int tr[2][D / 32];
  __device__ __forceinline__ OperandOffsets(int lane) {
    const int l32 = lane & 31, hh = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) plain[t] = l32 * D + 8 * ((2 * t + hh) ^ swz<D>(l32));
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const int row = 8 * r + 4 * hh + (i16 >> 2);
        const int c = 4 * cb + 2 * (g16 & 1) + ((i16 & 3) >> 1);
        tr[r][cb] = row * D + 8 * (c ^ swz<D>(row)) + 4 * (i16 & 1);
      }
  }
};

// Calls f(std::integral_constant<int, i>) for i = I .. N-1: a loop whose index is a
// compile-time constant in the body, so register arrays are never indexed dynamically.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Transposed operand of a 16-row step starting at `row0` of an LDS tile: rows become k.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const __bf16* tile, int row0, const OperandOffsets<D>& off, int cb) {
  const __bf16* p = tile + row0 * D;
  return join_bf16x8(lds_read_tr16(p + off.tr[0][cb]), lds_read_tr16(p + off.tr[1][cb]));
}

// Row-major store of a 32 x D accumulator block set (acc[cb] holds columns 32cb..32cb+31
// of this lane's row, the MFMA layout of an O^T-style product), times `mul`.
template <int D, typename OutT>
__device__ __forceinline__ void store_row(OutT* row, const f32x16 (&acc)[D / 32], float mul, int hh) {
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = cb * 32 + 8 * g + 4 * hh;
      const f32x4 v = {acc[cb][4 * g] * mul, acc[cb][4 * g + 1] * mul, acc[cb][4 * g + 2] * mul,
                       acc[cb][4 * g + 3] * mul};
      if constexpr (sizeof(OutT) == 4) {
        *reinterpret_cast<f32x4*>(row + c) = v;
      } else {
        *reinterpret_cast<bf16x4*>(row + c) = __builtin_convertvector(v, bf16x4);
      }
    }
}

// The same block in bf16 through a wave-private 32 x D LDS area, so each store writes whole
// rows (1 KB of consecutive rows per instruction) instead of 8 bytes of 32 rows.  `dst` is
// the block's first row; rows from n_valid on are not written.
template <int D>
__device__ __forceinline__ void store_rows_lds(__bf16* dst, int n_valid, __bf16* area,
                                               const f32x16 (&acc)[D / 32], float mul, int lane) {
  constexpr int CH = D / 8, RPI = 64 / CH;  // 16-byte chunks per row, rows per access
  int ln = lane;
  asm volatile("" : "+v"(ln));  // offsets made here, not hoisted into the main loop
  const int r32 = ln & 31, hh = ln >> 5;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // an earlier block is read back
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 v = {acc[cb][4 * g] * mul, acc[cb][4 * g + 1] * mul, acc[cb][4 * g + 2] * mul,
                       acc[cb][4 * g + 3] * mul};
      // chunk cb*4+g of row r32, XOR-swizzled by the row so the 32 rows spread over the banks
      *reinterpret_cast<bf16x4*>(area + r32 * D + (((cb * 4 + g) ^ (r32 & (CH - 1))) << 3) + 4 * hh) =
          __builtin_convertvector(v, bf16x4);
    }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = RPI * i + ln / CH, ch = ln % CH;
    const u32x4 val = *reinterpret_cast<const u32x4*>(area + row * D + ((ch ^ (row & (CH - 1))) << 3));
    if (row < n_valid) *reinterpret_cast<u32x4*>(dst + (size_t)row * D + ch * 8) = val;
  }
}

}  // namespace

// ---------------------------------------------------------------------------------------
// D = rowsum(dO * O) and the base-2 LSE, per 32-row record
// ---------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(const __bf16* __restrict__ O,
                                                            const __bf16* __restrict__ dO,
                                                            const float* __restrict__ LSE, float* __restrict__ rec,
                                                            int N_q, int n_rblk, long long n_slots) {
  constexpr int LPR = D / 8;  // lanes per row, 8 values each
  const long long t = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long slot = t / LPR;  // one slot per padded row
  const int part = (int)(t % LPR);
  float acc = 0.f;
  const long long bh = slot / ((long long)n_rblk * kRowBlk);
  const int row = (int)(slot - bh * n_rblk * kRowBlk);
  const bool valid = slot < n_slots && row < N_q;
  if (valid) {
    const size_t off = ((size_t)bh * N_q + row) * D + 8 * part;
    const bf16x8 o = *reinterpret_cast<const bf16x8*>(O + off);
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(dO + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf((float)o[i], (float)g[i], acc);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += shfl_xor_f(acc, m);
  if (part == 0 && slot < n_slots) {
    float l2 = kPosInf;  // rows past N_q and rows with no visible key: every P is 0
    if (valid) {
      const float l = LSE[(size_t)bh * N_q + row];
      if (l != kNegInf) l2 = l * kLog2e;
    }
    const long long blk = bh * n_rblk + row / kRowBlk;
    rec[blk * 64 + (row % kRowBlk)] = l2;
    rec[blk * 64 + 32 + (row % kRowBlk)] = valid ? acc : 0.f;
  }
}

// ---------------------------------------------------------------------------------------
// dQ: one workgroup per NW * 32 query rows (causal: a heavy and a light block), K/V streamed
// ---------------------------------------------------------------------------------------
template <int D, int BC, int NW, bool CAUSAL, typename OutT>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ rec, OutT* __restrict__ dQ, int H_q, int H_kv,
    int N_q, int N_k, float scale, float scale_log2, int n_qblocks, int n_units, int total_wg) {
  constexpr int BR = 32 * NW;
  constexpr int CHUNKS = D / 8;
  constexpr int STAGE = BC * D;
  constexpr int ROWS_PER_DMA = 1024 / (2 * D);
  constexpr int DMA = BC * D * 2 / 1024 / NW;  // per wave per tile, K and V each
  static_assert(DMA * 1024 * NW == BC * D * 2, "tile must split evenly over the waves");
  constexpr int NCB = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 Ks0[STAGE], Ks1[STAGE];
  __shared__ __attribute__((aligned(16))) __bf16 Vs0[STAGE], Vs1[STAGE];

  int bh, unit;
  map_workgroup(blockIdx.x, total_wg, n_units, bh, unit);
  const int b = bh / H_q;
  const int h = bh - b * H_q;
  const int hk = h / (H_q / H_kv);
  const __bf16* Kp = K + ((size_t)b * H_kv + hk) * N_k * D;
  const __bf16* Vp = V + ((size_t)b * H_kv + hk) * N_k * D;
  const int n_rblk = rec_blocks(N_q);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const OperandOffsets<D> off(lane);
  uint32_t dma_off[DMA];
#pragma unroll
  for (int i = 0; i < DMA; ++i) {
    const int r = ROWS_PER_DMA * (DMA * wave + i) + lane / CHUNKS;
    dma_off[i] = (uint32_t)(r * D + 8 * ((lane % CHUNKS) ^ swz<D>(r))) * 2u;
  }
  auto tile_rsrc = [&](const __bf16* base, int j) {
    const int kbase = j * BC;
    return make_rsrc(base + (size_t)kbase * D, range_bytes((long long)N_k - kbase, D * 2));
  };

  const int n_pass = (CAUSAL && 2 * unit + 1 < n_qblocks) ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    const int qb = !CAUSAL ? unit : (pass == 0 ? n_qblocks - 1 - unit : unit);
    const int q0 = qb * BR;
    const int wave_row0 = q0 + wave * 32;
    const int qrow = wave_row0 + l32;
    const int shift = N_k - N_q;
    const int qr = qrow < N_q ? qrow : N_q - 1;

    bf16x8 qf[D / 16], gf[D / 16];  // Q and dO rows as MFMA B fragments
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      qf[t] = *reinterpret_cast<const bf16x8*>(Q + ((size_t)bh * N_q + qr) * D + 16 * t + 8 * hh);
      gf[t] = *reinterpret_cast<const bf16x8*>(dO + ((size_t)bh * N_q + qr) * D + 16 * t + 8 * hh);
      if (qrow >= N_q) gf[t] = bf16x8{};
    }
    const float* r = rec + ((size_t)bh * n_rblk + qr / kRowBlk) * 64 + (qr % kRowBlk);
    const float lse2 = qrow < N_q ? r[0] : kPosInf;
    const float Dv = qrow < N_q ? r[32] : 0.f;

    int n_tiles = (N_k + BC - 1) / BC;
    if (CAUSAL) {
      const int max_key = min(q0 + BR - 1, N_q - 1) + shift;
      n_tiles = max_key < 0 ? 0 : min(n_tiles, max_key / BC + 1);
    }
    const int wave_last_key = min(wave_row0 + 31, N_q - 1) + shift;
    const int row_lim = CAUSAL ? min(N_k - 1, qrow + shift) : N_k - 1;

    f32x16 dq[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) dq[cb] = f32x16{};

    auto dma = [&](int i, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, __bf16* ks, __bf16* vs) {
      const int ii = i % DMA;
      buffer_load16_lds(i < DMA ? kr : vr, dma_off[ii], (i < DMA ? ks : vs) + (DMA * wave_u + ii) * 512);
    };
    if (n_tiles > 0) {
      const auto kr = tile_rsrc(Kp, 0), vr = tile_rsrc(Vp, 0);
#pragma unroll
      for (int i = 0; i < 2 * DMA; ++i) dma(i, kr, vr, Ks0, Vs0);
    }
    wait_vmem();
    __syncthreads();

    auto tile_step = [&](int j, const __bf16* ks, const __bf16* vs, __bf16* ks_next, __bf16* vs_next) {
      const auto kr_next = tile_rsrc(Kp, j + 1), vr_next = tile_rsrc(Vp, j + 1);
      constexpr int NDMA = 2 * DMA;
      constexpr int STEPS = (BC / 32) * (D / 16);
      constexpr int DMA_PER_STEP = (NDMA + STEPS - 1) / STEPS;
      const int kbase = j * BC;
      if (!CAUSAL || kbase <= wave_last_key) {
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb) {
          const int kb0 = kbase + kb * 32;
          if (CAUSAL && kb0 > wave_last_key) {
#pragma unroll
            for (int i = kb * (D / 16) * DMA_PER_STEP; i < (kb + 1) * (D / 16) * DMA_PER_STEP && i < NDMA; ++i)
              dma(i, kr_next, vr_next, ks_next, vs_next);
            continue;
          }
          // S^T and dP^T of 32 keys x this wave's 32 rows
          __builtin_amdgcn_s_setprio(1);
          f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
          for (int t = 0; t < D / 16; ++t) {
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(ks + kb * 32 * D + off.plain[t]);
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(vs + kb * 32 * D + off.plain[t]);
            s = mfma32x32x16(ka, qf[t], s);
            dp = mfma32x32x16(va, gf[t], dp);
            const int st = kb * (D / 16) + t;
#pragma unroll
            for (int i = st * DMA_PER_STEP; i < (st + 1) * DMA_PER_STEP && i < NDMA; ++i)
              dma(i, kr_next, vr_next, ks_next, vs_next);
          }
          // order: the K and V fragments of two k-steps in flight ahead of their MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
          for (int t = 0; t < D / 16; ++t) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if ((kb * (D / 16) + t) * DMA_PER_STEP < NDMA)
              __builtin_amdgcn_sched_group_barrier(0x020, DMA_PER_STEP, 0);
            if (t + 2 < D / 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          }
          __builtin_amdgcn_s_setprio(0);
          // P^T = 2^(s scale log2e - lse2), 0 past the mask; dS^T = P^T (dP^T - D)
          const bool need_mask = (kb0 + 32 > N_k) || (CAUSAL && kb0 + 31 > wave_row0 + shift);
          const int thr = row_lim - kb0 - 4 * hh;
          // (a block every row of this wave sees in full takes the variant without mask tests)
          f32x16 ds;
          auto soft = [&](auto maskc) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              float p = exp2f_hw(__builtin_fmaf(s[i], scale_log2, -lse2));
              if constexpr (decltype(maskc)::value) {
                if (8 * (i >> 2) + (i & 3) > thr) p = 0.f;
              }
              ds[i] = p * (dp[i] - Dv);
            }
          };
          if (need_mask) soft(std::true_type{});
          else soft(std::false_type{});
          bf16x8 dsf[2];
#pragma unroll
          for (int u = 0; u < 2; ++u)
            dsf[u] = to_bf16x8(f32x8{ds[8 * u], ds[8 * u + 1], ds[8 * u + 2], ds[8 * u + 3], ds[8 * u + 4],
                                     ds[8 * u + 5], ds[8 * u + 6], ds[8 * u + 7]});
          // dQ^T += K^T dS^T (K^T through the transposing LDS read)
          __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
              dq[cb] = mfma32x32x16(tr_frag<D>(ks, kb * 32 + 16 * u, off, cb), dsf[u], dq[cb]);
          __builtin_amdgcn_s_setprio(0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) dma(i, kr_next, vr_next, ks_next, vs_next);
      }
      wait_vmem();
      __syncthreads();
    };
    for (int j = 0; j < n_tiles; j += 2) {
      tile_step(j, Ks0, Vs0, Ks1, Vs1);
      if (j + 1 < n_tiles) tile_step(j + 1, Ks1, Vs1, Ks0, Vs0);
    }
    if constexpr (sizeof(OutT) == 2 && NW * 32 * D <= 2 * STAGE) {
      // bf16 out: through stage 1, which every wave has finished reading (the last tile's
      // barrier) and the next causal block refills only after its first barrier
      __bf16* area = (wave < NW / 2 ? Ks1 : Vs1) + (wave % (NW / 2)) * (32 * D);
      store_rows_lds<D>(reinterpret_cast<__bf16*>(dQ) + ((size_t)bh * N_q + wave_row0) * D, N_q - wave_row0, area,
                        dq, scale, lane);
    } else if (qrow < N_q) {
      store_row<D>(dQ + ((size_t)bh * N_q + qrow) * D, dq, scale, hh);
    }
  }
}

// ---------------------------------------------------------------------------------------
// dK, dV: one workgroup per 128 keys of a KV head (causal: a heavy and a light block);
// Q and dO of every query head of the group streamed past
// ---------------------------------------------------------------------------------------
template <int D, bool CAUSAL, typename OutT>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ rec, OutT* __restrict__ dK, OutT* __restrict__ dV,
    int H_q, int H_kv, int N_q, int N_k, float scale, float scale_log2, int n_kblocks, int n_units, int total_wg) {
  constexpr int BKV = 128, BQ = kRowBlk * kRecPerStep, NSB = kRecPerStep;  // NSB 32-row sub-blocks
  constexpr int CHUNKS = D / 8;
  constexpr int STAGE = BQ * D;
  constexpr int ROWS_PER_DMA = 1024 / (2 * D);
  constexpr int TDMA = BQ * D * 2 / 1024;  // 1 KB loads per tile (Q or dO)
  constexpr int DMA = 2 * TDMA / 4;        // per wave per step, Q and dO together
  constexpr int NCB = D / 32;
  static_assert(DMA * 4 == 2 * TDMA, "the Q and dO tiles must split evenly over the waves");
  __shared__ __attribute__((aligned(16))) __bf16 Qs0[STAGE], Qs1[STAGE];
  __shared__ __attribute__((aligned(16))) __bf16 Gs0[STAGE], Gs1[STAGE];
  __shared__ __attribute__((aligned(16))) float Rs0[64 * NSB], Rs1[64 * NSB];  // per 32 rows: log2 LSE[32], D[32]

  int bhk, unit;
  map_workgroup(blockIdx.x, total_wg, n_units, bhk, unit);
  const int b = bhk / H_kv;
  const int hk = bhk - b * H_kv;
  const int g = H_q / H_kv;
  const int n_rblk = rec_blocks(N_q);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const OperandOffsets<D> off(lane);
  // DMA i of this wave: global index gi = DMA*wave + i; the first TDMA fill Q, the rest dO
  uint32_t dma_off[DMA];
#pragma unroll
  for (int i = 0; i < DMA; ++i) {
    const int li = (DMA * wave + i) % TDMA;
    const int r = ROWS_PER_DMA * li + lane / CHUNKS;
    dma_off[i] = (uint32_t)(r * D + 8 * ((lane % CHUNKS) ^ swz<D>(r))) * 2u;
  }
  const int shift = N_k - N_q;
  const int n_qb = (N_q + BQ - 1) / BQ;

  const int n_pass = (CAUSAL && 2 * unit + 1 < n_kblocks) ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    // causal: early keys are seen by the most rows, so block `unit` is the heavy one
    const int kblk = !CAUSAL ? unit : (pass == 0 ? unit : n_kblocks - 1 - unit);
    const int k0 = kblk * BKV;
    const int kw0 = k0 + 32 * wave;
    const int key = kw0 + l32;
    const int kr_ = key < N_k ? key : N_k - 1;

    // this wave's K and V rows as MFMA B fragments (zero past N_k)
    bf16x8 kf[D / 16], vf[D / 16];
    const __bf16* Krow = K + (((size_t)b * H_kv + hk) * N_k + kr_) * D;
    const __bf16* Vrow = V + (((size_t)b * H_kv + hk) * N_k + kr_) * D;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      kf[t] = *reinterpret_cast<const bf16x8*>(Krow + 16 * t + 8 * hh);
      vf[t] = *reinterpret_cast<const bf16x8*>(Vrow + 16 * t + 8 * hh);
      if (key >= N_k) {
        kf[t] = bf16x8{};
        vf[t] = bf16x8{};
      }
    }
    f32x16 dk[NCB], dv[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      dk[cb] = f32x16{};
      dv[cb] = f32x16{};
    }

    // query blocks that see a key of this workgroup: rows i >= k0 - shift (causal)
    const int first_row = CAUSAL ? max(0, k0 - shift) : 0;
    const int qb_first = first_row / BQ;
    const int n_steps = first_row < N_q ? g * (n_qb - qb_first) : 0;
    const int wave_first_row = CAUSAL ? kw0 - shift : -1;  // rows below see none of this wave's keys

    auto step_rows = [&](int s, int& bh, int& q0) {
      const int hi = s / (n_qb - qb_first);
      bh = b * H_q + hk * g + hi;
      q0 = (qb_first + (s - hi * (n_qb - qb_first))) * BQ;
    };
    auto issue = [&](int s, __bf16* qs, __bf16* gs, float* rs) {
      int bh = 0, q0 = 0;
      if (s < n_steps) step_rows(s, bh, q0);
      const uint32_t bytes = s < n_steps ? range_bytes((long long)N_q - q0, D * 2) : 0u;
      const auto qr = make_rsrc(Q + ((size_t)bh * N_q + q0) * D, bytes);
      const auto gr = make_rsrc(dO + ((size_t)bh * N_q + q0) * D, bytes);
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        const int gi = DMA * wave_u + i;  // wave-uniform
        const int li = gi % TDMA;
        buffer_load16_lds(gi < TDMA ? qr : gr, dma_off[i], (gi < TDMA ? qs : gs) + li * 512);
      }
      if (wave_u == 0 && lane < 16 * NSB) {  // the 64-float LSE/D records of these rows
        const auto rr = make_rsrc(rec + ((size_t)bh * n_rblk + q0 / kRowBlk) * 64, s < n_steps ? 256u * NSB : 0u);
        buffer_load16_lds(rr, (uint32_t)lane * 16u, reinterpret_cast<__bf16*>(rs));
      }
    };

    issue(0, Qs0, Gs0, Rs0);
    wait_vmem();
    __syncthreads();

    // Masking: register i of a 32-row sub-block starting at row qs0 holds row
    // qs0 + 8(i/4) + 4hh + i%4, which sees this lane's key iff row + shift >= key; with
    // thr = qs0 + 4hh + shift - key that is 8(i/4) + i%4 + thr >= 0.  Keys past N_k are
    // never seen.
    const bool key_ok = key < N_k;
    auto step = [&](int s, const __bf16* qs_step, const __bf16* gs_step, const float* rs_step, __bf16* qs_n,
                    __bf16* gs_n, float* rs_n) {
      issue(s + 1, qs_n, gs_n, rs_n);
      int bh, q0_step;
      step_rows(s, bh, q0_step);
      // the step's rows in pairs of 32-row sub-blocks
#pragma unroll
      for (int pr = 0; pr < NSB / 2; ++pr) {
        const __bf16* qs = qs_step + pr * 64 * D;
        const __bf16* gs = gs_step + pr * 64 * D;
        const float* rs = rs_step + pr * 128;
        const int q0 = q0_step + 64 * pr;
        // One sub-block at a time (a causal step whose first sub-block sees none of this
        // wave's keys): S = Q K^T and dP = dO V^T for its 32 rows x this wave's 32 keys,
        auto scores = [&](int sb, f32x16& sc, f32x16& dp) {
          const __bf16* qsb = qs + sb * 32 * D;
          const __bf16* gsb = gs + sb * 32 * D;
          sc = f32x16{};
          dp = f32x16{};
#pragma unroll
          for (int t = 0; t < D / 16; ++t) {
            const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qsb + off.plain[t]);
            const bf16x8 ga = *reinterpret_cast<const bf16x8*>(gsb + off.plain[t]);
            sc = mfma32x32x16(qa, kf[t], sc);
            dp = mfma32x32x16(ga, vf[t], dp);
          }
        };
        // P = 2^(s scale log2e - lse2[row]) (0 past the mask; rows past N_q have lse2 = +inf)
        // and dS = P (dP - D[row]) as bf16 MFMA operands,
        auto softmax = [&](int sb, const f32x16& sc, const f32x16& dp, bf16x8 (&pf)[2], bf16x8 (&dsf)[2]) {
          const int qs0 = q0 + 32 * sb;
          const float* rsb = rs + sb * 64;
          const int thr = qs0 + 4 * hh + shift - key;
          f32x16 p, ds;
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(rsb + 8 * gq + 4 * hh);
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(rsb + 32 + 8 * gq + 4 * hh);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * gq + e;
              float pv = exp2f_hw(__builtin_fmaf(sc[i], scale_log2, -l4[e]));
              const bool vis = key_ok && (!CAUSAL || 8 * gq + e + thr >= 0);
              pv = vis ? pv : 0.f;
              p[i] = pv;
              ds[i] = pv * (dp[i] - d4[e]);
            }
          }
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            pf[u] = to_bf16x8(f32x8{p[8 * u], p[8 * u + 1], p[8 * u + 2], p[8 * u + 3], p[8 * u + 4], p[8 * u + 5],
                                    p[8 * u + 6], p[8 * u + 7]});
            dsf[u] = to_bf16x8(f32x8{ds[8 * u], ds[8 * u + 1], ds[8 * u + 2], ds[8 * u + 3], ds[8 * u + 4],
                                     ds[8 * u + 5], ds[8 * u + 6], ds[8 * u + 7]});
          }
        };
        // then dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T through the transposing LDS read)
        auto grads = [&](int sb, const bf16x8 (&pf)[2], const bf16x8 (&dsf)[2]) {
          const __bf16* qsb = qs + sb * 32 * D;
          const __bf16* gsb = gs + sb * 32 * D;
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
              dv[cb] = mfma32x32x16(tr_frag<D>(gsb, 16 * u, off, cb), pf[u], dv[cb]);
              dk[cb] = mfma32x32x16(tr_frag<D>(qsb, 16 * u, off, cb), dsf[u], dk[cb]);
            }
        };
        static_assert(NSB % 2 == 0, "the step is written for pairs of 32-row sub-blocks");
        // causal: sub-block rows below wave_first_row see none of this wave's keys
        if (!CAUSAL || q0 + 31 >= wave_first_row) {
          // Both sub-blocks, as one software-pipelined stream of MFMAs: the scores (S, dP) of
          // sub-blocks 0 and 1, then the gradients (dV, dK) of 0 and 1.  Each LDS operand is
          // read PD MFMAs ahead of its use (one wave per SIMD: nothing else hides the LDS
          // latency), and the softmax of a sub-block runs in the shadow of the MFMAs that
          // follow its scores, EPS elements per MFMA slot in two stages (exponential, then
          // mask and dS) one slot apart, so that each slot's VALU work is independent.  A
          // scheduling fence after each slot keeps this order.
          constexpr int NMS = 2 * (D / 16);  // score MFMAs per sub-block
          constexpr int NMG = 4 * NCB;       // gradient MFMAs per sub-block
          constexpr int NMT = 2 * NMS + 2 * NMG;
          constexpr int PD = 2;
          constexpr int kRecLead = 3;
          constexpr int EPS = D >= 128 ? 1 : 2;  // softmax elements per slot
          constexpr int NSL = 16 / EPS;          // slots of stage 1 per sub-block
          constexpr int S0[2] = {NMS + 1, 2 * NMS + 1};  // first softmax slot of each sub-block
          static_assert(S0[0] + 8 / EPS + 1 <= 2 * NMS && S0[0] + NSL + 1 <= 2 * NMS + 2 * NCB &&
                            S0[1] + 8 / EPS + 1 <= 2 * NMS + NMG && S0[1] + NSL + 1 <= 2 * NMS + NMG + 2 * NCB,
                        "each bf16 operand pair is complete before its first gradient MFMA");
          f32x16 sc[2], dp[2];
          float ex[2][16];
          f32x8 p8[2], d8[2];
          bf16x8 pf[2][2], dsf[2][2];
          f32x4 l4[2][4], d4[2][4];
          auto load_op = [&](auto mc) -> bf16x8 {
            constexpr int m = decltype(mc)::value;
            if constexpr (m < 2 * NMS) {
              constexpr int sb = m / NMS, j = m % NMS;
              return *reinterpret_cast<const bf16x8*>((j & 1 ? gs : qs) + sb * 32 * D + off.plain[j >> 1]);
            } else {
              constexpr int m2 = m - 2 * NMS, sb = m2 / NMG, j = m2 % NMG;
              return tr_frag<D>((j & 1 ? qs : gs) + sb * 32 * D, 16 * (j / (2 * NCB)), off, (j >> 1) % NCB);
            }
          };
          auto load_rec = [&](int sb, int gq) {
            l4[sb][gq] = *reinterpret_cast<const f32x4*>(rs + sb * 64 + 8 * gq + 4 * hh);
            d4[sb][gq] = *reinterpret_cast<const f32x4*>(rs + sb * 64 + 32 + 8 * gq + 4 * hh);
          };
          // register i of a sub-block holds row 8(i/4) + 4hh + i%4 of it
          auto stage1 = [&](int sb, int i) {  // e = 2^(s scale log2e - lse2[row])
            ex[sb][i] = exp2f_hw(__builtin_fmaf(sc[sb][i], scale_log2, -l4[sb][i >> 2][i & 3]));
          };
          auto stage2 = [&](auto maskc, int sb, int i) {  // P (0 past the mask), dS = P (dP - D[row])
            float pv = ex[sb][i];
            if constexpr (decltype(maskc)::value) {
              const int thr = q0 + 32 * sb + 4 * hh + shift - key;
              const bool vis = key_ok && (!CAUSAL || 8 * (i >> 2) + (i & 3) + thr >= 0);
              pv = vis ? pv : 0.f;
            }
            p8[sb][i & 7] = pv;
            d8[sb][i & 7] = pv * (dp[sb][i] - d4[sb][i >> 2][i & 3]);
            if ((i & 7) == 7) {
              pf[sb][i >> 3] = to_bf16x8(p8[sb]);
              dsf[sb][i >> 3] = to_bf16x8(d8[sb]);
            }
          };
          auto stream = [&](auto maskc) {
            sc[0] = sc[1] = dp[0] = dp[1] = f32x16{};
            bf16x8 ops[PD];
            static_for<0, PD>([&](auto mc) { ops[decltype(mc)::value] = load_op(mc); });
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, NMT>([&](auto mc) {
              constexpr int m = decltype(mc)::value;
              const bf16x8 a = ops[m % PD];
              if constexpr (m + PD < NMT) ops[m % PD] = load_op(std::integral_constant<int, m + PD>{});
#pragma unroll
              for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int gq = 0; gq < 4; ++gq)
                  if (m == S0[sb] + 4 * gq / EPS - kRecLead) load_rec(sb, gq);
              if constexpr (m < 2 * NMS) {
                constexpr int sb = m / NMS, j = m % NMS;
                if constexpr (j & 1) dp[sb] = mfma32x32x16(a, vf[j >> 1], dp[sb]);
                else sc[sb] = mfma32x32x16(a, kf[j >> 1], sc[sb]);
              } else {
                constexpr int m2 = m - 2 * NMS, sb = m2 / NMG, j = m2 % NMG;
                constexpr int u = j / (2 * NCB), cb = (j >> 1) % NCB;
                if constexpr (j & 1) dk[cb] = mfma32x32x16(a, dsf[sb][u], dk[cb]);
                else dv[cb] = mfma32x32x16(a, pf[sb][u], dv[cb]);
              }
#pragma unroll
              for (int sb = 0; sb < 2; ++sb) {
                const int k = m - S0[sb];
                if (k >= 0 && k < NSL) {
#pragma unroll
                  for (int e = 0; e < EPS; ++e) stage1(sb, EPS * k + e);
                }
                if (k >= 1 && k <= NSL) {
#pragma unroll
                  for (int e = 0; e < EPS; ++e) stage2(maskc, sb, EPS * (k - 1) + e);
                }
              }
              __builtin_amdgcn_sched_barrier(0);
            });
          };
          // masking only where this wave's keys run past N_k or past the first row's reach
          if (kw0 + 32 > N_k || (CAUSAL && kw0 + 31 > q0 + shift)) stream(std::true_type{});
          else stream(std::false_type{});
        } else if (q0 + 63 >= wave_first_row) {
          f32x16 sc1, dp1;
          bf16x8 pf1[2], ds1[2];
          scores(1, sc1, dp1);
          softmax(1, sc1, dp1, pf1, ds1);
          grads(1, pf1, ds1);
        }
      }
      wait_vmem();
      __syncthreads();
    };
    for (int s = 0; s < n_steps; s += 2) {
      step(s, Qs0, Gs0, Rs0, Qs1, Gs1, Rs1);
      if (s + 1 < n_steps) step(s + 1, Qs1, Gs1, Rs1, Qs0, Gs0, Rs0);
    }
    if constexpr (sizeof(OutT) == 2 && 4 * 32 * D <= 2 * STAGE) {
      // bf16 out: through stage 1, which every wave has finished reading (the last step's
      // barrier) and the next causal block refills only after its first barrier
      __bf16* area = (wave < 2 ? Qs1 : Gs1) + (wave & 1) * (32 * D);
      const size_t row0 = (((size_t)b * H_kv + hk) * N_k + kw0) * D;
      store_rows_lds<D>(reinterpret_cast<__bf16*>(dK) + row0, N_k - kw0, area, dk, scale, lane);
      store_rows_lds<D>(reinterpret_cast<__bf16*>(dV) + row0, N_k - kw0, area, dv, 1.f, lane);
    } else if (key < N_k) {
      const size_t row = (((size_t)b * H_kv + hk) * N_k + key) * D;
      store_row<D>(dK + row, dk, scale, hh);
      store_row<D>(dV + row, dv, 1.f, hh);
    }
  }
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
namespace {

template <int D, bool CAUSAL, typename OutT>
hipError_t launch_bwd_main(const BwdArgs& a) {
  hipStream_t st = (hipStream_t)a.stream;
  const float scale_log2 = a.scale * kLog2e;
  const float* rec = static_cast<const float*>(a.workspace);
  {
    // 4 waves (128 rows) over 64-key tiles, two workgroups per CU (8 waves over 128-key
    // tiles measured 2 % slower)
    constexpr int NW = 4, BC = 64;
    const int n_qblocks = (a.N_q + 32 * NW - 1) / (32 * NW);
    const int n_units = CAUSAL ? (n_qblocks + 1) / 2 : n_qblocks;
    const long long total = (long long)a.B * a.H_q * n_units;
    if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (total > 0) {  // N_q = 0: no dQ
      hipLaunchKernelGGL((bwd_dq_kernel<D, BC, NW, CAUSAL, OutT>), dim3((unsigned)total), dim3(64 * NW), 0, st,
                         (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (const __bf16*)a.dO, rec,
                         (OutT*)a.dQ, a.H_q, a.H_kv, a.N_q, a.N_k, a.scale, scale_log2, n_qblocks, n_units,
                         (int)total);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int n_kblocks = (a.N_k + 127) / 128;
  const int n_units = CAUSAL ? (n_kblocks + 1) / 2 : n_kblocks;
  const long long total = (long long)a.B * a.H_kv * n_units;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (total == 0) return hipSuccess;  // N_k = 0: no dK, dV
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, OutT>), dim3((unsigned)total), dim3(kThreads), 0, st,
                     (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (const __bf16*)a.dO, rec,
                     (OutT*)a.dK, (OutT*)a.dV, a.H_q, a.H_kv, a.N_q, a.N_k, a.scale, scale_log2, n_kblocks,
                     n_units, (int)total);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, bool out_f32) {
  const int n_rblk = rec_blocks(a.N_q);
  const long long n_slots = (long long)a.B * a.H_q * n_rblk * kRowBlk;
  const long long threads = n_slots * (D / 8);
  const long long grid = (threads + kThreads - 1) / kThreads;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (grid > 0) {  // N_q = 0: no records (dK, dV are then all zero)
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)a.stream,
                       (const __bf16*)a.O, (const __bf16*)a.dO, a.LSE, static_cast<float*>(a.workspace), a.N_q,
                       n_rblk, n_slots);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.causal)
    return out_f32 ? launch_bwd_main<D, true, float>(a) : launch_bwd_main<D, true, __bf16>(a);
  return out_f32 ? launch_bwd_main<D, false, float>(a) : launch_bwd_main<D, false, __bf16>(a);
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H_q, int N_q) {
  const size_t n_rblk = (size_t)rec_blocks(N_q);
  return ((size_t)B * H_q * n_rblk * 64 * sizeof(float) + 255) & ~(size_t)255;
}

hipError_t launch_bwd(const BwdArgs& a, bool out_f32) {
  return a.d == 128 ? launch_bwd_d<128>(a, out_f32) : launch_bwd_d<64>(a, out_f32);
}

}  // namespace fa
