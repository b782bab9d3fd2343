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
//     log of that sum, for the merge to weigh.  With a placement map (below) the merge runs
//     inside this kernel: the split of a group that completes last weighs the group's
//     partials, so no second launch follows.
//
// Per workgroup: 4 waves, 16 MFMA rows (stacked heads x tokens; a further row chunk is a
// further group); paged, two workgroups fit a CU, contiguous one (its stream keeps two
// chunks' registers live throughout; the automatic split count aims at one wave of one
// workgroup per CU either way).  Decode is a bytes problem, so the kernel is built around
// keeping loads in flight: each wave streams its own 32-key chunks of the split (chunks w,
// w+4, ...),
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
//
// Placement and the in-kernel merge.  Workgroups are dealt to the XCDs round-robin by
// linear index, so indices equal modulo the XCD count share an XCD and its L2.  The grid is
// one-dimensional and workgroup L takes group x + n_map * ((L / n_map) / ns) and split
// (L / n_map) % ns, x = L % n_map: with n_map a multiple of the XCD count, all splits of a
// group run on one XCD.  Each split stores its partial rows (plain stores, which reach that
// L2), waits until they are complete, stores its completion flag (a token unique to the
// call) and reads the group's flags back from the L2 (by atomics: the L1 of a CU may hold
// a copy read by an earlier workgroup); a split that finds every flag set merges the
// partials, read from the same L2, and returns the flags to 0.  The
// split completing last always finds them all (two completing together both merge and
// write the same values: the merge visits the splits in one fixed order).  No split waits
// for another.  The host enables this only after a probe of the XCD of every workgroup
// index has shown the round-robin placement on the GPU (flags == NULL otherwise: the
// partials go to the separate merge kernel).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr int kDecThreads = 256;
constexpr int kDecRows = kDecodeRows;
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

// The word at p as the L2 holds it.  Atomics run in the L2, never in a CU's L1 (which may
// still hold a line read earlier in the kernel by another workgroup on the same CU), and a
// compare-and-swap whose new value equals the expected one leaves memory as it is whatever
// it finds; the compiler keeps it an atomic (an idempotent add or or becomes a plain load).
__device__ __forceinline__ uint32_t read_at_l2(uint32_t* p) {
  uint32_t e = 0u;
  __hip_atomic_compare_exchange_strong(p, &e, 0u, __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return e;
}

template <int D, bool PAGED, typename OutT>
__global__ __launch_bounds__(kDecThreads, PAGED ? 2 : 1) void decode_split_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    OutT* __restrict__ O, float* __restrict__ LSE, float* __restrict__ O_part,
    float* __restrict__ LSE_part, uint32_t* __restrict__ flags, uint32_t token, int n_map, int n_groups,
    int n_zc, const int32_t* __restrict__ block_table, int page_size,
    int pages_per_seq, int H_q, int H_kv, int T, int N_k, int causal, int ns, int split_len,
    float scale_log2) {
  using C = DecChunk<D>;
  constexpr int VP = D + 16;                          // V row pitch in LDS (32-byte pad)
  constexpr int VT_ELEMS = kDecChunk * VP;            // per wave
  constexpr int MERGE_BYTES = (4 * kDecRows * 2 + 4 * kDecRows * D) * 4;
  constexpr int SMEM = 4 * VT_ELEMS * 2 > MERGE_BYTES ? 4 * VT_ELEMS * 2 : MERGE_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];

  // ---- which (split, group) this workgroup owns; a group is (b, hk, 16-row chunk zc) ----
  const int wgi = blockIdx.x;
  const int kq = wgi / n_map;
  const int group = wgi - kq * n_map + n_map * (kq / ns);
  if (group >= n_groups) return;            // the grid is rounded up to whole XCD rounds
  const int split = kq % ns;
  const int bk = group / n_zc;              // b * H_kv + hk
  const int zc = group - bk * n_zc;
  const int b = bk / H_kv;
  const int hk = bk - b * H_kv;
  const int g = H_q / H_kv;
  const int R = g * T;                      // stacked rows of this (b, hk)
  const int rows_total = (n_groups / n_zc) * R;  // B * H_q * T
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15;
  const int g4 = lane >> 4;

  // ---- this lane's MFMA row: (query head within the group, new token) ----
  const int rho = zc * kDecRows + l16;
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
  // A chunk past this wave's last one (looked up or loaded, never computed) takes the split's
  // first key in every lane: a few cache lines instead of a whole chunk.
  auto chunk_rows = [&](int i) -> int {
    const int key = i < my_chunks ? min(k0 + (wave + 4 * i) * kDecChunk + (lane & 31), k1 - 1) : k0;
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

  // ---- the stream: loads of chunk i+1 in flight while chunk i is computed ----
  if (my_chunks > 0) {
    C ca, cb_;
    if constexpr (!PAGED) {
      // Two chunks in flight from the start and every load of the loop issued
      // unconditionally (past-the-end chunks read one row), so every path into the loop
      // leaves the same loads outstanding and the compiler's wait counts keep the next chunk
      // in flight while one is computed (the 128K-key decode: 86.6 -> 84.9 us).  Both
      // register sets are then live at once: more than 256 registers, one workgroup per CU
      // (with many workgroups, as B=128 x 8 KV heads x 4096 keys, 0.9 % slower; B=16 x 8 x
      // 32768 keys at 2 splits 2.2 % faster).
      const int t0 = chunk_rows(0);
      const int t1 = chunk_rows(1);
      int t2 = chunk_rows(2);
      load(t0, ca);
      int t3 = chunk_rows(3);
      load(t1, cb_);
      int i = 0;
      for (; i + 1 < my_chunks; i += 2) {
        const int t4 = chunk_rows(i + 4);
        compute(i, ca);
        load(t2, ca);
        const int t5 = chunk_rows(i + 5);
        compute(i + 1, cb_);
        load(t3, cb_);
        t2 = t4;
        t3 = t5;
      }
      if (i < my_chunks) compute(i, ca);
    } else {
      // Table rows fetched one chunk earlier still, each lookup issued ahead of the K/V loads
      // that go out with it: vector loads complete in order, so a lookup issued after them
      // could only be used once they had all landed (paged B=64 decode: 4 splits 54.9 -> 52.6
      // us, 8 splits 53.2 -> 52.5).  (The contiguous loop's structure measured slower here:
      // 50.7 -> 57.4 us.)
      int rows_next = chunk_rows(0);
      int rows_after = chunk_rows(1);
      load(rows_next, ca);
      rows_next = rows_after;
      rows_after = chunk_rows(2);
      int i = 0;
      for (; i + 1 < my_chunks; i += 2) {
        const int rows_3 = chunk_rows(i + 3);
        load(rows_next, cb_);
        rows_next = rows_after;
        rows_after = rows_3;
        compute(i, ca);
        const int rows_4 = chunk_rows(i + 4);
        if (i + 2 < my_chunks) load(rows_next, ca);
        rows_next = rows_after;
        rows_after = rows_4;
        compute(i + 1, cb_);
      }
      if (i < my_chunks) compute(i, ca);
    }
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
  const int rr = zc * kDecRows + row;
  const bool has_row = rr < R;
  float out[CPT];
  float lse = kNegInf;
#pragma unroll
  for (int i = 0; i < CPT; ++i) out[i] = 0.f;
  if (has_row) {
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, Mw[w * kDecRows + row]);
    if (M != kNegInf) {
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
  }
  // rows of one group are consecutive rows of [B, H_q, T]
  const size_t grow0 = ((size_t)b * H_q + (size_t)hk * g) * T + (size_t)zc * kDecRows;
  const size_t grow = grow0 + row;
  auto store_out = [&](const float (&v)[CPT], float l) {
    OutT* Orow = O + grow * D + cpart * CPT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) Orow[i] = (OutT)v[i];
    if (LSE != nullptr && cpart == 0) LSE[grow] = l;
  };
  if (ns == 1) {
    if (has_row) store_out(out, lse);
    return;
  }
  if (has_row) {
    float* Orow = O_part + ((size_t)split * rows_total + grow) * D + cpart * CPT;
#pragma unroll
    for (int i = 0; i < CPT; i += 4) *reinterpret_cast<f32x4*>(Orow + i) = f32x4{out[i], out[i + 1], out[i + 2], out[i + 3]};
    if (cpart == 0) LSE_part[(size_t)split * rows_total + grow] = lse;
  }
  if (flags == nullptr) return;  // the merge kernel follows

  // ---- the LSE merge inside the kernel (all splits of the group share this XCD's L2) ----
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial stores have reached L2
  __syncthreads();                                    // and every other thread's
  int* last = reinterpret_cast<int*>(smem);           // the carries above are read: reuse
  if (wave == 0) {
    uint32_t* gf = flags + (size_t)group * ns;
    if (lane == 0) gf[split] = token;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    bool all = true;
    for (int s0 = 0; s0 < ns; s0 += 64) {
      const int sp = s0 + lane;
      const uint32_t f = sp < ns ? read_at_l2(gf + sp) : token;
      all = all && !wave_any(f != token);
    }
    // the next call may carry the same token (a replayed graph does): leave the flags at 0
    if (all)
      for (int sp = lane; sp < ns; sp += 64) gf[sp] = 0u;
    if (lane == 0) *last = all ? 1 : 0;
  }
  __syncthreads();
  if (*last == 0) return;

  // The merge.  A group has nrow <= 16 rows; with few rows and more than 8 splits the 16 row
  // slots of the workgroup form nsub shares (2 or 4) that divide the splits between them
  // (share k takes splits k, k + nsub, ...), and the shares of a row then meet in LDS by the
  // same rule.  Within a share: m* = max of lse_s, running, in rounds of 8 splits whose loads
  // go out together.  The partial rows are plain loads: a row of d floats fills whole cache
  // lines of its own and only this group's merge reads it, so no L1 of this XCD can hold an
  // old copy.  The lse values (4 bytes per row; other groups' rows share their lines) are
  // read at the L2.
  const int nrow = min(kDecRows, R - zc * kDecRows);
  const int nsub_rows = nrow <= 4 ? 4 : (nrow <= 8 ? 2 : 1);   // shares the row slots allow
  const int nsub = ns <= 8 ? 1 : (ns <= 16 || nsub_rows < 4 ? min(2, nsub_rows) : 4);
  const int rps = kDecRows / nsub;          // row slots per share
  const int sub = row / rps;
  const int mrow = row - sub * rps;         // the group row this thread merges
  const bool mrow_ok = mrow < nrow;
  const size_t mgrow = grow0 + (mrow_ok ? mrow : 0);  // clamped: slots past the rows load row 0
  float m = kNegInf, wsum = 0.f, acc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) acc[i] = 0.f;
  for (int s0 = sub; s0 < ns; s0 += 8 * nsub) {
    f32x4 v[8][CPT / 4];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = s0 + nsub * u;
#pragma unroll
      for (int i = 0; i < CPT / 4; ++i) v[u][i] = f32x4{};
      if (sp < ns) {   // a round may run past the last split
        const f32x4* Op = reinterpret_cast<const f32x4*>(O_part + ((size_t)sp * rows_total + mgrow) * D + cpart * CPT);
#pragma unroll
        for (int i = 0; i < CPT / 4; ++i) v[u][i] = Op[i];
      }
    }
    // lane cpart < 8 of the row reads the lse of split s0 + nsub * cpart, one atomic per
    // (row, split) word (atomics on one word queue at the L2), and the row's 16 lanes share it
    const int su = s0 + nsub * (cpart & 7);
    float mine = kNegInf;
    if (cpart < 8 && su < ns && mrow_ok)
      mine = __uint_as_float(read_at_l2(reinterpret_cast<uint32_t*>(LSE_part + (size_t)su * rows_total + mgrow)));
    float ls[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      ls[u] = __shfl(mine, (lane & ~15) | u, 64);
      if (s0 + nsub * u >= ns) ls[u] = kNegInf;   // past the last split: weight 0
    }
    float mb = kNegInf;
#pragma unroll
    for (int u = 0; u < 8; ++u) mb = fmaxf(mb, ls[u]);
    const float m_new = fmaxf(m, mb);
    // no branch on m_new: the partial loads above stay in flight with the lse loads
    const float m_use = m_new == kNegInf ? 0.f : m_new;  // no key seen yet: every weight is 0
    const float rescale = exp2f_hw((m - m_use) * kLog2e);  // 0 while m = -inf
    wsum *= rescale;
#pragma unroll
    for (int i = 0; i < CPT; ++i) acc[i] *= rescale;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = exp2f_hw((ls[u] - m_use) * kLog2e);   // 0 for an empty split (lse -inf)
      wsum += w;
#pragma unroll
      for (int i = 0; i < CPT; ++i) acc[i] = __builtin_fmaf(w, v[u][i / 4][i % 4], acc[i]);
    }
    m = m_new;
  }
  auto store_row = [&](const float (&a)[CPT], float M, float W) {
    OutT* Orow = O + mgrow * D + cpart * CPT;
    const float inv = M == kNegInf ? 0.f : 1.f / W;   // no split saw a key: O = 0, LSE = -inf
#pragma unroll
    for (int i = 0; i < CPT; ++i) Orow[i] = (OutT)(a[i] * inv);
    if (LSE != nullptr && cpart == 0) LSE[mgrow] = M == kNegInf ? kNegInf : M + log2f_hw(W) * kLn2;
  };
  if (nsub == 1) {
    if (mrow_ok) store_row(acc, m, wsum);
    return;
  }
  // the shares of a row meet in LDS, combined in share order (the same bits whichever split
  // merges)
  float* Mm = reinterpret_cast<float*>(smem);     // [16 slots]
  float* Ws = Mm + kDecRows;                      // [16 slots]
  float* Ac = Ws + kDecRows;                      // [16 slots][D]
  __syncthreads();                                // every thread has read *last
  if (cpart == 0) {
    Mm[row] = m;
    Ws[row] = wsum;
  }
#pragma unroll
  for (int i = 0; i < CPT; i += 4)
    *reinterpret_cast<f32x4*>(Ac + row * D + cpart * CPT + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
  __syncthreads();
  if (sub != 0 || !mrow_ok) return;
  float M = kNegInf;
  for (int k = 0; k < nsub; ++k) M = fmaxf(M, Mm[mrow + k * rps]);
  float W = 0.f, out2[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) out2[i] = 0.f;
  if (M != kNegInf) {
    for (int k = 0; k < nsub; ++k) {
      const int sl = mrow + k * rps;
      const float wt = exp2f_hw((Mm[sl] - M) * kLog2e);   // 0 for a share that saw no key
      W = __builtin_fmaf(Ws[sl], wt, W);
#pragma unroll
      for (int i = 0; i < CPT; ++i) out2[i] = __builtin_fmaf(Ac[sl * D + cpart * CPT + i], wt, out2[i]);
    }
  }
  store_row(out2, M, W);
}

template <int D, bool PAGED, typename OutT>
static hipError_t launch_dec(const DecodeArgs& a, int n_zc, int n_groups, int n_map, int n_wg) {
  hipLaunchKernelGGL((decode_split_kernel<D, PAGED, OutT>), dim3(n_wg), dim3(kDecThreads), 0, (hipStream_t)a.stream,
                     (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (OutT*)a.O, a.LSE, a.O_part,
                     a.LSE_part, a.flags, a.token, n_map, n_groups, n_zc, a.block_table, a.page_size,
                     a.pages_per_seq, a.H_q, a.H_kv, a.T, a.N_k, a.causal, a.num_splits, a.split_len,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_dec(const DecodeArgs& a, bool out_f32, int n_zc, int n_groups, int n_map, int n_wg) {
  if (a.block_table != nullptr)
    return out_f32 ? launch_dec<D, true, float>(a, n_zc, n_groups, n_map, n_wg)
                   : launch_dec<D, true, __bf16>(a, n_zc, n_groups, n_map, n_wg);
  return out_f32 ? launch_dec<D, false, float>(a, n_zc, n_groups, n_map, n_wg)
                 : launch_dec<D, false, __bf16>(a, n_zc, n_groups, n_map, n_wg);
}

hipError_t launch_decode_split(const DecodeArgs& a, bool out_f32) {
  const int R = (a.H_q / a.H_kv) * a.T;
  const long long n_zc = (R + kDecRows - 1) / kDecRows;
  const long long n_groups = (long long)a.B * a.H_kv * n_zc;
  const int n_map = a.flags != nullptr ? a.n_map : 1;
  if (n_map < 1 || a.num_splits < 1) return hipErrorInvalidValue;
  // whole rounds of n_map groups: the workgroups of a missing group return at once
  const long long n_wg = (n_groups + n_map - 1) / n_map * n_map * a.num_splits;
  if (n_groups > 0x7fffffffLL || n_wg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.d == 128) return dispatch_dec<128>(a, out_f32, (int)n_zc, (int)n_groups, n_map, (int)n_wg);
  return dispatch_dec<64>(a, out_f32, (int)n_zc, (int)n_groups, n_map, (int)n_wg);
}

// ---- placement probe: the XCD (XCC_ID hardware register) of every workgroup index ----
__global__ __launch_bounds__(64) void xcc_probe_kernel(uint32_t* out) {
  const uint32_t xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11)) & 0xffffu;  // XCC_ID[15:0]
  if (threadIdx.x == 0) out[blockIdx.x] = xcc;
}

hipError_t launch_xcc_probe(uint32_t* out, int n_wg, void* stream) {
  hipLaunchKernelGGL(xcc_probe_kernel, dim3(n_wg), dim3(64), 0, (hipStream_t)stream, out);
  return hipGetLastError();
}

}  // namespace fa
