// FlashAttention forward, bf16 inputs, fp32 accumulation, on gfx950 MFMA.
//
// Loop order (page "Softmax and FlashAttention", "Concept", FlashAttention-2): one
// workgroup owns a block of BR query rows of one (batch, head) and streams the K/V
// tiles of BC keys past it; each BR x BC score tile lives only in registers and is folded
// into the running output with the online-softmax carries of page "Kernel visualization:
// Flash Attention 1" ("Derivation", "The tiled version"): running max m, running sum l,
// unnormalized accumulator; one division by l at the end (page "Attention kernel chains",
// chain "The online softmax on numbers"), and the per-row LSE written once.
//
// MI355X mapping:
//   * d = 128: 8 waves x 32 query rows; d = 64: 4 waves x 64 rows, as two 32-row halves
//     that share every K and V fragment read from LDS.  Scores are computed transposed,
//     S^T = K Q^T, with the 32x32x16 bf16 MFMA: K (from LDS) is the A operand, the wave's
//     Q rows (registers, loaded once) the B operand.  In the accumulator layout each lane owns ONE query row
//     (lane % 32) and 16 keys per 32-key block, so the row max is a register reduction
//     plus one exchange between the two wave halves, the row sum stays a per-lane partial
//     until the end, and the rescale factor is a per-lane scalar.
//   * O^T = V^T P^T on the same MFMA: P^T comes straight from the score registers
//     (converted to bf16); V^T fragments are read from the row-major V tile in LDS with
//     the transposing LDS read (ds_read_b64_tr_b16), so V is staged exactly like K.
//   * K/V tiles: 16-byte buffer loads that write LDS directly (no register staging), one
//     tile ahead into a double-buffered LDS ring, issued a few at a time between the
//     score MFMAs; zero past the end of the sequence; one barrier per tile.  Rows are
//     stored unpadded with a 16-byte-chunk XOR swizzle that keeps the MFMA operand reads
//     (plain for K, transposing for V) bank-conflict free.
//   * Independent accumulators are interleaved; K fragments are read two k-steps ahead of
//     the score MFMAs that consume them, V fragments one step ahead.
//   * The reference max m is only moved (and l, O rescaled) when the weights computed
//     against it would sum above 2^30 on some lane of the wave (or no reference exists yet);
//     the row max itself is then computed, otherwise never.  O = acc / l and LSE = m + ln l
//     are exact for any reference m, so this only skips work (the test is wave-uniform).  O is divided by the sum of the same bf16-rounded P the PV product
//     uses (v_dot2 against (1, 1)), so the rounding of a dominant weight (which need not
//     be 1 under a lagging max) cancels in O = sum p V / sum p; the LSE uses the fp32 sum.
//   * The wave raises its issue priority for its MFMA sections (s_setprio; causal d = 64:
//     the PV section only), so the two waves sharing a SIMD tend to alternate: one on the
//     matrix core, one on the VALU.
//   * Workgroup order: each XCD owns a range of heads and works through them head by
//     head, so the K/V re-reads of the FlashAttention-2 order hit its L2.  A causal
//     workgroup takes two query blocks, the i-th heaviest and the i-th lightest of a head,
//     so that all workgroups cost the same.
//   * Softmax in base 2: p = 2^(s * scale * log2 e - m), with m kept in the same units.
#include "fa_device.h"
#include "fa_internal.h"

// Launch shape and schedule options, fixed at build time.  The shipped values are the
// defaults; the others are built on demand to compare tile shapes and workgroup orders.
#ifndef FA_FWD_D128_WAVES
#define FA_FWD_D128_WAVES 8      // d = 128: waves of 32 query rows per workgroup (Br = 32 x waves)
#endif
#ifndef FA_FWD_D128_BC
#define FA_FWD_D128_BC 128       // d = 128, contiguous K/V: keys per K/V tile
#endif
#ifndef FA_FWD_XCD_MAP
#define FA_FWD_XCD_MAP 1         // 1: each XCD walks its own heads; 0: plain blockIdx order
#endif
#ifndef FA_FWD_D128_VPF
#define FA_FWD_D128_VPF 1        // d = 128: key steps of V^T fragments read ahead of their MFMAs
#endif
#ifndef FA_FWD_D64_VPF
#define FA_FWD_D64_VPF 1         // d = 64: the same
#endif
#ifndef FA_FWD_D128_VEARLY
#define FA_FWD_D128_VEARLY 0     // d = 128, 1: the first of those reads are issued before the softmax
#endif
#ifndef FA_FWD_D64_RH
#define FA_FWD_D64_RH 2          // d = 64, contiguous K/V: 32-row halves per wave
#endif
#ifndef FA_FWD_D64_WAVES
#define FA_FWD_D64_WAVES 4       // d = 64, contiguous K/V: waves per workgroup
#endif
#ifndef FA_FWD_D64_BC
#define FA_FWD_D64_BC 64         // d = 64, contiguous K/V: keys per K/V tile
#endif
#ifndef FA_FWD_D64_QKPRIO
#define FA_FWD_D64_QKPRIO 0      // causal d = 64, 1: the score MFMA section also raises the issue priority
#endif
#ifndef FA_FWD_D64_VEARLY
#define FA_FWD_D64_VEARLY 1      // d = 64: the same (+3 % causal)
#endif

namespace fa {

// NW waves of RH x 32 query rows per workgroup, BR = 256 rows in both launches, two waves
// per SIMD on each CU (one 8-wave workgroup at d = 128, two 4-wave ones at d = 64): every
// K/V tile staged in LDS serves 256 rows, and at d = 128 the LDS a second workgroup would
// take holds 128-key tiles instead.
// A lane's tile sum of weights, 2^(s scale log2e - m) over its keys of one row, above which
// the reference m is moved to the tile max: the weights then stay below 2^30, far inside
// fp32 and bf16 range, and the fp32 sums keep their relative precision.
constexpr float kRescaleSum = 1073741824.0f;

template <int D, int BC, int NW, int RH>
struct FwdTile {
  static constexpr int BR = 32 * NW * RH;   // query rows per workgroup (RH 32-row halves per wave)
  static constexpr int CHUNKS = D / 8;      // 16-byte chunks per row
  static constexpr int STAGE = BC * D;      // elements of one K or V stage (no padding)
  static constexpr int ROWS_PER_DMA = 1024 / (2 * D);   // rows one wave-wide 16-byte DMA fills
  static constexpr int DMA = BC * D * 2 / 1024 / NW;  // DMAs per wave per tile (K, V each)
  static constexpr int NKB = BC / 32;       // 32-key blocks per tile
  static constexpr int NCB = D / 32;        // 32-column blocks of O^T
  static_assert(DMA * 1024 * NW == BC * D * 2, "tile must split evenly over the waves");
  // Logical 16-byte chunk c of row r sits at position c ^ swz(r) of the row.  Rows are not
  // padded (a DMA fills 1 KiB contiguously); the swizzle spreads both the plain K reads
  // (16 rows, one chunk) and the transposing V reads (4 rows x 4 chunks) over all banks.
  static __device__ __forceinline__ int swz(int r) {
    return D == 128 ? ((r & 3) << 2) | ((r >> 2) & 3) : (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
};

template <int D, int BC, int NW, int RH, bool CAUSAL, bool PAGED, typename OutT>
__global__ __launch_bounds__(64 * NW, 2) void fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    OutT* __restrict__ O, float* __restrict__ LSE, int H_q, int H_kv, int N_q, int N_k,
    float scale_log2, int n_qblocks, int n_units, int total_wg,
    const int32_t* __restrict__ block_table, int page_size, int pages_per_seq, float inv_page_size) {
  using T = FwdTile<D, BC, NW, RH>;
  // Two K and two V stages as separate arrays: with the stage known at compile time the
  // compiler can tell that a tile's LDS reads do not touch the stage being refilled, and
  // does not wait for the refill before reading.
  __shared__ __attribute__((aligned(16))) __bf16 Ks0[T::STAGE], Ks1[T::STAGE];
  __shared__ __attribute__((aligned(16))) __bf16 Vs0[T::STAGE], Vs1[T::STAGE];

  // ---- which (batch, head, query block) this workgroup owns ----
  // Workgroups are dispatched round-robin over the 8 XCDs (workgroup wg runs on XCD wg % 8).
  // Each XCD gets a contiguous range of heads and works through them head by head, so the
  // K/V re-reads of the FlashAttention-2 order stay in its L2.  Causal blocks differ in
  // cost (query block i visits about i+1 tiles), so a causal workgroup takes a pair of
  // blocks, the i-th heaviest and the i-th lightest of a head: every pair costs the same,
  // and no expensive block is left to start late.
  const int wg = blockIdx.x;
  const int n_bh = total_wg / n_units;
  int bh, unit;
  if (!FA_FWD_XCD_MAP) {
    bh = wg / n_units;
    unit = wg % n_units;
  } else if ((n_bh & 7) == 0) {
    const int hpx = n_bh >> 3;            // heads per XCD
    const int x = wg & 7, idx = wg >> 3;  // XCD, and position in its dispatch order
    bh = x * hpx + idx / n_units;
    unit = idx % n_units;
  } else {
    int logical = wg;
    if ((total_wg & 7) == 0) logical = (wg & 7) * (total_wg >> 3) + (wg >> 3);  // XCD-contiguous
    bh = logical / n_units;
    unit = logical % n_units;
  }
  const int b = bh / H_q;
  const int h = bh - b * H_q;
  const int hk = h / (H_q / H_kv);
  const __bf16* Qp = Q + (size_t)bh * N_q * D;
  // contiguous K/V: this head's rows; paged: the pools (rows found through the table)
  const __bf16* Kp = PAGED ? K : K + ((size_t)b * H_kv + hk) * N_k * D;
  const __bf16* Vp = PAGED ? V : V + ((size_t)b * H_kv + hk) * N_k * D;
  const int32_t* table_b = PAGED ? block_table + (size_t)b * pages_per_seq : nullptr;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;      // k-group of the MFMA operands
  const int g16 = lane >> 4;     // 16-lane group (transposing reads)
  const int i16 = lane & 15;
  const int n_pass = (CAUSAL && 2 * unit + 1 < n_qblocks) ? 2 : 1;
  for (int pass = 0; pass < n_pass; ++pass) {
    const int qb = !CAUSAL ? unit : (pass == 0 ? n_qblocks - 1 - unit : unit);
    const int q0 = qb * T::BR;
    const int wave_row0 = q0 + wave * 32 * RH;
    int qrow[RH];  // this lane's row in each 32-row half of the wave
#pragma unroll
    for (int x = 0; x < RH; ++x) qrow[x] = wave_row0 + 32 * x + l32;
    const int shift = N_k - N_q;   // bottom-right alignment: row i sees keys j <= i + shift

    // ---- Q block: read once, kept as MFMA B fragments ----
    bf16x8 qf[RH][D / 16];
#pragma unroll
    for (int x = 0; x < RH; ++x) {
      const int qr = qrow[x] < N_q ? qrow[x] : N_q - 1;  // clamped row; zeroed below
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        qf[x][t] = *reinterpret_cast<const bf16x8*>(Qp + (size_t)qr * D + 16 * t + 8 * hh);
        if (qrow[x] >= N_q) qf[x][t] = bf16x8{};
      }
    }

    // ---- which K/V tiles this block visits ----
    int n_tiles = (N_k + BC - 1) / BC;
    if (CAUSAL) {
      const int max_key = min(q0 + T::BR - 1, N_q - 1) + shift;
      n_tiles = max_key < 0 ? 0 : min(n_tiles, max_key / BC + 1);
    }
    const int wave_last_key = min(wave_row0 + 32 * RH - 1, N_q - 1) + shift;  // causal reach of this wave
    int row_lim[RH];  // last key each of this lane's rows sees
#pragma unroll
    for (int x = 0; x < RH; ++x) row_lim[x] = CAUSAL ? min(N_k - 1, qrow[x] + shift) : N_k - 1;

    // ---- carries, per row half ----
    float m_run[RH];   // reference max (log2 units of the scaled scores)
    float l_run[RH];   // this lane's partial sum of p over its keys (fp32 p: for the LSE)
    float lb_run[RH];  // the same sum over the bf16-rounded p the PV product uses (for O)
    f32x16 o[RH][T::NCB];
#pragma unroll
    for (int x = 0; x < RH; ++x) {
      m_run[x] = kNegInf;
      l_run[x] = 0.f;
      lb_run[x] = 0.f;
#pragma unroll
      for (int cb = 0; cb < T::NCB; ++cb) o[x][cb] = f32x16{};
    }

    // ---- K/V staging: global -> LDS directly (16-byte buffer loads with an LDS target) ----
    // Wave w's DMA i fills rows ROWS_PER_DMA * (DMA * w + i) + lane / CHUNKS; the lane fetches
    // the logical chunk that belongs at its position.  The descriptor starts at the tile and
    // ends at N_k: rows past the end of the sequence arrive as zeros (K: scores that get
    // masked; V: 0 * V = 0).
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t dma_off[T::DMA];
#pragma unroll
    for (int i = 0; i < T::DMA; ++i) {
      const int r = T::ROWS_PER_DMA * (T::DMA * wave + i) + lane / T::CHUNKS;
      const int pos = lane % T::CHUNKS;
      dma_off[i] = (uint32_t)(r * D + 8 * (pos ^ T::swz(r))) * 2u;
    }
    // DMA i (0 .. 2*DMA-1) of tile j: the K rows first, then the V rows.  Contiguous K/V:
    // buffer loads whose descriptor starts at the tile and ends at N_k, so rows past the end
    // of the sequence arrive as zeros.  Paged K/V (page "Attention kernel chains", chain
    // "The block-table cost of paged attention"): key j of sequence b is slot j % page_size
    // of pool page block_table[b][j / page_size]; each lane loads its row from its own
    // address, keys past the end are clamped to the last key (masked like any other), and
    // the table entries of a tile are read two tiles ahead so the dependent load is never
    // waited for.
    auto tile_rsrc = [&](const __bf16* base, int j) {
      const int kbase = j * BC;
      return make_rsrc(base + (size_t)kbase * D, range_bytes((long long)N_k - kbase, D * 2));
    };
    int dma_row[T::DMA];        // paged: tile row of this lane's DMA i
    uint32_t dma_chunk[T::DMA]; // paged: byte offset of its 16-byte chunk within the row
#pragma unroll
    for (int i = 0; i < T::DMA; ++i) {
      dma_row[i] = T::ROWS_PER_DMA * (T::DMA * wave + i) + lane / T::CHUNKS;
      dma_chunk[i] = (uint32_t)(16 * ((lane % T::CHUNKS) ^ T::swz(dma_row[i])));
    }
    auto key_page = [&](int key) {  // key / page_size, exact for key < 2^24
      int q = (int)((float)key * inv_page_size);
      q -= q * page_size > key ? 1 : 0;
      q += (q + 1) * page_size <= key ? 1 : 0;
      return q;
    };
    auto read_pages = [&](int j, int (&pg)[T::DMA]) {
#pragma unroll
      for (int i = 0; i < T::DMA; ++i) pg[i] = table_b[key_page(min(j * BC + dma_row[i], N_k - 1))];
    };
    auto pool_offset = [&](int j, const int (&pg)[T::DMA], int i) {  // bytes
      const int key = min(j * BC + dma_row[i], N_k - 1);
      const long long prow = (long long)pg[i] * page_size + (key - key_page(key) * page_size);
      return (size_t)(prow * H_kv + hk) * (D * 2) + dma_chunk[i];
    };
    auto dma = [&](int i, int j, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, const int (&pg)[T::DMA],
                   __bf16* ks, __bf16* vs) {
      const int ii = i % T::DMA;
      __bf16* dst = (i < T::DMA ? ks : vs) + (T::DMA * wave_u + ii) * 512;
      if constexpr (PAGED) {
        const char* src = reinterpret_cast<const char*>(i < T::DMA ? Kp : Vp) + pool_offset(j, pg, ii);
        global_load16_lds(src, dst);
      } else {
        buffer_load16_lds(i < T::DMA ? kr : vr, dma_off[ii], dst);
      }
    };
    int pg_next[T::DMA], pg_after[T::DMA];  // paged: pages of tiles j+1 and j+2
    // LDS read offsets (elements) of this lane's MFMA operands in a stage.  K fragment of
    // 32-key block kb, k-step t: row kb*32 + l32, logical chunk 2t + hh.  V^T fragment of
    // column block cb, key step u, half r: lane (16-group g16, index i16) points at key
    // 16u + 8r + 4hh + i16/4, columns 32cb + 16(g16%2) + 4(i16%4) .. +3.  The swizzle of a
    // row depends only on its index mod 16, so kb and u enter as plain immediates.
    int koff[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) koff[t] = l32 * D + 8 * ((2 * t + hh) ^ T::swz(l32));
    int voff[2][T::NCB];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int cb = 0; cb < T::NCB; ++cb) {
        const int row = 8 * r + 4 * hh + (i16 >> 2);
        const int c = 4 * cb + 2 * (g16 & 1) + ((i16 & 3) >> 1);
        voff[r][cb] = row * D + 8 * (c ^ T::swz(row)) + 4 * (i16 & 1);
      }

    if (n_tiles > 0) {
      const auto kr = tile_rsrc(Kp, 0), vr = tile_rsrc(Vp, 0);
      if constexpr (PAGED) {
        read_pages(0, pg_next);
        read_pages(1, pg_after);
      }
#pragma unroll
      for (int i = 0; i < 2 * T::DMA; ++i) dma(i, 0, kr, vr, pg_next, Ks0, Vs0);
      if constexpr (PAGED) {
#pragma unroll
        for (int i = 0; i < T::DMA; ++i) pg_next[i] = pg_after[i];
      }
    }
    wait_vmem();
    __syncthreads();

    // Tile j reads stage (ks, vs) while tile j+1 streams into (ks_next, vs_next), which
    // tile j-1 read before the last barrier.
    auto tile_step = [&](int j, const __bf16* ks, const __bf16* vs, __bf16* ks_next, __bf16* vs_next) {
      // Tile j+1 streams into (ks_next, vs_next), which tile j-1 read before the last
      // barrier.  Its DMAs are issued a few at a time between the score MFMAs: a wave that
      // issued them all at once would sit at the first one whose queue slot is not free.
      // (After the last tile the descriptors are empty: the stage gets zeros nobody reads.)
      const auto kr_next = tile_rsrc(Kp, j + 1), vr_next = tile_rsrc(Vp, j + 1);
      if constexpr (PAGED) read_pages(j + 2, pg_after);  // lands during this tile
      constexpr int NDMA = 2 * T::DMA;
      constexpr int DMA_PER_STEP = (NDMA + D / 16 - 1) / (D / 16);
      const int kbase = j * BC;

      if (!CAUSAL || kbase <= wave_last_key) {
        // ---- S^T = K_j Q^T: NKB independent accumulators, fragments read one step ahead ----
        // MFMA section: issue ahead of the other wave on this SIMD (causal d = 64: only the PV
        // section is raised, 2 % faster there)
        if constexpr (FA_FWD_D64_QKPRIO || D != 64 || !CAUSAL) __builtin_amdgcn_s_setprio(1);
        f32x16 s[RH][T::NKB];
#pragma unroll
        for (int x = 0; x < RH; ++x)
#pragma unroll
          for (int kb = 0; kb < T::NKB; ++kb) s[x][kb] = f32x16{};
        bf16x8 kf[2][T::NKB];
#pragma unroll
        for (int kb = 0; kb < T::NKB; ++kb)
          kf[0][kb] = *reinterpret_cast<const bf16x8*>(ks + kb * 32 * D + koff[0]);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          if (t + 1 < D / 16) {
#pragma unroll
            for (int kb = 0; kb < T::NKB; ++kb)
              kf[(t + 1) & 1][kb] =
                  *reinterpret_cast<const bf16x8*>(ks + kb * 32 * D + koff[t + 1]);
          }
#pragma unroll
          for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
            for (int x = 0; x < RH; ++x) s[x][kb] = mfma32x32x16(kf[t & 1][kb], qf[x][t], s[x][kb]);
#pragma unroll
          for (int i = t * DMA_PER_STEP; i < (t + 1) * DMA_PER_STEP && i < NDMA; ++i)
            dma(i, j + 1, kr_next, vr_next, pg_next, ks_next, vs_next);
        }
        // order: fragments of two k-steps in flight ahead of the MFMAs that use them
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * T::NKB, 0);
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          __builtin_amdgcn_sched_group_barrier(0x008, T::NKB * RH, 0);
          if (t * DMA_PER_STEP < NDMA) __builtin_amdgcn_sched_group_barrier(0x020, DMA_PER_STEP, 0);
          if (t + 2 < D / 16) __builtin_amdgcn_sched_group_barrier(0x100, T::NKB, 0);
        }

        __builtin_amdgcn_s_setprio(0);
        // ---- V^T fragments through transposing LDS reads, VP key steps ahead of the PV
        // MFMAs that use them; the first VEARLY steps are requested before the softmax, so
        // their LDS latency hides behind it ----
        auto vfrag = [&](int u, int cb) {
          const __bf16* p = vs + 16 * u * D;
          return join_bf16x8(lds_read_tr16(p + voff[0][cb]), lds_read_tr16(p + voff[1][cb]));
        };
        constexpr int VP = D == 64 ? FA_FWD_D64_VPF : FA_FWD_D128_VPF;
        // (not for the paged variant, whose table addressing leaves no registers for it)
        constexpr int VEARLY = (!PAGED && (D == 64 ? FA_FWD_D64_VEARLY : FA_FWD_D128_VEARLY)) ? VP : 0;
        bf16x8 vf[VP + 1][T::NCB];
#pragma unroll
        for (int u = 0; u < VEARLY; ++u)
#pragma unroll
          for (int cb = 0; cb < T::NCB; ++cb) vf[u][cb] = vfrag(u, cb);
        bf16x8 pf[RH][BC / 16];
#pragma unroll
        for (int x = 0; x < RH; ++x) {
          // ---- mask: ragged tail and the bottom-right causal edge ----
          const bool need_mask = (kbase + BC > N_k) || (CAUSAL && kbase + BC - 1 > wave_row0 + 32 * x + shift);
          if (need_mask) {
            const int thr = row_lim[x] - kbase - 4 * hh;  // key offset in this lane's numbering
#pragma unroll
            for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (kb * 32 + 8 * (r >> 2) + (r & 3) > thr) s[x][kb][r] = kNegInf;
          }

          // ---- online softmax (base 2, lazily rescaled) ----
          // Exponentiate against the running reference m as it stands; only when a lane's
          // tile sum comes out above kRescaleSum (or no reference exists yet) is the tile max
          // taken, the carries rescaled to it and the exponentials redone.  Any reference
          // gives the same O and LSE; this one only moves when the weights would grow large.
          auto exps = [&](float m_use) {
            float sum = 0.f;
#pragma unroll
            for (int u = 0; u < BC / 16; ++u) {
              const f32x16& sk = s[x][u >> 1];
              const int r0 = (u & 1) * 8;
              f32x8 e;
#pragma unroll
              for (int r = 0; r < 8; ++r) {
                e[r] = exp2f_hw(__builtin_fmaf(sk[r0 + r], scale_log2, -m_use));
                sum += e[r];
              }
              pf[x][u] = to_bf16x8(e);  // P^T operands (bf16, RNE) of the BC/16 key steps
            }
            return sum;
          };
          float tsum = m_run[x] == kNegInf ? 0.f : exps(m_run[x]);
          if (wave_any(m_run[x] == kNegInf || !(tsum <= kRescaleSum))) {
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < T::NKB; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[x][kb][r]);
            mx = max_halves(mx) * scale_log2;
            const float m_new = fmaxf(m_run[x], mx);
            if (m_new != m_run[x]) {
              // 0 when m_run = -inf; 1 for a row that still has no key (both -inf)
              const float alpha = m_new == kNegInf ? 1.f : exp2f_hw(m_run[x] - m_new);
              l_run[x] *= alpha;
              lb_run[x] *= alpha;
#pragma unroll
              for (int cb = 0; cb < T::NCB; ++cb) o[x][cb] *= alpha;
              m_run[x] = m_new;
            }
            tsum = exps(m_run[x] == kNegInf ? 0.f : m_run[x]);  // a row with no key yet: all p = 0
          }
          l_run[x] += tsum;
          // lb sums exactly the bf16 weights the PV product uses
#pragma unroll
          for (int u = 0; u < BC / 16; ++u) lb_run[x] = sum_bf16x8(pf[x][u], lb_run[x]);
        }

        // ---- O^T += V_j^T P^T ----
#pragma unroll
        for (int u = VEARLY; u < VP; ++u)
#pragma unroll
          for (int cb = 0; cb < T::NCB; ++cb) vf[u][cb] = vfrag(u, cb);
        __builtin_amdgcn_s_setprio(1);  // MFMA section: issue ahead of the other wave on this SIMD
#pragma unroll
        for (int u = 0; u < BC / 16; ++u) {
          if (u + VP < BC / 16) {
#pragma unroll
            for (int cb = 0; cb < T::NCB; ++cb) vf[(u + VP) % (VP + 1)][cb] = vfrag(u + VP, cb);
          }
#pragma unroll
          for (int cb = 0; cb < T::NCB; ++cb)
#pragma unroll
            for (int x = 0; x < RH; ++x) o[x][cb] = mfma32x32x16(vf[u % (VP + 1)][cb], pf[x][u], o[x][cb]);
        }
        __builtin_amdgcn_s_setprio(0);
      } else {
#pragma unroll
        for (int i = 0; i < NDMA; ++i) dma(i, j + 1, kr_next, vr_next, pg_next, ks_next, vs_next);
      }
      if constexpr (PAGED) {
#pragma unroll
        for (int i = 0; i < T::DMA; ++i) pg_next[i] = pg_after[i];
      }
      wait_vmem();      // this wave's DMAs of tile j+1 have landed
      __syncthreads();  // everyone's have; stage (ks, vs) is free for tile j+2
    };
    for (int j = 0; j < n_tiles; j += 2) {
      tile_step(j, Ks0, Vs0, Ks1, Vs1);
      if (j + 1 < n_tiles) tile_step(j + 1, Ks1, Vs1, Ks0, Vs0);
    }

    // ---- epilogue: one division, O and LSE written once ----
    if constexpr (sizeof(OutT) == 2 && !PAGED && NW * 32 * D <= 2 * T::STAGE) {
      // bf16 rows go out through LDS so each store writes whole rows (1 KB of consecutive
      // rows per instruction) instead of 8 bytes of 32 rows (+2-3 % at d = 128).  Each
      // 32-row half of the wave's block (32 x D) takes 64*D bytes of stage 1: every wave has
      // finished reading it (the tile loop's last barrier), and the next causal block
      // refills it only after its first barrier.
      constexpr int CH = D / 8;                   // 16-byte chunks per row
      constexpr int RPI = 64 / CH;                // rows per wave-wide 16-byte access
      constexpr int WPS = T::STAGE / (32 * D);    // waves per stage array
      __bf16* ost = (wave < WPS ? Ks1 : Vs1) + (wave % WPS) * (32 * D);
      // the lane-dependent offsets below are made here, not hoisted out of the pass loop
      // (kept live across the main loop they would crowd its registers)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int r32 = ln & 31, hh2 = ln >> 5;
#pragma unroll
      for (int x = 0; x < RH; ++x) {
        const float l_tot = l_run[x] + shfl_xor_f(l_run[x], 32);
        const float lb_tot = lb_run[x] + shfl_xor_f(lb_run[x], 32);
        const float inv = lb_tot > 0.f ? 1.f / lb_tot : 0.f;
        if (x > 0) {  // the previous half has been read back
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
#pragma unroll
        for (int cb = 0; cb < T::NCB; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v = {o[x][cb][4 * g] * inv, o[x][cb][4 * g + 1] * inv, o[x][cb][4 * g + 2] * inv,
                             o[x][cb][4 * g + 3] * inv};
            // chunk cb*4+g of row r32, XOR-swizzled by the row so the 32 rows spread over the banks
            *reinterpret_cast<bf16x4*>(ost + r32 * D + (((cb * 4 + g) ^ (r32 & (CH - 1))) << 3) + 4 * hh2) =
                __builtin_convertvector(v, bf16x4);
          }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int row0 = wave_row0 + 32 * x;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const int row = RPI * i + ln / CH, ch = ln % CH;
          const u32x4 val = *reinterpret_cast<const u32x4*>(ost + row * D + ((ch ^ (row & (CH - 1))) << 3));
          if (row0 + row < N_q)
            *reinterpret_cast<u32x4*>(O + ((size_t)bh * N_q + row0 + row) * D + ch * 8) = val;
        }
        if (LSE != nullptr && hh == 0 && qrow[x] < N_q)
          LSE[(size_t)bh * N_q + qrow[x]] = l_tot > 0.f ? (m_run[x] + log2f_hw(l_tot)) * kLn2 : kNegInf;
      }
      continue;
    }
#pragma unroll
    for (int x = 0; x < RH; ++x) {
      const float l_tot = l_run[x] + shfl_xor_f(l_run[x], 32);  // the two wave halves hold one row's keys
      const float lb_tot = lb_run[x] + shfl_xor_f(lb_run[x], 32);
      if (qrow[x] < N_q) {
        const float inv = lb_tot > 0.f ? 1.f / lb_tot : 0.f;
        OutT* Orow = O + ((size_t)bh * N_q + qrow[x]) * D;
#pragma unroll
        for (int cb = 0; cb < T::NCB; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c = cb * 32 + 8 * g + 4 * hh;
            const f32x4 v = {o[x][cb][4 * g] * inv, o[x][cb][4 * g + 1] * inv, o[x][cb][4 * g + 2] * inv,
                             o[x][cb][4 * g + 3] * inv};
            if constexpr (sizeof(OutT) == 4) {
              *reinterpret_cast<f32x4*>(Orow + c) = v;
            } else {
              *reinterpret_cast<bf16x4*>(Orow + c) = __builtin_convertvector(v, bf16x4);
            }
          }
        if (LSE != nullptr && hh == 0) {
          LSE[(size_t)bh * N_q + qrow[x]] = l_tot > 0.f ? (m_run[x] + log2f_hw(l_tot)) * kLn2 : kNegInf;
        }
      }
    }
  }
}

template <int D, int BC, bool CAUSAL, bool PAGED, typename OutT>
static hipError_t launch(const FwdArgs& a, const int32_t* block_table, int page_size, int pages_per_seq) {
  // d = 128: 8 waves of 32 rows (4 waves measured 1-5 % slower).  d = 64: 4 waves of two
  // 32-row halves, so each K or V fragment read from LDS feeds two MFMAs; the registers
  // this takes fit at d = 64 only
  constexpr int RH = D == 64 ? (PAGED ? 2 : FA_FWD_D64_RH) : 1;
  constexpr int NW = D == 64 ? (PAGED ? 4 : FA_FWD_D64_WAVES) : (PAGED ? 8 : FA_FWD_D128_WAVES);
  constexpr int BR = FwdTile<D, BC, NW, RH>::BR;
  const int n_qblocks = (a.N_q + BR - 1) / BR;
  const int n_units = CAUSAL ? (n_qblocks + 1) / 2 : n_qblocks;  // causal: block pairs
  const long long total = (long long)a.B * a.H_q * n_units;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, NW, RH, CAUSAL, PAGED, OutT>), dim3((unsigned)total), dim3(64 * NW), 0,
                     (hipStream_t)a.stream, (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V,
                     (OutT*)a.O, a.LSE, a.H_q, a.H_kv, a.N_q, a.N_k, a.scale * kLog2e, n_qblocks,
                     n_units, (int)total, block_table, page_size, pages_per_seq,
                     page_size > 0 ? 1.f / (float)page_size : 0.f);
  return hipGetLastError();
}

template <int D, bool PAGED>
static hipError_t dispatch_out(const FwdArgs& a, bool out_f32, const int32_t* bt, int ps, int pps) {
  // key tile: 128 keys for contiguous K/V at d = 128 (half the barriers per key); 64 keys for
  // the paged variant at d = 128 (its per-lane page addressing would not fit the registers
  // otherwise) and at d = 64 (two row halves per wave)
  constexpr int BC = PAGED ? 64 : (D == 128 ? FA_FWD_D128_BC : FA_FWD_D64_BC);
  if (a.causal)
    return out_f32 ? launch<D, BC, true, PAGED, float>(a, bt, ps, pps) : launch<D, BC, true, PAGED, __bf16>(a, bt, ps, pps);
  return out_f32 ? launch<D, BC, false, PAGED, float>(a, bt, ps, pps) : launch<D, BC, false, PAGED, __bf16>(a, bt, ps, pps);
}

hipError_t launch_fwd_bf16(const FwdArgs& a, bool out_f32) {
  if (a.d == 128) return dispatch_out<128, false>(a, out_f32, nullptr, 0, 0);
  return dispatch_out<64, false>(a, out_f32, nullptr, 0, 0);
}

hipError_t launch_fwd_bf16_paged(const FwdArgs& a, bool out_f32, const int32_t* block_table, int page_size,
                                 int pages_per_seq) {
  if (a.d == 128) return dispatch_out<128, true>(a, out_f32, block_table, page_size, pages_per_seq);
  return dispatch_out<64, true>(a, out_f32, block_table, page_size, pages_per_seq);
}

}  // namespace fa
