// The C ABI declared in include/fa.h: argument validation, kernel selection and launch
// on the caller's stream.  Nothing here allocates or frees, every check runs before the
// first HIP call, so an invalid call enqueues nothing, and nothing synchronises except the
// placement probe, once per GPU, at its first split decode call (placement_period).
#include <math.h>

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_internal.h"

namespace {

constexpr int kNumCU = 256;             // MI355X compute units
constexpr int kMaxPlacementPeriod = 64;  // largest workgroup placement period the probe accepts
constexpr int kResidentDecodeWgPerCu = 2;  // decode workgroups one CU holds at once

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

int status_of(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// A tensor of zero elements may be passed as NULL; any other must not.
bool present(const void* p, bool nonempty) { return p != nullptr || !nonempty; }

// a * b * c <= 2^31 - 1 for non-negative ints, without overflowing along the way
bool product_fits31(long long a, long long b, long long c) {
  const long long lim = 0x7fffffffLL;
  if (a == 0 || b == 0 || c == 0) return true;
  return a <= lim / b && a * b <= lim / c;
}

// Sizes: B, heads and d at least 1; the sequence lengths may be 0 (empty inputs).
int check_heads(int B, int H_q, int H_kv, int n_q, int n_k, int d) {
  if (B < 1 || H_q < 1 || H_kv < 1 || n_q < 0 || n_k < 0 || d < 1) return FA_ERR_BAD_SHAPE;
  if (H_q % H_kv != 0) return FA_ERR_BAD_SHAPE;
  // every row index (B*H*N) must fit a 32-bit int; the element offsets are 64-bit
  if (!product_fits31(B, H_q, n_q) || !product_fits31(B, H_kv, n_k)) return FA_ERR_BAD_SHAPE;
  return FA_OK;
}

// Keys per split: ceil(N_k / ns) rounded up to the decode chunk.
int split_len_of(int n_k, int ns) {
  const long long per = ((long long)n_k + ns - 1) / ns;
  return (int)((per + fa::kDecodeChunk - 1) / fa::kDecodeChunk * fa::kDecodeChunk);
}

// Workgroup groups of the decode kernel: one per (batch, KV head, 16 stacked query rows).
size_t decode_groups(int B, int H_q, int H_kv, int T) {
  return (size_t)B * H_kv * (((size_t)(H_q / H_kv) * T + fa::kDecodeRows - 1) / fa::kDecodeRows);
}

// A completion token unique to each decode call of the process (never 0, the value the
// kernel leaves its flags at).
uint32_t next_token() {
  static std::atomic<uint32_t> counter{0x5eed0000u};
  uint32_t t;
  do t = counter.fetch_add(1, std::memory_order_relaxed) + 1; while (t == 0);
  return t;
}

// Whether FA_MERGE_AUTO merges inside the decode kernel: all workgroups resident at once,
// and the merging workgroup's shares (up to 16 / rows of the group, at most 4) cover the
// splits in one round of 8 each.  Measured (paged B=64 decode, 8/1 heads; 128K-key decode,
// 32/8 heads; event-timed): 4 splits 51.3 us inside against the merge kernel's 52.5, 32 splits
// of the 128K decode 86.7 against 87.6; 16 splits of the paged decode (1024 workgroups)
// 60.4 against 54.1 and 64 splits of the 128K decode 95.8 against 90.3 lose.
bool in_kernel_pays(int B, int H_q, int H_kv, int T, int ns) {
  const long long rows = (long long)(H_q / H_kv) * T;
  const long long nrow = rows < fa::kDecodeRows ? rows : fa::kDecodeRows;
  const long long shares = nrow <= 4 ? 4 : (nrow <= 8 ? 2 : 1);
  const double wgs = (double)decode_groups(B, H_q, H_kv, T) * ns;
  return wgs <= (double)kNumCU * kResidentDecodeWgPerCu && ns <= 8 * shares;
}

// The decode grid (one dimension): the workgroup groups rounded up to whole placement rounds
// of at most kMaxPlacementPeriod, times the splits, must stay below 2^31.
bool grid_fits(int B, int H_q, int H_kv, int T, int ns) {
  const long long groups = (long long)decode_groups(B, H_q, H_kv, T);
  return (groups + kMaxPlacementPeriod - 1) / kMaxPlacementPeriod * kMaxPlacementPeriod * ns <= 0x7fffffffLL;
}

int auto_splits(int B, int H_q, int H_kv, int T, int N_k) {
  const long long row_chunks = ((long long)(H_q / H_kv) * T + 15) / 16;
  if (!product_fits31(B, H_kv, row_chunks)) return 1;       // far more workgroups than CUs already
  const long long base = (long long)B * H_kv * row_chunks;  // workgroups without splitting
  // One split workgroup per CU: one wave of workgroups, all resident, each streaming as long
  // a split as possible.  More splits only add partials to merge.  (Two workgroups per CU for
  // splits under 4096 keys measured better before the block-table lookups went out ahead of
  // the K/V loads and the merge moved into the kernel; since then the paged B=64 decode takes
  // 50.9 us at 4 splits and 52.7 us at 8.)
  const long long target = kNumCU;
  if (base < 1) return 1;  // no query row
  if (base >= target) return 1;
  long long ns = target / base;
  const long long max_useful = ((long long)N_k + 4 * fa::kDecodeChunk - 1) / (4 * fa::kDecodeChunk);
  if (ns > max_useful) ns = max_useful;  // at least one chunk per wave
  if (ns < 1) ns = 1;
  return (int)ns;
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL_PTR: return "FA_ERR_NULL_PTR: a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "FA_ERR_BAD_SHAPE: invalid size, head grouping, scale, split or page argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension or dtype not supported";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_ALIGNMENT: return "FA_ERR_ALIGNMENT: tensor pointer not 16-byte aligned";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error";
    default: return "unknown fa_status";
  }
}

int fa_version(void) { return 102; }

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H_q, int H_kv,
           int N_q, int N_k, int d, float scale, int causal, int dtype, void* stream) {
  if (!present(Q, N_q > 0) || !present(O, N_q > 0) || !present(K, N_k > 0) || !present(V, N_k > 0))
    return FA_ERR_NULL_PTR;
  int st = check_heads(B, H_q, H_kv, N_q, N_k, d);
  if (st != FA_OK) return st;
  if (!(scale > 0.f) || !isfinite(scale) || (causal != 0 && causal != 1)) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16 && dtype != FA_FP32 && dtype != FA_BF16_IN_FP32_OUT) return FA_ERR_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || (LSE && !aligned4(LSE)))
    return FA_ERR_ALIGNMENT;
  if (N_q == 0) return FA_OK;  // no query row: nothing to write (N_k == 0: every row gets O = 0, LSE = -inf)
  fa::FwdArgs a{Q, K, V, O, LSE, B, H_q, H_kv, N_q, N_k, d, scale, causal, stream};
  if (dtype == FA_FP32) return status_of(fa::launch_fwd_fp32(a));
  return status_of(fa::launch_fwd_bf16(a, dtype == FA_BF16_IN_FP32_OUT));
}

int fa_fwd_paged(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H_q, int H_kv,
                 int N_q, int N_k, int d, float scale, int causal, const int32_t* block_table, int page_size,
                 int pages_per_seq, int dtype, void* stream) {
  if (!present(Q, N_q > 0) || !present(O, N_q > 0) || !present(K, N_k > 0) || !present(V, N_k > 0) ||
      !present(block_table, N_k > 0))
    return FA_ERR_NULL_PTR;
  int st = check_heads(B, H_q, H_kv, N_q, N_k, d);
  if (st != FA_OK) return st;
  if (!(scale > 0.f) || !isfinite(scale) || (causal != 0 && causal != 1)) return FA_ERR_BAD_SHAPE;
  if (page_size < 1 || pages_per_seq < 0 || (long long)pages_per_seq * page_size < N_k) return FA_ERR_BAD_SHAPE;
  if ((long long)B * pages_per_seq > 0x7fffffffLL || N_k >= (1 << 24)) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16 && dtype != FA_BF16_IN_FP32_OUT) return FA_ERR_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || (LSE && !aligned4(LSE)) ||
      !aligned4(block_table))
    return FA_ERR_ALIGNMENT;
  if (N_q == 0) return FA_OK;
  fa::FwdArgs a{Q, K, V, O, LSE, B, H_q, H_kv, N_q, N_k, d, scale, causal, stream};
  return status_of(fa::launch_fwd_bf16_paged(a, dtype == FA_BF16_IN_FP32_OUT, block_table, page_size, pages_per_seq));
}

size_t fa_bwd_workspace_bytes(int B, int H_q, int N_q) {
  if (B < 1 || H_q < 1 || N_q < 1 || !product_fits31(B, H_q, N_q)) return 0;  // N_q = 0: none
  return fa::bwd_workspace_bytes(B, H_q, N_q);
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE, void* dQ,
           void* dK, void* dV, int B, int H_q, int H_kv, int N_q, int N_k, int d, float scale, int causal,
           void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  const bool hq = N_q > 0, hk = N_k > 0;
  if (!present(Q, hq) || !present(O, hq) || !present(dO, hq) || !present(LSE, hq) || !present(dQ, hq) ||
      !present(K, hk) || !present(V, hk) || !present(dK, hk) || !present(dV, hk))
    return FA_ERR_NULL_PTR;
  int st = check_heads(B, H_q, H_kv, N_q, N_k, d);
  if (st != FA_OK) return st;
  if (!(scale > 0.f) || !isfinite(scale) || (causal != 0 && causal != 1)) return FA_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16 && dtype != FA_BF16_IN_FP32_OUT) return FA_ERR_UNSUPPORTED;
  const size_t need = N_q > 0 ? fa::bwd_workspace_bytes(B, H_q, N_q) : 0;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) || !aligned4(LSE) ||
      !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) || !aligned16(workspace))
    return FA_ERR_ALIGNMENT;
  if (N_q == 0 && N_k == 0) return FA_OK;
  fa::BwdArgs a{Q, K, V, O, dO, LSE, dQ, dK, dV, B, H_q, H_kv, N_q, N_k, d, scale, causal, workspace, stream};
  return status_of(fa::launch_bwd(a, dtype == FA_BF16_IN_FP32_OUT));
}

int fa_decode_num_splits(int B, int H_q, int H_kv, int T, int N_k, int d) {
  if (check_heads(B, H_q, H_kv, T, N_k, d) != FA_OK) return 0;
  return auto_splits(B, H_q, H_kv, T, N_k);
}

size_t fa_decode_workspace_bytes(int B, int H_q, int H_kv, int T, int N_k, int d, int num_splits) {
  if (check_heads(B, H_q, H_kv, T, N_k, d) != FA_OK || num_splits < 0) return 0;
  const int ns = num_splits == 0 ? auto_splits(B, H_q, H_kv, T, N_k) : num_splits;
  if (ns <= 1) return 0;
  const size_t rows = (size_t)B * H_q * T;
  if ((long long)ns * (long long)rows > 0x7fffffffLL) return 0;  // partial index past 32 bits: rejected
  if (!grid_fits(B, H_q, H_kv, T, ns)) return 0;
  return round256((size_t)ns * rows * d * sizeof(float)) + round256((size_t)ns * rows * sizeof(float)) +
         round256((size_t)ns * decode_groups(B, H_q, H_kv, T) * sizeof(uint32_t));
}

}  // extern "C"

// The partial results of fa_decode_splitkv_noalloc: one array per GPU, resident for the
// process's lifetime, shared by every call on that GPU.  In host code its name is only a
// stand-in: the device address of each GPU's copy comes from hipGetSymbolAddress
// (scratch_on below), and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[FA_DECODE_NOALLOC_SCRATCH_BYTES];

// The placement probe's output: the XCD of each of its workgroups, per GPU (the same
// stand-in rule as `scratch`).
constexpr int kProbeWorkgroups = 1024;
static __device__ __align__(256) uint32_t xcc_probe_out[kProbeWorkgroups];

namespace {

constexpr int kMaxDevices = 64;

// GPU of `stream` (the current GPU for a NULL stream), or -1.
int device_of(void* stream) {
  int dev = -1;
  if (stream != nullptr) {
    if (hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return -1;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return -1;
  }
  return dev >= 0 && dev < kMaxDevices ? dev : -1;
}

// Device address of the array `sym` on GPU `dev`, looked up with that GPU current.
void* symbol_on(int dev, const void* sym) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, sym);
  if (cur != dev) (void)hipSetDevice(cur);
  return e == hipSuccess ? p : nullptr;
}

std::mutex placement_mutex;
int placement[kMaxDevices] = {};   // 0: not probed; -1: no usable period; p > 0: period
std::atomic<int> merge_mode{FA_MERGE_AUTO};

// The period p of the workgroup-to-XCD placement on the GPU of `stream`: every workgroup
// index L runs on the XCD of index L % p, and indices 0 .. p-1 run on p different XCDs.
// Probed once per GPU (1024 one-wave workgroups record their XCC_ID, the caller's stream is
// synchronised once); 0 when it cannot be known now (the stream is being captured into a
// graph, or a HIP call failed): the caller then uses the separate merge kernel.
int placement_period(void* stream) {
  if (merge_mode.load(std::memory_order_relaxed) == FA_MERGE_KERNEL) return 0;
  const int dev = device_of(stream);
  if (dev < 0) return 0;
  std::lock_guard<std::mutex> lock(placement_mutex);
  if (placement[dev] != 0) return placement[dev] > 0 ? placement[dev] : 0;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing((hipStream_t)stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return 0;
  uint32_t* d_out = static_cast<uint32_t*>(symbol_on(dev, HIP_SYMBOL(xcc_probe_out)));
  if (d_out == nullptr) return 0;
  uint32_t ids[kProbeWorkgroups];
  if (fa::launch_xcc_probe(d_out, kProbeWorkgroups, stream) != hipSuccess) return 0;
  if (hipMemcpyAsync(ids, d_out, sizeof(ids), hipMemcpyDeviceToHost, (hipStream_t)stream) != hipSuccess) return 0;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return 0;
  int period = -1;
  for (int p = 1; p <= kMaxPlacementPeriod && period < 0; p *= 2) {
    bool ok = true;
    for (int i = 0; i < p && ok; ++i)
      for (int j = 0; j < i && ok; ++j) ok = ids[i] != ids[j];
    for (int L = p; L < kProbeWorkgroups && ok; ++L) ok = ids[L] == ids[L % p];
    if (ok) period = p;
  }
  placement[dev] = period;
  return period > 0 ? period : 0;
}

// Validation shared by both decode entry points; on FA_OK, *ns_out holds the resolved split
// count and *need_out the partial-result bytes it takes (0 with one split).
int check_decode(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H_q, int H_kv,
                 int T, int N_k, int d, float scale, int causal, int num_splits, const int32_t* block_table,
                 int page_size, int pages_per_seq, int dtype, int* ns_out, size_t* need_out) {
  if (!present(Q, T > 0) || !present(O, T > 0) || !present(K, N_k > 0) || !present(V, N_k > 0))
    return FA_ERR_NULL_PTR;
  int st = check_heads(B, H_q, H_kv, T, N_k, d);
  if (st != FA_OK) return st;
  if (!(scale > 0.f) || !isfinite(scale) || (causal != 0 && causal != 1) || num_splits < 0) return FA_ERR_BAD_SHAPE;
  if (block_table != nullptr) {
    if (page_size < 1 || pages_per_seq < 0 || (long long)pages_per_seq * page_size < N_k) return FA_ERR_BAD_SHAPE;
    if ((long long)B * pages_per_seq > 0x7fffffffLL) return FA_ERR_BAD_SHAPE;
  }
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_BF16 && dtype != FA_BF16_IN_FP32_OUT) return FA_ERR_UNSUPPORTED;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || (LSE && !aligned4(LSE)) ||
      (block_table && !aligned4(block_table)))
    return FA_ERR_ALIGNMENT;
  const int ns = num_splits == 0 ? auto_splits(B, H_q, H_kv, T, N_k) : num_splits;
  // every partial row index (split * rows + row) must fit 32 bits, as in fa_lse_merge
  if (ns > 1 && (long long)B * H_q * T * ns > 0x7fffffffLL) return FA_ERR_BAD_SHAPE;  // B*H_q*T < 2^31 here
  if (!grid_fits(B, H_q, H_kv, T, ns)) return FA_ERR_BAD_SHAPE;
  *ns_out = ns;
  *need_out = fa_decode_workspace_bytes(B, H_q, H_kv, T, N_k, d, ns);
  return FA_OK;
}

// Launch the split kernel and, with more than one split, the merge, with the partials in
// `workspace` (laid out as fa_decode_workspace_bytes describes).
int run_decode(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H_q, int H_kv, int T,
               int N_k, int d, float scale, int causal, int ns, const int32_t* block_table, int page_size,
               int pages_per_seq, void* workspace, int dtype, void* stream) {
  if (T == 0) return FA_OK;  // no query: nothing to write (N_k == 0: O = 0, LSE = -inf)
  const size_t rows = (size_t)B * H_q * T;
  float* O_part = nullptr;
  float* LSE_part = nullptr;
  uint32_t* flags = nullptr;
  int n_map = 1;
  if (ns > 1) {
    char* w = static_cast<char*>(workspace);
    O_part = reinterpret_cast<float*>(w);
    w += round256((size_t)ns * rows * d * sizeof(float));
    LSE_part = reinterpret_cast<float*>(w);
    w += round256((size_t)ns * rows * sizeof(float));
    // With a known placement the kernel can merge the partials itself (one launch).  Its
    // merge is a chain of L2 round trips after the stream, which pays while every workgroup
    // is resident at once (no second round of workgroups waits behind a merge) and one round
    // of 8 splits per share of the merging workgroup covers the group (in_kernel_pays).
    const int mode = merge_mode.load(std::memory_order_relaxed);
    const int p = placement_period(stream);
    if (p > 0 && (mode == FA_MERGE_IN_KERNEL || in_kernel_pays(B, H_q, H_kv, T, ns))) {
      flags = reinterpret_cast<uint32_t*>(w);
      n_map = p;
    }
  }
  fa::DecodeArgs a{Q, K, V, O, LSE, B, H_q, H_kv, T, N_k, d, scale, causal, ns, split_len_of(N_k, ns),
                   block_table, page_size, pages_per_seq, O_part, LSE_part, flags,
                   flags != nullptr ? next_token() : 0u, n_map, stream};
  const bool out_f32 = dtype == FA_BF16_IN_FP32_OUT;
  hipError_t e = fa::launch_decode_split(a, out_f32);
  if (e != hipSuccess) return FA_ERR_HIP;
  if (ns > 1 && flags == nullptr) e = fa::launch_lse_merge(O_part, LSE_part, O, LSE, ns, (int)rows, d, out_f32, stream);
  return status_of(e);
}

std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the GPU `stream` belongs to (the current GPU for a NULL
// stream), looked up once per GPU with that GPU current.  NULL on any HIP error.
void* scratch_on(void* stream) {
  const int dev = device_of(stream);
  if (dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) scratch_ptr[dev] = symbol_on(dev, HIP_SYMBOL(scratch));
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int fa_decode_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H_q,
                      int H_kv, int T, int N_k, int d, float scale, int causal, int num_splits,
                      const int32_t* block_table, int page_size, int pages_per_seq, void* workspace,
                      size_t workspace_bytes, int dtype, void* stream) {
  int ns = 0;
  size_t need = 0;
  const int st = check_decode(Q, K, V, O, LSE, B, H_q, H_kv, T, N_k, d, scale, causal, num_splits, block_table,
                              page_size, pages_per_seq, dtype, &ns, &need);
  if (st != FA_OK) return st;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return FA_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return FA_ERR_ALIGNMENT;
  return run_decode(Q, K, V, O, LSE, B, H_q, H_kv, T, N_k, d, scale, causal, ns, block_table, page_size,
                    pages_per_seq, workspace, dtype, stream);
}

int fa_decode_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H_q,
                              int H_kv, int T, int N_k, int d, float scale, int causal, int num_splits,
                              const int32_t* block_table, int page_size, int pages_per_seq, int dtype,
                              void* stream) {
  int ns = 0;
  size_t need = 0;
  const int st = check_decode(Q, K, V, O, LSE, B, H_q, H_kv, T, N_k, d, scale, causal, num_splits, block_table,
                              page_size, pages_per_seq, dtype, &ns, &need);
  if (st != FA_OK) return st;
  if (need > (size_t)FA_DECODE_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  if (T == 0) return FA_OK;
  void* ws = nullptr;
  if (need > 0 && (ws = scratch_on(stream)) == nullptr) return FA_ERR_HIP;
  return run_decode(Q, K, V, O, LSE, B, H_q, H_kv, T, N_k, d, scale, causal, ns, block_table, page_size,
                    pages_per_seq, ws, dtype, stream);
}

int fa_decode_merge_period(void* stream) { return placement_period(stream); }

int fa_decode_merge_in_kernel(int B, int H_q, int H_kv, int T, int N_k, int d, int num_splits, void* stream) {
  if (check_heads(B, H_q, H_kv, T, N_k, d) != FA_OK || num_splits < 0) return -1;
  const int ns = num_splits == 0 ? auto_splits(B, H_q, H_kv, T, N_k) : num_splits;
  if (ns <= 1 || T == 0) return 0;
  const int mode = merge_mode.load(std::memory_order_relaxed);
  if (placement_period(stream) <= 0) return 0;
  return mode == FA_MERGE_IN_KERNEL || in_kernel_pays(B, H_q, H_kv, T, ns) ? 1 : 0;
}

int fa_decode_set_merge(int mode) {
  if (mode != FA_MERGE_AUTO && mode != FA_MERGE_KERNEL && mode != FA_MERGE_IN_KERNEL) return FA_ERR_BAD_SHAPE;
  return merge_mode.exchange(mode);
}

int fa_lse_merge(const float* O_part, const float* LSE_part, void* O, float* LSE, int num_splits, int rows,
                 int d, int out_dtype, void* stream) {
  if (!present(O_part, rows > 0) || !present(LSE_part, rows > 0) || !present(O, rows > 0)) return FA_ERR_NULL_PTR;
  if (num_splits < 1 || rows < 0 || d < 1 || d > 512) return FA_ERR_BAD_SHAPE;
  if ((long long)num_splits * rows > 0x7fffffffLL) return FA_ERR_BAD_SHAPE;
  if (out_dtype != FA_BF16 && out_dtype != FA_FP32) return FA_ERR_UNSUPPORTED;
  if (!aligned4(O_part) || !aligned4(LSE_part) || !aligned4(O) || (LSE && !aligned4(LSE))) return FA_ERR_ALIGNMENT;
  if (rows == 0) return FA_OK;
  return status_of(fa::launch_lse_merge(O_part, LSE_part, O, LSE, num_splits, rows, d, out_dtype == FA_FP32, stream));
}

}  // extern "C"
