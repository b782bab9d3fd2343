// Host-side checks of the C ABI (include/fa.h, include/fa_calib.h), built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code of fa_api.hip and fa_calib.hip.  Every call
// here breaks at least one documented rule, so it is rejected before any HIP call: the
// driver runs on a host without a GPU.  The size helpers are called with extreme values so
// that every overflow guard of the validation runs under the sanitizers.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <climits>

#include "fa.h"
#include "fa_calib.h"

static int failures = 0;

static void expect(const char* what, long long got, long long want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %lld, want %lld\n", what, got, want);
    ++failures;
  }
}

int main() {
  void* P = reinterpret_cast<void*>(uintptr_t{0x10000});        // never dereferenced
  void* P8 = reinterpret_cast<void*>(uintptr_t{0x10008});       // not 16-byte aligned
  float* F = static_cast<float*>(P);
  const int32_t* BT = static_cast<const int32_t*>(P);

  // status strings and version
  for (int s = -3; s < 12; ++s) {
    const char* t = fa_status_string(s);
    expect("status string non-null", t != nullptr, 1);
    expect("status string non-empty", t != nullptr && strlen(t) > 0, 1);
  }
  expect("version", fa_version(), 102);

  // fa_fwd
  expect("fwd null Q", fa_fwd(nullptr, P, P, P, F, 1, 2, 1, 8, 8, 64, 0.125f, 0, FA_BF16, nullptr), FA_ERR_NULL_PTR);
  expect("fwd B=0", fa_fwd(P, P, P, P, F, 0, 2, 1, 8, 8, 64, 0.125f, 0, FA_BF16, nullptr), FA_ERR_BAD_SHAPE);
  expect("fwd H_q%H_kv", fa_fwd(P, P, P, P, F, 1, 3, 2, 8, 8, 64, 0.125f, 0, FA_BF16, nullptr), FA_ERR_BAD_SHAPE);
  expect("fwd huge rows", fa_fwd(P, P, P, P, F, INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, 64, 0.125f, 0, FA_BF16,
                                 nullptr), FA_ERR_BAD_SHAPE);
  expect("fwd scale nan", fa_fwd(P, P, P, P, F, 1, 2, 1, 8, 8, 64, __builtin_nanf(""), 0, FA_BF16, nullptr),
         FA_ERR_BAD_SHAPE);
  expect("fwd causal 2", fa_fwd(P, P, P, P, F, 1, 2, 1, 8, 8, 64, 0.125f, 2, FA_BF16, nullptr), FA_ERR_BAD_SHAPE);
  expect("fwd d=96", fa_fwd(P, P, P, P, F, 1, 2, 1, 8, 8, 96, 0.125f, 0, FA_BF16, nullptr), FA_ERR_UNSUPPORTED);
  expect("fwd dtype", fa_fwd(P, P, P, P, F, 1, 2, 1, 8, 8, 64, 0.125f, 0, 9, nullptr), FA_ERR_UNSUPPORTED);
  expect("fwd align", fa_fwd(P8, P, P, P, F, 1, 2, 1, 8, 8, 64, 0.125f, 0, FA_BF16, nullptr), FA_ERR_ALIGNMENT);

  // fa_fwd_paged
  expect("paged null table", fa_fwd_paged(P, P, P, P, F, 2, 4, 2, 16, 100, 128, 0.1f, 1, nullptr, 16, 7, FA_BF16,
                                          nullptr), FA_ERR_NULL_PTR);
  expect("paged short table", fa_fwd_paged(P, P, P, P, F, 2, 4, 2, 16, 100, 128, 0.1f, 1, BT, 16, 6, FA_BF16, nullptr),
         FA_ERR_BAD_SHAPE);
  expect("paged huge table", fa_fwd_paged(P, P, P, P, F, INT_MAX, 4, 2, 16, 100, 128, 0.1f, 1, BT, 16, INT_MAX,
                                          FA_BF16, nullptr), FA_ERR_BAD_SHAPE);
  expect("paged N_k 2^24", fa_fwd_paged(P, P, P, P, F, 1, 4, 2, 16, 1 << 24, 128, 0.1f, 1, BT, 16, 1 << 20, FA_BF16,
                                        nullptr), FA_ERR_BAD_SHAPE);
  expect("paged fp32", fa_fwd_paged(P, P, P, P, F, 2, 4, 2, 16, 100, 128, 0.1f, 1, BT, 16, 7, FA_FP32, nullptr),
         FA_ERR_UNSUPPORTED);

  // fa_bwd and its workspace size
  expect("bwd ws bytes 0", (long long)fa_bwd_workspace_bytes(0, 1, 1), 0);
  expect("bwd ws bytes huge", (long long)fa_bwd_workspace_bytes(INT_MAX, INT_MAX, INT_MAX), 0);
  expect("bwd ws bytes", (long long)fa_bwd_workspace_bytes(4, 16, 4096), 4LL * 16 * 128 * 256);
  expect("bwd null dO", fa_bwd(P, P, P, P, nullptr, F, P, P, P, 1, 2, 1, 8, 8, 64, 0.125f, 0, P, 1 << 20, FA_BF16,
                               nullptr), FA_ERR_NULL_PTR);
  expect("bwd no workspace", fa_bwd(P, P, P, P, P, F, P, P, P, 1, 2, 1, 8, 8, 64, 0.125f, 0, nullptr, 0, FA_BF16,
                                    nullptr), FA_ERR_WORKSPACE);
  expect("bwd fp32 in", fa_bwd(P, P, P, P, P, F, P, P, P, 1, 2, 1, 8, 8, 64, 0.125f, 0, P, 1 << 20, FA_FP32,
                               nullptr), FA_ERR_UNSUPPORTED);

  // decode: split count and workspace helpers at the edges
  expect("num splits bad", fa_decode_num_splits(0, 1, 1, 1, 1, 128), 0);
  expect("num splits huge", fa_decode_num_splits(INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, 128), 0);
  expect("num splits C4", fa_decode_num_splits(1, 32, 8, 1, 131072, 128) >= 1, 1);
  expect("dec ws huge splits", (long long)fa_decode_workspace_bytes(1, 32, 8, 1, 131072, 128, INT_MAX), 0);
  expect("dec ws one split", (long long)fa_decode_workspace_bytes(1, 32, 8, 1, 131072, 128, 1), 0);
  expect("dec huge splits", fa_decode_splitkv(P, P, P, P, F, 1, 4, 2, 1, 100, 128, 0.1f, 1, INT_MAX, nullptr, 0, 0,
                                              P, (size_t)-1, FA_BF16, nullptr), FA_ERR_BAD_SHAPE);
  expect("dec no workspace", fa_decode_splitkv(P, P, P, P, F, 1, 4, 2, 1, 100, 128, 0.1f, 1, 4, nullptr, 0, 0,
                                               nullptr, 0, FA_BF16, nullptr), FA_ERR_WORKSPACE);
  // one workgroup group: the grid, groups rounded up to 64 times the splits, passes 2^31
  expect("dec grid", fa_decode_splitkv(P, P, P, P, F, 1, 1, 1, 1, 100, 128, 0.1f, 1, 1 << 25, nullptr, 0, 0, P,
                                       (size_t)-1, FA_BF16, nullptr), FA_ERR_BAD_SHAPE);
  expect("dec table short", fa_decode_splitkv(P, P, P, P, F, 1, 4, 2, 1, 100, 128, 0.1f, 1, 4, BT, 16, 6, P,
                                              (size_t)-1, FA_BF16, nullptr), FA_ERR_BAD_SHAPE);
  expect("noalloc scratch", fa_decode_splitkv_noalloc(P, P, P, P, F, 1, 4, 2, 1, 100, 128, 0.1f, 1, 8193, nullptr, 0,
                                                      0, FA_BF16, nullptr), FA_ERR_WORKSPACE);
  expect("noalloc no rows", fa_decode_splitkv_noalloc(P, P, P, P, F, 1, 4, 2, 0, 100, 128, 0.1f, 1, 4, nullptr, 0, 0,
                                                      FA_BF16, nullptr), FA_OK);

  // merge
  expect("merge ns 0", fa_lse_merge(F, F, P, F, 0, 8, 128, FA_BF16, nullptr), FA_ERR_BAD_SHAPE);
  expect("merge huge", fa_lse_merge(F, F, P, F, INT_MAX, INT_MAX, 128, FA_BF16, nullptr), FA_ERR_BAD_SHAPE);
  expect("merge d 513", fa_lse_merge(F, F, P, F, 4, 8, 513, FA_BF16, nullptr), FA_ERR_BAD_SHAPE);
  expect("merge no rows", fa_lse_merge(F, F, P, F, 4, 0, 128, FA_BF16, nullptr), FA_OK);

  // calibration kernels
  expect("calib mfma", fa_calib_mfma(nullptr, static_cast<uint64_t*>(P), 1, 1, nullptr), 1);
  expect("calib stream", fa_calib_stream_read(P, 24, F, 1, nullptr), 2);
  expect("calib clock", fa_calib_clock(static_cast<uint64_t*>(P), 0, nullptr), 2);

  if (failures == 0) printf("abi driver ok\n");
  return failures == 0 ? 0 : 1;
}
