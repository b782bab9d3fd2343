// Host-side argument bundles and launcher entry points shared between the C-ABI layer
// (fa_api.hip) and the kernel files.  Validation happens in fa_api.hip before any of
// these is called; the launchers assume valid arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  int B, H_q, H_kv, N_q, N_k, d;
  float scale;
  int causal;
  void* stream;
};

struct DecodeArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  int B, H_q, H_kv, T, N_k, d;
  float scale;
  int causal;
  int num_splits;   // resolved, >= 1
  int split_len;    // keys per split (multiple of the decode chunk)
  const int32_t* block_table;  // NULL: contiguous K/V
  int page_size, pages_per_seq;
  float* O_part;    // [num_splits, B*H_q*T, d] (unused when num_splits == 1)
  float* LSE_part;  // [num_splits, B*H_q*T]
  uint32_t* flags;  // [groups, num_splits] completion flags for the in-kernel merge; NULL: merge kernel
  uint32_t token;   // this call's completion token (never 0)
  int n_map;        // placement period: workgroup indices equal modulo n_map share an XCD
  void* stream;
};

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* LSE;
  void* dQ;
  void* dK;
  void* dV;
  int B, H_q, H_kv, N_q, N_k, d;
  float scale;
  int causal;
  void* workspace;  // >= bwd_workspace_bytes(B, H_q, N_q)
  void* stream;
};

hipError_t launch_fwd_bf16(const FwdArgs& a, bool out_f32);
hipError_t launch_fwd_bf16_paged(const FwdArgs& a, bool out_f32, const int32_t* block_table, int page_size,
                                 int pages_per_seq);
hipError_t launch_fwd_fp32(const FwdArgs& a);
hipError_t launch_decode_split(const DecodeArgs& a, bool out_f32);
hipError_t launch_xcc_probe(uint32_t* out, int n_wg, void* stream);
hipError_t launch_lse_merge(const float* O_part, const float* LSE_part, void* O, float* LSE,
                            int num_splits, int rows, int d, bool out_f32, void* stream);

size_t bwd_workspace_bytes(int B, int H_q, int N_q);
hipError_t launch_bwd(const BwdArgs& a, bool out_f32);

constexpr int kDecodeChunk = 64;  // keys per wave iteration in the decode kernel
constexpr int kDecodeRows = 16;   // stacked query rows per decode workgroup

}  // namespace fa
