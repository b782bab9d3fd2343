/*
 * fa.h -- FlashAttention forward and backward passes and split-KV decode for AMD Instinct
 * MI355X (gfx950).
 *
 * C linkage; no C++ or framework types cross this boundary.  Every tensor argument is a
 * DEVICE pointer owned by the caller.  The library never allocates, frees or synchronises:
 * each call validates its arguments, enqueues its kernels on `stream` and returns.  Outputs
 * are valid once the stream reaches the enqueued work; inputs must stay alive until then.
 * There is no global mutable state apart from the scratch of fa_decode_splitkv_noalloc, the
 * per-GPU placement probe result and the merge switch of the decode (below), each guarded,
 * so calls from several host threads are safe.
 *
 * Layouts (all contiguous, head dimension fastest, as the Flash Attention 1 kernel of the
 * page "Kernel visualization: Flash Attention 1" ("Initial setup") offsets its pointers by
 * batch*head*N*D):
 *   Q, O            [B, H_q,  N_q, d]          (decode: N_q = T new queries)
 *   K, V            [B, H_kv, N_k, d]          (contiguous cache)
 *   K, V pools      [num_pages, page_size, H_kv, d]   (paged cache: fa_fwd_paged, decode)
 *   LSE             [B, H_q, N_q] fp32
 *   dQ / dK, dV     as Q / as K, V   (fa_bwd)
 *   block_table     [B, pages_per_seq] int32
 *
 * Semantics (each output row is exact attention up to rounding):
 *   x_j   = scale * <Q[b,h,i,:], K[b,h_kv,j,:]>,  h_kv = h / (H_q / H_kv)
 *           (GQA: contiguous groups of H_q/H_kv query heads share one KV head; page
 *            "Attention kernel chains", chain "GQA loads KV once per group")
 *   visible keys: all j < N_k, or with causal != 0 only j <= i + (N_k - N_q): the mask is
 *           aligned to the bottom-right corner, query row i sits at position N_k - N_q + i
 *           (chain "The causal mask for a decode step")
 *   O[b,h,i,:] = sum_j p_j V[b,h_kv,j,:],  p = softmax of the visible x
 *           (page "Kernel visualization: Flash Attention 1", "Derivation")
 *   LSE[b,h,i] = ln sum_j e^{x_j}  over visible j  (natural log of the scaled scores; chain
 *           "What the backward pass saves": the forward keeps this one fp32 value per row)
 *   A row with no visible key (causal with N_q > N_k, or N_k = 0) gets O = 0 and LSE = -inf.
 *
 * Sizes: B, H_q, H_kv and d are >= 1; the sequence lengths (N_q, N_k, T, rows) may be 0.
 * A forward, decode or merge call with no query row validates its arguments and returns
 * FA_OK without enqueuing anything.  A pointer to a tensor of zero elements may be NULL;
 * any other may not.
 *
 * Errors: arguments are validated before anything is enqueued; on any failure nothing is
 * enqueued and a non-zero fa_status is returned.  A failed launch returns FA_ERR_HIP.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL_PTR = 1,     /* a required pointer is NULL */
  FA_ERR_BAD_SHAPE = 2,    /* B, H or d <= 0, a length < 0, H_q % H_kv != 0, scale not > 0, bad split/page args */
  FA_ERR_UNSUPPORTED = 3,  /* head dimension or dtype the library has no kernel for */
  FA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than fa_decode_workspace_bytes() */
  FA_ERR_ALIGNMENT = 5,    /* a tensor pointer is not 16-byte aligned */
  FA_ERR_HIP = 6           /* the HIP runtime reported an error at launch */
} fa_status;

typedef enum fa_dtype {
  FA_BF16 = 0,             /* bf16 Q/K/V and O; fp32 accumulation and LSE */
  FA_FP32 = 1,             /* fp32 Q/K/V and O (fa_fwd only) */
  FA_BF16_IN_FP32_OUT = 2  /* bf16 Q/K/V, O stored as fp32 before any rounding to bf16 */
} fa_dtype;

/*
 * fa_fwd -- the FlashAttention forward pass in FlashAttention-2 loop order.
 *
 * Defined by: page "Softmax and FlashAttention" ("Concept": a block of Br queries, K and V
 * streamed past in blocks of Bc, each Br x Bc score tile computed on chip and folded into
 * a running output) with the online-softmax carries of page "Kernel visualization: Flash
 * Attention 1" ("Derivation", "The tiled version": running max, running sum, unnormalized
 * accumulator) and the single division at the end (page "Attention kernel chains", chain
 * "The online softmax on numbers").
 *
 *   Q [B,H_q,N_q,d], K/V [B,H_kv,N_k,d] in `dtype`'s input type; O [B,H_q,N_q,d] in its
 *   output type; LSE [B,H_q,N_q] fp32 (may be NULL if not wanted).
 *   d in {64, 128}.  scale > 0 (typically 1/sqrt(d)).  causal: 0 or 1 (bottom-right).
 *   N_q, N_k >= 0, any value (ragged tails are masked).  stream: a hipStream_t or NULL.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
           int B, int H_q, int H_kv, int N_q, int N_k, int d,
           float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_paged -- fa_fwd over a paged KV cache: chunked prefill, where the N_q new tokens
 * of each sequence attend to the N_k cached ones (the last N_q of which are usually those
 * same new tokens), read through a block table.
 *
 * Defined by: the same passages as fa_fwd for the arithmetic and loop order; page
 * "Attention kernel chains", chain "The block-table cost of paged attention" (one int32
 * page index per page_size-token block) for the key addressing, and chain "The causal mask
 * for a decode step" for the mask: with N_q < N_k the queries are the LAST N_q positions,
 * so query i sees keys j <= i + N_k - N_q.
 *
 *   Q [B,H_q,N_q,d] bf16; O [B,H_q,N_q,d] bf16 (FA_BF16) or fp32 (FA_BF16_IN_FP32_OUT);
 *   LSE [B,H_q,N_q] fp32 (may be NULL).
 *   K/V pools [num_pages,page_size,H_kv,d] bf16 (the layout fa_decode_splitkv reads): key j
 *     of sequence b is slot j%page_size of page block_table[b*pages_per_seq + j/page_size].
 *   page_size >= 1, pages_per_seq >= 0, pages_per_seq*page_size >= N_k, N_k < 2^24 (the table
 *     may be NULL when N_k = 0).  Table contents are not
 *     checked: an entry outside the pool is undefined behaviour, as in any gather.
 *   d in {64, 128}.  scale > 0.  causal: 0 or 1 (bottom-right).  stream: hipStream_t or NULL.
 */
int fa_fwd_paged(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int B, int H_q, int H_kv, int N_q, int N_k, int d, float scale, int causal,
                 const int32_t* block_table, int page_size, int pages_per_seq,
                 int dtype, void* stream);

/*
 * fa_bwd_workspace_bytes -- bytes of device workspace fa_bwd needs: one 64-float record
 * per 32 query rows of each (batch, query head) (the base-2 LSE and D of those rows), the
 * rows padded to a multiple of 64, rounded up to 256 bytes.  Returns 0 on invalid sizes.
 */
size_t fa_bwd_workspace_bytes(int B, int H_q, int N_q);

/*
 * fa_bwd -- gradients of the forward pass: dQ, dK, dV for the upstream gradient dO.
 *
 * Defined by: page "Attention kernel chains", chain "What the backward pass saves": the
 * forward keeps its inputs, its output O and the fp32 LSE of every row (fa_fwd's LSE output), each
 * probability tile is rebuilt on chip as P = exp(S - LSE), and one extra row vector
 * D = rowsum(dO * O) is computed before the main loops.  The rest is the chain rule of
 * the forward definition: dP = dO V^T, dS = P * (dP - D), dV = P^T dO, dK = scale dS^T Q,
 * dQ = scale dS K.  GQA: dK and dV of a KV head are summed over its H_q/H_kv query heads.
 * The same bottom-right causal rule as fa_fwd.
 *
 *   Q, dO, O [B,H_q,N_q,d] bf16; K, V [B,H_kv,N_k,d] bf16; LSE [B,H_q,N_q] fp32 (from fa_fwd
 *   on the same inputs, natural log; -inf for a row that sees no key).
 *   dQ [B,H_q,N_q,d], dK and dV [B,H_kv,N_k,d]: bf16 (FA_BF16) or fp32 (FA_BF16_IN_FP32_OUT);
 *   every element is written (keys no query sees get 0: with N_q = 0, dK = dV = 0; with
 *   N_k = 0, dQ = 0).
 *   workspace: >= fa_bwd_workspace_bytes(B, H_q, N_q) bytes of device memory, 16-byte aligned
 *   (may be NULL when that is 0).
 *   d in {64, 128}.  scale > 0.  causal: 0 or 1.  stream: hipStream_t or NULL.
 *   The result does not depend on scheduling (no atomics): repeated calls agree bit for bit.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* LSE, void* dQ, void* dK, void* dV,
           int B, int H_q, int H_kv, int N_q, int N_k, int d, float scale, int causal,
           void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * fa_decode_num_splits -- the split count fa_decode_splitkv uses when called with
 * num_splits == 0.  Splitting pays when batch x KV heads is far below the number of
 * compute units; the aim is about one full wave of workgroups and no mostly idle second
 * wave (page "Attention kernel chains", chain "How many splits for decode"), here for the
 * MI355X's 256 compute units: one workgroup per CU.  Never more splits than 256-key pieces
 * of the cache.  Returns >= 1, or 0 on invalid sizes.
 */
int fa_decode_num_splits(int B, int H_q, int H_kv, int T, int N_k, int d);

/*
 * fa_decode_workspace_bytes -- bytes of device workspace fa_decode_splitkv needs for
 * `num_splits` splits (0 = the automatic count): the normalized partial outputs
 * O_part [ns, B*H_q*T, d] fp32, then LSE_part [ns, B*H_q*T] fp32, then the completion flags
 * of the in-kernel merge, uint32 [G, ns] with G = B*H_kv*ceil(H_q/H_kv*T/16) workgroup
 * groups, each part 256-byte aligned.  Returns 0 when num_splits resolves to 1 (no
 * workspace needed) or on bad sizes.
 */
size_t fa_decode_workspace_bytes(int B, int H_q, int H_kv, int T, int N_k, int d, int num_splits);

/*
 * fa_decode_splitkv -- split-KV ("flash decoding") attention of T new queries over a cache
 * of N_k keys, with the partial results combined by the LSE merge: inside the decode kernel
 * (one launch; the split of each group that completes last merges) when the GPU's
 * workgroup placement is known (fa_decode_merge_period), every workgroup of the call is
 * resident at once (at most 512) and the merging workgroup covers the splits in one round
 * (at most 8, 16 or 32 splits for groups of more than 8, 5-8 or at most 4 stacked rows),
 * else by the merge kernel (fa_decode_set_merge changes this).
 *
 * Defined by: page "Attention kernel chains", chains "How many splits for decode" (the key
 * axis is cut into num_splits contiguous chunks, one worker each), "The log-sum-exp merge"
 * (every split stores its own output, already divided by its own sum, plus the log of that
 * sum; the merge recovers the exact result for any split), "GQA
 * loads KV once per group" (the H_q/H_kv query heads of a group are stacked as the rows of
 * one tile so each KV tile is read once per group) and "The block-table cost of paged
 * attention" (one int32 page index per page_size-token block).
 *
 *   Q [B,H_q,T,d] bf16; O [B,H_q,T,d] bf16 (FA_BF16) or fp32 (FA_BF16_IN_FP32_OUT);
 *   LSE [B,H_q,T] fp32 (may be NULL).
 *   block_table == NULL: K/V contiguous [B,H_kv,N_k,d] bf16.
 *   block_table != NULL: K/V pools [num_pages,page_size,H_kv,d] bf16; token j of sequence b
 *     is in page block_table[b*pages_per_seq + j/page_size], slot j%page_size; requires
 *     page_size >= 1, pages_per_seq >= 0 and pages_per_seq*page_size >= N_k.  Table contents are not checked:
 *     an entry outside the pool is undefined behaviour, as in any gather.
 *   causal: 0 (every cached key visible) or 1 (bottom-right: query t sees j <= N_k - T + t).
 *   num_splits: >= 1, or 0 for fa_decode_num_splits().  Splits are contiguous key ranges of
 *     equal length rounded up to 64 keys; trailing splits may be empty.  num_splits * B*H_q*T
 *     and the workgroup count, num_splits * G rounded up to a multiple of 64 groups (G as in
 *     fa_decode_workspace_bytes), must stay below 2^31 (FA_ERR_BAD_SHAPE otherwise;
 *     fa_decode_workspace_bytes returns 0).
 *   workspace: >= fa_decode_workspace_bytes(...) bytes of device memory (may be NULL when
 *     that is 0), any content: the completion flags carry a token unique to each call and
 *     the kernel leaves them at 0, so nothing needs clearing, before the first call, between
 *     calls or between replays of a captured call.  Afterwards O_part and LSE_part hold the
 *     call's partials (fa_lse_merge's layout).  Calls that may overlap in time must not
 *     share a workspace.  d == 128 or 64.
 *   The first call with more than one split on a GPU probes its placement (below), which
 *   synchronises `stream` once; a first call made while `stream` is being captured into a
 *   graph skips the probe and uses the merge kernel.
 */
int fa_decode_splitkv(const void* Q, const void* K, const void* V, void* O, float* LSE,
                      int B, int H_q, int H_kv, int T, int N_k, int d,
                      float scale, int causal, int num_splits,
                      const int32_t* block_table, int page_size, int pages_per_seq,
                      void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * fa_decode_merge_period -- how fa_decode_splitkv merges on the GPU of `stream` (the current
 * GPU for NULL): the placement period p > 0 when the merge runs inside the decode kernel,
 * 0 when calls there launch the merge kernel.  The in-kernel merge relies on the GPU
 * dealing workgroups to its XCDs round-robin, so that workgroup indices equal modulo p run
 * on one XCD and share its L2 (the decode kernel puts all splits of a group on such
 * indices).  The first query on a GPU (or its first split decode call) probes that: a
 * kernel of 1024 workgroups records the XCC_ID register of each, and p is the smallest
 * power of two <= 64 with index L always on the XCD of index L % p and indices 0 .. p-1
 * on p different XCDs; none found: 0 for the process's lifetime.  The probe synchronises
 * `stream` once; while `stream` is being captured it is skipped (0 for now).  Returns 0
 * under fa_decode_set_merge(FA_MERGE_KERNEL) or on a HIP error.
 */
int fa_decode_merge_period(void* stream);

/*
 * fa_decode_merge_in_kernel -- whether a fa_decode_splitkv call with these sizes and
 * num_splits (0 = automatic) on `stream`'s GPU merges inside the decode kernel (1) or
 * launches the merge kernel or needs no merge (0); -1 on invalid sizes.  Probes the GPU's
 * placement on first use, as fa_decode_merge_period.
 */
int fa_decode_merge_in_kernel(int B, int H_q, int H_kv, int T, int N_k, int d, int num_splits, void* stream);

/*
 * fa_decode_set_merge -- process-wide choice of the decode merge: FA_MERGE_AUTO (the
 * default: in the decode kernel where fa_decode_merge_period allows it and the call meets
 * the conditions under fa_decode_splitkv, the separate merge kernel otherwise),
 * FA_MERGE_KERNEL (always the merge
 * kernel) or FA_MERGE_IN_KERNEL (in the decode kernel wherever the placement allows, any
 * split count).  All give the same result up to rounding order.  Affects calls that start
 * after it returns.  Returns the previous choice, or FA_ERR_BAD_SHAPE for another value
 * (the choice is then unchanged).
 */
#define FA_MERGE_AUTO 0
#define FA_MERGE_KERNEL 1
#define FA_MERGE_IN_KERNEL 2
int fa_decode_set_merge(int mode);

/*
 * fa_decode_splitkv_noalloc -- fa_decode_splitkv for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, kernels and results, with the partial results kept in
 * a scratch array of FA_DECODE_NOALLOC_SCRATCH_BYTES (16 MiB) that the library holds on
 * each GPU it runs on until the process ends, instead of a caller's workspace.
 *
 *   Arguments as fa_decode_splitkv without the workspace.  A call whose partials need more
 *   than FA_DECODE_NOALLOC_SCRATCH_BYTES (fa_decode_workspace_bytes(...) of its sizes and
 *   split count) returns FA_ERR_WORKSPACE and enqueues nothing; FA_ERR_HIP if the scratch
 *   address cannot be looked up.  Nothing here calls hipMalloc or hipFree; the first call
 *   on a GPU looks up that GPU's copy of the array (hipGetSymbolAddress) once.
 *   Every split writes all of its partial rows before the merge reads them and the merge
 *   leaves the completion flags at 0, so the scratch keeps no state from one call to the
 *   next that matters (replays of a captured call included).  All calls on one GPU share
 *   its scratch: calls that may overlap in time on one GPU (different streams, or several
 *   host threads without ordering) race and must not be made.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (16u << 20)
int fa_decode_splitkv_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                              int B, int H_q, int H_kv, int T, int N_k, int d,
                              float scale, int causal, int num_splits,
                              const int32_t* block_table, int page_size, int pages_per_seq,
                              int dtype, void* stream);

/*
 * fa_lse_merge -- combine normalized partial results over disjoint key sets.
 *
 * Defined by: page "Attention kernel chains", chain "The log-sum-exp merge":
 *   lse = ln sum_s e^{lse_s},   O = sum_s e^{lse_s - lse} O_s,
 * computed against m* = max_s lse_s.  Partials with lse_s = -inf (a worker that saw no
 * key) get weight 0; a row whose partials are all -inf gets O = 0 and lse = -inf.
 *
 *   O_part [num_splits, rows, d] fp32, LSE_part [num_splits, rows] fp32 (the workspace
 *   layout of fa_decode_splitkv); O [rows, d] in out_dtype (FA_BF16 or FA_FP32);
 *   LSE [rows] fp32 (may be NULL).  num_splits >= 1, rows >= 0, 1 <= d <= 512.
 */
int fa_lse_merge(const float* O_part, const float* LSE_part, void* O, float* LSE,
                 int num_splits, int rows, int d, int out_dtype, void* stream);

/* Human-readable name of an fa_status value (static storage; never NULL). */
const char* fa_status_string(int status);

/* Library ABI version (major*100 + minor). */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
