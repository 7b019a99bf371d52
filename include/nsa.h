/*
 * nsa.h -- C ABI of the MI355X (gfx950) native sparse attention forward.
 *
 * The operation (ejKernel "native_sparse_attention" API page: the module
 * description, and "Parameters" of `run` / `native_sparse_attention`): every
 * query token's group of query heads attends only to the key/value blocks
 * listed in its row of `block_indices`, truncated to `block_counts` entries,
 * each block being `block_size` consecutive keys.  Scores are scale * q.k,
 * normalised by a softmax over the visible keys, and the output is the
 * probability-weighted sum of the values.  Inside the query's own block only
 * keys at or before the query position are visible (causal, inclusive
 * diagonal: the causal block rule of the ejKernel block-sparse mask page).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the
 *    library allocates nothing, keeps no pointer after a call returns and
 *    holds no global state.  Work is enqueued asynchronously on `stream`
 *    (a hipStream_t; NULL means the default stream).
 *  - Tensors are contiguous row-major with the last dimension fastest:
 *      q   [B, T, Hq,  D]      (dtype)
 *      k,v [B, T, Hkv, D]      (dtype)
 *      block_indices [B, T, Hkv, S]  int32, block ids relative to the
 *                                     sequence start
 *      block_counts  [B, T, Hkv]     int32
 *      out [B, T, Hq,  D]      (dtype, rounded once from fp32)
 *      lse [B, T, Hq]          float32, natural log of the softmax
 *                              denominator: log sum_s exp(scale * q.k_s)
 *    q, k, v and out must be 16-byte aligned.
 *  - Query head hq uses kv head hq / (Hq / Hkv).
 *  - Only entries i < clamp(block_counts, 0, S) are read.  Entries that are
 *    negative, beyond the query's own block or beyond the sequence
 *    contribute nothing; a block listed twice counts once.  Index contents
 *    are never an error.  A row with no visible key gets out = 0 and
 *    lse = -inf.
 *  - Host-detectable argument errors return synchronously before anything is
 *    enqueued; a failed launch returns NSA_ERROR_LAUNCH_FAILED.
 *  - NSA_SUCCESS from an enqueuing call means the arguments were valid and
 *    the work was enqueued; it says nothing about how the device run ended.
 *    The forward kernels' waits are bounded: a wait that expires leaves the
 *    affected out / lse rows unwritten and is reported ONLY through
 *    nsa_fwd_device_status (below), which a caller must read before
 *    trusting the results of nsa_fwd, nsa_fwd_varlen, nsa_fwd_qblock or
 *    nsa_fwd_execute.
 *  - The workspace is caller-owned device memory of at least
 *    nsa_fwd_workspace_size() bytes, 256-byte aligned; its contents need no
 *    initialisation and are overwritten.  Two calls that share a workspace
 *    must be ordered on one stream.
 */
#ifndef NSA_H
#define NSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NSA_ABI_VERSION 3

typedef enum {
  NSA_SUCCESS = 0,
  NSA_ERROR_INVALID_VALUE = 1,      /* null pointer, bad size, misalignment, non-finite scale */
  NSA_ERROR_NOT_SUPPORTED = 2,      /* head_dim, block_size, group size or dtype not built */
  NSA_ERROR_WORKSPACE_TOO_SMALL = 3,
  NSA_ERROR_LAUNCH_FAILED = 4
} nsa_status;

typedef enum { NSA_DTYPE_F32 = 0, NSA_DTYPE_BF16 = 1 } nsa_dtype;

typedef struct {
  int32_t batch;        /* B; must be 1 for the varlen entry point            */
  int32_t seqlen;       /* T; total packed tokens for the varlen entry point  */
  int32_t num_q_heads;  /* Hq, a multiple of num_kv_heads                     */
  int32_t num_kv_heads; /* Hkv                                                */
  int32_t head_dim;     /* D: 64 or 128                                       */
  int32_t num_selected; /* S, last dimension of block_indices (1..1024)       */
  int32_t dtype;        /* nsa_dtype of q, k, v and out (other values: NOT_SUPPORTED) */
} nsa_dims;

/*
 * Bytes of workspace nsa_fwd / nsa_fwd_varlen need for these dims.
 * num_seqs = 0 for the fixed-length entry point, else the number of packed
 * sequences.  Returns 0 if the dims are invalid or not supported.
 */
size_t nsa_fwd_workspace_size(const nsa_dims* dims, int32_t block_size, int32_t num_seqs);

/*
 * Fixed-length forward: B independent sequences of length T.
 *  block_size: 32, 64 or 128.
 *  scale: softmax scale applied to q.k (finite).
 *  lse: may be NULL (then not written).
 */
nsa_status nsa_fwd(const nsa_dims* dims, const void* q, const void* k, const void* v,
                   const int32_t* block_indices, const int32_t* block_counts,
                   int32_t block_size, float scale, void* out, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * nsa_fwd for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same
 * computation, kernels and results as nsa_fwd, with the workspace taken
 * from a static device array of 32 MiB (NSA_NOALLOC_SCRATCH_BYTES) that every
 * GPU the library runs on holds until the process ends.  It calls no
 * allocating routine.  The current device's array is used, so `stream` must
 * belong to the current device.
 *  - Dims whose nsa_fwd_workspace_size exceeds the array return
 *    NSA_ERROR_WORKSPACE_TOO_SMALL before anything is enqueued (the five
 *    named workloads of the design notes need at most 24.4 MiB).
 *  - Every call on a GPU uses that GPU's one array: calls that overlap on one
 *    GPU (different streams, or host threads without ordering) race and give
 *    undefined results.  Order them on one stream.
 *  - device_status: NULL, or a DEVICE int32 that receives the run's status
 *    word (0 = every bounded wait completed; NSA_DEVICE_WAIT_EXPIRED
 *    otherwise) once the work on `stream` has completed.
 *  - Other arguments, layouts and errors as nsa_fwd.
 */
#define NSA_NOALLOC_SCRATCH_BYTES (32u << 20)
nsa_status nsa_fwd_noalloc(const nsa_dims* dims, const void* q, const void* k, const void* v,
                           const int32_t* block_indices, const int32_t* block_counts,
                           int32_t block_size, float scale, void* out, float* lse,
                           int32_t* device_status, void* stream);

/*
 * Variable-length forward (the `cu_seqlens` argument of the same page):
 * dims->batch == 1, dims->seqlen = total packed tokens, and the sequences
 * are packed back to back.  cu_seqlens [num_seqs + 1] int32 DEVICE array,
 * cu_seqlens[0] = 0, non-decreasing, cu_seqlens[num_seqs] = T (a contract
 * the device does not check).  Block j of a sequence starting at bos covers
 * tokens [bos + j*block_size, bos + (j+1)*block_size) clipped to the
 * sequence; keys never come from another sequence.
 */
nsa_status nsa_fwd_varlen(const nsa_dims* dims, const void* q, const void* k, const void* v,
                          const int32_t* block_indices, const int32_t* block_counts,
                          const int32_t* cu_seqlens, int32_t num_seqs,
                          int32_t block_size, float scale, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fixed-length forward with indices shared by the tokens of a query block
 * (the `block_indices` parameter description of the same page: indices of
 * key blocks per query block, [batch, num_kv_heads, num_query_blocks, ...],
 * and `block_counts`, the number of key blocks per query block).
 *  block_indices [B, Hkv, NQB, S] int32, NQB = ceil(T / block_size);
 *  block_counts  [B, Hkv, NQB]    int32.
 * Query token t uses row t / block_size (query blocks have the key blocks'
 * size).  Everything else -- entries read, skipped and merged, the causal
 * rule inside the token's own block, q/k/v/out/lse layouts, errors and the
 * workspace (nsa_fwd_workspace_size with num_seqs = 0) -- is as for
 * nsa_fwd, so the result equals nsa_fwd with every token's row copied from
 * its query block's row.  Packed (varlen) sequences are not supported by
 * this layout.
 */
nsa_status nsa_fwd_qblock(const nsa_dims* dims, const void* q, const void* k, const void* v,
                          const int32_t* block_indices, const int32_t* block_counts,
                          int32_t block_size, float scale, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode step: one query token per sequence against its KV cache, with the
 * block selection applied (the NSA page's operation restricted to the
 * newest token, with the ragged per-sequence key range of the
 * ragged-decode page's `ragged_decode_mqa_xla`: query [B, Hq, D], cache
 * [B, S, Hkv, D] and a key range per sequence).
 *  dims->batch   B sequences; dims->seqlen = Smax, cache rows per sequence;
 *  dims->dtype   NSA_DTYPE_BF16 only; dims->num_selected = S <= 64.
 *  q        [B, Hq, D]        bf16, the newest token of each sequence
 *  k, v     [B, Smax, Hkv, D] bf16 cache; row s of sequence b is key s
 *  seq_lens [B] int32 DEVICE array: len_b, clamped to [0, Smax]; keys
 *           0 .. len_b - 1 exist and the query sits at t = len_b - 1
 *  block_indices [B, Hkv, S] int32 and block_counts [B, Hkv] int32: the
 *           query's row, read with the rules of nsa_fwd (entries past the
 *           count, negative or past t's own block t / block_size contribute
 *           nothing, repeats count once, keys after t are masked)
 *  out      [B, Hq, D] bf16;  lse [B, Hq] float32 or NULL.
 * len_b = 0 (or no visible key) gives out = 0 and lse = -inf.  No
 * workspace.  Argument errors return synchronously as for nsa_fwd;
 * NSA_ERROR_NOT_SUPPORTED for fp32, S > 64 and the head_dim / block_size /
 * group limits of nsa_fwd.
 */
nsa_status nsa_decode(const nsa_dims* dims, const void* q, const void* k, const void* v,
                      const int32_t* seq_lens, const int32_t* block_indices,
                      const int32_t* block_counts, int32_t block_size, float scale, void* out,
                      float* lse, void* stream);

/*
 * Backward of nsa_fwd (fixed-length sequences, bf16): the gradients of the
 * forward's out with respect to q, k and v, given dout.  With P the
 * forward's probabilities over each token's visible keys (recomputed from
 * q, k and the forward's lse):
 *   Delta = dout . out,  dS = P (dout . v - Delta),
 *   dq = scale sum dS k,  dk = scale sum dS q,  dv = sum P dout
 * (the chain rule through the masked softmax of the NSA page's operation).
 *  q, k, v, out, dout bf16 in the layouts of nsa_fwd; lse [B, T, Hq]
 *  float32 from the same forward; dq [B, T, Hq, D], dk, dv [B, T, Hkv, D]
 *  float32, fully written (rows of keys no token reads get zeros).
 *  The index rows and their rules are those of nsa_fwd; S <= 64.
 *  Workspace: nsa_bwd_workspace_size() bytes (Delta [B, T, Hq] float32, a
 *  reader bitmap per key block: B * Hkv * ceil(T / block_size) *
 *  ceil(T / 32) words, and each token segment's partial dK and dV sums:
 *  2 * ceil(T / L) * B * T * Hkv * D float32 with segments of L = 512
 *  tokens up to T = 4096, 1024 up to 8192, 2048 up to 16384, else 4096,
 *  times 16 / G where G = Hq / Hkv <= 16, at most 4096 and at most T (none
 *  when one segment covers T: dk and dv are then written directly),
 *  then the forward's schedule of the same indices: dq runs as the
 *  gradient mode of the forward's gather over it),
 *  256-byte aligned, no initialisation needed.  Past T = 16384 the
 *  segment length stays 4096, so the partial sums grow as T^2: about
 *  1.07 GB at B = 1, T = 32768, Hkv = 4, D = 128, 4.3 GB at T = 65536.
 *  Dims whose kernels would exceed a grid of 2^32 work-items return
 *  NSA_ERROR_NOT_SUPPORTED.
 * dk and dv sum over a block's readers in token order, so results are
 * deterministic.  NSA_ERROR_NOT_SUPPORTED for fp32, S > 64 and wherever
 * nsa_fwd does not take the same fixed-length dims and block_size.  The
 * waits of the dq gather are bounded like the forward's: see
 * nsa_bwd_device_status.
 */
size_t nsa_bwd_workspace_size(const nsa_dims* dims, int32_t block_size);
nsa_status nsa_bwd(const nsa_dims* dims, const void* q, const void* k, const void* v,
                   const void* out, const float* lse, const void* dout,
                   const int32_t* block_indices, const int32_t* block_counts,
                   int32_t block_size, float scale, float* dq, float* dk, float* dv,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two halves of a forward call.  nsa_fwd(...) is exactly
 * nsa_fwd_schedule(...) followed by nsa_fwd_execute(...) on the same stream.
 *
 * nsa_fwd_schedule reads block_indices / block_counts (and cu_seqlens when
 * not NULL: varlen, num_seqs sequences; NULL: fixed length, num_seqs
 * ignored) and writes into the workspace each work item's merged block
 * list and the longest-first order of the items.  A sparsity pattern known
 * ahead of time may be indexed once and used many times (module description
 * of the page), so a schedule stays valid for any number of nsa_fwd_execute
 * calls with the same dims, block_size and num_seqs while the indices are
 * unchanged.
 * If list_offset / list_len are not NULL they receive the byte offset in
 * the workspace of the int32 work list (processing order, a permutation of
 * 0 .. *list_len - 1) and its length, for inspection.
 *
 * nsa_fwd_execute runs the attention kernel from a schedule previously
 * written into `workspace` (num_seqs = 0 for fixed length).  It does not
 * read the indices.  With a workspace that does not hold a schedule for the
 * same dims, block_size and num_seqs the results are undefined, but the
 * kernel still reads and writes only inside q, k, v, out, lse and the
 * workspace (every scheduled value is range-checked before use).
 */
nsa_status nsa_fwd_schedule(const nsa_dims* dims, const int32_t* block_indices,
                            const int32_t* block_counts, const int32_t* cu_seqlens,
                            int32_t num_seqs, int32_t block_size, void* workspace,
                            size_t workspace_bytes, void* stream, size_t* list_offset,
                            int32_t* list_len);

/*
 * Scheduler half of nsa_fwd_qblock: the indices in the query-block layout
 * described there, otherwise as nsa_fwd_schedule for fixed length.  The
 * schedule it writes is run by nsa_fwd_execute with num_seqs = 0.
 */
nsa_status nsa_fwd_schedule_qblock(const nsa_dims* dims, const int32_t* block_indices,
                                   const int32_t* block_counts, int32_t block_size,
                                   void* workspace, size_t workspace_bytes, void* stream,
                                   size_t* list_offset, int32_t* list_len);

nsa_status nsa_fwd_execute(const nsa_dims* dims, const void* q, const void* k, const void* v,
                           int32_t num_seqs, int32_t block_size, float scale, void* out,
                           float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Device status of the forward calls that used `workspace` since the last
 * nsa_fwd_schedule (or nsa_fwd / nsa_fwd_varlen, which schedule first) on it.
 * Every wait inside the kernels is bounded; if one expired, bit 0
 * (NSA_DEVICE_WAIT_EXPIRED) is set and the results of those calls are
 * incomplete.  0 means every run completed normally.  The dims, block_size
 * and num_seqs (0 = fixed length) must be those of the calls.  This waits
 * for `stream` to finish and copies one word to the host.
 */
#define NSA_DEVICE_WAIT_EXPIRED 1
nsa_status nsa_fwd_device_status(const nsa_dims* dims, int32_t block_size, int32_t num_seqs,
                                 const void* workspace, size_t workspace_bytes, void* stream,
                                 int32_t* status);

/*
 * Device status of the last nsa_bwd call that used `workspace`: bit 0
 * (NSA_DEVICE_WAIT_EXPIRED) set if a bounded wait of its dq gather expired
 * (its dq, and the dk / dv that follow from its reader bitmaps, are then
 * incomplete); 0 if the call completed normally.  dims and block_size must
 * be those of the call.  Waits for `stream` to finish and copies one word
 * to the host.
 */
nsa_status nsa_bwd_device_status(const nsa_dims* dims, int32_t block_size, const void* workspace,
                                 size_t workspace_bytes, void* stream, int32_t* status);

/* Human-readable name of a status code (static storage). */
const char* nsa_status_string(nsa_status status);

/* NSA_ABI_VERSION of the built library. */
int32_t nsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NSA_H */
