/*
 * swa.h -- C ABI of libswa.so: sliding-window grouped-query attention over a
 * rolling-buffer KV cache, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (Mistral 7B (Chinese translation), section 2
 * "Architectural details"):
 *   - paragraph "Sliding Window Attention" and the Figure 1 caption: the token
 *     at position i attends to the W positions i-W+1 .. i (no more than W,
 *     ending at itself; positions below 0 do not exist);
 *   - section 1 "Introduction": grouped-query attention; here query head h
 *     reads key/value head h / G with G = n_q_heads / n_kv_heads;
 *   - paragraph "Rolling Buffer Cache" and the Figure 2 caption: keys and
 *     values of position i live in cache slot i mod W; later positions
 *     overwrite earlier ones;
 *   - paragraph "Pre-fill and Chunking" and the Figure 3 caption: a prompt is
 *     processed chunk by chunk; a chunk attends causally to itself and,
 *     through the window, to the cache; afterwards tokens are generated one at
 *     a time.
 *
 * Conventions shared by every entry point
 *   - Pointers named in the structs and arguments are DEVICE pointers owned by
 *     the caller, except the fields prefixed h_ (host pointers).  The library
 *     allocates nothing, keeps no pointer after returning and has no global
 *     mutable state; calls are re-entrant.  (The one exception is
 *     swa_decode_step_noalloc, whose merge partials live in a device array of
 *     the library's own; see there.)
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *     null stream) and never synchronizes.  Buffers must stay alive until the
 *     enqueued work has finished.
 *   - Layouts are dense and row-major:
 *       cache k / v        [n_cache][n_kv_heads][window][head_dim]
 *       q, out             [total_tokens][n_q_heads][head_dim]
 *       k_new, v_new       [total_tokens][n_kv_heads][head_dim]
 *     Tokens of a batch are packed sequence after sequence: the tokens of
 *     sequence b are rows cu_seqlens[b] .. cu_seqlens[b+1]-1 and token t of
 *     sequence b has absolute position start_pos[b] + (t - cu_seqlens[b]).
 *     All tensors of one call share the cache dtype.  Base pointers must be
 *     16-byte aligned.
 *   - Errors are returned, never raised.  Arguments are validated before
 *     anything is enqueued: on any status other than SWA_OK nothing has been
 *     launched and no buffer has been touched, except SWA_ERR_HIP, which
 *     reports a failed launch.  Device-resident metadata (cu_seqlens,
 *     start_pos, cache_idx) is trusted unless the host mirrors are given, in
 *     which case the mirrors are checked.  Faults in device work surface at the
 *     caller's next synchronization.
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWA_ABI_VERSION 3  /* 2: swa_decode_step added; 3: swa_decode_step_noalloc */

typedef enum swa_dtype {
  SWA_DTYPE_BF16 = 0, /* bfloat16 storage, fp32 arithmetic, bf16 output (round to nearest even) */
  SWA_DTYPE_F32 = 1   /* fp32 storage and arithmetic */
} swa_dtype;

typedef enum swa_status {
  SWA_OK = 0,
  SWA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misalignment, inconsistent metadata */
  SWA_ERR_UNSUPPORTED = 2,      /* valid request outside the compiled shapes (dtype / head_dim / group) */
  SWA_ERR_WORKSPACE = 3,        /* decode workspace missing or smaller than swa_decode_workspace_size() */
  SWA_ERR_HIP = 4,              /* a HIP launch reported an error */
  SWA_ERR_INTERNAL = 5
} swa_status;

/*
 * The rolling buffer of one attention layer (paragraph "Rolling Buffer Cache").
 * Row r of the cache is one sequence's ring: for each KV head g it holds
 * `window` slots of head_dim elements.  After positions 0..e of a sequence
 * have been written, slot t holds position e - ((e - t) mod window) when that
 * is >= 0; other slots hold whatever the caller put there.
 * Supported: head_dim in {16, 64, 128} for both dtypes; 1 <= window <= 2^30;
 * n_kv_heads >= 1.
 */
typedef struct swa_cache {
  void *k;             /* device, [n_cache][n_kv_heads][window][head_dim] */
  void *v;             /* device, same layout as k */
  int32_t n_cache;     /* number of rings (cache rows) */
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t window;      /* W: slots per ring = keys per query */
  int32_t dtype;       /* swa_dtype */
  int32_t reserved;    /* must be 0 */
} swa_cache;

/*
 * The sequences of one call.  total_tokens and max_new_tokens size the launch
 * grid; they must match the device metadata.  cache_idx may be NULL (sequence b
 * uses cache row b).  The h_ mirrors are optional host copies of the device
 * arrays; when given they are validated (monotone cu_seqlens ending at
 * total_tokens, no sequence longer than max_new_tokens, start_pos >= 0,
 * start_pos + length <= 2^31 - 1, cache rows in range) and an error is returned
 * before any launch.
 */
typedef struct swa_batch {
  int32_t num_seqs;
  int32_t total_tokens;
  int32_t max_new_tokens;
  int32_t reserved;              /* must be 0 */
  const int32_t *cu_seqlens;     /* device [num_seqs + 1], cu_seqlens[0] = 0 */
  const int32_t *start_pos;      /* device [num_seqs] absolute position of each sequence's first new token */
  const int32_t *cache_idx;      /* device [num_seqs] cache row of each sequence, or NULL */
  const int32_t *h_cu_seqlens;   /* optional host mirror of cu_seqlens */
  const int32_t *h_start_pos;    /* optional host mirror of start_pos */
  const int32_t *h_cache_idx;    /* optional host mirror of cache_idx */
} swa_batch;

/* SWA_ABI_VERSION of the library that is loaded. */
int swa_abi_version(void);

/* Static, never-NULL description of a status code. */
const char *swa_status_string(int status);

/*
 * Cache write (paragraph "Rolling Buffer Cache", Figure 2 caption).
 * For every new token of every sequence, at absolute position p:
 *     cache.k[row][g][p mod W][:] = k_new[token][g][:]   (and the same for v)
 * with row = cache_idx[b] (or b).  When a sequence brings more than W tokens,
 * several of them map to one slot; the highest position wins, exactly as if
 * the writes were applied in position order (only the last W tokens are
 * copied).  The copy is bitwise.  Slots not written keep their contents.
 * k_new, v_new: device [total_tokens][n_kv_heads][head_dim].
 * Sequences must use distinct cache rows within one call.
 */
int swa_cache_write(const swa_cache *cache, const swa_batch *batch,
                    const void *k_new, const void *v_new, void *stream);

/*
 * Chunked prefill (paragraph "Pre-fill and Chunking", Figure 3 caption).
 * For each new token at absolute position i of sequence b and each query head h:
 *     out[token][h] = softmax_j( sm_scale * q[token][h] . k_j ) v_j,  j in [max(0, i-W+1), i]
 * where k_j / v_j (KV head h / G) come from
 *     - the cache ring of the sequence, slot j mod W, when j < start_pos[b]
 *       (that slot must hold position j: the earlier chunks have been written);
 *     - k_new / v_new of this call, when j >= start_pos[b].
 * The cache is only read.  To continue the sequence, enqueue swa_cache_write
 * for the same tokens afterwards on the same stream (writing first would
 * overwrite positions the chunk still reads when the chunk is as long as W).
 * Any chunk length >= 0 is accepted; the window rule is applied on absolute
 * positions, so a chunk longer than W also sees the window inside itself.
 * q, out: device [total_tokens][n_q_heads][head_dim]; n_q_heads must be a
 * multiple of n_kv_heads with G = n_q_heads / n_kv_heads in {1, 2, 4, 8}.
 * cache.k / cache.v may be NULL only if the host mirror h_start_pos is given
 * and every start_pos is 0.
 */
int swa_prefill_chunk(const swa_cache *cache, const swa_batch *batch,
                      const void *q, int32_t n_q_heads,
                      const void *k_new, const void *v_new,
                      float sm_scale, void *out, void *stream);

/*
 * Measurement aid for the tile skip of swa_prefill_chunk (paragraph "Sliding
 * Window Attention": the window cuts the work per token to W keys, which the
 * paper credits for its speed-up over standard attention at 16K tokens).
 * Same arguments and the same result, bit for bit, as swa_prefill_chunk, but
 * every key tile from position 0 up to the query tile is visited -- the whole
 * causal triangle, as attention without the band skip computes it -- and the
 * keys outside each query's window are masked.  Keys below the band are read
 * where the call holds them (positions >= max(0, start_pos - W + 1)).
 * SWA_DTYPE_BF16 only (SWA_ERR_UNSUPPORTED for SWA_DTYPE_F32).
 */
int swa_prefill_chunk_no_tile_skip(const swa_cache *cache, const swa_batch *batch,
                                   const void *q, int32_t n_q_heads,
                                   const void *k_new, const void *v_new,
                                   float sm_scale, void *out, void *stream);

/*
 * Bytes of device workspace swa_decode and swa_decode_step need for this cache
 * shape, batch size and head count (0 when the plan needs none).  Returns 0 for
 * invalid input.  When one workgroup per (sequence, KV head) would leave the
 * GPU short of work, the plan spreads the attention over more workgroups; the
 * workspace holds their partial results (head_dim + 2 floats per query head)
 * and a merge launch combines them.  Two plans:
 *   - split: each window in S parts, one partial per (sequence, query head,
 *     part): num_seqs * n_q_heads * S * (head_dim + 2) * 4 bytes,
 *     2 <= S <= window / 256;
 *   - stream (bf16 on the matrix-core kernel -- G >= 2 at head_dim 128, any
 *     G at head_dim 64 -- with 2 to 64 sequences): the valid slots of the
 *     whole batch in equal ranges, one per workgroup, which leaves at most two
 *     partials of the G query heads of a KV head: N * 2 * G * (head_dim + 2)
 *     * 4 bytes for N <= 512 workgroups.
 * Guarantees: the size depends only on the arguments of this call; it is 0 for
 * SWA_DTYPE_F32, for window < 512 and when num_seqs * n_kv_heads >= 2048; it
 * never exceeds SWA_DECODE_WORKSPACE_MAX_BYTES.
 */
#define SWA_DECODE_WORKSPACE_MAX_BYTES ((size_t)8 << 20)
size_t swa_decode_workspace_size(const swa_cache *cache, int32_t num_seqs, int32_t n_q_heads);

/*
 * Single-token decode (paragraph "Pre-fill and Chunking": generation is token
 * by token).  Sequence b has exactly one new token, row b of q / out, at
 * absolute position pos = start_pos[b]; its keys and values must already be in
 * the cache (enqueue swa_cache_write first: slot pos mod W then held pos - W,
 * which is outside the window of pos).  The query attends to the
 * min(pos + 1, W) valid slots of its ring, which hold positions
 * max(0, pos-W+1) .. pos.
 * batch.total_tokens must equal num_seqs and max_new_tokens must be 1;
 * cu_seqlens is not read.
 * q, out: device [num_seqs][n_q_heads][head_dim].
 * workspace: device, at least swa_decode_workspace_size() bytes (may be NULL
 * when that is 0).  Calls that share a workspace must not overlap.
 */
int swa_decode(const swa_cache *cache, const swa_batch *batch,
               const void *q, int32_t n_q_heads, float sm_scale, void *out,
               void *workspace, size_t workspace_bytes, void *stream);

/*
 * Fused decode step (paragraphs "Rolling Buffer Cache" and "Pre-fill and
 * Chunking": a generated token's keys and values go to slot pos mod W, and the
 * token then attends to the window).  Same result as
 *     swa_cache_write(cache, batch, k_new, v_new, stream);
 *     swa_decode(cache, batch, q, n_q_heads, sm_scale, out, workspace, workspace_bytes, stream);
 * -- cache contents and output bit for bit -- in one attention launch (plus the
 * split-merge launch when the plan splits the window): the new token's K/V
 * enter the attention directly from k_new / v_new and are written to their
 * slot by the same launch.  It removes a launch per generated token and, like
 * every entry point, calls no memset and allocates nothing, so a step can be
 * captured in a HIP graph and replayed.
 * k_new, v_new: device [num_seqs][n_kv_heads][head_dim], 16-byte aligned,
 * NULL rejected.  Batch, q, out and workspace as for swa_decode (the workspace
 * size is swa_decode_workspace_size()).  Sequences must use distinct cache
 * rows (checked when h_cache_idx is given).
 */
int swa_decode_step(const swa_cache *cache, const swa_batch *batch,
                    const void *q, int32_t n_q_heads,
                    const void *k_new, const void *v_new,
                    float sm_scale, void *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * swa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, validation and result
 * as swa_decode_step -- output and cache bit for bit -- but the merge
 * partials go to a device array inside the library of
 * SWA_DECODE_WORKSPACE_MAX_BYTES bytes (8 MiB), one per GPU, held until the
 * process ends.  It calls no allocator.  The first call on a GPU looks up the
 * array's address (make it outside a graph capture); later calls only
 * launch.  Limits and hazards:
 *   - SWA_ERR_WORKSPACE if the plan would need more than the array holds
 *     (swa_decode_workspace_size() > SWA_DECODE_WORKSPACE_MAX_BYTES; never
 *     the case for head_dim <= 128);
 *   - `stream` must belong to the current device (SWA_ERR_INVALID_ARGUMENT);
 *   - all calls on one GPU share the array: calls that overlap in time on one
 *     GPU (different streams, or concurrent graph replays) race and give wrong
 *     results.  Calls ordered on one stream are safe.
 */
int swa_decode_step_noalloc(const swa_cache *cache, const swa_batch *batch,
                            const void *q, int32_t n_q_heads,
                            const void *k_new, const void *v_new,
                            float sm_scale, void *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
