// Launch parameters and launchers shared between the C-ABI layer (api.hip) and
// the kernels.  Plain structs passed by value to the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swa {

// Metadata of the sequences of one call (device pointers).
struct SeqMeta {
  const int32_t *cu_seqlens;  // [num_seqs + 1]; NULL in decode (token b = sequence b)
  const int32_t *start_pos;   // [num_seqs]
  const int32_t *cache_idx;   // [num_seqs] or NULL (row b)
  int32_t num_seqs;
  int32_t max_new_tokens;
};

struct CacheRef {
  const void *k;
  const void *v;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t window;
  int32_t elt_bytes;
};

struct CacheWriteParams {
  SeqMeta seq;
  void *cache_k;
  void *cache_v;
  const void *k_new;
  const void *v_new;
  int32_t n_kv_heads;
  int32_t window;
  int32_t row_chunks;  // 16-byte chunks per row (head_dim * elt / 16)
};

struct PrefillParams {
  SeqMeta seq;
  CacheRef cache;
  const void *q;
  const void *k_new;
  const void *v_new;
  void *out;
  void *cache_k_out;  // fp32 fused decode step only: the writable cache
  void *cache_v_out;
  int32_t n_q_heads;
  int32_t tiles_per_seq;  // query tiles per sequence (ceil(max_new_tokens / tile))
  int32_t n_work;         // num_seqs * tiles_per_seq * n_kv_heads
  float scale_log2;       // sm_scale * log2(e)
  float sm_scale;
  int32_t visit_all_tiles;  // measurement variant: no band tile skip (bf16 prefill)
};

struct DecodeParams {
  SeqMeta seq;
  CacheRef cache;
  const void *q;
  void *out;
  // Fused step (write, then attend, in one launch): the new token's K/V rows
  // [num_seqs][n_kv_heads][head_dim] and the writable cache.  NULL k_new:
  // plain decode over a cache that already holds the new token.
  const void *k_new;
  const void *v_new;
  void *cache_k_out;
  void *cache_v_out;
  // Partial results: split mode [num_seqs][n_q_heads][splits][head_dim] and
  // [..][2] (max in log2 units, sum); stream mode [stream_wg][2][G][head_dim]
  // and [..][2], two slots per workgroup.
  float *ws_acc;
  float *ws_ml;
  int32_t n_q_heads;
  int32_t splits;
  int32_t split_len;  // slots per split for a full window (see seq_split_len)
  int32_t stream_wg;  // > 0: stream mode with this many workgroups (see stream_range_rows)
  float scale_log2;
  float sm_scale;
};

// Slots per split of one sequence in a decode launch.  The plan fixes the
// number of splits and a split length that covers the whole window; a
// sequence with fewer valid slots spreads them evenly over all its splits
// instead (multiples of 32, at least kMinSplitRows), so a short context still
// runs on every split.  splits * result >= n_valid always holds.
constexpr int kMinSplitRows = 128;
__device__ __forceinline__ int seq_split_len(int n_valid, int splits, int plan_len) {
  int len = (n_valid + splits - 1) / splits;
  len = (len + 31) & ~31;
  len = len > kMinSplitRows ? len : kMinSplitRows;
  return len < plan_len ? len : plan_len;
}

// Stream mode of the matrix-core decode (small batches): the valid slots of
// all (sequence, KV head) pairs, laid end to end sequence-major, are cut into
// stream_wg contiguous ranges of equal length, one per workgroup, so that
// sequences of different context lengths cost the same per slot.  The plan
// sizes the grid for ranges of kStreamWgRows slots of full windows; the range
// length is a multiple of 32, at least kStreamMinRows, so short contexts still
// spread over many workgroups.  total_rows <= 2^30 (the plan checks pairs x W).
constexpr int kStreamWgRows = 256;
constexpr int kStreamMinRows = 128;
constexpr int kStreamMaxSeqs = 64;  // one wave scans the batch
__host__ __device__ __forceinline__ int stream_range_rows(int total_rows, int stream_wg) {
  int len = (total_rows + stream_wg - 1) / stream_wg;
  len = (len + 31) & ~31;
  return len > kStreamMinRows ? len : kStreamMinRows;
}

// Decode plan: how the window of each (sequence, KV head) is split across
// workgroups (split mode), or how many workgroups share the batch's slots
// (stream mode, stream_wg > 0).
struct DecodePlan {
  int32_t splits;
  int32_t split_len;
  int32_t stream_wg;
  size_t acc_floats;  // floats of ws_acc; ws_ml follows them
  size_t workspace_bytes;
};
DecodePlan plan_decode(int32_t num_seqs, int32_t n_kv_heads, int32_t n_q_heads, int32_t head_dim,
                       int32_t window, int32_t dtype);

hipError_t launch_cache_write(const CacheWriteParams &p, hipStream_t stream);
int prefill_bf16_tile_rows(int group);
hipError_t launch_prefill_bf16(const PrefillParams &p, int group, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillParams &p, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams &p, int group, hipStream_t stream);       // group 1
hipError_t launch_decode_mfma_bf16(const DecodeParams &p, int group, hipStream_t stream);  // group 2, 4, 8
hipError_t launch_decode_combine_bf16(const DecodeParams &p, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeParams &p, hipStream_t stream);

}  // namespace swa
