// Rolling-buffer cache write for gfx950.
//
// Mistral 7B (Chinese translation), section 2, paragraph "Rolling Buffer
// Cache" and the Figure 2 caption: the keys and values of time step i are
// stored at slot i mod W of a cache of fixed size W, overwriting what an
// earlier position left there.
//
// One thread moves one 16-byte piece of one row (token, KV head).  Only the
// last min(C, W) tokens of a sequence are copied: every earlier token maps to
// a slot that a later token of the same call overwrites, so skipping them
// gives exactly the in-order result and no two threads ever write the same
// bytes.  Pure HBM copy: 2 (K, V) x 2 (read + write) x tokens x Hkv x row bytes.
#include "device_common.h"
#include "swa_internal.h"

namespace swa {

__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p) {
  const int b = blockIdx.y;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_token = p.n_kv_heads * p.row_chunks;
  const int64_t t = idx / per_token;
  const int rem = (int)(idx - t * per_token);
  const int g = rem / p.row_chunks;
  const int ch = rem - g * p.row_chunks;

  const int32_t tok0 = p.seq.cu_seqlens[b];
  const int32_t n_new = p.seq.cu_seqlens[b + 1] - tok0;
  if (t >= n_new || t < (int64_t)n_new - p.window) return;

  const int64_t pos = (int64_t)p.seq.start_pos[b] + t;
  const int64_t slot = pos % p.window;
  const int64_t row = p.seq.cache_idx ? p.seq.cache_idx[b] : b;
  const int64_t dst = (((row * p.n_kv_heads + g) * p.window + slot) * p.row_chunks + ch);
  const int64_t src = (((int64_t)tok0 + t) * p.n_kv_heads + g) * p.row_chunks + ch;

  const u32x4 *src_v = (const u32x4 *)(blockIdx.z == 0 ? p.k_new : p.v_new);
  u32x4 *dst_v = (u32x4 *)(blockIdx.z == 0 ? p.cache_k : p.cache_v);
  dst_v[dst] = __builtin_nontemporal_load(src_v + src);
}

hipError_t launch_cache_write(const CacheWriteParams &p, hipStream_t stream) {
  if (p.seq.num_seqs == 0 || p.seq.max_new_tokens == 0) return hipSuccess;
  // One thread per 16-byte piece of the first max_new_tokens tokens of each
  // sequence (grid.y = sequence, grid.z = K or V); threads past a sequence's
  // length, or of tokens overwritten later in the same call, return at once.
  const int64_t threads = (int64_t)p.seq.max_new_tokens * p.n_kv_heads * p.row_chunks;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks, (unsigned)p.seq.num_seqs, 2), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace swa
