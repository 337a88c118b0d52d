// Rolling-buffer cache write for gfx950.
//
// Mistral 7B (Chinese translation), section 2, paragraph "Rolling Buffer
// Cache" and the Figure 2 caption: the keys and values of time step i are
// stored at slot i mod W of a cache of fixed size W, overwriting what an
// earlier position left there.
//
// One thread moves one 16-byte piece of one row (token, KV head) of K and the
// same piece of V.  Only the last min(C, W) tokens of a sequence are copied:
// every earlier token maps to a slot that a later token of the same call
// overwrites, so skipping them gives exactly the in-order result and no two
// threads ever write the same bytes.  Pure HBM copy: 2 (K, V) x 2 (read + write) x tokens x Hkv x row bytes.
#include "device_common.h"
#include "swa_internal.h"

namespace swa {

__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p) {
  const int b = wg_y();
  const int64_t idx = (int64_t)wg_x() * 256 + thread_x();
  const int per_token = p.n_kv_heads * p.row_chunks;
  const int64_t tw = idx / per_token;  // index among the tokens this sequence writes
  const int rem = (int)(idx - tw * per_token);
  const int g = rem / p.row_chunks;
  const int ch = rem - g * p.row_chunks;

  const int32_t tok0 = p.seq.cu_seqlens[b];
  const int32_t n_new = p.seq.cu_seqlens[b + 1] - tok0;
  const int32_t n_write = n_new < p.window ? n_new : p.window;  // the last min(C, W) tokens
  if (tw >= n_write) return;
  const int64_t t = (int64_t)(n_new - n_write) + tw;

  const int64_t pos = (int64_t)p.seq.start_pos[b] + t;
  const int64_t slot = pos % p.window;
  const int64_t row = p.seq.cache_idx ? p.seq.cache_idx[b] : b;
  const int64_t dst = (((row * p.n_kv_heads + g) * p.window + slot) * p.row_chunks + ch);
  const int64_t src = (((int64_t)tok0 + t) * p.n_kv_heads + g) * p.row_chunks + ch;

  // both loads in flight before either store
  const u32x4 kx = __builtin_nontemporal_load((const u32x4 *)p.k_new + src);
  const u32x4 vx = __builtin_nontemporal_load((const u32x4 *)p.v_new + src);
  ((u32x4 *)p.cache_k)[dst] = kx;
  ((u32x4 *)p.cache_v)[dst] = vx;
}

hipError_t launch_cache_write(const CacheWriteParams &p, hipStream_t stream) {
  if (p.seq.num_seqs == 0 || p.seq.max_new_tokens == 0) return hipSuccess;
  // One thread per 16-byte piece (of K and of V) of the tokens that are
  // written: grid.y = sequence, grid.x covers min(max_new_tokens, W) tokens.
  const int64_t rows = p.seq.max_new_tokens < p.window ? p.seq.max_new_tokens : p.window;
  const int64_t threads = rows * p.n_kv_heads * p.row_chunks;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks, (unsigned)p.seq.num_seqs), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace swa
