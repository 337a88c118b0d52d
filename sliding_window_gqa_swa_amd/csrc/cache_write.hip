// Rolling-buffer cache write for gfx950.
//
// Mistral 7B (Chinese translation), section 2, paragraph "Rolling Buffer
// Cache" and the Figure 2 caption: the keys and values of time step i are
// stored at slot i mod W of a cache of fixed size W, overwriting what an
// earlier position left there.
//
// A thread moves 16-byte pieces of rows (token, KV head) of K and the same
// pieces of V.  Only the last min(C, W) tokens of a sequence are copied:
// every earlier token maps to a slot that a later token of the same call
// overwrites, so skipping them gives exactly the in-order result and no two
// threads ever write the same bytes.  Pure HBM copy: 2 (K, V) x 2 (read + write) x tokens x Hkv x row bytes.
#include "device_common.h"
#include "swa_internal.h"

namespace swa {

constexpr int kThreads = 1024;
constexpr int kPiecesPerThread = 2;

// Each thread streams pieces idx, idx + stride, ... of its sequence, issuing
// the loads of the next piece before it stores the current one.  With one
// piece per thread every wave loads, waits, then stores, so the launch reads
// everything before it writes anything; two pieces per thread overlap the
// second half's reads with the first half's writes.  The loads are ordinary
// (cached) loads: the chunk's K/V were just read by the prefill of the same
// chunk, and cached loads find them where non-temporal ones went to memory
// (16384-token chunk right after its prefill: 11.0 -> 9.8 us between events).
// 1024-thread workgroups, a quarter as many as with 256, measured fastest
// there (256 x 4 or 512 x 2 or 4 pieces: 10.3-10.7 us).
__global__ __launch_bounds__(kThreads) void cache_write_kernel(CacheWriteParams p, int n_wg_x) {
  const int b = wg_y();
  const int32_t tok0 = p.seq.cu_seqlens[b];
  const int32_t n_new = p.seq.cu_seqlens[b + 1] - tok0;
  const int32_t n_write = n_new < p.window ? n_new : p.window;  // the last min(C, W) tokens
  const int per_token = p.n_kv_heads * p.row_chunks;
  const int64_t total = (int64_t)n_write * per_token;          // pieces this sequence writes
  const int64_t stride = (int64_t)n_wg_x * kThreads;
  int64_t idx = (int64_t)wg_x() * kThreads + thread_x();
  if (idx >= total) return;
  const int64_t t_skip = (int64_t)(n_new - n_write);           // tokens whose slots a later token takes
  const int64_t pos0 = (int64_t)p.seq.start_pos[b] + t_skip;
  const int64_t row = p.seq.cache_idx ? p.seq.cache_idx[b] : b;
  const u32x4 *ksrc = (const u32x4 *)p.k_new + ((int64_t)tok0 + t_skip) * per_token;
  const u32x4 *vsrc = (const u32x4 *)p.v_new + ((int64_t)tok0 + t_skip) * per_token;
  // piece i = (token tw, KV head g, 16-byte chunk ch) -> slot (pos0 + tw) mod W of ring (row, g)
  auto dst_of = [&](int64_t i) {
    const int64_t tw = i / per_token;
    const int rem = (int)(i - tw * per_token);
    const int g = rem / p.row_chunks;
    const int ch = rem - g * p.row_chunks;
    return ((row * p.n_kv_heads + g) * p.window + (pos0 + tw) % p.window) * p.row_chunks + ch;
  };

  u32x4 kx = ksrc[idx];
  u32x4 vx = vsrc[idx];
  for (;;) {
    const int64_t nx = idx + stride;
    u32x4 kn = kx, vn = vx;
    if (nx < total) {
      kn = ksrc[nx];
      vn = vsrc[nx];
    }
    const int64_t d = dst_of(idx);
    ((u32x4 *)p.cache_k)[d] = kx;
    ((u32x4 *)p.cache_v)[d] = vx;
    if (nx >= total) break;
    idx = nx;
    kx = kn;
    vx = vn;
  }
}

hipError_t launch_cache_write(const CacheWriteParams &p, hipStream_t stream) {
  if (p.seq.num_seqs == 0 || p.seq.max_new_tokens == 0) return hipSuccess;
  // grid.y = sequence; grid.x covers min(max_new_tokens, W) tokens at
  // kPiecesPerThread 16-byte pieces (of K and of V) per thread.
  const int64_t rows = p.seq.max_new_tokens < p.window ? p.seq.max_new_tokens : p.window;
  const int64_t pieces = rows * p.n_kv_heads * p.row_chunks;
  const int64_t blocks = (pieces + kThreads * kPiecesPerThread - 1) / (kThreads * kPiecesPerThread);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks, (unsigned)p.seq.num_seqs), dim3(kThreads), 0, stream,
                     p, (int)blocks);
  return hipGetLastError();
}

}  // namespace swa
