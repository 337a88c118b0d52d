// C ABI of libswa: argument validation, launch planning and dispatch.
// The operations are defined in include/swa.h; every check here runs on the
// host before anything is enqueued.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "../../include/swa.h"
#include "swa_internal.h"

namespace swa {

static int elt_bytes(int32_t dtype) {
  switch (dtype) {
    case SWA_DTYPE_BF16: return 2;
    case SWA_DTYPE_F32: return 4;
    default: return 0;
  }
}

static bool aligned16(const void *p) { return (((uintptr_t)p) & 15u) == 0; }

// Shapes the kernels are compiled for.
static bool head_dim_supported(int32_t dtype, int32_t d) {
  (void)dtype;  // both dtypes are compiled for the same head dims
  return d == 16 || d == 64 || d == 128;
}

static swa_status check_cache(const swa_cache *c, bool need_ptrs) {
  if (!c) return SWA_ERR_INVALID_ARGUMENT;
  if (c->reserved != 0) return SWA_ERR_INVALID_ARGUMENT;
  if (c->n_cache < 1 || c->n_kv_heads < 1 || c->head_dim < 1 || c->window < 1) return SWA_ERR_INVALID_ARGUMENT;
  if (c->window > (1 << 30)) return SWA_ERR_UNSUPPORTED;  // keeps window + tile offsets inside int32
  const int eb = elt_bytes(c->dtype);
  if (eb == 0) return SWA_ERR_INVALID_ARGUMENT;
  if (need_ptrs && (!c->k || !c->v)) return SWA_ERR_INVALID_ARGUMENT;
  if ((c->k && !aligned16(c->k)) || (c->v && !aligned16(c->v))) return SWA_ERR_INVALID_ARGUMENT;
  // element count must fit comfortably in 64-bit byte offsets
  const double elems = (double)c->n_cache * c->n_kv_heads * (double)c->window * c->head_dim;
  if (elems * eb > 9.0e18) return SWA_ERR_INVALID_ARGUMENT;
  if (((int64_t)c->head_dim * eb) % 16 != 0) return SWA_ERR_UNSUPPORTED;
  if (!head_dim_supported(c->dtype, c->head_dim)) return SWA_ERR_UNSUPPORTED;
  return SWA_OK;
}

// Checks shared by every entry point.  `decode`: one token per sequence.
static swa_status check_batch(const swa_batch *bt, const swa_cache *c, bool decode, bool distinct_rows) {
  if (!bt) return SWA_ERR_INVALID_ARGUMENT;
  if (bt->reserved != 0) return SWA_ERR_INVALID_ARGUMENT;
  if (bt->num_seqs < 0 || bt->total_tokens < 0 || bt->max_new_tokens < 0) return SWA_ERR_INVALID_ARGUMENT;
  if (bt->num_seqs > 65535) return SWA_ERR_UNSUPPORTED;
  const int n = bt->num_seqs;
  if (n == 0) return (bt->total_tokens == 0) ? SWA_OK : SWA_ERR_INVALID_ARGUMENT;
  if (!bt->start_pos) return SWA_ERR_INVALID_ARGUMENT;
  if (!bt->cache_idx && n > c->n_cache) return SWA_ERR_INVALID_ARGUMENT;
  if (decode) {
    if (bt->total_tokens != n || bt->max_new_tokens != 1) return SWA_ERR_INVALID_ARGUMENT;
  } else {
    if (!bt->cu_seqlens) return SWA_ERR_INVALID_ARGUMENT;
    if (bt->max_new_tokens > bt->total_tokens) return SWA_ERR_INVALID_ARGUMENT;
    if ((int64_t)bt->max_new_tokens * n < bt->total_tokens) return SWA_ERR_INVALID_ARGUMENT;
  }
  if (!decode && bt->h_cu_seqlens) {
    const int32_t *cu = bt->h_cu_seqlens;
    if (cu[0] != 0 || cu[n] != bt->total_tokens) return SWA_ERR_INVALID_ARGUMENT;
    for (int b = 0; b < n; b++) {
      const int64_t len = (int64_t)cu[b + 1] - cu[b];
      if (len < 0 || len > bt->max_new_tokens) return SWA_ERR_INVALID_ARGUMENT;
    }
  }
  if (bt->h_start_pos) {
    for (int b = 0; b < n; b++) {
      const int64_t sp = bt->h_start_pos[b];
      int64_t len = decode ? 1 : bt->max_new_tokens;
      if (!decode && bt->h_cu_seqlens) len = (int64_t)bt->h_cu_seqlens[b + 1] - bt->h_cu_seqlens[b];
      if (sp < 0 || sp + len > INT32_MAX) return SWA_ERR_INVALID_ARGUMENT;
    }
  }
  if (bt->cache_idx && bt->h_cache_idx) {
    for (int b = 0; b < n; b++)
      if (bt->h_cache_idx[b] < 0 || bt->h_cache_idx[b] >= c->n_cache) return SWA_ERR_INVALID_ARGUMENT;
    if (distinct_rows) {
      std::vector<int32_t> rows(bt->h_cache_idx, bt->h_cache_idx + n);
      std::sort(rows.begin(), rows.end());
      if (std::adjacent_find(rows.begin(), rows.end()) != rows.end()) return SWA_ERR_INVALID_ARGUMENT;
    }
  }
  return SWA_OK;
}

static SeqMeta seq_meta(const swa_batch *bt, bool decode) {
  SeqMeta s;
  s.cu_seqlens = decode ? nullptr : bt->cu_seqlens;
  s.start_pos = bt->start_pos;
  s.cache_idx = bt->cache_idx;
  s.num_seqs = bt->num_seqs;
  s.max_new_tokens = bt->max_new_tokens;
  return s;
}

static CacheRef cache_ref(const swa_cache *c) {
  CacheRef r;
  r.k = c->k;
  r.v = c->v;
  r.n_kv_heads = c->n_kv_heads;
  r.head_dim = c->head_dim;
  r.window = c->window;
  r.elt_bytes = elt_bytes(c->dtype);
  return r;
}

static swa_status check_heads(const swa_cache *c, int32_t n_q_heads) {
  if (n_q_heads < 1 || n_q_heads % c->n_kv_heads != 0) return SWA_ERR_INVALID_ARGUMENT;
  const int group = n_q_heads / c->n_kv_heads;
  if (c->dtype == SWA_DTYPE_BF16 && group != 1 && group != 2 && group != 4 && group != 8) return SWA_ERR_UNSUPPORTED;
  return SWA_OK;
}

static bool scale_ok(float s) { return isfinite(s) && s > 0.f; }

// bf16 decode runs on the matrix cores (decode_mfma.hip), except G = 1 at
// head_dim 128, which has its own VALU kernel (decode_bf16.hip).
static bool decode_on_valu(int32_t group, int32_t head_dim) { return group == 1 && head_dim == 128; }

DecodePlan plan_decode(int32_t num_seqs, int32_t n_kv_heads, int32_t n_q_heads, int32_t head_dim, int32_t window,
                       int32_t dtype) {
  DecodePlan pl{1, window, 0, 0, 0};
  if (dtype != SWA_DTYPE_BF16 || num_seqs <= 0) return pl;
  // Workgroups per launch to aim for.  The VALU kernel (G = 1) wants >= ~2048
  // (8 per CU).  The matrix-core kernel (G >= 2) holds 2 workgroups per CU, so
  // 512 fill the chip once: 64 sequences x 8 KV heads then take one split per
  // ring and need no merge launch.  A split of a full window keeps >= 256
  // slots either way, so that each wave streams several 16 KiB steps; smaller
  // batches on the matrix-core kernel go to the stream plan below.
  const int64_t pairs = (int64_t)num_seqs * n_kv_heads;
  const int32_t group = n_q_heads / n_kv_heads;
  const bool valu = decode_on_valu(group, head_dim);
  const int64_t target_wg = valu ? 2048 : 512;
  int64_t max_splits = std::max<int64_t>(1, window / 256);
  int64_t splits = std::min<int64_t>(max_splits, std::max<int64_t>(1, (target_wg + pairs - 1) / pairs));
  int64_t len = (window + splits - 1) / splits;
  len = (len + 31) / 32 * 32;
  splits = (window + len - 1) / len;
  if (splits == 1) return pl;
  if (!valu && head_dim >= 64 && num_seqs >= 2 && num_seqs <= kStreamMaxSeqs &&
      pairs * window <= (int64_t(1) << 30)) {
    // Too few rings to fill the chip one workgroup each: the matrix-core
    // kernel runs in stream mode, where every workgroup takes an equal share
    // of the batch's valid slots whatever each sequence's context length,
    // with at most two partial results per workgroup.  (One sequence has the
    // same context in every KV head: its split plan is balanced already.  At
    // head_dim 16 the whole launch is short and latency-bound, and the stream
    // prologue and piece changes cost more than the balance gains.)
    const int64_t wg = std::min<int64_t>(target_wg, (pairs * window + kStreamWgRows - 1) / kStreamWgRows);
    pl.stream_wg = (int32_t)wg;
    pl.acc_floats = (size_t)wg * 2 * group * head_dim;
    pl.workspace_bytes = (size_t)wg * 2 * group * (head_dim + 2) * sizeof(float);
    return pl;
  }
  pl.splits = (int32_t)splits;
  pl.split_len = (int32_t)len;
  pl.acc_floats = (size_t)num_seqs * n_q_heads * splits * head_dim;
  pl.workspace_bytes = (size_t)num_seqs * n_q_heads * splits * (head_dim + 2) * sizeof(float);
  return pl;
}

// swa_decode (k_new == NULL) and swa_decode_step (k_new, v_new given).
static int decode_impl(const swa_cache *cache, const swa_batch *batch, const void *q, int32_t n_q_heads,
                       const void *k_new, const void *v_new, float sm_scale, void *out, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  const bool fused = k_new != nullptr;
  swa_status st = check_cache(cache, true);
  if (st != SWA_OK) return st;
  st = check_heads(cache, n_q_heads);
  if (st != SWA_OK) return st;
  st = check_batch(batch, cache, true, fused);  // the fused step writes: rows must be distinct
  if (st != SWA_OK) return st;
  if (!scale_ok(sm_scale)) return SWA_ERR_INVALID_ARGUMENT;
  if (batch->num_seqs == 0) return SWA_OK;
  if (!q || !out || !aligned16(q) || !aligned16(out)) return SWA_ERR_INVALID_ARGUMENT;
  if (fused && (!aligned16(k_new) || !aligned16(v_new))) return SWA_ERR_INVALID_ARGUMENT;
  const DecodePlan pl = plan_decode(batch->num_seqs, cache->n_kv_heads, n_q_heads, cache->head_dim, cache->window,
                                    cache->dtype);
  if (pl.workspace_bytes > 0) {
    if (!workspace || workspace_bytes < pl.workspace_bytes) return SWA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SWA_ERR_INVALID_ARGUMENT;
  }
  DecodeParams p{};
  p.seq = seq_meta(batch, true);
  p.cache = cache_ref(cache);
  p.q = q;
  p.out = out;
  if (fused) {
    p.k_new = k_new;
    p.v_new = v_new;
    p.cache_k_out = cache->k;
    p.cache_v_out = cache->v;
  }
  p.n_q_heads = n_q_heads;
  p.splits = pl.splits;
  p.split_len = pl.split_len;
  p.stream_wg = pl.stream_wg;
  p.sm_scale = sm_scale;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  if (pl.workspace_bytes > 0) {
    p.ws_acc = (float *)workspace;
    p.ws_ml = p.ws_acc + pl.acc_floats;
  }
  hipError_t e;
  const int group = n_q_heads / cache->n_kv_heads;
  if (cache->dtype == SWA_DTYPE_BF16)
    e = decode_on_valu(group, cache->head_dim) ? launch_decode_bf16(p, group, stream)
                                               : launch_decode_mfma_bf16(p, group, stream);
  else
    e = launch_decode_f32(p, stream);
  return e == hipSuccess ? SWA_OK : SWA_ERR_HIP;
}

}  // namespace swa

// Split partials of swa_decode_step_noalloc, for callers that cannot allocate
// device memory.  Each GPU the library runs on holds its own copy until the
// process ends; every call on that GPU shares it.  The decode kernels write
// every partial they later read, so nothing needs to start at zero.
static __device__ __align__(256) unsigned char scratch[SWA_DECODE_WORKSPACE_MAX_BYTES];

namespace swa {

constexpr int kMaxDevices = 1024;
static std::mutex g_scratch_mutex;
static void *g_scratch_ptr[kMaxDevices];

// Device address of the current GPU's copy of `scratch`.  In host code the
// array's name is only a host-side handle, so the address is looked up once
// per device, with that device current, and only this pointer reaches kernels.
static swa_status scratch_of_current_device(hipStream_t stream, void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SWA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SWA_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return SWA_ERR_HIP;
    if ((int)sdev != dev) return SWA_ERR_INVALID_ARGUMENT;  // the stream must belong to the current device
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SWA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SWA_OK;
}

}  // namespace swa

using namespace swa;

extern "C" {

int swa_abi_version(void) { return SWA_ABI_VERSION; }

const char *swa_status_string(int status) {
  switch (status) {
    case SWA_OK: return "SWA_OK";
    case SWA_ERR_INVALID_ARGUMENT: return "SWA_ERR_INVALID_ARGUMENT: invalid argument";
    case SWA_ERR_UNSUPPORTED: return "SWA_ERR_UNSUPPORTED: shape or dtype not compiled into this library";
    case SWA_ERR_WORKSPACE: return "SWA_ERR_WORKSPACE: decode workspace missing or too small";
    case SWA_ERR_HIP: return "SWA_ERR_HIP: a HIP launch failed";
    case SWA_ERR_INTERNAL: return "SWA_ERR_INTERNAL: internal error";
    default: return "unknown swa_status";
  }
}

int swa_cache_write(const swa_cache *cache, const swa_batch *batch, const void *k_new, const void *v_new,
                    void *stream) {
  try {
    swa_status st = check_cache(cache, true);
    if (st != SWA_OK) return st;
    st = check_batch(batch, cache, false, true);
    if (st != SWA_OK) return st;
    if (batch->num_seqs == 0 || batch->total_tokens == 0) return SWA_OK;
    if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return SWA_ERR_INVALID_ARGUMENT;
    CacheWriteParams p;
    p.seq = seq_meta(batch, false);
    p.cache_k = cache->k;
    p.cache_v = cache->v;
    p.k_new = k_new;
    p.v_new = v_new;
    p.n_kv_heads = cache->n_kv_heads;
    p.window = cache->window;
    p.row_chunks = cache->head_dim * elt_bytes(cache->dtype) / 16;
    return launch_cache_write(p, (hipStream_t)stream) == hipSuccess ? SWA_OK : SWA_ERR_HIP;
  } catch (...) {
    return SWA_ERR_INTERNAL;
  }
}

}  // extern "C"

// swa_prefill_chunk, and (visit_all_tiles) its measurement variant without the band tile skip.
static int prefill_impl(const swa_cache *cache, const swa_batch *batch, const void *q, int32_t n_q_heads,
                        const void *k_new, const void *v_new, float sm_scale, void *out, void *stream,
                        bool visit_all_tiles) {
  try {
    swa_status st = check_cache(cache, false);
    if (st != SWA_OK) return st;
    st = check_heads(cache, n_q_heads);
    if (st != SWA_OK) return st;
    st = check_batch(batch, cache, false, false);
    if (st != SWA_OK) return st;
    if (!scale_ok(sm_scale)) return SWA_ERR_INVALID_ARGUMENT;
    if (batch->num_seqs == 0 || batch->total_tokens == 0) return SWA_OK;
    if (!q || !k_new || !v_new || !out) return SWA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out)) return SWA_ERR_INVALID_ARGUMENT;
    if (!cache->k || !cache->v) {
      // no cache: only allowed when every sequence starts at position 0
      if (cache->k || cache->v || !batch->h_start_pos) return SWA_ERR_INVALID_ARGUMENT;
      for (int b = 0; b < batch->num_seqs; b++)
        if (batch->h_start_pos[b] != 0) return SWA_ERR_INVALID_ARGUMENT;
    }
    PrefillParams p{};
    p.seq = seq_meta(batch, false);
    p.cache = cache_ref(cache);
    p.q = q;
    p.k_new = k_new;
    p.v_new = v_new;
    p.out = out;
    p.n_q_heads = n_q_heads;
    p.sm_scale = sm_scale;
    p.scale_log2 = sm_scale * 1.4426950408889634f;
    p.visit_all_tiles = visit_all_tiles ? 1 : 0;
    hipError_t e;
    if (cache->dtype == SWA_DTYPE_BF16) {
      const int group = n_q_heads / cache->n_kv_heads;
      const int rows = prefill_bf16_tile_rows(group);
      const int64_t tps = (batch->max_new_tokens + rows - 1) / rows;
      const int64_t n_work = tps * batch->num_seqs * cache->n_kv_heads;
      if (n_work > INT32_MAX) return SWA_ERR_UNSUPPORTED;
      p.tiles_per_seq = (int32_t)tps;
      p.n_work = (int32_t)n_work;
      e = launch_prefill_bf16(p, group, (hipStream_t)stream);
    } else {
      if (visit_all_tiles) return SWA_ERR_UNSUPPORTED;  // the fp32 path has no key tiles
      e = launch_prefill_f32(p, (hipStream_t)stream);
    }
    return e == hipSuccess ? SWA_OK : SWA_ERR_HIP;
  } catch (...) {
    return SWA_ERR_INTERNAL;
  }
}

extern "C" {

int swa_prefill_chunk(const swa_cache *cache, const swa_batch *batch, const void *q, int32_t n_q_heads,
                      const void *k_new, const void *v_new, float sm_scale, void *out, void *stream) {
  return prefill_impl(cache, batch, q, n_q_heads, k_new, v_new, sm_scale, out, stream, false);
}

int swa_prefill_chunk_no_tile_skip(const swa_cache *cache, const swa_batch *batch, const void *q,
                                   int32_t n_q_heads, const void *k_new, const void *v_new, float sm_scale,
                                   void *out, void *stream) {
  return prefill_impl(cache, batch, q, n_q_heads, k_new, v_new, sm_scale, out, stream, true);
}

size_t swa_decode_workspace_size(const swa_cache *cache, int32_t num_seqs, int32_t n_q_heads) {
  if (check_cache(cache, false) != SWA_OK || num_seqs < 0 || check_heads(cache, n_q_heads) != SWA_OK) return 0;
  return plan_decode(num_seqs, cache->n_kv_heads, n_q_heads, cache->head_dim, cache->window, cache->dtype)
      .workspace_bytes;
}

int swa_decode(const swa_cache *cache, const swa_batch *batch, const void *q, int32_t n_q_heads, float sm_scale,
               void *out, void *workspace, size_t workspace_bytes, void *stream) {
  try {
    return decode_impl(cache, batch, q, n_q_heads, nullptr, nullptr, sm_scale, out, workspace, workspace_bytes,
                       (hipStream_t)stream);
  } catch (...) {
    return SWA_ERR_INTERNAL;
  }
}

int swa_decode_step(const swa_cache *cache, const swa_batch *batch, const void *q, int32_t n_q_heads,
                    const void *k_new, const void *v_new, float sm_scale, void *out, void *workspace,
                    size_t workspace_bytes, void *stream) {
  try {
    if (!k_new || !v_new) return SWA_ERR_INVALID_ARGUMENT;
    return decode_impl(cache, batch, q, n_q_heads, k_new, v_new, sm_scale, out, workspace, workspace_bytes,
                       (hipStream_t)stream);
  } catch (...) {
    return SWA_ERR_INTERNAL;
  }
}

int swa_decode_step_noalloc(const swa_cache *cache, const swa_batch *batch, const void *q, int32_t n_q_heads,
                            const void *k_new, const void *v_new, float sm_scale, void *out, void *stream) {
  try {
    if (!k_new || !v_new) return SWA_ERR_INVALID_ARGUMENT;
    // the validation of swa_decode_step, before the scratch is looked up
    swa_status st = check_cache(cache, true);
    if (st != SWA_OK) return st;
    st = check_heads(cache, n_q_heads);
    if (st != SWA_OK) return st;
    st = check_batch(batch, cache, true, true);
    if (st != SWA_OK) return st;
    if (!scale_ok(sm_scale)) return SWA_ERR_INVALID_ARGUMENT;
    if (batch->num_seqs == 0) return SWA_OK;
    if (!q || !out || !aligned16(q) || !aligned16(out) || !aligned16(k_new) || !aligned16(v_new))
      return SWA_ERR_INVALID_ARGUMENT;
    const size_t need = swa_decode_workspace_size(cache, batch->num_seqs, n_q_heads);
    if (need > SWA_DECODE_WORKSPACE_MAX_BYTES) return SWA_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
      st = scratch_of_current_device((hipStream_t)stream, &ws);
      if (st != SWA_OK) return st;
    }
    return decode_impl(cache, batch, q, n_q_heads, k_new, v_new, sm_scale, out, ws, need, (hipStream_t)stream);
  } catch (...) {
    return SWA_ERR_INTERNAL;
  }
}

}  // extern "C"
