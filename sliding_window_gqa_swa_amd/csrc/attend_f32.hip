// fp32 sliding-window GQA attention (prefill and decode) for gfx950.
//
// The fp32 storage path exists for exactness checks at small sizes (fp32
// inputs, fp32 arithmetic end to end); the bf16 MFMA / streaming kernels are
// the performance path.  Same semantics as those kernels:
//   Mistral 7B (Chinese translation), section 2, paragraph "Sliding Window
//   Attention": the query at position i reads keys j, i-W < j <= i;
//   paragraph "Rolling Buffer Cache": key j lives in ring slot j mod W;
//   paragraph "Pre-fill and Chunking": keys inside the current chunk come from
//   the chunk itself, keys before it from the cache;
//   section 1: query head h reads KV head h / G.
//
// One wave per (token, query head).  Lanes take keys j = lo + lane, lo + lane
// + 64, ...; each lane keeps its own online-softmax state and full-width
// accumulator; the wave then merges the 64 partial states (log-sum-exp).
#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kWaves = 4;

// mode: 0 prefill, 1 decode (the new token is already in the ring), 2 fused
// decode step (the new token comes from k_new / v_new and is written to its
// slot by the first query head of each KV head)
template <int D>
__global__ __launch_bounds__(64 * kWaves) void attend_f32_kernel(PrefillParams p, int mode) {
  const bool decode = mode != 0;
  __shared__ float sq[kWaves][D];
  const int lane = thread_x() & 63, wave = thread_x() >> 6;
  const int b = wg_y();
  const int t = wg_x();
  const int h = wg_z() * kWaves + wave;
  const int hq = p.n_q_heads;
  const int hkv = p.cache.n_kv_heads;
  const int G = hq / hkv;
  const int g = h / G;

  int tok0, n_new;
  if (decode) {
    tok0 = b;
    n_new = 1;
  } else {
    tok0 = p.seq.cu_seqlens[b];
    n_new = p.seq.cu_seqlens[b + 1] - tok0;
  }
  const bool active = t < n_new && h < hq;
  const int s = p.seq.start_pos[b];
  const int i = s + t;               // absolute query position
  const int W = p.cache.window;
  // keys below ring_end come from the ring; in decode the query's own key is
  // already there, in prefill the chunk's keys come from k_new / v_new
  const int ring_end = mode == 1 ? s + 1 : s;
  const int crow = p.seq.cache_idx ? p.seq.cache_idx[b] : b;
  const float *Q = (const float *)p.q;
  if (active)
    for (int d = lane; d < D; d += 64) sq[wave][d] = Q[((size_t)(tok0 + t) * hq + h) * D + d];
  __syncthreads();
  if (!active) return;

  const float *ck = (const float *)p.cache.k, *cv = (const float *)p.cache.v;
  const float *kn = (const float *)p.k_new, *vn = (const float *)p.v_new;
  const size_t ring0 = ((size_t)crow * hkv + g) * (size_t)W;
  if (mode == 2 && h == g * G) {
    // slot i mod W held position i - W, outside the window of i: nobody reads it here
    float *wk = (float *)p.cache_k_out + (ring0 + (size_t)(i % W)) * D;
    float *wv = (float *)p.cache_v_out + (ring0 + (size_t)(i % W)) * D;
    const size_t off = ((size_t)tok0 * hkv + g) * D;
    for (int d = lane; d < D; d += 64) {
      wk[d] = kn[off + d];
      wv[d] = vn[off + d];
    }
  }
  const int lo = max(0, i - W + 1);
  const float cs = p.scale_log2;

  float m = -INFINITY, l = 0.f;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; d++) acc[d] = 0.f;

  const int n_keys = i - lo + 1;
  for (int r = lane; r < n_keys; r += 64) {  // relative index: no overflow near 2^31
    const int j = lo + r;
    const float *kr, *vr;
    if (j < ring_end) {
      const size_t off = (ring0 + (size_t)(j % W)) * D;
      kr = ck + off;
      vr = cv + off;
    } else {
      const size_t off = ((size_t)(tok0 + j - s) * hkv + g) * D;
      kr = kn + off;
      vr = vn + off;
    }
    float dot = 0.f;
#pragma unroll
    for (int d = 0; d < D; d++) dot = __builtin_fmaf(sq[wave][d], kr[d], dot);
    float sc, mn, alpha, pv;
    {
      // the rounded score is kept as is (no fusion of the product into the
      // subtraction), so a key that sets the running max gets weight exactly 1
#pragma clang fp contract(off)
      sc = dot * cs;
      mn = fmaxf(m, sc);
      alpha = exp2f(m - mn);  // m = -inf on the first key: 0
      pv = exp2f(sc - mn);
    }
    l = l * alpha + pv;
#pragma unroll
    for (int d = 0; d < D; d++) acc[d] = __builtin_fmaf(pv, vr[d], acc[d] * alpha);
    m = mn;
  }

  // log-sum-exp merge of the 64 lanes (lanes without keys have m = -inf, l = 0)
  float mx = m;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const float f = (m == -INFINITY) ? 0.f : exp2f(m - mx);
  l *= f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) l += __shfl_xor(l, off);
  const float inv = 1.0f / l;
  float *O = (float *)p.out + ((size_t)(tok0 + t) * hq + h) * D;
#pragma unroll
  for (int d = 0; d < D; d++) {
    float a = acc[d] * f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a += __shfl_xor(a, off);
    if (lane == (d & 63)) O[d] = a * inv;
  }
}

hipError_t launch(const PrefillParams &p, int mode, int max_new, hipStream_t stream) {
  if (p.seq.num_seqs == 0 || max_new == 0) return hipSuccess;
  dim3 grid((unsigned)max_new, (unsigned)p.seq.num_seqs, (unsigned)((p.n_q_heads + kWaves - 1) / kWaves));
  switch (p.cache.head_dim) {
    case 16: hipLaunchKernelGGL(attend_f32_kernel<16>, grid, dim3(64 * kWaves), 0, stream, p, mode); break;
    case 64: hipLaunchKernelGGL(attend_f32_kernel<64>, grid, dim3(64 * kWaves), 0, stream, p, mode); break;
    case 128: hipLaunchKernelGGL(attend_f32_kernel<128>, grid, dim3(64 * kWaves), 0, stream, p, mode); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams &p, hipStream_t stream) {
  return launch(p, 0, p.seq.max_new_tokens, stream);
}

hipError_t launch_decode_f32(const DecodeParams &d, hipStream_t stream) {
  PrefillParams p{};
  p.seq = d.seq;
  p.cache = d.cache;
  p.q = d.q;
  p.out = d.out;
  p.n_q_heads = d.n_q_heads;
  p.scale_log2 = d.scale_log2;
  p.sm_scale = d.sm_scale;
  p.k_new = d.k_new;
  p.v_new = d.v_new;
  p.cache_k_out = d.cache_k_out;
  p.cache_v_out = d.cache_v_out;
  return launch(p, d.k_new ? 2 : 1, 1, stream);
}

}  // namespace swa
