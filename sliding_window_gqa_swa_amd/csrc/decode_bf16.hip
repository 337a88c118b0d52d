// Single-token sliding-window GQA decode over the rolling buffer, bf16, gfx950.
//
// Mistral 7B (Chinese translation), section 2: tokens are generated one at a
// time (paragraph "Pre-fill and Chunking"); the keys/values of the last W
// positions sit in the W slots of the ring (paragraph "Rolling Buffer Cache");
// the query attends to those W positions (paragraph "Sliding Window
// Attention").  Section 1: with grouped-query attention the G query heads of
// a KV head read the same keys and values, which is what makes decoding
// cheaper in memory.
//
// After position pos has been written, slots [0, min(pos+1, W)) hold exactly
// positions max(0, pos-W+1) .. pos, so the query attends to every valid slot;
// softmax attention is a sum over keys and needs no slot -> position map.
//
// The library launches this kernel for G = 1 at head_dim 128 only; G = 2, 4,
// 8 (and head_dim 16 / 64 at any G) run on the matrix cores (decode_mfma.hip),
// because the per-head VALU work here grows with G.  The template still
// handles G <= 8, and the split merge (combine kernel) below serves both
// kernels' split plans at every head_dim (the matrix-core kernel's stream plan
// has its own merge, on the same merge_partials routine).
//
// Design (HBM-bound: 4 FLOP per byte of K/V):
//   * One workgroup = (sequence, KV head, split of the window): 4 waves.  All
//     G query heads are served from the same loaded K/V rows (GQA sharing).
//   * Loads: 8 lanes per 256-byte row, two 16-byte loads per lane (one per
//     128-byte half): each wave-wide load instruction reads whole cache lines
//     of 8 consecutive rows; a wave streams 32 rows (16 KiB of K+V) per step.
//   * Scores: v_dot2_f32_bf16 on packed pairs, then a 3-step DPP sum over the
//     8 lanes of a row; online softmax with one max per head per wave (shared
//     by all lanes), exp2 with the scale folded in.
//   * Merge: lane groups by DPP/permute sums, waves through LDS with a
//     log-sum-exp merge, splits through the workspace + a combine kernel.
#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerStep = 32;

template <int G>
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(DecodeParams p) {
  // A wave serves at most 4 query heads (registers: accumulators and query
  // slices grow with the heads).  With G = 8 the waves split into two head
  // groups of 4; both groups stream every row of the split (the second read of
  // a row is served by the caches).
  constexpr int GW = G < 4 ? G : 4;          // query heads per wave
  constexpr int NHG = G / GW;                // head groups
  constexpr int kRowWaves = kWaves / NHG;    // waves streaming the rows for one head group
  __shared__ float sm_acc[kRowWaves][G][kD];
  __shared__ float sm_m[kRowWaves][G];
  __shared__ float sm_l[kRowWaves][G];

  const int tid = thread_x(), lane = tid & 63, wave = tid >> 6;
  const int hg = wave % NHG, rw = wave / NHG;
  const int grp = lane >> 3, c = lane & 7;
  const int splits = p.splits;
  const int sp = wg_x() % splits;
  const int bg = wg_x() / splits;
  const int hkv = p.cache.n_kv_heads;
  const int g = bg % hkv, b = bg / hkv;
  const int W = p.cache.window;
  const int hq = p.n_q_heads;

  const int pos = p.seq.start_pos[b];
  const int n_valid = min(pos + 1, W);
  const int crow = p.seq.cache_idx ? p.seq.cache_idx[b] : b;
  const int len = seq_split_len(n_valid, splits, p.split_len);
  const int r_begin = sp * len;
  const int r_end = min(r_begin + len, n_valid);
  const float cs = p.scale_log2;

  const size_t ring0 = ((size_t)crow * hkv + g) * (size_t)W * kD;
  const uint16_t *kring = (const uint16_t *)p.cache.k + ring0;
  const uint16_t *vring = (const uint16_t *)p.cache.v + ring0;

  // Fused step: the new token (position pos) belongs in slot pos mod W.  The
  // workgroup whose split holds that slot reads the token's K/V from k_new /
  // v_new instead of the ring and also writes them there; no other workgroup
  // of this launch reads the slot, so the result is that of write-then-attend.
  const bool fused = p.k_new != nullptr;
  const int new_slot = fused ? pos % W : -1;
  const uint16_t *knew = fused ? (const uint16_t *)p.k_new + ((size_t)b * hkv + g) * kD : nullptr;
  const uint16_t *vnew = fused ? (const uint16_t *)p.v_new + ((size_t)b * hkv + g) * kD : nullptr;
  if (new_slot >= r_begin && new_slot < r_end && wave == 0 && lane < 32) {
    // 16 lanes copy the 256-byte K row, 16 lanes the V row
    const int ch = lane & 15;
    const uint16_t *src = lane < 16 ? knew : vnew;
    uint16_t *dst = (uint16_t *)(lane < 16 ? p.cache_k_out : p.cache_v_out) + ring0 + (size_t)new_slot * kD;
    *(u32x4 *)(dst + 8 * ch) = *(const u32x4 *)(src + 8 * ch);
  }

  // query slices of this wave's GW heads matching this lane's two 8-element chunks
  u32x4 qa[GW], qb[GW];
  const uint16_t *Q = (const uint16_t *)p.q;
#pragma unroll
  for (int hh = 0; hh < GW; hh++) {
    const uint16_t *qrow = Q + ((size_t)b * hq + g * G + hg * GW + hh) * kD;
    qa[hh] = *(const u32x4 *)(qrow + 8 * c);
    qb[hh] = *(const u32x4 *)(qrow + 64 + 8 * c);
  }

  float m[GW], l[GW], acc[GW][16];
#pragma unroll
  for (int hh = 0; hh < GW; hh++) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; e++) acc[hh][e] = 0.f;
  }

  for (int r0 = r_begin + kRowsPerStep * rw; r0 < r_end; r0 += kRowsPerStep * kRowWaves) {
    u32x4 ka[4], kb[4], va[4], vb[4];
    bool ok[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int r = r0 + 8 * k + grp;
      ok[k] = r < r_end;
      const u32x4 z = {0, 0, 0, 0};
      ka[k] = z; kb[k] = z; va[k] = z; vb[k] = z;
      if (ok[k]) {
        const bool is_new = r == new_slot;
        const uint16_t *kr = is_new ? knew : kring + (size_t)r * kD;
        const uint16_t *vr = is_new ? vnew : vring + (size_t)r * kD;
        ka[k] = __builtin_nontemporal_load((const u32x4 *)(kr + 8 * c));
        kb[k] = __builtin_nontemporal_load((const u32x4 *)(kr + 64 + 8 * c));
        va[k] = __builtin_nontemporal_load((const u32x4 *)(vr + 8 * c));
        vb[k] = __builtin_nontemporal_load((const u32x4 *)(vr + 64 + 8 * c));
      }
    }
    float sc[GW][4];
#pragma unroll
    for (int k = 0; k < 4; k++)
#pragma unroll
      for (int hh = 0; hh < GW; hh++) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < 4; e++) d = fdot2_bf16(ka[k][e], qa[hh][e], d);
#pragma unroll
        for (int e = 0; e < 4; e++) d = fdot2_bf16(kb[k][e], qb[hh][e], d);
        d = sum8(d);
        sc[hh][k] = ok[k] ? d * cs : -INFINITY;
      }
    float pk[GW][4];
#pragma unroll
    for (int hh = 0; hh < GW; hh++) {
      float mb = fmaxf(fmaxf(sc[hh][0], sc[hh][1]), fmaxf(sc[hh][2], sc[hh][3]));
      mb = max_over_groups8(mb);  // row r0 is valid, so mb is finite
      const float mn = fmaxf(m[hh], mb);
      if (mn > m[hh]) {
        const float alpha = exp2f(m[hh] - mn);  // 0 on the first step
        l[hh] *= alpha;
#pragma unroll
        for (int e = 0; e < 16; e++) acc[hh][e] *= alpha;
        m[hh] = mn;
      }
#pragma unroll
      for (int k = 0; k < 4; k++) {
        pk[hh][k] = exp2f(sc[hh][k] - mn);
        l[hh] += pk[hh][k];
      }
    }
#pragma unroll
    for (int k = 0; k < 4; k++) {
      float vf[16];
#pragma unroll
      for (int e = 0; e < 4; e++) {
        vf[2 * e] = bf16lo(va[k][e]);
        vf[2 * e + 1] = bf16hi(va[k][e]);
        vf[8 + 2 * e] = bf16lo(vb[k][e]);
        vf[8 + 2 * e + 1] = bf16hi(vb[k][e]);
      }
#pragma unroll
      for (int hh = 0; hh < GW; hh++)
#pragma unroll
        for (int e = 0; e < 16; e++) acc[hh][e] = __builtin_fmaf(pk[hh][k], vf[e], acc[hh][e]);
    }
  }

  // combine the 8 lane groups of the wave (they share m), then the waves
#pragma unroll
  for (int hh = 0; hh < GW; hh++) {
    l[hh] = sum_over_groups8(l[hh]);
#pragma unroll
    for (int e = 0; e < 16; e++) acc[hh][e] = sum_over_groups8(acc[hh][e]);
  }
  if (grp == 0) {
#pragma unroll
    for (int hh = 0; hh < GW; hh++) {
      const int hw = hg * GW + hh;  // head index within the group of G
#pragma unroll
      for (int e = 0; e < 8; e++) {
        sm_acc[rw][hw][8 * c + e] = acc[hh][e];
        sm_acc[rw][hw][64 + 8 * c + e] = acc[hh][8 + e];
      }
      if (c == 0) {
        sm_m[rw][hw] = m[hh];
        sm_l[rw][hw] = l[hh];
      }
    }
  }
  __syncthreads();

  for (int idx = tid; idx < G * kD; idx += kThreads) {
    const int hh = idx / kD, d = idx % kD;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kRowWaves; w++) mx = fmaxf(mx, sm_m[w][hh]);
    float ls = 0.f, os = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kRowWaves; w++) {
        const float f = exp2f(sm_m[w][hh] - mx);
        ls += sm_l[w][hh] * f;
        os += sm_acc[w][hh][d] * f;
      }
    }
    const int h = g * G + hh;
    if (splits == 1) {
      ((uint16_t *)p.out)[((size_t)b * hq + h) * kD + d] = (uint16_t)pack_bf16(os / ls, 0.f);
    } else {
      const size_t slot = ((size_t)b * hq + h) * splits + sp;
      p.ws_acc[slot * kD + d] = os;
      if (d == 0) {
        p.ws_ml[slot * 2] = mx;
        p.ws_ml[slot * 2 + 1] = ls;
      }
    }
  }
}

// Merge the per-split partials of each (sequence, query head), in split
// order (merge_partials).  One thread per output element, 64 ceil(head_dim /
// 64) threads so that the waves are whole; threads past head_dim repeat the
// last column and store nothing.
__global__ __launch_bounds__(kD) void decode_combine_bf16_kernel(DecodeParams p) {
  const int bh = wg_x(), d = thread_x();
  const int D = p.cache.head_dim;
  const int S = p.splits;
  const int dd = min(d, D - 1);
  const float *ml = p.ws_ml + (size_t)bh * S * 2;
  const float *acc = p.ws_acc + (size_t)bh * S * D + dd;
  const float o = merge_partials(
      S, d & 63, [&](int j) { return ml + 2 * j; }, [&](int j) { return acc + (size_t)j * D; });
  if (d < D) ((uint16_t *)p.out)[(size_t)bh * D + d] = (uint16_t)pack_bf16(o, 0.f);
}

template <int G>
hipError_t launch_g(const DecodeParams &p, hipStream_t stream) {
  const unsigned n_wg = (unsigned)p.seq.num_seqs * p.cache.n_kv_heads * p.splits;
  hipLaunchKernelGGL(decode_bf16_kernel<G>, dim3(n_wg), dim3(kThreads), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine_bf16(p, stream);
}

}  // namespace

hipError_t launch_decode_combine_bf16(const DecodeParams &p, hipStream_t stream) {
  if (p.seq.num_seqs == 0 || p.splits == 1) return hipSuccess;
  hipLaunchKernelGGL(decode_combine_bf16_kernel, dim3((unsigned)p.seq.num_seqs * p.n_q_heads),
                     dim3((unsigned)(64 * ((p.cache.head_dim + 63) / 64))), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeParams &p, int group, hipStream_t stream) {
  if (p.seq.num_seqs == 0) return hipSuccess;
  if (group != 1 || p.cache.head_dim != kD) return hipErrorInvalidValue;
  return launch_g<1>(p, stream);
}

}  // namespace swa
