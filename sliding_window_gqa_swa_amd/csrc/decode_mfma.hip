// Single-token sliding-window GQA decode on the matrix cores, bf16, gfx950
// (G = 2, 4, 8 query heads per KV head at head_dim 128; every G at head_dim
// 16 and 64).
//
// Same operation as decode_bf16.hip (Mistral 7B (Chinese translation),
// section 2, paragraphs "Rolling Buffer Cache" and "Pre-fill and Chunking";
// section 1 for GQA): each query attends to the min(pos+1, W) valid slots of
// its ring; with the fused step the new token's K/V come from k_new / v_new
// and are written to slot pos mod W by the workgroup whose split holds it.
//
// With G query heads per KV head the per-row work is a small matrix product,
// so it runs on v_mfma_f32_16x16x32_bf16 (the G heads padded to 16 columns)
// instead of per-head VALU dot products, which cost more per byte as G grows:
//   * Split mode: one workgroup = (sequence, KV head, split of the window),
//     4 waves (16 at head_dim 16); a wave takes 32-key steps
//     r0 = split start + 32 w + 32 kWaves j.
//   * Stream mode (batches too small to fill the chip with whole windows):
//     the valid slots of all (sequence, KV head) pairs are laid end to end and
//     cut into equal ranges, one per workgroup, which attends to its range one
//     pair piece at a time, so that short and long contexts in one batch cost
//     the same per slot.  Pieces that are parts of pairs leave partial results
//     (at most two per workgroup) for a merge launch.
//   * S^T (keys x heads) = K Q^T: the K rows are loaded from HBM straight into
//     the MFMA A-operand layout (lane -> row lane % 16, 8 consecutive d);
//     Q^T is the B operand, loaded once.
//   * O^T (d x heads) += V^T P^T: the V rows go to a per-wave LDS buffer with
//     global_load_lds (XOR-swizzled 16-byte chunks) and come back transposed
//     with ds_read_b64_tr_b16; P^T stays in registers (the S^T accumulator
//     layout is the B-operand layout).
//   * Two K register sets and two V buffers: once a step has its scores, the
//     next step's K (registers) and V (the other LDS buffer) are issued and
//     stay in flight through this step's softmax and P V.  The two V buffers
//     are distinct LDS objects and the loop is unrolled by two, so the
//     compiler can tell a buffer being filled from the one being read and
//     does not wait for the prefetch before reading.
//   * Keys past the split (a partial last step) read the split's last valid
//     row and are masked to -inf: unwritten slots are never read.
//   * Waves merge through LDS (log-sum-exp); splits through the workspace and
//     the combine kernel of decode_bf16.hip, stream pieces through the
//     workspace and the stream combine kernel below.
#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kStep = 32;                  // keys per wave step
constexpr float kRescaleSlack = 8.0f;      // log2 units, as in the prefill
constexpr uint32_t kBf16OnePair = 0x3F803F80u;
constexpr int kNonTemporal = 2;  // cache-policy bit "nt" of a global_load_lds (K rows use nontemporal loads too)

typedef __attribute__((address_space(3))) void lds_void;

// Waits, each fenced so that the scheduler moves no instruction across it:
// vmcnt(0) ends the outstanding loads (registers and LDS), lgkmcnt(0) the
// outstanding LDS reads.
__device__ __forceinline__ void wait_vm0() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void wait_lds_reads() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row geometry for head_dim D (128, 64 or 16): a row is 2D bytes in kC
// chunks of 16 bytes; one global_load_lds moves 1 KiB = kRpl rows; the V rows
// are stored in 32-byte segments XOR-swizzled by vseg(row) (the prefill's V
// layout), so a transposed read of 8 consecutive rows hits 8 different bank
// groups.
template <int D>
struct RowGeo {
  // waves per workgroup: at head_dim 16 a row is 32 bytes, so more waves keep
  // enough bytes in flight (the kernel is small in registers and LDS there)
  static constexpr int kWaves = D == 16 ? 16 : 4;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRowB = 2 * D;
  static constexpr int kVBufB = kStep * kRowB;         // one wave step of V rows
  static constexpr int kC = D / 8;
  static constexpr int kRpl = 64 / kC;
  static constexpr int kVLoads = kStep / kRpl;         // 1 KiB loads per V step (8, 4, 1)
  static constexpr int kKS = D >= 32 ? D / 32 : 1;     // 32-deep steps of QK (D = 16: zero-padded)
  static constexpr int kDB = D / 16;
  static __device__ __forceinline__ int vseg(int row) {
    if constexpr (D == 128) return (row & 3) + 4 * ((row >> 2) & 1);
    else if constexpr (D == 64) return (row >> 1) & 3;
    else return 0;
  }
};

template <int D>
using VBuf = unsigned char[RowGeo<D>::kWaves][RowGeo<D>::kVBufB];

// Where the result of one attended range goes: the final bf16 rows of out
// (acc == nullptr), or partial results -- unnormalised output sums, running
// max in log2 units and weight sum -- of query head hh of the group at
// acc[(base + hh * stride) * D] and ml[(base + hh * stride) * 2].
struct RangeOut {
  float *acc;
  float *ml;
  size_t base;
  int stride;
};

// The G query heads of KV head g of sequence b (at position pos, cache row
// crow) attend to ring slots [r_begin, r_end), by the whole workgroup.  On
// return each wave is past its own LDS reads, but vbuf_a, which held the wave
// merge, may still be read by the others: a barrier comes before it is refilled.
template <int G, int D>
__device__ __forceinline__ void attend_range(const DecodeParams &p, VBuf<D> &vbuf_a, VBuf<D> &vbuf_b, int b, int g,
                                             int pos, int crow, int r_begin, int r_end, RangeOut dst) {
  using Rg = RowGeo<D>;
  constexpr int kD = D, kRowB = Rg::kRowB, kVBufB = Rg::kVBufB, kC = Rg::kC, kRpl = Rg::kRpl;
  constexpr int kKS = Rg::kKS, kDB = Rg::kDB;
  constexpr int kWaves = Rg::kWaves, kThreads = Rg::kThreads;
  static_assert(kWaves * G * (kD + 2) * 4 <= kWaves * kVBufB, "the wave merge fits in vbuf_a");

  const int tid = thread_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, lg = lane >> 4;  // MFMA column (query head) and lane group
  const int hkv = p.cache.n_kv_heads;
  const int W = p.cache.window;
  const int hq = p.n_q_heads;
  const float c = p.scale_log2;

  const size_t ring0 = ((size_t)crow * hkv + g) * (size_t)W * kD;
  const uint16_t *kring = (const uint16_t *)p.cache.k + ring0;
  const uint16_t *vring = (const uint16_t *)p.cache.v + ring0;

  // fused step: the new token's row comes from k_new / v_new and is written to
  // its slot by the workgroup whose range holds it (nobody else reads the slot)
  const bool fused = p.k_new != nullptr;
  const int new_slot = fused ? pos % W : -1;
  const uint16_t *knew = fused ? (const uint16_t *)p.k_new + ((size_t)b * hkv + g) * kD : nullptr;
  const uint16_t *vnew = fused ? (const uint16_t *)p.v_new + ((size_t)b * hkv + g) * kD : nullptr;
  if (new_slot >= r_begin && new_slot < r_end && wave == 0 && lane < 2 * kC) {
    // kC lanes copy the K row, kC lanes the V row, 16 bytes each
    const int ch = lane % kC;
    const uint16_t *src = lane < kC ? knew : vnew;
    uint16_t *row = (uint16_t *)(lane < kC ? p.cache_k_out : p.cache_v_out) + ring0 + (size_t)new_slot * kD;
    *(u32x4 *)(row + 8 * ch) = *(const u32x4 *)(src + 8 * ch);
  }

  bf16x8 qf[kKS];  // Q^T as the B operand, loaded after the first K/V loads are issued

  // LDS offsets of the transposed V reads (the prefill's mapping for one
  // 32-key slice): rows 4 lg + (col / 4) and +16, 8 bytes at segment-swizzled
  // columns of d-block db
  int v_off[kDB];
  {
    const int vr = 4 * lg + (col >> 2);
    const int vb = vr * kRowB + 8 * (lane & 3);
#pragma unroll
    for (int db = 0; db < kDB; db++) v_off[db] = vb + 32 * (db ^ Rg::vseg(vr));
  }
  // global_load_lds of a V step: load i covers rows kRpl i .. kRpl (i + 1) - 1;
  // lane -> row kRpl i + lane / kC, LDS chunk lane % kC, holding logical chunk
  // (lane % kC) ^ 2 vseg(row).  vseg of those rows depends on i only through
  // its parity (D = 128: rows 4 i + lane / 16), so two values per lane suffice.
  const int vchunk_even = (lane % kC) ^ (2 * Rg::vseg(lane / kC));
  const int vchunk_odd = (lane % kC) ^ (2 * Rg::vseg(kRpl + lane / kC));

  f32x4 o[kDB];
#pragma unroll
  for (int db = 0; db < kDB; db++) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;  // running max of this lane's column, log2 units
  float l = 0.f;        // this lane's share of the column's sum

  // issue the loads of the step at r0: K rows into kf, V rows into vb (LDS).
  // (D = 16: lanes 32-63 load the row's two chunks again; their Q is zero)
  auto issue = [&](int r0, bf16x8 (&kf)[2][kKS], unsigned char *vb) __attribute__((always_inline)) {
    const int last = r_end - 1;
#pragma unroll
    for (int kbi = 0; kbi < 2; kbi++) {
      const int r = min(r0 + 16 * kbi + col, last);
      const uint16_t *kr = r == new_slot ? knew : kring + (size_t)r * kD;
#pragma unroll
      for (int ks = 0; ks < kKS; ks++)
        kf[kbi][ks] = __builtin_nontemporal_load((const bf16x8 *)(kr + 32 * ks + 8 * (lg & (kC - 1))));
    }
#pragma unroll
    for (int i = 0; i < Rg::kVLoads; i++) {
      const int r = min(r0 + kRpl * i + lane / kC, last);
      const uint16_t *vr = r == new_slot ? vnew : vring + (size_t)r * kD;
      const int ch = (i & 1) ? vchunk_odd : vchunk_even;
      __builtin_amdgcn_global_load_lds(vr + 8 * ch, (lds_void *)(vb + i * 1024), 16, 0, kNonTemporal);
    }
  };

  // S^T of a step: keys 16 kbi + 4 lg + i of the step in sa[kbi][i], column = head
  auto scores = [&](const bf16x8 (&kf)[2][kKS], f32x4 (&sa)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kbi = 0; kbi < 2; kbi++) {
      sa[kbi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < kKS; ks++) sa[kbi] = mfma16(kf[kbi][ks], qf[ks], sa[kbi]);
    }
  };

  // the rest of a step: online softmax of every column, O^T += V^T P^T
  auto softmax_pv = [&](int r0, f32x4 (&sa)[2], const unsigned char *vb) __attribute__((always_inline)) {
    // keys past the split are masked (their rows repeat a valid one)
    const int k0 = r0 + 4 * lg;
#pragma unroll
    for (int kbi = 0; kbi < 2; kbi++)
#pragma unroll
      for (int i = 0; i < 4; i++)
        if (k0 + 16 * kbi + i >= r_end) sa[kbi][i] = -INFINITY;
    float mt = fmaxf(fmaxf(fmaxf(sa[0][0], sa[0][1]), fmaxf(sa[0][2], sa[0][3])),
                     fmaxf(fmaxf(sa[1][0], sa[1][1]), fmaxf(sa[1][2], sa[1][3])));
    mt = max_pair32(max_pair16(mt));  // key r0 is valid: finite
    const float mts = mt * c;
    const bool upd = mts > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(upd)) {
      const float mn = upd ? mts : m;
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < kDB; db++) o[db] *= alpha;
    }
#pragma unroll
    for (int kbi = 0; kbi < 2; kbi++)
#pragma unroll
      for (int i = 0; i < 4; i++) sa[kbi][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[kbi][i], c, -m));
    u32x4 w;
    w[0] = pack_bf16(sa[0][0], sa[0][1]);
    w[1] = pack_bf16(sa[0][2], sa[0][3]);
    w[2] = pack_bf16(sa[1][0], sa[1][1]);
    w[3] = pack_bf16(sa[1][2], sa[1][3]);
#pragma unroll
    for (int e = 0; e < 4; e++) l = fdot2_bf16(w[e], kBf16OnePair, l);  // sum of what enters P V
    const bf16x8 pf = __builtin_bit_cast(bf16x8, w);
#pragma unroll
    for (int db = 0; db < kDB; db++) {
      const unsigned char *va = vb + v_off[db];
      const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)va);
      const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(va + 16 * kRowB));
      u32x4 vv;
      vv[0] = __builtin_bit_cast(u32x2, v1)[0];
      vv[1] = __builtin_bit_cast(u32x2, v1)[1];
      vv[2] = __builtin_bit_cast(u32x2, v2)[0];
      vv[3] = __builtin_bit_cast(u32x2, v2)[1];
      o[db] = mfma16(__builtin_bit_cast(bf16x8, vv), pf, o[db]);
    }
  };

  // this wave's n steps r0, r0 + stride, ..., two per iteration (buffers a, b).
  // A step waits for its own loads, computes its scores, then issues the next
  // step's loads (into the K registers it has just consumed and the other V
  // buffer), so they are in flight during this step's softmax and P V.
  const int stride = kStep * kWaves;
  int r0 = r_begin + kStep * wave;
  const int n = r0 < r_end ? (r_end - r0 + stride - 1) / stride : 0;
  bf16x8 ka[2][kKS], kb[2][kKS];
  unsigned char *va = vbuf_a[wave], *vbb = vbuf_b[wave];
  if (n > 0) issue(r0, ka, va);
  // Q^T: lane -> head `col` (zero when col >= G), d-group lg (zero for lg >= 2 when D = 16)
  {
    const bool ok = col < G && (kD >= 32 || lg < 2);
    const uint16_t *qrow = (const uint16_t *)p.q + ((size_t)b * hq + g * G + (ok ? col : 0)) * kD + 8 * (lg & (kC - 1));
#pragma unroll
    for (int ks = 0; ks < kKS; ks++) {
      u32x4 v = {0, 0, 0, 0};
      if (ok) v = *(const u32x4 *)(qrow + 32 * ks);
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  for (int s = 0; s < n; s += 2) {
    f32x4 sa[2];
    wait_vm0();
    scores(ka, sa);
    if (s + 1 < n) {
      wait_lds_reads();  // the last step's reads of vbb are done before it is refilled
      issue(r0 + stride, kb, vbb);
    }
    softmax_pv(r0, sa, va);
    r0 += stride;
    if (s + 1 >= n) break;
    wait_vm0();
    scores(kb, sa);
    if (s + 2 < n) {
      wait_lds_reads();
      issue(r0 + stride, ka, va);
    }
    softmax_pv(r0, sa, vbb);
    r0 += stride;
  }

  // merge the waves: each writes its columns' partials, vbuf_a becomes the
  // merge area (every wave is past its last LDS read after the barrier)
  l = add_pair32(add_pair16(l));
  __syncthreads();
  float *sm_acc = (float *)&vbuf_a[0][0];          // [kWaves][G][kD]
  float *sm_ml = sm_acc + kWaves * G * kD;          // [kWaves][G][2]
  if (col < G) {
#pragma unroll
    for (int db = 0; db < kDB; db++)
#pragma unroll
      for (int i = 0; i < 4; i++) sm_acc[(wave * G + col) * kD + 16 * db + 4 * lg + i] = o[db][i];
    if (lg == 0) {
      sm_ml[(wave * G + col) * 2] = m;
      sm_ml[(wave * G + col) * 2 + 1] = l;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * kD; idx += kThreads) {
    const int hh = idx / kD, d = idx % kD;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; w++) mx = fmaxf(mx, sm_ml[(w * G + hh) * 2]);
    float ls = 0.f, os = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; w++) {
        const float mw = sm_ml[(w * G + hh) * 2];
        if (mw == -INFINITY) continue;  // a wave without keys
        const float f = __builtin_amdgcn_exp2f(mw - mx);
        ls += sm_ml[(w * G + hh) * 2 + 1] * f;
        os += sm_acc[(w * G + hh) * kD + d] * f;
      }
    }
    if (dst.acc == nullptr) {
      ((uint16_t *)p.out)[((size_t)b * hq + g * G + hh) * kD + d] = (uint16_t)pack_bf16(os / ls, 0.f);
    } else {
      const size_t slot = dst.base + (size_t)hh * dst.stride;
      dst.acc[slot * kD + d] = os;
      if (d == 0) {
        dst.ml[slot * 2] = mx;
        dst.ml[slot * 2 + 1] = ls;
      }
    }
  }
}

template <int G, int D, bool kStream>
__global__ __launch_bounds__(RowGeo<D>::kThreads) void decode_mfma_kernel(DecodeParams p) {
  // two V buffers per wave, as two objects; after a range vbuf_a holds the merge
  __shared__ __attribute__((aligned(16))) unsigned char vbuf_a[RowGeo<D>::kWaves][RowGeo<D>::kVBufB];
  __shared__ __attribute__((aligned(16))) unsigned char vbuf_b[RowGeo<D>::kWaves][RowGeo<D>::kVBufB];
  const int hkv = p.cache.n_kv_heads;
  const int W = p.cache.window;
  if constexpr (!kStream) {
    // split mode: one workgroup = (sequence, KV head, split of the window)
    const int splits = p.splits;
    const int sp = wg_x() % splits;
    const int bg = wg_x() / splits;
    const int g = bg % hkv, b = bg / hkv;
    // both per-sequence loads issued together (no branch on cache_idx between them)
    const int32_t *ci = p.seq.cache_idx ? p.seq.cache_idx : p.seq.start_pos;
    const int pos = __builtin_amdgcn_readfirstlane(p.seq.start_pos[b]);
    const int ci_b = __builtin_amdgcn_readfirstlane(ci[b]);
    const int crow = p.seq.cache_idx ? ci_b : b;
    const int n_valid = min(pos + 1, W);
    // uniform by construction; readfirstlane lets the compiler branch on them with scalar branches
    const int len = __builtin_amdgcn_readfirstlane(seq_split_len(n_valid, splits, p.split_len));
    const int r_begin = __builtin_amdgcn_readfirstlane(sp * len);
    const int r_end = __builtin_amdgcn_readfirstlane(min(r_begin + len, n_valid));
    RangeOut dst{nullptr, nullptr, 0, 0};
    if (splits > 1) dst = RangeOut{p.ws_acc, p.ws_ml, ((size_t)b * p.n_q_heads + g * G) * splits + sp, splits};
    attend_range<G, D>(p, vbuf_a, vbuf_b, b, g, pos, crow, r_begin, r_end, dst);
  } else {
    // stream mode: the valid slots of the pairs (b, g), laid end to end
    // sequence-major -- pair (b, g) holds rows hkv S(b) + g nv(b) .. + nv(b) - 1,
    // with nv(b) its valid slots and S(b) those of the sequences before b --
    // are cut into ranges of L rows; this workgroup attends to range wg_x(),
    // piece by piece (one piece per pair it meets).  A piece that is a whole
    // pair gives final rows; the first and the last piece may be parts of pairs
    // and go to the workgroup's partial slots 0 and 1.  Every wave computes
    // the same plan from the batch (2 to 64 sequences, one per lane).
    const int lane = thread_x() & 63;
    const int ns = p.seq.num_seqs;
    const int32_t *ci = p.seq.cache_idx ? p.seq.cache_idx : p.seq.start_pos;  // both loads issued together
    const int pos_l = lane < ns ? p.seq.start_pos[lane] : 0;
    const int ci_l = lane < ns ? ci[lane] : 0;
    const int crow_l = p.seq.cache_idx ? ci_l : lane;
    const int nv_l = lane < ns ? max(0, min(pos_l + 1, W)) : 0;
    const int incl = wave_incl_scan_i32(nv_l);  // inclusive prefix sum over the sequences
    const int total = hkv * __builtin_amdgcn_readlane(incl, 63);
    const int L = stream_range_rows(total, p.stream_wg);
    const int R0 = wg_x() * L;
    if (R0 >= total) return;
    const int R1 = min(R0 + L, total);
    // the first sequence whose pairs reach past R0 (lanes past the batch hold
    // the total, so a lane below ns is found first)
    int b = __builtin_ffsll((long long)__builtin_amdgcn_ballot_w64(hkv * incl > R0)) - 1;
    int nvb = __builtin_amdgcn_readlane(nv_l, b);
    const int off = R0 - hkv * (__builtin_amdgcn_readlane(incl, b) - nvb);  // 0 <= off < hkv nvb
    if (off < 0 || off >= hkv * nvb) return;  // cannot happen with a monotone prefix; no ring access outside it
    int g = off / nvb;
    int r_begin = off - g * nvb;
    int cur = R0;
    for (;;) {
      const int r_end = min(nvb, r_begin + (R1 - cur));
      RangeOut dst{nullptr, nullptr, 0, 0};
      if (r_begin > 0 || r_end < nvb)
        dst = RangeOut{p.ws_acc, p.ws_ml, ((size_t)wg_x() * 2 + (cur == R0 ? 0 : 1)) * G, 1};
      attend_range<G, D>(p, vbuf_a, vbuf_b, b, g, __builtin_amdgcn_readlane(pos_l, b),
                         __builtin_amdgcn_readlane(crow_l, b), r_begin, r_end, dst);
      cur += r_end - r_begin;
      if (cur >= R1) break;
      r_begin = 0;
      if (++g == hkv) {
        g = 0;
        if (++b >= ns) break;
        nvb = __builtin_amdgcn_readlane(nv_l, b);
      }
      __syncthreads();  // vbuf_a held the wave merge
    }
  }
}

// Stream mode: merge the partial results of each (sequence, query head) whose
// pair of slots spans several workgroups' ranges; pairs inside one range
// already have their rows.  Each wave recomputes the decode kernel's plan from
// the batch (lane i holds sequence i; the same prefix sum).  The partials come from workgroups
// w0 .. w1 (slot 1 of w0 when the pair starts inside w0's range, else slot 0)
// and are merged as in the split merge (decode_bf16.hip).  One thread per
// output element; 64 ceil(D / 64) threads, so that every wave is whole for
// the sums over the batch and the partials.
__global__ __launch_bounds__(128) void decode_combine_stream_kernel(DecodeParams p) {
  const int bh = wg_x(), d = thread_x(), lane = d & 63;
  const int D = p.cache.head_dim, W = p.cache.window;
  const int hq = p.n_q_heads, hkv = p.cache.n_kv_heads, G = hq / hkv;
  const int b = bh / hq, h = bh % hq, g = h / G, hh = h % G;
  const int ns = p.seq.num_seqs;
  const int nv = lane < ns ? max(0, min(p.seq.start_pos[lane] + 1, W)) : 0;
  const int incl = wave_incl_scan_i32(nv);
  const int total = hkv * __builtin_amdgcn_readlane(incl, 63);
  const int nvb = __builtin_amdgcn_readlane(nv, b);
  const int before = __builtin_amdgcn_readlane(incl, b) - nvb;
  if (nvb == 0) return;
  const int dd = min(d, D - 1);  // threads past D repeat the last column and store nothing
  const int L = stream_range_rows(total, p.stream_wg);
  const int P = hkv * before + g * nvb;
  const int w0 = P / L, w1 = (P + nvb - 1) / L;
  if (w0 == w1 || P < 0 || w1 >= p.stream_wg) return;  // (the last two cannot happen: slots in range)
  const int s0 = P == w0 * L ? 0 : 1;
  // partial j comes from workgroup w0 + j
  auto slot_of = [&](int j) { return ((size_t)(w0 + j) * 2 + (j == 0 ? s0 : 0)) * G + hh; };
  const float o = merge_partials(
      w1 - w0 + 1, lane, [&](int j) { return p.ws_ml + slot_of(j) * 2; },
      [&](int j) { return p.ws_acc + slot_of(j) * D + dd; });
  if (d < D) ((uint16_t *)p.out)[(size_t)bh * D + d] = (uint16_t)pack_bf16(o, 0.f);
}

template <int G, int D>
hipError_t launch_gd(const DecodeParams &p, hipStream_t stream) {
  if (p.stream_wg > 0) {
    if (p.seq.num_seqs > kStreamMaxSeqs) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_mfma_kernel<G, D, true>), dim3((unsigned)p.stream_wg), dim3(RowGeo<D>::kThreads), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_stream_kernel, dim3((unsigned)p.seq.num_seqs * p.n_q_heads),
                       dim3((unsigned)(64 * ((D + 63) / 64))), 0, stream, p);
    return hipGetLastError();
  }
  const unsigned n_wg = (unsigned)p.seq.num_seqs * p.cache.n_kv_heads * p.splits;
  hipLaunchKernelGGL((decode_mfma_kernel<G, D, false>), dim3(n_wg), dim3(RowGeo<D>::kThreads), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_combine_bf16(p, stream);
}

template <int D>
hipError_t launch_d(const DecodeParams &p, int group, hipStream_t stream) {
  switch (group) {
    case 1:
      if constexpr (D != 128) return launch_gd<1, D>(p, stream);  // D = 128, G = 1: the VALU kernel
      return hipErrorInvalidValue;
    case 2: return launch_gd<2, D>(p, stream);
    case 4: return launch_gd<4, D>(p, stream);
    case 8: return launch_gd<8, D>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_mfma_bf16(const DecodeParams &p, int group, hipStream_t stream) {
  if (p.seq.num_seqs == 0) return hipSuccess;
  switch (p.cache.head_dim) {
    case 128: return launch_d<128>(p, group, stream);
    case 64: return launch_d<64>(p, group, stream);
    case 16: return launch_d<16>(p, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swa
