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
//   * One workgroup = (sequence, KV head, split of the window), 4 waves; a
//     wave takes 32-key steps r0 = split start + 32 w + 128 j.
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
//   * Waves merge through LDS (log-sum-exp), splits through the workspace and
//     the combine kernel of decode_bf16.hip.
#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
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

template <int G, int D>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(DecodeParams p) {
  using Rg = RowGeo<D>;
  constexpr int kD = D, kRowB = Rg::kRowB, kVBufB = Rg::kVBufB, kC = Rg::kC, kRpl = Rg::kRpl;
  constexpr int kKS = Rg::kKS, kDB = Rg::kDB;
  // two V buffers per wave, as two objects; after the loop vbuf_a holds the merge
  __shared__ __attribute__((aligned(16))) unsigned char vbuf_a[kWaves][kVBufB];
  __shared__ __attribute__((aligned(16))) unsigned char vbuf_b[kWaves][kVBufB];
  static_assert(kWaves * G * (kD + 2) * 4 <= kWaves * kVBufB, "the wave merge fits in vbuf_a");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, lg = lane >> 4;  // MFMA column (query head) and lane group
  const int splits = p.splits;
  const int sp = blockIdx.x % splits;
  const int bg = blockIdx.x / splits;
  const int hkv = p.cache.n_kv_heads;
  const int g = bg % hkv, b = bg / hkv;
  const int W = p.cache.window;
  const int hq = p.n_q_heads;

  const int pos = __builtin_amdgcn_readfirstlane(p.seq.start_pos[b]);
  const int n_valid = min(pos + 1, W);
  const int crow = p.seq.cache_idx ? __builtin_amdgcn_readfirstlane(p.seq.cache_idx[b]) : b;
  // uniform by construction; readfirstlane lets the compiler branch on them with scalar branches
  const int len = __builtin_amdgcn_readfirstlane(seq_split_len(n_valid, splits, p.split_len));
  const int r_begin = __builtin_amdgcn_readfirstlane(sp * len);
  const int r_end = __builtin_amdgcn_readfirstlane(min(r_begin + len, n_valid));
  const float c = p.scale_log2;

  const size_t ring0 = ((size_t)crow * hkv + g) * (size_t)W * kD;
  const uint16_t *kring = (const uint16_t *)p.cache.k + ring0;
  const uint16_t *vring = (const uint16_t *)p.cache.v + ring0;

  // fused step: the new token's row comes from k_new / v_new and is written to
  // its slot by the workgroup whose split holds it (nobody else reads the slot)
  const bool fused = p.k_new != nullptr;
  const int new_slot = fused ? pos % W : -1;
  const uint16_t *knew = fused ? (const uint16_t *)p.k_new + ((size_t)b * hkv + g) * kD : nullptr;
  const uint16_t *vnew = fused ? (const uint16_t *)p.v_new + ((size_t)b * hkv + g) * kD : nullptr;
  if (new_slot >= r_begin && new_slot < r_end && wave == 0 && lane < 2 * kC) {
    // kC lanes copy the K row, kC lanes the V row, 16 bytes each
    const int ch = lane % kC;
    const uint16_t *src = lane < kC ? knew : vnew;
    uint16_t *dst = (uint16_t *)(lane < kC ? p.cache_k_out : p.cache_v_out) + ring0 + (size_t)new_slot * kD;
    *(u32x4 *)(dst + 8 * ch) = *(const u32x4 *)(src + 8 * ch);
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

template <int G, int D>
hipError_t launch_gd(const DecodeParams &p, hipStream_t stream) {
  const unsigned n_wg = (unsigned)p.seq.num_seqs * p.cache.n_kv_heads * p.splits;
  hipLaunchKernelGGL((decode_mfma_kernel<G, D>), dim3(n_wg), dim3(kThreads), 0, stream, p);
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
