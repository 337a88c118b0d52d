// Chunked sliding-window GQA prefill, bf16 in / bf16 out, fp32 accumulation, gfx950.
//
// What it computes (Mistral 7B (Chinese translation), section 2):
//   paragraph "Sliding Window Attention" / Figure 1 caption -- the query at
//   absolute position i attends to keys j with i-W < j <= i;
//   paragraph "Pre-fill and Chunking" / Figure 3 caption -- a chunk attends
//   causally to itself and through the window to the cache; keys j below the
//   chunk start come from ring slot j mod W (paragraph "Rolling Buffer Cache"),
//   keys inside the chunk from the chunk's own k_new / v_new;
//   section 1 -- grouped-query attention: the G query heads of KV head g share
//   its keys and values.
//
// Design (MI355X / CDNA4):
//   * One workgroup = (sequence, KV head g, BQ = 256/G query positions) x the G
//     query heads of g = 256 query rows in 8 waves of 32 rows.  Every K/V tile
//     (64 keys) is staged ONCE in LDS and consumed by all G heads.
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16.  The S^T
//     accumulator layout (lane = query, registers = keys) is reused directly
//     as the B operand of the PV product, so P never leaves registers; V^T is
//     read with ds_read_b64_tr_b16 (4-key transposed loads).
//   * Ping-pong: waves w and w+4 share a SIMD and belong to different groups
//     (A = waves 0-3, B = waves 4-7).  Each tile is a softmax half-step (VALU)
//     and a matrix half-step (PV of this tile + QK of the next, MFMA + LDS
//     reads); group B runs one half-step behind A, so on every SIMD one wave
//     issues MFMAs while the other runs the softmax.
//   * Tiles go straight from global memory into LDS (global_load_lds, 16 bytes
//     per lane): group A streams the K tiles (3 LDS slots), group B the V
//     tiles (2 slots); no staging registers.  LDS rows are 2 head_dim bytes
//     (256 B at head_dim 128) with XOR swizzles of the 16-byte chunks: at
//     head_dim 128, K chunk ^ (row % 16) (the 16-byte K reads of 16 rows hit
//     16 different chunks), V chunk ^ (2 (row % 4) + 8 ((row / 4) % 2)): a
//     transposed read of 32 lanes covers rows 8k..8k+7, 32 B each, and these
//     land in 8 different 32-byte segments, i.e. all 64 banks once (Geo<D>
//     holds the same rules for head_dim 64 and 16).
//   * head_dim 16 runs the 32-deep QK step with zero-padded Q (lanes 32-63).
//   * Only tiles intersecting the workgroup's band [q0-W+1, q_last] are
//     visited; only tiles crossing a row's window edge or the diagonal run the
//     mask code.  Keys outside the band are never read from outside it: their
//     rows are loaded from the nearest key of the band (always written data)
//     and masked, so unwritten cache slots cannot reach the arithmetic.
//   * The matrix half-step is an explicit pipeline over operand fragments
//     (the next tile's K fragments, then this tile's V fragments): each is
//     read from LDS three fragments before the two MFMAs that use it, and
//     every step of the pipeline is pinned in place.
//   * Online softmax in fp32 with exp2.  The softmax half-step competes with
//     the other wave's MFMAs for the VALU issue port; it is kept small:
//       - the score accumulators start at -M (the running max of q.k), so
//         a weight is exp2(c * accumulator), one multiply per score;
//       - the row sums are an MFMA of the bf16 weights with a ones operand,
//         which also leaves every lane with its query's complete sum;
//       - the rescale test is one compare of each lane's tile max against
//         the row's threshold; the cross-lane row max is only formed on the
//         rare tiles that rescale;
//       - the unmasked interior loop is unrolled by 6 (3 K slots x 2 V slots),
//         so LDS slot addresses are immediate offsets.
//   * Epilogue: each wave stages its normalised bf16 rows in LDS and writes
//     them as whole rows with non-temporal 16-byte stores.
//   * Work order (KV head, sequence, query tile from the last), dealt to the
//     XCDs in contiguous ranges: one KV head per XCD balances ragged batches
//     and keeps each head's K/V in one L2.
#include "device_common.h"
#include "swa_internal.h"

#include <type_traits>

namespace swa {
namespace {

constexpr int kBN = 64;                       // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr float kRescaleSlack = 8.0f;         // log2 units: weights stay <= 256
constexpr uint32_t kBf16OnePair = 0x3F803F80u;

// Tile geometry for head_dim D (128, 64 or 16).  An LDS row holds one key (or
// value) row of 2D bytes in 16-byte chunks; a tile is kBN rows.  One
// global_load_lds instruction moves 1 KiB: kRpl rows of kC chunks.
template <int D>
struct Geo {
  static constexpr int kRowB = 2 * D;                  // bytes per LDS row
  static constexpr int kTileB = kBN * kRowB;           // 16 / 8 / 2 KiB
  static constexpr int kLdsBytes = 5 * kTileB;         // 3 K slots + 2 V slots
  static constexpr int kC = D / 8;                     // 16-byte chunks per row
  static constexpr int kRpl = 64 / kC;                 // rows per 1 KiB wave-load
  static constexpr int kNL = kBN / kRpl;               // wave-loads per tile
  static constexpr int kLoads = (kNL + 3) / 4;         // wave-loads per wave of a group
  static constexpr int kKS = D >= 32 ? D / 32 : 1;     // 32-deep steps of QK (D = 16: one, zero-padded)
  static constexpr int kDB = D / 16;                   // 16-column blocks of O
  // K rows: physical chunk = logical chunk ^ kswz(row).  The 16-byte operand
  // reads of 16 consecutive rows then cover all 64 banks once.
  static __device__ __forceinline__ int kswz(int row) { return (row / (16 / kC)) % kC; }
  // V rows, in 32-byte segments: physical segment = logical ^ vseg(row).  A
  // transposed read of 32 lanes covers 8 consecutive rows x 32 bytes of one
  // logical segment, and these land in 8 different 32-byte bank groups.
  static __device__ __forceinline__ int vseg(int row) {
    if constexpr (D == 128) return (row & 3) + 4 * ((row >> 2) & 1);
    else if constexpr (D == 64) return (row >> 1) & 3;
    else return 0;
  }
};

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Wait for this wave's outstanding global loads (including those that write
// LDS directly); expcnt and lgkmcnt are left unconstrained.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int G, int D>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillParams p) {
  using Gm = Geo<D>;
  constexpr int kRowB = Gm::kRowB, kTileB = Gm::kTileB, kC = Gm::kC, kRpl = Gm::kRpl;
  constexpr int kKS = Gm::kKS, kDB = Gm::kDB;
  constexpr int kWph = kWaves / G;  // waves per query head
  constexpr int kBQ = 32 * kWph;    // query positions per workgroup
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = thread_x(), lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave choices scalar
  // Work order (KV head, sequence, query tile from the last), dealt to the XCDs
  // in contiguous ranges: with 8 KV heads every XCD takes one head of every
  // sequence -- the same share of a ragged batch -- and only that head's K/V
  // passes through its L2; the workgroups resident on an XCD at a time work on
  // neighbouring query tiles of one sequence, whose windows overlap.
  const int work = __builtin_amdgcn_readfirstlane(xcd_logical_id(wg_x(), p.n_work));
  const int tps = p.tiles_per_seq;
  const int nseq = p.seq.num_seqs;
  const int hkv = p.cache.n_kv_heads;
  const int g = __builtin_amdgcn_readfirstlane(work / (nseq * tps));
  const int rem = work % (nseq * tps);
  const int b = __builtin_amdgcn_readfirstlane(rem / tps);
  const int qt = __builtin_amdgcn_readfirstlane(tps - 1 - rem % tps);  // heaviest (latest) first

  // workgroup-uniform metadata (kept in scalar registers)
  const int tok0 = __builtin_amdgcn_readfirstlane(p.seq.cu_seqlens[b]);
  const int n_new = __builtin_amdgcn_readfirstlane(p.seq.cu_seqlens[b + 1]) - tok0;
  if (qt * kBQ >= n_new) return;
  const int s = __builtin_amdgcn_readfirstlane(p.seq.start_pos[b]);
  const int crow = p.seq.cache_idx ? __builtin_amdgcn_readfirstlane(p.seq.cache_idx[b]) : b;
  const int W = p.cache.window;
  const int q0 = s + qt * kBQ;
  const int q_end = s + n_new;                    // one past the last query position
  // (positions go up to 2^31 - 1: sums that may pass it are formed in 64 bits)
  const int hi = q0 + min(kBQ, q_end - q0) - 1;   // last key any row needs
  const int lo = max(0, q0 - W + 1);              // first key any row needs
  // Measurement variant without the band tile skip (visit_all_tiles): the
  // tiles start at key 0, as in attention that visits the whole causal
  // triangle and masks; keys below the band are read where the call holds
  // them (from max(0, s - W + 1) on) and masked.  Same result.
  const int kt0 = p.visit_all_tiles ? 0 : (lo / kBN) * kBN;
  const int lo_rd = p.visit_all_tiles ? max(0, s - W + 1) : lo;  // first key row that may be read
  const int n_tiles = (hi - kt0) / kBN + 1;
  // tiles starting at or after nomask_lo (and ending by q0) need no mask
  const int64_t nomask_lo = (int64_t)q0 + kBQ - W;

  const int h = g * G + wave / kWph;
  const int qoff = (wave % kWph) * 32;            // this wave's first query, relative to q0
  const int n_rows = q_end - q0;                  // valid query positions from q0 on
  const int hq = p.n_q_heads;
  const float c = p.scale_log2;

  // ---- Q^T as MFMA B operand: lane -> query (lane & 15) of block qb, d-group (lane >> 4)
  // (D = 16: the 32-deep MFMA step is zero-padded; lanes 32-63 hold zeros)
  const uint16_t *Q = (const uint16_t *)p.q;
  bf16x8 qf[kKS][2];
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const int qrel = qoff + 16 * qb + (lane & 15);
    const bool ok = qrel < n_rows && (D >= 32 || lane < 32);
    const uint16_t *qrow = Q + ((size_t)(tok0 + (q0 - s) + qrel) * hq + h) * D + 8 * ((lane >> 4) & (kC - 1));
#pragma unroll
    for (int ks = 0; ks < kKS; ks++) {
      u32x4 v = {0, 0, 0, 0};
      if (ok) v = *(const u32x4 *)(qrow + 32 * ks);
      qf[ks][qb] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- Tile streaming.  Group A (waves 0-3) loads K tiles, group B (waves
  // 4-7) V tiles.  A tile is kNL loads of 1 KiB (kRpl rows each); wave wg of
  // its group issues loads wg, wg+4, ..., i.e. rows kRpl*wg + 4*kRpl*m +
  // (lane/kC), and its lane writes LDS chunk (lane % kC) of that row, which
  // holds the logical chunk (lane % kC) ^ swizzle(row) -- a per-lane constant
  // (the swizzles repeat every 4*kRpl rows).
  const int grp = wave >> 2, wg = wave & 3;
  const int row_l = kRpl * wg + lane / kC;           // row of load m is row_l + 4 kRpl m
  const int pchunk = lane % kC;
  const int lchunk = grp == 0 ? (pchunk ^ Gm::kswz(row_l)) : (pchunk ^ (2 * Gm::vseg(row_l)));
  const char *src_ring = (const char *)(grp == 0 ? p.cache.k : p.cache.v);
  const char *src_new = (const char *)(grp == 0 ? p.k_new : p.v_new);
  const int64_t ring_row0 = ((int64_t)crow * hkv + g) * (int64_t)W;     // ring rows of (crow, g)
  const int64_t new_stride = (int64_t)hkv * kRowB;                     // bytes between tokens
  const int64_t new_tok0 = (int64_t)(tok0 - s);                        // token index of position 0
  const uint32_t lane_off_new = (uint32_t)(row_l * hkv * kRowB + lchunk * 16);
  const uint32_t lane_off_ring = (uint32_t)(row_l * kRowB + lchunk * 16);
  auto load_tile = [&](unsigned char *dst, int ts) __attribute__((always_inline)) {
    if (Gm::kNL < 4 && wg >= Gm::kNL) return;  // D = 16: a tile is two loads
    const bool all_valid = ts >= lo_rd && ts + kBN - 1 <= hi;
    const int ts_mod = ts % W;
    // fast paths: a uniform base (scalar registers) plus this lane's 32-bit offset
    if (all_valid && ts >= s) {
      const char *base = src_new + ((new_tok0 + ts) * hkv + g) * (int64_t)kRowB;
#pragma unroll
      for (int m = 0; m < Gm::kLoads; m++)
        __builtin_amdgcn_global_load_lds(base + (int64_t)(4 * kRpl * m) * new_stride + lane_off_new,
                                         (lds_void *)(dst + (wg + 4 * m) * 1024), 16, 0, 0);
    } else if (all_valid && ts + kBN - 1 < s && ts_mod + kBN <= W) {
      const char *base = src_ring + (ring_row0 + ts_mod) * kRowB;
#pragma unroll
      for (int m = 0; m < Gm::kLoads; m++)
        __builtin_amdgcn_global_load_lds(base + 4 * kRpl * m * kRowB + lane_off_ring,
                                         (lds_void *)(dst + (wg + 4 * m) * 1024), 16, 0, 0);
    } else {
      // edge tile: rows outside [lo, hi] read the nearest key of the band
#pragma unroll
      for (int m = 0; m < Gm::kLoads; m++) {
        const int j = min(max(ts + row_l + 4 * kRpl * m, lo_rd), hi);
        const char *src = j < s ? src_ring + (ring_row0 + j % W) * kRowB
                                : src_new + ((new_tok0 + j) * hkv + g) * (int64_t)kRowB;
        __builtin_amdgcn_global_load_lds(src + lchunk * 16, (lds_void *)(dst + (wg + 4 * m) * 1024), 16, 0, 0);
      }
    }
  };
  auto kslot = [&](int i) __attribute__((always_inline)) { return smem + i * kTileB; };
  auto vslot = [&](int i) __attribute__((always_inline)) { return smem + (3 + i) * kTileB; };

  // LDS offsets of this lane's MFMA operand reads.
  //   K (A operand of S^T): row 16*kbi + lane%16, logical chunk 4*ks + lane/16
  //     (D = 16: chunk (lane/16) % 2; lanes 32-63 meet zero Q) -> k_off[ks] + 16*kRowB*kbi
  //   V (transposed reads): rows 32*kk + 16*half + 4*(lane/16) + (lane%16)/4,
  //     columns 16*db + 4*(lane%4) .. +4 -> v_off[db] + rows*kRowB
  // (the swizzles of rows r and r + 16 agree, so the offsets are per lane)
  int k_off[kKS], v_off[kDB];
  {
    const int r = lane & 15;
#pragma unroll
    for (int ks = 0; ks < kKS; ks++) k_off[ks] = r * kRowB + ((((4 * ks + (lane >> 4)) & (kC - 1)) ^ Gm::kswz(r)) << 4);
    const int vr = 4 * (lane >> 4) + ((lane & 15) >> 2);
    const int vb = vr * kRowB + 8 * (lane & 3);
#pragma unroll
    for (int db = 0; db < kDB; db++) v_off[db] = vb + 32 * (db ^ Gm::vseg(vr));
  }

  f32x4 o[kDB][2];
#pragma unroll
  for (int db = 0; db < kDB; db++)
#pragma unroll
    for (int qb = 0; qb < 2; qb++) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Running max M of each query row's raw scores q.k, kept as the accumulator
  // start negm = -M (0 while M = -inf) and the rescale threshold gap on the
  // tile max of the accumulators (kRescaleSlack / c while M is finite, -inf
  // before).
  f32x4 negm[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float gap[2] = {-INFINITY, -INFINITY};
  const float gap_finite = kRescaleSlack / c;
  // Row sums on the matrix cores: lsum[qb] += ones P^T, so every register of a
  // lane holds the whole sum of its query column (no cross-lane reduction).
  f32x4 lsum[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{kBf16OnePair, kBf16OnePair, kBf16OnePair, kBf16OnePair});
  f32x4 sa[4][2];                       // S^T of the tile in flight: 4 key blocks x 2 query blocks
  u32x4 pw[2][2];                       // P^T (bf16 pairs) of the softmaxed tile: [32-key slice][qb]

  // S^T - M = K Q^T + negm (the prologue's first tile; the matrix half-step
  // below computes the same for the tiles after it)
  auto qk = [&](const unsigned char *kb) __attribute__((always_inline)) {
#pragma unroll
    for (int kbi = 0; kbi < 4; kbi++)
#pragma unroll
      for (int qb = 0; qb < 2; qb++) sa[kbi][qb] = negm[qb];
#pragma unroll
    for (int ks = 0; ks < kKS; ks++) {
#pragma unroll
      for (int kbi = 0; kbi < 4; kbi++) {
        const bf16x8 kf = *(const bf16x8 *)(kb + k_off[ks] + 16 * kRowB * kbi);
        sa[kbi][0] = mfma16(kf, qf[ks][0], sa[kbi][0]);
        sa[kbi][1] = mfma16(kf, qf[ks][1], sa[kbi][1]);
      }
    }
  };

  // V^T fragment for O^T += V^T P^T: 16 d-columns (block db) x 32 keys (slice kk)
  // of the V tile at vbase, as two 4-key transposed reads per lane.
  auto vread = [&](const unsigned char *vbase, int kk, int db) __attribute__((always_inline)) {
    const unsigned char *va = vbase + v_off[db] + 32 * kk * kRowB;
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)va);
    const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(va + 16 * kRowB));
    u32x4 w;
    w[0] = __builtin_bit_cast(u32x2, v1)[0];
    w[1] = __builtin_bit_cast(u32x2, v1)[1];
    w[2] = __builtin_bit_cast(u32x2, v2)[0];
    w[3] = __builtin_bit_cast(u32x2, v2)[1];
    return __builtin_bit_cast(bf16x8, w);
  };

  // mask (edge tiles), online softmax, P^T as bf16 into pw.
  // A query's 64 keys sit in lanes l, l^16, l^32, l^48.  The running max M
  // only moves when a tile's max exceeds it by more than kRescaleSlack in log2
  // units (c (q.k - M)): the weights then stay <= 2^kRescaleSlack, O and the
  // row sums are rescaled only on those (rare) tiles, and the result is
  // unchanged because they share M.
  auto softmax = [&](int ts, bool masked) __attribute__((always_inline)) {
    if (masked) {
      __asm__ volatile("");  // keep this a branch: only edge tiles pay for the mask
      // key - query for this lane's first element; valid iff -W < key - query <= 0
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
        const int d0 = (ts - q0) + 4 * (lane >> 4) - (qoff + 16 * qb + (lane & 15)) + W - 1;
#pragma unroll
        for (int kbi = 0; kbi < 4; kbi++)
#pragma unroll
          for (int i = 0; i < 4; i++)
            if ((unsigned)(d0 + 16 * kbi + i) >= (unsigned)W) sa[kbi][qb][i] = -INFINITY;
      }
    }
    // sa already holds q.k - mc (the accumulators started at negm = -mc),
    // where mc is the running max M when this tile's scores were computed, or
    // 0 while M = -inf.  The weight of a key is exp2(c (q.k - M)).  The tile
    // needs a rescale iff its max exceeds M by more than kRescaleSlack / c,
    // i.e. iff max(sa) > gap.
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      // tile max of this lane's 16 values as a chain of 3-input maxima
      float mt = fmaxf(sa[0][qb][0], sa[0][qb][1]);
#pragma unroll
      for (int e = 2; e < 16; e += 2)
        mt = fmaxf(fmaxf(mt, sa[e / 4][qb][e % 4]), sa[e / 4][qb][e % 4 + 1]);
      // The test runs on each lane's own 16 values: the 4 lanes of a query
      // share its threshold, so the query's max exceeds it iff one of its
      // lanes does.  The cross-lane max is only formed on the rare tiles that
      // rescale.
      if (__builtin_amdgcn_ballot_w64(mt > gap[qb])) {
        mt = max_pair32(max_pair16(mt));
        const bool upd = mt > gap[qb];
        const bool m_inf = gap[qb] == -INFINITY;
        const float mc = -negm[qb][0];
        const float mn = upd ? mt + mc : (m_inf ? -INFINITY : mc);
        const float alpha = m_inf ? 0.f : __builtin_amdgcn_exp2f((mc - mn) * c);
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < kDB; db++) o[db][qb] *= alpha;
        const bool mn_inf = mn == -INFINITY;
        const float shift = mn_inf ? 0.f : mn - mc;  // 0 where M did not move
#pragma unroll
        for (int kbi = 0; kbi < 4; kbi++) sa[kbi][qb] -= shift;
        const float nm = mn_inf ? 0.f : -mn;
        negm[qb] = f32x4{nm, nm, nm, nm};
        gap[qb] = mn_inf ? -INFINITY : gap_finite;
      }
#pragma unroll
      for (int kbi = 0; kbi < 4; kbi++)
#pragma unroll
        for (int i = 0; i < 4; i++) sa[kbi][qb][i] = __builtin_amdgcn_exp2f(sa[kbi][qb][i] * c);
#pragma unroll
      for (int kk = 0; kk < 2; kk++) {
        u32x4 w;
        w[0] = pack_bf16(sa[2 * kk][qb][0], sa[2 * kk][qb][1]);
        w[1] = pack_bf16(sa[2 * kk][qb][2], sa[2 * kk][qb][3]);
        w[2] = pack_bf16(sa[2 * kk + 1][qb][0], sa[2 * kk + 1][qb][1]);
        w[3] = pack_bf16(sa[2 * kk + 1][qb][2], sa[2 * kk + 1][qb][3]);
        pw[kk][qb] = w;
      }
    }
  };

  // ---- Schedule.  Tile t = softmax half-step V_t and matrix half-step
  // M_t = { O += P(t) V(t);  S = K(t+1) Q^T }, separated by barriers; group B
  // runs one half-step behind group A.  During V_t group A streams K(t+2)
  // into K slot (t+2) mod 3 and group B streams V(t+1) into V slot (t+1) mod 2.
  // With A's V_t in half-step 2t and B's in 2t+1 (M_t one later), a slot is
  // rewritten only after its last reader (B's M of two tiles back, or of the
  // previous tile for V) has passed a barrier, and each tile is complete (its
  // loads waited for) one barrier before its first reader.  Every wave executes
  // the same number of barriers.
  //
  // Tiles needing a mask form a prefix (the window's lower edge) and a suffix
  // (the diagonal) of the tile range; the interior runs without mask code.
  //   unmasked  <=>  ts >= nomask_lo  and  ts + kBN - 1 <= q0
  const int n_lead = (int)min((int64_t)n_tiles, max((int64_t)0, (nomask_lo - kt0 + kBN - 1) / kBN));
  const int n_diag_free = (q0 - kBN + 1 - kt0) >= 0 ? (q0 - kBN + 1 - kt0) / kBN + 1 : 0;
  const int t_mid_end = max(n_lead, min(n_tiles, n_diag_free));

  // The matrix half-step M_t = { row sums; S^T(t+1) - M = K(t+1) Q^T + negm;
  // O^T += V^T P^T(t) } as a pipeline over operand fragments: first the 4 kKS K
  // fragments of the next tile's scores (step ks, key block kbi; one read
  // each), then the 2 kDB V fragments of P V (key slice kk, d-block db; two
  // transposed reads each), each feeding two MFMAs (query blocks 0 and 1).  The
  // scores come first because the next softmax half-step needs them; O is not
  // read before the next matrix half-step.  Fragment f is read kFragLead
  // fragments ahead of its MFMAs, the four row-sum MFMAs (no LDS operand) run
  // under the latency of the first reads, and every iteration ends in a
  // scheduling barrier, so the compiler keeps this order (its wait counts
  // follow the reads).
  constexpr int kFragLead = 3;
  auto matrix_half_step = [&](const unsigned char *vbase, const unsigned char *kb, auto with_qk)
                              __attribute__((always_inline)) {
    constexpr int kNK = decltype(with_qk)::value ? 4 * kKS : 0;
    constexpr int kNF = kNK + 2 * kDB;
    bf16x8 fr[kFragLead];
    auto load = [&](int f) __attribute__((always_inline)) {
      if (f < kNK) return *(const bf16x8 *)(kb + k_off[f / 4] + 16 * kRowB * (f % 4));
      const int g = f - kNK;
      return vread(vbase, g / kDB, g % kDB);
    };
    auto use = [&](int f, bf16x8 x) __attribute__((always_inline)) {
      if (f < kNK) {
        const int ks = f / 4, kbi = f % 4;
        sa[kbi][0] = mfma16(x, qf[ks][0], ks == 0 ? negm[0] : sa[kbi][0]);
        sa[kbi][1] = mfma16(x, qf[ks][1], ks == 0 ? negm[1] : sa[kbi][1]);
      } else {
        const int g = f - kNK, kk = g / kDB, db = g % kDB;
        o[db][0] = mfma16(x, __builtin_bit_cast(bf16x8, pw[kk][0]), o[db][0]);
        o[db][1] = mfma16(x, __builtin_bit_cast(bf16x8, pw[kk][1]), o[db][1]);
      }
    };
#pragma unroll
    for (int i = 0; i < kNF + kFragLead; i++) {
      if (i >= kFragLead) use(i - kFragLead, fr[(i - kFragLead) % kFragLead]);
      if (i < kNF) fr[i % kFragLead] = load(i);
      if (i == kFragLead - 1) {
        // row sums of exactly the bf16 weights that enter P V
#pragma unroll
        for (int kk = 0; kk < 2; kk++) {
          lsum[0] = mfma16(ones, __builtin_bit_cast(bf16x8, pw[kk][0]), lsum[0]);
          lsum[1] = mfma16(ones, __builtin_bit_cast(bf16x8, pw[kk][1]), lsum[1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One tile: t is the tile index; R = t mod 6 when it is known at compile
  // time (then every LDS slot address is a constant offset), -1 otherwise.
  auto step_r = [&](int t, bool masked, auto with_qk, auto res) __attribute__((always_inline)) {
    constexpr int R = decltype(res)::value;
    const int nt = grp == 0 ? t + 2 : t + 1;  // the tile this group streams now
    const int kl = R < 0 ? (t + 2) % 3 : (R + 2) % 3, vl = R < 0 ? (t + 1) & 1 : (R + 1) & 1;
    const int kq = R < 0 ? (t + 1) % 3 : (R + 1) % 3, vp = R < 0 ? t & 1 : R & 1;
    if (nt < n_tiles) load_tile(grp == 0 ? kslot(kl) : vslot(vl), kt0 + nt * kBN);
    softmax(kt0 + t * kBN, masked);
    wait_vmem();
    __syncthreads();
    // the matrix half-step's wave issues first when both waves of the SIMD are
    // ready (MFMAs and operand reads ahead of the other wave's softmax VALU)
    __builtin_amdgcn_s_setprio(3);
    matrix_half_step(vslot(vp), kslot(kq), with_qk);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  };
  constexpr std::integral_constant<int, -1> kRt{};
  auto step = [&](int t, bool masked, auto with_qk) __attribute__((always_inline)) { step_r(t, masked, with_qk, kRt); };

  if (grp == 0) {
    load_tile(kslot(0), kt0);
    if (n_tiles > 1) load_tile(kslot(1), kt0 + kBN);
  } else {
    load_tile(vslot(0), kt0);
  }
  wait_vmem();
  __syncthreads();
  if (grp == 1) __builtin_amdgcn_s_barrier();  // group B: half a step behind
  qk(kslot(0));
  // every tile but the last also computes the scores of its successor
  constexpr std::true_type kNext{};
  constexpr std::false_type kLast{};
  const int t_last = n_tiles - 1;
  int t = 0;
  for (; t < min(n_lead, t_last); t++) step(t, true, kNext);
  {
    // the unmasked interior, unrolled by 6 (3 K slots x 2 V slots) from a tile
    // index that is a multiple of 6, so its slot addresses are immediates
    const int mid_end = min(t_mid_end, t_last);
    for (; t < mid_end && t % 6 != 0; t++) step(t, false, kNext);
    for (; t + 6 <= mid_end; t += 6) {
      step_r(t, false, kNext, std::integral_constant<int, 0>{});
      step_r(t + 1, false, kNext, std::integral_constant<int, 1>{});
      step_r(t + 2, false, kNext, std::integral_constant<int, 2>{});
      step_r(t + 3, false, kNext, std::integral_constant<int, 3>{});
      step_r(t + 4, false, kNext, std::integral_constant<int, 4>{});
      step_r(t + 5, false, kNext, std::integral_constant<int, 5>{});
    }
    for (; t < mid_end; t++) step(t, false, kNext);
  }
  for (; t < t_last; t++) step(t, true, kNext);
  step(t_last, !(t_last >= n_lead && t_last < t_mid_end), kLast);
  if (grp == 0) __builtin_amdgcn_s_barrier();  // group A: matches B's extra barrier

  // epilogue: normalise by the row sums (every lane holds its query's whole
  // sum), round to bf16 and store.  The output goes out in whole rows: each
  // wave stages its 32 rows x D in LDS (free once every wave has passed the
  // last barrier; 16-byte chunks XOR-swizzled by row so that the 16 rows of one
  // write hit different banks), then each lane stores 16-byte pieces, a wave
  // instruction covering 1024 / (2 D) complete rows.  The stores are
  // non-temporal: the output is never read back here, and kept out of the L2
  // it leaves that to the K/V tiles.  Against 8-byte stores straight from the
  // accumulators (a quarter row per 16 rows and instruction): +3 % at head_dim
  // 128 for G = 1, 2 and 4, +2 % at G = 8, level at head_dim 16; the output is
  // the same bit for bit.  Non-temporal 8-byte stores wrote partial lines (the
  // write counter read 1.8x the output's bytes).
  {
    unsigned char *stage = smem + wave * (32 * kRowB);
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      const float inv = 1.0f / lsum[qb][0];
      const int r = 16 * qb + (lane & 15);
#pragma unroll
      for (int db = 0; db < kDB; db++) {
        u32x2 w;
        w[0] = pack_bf16(o[db][qb][0] * inv, o[db][qb][1] * inv);
        w[1] = pack_bf16(o[db][qb][2] * inv, o[db][qb][3] * inv);
        const int byte = 32 * db + 8 * (lane >> 4);  // columns 16 db + 4 (lane / 16) .. + 3
        *(u32x2 *)(stage + r * kRowB + (((byte >> 4) ^ (r & (kC - 1))) << 4) + (byte & 15)) = w;
      }
    }
    __syncthreads();
    uint16_t *O = (uint16_t *)p.out;
    constexpr int kPieces = 32 * kC / 64;  // 16-byte pieces per lane
#pragma unroll
    for (int i = 0; i < kPieces; i++) {
      const int idx = 64 * i + lane;
      const int r = idx / kC, ch = idx % kC;
      const u32x4 x = *(const u32x4 *)(stage + r * kRowB + ((ch ^ (r & (kC - 1))) << 4));
      const int qrel = qoff + r;
      if (qrel < n_rows) {
        u32x4 *dst = (u32x4 *)(O + ((size_t)(tok0 + (q0 - s) + qrel) * hq + h) * D) + ch;
        __builtin_nontemporal_store(x, dst);
      }
    }
  }
}

template <int G, int D>
hipError_t launch_gd(const PrefillParams &p, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_bf16_kernel<G, D>), dim3((unsigned)p.n_work), dim3(kThreads), Geo<D>::kLdsBytes,
                     stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillParams &p, int group, hipStream_t stream) {
  switch (group) {
    case 1: return launch_gd<1, D>(p, stream);
    case 2: return launch_gd<2, D>(p, stream);
    case 4: return launch_gd<4, D>(p, stream);
    case 8: return launch_gd<8, D>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int prefill_bf16_tile_rows(int group) { return 32 * (kWaves / group); }

hipError_t launch_prefill_bf16(const PrefillParams &p, int group, hipStream_t stream) {
  if (p.n_work == 0) return hipSuccess;
  switch (p.cache.head_dim) {
    case 128: return launch_d<128>(p, group, stream);
    case 64: return launch_d<64>(p, group, stream);
    case 16: return launch_d<16>(p, group, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swa
