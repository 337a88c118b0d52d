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
//     tiles (2 slots); no staging registers.  LDS rows are 256 B with XOR
//     swizzles of the 16-byte chunks: K chunk ^ (row % 16) (the 16-byte K
//     reads of 16 rows hit 16 different chunks), V chunk ^ (2 (row % 4) +
//     8 ((row / 4) % 2)): a transposed read of 32 lanes covers rows 8k..8k+7,
//     32 B each, and these land in 8 different 32-byte segments, i.e. all 64
//     banks once.
//   * Only tiles intersecting the workgroup's band [q0-W+1, q_last] are
//     visited; only tiles crossing a row's window edge or the diagonal run the
//     mask code.  Keys outside the band are never read from outside it: their
//     rows are loaded from the nearest key of the band (always written data)
//     and masked, so unwritten cache slots cannot reach the arithmetic.
//   * Online softmax in fp32 with exp2.  The softmax half-step competes with
//     the other wave's MFMAs for the VALU issue port, so its instruction count
//     per tile bounds the matrix rate; it is kept small:
//       - the score accumulators start at -M (the running max of q.k), so
//         a weight is exp2(c * accumulator), one multiply per score;
//       - the row sums are an MFMA of the bf16 weights with a ones operand,
//         which also leaves every lane with its query's complete sum;
//       - the rescale test is one compare of the tile max against a per-row
//         threshold.
//   * Work order (KV head, sequence, query tile from the last), dealt to the
//     XCDs in contiguous ranges: one KV head per XCD balances ragged batches
//     and keeps each head's K/V in one L2.
#include "device_common.h"
#include "swa_internal.h"

#include <type_traits>

namespace swa {
namespace {

constexpr int kD = 128;
constexpr int kBN = 64;                       // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowB = kD * 2;                 // 256-byte LDS rows
constexpr int kTileB = kBN * kRowB;           // 16 KiB
constexpr int kLdsBytes = 5 * kTileB;         // 3 K slots + 2 V slots
constexpr float kRescaleSlack = 8.0f;         // log2 units: weights stay <= 256
constexpr uint32_t kBf16OnePair = 0x3F803F80u;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Wait for this wave's outstanding global loads (including those that write
// LDS directly); expcnt and lgkmcnt are left unconstrained.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int G>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillParams p) {
  constexpr int kWph = kWaves / G;  // waves per query head
  constexpr int kBQ = 32 * kWph;    // query positions per workgroup
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave choices scalar
  // Work order (KV head, sequence, query tile from the last), dealt to the XCDs
  // in contiguous ranges: with 8 KV heads every XCD takes one head of every
  // sequence -- the same share of a ragged batch -- and only that head's K/V
  // passes through its L2; the workgroups resident on an XCD at a time work on
  // neighbouring query tiles of one sequence, whose windows overlap.
  const int work = __builtin_amdgcn_readfirstlane(xcd_logical_id(blockIdx.x, p.n_work));
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
  const int kt0 = (lo / kBN) * kBN;
  const int n_tiles = (hi - kt0) / kBN + 1;
  // tiles starting at or after nomask_lo (and ending by q0) need no mask
  const int64_t nomask_lo = (int64_t)q0 + kBQ - W;

  const int h = g * G + wave / kWph;
  const int qoff = (wave % kWph) * 32;            // this wave's first query, relative to q0
  const int n_rows = q_end - q0;                  // valid query positions from q0 on
  const int hq = p.n_q_heads;
  const float c = p.scale_log2;

  // ---- Q^T as MFMA B operand: lane -> query (lane & 15) of block qb, d-group (lane >> 4)
  const uint16_t *Q = (const uint16_t *)p.q;
  bf16x8 qf[4][2];
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const int qrel = qoff + 16 * qb + (lane & 15);
    const bool ok = qrel < n_rows;
    const uint16_t *qrow = Q + ((size_t)(tok0 + (q0 - s) + qrel) * hq + h) * kD + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      u32x4 v = {0, 0, 0, 0};
      if (ok) v = *(const u32x4 *)(qrow + 32 * ks);
      qf[ks][qb] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- Tile streaming.  Group A (waves 0-3) loads K tiles, group B (waves
  // 4-7) V tiles.  A tile is 16 loads of 1 KiB (4 rows each); wave wg of its
  // group issues loads wg, wg+4, wg+8, wg+12, i.e. rows 4*wg + 16*m + (lane/16),
  // and its lane writes LDS chunk (lane % 16) of that row, which holds the
  // logical chunk (lane % 16) ^ swizzle(row) -- a per-lane constant.
  const int grp = wave >> 2, wg = wave & 3;
  const int row_l = 4 * wg + (lane >> 4);            // row of load m is row_l + 16 m
  const int pchunk = lane & 15;
  const int lchunk = grp == 0 ? (pchunk ^ (row_l & 15)) : (pchunk ^ (2 * (row_l & 3)) ^ (8 * ((row_l >> 2) & 1)));
  const char *src_ring = (const char *)(grp == 0 ? p.cache.k : p.cache.v);
  const char *src_new = (const char *)(grp == 0 ? p.k_new : p.v_new);
  const int64_t ring_row0 = ((int64_t)crow * hkv + g) * (int64_t)W;     // ring rows of (crow, g)
  const int64_t new_stride = (int64_t)hkv * kRowB;                     // bytes between tokens
  const int64_t new_tok0 = (int64_t)(tok0 - s);                        // token index of position 0
  const uint32_t lane_off_new = (uint32_t)(row_l * hkv * kRowB + lchunk * 16);
  const uint32_t lane_off_ring = (uint32_t)(row_l * kRowB + lchunk * 16);
  auto load_tile = [&](unsigned char *dst, int ts) __attribute__((always_inline)) {
    const bool all_valid = ts >= lo && ts + kBN - 1 <= hi;
    const int ts_mod = ts % W;
    // fast paths: a uniform base (scalar registers) plus this lane's 32-bit offset
    if (all_valid && ts >= s) {
      const char *base = src_new + ((new_tok0 + ts) * hkv + g) * (int64_t)kRowB;
#pragma unroll
      for (int m = 0; m < 4; m++)
        __builtin_amdgcn_global_load_lds(base + (int64_t)(16 * m) * new_stride + lane_off_new,
                                         (lds_void *)(dst + (wg + 4 * m) * 1024), 16, 0, 0);
    } else if (all_valid && ts + kBN - 1 < s && ts_mod + kBN <= W) {
      const char *base = src_ring + (ring_row0 + ts_mod) * kRowB;
#pragma unroll
      for (int m = 0; m < 4; m++)
        __builtin_amdgcn_global_load_lds(base + 16 * m * kRowB + lane_off_ring,
                                         (lds_void *)(dst + (wg + 4 * m) * 1024), 16, 0, 0);
    } else {
      // edge tile: rows outside [lo, hi] read the nearest key of the band
#pragma unroll
      for (int m = 0; m < 4; m++) {
        const int j = min(max(ts + row_l + 16 * m, lo), hi);
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
  //     -> k_off[ks] + 4096*kbi
  //   V (transposed reads): rows 32*kk + 16*half + 4*(lane/16) + (lane%16)/4,
  //     columns 16*db + 4*(lane%4) .. +4 -> v_off[db/4][db%4] + rows*256
  int k_off[4], v_off[2][4];
  {
    const int r = lane & 15;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) k_off[ks] = r * kRowB + (((4 * ks + (lane >> 4)) ^ r) << 4);
    const int vr = 4 * (lane >> 4) + ((lane & 15) >> 2);
    const int j = vr & 3, hv = (vr >> 2) & 1;
    const int vb = vr * kRowB + 8 * (lane & 3);
#pragma unroll
    for (int dl = 0; dl < 4; dl++) {
      v_off[0][dl] = vb + 32 * (dl ^ j) + 128 * hv;
      v_off[1][dl] = vb + 32 * (dl ^ j) + 128 * (hv ^ 1);
    }
  }

  f32x4 o[8][2];
#pragma unroll
  for (int db = 0; db < 8; db++)
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

  // S^T - M = K Q^T + negm (the order of LDS reads and MFMAs is set by the
  // half-step schedule)
  auto qk = [&](const unsigned char *kb) __attribute__((always_inline)) {
#pragma unroll
    for (int kbi = 0; kbi < 4; kbi++)
#pragma unroll
      for (int qb = 0; qb < 2; qb++) sa[kbi][qb] = negm[qb];
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
#pragma unroll
      for (int kbi = 0; kbi < 4; kbi++) {
        const bf16x8 kf = *(const bf16x8 *)(kb + k_off[ks] + 4096 * kbi);
        sa[kbi][0] = mfma16(kf, qf[ks][0], sa[kbi][0]);
        sa[kbi][1] = mfma16(kf, qf[ks][1], sa[kbi][1]);
      }
    }
  };

  // V^T fragment for O^T += V^T P^T: 16 d-columns (block db) x 32 keys (slice kk)
  // of the V tile at vbase, as two 4-key transposed reads per lane.
  auto vread = [&](const unsigned char *vbase, int kk, int db) __attribute__((always_inline)) {
    const unsigned char *va = vbase + v_off[db >> 2][db & 3] + 32 * kk * kRowB;
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)va);
    const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(va + 16 * kRowB));
    u32x4 w;
    w[0] = __builtin_bit_cast(u32x2, v1)[0];
    w[1] = __builtin_bit_cast(u32x2, v1)[1];
    w[2] = __builtin_bit_cast(u32x2, v2)[0];
    w[3] = __builtin_bit_cast(u32x2, v2)[1];
    return __builtin_bit_cast(bf16x8, w);
  };

  // row sums and O^T += V^T P^T (order of reads and MFMAs as for qk)
  auto pv = [&](const unsigned char *vbase) __attribute__((always_inline)) {
    // row sums of exactly the bf16 weights that enter P V; these MFMAs need no
    // LDS data, so they go first, under the latency of the first operand reads
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      lsum[0] = mfma16(ones, __builtin_bit_cast(bf16x8, pw[kk][0]), lsum[0]);
      lsum[1] = mfma16(ones, __builtin_bit_cast(bf16x8, pw[kk][1]), lsum[1]);
    }
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      const bf16x8 p0 = __builtin_bit_cast(bf16x8, pw[kk][0]);
      const bf16x8 p1 = __builtin_bit_cast(bf16x8, pw[kk][1]);
#pragma unroll
      for (int db = 0; db < 8; db++) {
        const bf16x8 vf = vread(vbase, kk, db);
        o[db][0] = mfma16(vf, p0, o[db][0]);
        o[db][1] = mfma16(vf, p1, o[db][1]);
      }
    }
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
      mt = max_pair32(max_pair16(mt));
      const bool upd = mt > gap[qb];
      if (__builtin_amdgcn_ballot_w64(upd)) {
        const bool m_inf = gap[qb] == -INFINITY;
        const float mc = -negm[qb][0];
        const float mn = upd ? mt + mc : (m_inf ? -INFINITY : mc);
        const float alpha = m_inf ? 0.f : __builtin_amdgcn_exp2f((mc - mn) * c);
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; db++) o[db][qb] *= alpha;
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

  // Order of the matrix half-step's 48 LDS reads (32 V, then 16 K) and 68
  // MFMAs (4 row sums, 32 PV, then 32 QK): eight reads first, then the four
  // row-sum MFMAs, then two MFMAs and two reads alternately, so reads run
  // about four MFMA pairs ahead of their consumers and the K reads of the next
  // QK overlap the tail of PV.  (The compiler may
  // still move the last QK MFMAs past the closing barrier; measured, that
  // beats keeping them inside.)
  auto schedule_matrix_half_step = [&]() __attribute__((always_inline)) {
    constexpr int kReads = 48, kLead = 8, kPairs = (kReads - kLead) / 2;
    __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);  // 0x100: LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);      // the row-sum MFMAs
#pragma unroll
    for (int i = 0; i < kPairs; i++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);    // 0x008: MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 64 - 2 * kPairs, 0);
  };

  auto step = [&](int t, bool masked, auto with_qk) __attribute__((always_inline)) {
    const int nt = grp == 0 ? t + 2 : t + 1;  // the tile this group streams now
    if (nt < n_tiles) load_tile(grp == 0 ? kslot(nt % 3) : vslot(nt & 1), kt0 + nt * kBN);
    softmax(kt0 + t * kBN, masked);
    wait_vmem();
    __syncthreads();
    // the matrix half-step's wave issues first when both waves of the SIMD are
    // ready (MFMAs and operand reads ahead of the other wave's softmax VALU)
    __builtin_amdgcn_s_setprio(3);
    pv(vslot(t & 1));
    if constexpr (decltype(with_qk)::value) {
      qk(kslot((t + 1) % 3));
      schedule_matrix_half_step();
    }
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
  };

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
  for (; t < min(t_mid_end, t_last); t++) step(t, false, kNext);
  for (; t < t_last; t++) step(t, true, kNext);
  step(t_last, !(t_last >= n_lead && t_last < t_mid_end), kLast);
  if (grp == 0) __builtin_amdgcn_s_barrier();  // group A: matches B's extra barrier

  // epilogue: finish the row sums across the 4 lane groups, normalise, store bf16
  uint16_t *O = (uint16_t *)p.out;
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    const float lt = lsum[qb][0];
    const float inv = 1.0f / lt;
    const int qrel = qoff + 16 * qb + (lane & 15);
    if (qrel < n_rows) {
      uint16_t *orow = O + ((size_t)(tok0 + (q0 - s) + qrel) * hq + h) * kD + 4 * (lane >> 4);
#pragma unroll
      for (int db = 0; db < 8; db++) {
        u32x2 w;
        w[0] = pack_bf16(o[db][qb][0] * inv, o[db][qb][1] * inv);
        w[1] = pack_bf16(o[db][qb][2] * inv, o[db][qb][3] * inv);
        *(u32x2 *)(orow + 16 * db) = w;
      }
    }
  }
}

template <int G>
hipError_t launch_g(const PrefillParams &p, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_bf16_kernel<G>, dim3((unsigned)p.n_work), dim3(kThreads), kLdsBytes, stream, p);
  return hipGetLastError();
}

}  // namespace

int prefill_bf16_tile_rows(int group) { return 32 * (kWaves / group); }

hipError_t launch_prefill_bf16(const PrefillParams &p, int group, hipStream_t stream) {
  if (p.n_work == 0) return hipSuccess;
  switch (group) {
    case 1: return launch_g<1>(p, stream);
    case 2: return launch_g<2>(p, stream);
    case 4: return launch_g<4>(p, stream);
    case 8: return launch_g<8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace swa
