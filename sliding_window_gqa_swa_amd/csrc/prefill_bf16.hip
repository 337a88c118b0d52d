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
//   * One workgroup = (sequence, KV head g, tile of BQ query positions) x the G
//     query heads of g: 8 waves, 32 query rows each, 256 rows per workgroup.
//     Every K/V tile is staged ONCE in LDS and consumed by all G heads.
//   * S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16.  The S^T
//     accumulator layout (lane = query, registers = keys) is reused directly
//     as the B operand of the PV product, so P never leaves registers; V^T is
//     read with ds_read_b64_tr_b16 (4-key transposed loads).
//   * K/V tiles are BN = 64 keys aligned to multiples of 64 in absolute
//     position.  Only the tiles intersecting the workgroup's band
//     [q0-W+1, q_last] are visited; tiles wholly inside every row's band run
//     without a mask.  Keys outside the band are zero-filled in LDS, never
//     loaded, so unwritten cache slots cannot reach the arithmetic.
//   * LDS rows are padded: K rows to 272 B (consecutive rows 4 banks apart: the
//     16-byte K reads of 8 rows cover all 32 banks), V rows to 288 B (rows 8
//     banks apart: the 4 rows x 32 B of a transposed read of 16 lanes hit
//     disjoint banks).  Every operand address is a per-lane base plus an
//     immediate.  K and V are double-buffered (70 KiB), one barrier per tile.
//   * Online softmax in fp32 with exp2 (scale * log2 e folded into one FMA).
//   * Workgroups are ordered heaviest-first and mapped XCD-contiguously.
#include "device_common.h"
#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kD = 128;
constexpr int kBN = 64;                       // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kKRow = kD * 2 + 16;            // K rows: 256 B of data + 16 B of padding
constexpr int kVRow = kD * 2 + 32;            // V rows: 256 B of data + 32 B of padding
constexpr int kKTile = kBN * kKRow;
constexpr int kVTile = kBN * kVRow;
constexpr int kBufBytes = kKTile + kVTile;    // one K tile + one V tile
constexpr int kLdsBytes = 2 * kBufBytes;      // double-buffered
constexpr float kRescaleSlack = 8.0f;         // log2 units: weights stay <= 256
constexpr uint32_t kBf16OnePair = 0x3F803F80u;


__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int G>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillParams p) {
  constexpr int kWph = kWaves / G;  // waves per query head
  constexpr int kBQ = 32 * kWph;    // query positions per workgroup
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int work = __builtin_amdgcn_readfirstlane(xcd_logical_id(blockIdx.x, p.n_work));
  const int tps = p.tiles_per_seq;
  const int qt = tps - 1 - (work % tps);  // heaviest (latest) query tile first
  const int bg = work / tps;
  const int hkv = p.cache.n_kv_heads;
  const int g = __builtin_amdgcn_readfirstlane(bg % hkv), b = __builtin_amdgcn_readfirstlane(bg / hkv);

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

  // ---- K/V tile staging: thread -> rows r0, r0 + 32 of a tile, 16-byte chunk cc.
  // Keys below the chunk start come from ring slot j mod W (advanced
  // incrementally by 64 per tile), keys from the chunk on from k_new / v_new.
  const int r0 = tid >> 4, cc = tid & 15;
  const uint16_t *ck = (const uint16_t *)p.cache.k, *cv = (const uint16_t *)p.cache.v;
  const uint16_t *kn = (const uint16_t *)p.k_new, *vn = (const uint16_t *)p.v_new;
  const int64_t ring_base = ((int64_t)crow * hkv + g) * (int64_t)W * kD + cc * 8;
  const int64_t new_stride = (int64_t)hkv * kD;
  const int64_t new_base = ((int64_t)(tok0 - s) * hkv + g) * kD + cc * 8;  // + j * new_stride
  const int slot_step = kBN % W;
  int slot[2] = {(kt0 + r0) % W, (kt0 + r0 + 32) % W};
  u32x4 stg[4];
  auto load_tile = [&](int ts) {
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int j = ts + r0 + 32 * u;
      u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (j >= lo && j <= hi) {
        const bool ring = j < s;
        const int64_t off = ring ? ring_base + (int64_t)slot[u] * kD : new_base + (int64_t)j * new_stride;
        const uint16_t *kp = ring ? ck : kn;
        const uint16_t *vp = ring ? cv : vn;
        kv = *(const u32x4 *)(kp + off);
        vv = *(const u32x4 *)(vp + off);
      }
      stg[u] = kv;
      stg[2 + u] = vv;
      slot[u] += slot_step;
      if (slot[u] >= W) slot[u] -= W;
    }
  };
  const int kst = r0 * kKRow + cc * 16, vst = r0 * kVRow + cc * 16;
  auto store_tile = [&](int buf) {
    unsigned char *kb = smem + buf * kBufBytes;
    unsigned char *vb = kb + kKTile;
    *(u32x4 *)(kb + kst) = stg[0];
    *(u32x4 *)(kb + kst + 32 * kKRow) = stg[1];
    *(u32x4 *)(vb + vst) = stg[2];
    *(u32x4 *)(vb + vst + 32 * kVRow) = stg[3];
  };
  // LDS byte offsets of this lane's MFMA operand reads.  With padded rows every
  // read is this per-lane base plus a compile-time constant.
  //   K (A operand of S^T): row 16*kbi + lane%16, columns 32*ks + 8*(lane/16) .. +8
  //   V (transposed reads): rows 32*kk + 4*(lane/16) + (lane%16)/4 (+16),
  //                         columns 16*db + 4*(lane%4) .. +4
  const int k_lane = (lane & 15) * kKRow + (lane >> 4) * 16;
  const int v_lane = (4 * (lane >> 4) + ((lane & 15) >> 2)) * kVRow + 8 * (lane & 3);

  f32x4 o[8][2];
#pragma unroll
  for (int db = 0; db < 8; db++)
#pragma unroll
    for (int qb = 0; qb < 2; qb++) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[2] = {-INFINITY, -INFINITY};  // running max, log2 units
  float l[2] = {0.f, 0.f};              // this lane's share of the row sums

  // One K/V tile: S^T = K Q^T, (mask), online softmax, O^T += V^T P^T.
  auto tile = [&](const unsigned char *kb, const unsigned char *vb, int ts, bool masked, bool has_next) {
    f32x4 sa[4][2];
#pragma unroll
    for (int kbi = 0; kbi < 4; kbi++)
#pragma unroll
      for (int qb = 0; qb < 2; qb++) sa[kbi][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K fragments are read one 32-wide d-step ahead of the MFMAs that use them,
    // so the LDS latency overlaps the matrix work of the previous step.
    bf16x8 kf[2][4];
#pragma unroll
    for (int kbi = 0; kbi < 4; kbi++) kf[0][kbi] = *(const bf16x8 *)(kb + k_lane + 16 * kbi * kKRow);
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      if (ks + 1 < 4) {
#pragma unroll
        for (int kbi = 0; kbi < 4; kbi++)
          kf[(ks + 1) & 1][kbi] = *(const bf16x8 *)(kb + k_lane + 16 * kbi * kKRow + 64 * (ks + 1));
      }
#pragma unroll
      for (int kbi = 0; kbi < 4; kbi++) {
        sa[kbi][0] = mfma16(kf[ks & 1][kbi], qf[ks][0], sa[kbi][0]);
        sa[kbi][1] = mfma16(kf[ks & 1][kbi], qf[ks][1], sa[kbi][1]);
      }
    }
    // the next tile's global loads are issued here, after the K fragments of
    // this tile are consumed (shorter register live ranges); their latency is
    // covered by the softmax and PV work below
    if (has_next) load_tile(ts + kBN);
    if (masked) {
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
    // Online softmax per query; a query's 64 keys sit in lanes l, l^16, l^32, l^48.
    // The running max m is kept in log2 units (score * scale * log2 e) and only
    // moves when a tile's max exceeds it by more than kRescaleSlack: the
    // weights then stay <= 2^kRescaleSlack, the O/l rescale runs only on those
    // (rare) tiles, and the result is unchanged because O and l share m.
#pragma unroll
    for (int qb = 0; qb < 2; qb++) {
      float mt = -INFINITY;
#pragma unroll
      for (int kbi = 0; kbi < 4; kbi++)
        mt = fmaxf(mt, fmaxf(fmaxf(sa[kbi][qb][0], sa[kbi][qb][1]), fmaxf(sa[kbi][qb][2], sa[kbi][qb][3])));
      mt = fmaxf(mt, xor16(mt));
      mt = fmaxf(mt, xor32(mt));
      const float mts = mt * c;
      const bool upd = mts > m[qb] + kRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(upd)) {
        const float mn = upd ? mts : m[qb];
        const float alpha = (m[qb] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[qb] - mn);
        m[qb] = mn;
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; db++) o[db][qb] *= alpha;
      }
      const float mc = (m[qb] == -INFINITY) ? 0.f : m[qb];
#pragma unroll
      for (int kbi = 0; kbi < 4; kbi++)
#pragma unroll
        for (int i = 0; i < 4; i++) sa[kbi][qb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[kbi][qb][i], c, -mc));
    }
    // O^T += V^T P^T over two 32-key slices
#pragma unroll
    for (int kk = 0; kk < 2; kk++) {
      bf16x8 pf[2];
#pragma unroll
      for (int qb = 0; qb < 2; qb++) {
        u32x4 w;
        w[0] = pack_bf16(sa[2 * kk][qb][0], sa[2 * kk][qb][1]);
        w[1] = pack_bf16(sa[2 * kk][qb][2], sa[2 * kk][qb][3]);
        w[2] = pack_bf16(sa[2 * kk + 1][qb][0], sa[2 * kk + 1][qb][1]);
        w[3] = pack_bf16(sa[2 * kk + 1][qb][2], sa[2 * kk + 1][qb][3]);
        pf[qb] = __builtin_bit_cast(bf16x8, w);
        // row sum of the bf16-rounded weights, i.e. of exactly what enters P V
#pragma unroll
        for (int e = 0; e < 4; e++) l[qb] = fdot2_bf16(w[e], kBf16OnePair, l[qb]);
      }
      // V fragments are read one 16-column block ahead of their MFMAs.
      auto vread = [&](int db) {
        const unsigned char *va = vb + v_lane + 32 * kk * kVRow + 32 * db;
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)va);
        const i16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(va + 16 * kVRow));
        u32x4 w;
        w[0] = __builtin_bit_cast(u32x2, v1)[0];
        w[1] = __builtin_bit_cast(u32x2, v1)[1];
        w[2] = __builtin_bit_cast(u32x2, v2)[0];
        w[3] = __builtin_bit_cast(u32x2, v2)[1];
        return __builtin_bit_cast(bf16x8, w);
      };
      bf16x8 vf[2];
      vf[0] = vread(0);
#pragma unroll
      for (int db = 0; db < 8; db++) {
        if (db + 1 < 8) vf[(db + 1) & 1] = vread(db + 1);
        o[db][0] = mfma16(vf[db & 1], pf[0], o[db][0]);
        o[db][1] = mfma16(vf[db & 1], pf[1], o[db][1]);
      }
    }
  };

  // Tiles needing a mask form a prefix (window's lower edge) and a suffix (the
  // diagonal) of the tile range; the interior runs the unmasked body.
  //   unmasked  <=>  ts >= nomask_lo  and  ts + kBN - 1 <= q0
  const int n_lead = (int)min((int64_t)n_tiles, max((int64_t)0, (nomask_lo - kt0 + kBN - 1) / kBN));
  const int n_diag_free = (q0 - kBN + 1 - kt0) >= 0 ? (q0 - kBN + 1 - kt0) / kBN + 1 : 0;
  const int t_mid_end = max(n_lead, min(n_tiles, n_diag_free));

  auto step = [&](int t, bool masked) {
    const int ts = kt0 + t * kBN;
    const bool has_next = t + 1 < n_tiles;
    const unsigned char *kb = smem + (t & 1) * kBufBytes;
    tile(kb, kb + kKTile, ts, masked, has_next);
    if (has_next) store_tile((t + 1) & 1);
    __syncthreads();
  };

  load_tile(kt0);
  store_tile(0);
  __syncthreads();
  int t = 0;
  for (; t < n_lead; t++) step(t, true);
  for (; t < t_mid_end; t++) step(t, false);
  for (; t < n_tiles; t++) step(t, true);

  // epilogue: finish the row sums across the 4 lane groups, normalise, store bf16
  uint16_t *O = (uint16_t *)p.out;
#pragma unroll
  for (int qb = 0; qb < 2; qb++) {
    float lt = l[qb];
    lt += xor16(lt);
    lt += xor32(lt);
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
