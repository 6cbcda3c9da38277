// Lightning-indexer scores (DeepSeek-V4 digest, 模块 B eq 16; jsqmd blog 第二阶段):
//   I[b, t, s] = sum_h wI[b, t, h] * ReLU(qI[b, t, h, :] . K[b, s, :])
// for compressed entries visible to the query (m (s+1) <= p+1), -inf otherwise.
//
// MFMA path (bf16 queries, BF16 or MXFP4 keys, hI = 32, cI in {32, 64, 128}):
// the 32 heads of a query are the M dimension of v_mfma_f32_32x32x16_bf16 and
// 32 keys its N dimension.  Query fragments stay in registers for the whole
// key loop; a 256-key tile is decoded once into LDS as bf16 (MXFP4 through the
// gfx950 scaled fp4->bf16 conversion, which is exact) and shared by the four
// waves.  The head reduction sum_h w_h ReLU(acc) runs on the accumulator
// registers: 16 heads per lane plus one cross-lane add.
//
// Candidate mode (EM): the same scores, but instead of the score row a block
// keeps, per query, the composites (order key << 32 | ~index) of the visible
// keys whose order key reaches the query's threshold key, appended to the
// query's list for the block's key range; nothing else is stored.
#include <type_traits>

#include "dsv4_common.h"
#include "dsv4_internal.h"

namespace dsv4 {

// ------------------------------------------------------------------ generic
__device__ __forceinline__ float key_elem(const IndexerArgs& a, int64_t b, int64_t s, int j) {
  const int64_t row = key_row(a, b, s);
  if (a.k_layout == ROW_MXFP4) {
    const uint8_t* codes = reinterpret_cast<const uint8_t*>(a.keys) + row * (a.cI / 2);
    const uint32_t byte = codes[j >> 1];
    const uint32_t nib = (j & 1) ? (byte >> 4) : (byte & 15u);
    const uint32_t E = a.k_scales[row * (a.cI / 32) + (j >> 5)];
    return e2m1_to_f32(nib) * e8m0_to_f32(E);
  }
  const uint8_t* r = reinterpret_cast<const uint8_t*>(a.keys) + row * row_bytes(a.k_layout, a.cI);
  return load_row_elem(r, a.k_layout, a.cI, j);
}

__global__ void indexer_generic(IndexerArgs a, PosTable pt, int b0, int nb) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_b = a.nq * a.S;
  if (gid >= per_b * nb) return;
  const int64_t bl = gid / per_b;
  const int64_t b = b0 + bl;
  const int64_t t = (gid % per_b) / a.S;
  const int64_t s = gid % a.S;
  if (a.row_flags && !a.row_flags[b * a.nq + t]) return;
  const int64_t p = pt.q_pos0[bl] + t;
  float* out = a.scores + (b * a.nq + t) * a.S + s;
  if (s >= visible_count(p, a.m, a.S)) { *out = -INFINITY; return; }
  float score = 0.0f;
  for (int h = 0; h < a.hI; ++h) {
    const int64_t qbase = ((b * a.nq + t) * a.hI + h) * a.cI;
    float dot = 0.0f;
    for (int j = 0; j < a.cI; ++j) dot = fmaf(load_act(a.qI, a.q_dtype, qbase + j), key_elem(a, b, s, j), dot);
    score = fmaf(a.wI[(b * a.nq + t) * a.hI + h], fmaxf(dot, 0.0f), score);
  }
  *out = score;
}

// value of element j of a query head quantised to MXFP4 (QF = 4: its
// 32-element block scaled by 2^(floor(log2 amax) - 2), elements rounded to
// E2M1) or MXFP8 (QF = 8: scale 2^(floor(log2 amax) - 8), E4M3 elements)
template <int QF>
__device__ __forceinline__ float qx_elem(const IndexerArgs& a, int64_t qbase, int j) {
  const int j0 = j & ~31;
  float amax = 0.f;
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(load_act(a.qI, a.q_dtype, qbase + j0 + i)));
  const uint32_t E = QF == 8 ? mx8_scale_code(amax) : mx_scale_code(amax);
  const float inv = __uint_as_float((254u - E) << 23);            // 2^(127 - E)
  const float v = load_act(a.qI, a.q_dtype, qbase + j) * inv;
  return (QF == 8 ? e4m3_to_f32(f32_to_e4m3(v)) : e2m1_to_f32(f32_to_e2m1(v))) * e8m0_to_f32(E);
}

// generic path of the FP4- / FP8-query scores: one thread per (b, t, s)
template <int QF>
__global__ void indexer_generic_qx(IndexerArgs a, PosTable pt, int b0, int nb) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per_b = a.nq * a.S;
  if (gid >= per_b * nb) return;
  const int64_t bl = gid / per_b;
  const int64_t b = b0 + bl;
  const int64_t t = (gid % per_b) / a.S;
  const int64_t s = gid % a.S;
  const int64_t p = pt.q_pos0[bl] + t;
  float* out = a.scores + (b * a.nq + t) * a.S + s;
  if (s >= visible_count(p, a.m, a.S)) { *out = -INFINITY; return; }
  float score = 0.0f;
  for (int h = 0; h < a.hI; ++h) {
    const int64_t qbase = ((b * a.nq + t) * a.hI + h) * a.cI;
    float dot = 0.0f;
    for (int j = 0; j < a.cI; ++j) dot = fmaf(qx_elem<QF>(a, qbase, j), key_elem(a, b, s, j), dot);
    score = fmaf(a.wI[(b * a.nq + t) * a.hI + h], fmaxf(dot, 0.0f), score);
  }
  *out = score;
}

// 32 values -> one MXFP4 block: 16 bytes of E2M1 codes (element 2j in the low
// nibble of byte j) and the E8M0 scale code
__device__ __forceinline__ void mxfp4_block(const float (&x)[32], u32x4& codes, uint32_t& E) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  E = mx_scale_code(amax);
  const float inv = __uint_as_float((254u - E) << 23);            // 2^(127 - E)
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) w |= f32_to_e2m1(x[8 * d + e] * inv) << (4 * e);
    codes[d] = w;
  }
}

// 32 values -> one MXFP8 block: 32 E4M3 code bytes (element i in byte i; lo
// holds elements 0..15, hi 16..31) and the E8M0 scale code
__device__ __forceinline__ void mxfp8_block(const float (&x)[32], u32x4& lo, u32x4& hi, uint32_t& E) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  E = mx8_scale_code(amax);
  const float inv = __uint_as_float((254u - E) << 23);            // 2^(127 - E)
#pragma unroll
  for (int d = 0; d < 8; ++d) {
    uint32_t w = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) w |= f32_to_e4m3(x[4 * d + e] * inv) << (8 * e);
    if (d < 4) lo[d] = w;
    else hi[d - 4] = w;
  }
}

// ------------------------------------------------------------------ MFMA path
constexpr int KT = IDX_KT;   // keys per LDS tile
typedef int i32x8 __attribute__((ext_vector_type(8)));

// WQ waves split the queries, 4/WQ waves split the 8 n-tiles of a key tile;
// each wave holds QPW queries.  QF = 4 or 8: the queries are quantised to
// MXFP4 or MXFP8 in registers and the MXFP4 key tile stays in its stored form
// in LDS; each 64-channel k-step is one v_mfma_scale_f32_32x32x64_f8f6f4 on
// E2M1 or E4M3 queries against E2M1 keys with their E8M0 block scales.  Lane
// l of either operand holds row/column l % 32 and the scale of 32-channel block
// l / 32 of the k-step; an E2M1 lane holds that block's 32 codes in 16 bytes,
// an E4M3 lane holds channels 16 (l / 32) .. + 15 of block 0 in bytes 0..15 and
// the same channels of block 1 in bytes 16..31.
template <int CI, int KL, int WQ, int QPW, int QF, bool EM>
__global__ __launch_bounds__(256, 2) void indexer_mfma(IndexerArgs a, PosTable pt, int b0,
                                                        int qblocks, int tiles_per_split) {
  constexpr int WK = 4 / WQ;          // waves along the key tile
  constexpr int QB = WQ * QPW;        // queries per block
  constexpr int NTW = 8 / WK;         // 32-key n-tiles per wave
  constexpr int KS = CI / 16;         // bf16 MFMA k-steps
  constexpr bool Q4 = QF != 0;        // scaled path: quantised queries, stored MXFP4 key tile
  constexpr int K4 = CI / 64;         // scaled-MFMA k-steps
  constexpr int LDK = CI + 8;
  constexpr int CB = CI / 2, NBS = CI / 32;              // MXFP4 code / scale bytes per key
  constexpr int LDC = CB + (CI >= 128 ? 16 : 0);         // LDS code row stride (bytes)
  static_assert(!Q4 || (KL == ROW_MXFP4 && CI % 64 == 0), "FP4 queries need MXFP4 keys, cI % 64 == 0");
  __shared__ uint16_t Ks[Q4 ? 8 : KT * LDK];
  __shared__ __align__(16) uint8_t Kc[Q4 ? KT * LDC : 16];
  __shared__ uint8_t Kscl[Q4 ? KT * NBS : 4];

  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int wq = wv / WK, wk = wv % WK;
  const int bl = blockIdx.x / qblocks;
  const int64_t b = b0 + bl;
  const int64_t t0 = (int64_t)(blockIdx.x % qblocks) * QB;
  const int64_t S = a.S;
  const int64_t ntiles = (S + KT - 1) / KT;
  const int64_t tile_lo = (int64_t)blockIdx.y * tiles_per_split;
  const int64_t tile_hi = tile_lo + tiles_per_split < ntiles ? tile_lo + tiles_per_split : ntiles;
  static_assert(!EM || QF == 0, "candidate mode: bf16 queries");
  if (!EM && tile_lo >= tile_hi) return;
  if (a.row_flags) {                          // restricted: only blocks holding a flagged row
    bool any = false;
    for (int qi = 0; qi < QB; ++qi)
      if (t0 + qi < a.nq && a.row_flags[b * a.nq + t0 + qi]) any = true;
    if (!any) return;
  }

  // query fragments (B operand is the key; A operand is the 32 heads x cI)
  bf16x8 qf[QPW][Q4 ? 1 : KS];
  u32x4 q4c[QPW][Q4 ? K4 : 1];
  u32x4 q8h[QPW][QF == 8 ? K4 : 1];    // E4M3 code bytes 16..31 (MXFP8 queries)
  uint32_t q4s[QPW][Q4 ? K4 : 1];
  float wh[QPW][16];
  int64_t nvis[QPW];
  bool qvalid[QPW];
  int64_t nvis_max = 0, nvis_min = S;
  for (int qi = 0; qi < QB; ++qi) {           // block-wide maximum and minimum (uniform)
    const int64_t t = t0 + qi;
    if (t < a.nq) {
      const int64_t v = visible_count(pt.q_pos0[bl] + t, a.m, S);
      nvis_max = v > nvis_max ? v : nvis_max;
      nvis_min = v < nvis_min ? v : nvis_min;
    }
  }
#pragma unroll
  for (int qi = 0; qi < QPW; ++qi) {
    const int64_t t = t0 + wq * QPW + qi;
    qvalid[qi] = t < a.nq;
    const int64_t tt = qvalid[qi] ? t : a.nq - 1;
    nvis[qi] = qvalid[qi] ? visible_count(pt.q_pos0[bl] + t, a.m, S) : 0;
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.qI) + ((b * a.nq + tt) * 32 + (l & 31)) * CI;
    if constexpr (Q4) {
#pragma unroll
      for (int k4 = 0; k4 < K4; ++k4) {
        float x[32];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 64 * k4 + 32 * (l >> 5) + 8 * v);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[8 * v + 2 * e] = __uint_as_float(w[e] << 16);
            x[8 * v + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
          }
        }
        if constexpr (QF == 8) {
          // lane half G quantises block G of the k-step (its scale is the one
          // the MFMA applies to block G), but the 8-bit operand wants channels
          // 16 G .. 16 G + 15 of both blocks: trade halves with lane l ^ 32
          u32x4 lo, hi;
          mxfp8_block(x, lo, hi, q4s[qi][k4]);
          const u32x4 send = (l >> 5) ? lo : hi;
          u32x4 recv;
#pragma unroll
          for (int d = 0; d < 4; ++d) recv[d] = (uint32_t)__shfl_xor((int)send[d], 32);
          q4c[qi][k4] = (l >> 5) ? recv : lo;
          q8h[qi][QF == 8 ? k4 : 0] = (l >> 5) ? hi : recv;
        } else {
          mxfp4_block(x, q4c[qi][k4], q4s[qi][k4]);
        }
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        qf[qi][kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * (l >> 5)));
    }
    const float* wrow = a.wI + (b * a.nq + tt) * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) wh[qi][r] = wrow[(r >> 2) * 8 + 4 * (l >> 5) + (r & 3)];
  }

  // query pairs: lane half G finishes query 2 p + G of pair p (one query per
  // pair when QPW = 1, upper half idle); per-lane row, visible count, validity
  constexpr int NPAIR = QPW > 1 ? QPW / 2 : 1;
  // Scores go out through a buffer resource over the block's valid query
  // rows: a lane whose key is past S, or that finishes no query, gets an
  // offset beyond the range and the hardware drops its store, so the store
  // needs no branch and the unrolled n-tile loop stays one scheduling region.
  const int64_t nrows = a.nq - t0 < QB ? a.nq - t0 : QB;
  const uint64_t sbase = EM ? 0ull : reinterpret_cast<uint64_t>(a.scores + (b * a.nq + t0) * S);
  const uint32_t sb_lo = __builtin_amdgcn_readfirstlane((uint32_t)sbase);
  const uint32_t sb_hi = __builtin_amdgcn_readfirstlane((uint32_t)(sbase >> 32));
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<float*>(((uint64_t)sb_hi << 32) | sb_lo), (short)0,
      __builtin_amdgcn_readfirstlane((int)(nrows * S * 4)), 0x00020000);
  uint32_t prow[NPAIR];              // byte offset of the lane's output row
  int pvis[NPAIR];
  bool pok[NPAIR];
  const bool hi = l >= 32;
#pragma unroll
  for (int pp = 0; pp < NPAIR; ++pp) {
    const int qa = QPW > 1 ? 2 * pp : 0, qb = QPW > 1 ? 2 * pp + 1 : 0;
    prow[pp] = (uint32_t)((wq * QPW + (hi ? qb : qa)) * S) * 4u;
    pvis[pp] = (int)(hi ? nvis[qb] : nvis[qa]);
    pok[pp] = (hi ? qvalid[qb] : qvalid[qa]) && (QPW > 1 || !hi);
  }
  // full-tile stores: the same row offsets; a lane that finishes no query
  // points past the range (which is below 2^31: nrows <= 16, S < 2^25), and
  // a query past nq has its row at or beyond nrows, also past the range
  uint32_t prow_f[NPAIR];
#pragma unroll
  for (int pp = 0; pp < NPAIR; ++pp) prow_f[pp] = (QPW > 1 || !hi) ? prow[pp] : 0x80000000u;
  const int S32 = (int)S;
  // candidate mode: per lane, the threshold of the query it finishes, the
  // start of that query's list for this key range, and (one wave per query
  // set) the list length so far; blocks whose waves share queries count in LDS
  __shared__ uint32_t s_ccnt[EM && WK > 1 ? QB : 1];
  float plk[NPAIR];
  uint32_t ccnt[NPAIR];
  uint64_t crow[NPAIR];
  if constexpr (EM) {
#pragma unroll
    for (int pp = 0; pp < NPAIR; ++pp) {
      const int qa = QPW > 1 ? 2 * pp : 0, qb = QPW > 1 ? 2 * pp + 1 : 0;
      const int64_t tq = t0 + wq * QPW + (hi ? qb : qa);
      const int64_t grow = b * a.nq + (tq < a.nq ? tq : a.nq - 1);
      plk[pp] = a.lval[grow];
      crow[pp] = ((uint64_t)grow * gridDim.y + blockIdx.y) * (uint64_t)a.cap;
      ccnt[pp] = 0;
    }
    if constexpr (WK > 1) {
      if (threadIdx.x < QB) s_ccnt[threadIdx.x] = 0;
      __syncthreads();
    }
  }

  for (int64_t tile = tile_lo; tile < tile_hi; ++tile) {
    const int64_t s0 = tile * KT;
    if (s0 >= nvis_max) {
      if constexpr (EM) continue;
      // nothing visible to any query of the block: -inf only
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi) {
        if (!qvalid[qi]) continue;
        float* orow = a.scores + (b * a.nq + t0 + wq * QPW + qi) * S;
        for (int nt = 0; nt < NTW; ++nt) {
          const int64_t s = s0 + (wk * NTW + nt) * 32 + (l & 31);
          if (l < 32 && s < S) orow[s] = -INFINITY;
        }
      }
      continue;
    }
    // ---- the key tile into LDS: stored MXFP4 bytes (Q4), else decoded to bf16
    if constexpr (Q4) {
      const int64_t s = s0 + threadIdx.x;
      const bool in = s < S;
      const int64_t kr = key_row(a, b, in ? s : 0);
      const uint8_t* cr = reinterpret_cast<const uint8_t*>(a.keys) + kr * CB;
      const uint8_t* sr = a.k_scales + kr * NBS;
#pragma unroll
      for (int i = 0; i < CB / 16; ++i) {
        u32x4 v = *reinterpret_cast<const u32x4*>(cr + 16 * i);
        if (!in) v = (u32x4){0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(Kc + threadIdx.x * LDC + 16 * i) = v;
      }
#pragma unroll
      for (int i = 0; i < NBS; ++i) Kscl[threadIdx.x * NBS + i] = in ? sr[i] : (uint8_t)0;
    } else if (KL == ROW_MXFP4) {
      constexpr int CB = CI / 2;            // code bytes per key
      constexpr int NB = CI / 32;           // scale bytes per key
      const int64_t s = s0 + threadIdx.x;
      uint32_t out[CI / 2];
      if (s < S) {
        const int64_t kr = key_row(a, b, s);
        const uint8_t* cr = reinterpret_cast<const uint8_t*>(a.keys) + kr * CB;
        const uint8_t* sr = a.k_scales + kr * NB;
#pragma unroll
        for (int blk = 0; blk < NB; ++blk) {
          const float sc = e8m0_to_f32(sr[blk]);
          const u32x4 w = *reinterpret_cast<const u32x4*>(cr + 16 * blk);
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
#pragma unroll
            for (int by = 0; by < 4; ++by) out[blk * 16 + dw * 4 + by] = fp4x2_to_bf16x2(w[dw], by, sc);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < CI / 2; ++i) out[i] = 0u;
      }
#pragma unroll
      for (int i = 0; i < CI / 8; ++i)
        *reinterpret_cast<u32x4*>(Ks + threadIdx.x * LDK + 8 * i) =
            (u32x4){out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
    } else {   // BF16 keys
      constexpr int CH = CI / 8;            // 16-byte chunks per key
      for (int i = threadIdx.x; i < KT * CH; i += 256) {
        const int kr = i / CH, cc = i % CH;
        const int64_t s = s0 + kr;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (s < S) v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.keys) + key_row(a, b, s) * CI + 8 * cc);
        *reinterpret_cast<u32x4*>(Ks + kr * LDK + 8 * cc) = v;
      }
    }
    __syncthreads();
    // ---- scores.  FULL: every key of the tile is visible to every query of
    // the block, so a store needs no per-lane test (rows of queries past nq,
    // and lanes that finish no query, lie beyond the buffer's range)
    auto ntile_loop = [&](auto fullc) {
    constexpr bool FULL = decltype(fullc)::value;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int ntile = wk * NTW + nt;
      bf16x8 kf[Q4 ? 1 : KS];
      i32x8 k4c[Q4 ? K4 : 1];
      int k4s[Q4 ? K4 : 1];
      if constexpr (Q4) {
#pragma unroll
        for (int k4 = 0; k4 < K4; ++k4) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(Kc + (ntile * 32 + (l & 31)) * LDC + 32 * k4 + 16 * (l >> 5));
          k4c[k4] = (i32x8){(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
          k4s[k4] = Kscl[(ntile * 32 + (l & 31)) * NBS + 2 * k4 + (l >> 5)];
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
          kf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(Ks + (ntile * 32 + (l & 31)) * LDK + 16 * kk + 8 * (l >> 5)));
      }
      const int64_t s = s0 + ntile * 32 + (l & 31);
      // lane half G holds heads 8 (r/4) + 4 G + r%4 of key s: partial sums
      float part[QPW];
#pragma unroll
      for (int qi = 0; qi < QPW; ++qi) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
        if constexpr (Q4) {
#pragma unroll
          for (int k4 = 0; k4 < K4; ++k4) {
            const u32x4 qc = q4c[qi][k4];
            if constexpr (QF == 8) {                  // E4M3 queries: format 0, 32 bytes per lane
              const u32x4 qh = q8h[qi][k4];
              acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  (i32x8){(int)qc[0], (int)qc[1], (int)qc[2], (int)qc[3], (int)qh[0], (int)qh[1], (int)qh[2], (int)qh[3]},
                  k4c[k4], acc, 0, 4, 0, (int)q4s[qi][k4], 0, k4s[k4]);
            } else {                                  // E2M1 queries: format 4, 16 bytes per lane
              acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  (i32x8){(int)qc[0], (int)qc[1], (int)qc[2], (int)qc[3], 0, 0, 0, 0}, k4c[k4], acc,
                  4, 4, 0, (int)q4s[qi][k4], 0, k4s[k4]);
            }
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < KS; ++kk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[qi][kk], kf[kk], acc, 0, 0, 0);
        }
        // (this file is built with IEEE mode off: the max is one instruction)
        float sc = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sc = fmaf(wh[qi][r], fmaxf(acc[r], 0.0f), sc);
        part[qi] = sc;
      }
      // queries in pairs: the lower half finishes query 2 p, the upper half
      // 2 p + 1; one v_permlane32_swap of the two partials leaves each lane
      // with its own partial of that query and its partner's (lanes l ^ 32),
      // without a trip through LDS; one 64-lane store per pair
      const int s32 = (int)s;
      auto finish_pair = [&](auto ppc) {
        constexpr int pp = decltype(ppc)::value;
        constexpr int qa = QPW > 1 ? 2 * pp : 0, qb = QPW > 1 ? 2 * pp + 1 : 0;
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[qa]), __float_as_uint(part[qb]),
                                                         false, false);
        const float total = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        if constexpr (EM) {
          // (scores are finite: the float order is the order of their keys)
          const bool keep = (FULL ? pok[pp] : (pok[pp] && s32 < pvis[pp])) && total >= plk[pp];
          const uint64_t bal = __ballot(keep);
          if (bal != 0) {
            const uint32_t lo32 = (uint32_t)bal, hi32 = (uint32_t)(bal >> 32);
            // rank among the kept lanes of the same half (the same query)
            const uint32_t below = __builtin_amdgcn_mbcnt_hi(hi32, __builtin_amdgcn_mbcnt_lo(lo32, 0u)) -
                                   (hi ? (uint32_t)__popc(lo32) : 0u);
            const uint32_t n = (uint32_t)__popc(hi ? hi32 : lo32);
            uint32_t base;
            if constexpr (WK == 1) {
              base = ccnt[pp];
              ccnt[pp] += n;
            } else {
              const int qrow = wq * QPW + (hi ? qb : qa);
              uint32_t got = 0;
              if ((l & 31) == 0 && n != 0) got = atomicAdd(&s_ccnt[qrow], n);
              base = (uint32_t)__shfl((int)got, l & 32);
            }
            const uint32_t pos = base + below;
            if (keep && pos < (uint32_t)a.cap) a.cand[crow[pp] + pos] = composite(score_key(total), (uint32_t)s32);
          }
        } else if constexpr (FULL) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(total), srsrc, (int)(prow_f[pp] + 4u * (uint32_t)s32),
                                                0, 0);
        } else {
          const uint32_t off = pok[pp] && s32 < S32 ? prow[pp] + 4u * (uint32_t)s32 : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s32 < pvis[pp] ? total : -INFINITY), srsrc,
                                                (int)off, 0, 0);
        }
      };
      finish_pair(std::integral_constant<int, 0>());
      if constexpr (NPAIR > 1) finish_pair(std::integral_constant<int, 1>());
      static_assert(NPAIR <= 2, "pairs");
    }
    };
    if (s0 + KT <= nvis_min) ntile_loop(std::true_type());
    else ntile_loop(std::false_type());
    __syncthreads();
  }
  if constexpr (EM) {
    // list lengths (the true count, also when it exceeds cap)
    if constexpr (WK == 1) {
#pragma unroll
      for (int pp = 0; pp < NPAIR; ++pp)
        if (pok[pp] && (l & 31) == 0) a.ccount[crow[pp] / (uint64_t)a.cap] = ccnt[pp];
    } else {
      if (threadIdx.x < QB && t0 + threadIdx.x < a.nq)
        a.ccount[((uint64_t)(b * a.nq + t0 + threadIdx.x)) * gridDim.y + blockIdx.y] = s_ccnt[threadIdx.x];
    }
  }
}

template <int CI, int KL, int QF, int WQ, int QPW>
static void launch_mfma_grid(const IndexerArgs& a, const PosTable& pt, int b0, int nb, hipStream_t s) {
  const IndexerGrid g = indexer_grid(a, nb);
  const dim3 grid((unsigned)(g.qblocks * nb), (unsigned)g.splits);
  if constexpr (QF == 0) {
    if (a.cand) {
      hipLaunchKernelGGL((indexer_mfma<CI, KL, WQ, QPW, 0, true>), grid, dim3(256), 0, s, a, pt, b0, (int)g.qblocks,
                         g.tps);
      return;
    }
  }
  hipLaunchKernelGGL((indexer_mfma<CI, KL, WQ, QPW, QF, false>), grid, dim3(256), 0, s, a, pt, b0, (int)g.qblocks,
                     g.tps);
}

template <int CI, int KL, int QF = 0>
static void launch_mfma_variant(const IndexerArgs& a, const PosTable& pt, int b0, int nb, hipStream_t s) {
  // four queries per wave (16 per block); two for bf16 queries at cI = 128,
  // whose query fragments alone would take 128 registers at four; single
  // queries when a sequence has fewer than 16 (indexer_grid matches these)
  if (a.nq >= 16) launch_mfma_grid<CI, KL, QF, 4, QF == 0 && CI == 128 ? 2 : 4>(a, pt, b0, nb, s);
  else launch_mfma_grid<CI, KL, QF, 1, 1>(a, pt, b0, nb, s);
}

hipError_t launch_indexer(const IndexerArgs& a, const int64_t* q_pos0, hipStream_t s) {
  if (a.nq <= 0 || a.S <= 0 || a.B <= 0) return hipSuccess;
  if (a.cand && (a.qfmt != 0 || !indexer_mfma_ok(a) || a.B > MAXB)) return hipErrorInvalidValue;
  for (int64_t b0 = 0; b0 < a.B; b0 += MAXB) {
    const int nb = (int)(a.B - b0 < MAXB ? a.B - b0 : MAXB);
    PosTable pt;
    for (int i = 0; i < nb; ++i) { pt.q_pos0[i] = q_pos0[b0 + i]; pt.win_pos0[i] = 0; }
    if (a.qfmt != 0) {
      const bool q8 = a.qfmt == 8;
      if (a.q_dtype == ACT_BF16 && a.hI == 32 && (a.cI == 64 || a.cI == 128) && a.S < ((int64_t)1 << 25)) {
        if (a.cI == 64) q8 ? launch_mfma_variant<64, ROW_MXFP4, 8>(a, pt, (int)b0, nb, s)
                           : launch_mfma_variant<64, ROW_MXFP4, 4>(a, pt, (int)b0, nb, s);
        else q8 ? launch_mfma_variant<128, ROW_MXFP4, 8>(a, pt, (int)b0, nb, s)
                : launch_mfma_variant<128, ROW_MXFP4, 4>(a, pt, (int)b0, nb, s);
      } else {
        const int64_t total = a.nq * a.S * nb;
        if (q8) hipLaunchKernelGGL(indexer_generic_qx<8>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, pt, (int)b0, nb);
        else hipLaunchKernelGGL(indexer_generic_qx<4>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, pt, (int)b0, nb);
      }
    } else if (indexer_mfma_ok(a)) {
      const bool mx = a.k_layout == ROW_MXFP4;
      switch (a.cI) {
        case 32: mx ? launch_mfma_variant<32, ROW_MXFP4>(a, pt, (int)b0, nb, s) : launch_mfma_variant<32, ROW_BF16>(a, pt, (int)b0, nb, s); break;
        case 64: mx ? launch_mfma_variant<64, ROW_MXFP4>(a, pt, (int)b0, nb, s) : launch_mfma_variant<64, ROW_BF16>(a, pt, (int)b0, nb, s); break;
        default: mx ? launch_mfma_variant<128, ROW_MXFP4>(a, pt, (int)b0, nb, s) : launch_mfma_variant<128, ROW_BF16>(a, pt, (int)b0, nb, s); break;
      }
    } else {
      const int64_t total = a.nq * a.S * nb;
      hipLaunchKernelGGL(indexer_generic, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, a, pt, (int)b0, nb);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dsv4
