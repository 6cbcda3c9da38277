// Shared-KV multi-query attention cores of CSA and HCA (DeepSeek-V4 digest,
// 模块 B eq 18-19, 模块 C eq 24-26, 模块 D sliding window and attention sink;
// jsqmd blog 第三阶段 and 2.) HCA).
//
// For query (b, t) at position p and head h, the key set is
//   sparse: { kv_comp[b, s] : s in idx[b, t] }   ++ window rows of [p-n_win+1, p]
//   dense:  { kv_comp[b, s] : m'(s+1) <= p+1 }   ++ window rows of [p-n_win+1, p]
// each key is also its value, and
//   out = sum_x e^{l_x - M} key_x / (sum_x e^{l_x - M} + e^{z'_h - M}),
//   l_x = scale * q_h . key_x,   M = max(max_x l_x, z'_h).
//
// MFMA path (bf16 queries, BF16 or FP8+bf16-RoPE rows, c in {128, 512}): see
// the comment above attn_mfma.  The running maximum is only raised when a tile
// exceeds it by 2^8 (exact after the final normalisation; bf16 P stays well
// inside range).  Short key sets with few queries are split across blocks and
// merged in a fixed order.
#include <type_traits>

#include "dsv4_common.h"
#include "dsv4_internal.h"

namespace dsv4 {

struct UnitInfo {
  int64_t t0, tl;        // first and last query of the group
  int64_t ncomp;         // compressed-entry slots
  int64_t wlo, wlen;     // window positions [wlo, wlo + wlen)
  int64_t total;
};

__device__ __forceinline__ UnitInfo unit_info(const AttnArgs& a, const AttnPlan& pl, int64_t p0, int64_t u) {
  UnitInfo ui;
  ui.t0 = u * pl.qpw;
  ui.tl = (ui.t0 + pl.qpw < a.nq ? ui.t0 + pl.qpw : a.nq) - 1;
  const int64_t pf = p0 + ui.t0, pl_ = p0 + ui.tl;
  ui.ncomp = pl.dense ? visible_count(pl_, a.ratio, a.S) : a.k;
  if (a.n_win > 0) {
    ui.wlo = pf - a.n_win + 1 > 0 ? pf - a.n_win + 1 : 0;
    ui.wlen = pl_ - ui.wlo + 1;
  } else {
    ui.wlo = 0;
    ui.wlen = 0;
  }
  ui.total = ui.ncomp + ui.wlen;
  return ui;
}

// Split partials in the workspace: {m, l} in fp32 for every (unit, split,
// row), then the unnormalised O rows in bf16, [unit][split][row][c] (half
// the bytes of fp32 rows; the merge reads every split's row, so at decode
// these bytes are of the order of the key rows themselves).
struct PartialRow {
  float* ml;
  uint16_t* o;
};
__device__ __forceinline__ PartialRow partial_row(const AttnArgs& a, const AttnPlan& pl, int64_t units, int64_t unit,
                                                  int64_t split, int64_t rows, int64_t row, int c) {
  float* mlb = reinterpret_cast<float*>(a.ws);
  uint16_t* ob = reinterpret_cast<uint16_t*>(mlb + units * pl.max_splits * rows * 2);
  const int64_t i = (unit * pl.max_splits + split) * rows + row;
  return {mlb + i * 2, ob + i * c};
}

// bf16 of 4 partial channels at dst (8-byte aligned)
__device__ __forceinline__ void store_partial4(uint16_t* dst, float v0, float v1, float v2, float v3) {
  *reinterpret_cast<u32x2*>(dst) = (u32x2){pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
}

// row of key slot `slot` (null if padding); *pos = entry index or position,
// *win = window row
__device__ __forceinline__ const uint8_t* slot_row(const AttnArgs& a, int64_t b, int64_t t, const UnitInfo& ui,
                                                   int64_t wpos0, int64_t slot, int rb, int64_t* pos, bool* win) {
  if (slot < ui.ncomp) {
    *win = false;
    int64_t s = slot;
    if (a.idx) s = a.idx[(b * a.nq + t) * a.k + slot];
    *pos = s;
    if (s < 0 || s >= a.S) { *pos = -1; return nullptr; }
    return reinterpret_cast<const uint8_t*>(a.kv_comp) + (b * a.S + s) * (int64_t)rb;
  }
  *win = true;
  const int64_t u = ui.wlo + (slot - ui.ncomp);
  *pos = u;
  return reinterpret_cast<const uint8_t*>(a.kv_win) + (b * a.W + (u - wpos0)) * (int64_t)rb;
}

__device__ __forceinline__ bool slot_visible(bool win, int64_t pos, int64_t p, int64_t nvis, int n_win) {
  if (win) return pos <= p && pos >= p - n_win + 1;
  return pos >= 0 && pos < nvis;
}

// ------------------------------------------------------------------ output rotation in the store
// (DeepSeek-V4 digest, 模块 D: the output's RoPE dims are rotated back by the
// query's position.)  The result is what storing the output and then rotating
// the stored row gives: a bf16 output is rounded to bf16 first, the pair is
// rotated in fp32 by rope_pair and rounded again.  Pairs are whole within
// any 4 aligned channels (c and the rotated width are multiples of 8).

// cos / sin of the rotation of nqb queries from position pfirst on: pair j of
// query q at tcs / tsn[q * R / 2 + j] (block-wide)
__device__ __forceinline__ void out_rot_table(float* tcs, float* tsn, int nqb, int64_t pfirst, int R, float theta) {
  const int np = R >> 1;
  for (int i = threadIdx.x; i < nqb * np; i += blockDim.x)
    rope_cs(-(pfirst + i / np), i % np, R, theta, &tcs[i], &tsn[i]);
}

__device__ __forceinline__ float bf16_round(float x) {
  return __builtin_bit_cast(float, (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x) << 16);
}

// bf16 store of channels e0 .. e0 + 3 (e0 % 4 == 0) of a row; rotated when
// they lie in the last R channels (cs / sn: the row's query's table)
__device__ __forceinline__ void store4_bf16_rot(uint16_t* dst, float v0, float v1, float v2, float v3, int e0, int c,
                                                int R, const float* cs, const float* sn) {
  if (R > 0 && e0 >= c - R) {
    float x0 = bf16_round(v0), x1 = bf16_round(v1), x2 = bf16_round(v2), x3 = bf16_round(v3);
    const int j = (e0 - (c - R)) >> 1;
    rope_pair(x0, x1, cs[j], sn[j]);
    rope_pair(x2, x3, cs[j + 1], sn[j + 1]);
    *reinterpret_cast<u32x2*>(dst) = (u32x2){pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
  } else {
    *reinterpret_cast<u32x2*>(dst) = (u32x2){__builtin_bit_cast(uint32_t, (bf16x2){(__bf16)v0, (__bf16)v1}),
                                             __builtin_bit_cast(uint32_t, (bf16x2){(__bf16)v2, (__bf16)v3})};
  }
}

// ------------------------------------------------------------------ generic (fp32 math)
// one block of 256 threads per (b, t, h); keys in chunks of 256 with an online softmax
__global__ __launch_bounds__(256) void attn_generic(AttnArgs a, PosTable pt, int b0, AttnPlan pl) {
  __shared__ float qs[1024];
  __shared__ float L[256];
  __shared__ const uint8_t* rows[256];
  __shared__ float red[8];
  const int64_t gid = blockIdx.x;
  const int64_t bl = gid / (a.nq * a.nh);
  const int64_t t = (gid / a.nh) % a.nq;
  const int h = (int)(gid % a.nh);
  const int64_t b = b0 + bl;
  const int c = a.c;
  const int rb = row_bytes(a.kv_layout, c);
  const int64_t p = pt.q_pos0[bl] + t;
  AttnPlan one = pl;
  one.qpw = 1;
  const UnitInfo ui = unit_info(a, one, pt.q_pos0[bl], t);
  const int64_t nvis = pl.dense ? visible_count(p, a.ratio, a.S) : a.S;
  const int64_t qbase = ((b * a.nq + t) * a.nh + h) * c;
  for (int j = threadIdx.x; j < c; j += 256) qs[j] = load_act(a.q, a.q_dtype, qbase + j);
  float o[4] = {0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  __syncthreads();
  for (int64_t s0 = 0; s0 < ui.total; s0 += 256) {
    const int64_t slot = s0 + threadIdx.x;
    float lg = -INFINITY;
    const uint8_t* row = nullptr;
    if (slot < ui.total) {
      int64_t pos;
      bool win;
      row = slot_row(a, b, t, ui, pt.win_pos0[bl], slot, rb, &pos, &win);
      if (row && slot_visible(win, pos, p, nvis, a.n_win)) {
        float d = 0.f;
        for (int j = 0; j < c; ++j) d = fmaf(qs[j], load_row_elem(row, a.kv_layout, c, j), d);
        lg = d * a.scale;
      } else {
        row = nullptr;
      }
    }
    rows[threadIdx.x] = row;
    float mx = wave_max(lg);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
    const float pv = (lg == -INFINITY) ? 0.f : __expf(lg - m_new);
    L[threadIdx.x] = pv;
    float sm = wave_sum(pv);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[4 + (threadIdx.x >> 6)] = sm;
    __syncthreads();
    sm = (red[4] + red[5]) + (red[6] + red[7]);
    l_run = l_run * alpha + sm;
    m_run = m_new;
    const int nslots = (int)(ui.total - s0 < 256 ? ui.total - s0 : 256);
    for (int jj = 0; jj < 4; ++jj) {
      const int j = threadIdx.x + 256 * jj;
      if (j >= c) break;
      float acc = o[jj] * alpha;
      for (int x = 0; x < nslots; ++x)
        if (rows[x]) acc = fmaf(L[x], load_row_elem(rows[x], a.kv_layout, c, j), acc);
      o[jj] = acc;
    }
    __syncthreads();
  }
  float den = l_run, f = 1.0f;
  if (a.sink) {
    const float z = a.sink[h];
    const float M = fmaxf(m_run, z);
    f = m_run == -INFINITY ? 0.f : __expf(m_run - M);
    den = l_run * f + __expf(z - M);
  }
  const float inv = den > 0.f ? f / den : 0.f;
  const int R = a.rot_dims;
  for (int jj = 0; jj < 4; ++jj) {
    const int j = threadIdx.x + 256 * jj;
    float v = j < c ? o[jj] * inv : 0.f;
    if (R > 0) {                          // pairs (j, j ^ 1): neighbouring lanes of one wave
      if (a.q_dtype == ACT_BF16) v = bf16_round(v);
      const float pv = __shfl_xor(v, 1);
      if (j < c && j >= c - R) {
        float cs, sn;
        rope_cs(-(pt.q_pos0[bl] + t), (j - (c - R)) >> 1, R, a.rot_theta, &cs, &sn);
        float x0 = (j & 1) ? pv : v, x1 = (j & 1) ? v : pv;
        rope_pair(x0, x1, cs, sn);
        v = (j & 1) ? x1 : x0;
      }
    }
    if (j < c) store_act(a.out, a.q_dtype, qbase + j, v);
  }
}

// ------------------------------------------------------------------ MFMA path
// Rows are (query, head) pairs.  A block owns R = 32*NRG rows (one query for
// the sparse core; queries that share their keys for the dense core) and
// streams its key slots in tiles of 32:
//   * the raw stored rows of a tile are copied global -> LDS with
//     global_load_lds_dwordx4 two tiles ahead (double-buffered stage, no
//     registers held while the copies are in flight);
//   * the stage is decoded once into a bf16 key tile [32][c] whose 16-byte
//     chunks are XOR-swizzled by row, so that both the row reads of S^T and
//     the transposed reads of V^T are free of bank conflicts;
//   * wave (rg, ch) owns the 32 rows of row group rg and channel slice ch: it
//     keeps Q^T and O^T of that slice in registers, computes the partial
//     S^T = K Q^T with v_mfma_f32_32x32x16_bf16 and adds the partner slice's
//     partial through LDS; each lane then owns the logits of one row for half
//     of the tile's keys (the other half is in lane ^ 32);
//   * O^T += V^T P^T takes its V^T operand straight from the row-major key
//     tile with ds_read_b64_tr_b16 (K = V).
constexpr int TS = 32;           // key slots per tile

// A zero row (at least as long as any stored row, 2 c bytes at c = 512):
// padding key slots are copied from it, so their keys and values are exactly
// zero (their logits are masked; a zero value keeps P = 0 from meeting a
// non-finite byte pattern in PV).  Read-only; zero-initialised at load.
__device__ __align__(16) uint8_t g_zero_row[1024];
constexpr int SIDX_CAP = ATTN_SIDX_CAP;   // index-list slots a sparse block caches in LDS

// The copies of one wave for one tile: copy q = wv + NW i (q < NDMA) takes
// bytes 32 q + 16 G of each lane's row (offset 32 NW i from `base`, which
// already holds 32 wv + 16 G) into stage bytes [1024 q, 1024 q + 1024).
template <int I, int N, int NW, int NDMA>
struct DmaCopies {
  __device__ __forceinline__ static void run(const uint8_t* base, uint32_t lds0, int wv) {
    if (NW * (I + 1) <= NDMA || wv + NW * I < NDMA) dma16<32 * NW * I>(base, lds0 + 1024 * NW * I);
    DmaCopies<I + 1, N, NW, NDMA>::run(base, lds0, wv);
  }
};
template <int N, int NW, int NDMA>
struct DmaCopies<N, N, NW, NDMA> {
  __device__ __forceinline__ static void run(const uint8_t*, uint32_t, int) {}
};

// Barrier for LDS traffic only: waits for this wave's LDS operations, not for
// the global->LDS copies still in flight (their completion is waited for
// explicitly with vmcnt before the stage is read).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
}

// Layout of the bf16 key tile: rows of C + 16 elements (a stride of 32 bytes
// mod 128), and 16-byte chunk j of row r stored at chunk j ^ ksw(r) with
// ksw(r) = (r >> 2) & 3.  Eight consecutive rows then cover 8 distinct
// 16-byte bank groups (row reads of S^T, the decode writes), and 4 consecutive
// rows x 32 bytes cover all 32 banks (transposed reads of V^T).  The XOR only
// touches the two low chunk bits, so every loop-varying part of an address is
// an immediate offset.
constexpr int KPAD = 16;
template <int V> struct Par { static constexpr int value = V; };   // a buffer parity known at compile time
__device__ __forceinline__ int ksw(int r) { return (r >> 2) & 3; }

template <int C, int KVL, int CS, int NRG>
struct AttnCfg {
  static constexpr int NW = NRG * CS;
  static constexpr int NT = 64 * NW;
  static constexpr int R = 32 * NRG;
  static constexpr int CH = C / CS;                 // channels per wave
  static constexpr int KQ = CH / 16;                // S^T k-steps per wave
  static constexpr int MO = CH / 32;                // O^T m-tiles per wave
  static constexpr int RB = KVL == ROW_FP8 ? C + ROPE_DIMS : 2 * C;   // stored row bytes
  static constexpr int NP = RB / 16;                // 16-byte pieces per stored row
  static constexpr int NF8 = KVL == ROW_FP8 ? (C - ROPE_DIMS) / 16 : 0;   // fp8 pieces (16 channels each)
  static constexpr int NDMA = TS * NP / 64;         // wave copies per tile
  static constexpr int STAGE = TS * RB;             // bytes per stage buffer
};

template <int C, int KVL, int CS, int NRG>
__global__ __launch_bounds__(64 * NRG * CS)
__attribute__((amdgpu_waves_per_eu(C >= 512 ? 1 : 2, C >= 512 ? 1 : 2)))
void attn_mfma(AttnArgs a, PosTable pt, int b0, AttnPlan pl) {
  using Cf = AttnCfg<C, KVL, CS, NRG>;
  constexpr int KQ = Cf::KQ, MO = Cf::MO, CH = Cf::CH, NP = Cf::NP, RB = Cf::RB;
  constexpr int KT = TS * (C + KPAD);     // elements of one key tile
  // two stage buffers (raw rows, piece-major: [piece][slot][16 B]) and three
  // bf16 key tiles (chunk-swizzled); tile t lives in key tile t % 3, chosen at
  // compile time (separate objects: addresses fold into the LDS instructions
  // and alias analysis keeps the tiles apart)
  constexpr int HK = CS > 1 ? 8 : 16;     // score registers a wave keeps per tile: its key half
  __shared__ __align__(16) uint8_t s_stage[2 * Cf::STAGE];
  __shared__ __align__(16) uint16_t s_K0[KT];
  __shared__ __align__(16) uint16_t s_K1[KT];
  __shared__ __align__(16) uint16_t s_K2[KT];
  // exchange within a channel pair: the partner's half of the partial scores,
  // this wave's half of P (bf16 pairs), its per-row half maximum
  __shared__ __align__(16) float s_xs[CS > 1 ? Cf::NW * 2 * 64 * 4 : 4];   // [wave][r/4][lane][4]
  __shared__ __align__(16) uint32_t s_xp[CS > 1 ? Cf::NW * 64 * 4 : 4];   // [wave][lane][4]
  __shared__ float s_xm[CS > 1 ? Cf::NW * 64 : 1];                        // [wave][lane]
  __shared__ uint32_t s_vmask[3][8];                         // per key tile and query: visible slots
  __shared__ int s_nvisq[8];
  __shared__ int s_sidx[SIDX_CAP];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int l = threadIdx.x & 63, G = l >> 5, col = l & 31;
  const int rg = wv / CS, ch = wv % CS;
  const int64_t bl = blockIdx.x / pl.units_per_b, u = blockIdx.x % pl.units_per_b;
  const int64_t b = b0 + bl;
  const int64_t p0 = pt.q_pos0[bl], wpos0 = pt.win_pos0[bl];
  const UnitInfo ui = unit_info(a, pl, p0, u);
  const int64_t nsplit = pl.max_splits == 1 ? 1 : (ui.total + pl.chunk - 1) / pl.chunk;
  const int split = blockIdx.y;
  if (split > 0 && split >= nsplit) return;
  const int slot_lo = split * pl.chunk;
  const int slot_hi = (int)(pl.max_splits == 1 ? ui.total : (slot_lo + pl.chunk < ui.total ? slot_lo + pl.chunk : ui.total));
  const int ncomp = (int)ui.ncomp;
  const uint8_t* comp_base = reinterpret_cast<const uint8_t*>(a.kv_comp) + b * a.S * (int64_t)RB;
  const uint8_t* win_base = reinterpret_cast<const uint8_t*>(a.kv_win) + (b * a.W + (ui.wlo - wpos0)) * (int64_t)RB;
  static_assert(Cf::RB <= (int)sizeof(g_zero_row), "zero row shorter than a stored row");
  const uint8_t* dummy = g_zero_row;                                 // padding slots
  const int nq_blk = (int)(ui.tl - ui.t0 + 1);
  const int pfirst = (int)(p0 + ui.t0);
  const int ntiles = slot_hi > slot_lo ? (slot_hi - slot_lo + TS - 1) / TS : 0;

  // block-level tables: visible compressed entries per query, cached index list
  if (threadIdx.x < 8) s_nvisq[threadIdx.x] = pl.dense ? (int)visible_count(pfirst + threadIdx.x, a.ratio, a.S) : (int)a.S;
  int bad_idx = 0;      // an index outside [0, S) in this block's list
  if (a.idx) {
    const int32_t* irow = a.idx + (b * a.nq + ui.t0) * a.k;
    const int n_i = (ncomp < slot_hi ? ncomp : slot_hi) - slot_lo;
    for (int i = threadIdx.x; i < n_i; i += Cf::NT) {
      const int e = irow[slot_lo + i];
      s_sidx[i] = e;
      bad_idx |= (e < 0 || e >= a.S) ? 1 : 0;
    }
  }
  const bool idx_ok = !__syncthreads_or(bad_idx);
  const int plast = (int)(p0 + ui.tl);
  const int nvis_first = pl.dense ? (int)visible_count(pfirst, a.ratio, a.S) : (int)a.S;

  // the row this lane owns: (query t, head h)
  const int row = 32 * rg + col;
  const int qloc = row / a.nh;
  const int h = row % a.nh;
  const int64_t t = ui.t0 + qloc;
  const bool qvalid = t <= ui.tl;
  const int64_t tq = qvalid ? t : ui.tl;

  bf16x8 qf[KQ];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((b * a.nq + tq) * a.nh + h) * C + ch * CH;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * G));
    // land the query fragments before the tile copies start: a later wait for
    // them would also wait for every copy issued after them
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  }
  f32x16 acc[MO];
#pragma unroll
  for (int i = 0; i < MO; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl = pl.scale_log2;     // > 0

  // stored row of slot s, or nullptr for padding; *pos, *win describe it
  auto slot_src = [&](int s, int* pos, bool* win) -> const uint8_t* {
    if (s < ncomp) {
      *win = false;
      const int e = a.idx ? s_sidx[s - slot_lo] : s;
      *pos = e;
      if (e < 0 || e >= a.S) return nullptr;
      return comp_base + (int64_t)e * RB;
    }
    *win = true;
    *pos = (int)ui.wlo + (s - ncomp);
    return win_base + (int64_t)(s - ncomp) * RB;
  };

  // copies of tile `it` into a stage buffer.  Stage piece P = piece * TS +
  // slot and wave copy q covers P in [64 q, 64 q + 64): lane l always serves
  // slot s0 + l % 32 (piece 2 q + l / 32), so its row address is found once
  // per tile and the copies differ by immediate offsets.  Padding slots copy
  // the zero row.
  auto issue = [&](int it, uint8_t* stg) {
    const int slot = slot_lo + it * TS + (l & 31);
    int pos;
    bool win;
    const uint8_t* row = slot < slot_hi ? slot_src(slot, &pos, &win) : nullptr;
    const uint8_t* base = (row ? row : dummy) + 16 * G + 32 * wv;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)(stg + wv * 1024));
    DmaCopies<0, (Cf::NDMA + Cf::NW - 1) / Cf::NW, Cf::NW, Cf::NDMA>::run(base, lds0, wv);
  };
  // copies per wave and tile: waves below NDMA % NW issue one more
  const int my_dma = Cf::NDMA / Cf::NW + (wv < Cf::NDMA % Cf::NW ? 1 : 0);
  // wait until at most n of this wave's tile copies are still in flight
  auto wait_copies = [&](int n) {
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;   // vmcnt(0)
      case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
      case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
      case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
      case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
      case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
      case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
      case 7: __builtin_amdgcn_s_waitcnt(0x0F77); break;
      case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
      case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
      case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
      case 11: __builtin_amdgcn_s_waitcnt(0x0F7B); break;
      case 12: __builtin_amdgcn_s_waitcnt(0x0F7C); break;
      default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
  };

  // Is every slot of tile `it` visible to every query of the block?  Scalar
  // arithmetic: the first query sees the fewest compressed entries, the first
  // query's position bounds the window from above and the last query's window
  // start bounds it from below; an index list is all visible when every
  // entry lies in [0, S).
  auto tile_full = [&](int it) -> bool {
    const int s0 = slot_lo + it * TS, s1 = s0 + TS;
    if (s1 > slot_hi) return false;
    if (s0 < ncomp) {
      if (a.idx ? !idx_ok : (s1 < ncomp ? s1 : ncomp) > nvis_first) return false;
    }
    if (s1 > ncomp) {
      const int lo = (int)ui.wlo + ((s0 > ncomp ? s0 : ncomp) - ncomp), hi = (int)ui.wlo + (s1 - 1 - ncomp);
      if (hi > pfirst || lo < plast - a.n_win + 1) return false;
    }
    return true;
  };
  // per-query visibility bits of a tile that is not full (wave 0)
  auto masks = [&](int it, int buf) {
    if (wv != 0 || tile_full(it)) return;
    const int s0 = slot_lo + it * TS;
    uint32_t vbits = 0;
    const int slot = s0 + l;
    if (l < TS && slot < slot_hi) {
      int pos;
      bool win;
      if (slot_src(slot, &pos, &win)) {
        for (int q = 0; q < nq_blk; ++q) {
          const int pq = pfirst + q;
          const bool ok = win ? (pos <= pq && pos >= pq - a.n_win + 1) : (pos < s_nvisq[q]);
          vbits |= (ok ? 1u : 0u) << q;
        }
      }
    }
    for (int q = 0; q < nq_blk; ++q) {
      const uint32_t bal = (uint32_t)__ballot((vbits >> q) & 1u);
      if (l == 0) s_vmask[buf][q] = bal;
    }
  };

  // Decode of a stage into a bf16 key tile, as a load step and a convert-and-
  // store step, both free of branches.  Stage unit un (16 bytes) is piece
  // un / TS of slot un % TS, E4M3 units first.  Each thread takes F8 whole
  // E4M3 units, then (when the E4M3 units leave half a round) half of one
  // more E4M3 unit, then FB bf16 units.
  constexpr int U8 = Cf::NF8 * TS, UB = (NP - Cf::NF8) * TS;
  constexpr int F8 = U8 / Cf::NT, R8 = U8 % Cf::NT, FB = UB / Cf::NT;
  static_assert((R8 == 0 || 2 * R8 == Cf::NT) && UB % Cf::NT == 0, "decode work splits evenly");
  constexpr bool HALF = R8 != 0;
  struct DecRegs {
    u32x4 w8[F8 > 0 ? F8 : 1];
    u32x2 wh;
    u32x4 wb[FB > 0 ? FB : 1];
  };
  const int tid = threadIdx.x;
  auto dec_load = [&](const uint8_t* stg) -> DecRegs {
    DecRegs d;
#pragma unroll
    for (int j = 0; j < F8; ++j) d.w8[j] = *reinterpret_cast<const u32x4*>(stg + (tid + Cf::NT * j) * 16);
    if constexpr (HALF) d.wh = *reinterpret_cast<const u32x2*>(stg + (F8 * Cf::NT + (tid >> 1)) * 16 + 8 * (tid & 1));
#pragma unroll
    for (int j = 0; j < FB; ++j) d.wb[j] = *reinterpret_cast<const u32x4*>(stg + (U8 + tid + Cf::NT * j) * 16);
    return d;
  };
  // 8 E4M3 bytes -> one 16-byte bf16 chunk
  auto e4m3x8 = [](u32x2 w) -> u32x4 {
    return (u32x4){e4m3x2_to_bf16x2(w[0], false), e4m3x2_to_bf16x2(w[0], true),
                   e4m3x2_to_bf16x2(w[1], false), e4m3x2_to_bf16x2(w[1], true)};
  };
  auto dec_store = [&](const DecRegs& d, uint16_t* kt) {
#pragma unroll
    for (int j = 0; j < F8; ++j) {               // 16 E4M3 channels -> chunks 2 piece, 2 piece + 1
      const int un = tid + Cf::NT * j, piece = un / TS, ks = un % TS;
      uint16_t* krow = kt + ks * (C + KPAD);
      *reinterpret_cast<u32x4*>(krow + 8 * ((2 * piece) ^ ksw(ks))) = e4m3x8((u32x2){d.w8[j][0], d.w8[j][1]});
      *reinterpret_cast<u32x4*>(krow + 8 * ((2 * piece + 1) ^ ksw(ks))) = e4m3x8((u32x2){d.w8[j][2], d.w8[j][3]});
    }
    if constexpr (HALF) {                        // 8 E4M3 channels -> chunk 2 piece + half
      const int un = F8 * Cf::NT + (tid >> 1), piece = un / TS, ks = un % TS;
      *reinterpret_cast<u32x4*>(kt + ks * (C + KPAD) + 8 * ((2 * piece + (tid & 1)) ^ ksw(ks))) = e4m3x8(d.wh);
    }
#pragma unroll
    for (int j = 0; j < FB; ++j) {               // 8 bf16 channels -> one chunk
      const int un = U8 + tid + Cf::NT * j, piece = un / TS, ks = un % TS;
      const int chunk = 2 * Cf::NF8 + (piece - Cf::NF8);
      *reinterpret_cast<u32x4*>(kt + ks * (C + KPAD) + 8 * (chunk ^ ksw(ks))) = d.wb[j];
    }
  };
  auto decode = [&](const uint8_t* stg, uint16_t* kt) { dec_store(dec_load(stg), kt); };

  auto ktile = [&](auto kbc) -> uint16_t* {
    constexpr int KB = decltype(kbc)::value;
    if constexpr (KB == 0) return s_K0;
    else if constexpr (KB == 1) return s_K1;
    else return s_K2;
  };
  // ---- pieces of the pipeline
  // partial S^T[32 keys][32 rows] of the tile in key tile KB over this wave's
  // channel slice: register r holds key slot 8 (r/4) + 4 G + r%4 of row col
  auto score_tile = [&](auto kbc) -> f32x16 {
    const uint16_t* kt = ktile(kbc);
    f32x16 s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) { s0[r] = 0.f; s1[r] = 0.f; }
    // logical chunk of k-step kk: ch*CH/8 + 2 kk + G; only its two low bits
    // meet the swizzle, so even and odd kk each get one base address
    const uint16_t* krow = kt + col * (C + KPAD);
    const int x0 = ch * (CH / 8) + G;
    const uint16_t* kb0 = krow + 8 * (x0 ^ ksw(col));
    const uint16_t* kb1 = krow + 8 * ((x0 + 2) ^ ksw(col));
#pragma unroll
    for (int kk = 0; kk < KQ; kk += 2) {
      const int hop = 8 * 4 * (kk >> 1);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(kb0 + hop)), qf[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(*reinterpret_cast<const u32x4*>(kb1 + hop)), qf[kk + 1], s1, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] += s1[r];
    return s0;
  };
  const int partner = wv ^ 1;                       // CS == 2: the wave with the other channel half
  // the partner's key half of a partial S^T goes to LDS
  auto put_partial = [&](const f32x16& sp) {
    const bool lo = ch != 0;                        // partner owns keys 0..15 (registers 0..7)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
      *reinterpret_cast<f32x4*>(s_xs + ((wv * 2 + rr) * 64 + l) * 4) =
          (f32x4){lo ? sp[4 * rr] : sp[8 + 4 * rr], lo ? sp[4 * rr + 1] : sp[8 + 4 * rr + 1],
                  lo ? sp[4 * rr + 2] : sp[8 + 4 * rr + 2], lo ? sp[4 * rr + 3] : sp[8 + 4 * rr + 3]};
  };
  // this wave's key half of the full scores: own registers 8 ch .. 8 ch + 7 plus the partner's
  auto take_half = [&](const f32x16& sp, float (&hn)[HK]) {
    if constexpr (CS > 1) {
      const bool hi = ch != 0;
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        const f32x4 o = *reinterpret_cast<const f32x4*>(s_xs + ((partner * 2 + rr) * 64 + l) * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) hn[4 * rr + j] = (hi ? sp[8 + 4 * rr + j] : sp[4 * rr + j]) + o[j];
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) hn[r] = sp[r];
    }
  };
  // mask a tile's half scores (tiles not seen whole by every query) and
  // return this lane's row maximum over the half (both lane halves)
  auto mask_max = [&](int t, int kbuf, float (&hn)[HK]) -> float {
    if (!tile_full(t)) {
      const uint32_t m16 = (s_vmask[kbuf][qloc] >> (4 * G)) & 0x0F0F0F0Fu;
      const uint32_t mh = CS > 1 ? m16 >> (16 * ch) : m16;
#pragma unroll
      for (int i = 0; i < HK; ++i) hn[i] = ((mh >> (8 * (i >> 2) + (i & 3))) & 1u) ? hn[i] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < HK; ++i) mx = fmaxf(mx, hn[i]);
    return max_halves(mx);
  };

  // PV of the tile in key tile KB: O^T[c][row] += V^T[c][keys] P^T[keys][row].
  // MFMA over key half s covers slots [16s + 4G, +4) and [16s + 8 + 4G, +4);
  // each half of its A operand comes from one transposed read: lane (lambda =
  // l % 16) of a 16-lane group addresses key row key0 + lambda/4, channels
  // c0 + 4 (lambda % 4) .. + 4, and receives channel c0 + lambda of keys
  // key0 .. key0 + 3.  Key rows 16 s + 8 hf + 4 G + lambda/4 have the swizzle
  // (2 hf + G) & 3 for either s, so a half only moves the base by 16 rows.
  typedef short v4s __attribute__((ext_vector_type(4)));
  const int lam = l & 15, grp = (l >> 4) & 1;
  const int e8 = (ch * CH + 16 * grp + 4 * (lam & 3)) >> 2;            // 8-byte chunk for mo = 0
  const int rowl = 4 * G + (lam >> 2);
  const int tb0 = rowl * (C + KPAD) + 8 * ((e8 >> 1) ^ ((0 + G) & 3)) + 4 * (e8 & 1);
  const int tb1 = (rowl + 8) * (C + KPAD) + 8 * ((e8 >> 1) ^ ((2 + G) & 3)) + 4 * (e8 & 1);
  auto pv_half = [&](const uint16_t* kt, int half, const bf16x8& pf) {
    const uint16_t* t0p = kt + 16 * half * (C + KPAD) + tb0;
    const uint16_t* t1p = kt + 16 * half * (C + KPAD) + tb1;
#pragma unroll
    for (int mo = 0; mo < MO; ++mo) {
      const v4s t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(t0p + 32 * mo));
      const v4s t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(t1p + 32 * mo));
      const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
      acc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8((u32x4){w0[0], w0[1], w1[0], w1[1]}), pf,
                                                        acc[mo], 0, 0, 0);
    }
  };

  // Software pipeline, two block barriers per tile.  Iteration it (tile it's
  // scores of this wave's key half, hc, and its row maximum are in registers):
  //   copies of tile it+3 go out (into the stage tile it+1 was decoded from);
  //   P of tile it, next to the S^T MFMAs of tile it+1;
  //   partner exchange of partial scores (tile it+1) and P (tile it);
  //   [wait for this wave's copies of tile it+2]  B_a;
  //   scores of tile it+1 completed, masked, half maximum published;
  //   PV of tile it, next to the decode of tile it+2 (key tile (it+2) % 3,
  //   last read by PV of tile it-1);  B_b.
  // The running maximum is raised only when a row's tile maximum passes it by
  // more than 8 (log2 units); that rescale sits outside the inner loop, which
  // keeps the O^T accumulator in place.
  float hc[HK];
#pragma unroll
  for (int i = 0; i < HK; ++i) hc[i] = -INFINITY;
  float hmc = -INFINITY, tmax = -INFINITY;
  auto check = [&]() -> bool {
    const float pm = CS > 1 ? s_xm[partner * 64 + l] : -INFINITY;
    tmax = fmaxf(hmc, pm) * sl;
    return __builtin_amdgcn_ballot_w64(tmax > m_run + 8.0f) != 0;
  };
  auto raise_max = [&]() {
    float alpha = 1.f;
    if (tmax > m_run + 8.0f) {
      alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - tmax);
      m_run = tmax;
    }
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < MO; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
  };
  // The two overlapped stretches (P of tile it with the S^T MFMAs of tile it+1;
  // PV of tile it with the decode of tile it+2) are branch-free so that the
  // scheduler can interleave them: past the last tile they run on key tiles
  // and stages nobody reads again.
  auto finish = [&](auto kbc, int it) {
    constexpr int KB = decltype(kbc)::value;
    const Par<(KB + 1) % 3> kb1;
    const Par<(KB + 2) % 3> kb2;
    if (it + 3 < ntiles) issue(it + 3, s_stage + ((it + 1) & 1) * Cf::STAGE);
    // P of tile it over this wave's key half; l accumulates over it
    const float mneg = m_run == -INFINITY ? 0.f : -m_run;
    uint32_t pk[HK / 2];
#pragma unroll
    for (int i = 0; i < HK; i += 2) {
      // v_exp_f32 directly: results below 2^-126 flush to zero, which leaves
      // the normalised output unchanged at fp32 resolution
      const float e0 = __builtin_amdgcn_exp2f(fmaf(hc[i], sl, mneg));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(hc[i + 1], sl, mneg));
      l_run += e0 + e1;
      pk[i >> 1] = __builtin_bit_cast(uint32_t, (bf16x2){(__bf16)e0, (__bf16)e1});
    }
    const f32x16 sn = score_tile(kb1);
    if constexpr (CS > 1) {
      put_partial(sn);
      *reinterpret_cast<u32x4*>(s_xp + (wv * 64 + l) * 4) = (u32x4){pk[0], pk[1], pk[2], pk[3]};
    }
    // this wave's copies of tile it+2 have landed once at most those of it+3 remain
    wait_copies(it + 3 < ntiles ? my_dma : 0);
    lds_barrier();                                                    // B_a
    const DecRegs dr = dec_load(s_stage + (it & 1) * Cf::STAGE);     // tile it+2
    float hn[HK];
    take_half(sn, hn);
    const float hmn = mask_max(it + 1, (KB + 1) % 3, hn);
    if constexpr (CS > 1) s_xm[wv * 64 + l] = hmn;
    const uint16_t* kt = ktile(kbc);
    if constexpr (CS > 1) {
      const u32x4 pp = *reinterpret_cast<const u32x4*>(s_xp + (partner * 64 + l) * 4);
      pv_half(kt, ch, as_bf16x8((u32x4){pk[0], pk[1], pk[2], pk[3]}));
      pv_half(kt, ch ^ 1, as_bf16x8(pp));
    } else {
      pv_half(kt, 0, as_bf16x8((u32x4){pk[0], pk[1], pk[2], pk[3]}));
      pv_half(kt, 1, as_bf16x8((u32x4){pk[4], pk[5], pk[6], pk[7]}));
    }
    dec_store(dr, ktile(kb2));
    masks(it + 2, (KB + 2) % 3);
    lds_barrier();                                                    // B_b
#pragma unroll
    for (int i = 0; i < HK; ++i) hc[i] = hn[i];
    hmc = hmn;
  };

  // prologue: tiles 0 and 1 decoded, tile 2 in flight, scores of tile 0 ready
  if (ntiles > 0) {
    issue(0, s_stage);
    if (ntiles > 1) issue(1, s_stage + Cf::STAGE);
    wait_copies(ntiles > 1 ? my_dma : 0);
    lds_barrier();                                   // copies of tile 0 visible
    decode(s_stage, s_K0);
    masks(0, 0);
    wait_copies(0);
    lds_barrier();                                   // key tile 0 complete, copies of tile 1 visible
    if (ntiles > 2) issue(2, s_stage);
    if (ntiles > 1) {
      decode(s_stage + Cf::STAGE, s_K1);
      masks(1, 1);
    }
    const f32x16 s0v = score_tile(Par<0>());
    if constexpr (CS > 1) put_partial(s0v);
    lds_barrier();                                   // partials of tile 0, key tile 1 complete
    take_half(s0v, hc);
    hmc = mask_max(0, 0, hc);
    if constexpr (CS > 1) s_xm[wv * 64 + l] = hmc;
    lds_barrier();                                   // half maxima of tile 0
  }
  // inner loop unrolled by three (key tile it % 3 known at compile time); it
  // resumes at any phase after a rescale
  for (int it = 0; it < ntiles;) {
    bool up = false;
    for (;;) {
      const int ph = it % 3;
      if (ph == 0) {
        up = check();
        if (up) break;
        finish(Par<0>(), it);
        if (++it >= ntiles) break;
      }
      if (ph <= 1) {
        up = check();
        if (up) break;
        finish(Par<1>(), it);
        if (++it >= ntiles) break;
      }
      up = check();
      if (up) break;
      finish(Par<2>(), it);
      if (++it >= ntiles) break;
    }
    if (up) {
      raise_max();
      switch (it % 3) {
        case 0: finish(Par<0>(), it); break;
        case 1: finish(Par<1>(), it); break;
        default: finish(Par<2>(), it); break;
      }
      ++it;
    }
  }

  l_run = sum_halves(l_run);
  if constexpr (CS > 1) {            // each wave of a pair summed P over its own key half
    s_xm[wv * 64 + l] = l_run;
    lds_barrier();
    l_run += s_xm[partner * 64 + l];
  }
  // output rotation table in the stage (every wave is done with it)
  const int R = pl.max_splits == 1 ? a.rot_dims : 0;
  float* tcs = reinterpret_cast<float*>(s_stage);
  float* tsn = tcs + nq_blk * (R >> 1);
  if (R > 0) {
    lds_barrier();
    out_rot_table(tcs, tsn, nq_blk, pfirst, R, a.rot_theta);
    lds_barrier();
  }
  if (!qvalid) return;
  // register r of m-tile mo holds channel ch*CH + 32 mo + 8 (r/4) + 4 G + r%4 of this lane's row
  if (pl.max_splits == 1) {
    float f = m_run == -INFINITY ? 0.f : 1.f, den = l_run;
    if (a.sink) {
      const float z = a.sink[h] * LOG2E;
      const float M = fmaxf(m_run, z);
      f = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
      den = l_run * f + exp2f(z - M);
    }
    const float inv = den > 0.f ? f / den : 0.f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + ((b * a.nq + t) * a.nh + h) * C + ch * CH;
    const float* qcs = tcs + qloc * (R >> 1);
    const float* qsn = tsn + qloc * (R >> 1);
#pragma unroll
    for (int mo = 0; mo < MO; ++mo)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store4_bf16_rot(orow + 32 * mo + 8 * j + 4 * G, acc[mo][4 * j] * inv, acc[mo][4 * j + 1] * inv,
                        acc[mo][4 * j + 2] * inv, acc[mo][4 * j + 3] * inv, ch * CH + 32 * mo + 8 * j + 4 * G, C, R,
                        qcs, qsn);
  } else {
    const int64_t unit = blockIdx.x;
    const int64_t rows = Cf::R;
    const PartialRow pr = partial_row(a, pl, gridDim.x, unit, split, rows, row, C);
    uint16_t* ow = pr.o + ch * CH;
    if (G == 0 && ch == 0) { pr.ml[0] = m_run; pr.ml[1] = l_run; }
#pragma unroll
    for (int mo = 0; mo < MO; ++mo)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store_partial4(ow + 32 * mo + 8 * j + 4 * G, acc[mo][4 * j], acc[mo][4 * j + 1], acc[mo][4 * j + 2],
                       acc[mo][4 * j + 3]);
  }
}

// ------------------------------------------------------------------ FP8 rows at c = 512
// Two blocks per CU.  The decoded bf16 key tiles are gone: the MFMA operands
// come straight from the raw stage (E4M3 bytes converted in registers, the 64
// bf16 RoPE channels as they are), which halves the LDS bytes per MFMA and
// leaves LDS for three stages of copies in flight.
//   * wave (rg, ch) holds Q^T and O^T of 32 rows x 256 channels: E4M3
//     channels 224 ch .. 224 ch + 223 and bf16 RoPE channels 448 + 32 ch ..
//     448 + 32 ch + 31, so that both waves of a pair convert the same number
//     of E4M3 operands (they meet at every barrier);
//   * S^T over the wave's channel half: A = K rows (ds_read_b64 of 8 E4M3
//     bytes per lane, or ds_read_b128 of 8 bf16), B = Q^T;
//   * both waves of a pair write their whole partial S^T and read the other's,
//     so each holds the full scores of its 32 rows and computes the softmax of
//     all 32 keys itself (no exchange of maxima or P);
//   * O^T += V^T P^T with V^T from ds_read_b64_tr_b8: in a 16-lane group, lane
//     s reads 8 bytes at key k0 + s/2, channels c0 + 8 (s % 2); lane i then
//     holds channel c0 + i of keys k0 .. k0 + 7.  The stage keeps key j of a
//     tile at slot kperm(j) (bits 2 and 3 of j swapped), so those 8 slots are
//     the keys 16 s + 4 G + {0..3}, 16 s + 8 + 4 G + {0..3} that the P^T
//     fragment of lane half G holds (registers 8 s .. 8 s + 7 of S^T);
//   * a piece (16 bytes of a row) of the 32 keys is a 512-byte run of slots,
//     and in odd pieces slot j sits at position j ^ 8: the transposed reads
//     take the same 8 slots of pieces 2 i and 2 i + 1 together, which would
//     otherwise lie 512 bytes apart, in the same LDS banks;
//   * per tile: [copies of tile it landed] barrier, copies of tile it+2, S^T,
//     partial out, barrier, softmax, PV.
constexpr int F8_NSTG = 3;
constexpr int F8_K8 = 14;   // E4M3 k-steps (and pieces) of each channel half
__device__ __forceinline__ int kperm(int x) { return (x & ~12) | ((x >> 1) & 4) | ((x << 1) & 8); }

template <int NRG>
__global__ __launch_bounds__(128 * NRG, 2) void attn_f8(AttnArgs a, PosTable pt, int b0, AttnPlan pl) {
  constexpr int C = 512, CS = 2;
  using Cf = AttnCfg<C, ROW_FP8, CS, NRG>;
  constexpr int KQ = Cf::KQ, MO = Cf::MO, RB = Cf::RB, NF8 = Cf::NF8;   // 16, 8, 576, 28
  static_assert(KQ == 16 && MO == 8 && NF8 == 28, "c = 512, FP8 + 64 bf16 RoPE dims");
  __shared__ __align__(16) uint8_t s_stage[F8_NSTG * Cf::STAGE];
  __shared__ __align__(16) float s_x[Cf::NW * 16 * 64];            // [wave][r/4][lane][4]
  __shared__ uint32_t s_vmask[F8_NSTG][8];
  __shared__ int s_nvisq[8];
  __shared__ int s_sidx[SIDX_CAP];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, G = l >> 5, col = l & 31;
  const int rg = wv / CS, ch = wv % CS;
  const int64_t bl = blockIdx.x / pl.units_per_b, u = blockIdx.x % pl.units_per_b;
  const int64_t b = b0 + bl;
  const int64_t p0 = pt.q_pos0[bl], wpos0 = pt.win_pos0[bl];
  const UnitInfo ui = unit_info(a, pl, p0, u);
  const int64_t nsplit = pl.max_splits == 1 ? 1 : (ui.total + pl.chunk - 1) / pl.chunk;
  const int split = blockIdx.y;
  if (split > 0 && split >= nsplit) return;
  const int slot_lo = split * pl.chunk;
  const int slot_hi = (int)(pl.max_splits == 1 ? ui.total : (slot_lo + pl.chunk < ui.total ? slot_lo + pl.chunk : ui.total));
  const int ncomp = (int)ui.ncomp;
  const uint8_t* comp_base = reinterpret_cast<const uint8_t*>(a.kv_comp) + b * a.S * (int64_t)RB;
  const uint8_t* win_base = reinterpret_cast<const uint8_t*>(a.kv_win) + (b * a.W + (ui.wlo - wpos0)) * (int64_t)RB;
  static_assert(RB <= (int)sizeof(g_zero_row), "zero row shorter than a stored row");
  const uint8_t* dummy = g_zero_row;
  const int nq_blk = (int)(ui.tl - ui.t0 + 1);
  const int pfirst = (int)(p0 + ui.t0);
  const int ntiles = slot_hi > slot_lo ? (slot_hi - slot_lo + TS - 1) / TS : 0;

  if (threadIdx.x < 8) s_nvisq[threadIdx.x] = pl.dense ? (int)visible_count(pfirst + threadIdx.x, a.ratio, a.S) : (int)a.S;
  int bad_idx = 0;
  if (a.idx) {
    const int32_t* irow = a.idx + (b * a.nq + ui.t0) * a.k;
    const int n_i = (ncomp < slot_hi ? ncomp : slot_hi) - slot_lo;
    for (int i = threadIdx.x; i < n_i; i += Cf::NT) {
      const int e = irow[slot_lo + i];
      s_sidx[i] = e;
      bad_idx |= (e < 0 || e >= a.S) ? 1 : 0;
    }
  }
  const bool idx_ok = !__syncthreads_or(bad_idx);
  const int plast = (int)(p0 + ui.tl);
  const int nvis_first = pl.dense ? (int)visible_count(pfirst, a.ratio, a.S) : (int)a.S;

  const int row = 32 * rg + col;
  const int qloc = row / a.nh;
  const int h = row % a.nh;
  const int64_t t = ui.t0 + qloc;
  const bool qvalid = t <= ui.tl;
  const int64_t tq = qvalid ? t : ui.tl;

  // Q^T in the contraction order of S^T: k-step 2 j + hh (< 14) of lane half
  // G takes E4M3 channels 224 ch + 16 (2 j + G) + 8 hh .. + 8, k-steps 14 and
  // 15 the bf16 channels 448 + 32 ch + 16 (kk - 14) + 8 G .. + 8
  bf16x8 qf[KQ];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((b * a.nq + tq) * a.nh + h) * C;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const int c8 = kk < F8_K8 ? 224 * ch + 16 * (2 * (kk >> 1) + G) + 8 * (kk & 1)
                                : (C - ROPE_DIMS) + 32 * ch + 16 * (kk - F8_K8) + 8 * G;
      qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + c8));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): only tile copies are counted from here on
  }
  f32x16 acc[MO];
#pragma unroll
  for (int i = 0; i < MO; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl = pl.scale_log2;

  auto slot_src = [&](int s, int* pos, bool* win) -> const uint8_t* {
    if (s < ncomp) {
      *win = false;
      const int e = a.idx ? s_sidx[s - slot_lo] : s;
      *pos = e;
      if (e < 0 || e >= a.S) return nullptr;
      return comp_base + (int64_t)e * RB;
    }
    *win = true;
    *pos = (int)ui.wlo + (s - ncomp);
    return win_base + (int64_t)(s - ncomp) * RB;
  };
  // copies of tile `it`: lane l fills position l % 32 of a piece of parity G,
  // which holds slot (l % 32) ^ 8 G, that is key kperm((l % 32) ^ 8 G)
  const int kp = kperm((l & 31) ^ (8 * G));
  auto issue = [&](int it, uint8_t* stg) {
    const int s0 = slot_lo + it * TS;
    const uint8_t* rowp;
    if (s0 + TS <= ncomp && s0 + TS <= slot_hi && (!a.idx || idx_ok)) {
      // a whole tile of compressed entries (indices already checked): no per-lane tests
      const int e = a.idx ? s_sidx[s0 + kp - slot_lo] : s0 + kp;
      rowp = comp_base + (int64_t)e * RB;
    } else {
      const int slot = s0 + kp;
      int pos;
      bool win;
      rowp = slot < slot_hi ? slot_src(slot, &pos, &win) : nullptr;
      rowp = rowp ? rowp : dummy;
    }
    const uint8_t* base = rowp + 16 * G + 32 * wv;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)(stg + wv * 1024));
    DmaCopies<0, (Cf::NDMA + Cf::NW - 1) / Cf::NW, Cf::NW, Cf::NDMA>::run(base, lds0, wv);
  };
  const int my_dma = Cf::NDMA / Cf::NW + (wv < Cf::NDMA % Cf::NW ? 1 : 0);
  auto wait_copies = [&](int n) {
    switch (n) {
      case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
      case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
      case 9: __builtin_amdgcn_s_waitcnt(0x0F79); break;
      case 10: __builtin_amdgcn_s_waitcnt(0x0F7A); break;
      default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
  };
  auto tile_full = [&](int it) -> bool {
    const int s0 = slot_lo + it * TS, s1 = s0 + TS;
    if (s1 > slot_hi) return false;
    if (s0 < ncomp) {
      if (a.idx ? !idx_ok : (s1 < ncomp ? s1 : ncomp) > nvis_first) return false;
    }
    if (s1 > ncomp) {
      const int lo = (int)ui.wlo + ((s0 > ncomp ? s0 : ncomp) - ncomp), hi = (int)ui.wlo + (s1 - 1 - ncomp);
      if (hi > pfirst || lo < plast - a.n_win + 1) return false;
    }
    return true;
  };
  // per-query visibility bits of a tile that is not full, in key order (wave 0)
  auto masks = [&](int it, int buf) {
    if (wv != 0 || tile_full(it)) return;
    const int s0 = slot_lo + it * TS;
    uint32_t vbits = 0;
    const int slot = s0 + l;
    if (l < TS && slot < slot_hi) {
      int pos;
      bool win;
      if (slot_src(slot, &pos, &win)) {
        for (int q = 0; q < nq_blk; ++q) {
          const int pq = pfirst + q;
          const bool ok = win ? (pos <= pq && pos >= pq - a.n_win + 1) : (pos < s_nvisq[q]);
          vbits |= (ok ? 1u : 0u) << q;
        }
      }
    }
    for (int q = 0; q < nq_blk; ++q) {
      const uint32_t bal = (uint32_t)__ballot((vbits >> q) & 1u);
      if (l == 0) s_vmask[buf][q] = bal;
    }
  };

  auto e4m3x8 = [](u32x2 w) -> bf16x8 {
    return as_bf16x8((u32x4){e4m3x2_to_bf16x2(w[0], false), e4m3x2_to_bf16x2(w[0], true),
                             e4m3x2_to_bf16x2(w[1], false), e4m3x2_to_bf16x2(w[1], true)});
  };
  typedef short v4s __attribute__((ext_vector_type(4)));
  typedef int v2i __attribute__((ext_vector_type(2)));
  // S^T operand: key m = l % 32 at stage slot kperm(m); channel half ch: E4M3
  // pieces 14 ch + 2 j + G, then bf16 pieces 28 + 4 ch + 2 (kk - 14) + G
  // (every piece a lane half reads has parity G)
  const int kslot = (kperm(col) ^ (8 * G)) * 16;
  auto score_tile = [&](auto chc, const uint8_t* stg) -> f32x16 {
    constexpr int CHW = decltype(chc)::value;
    constexpr int P8 = F8_K8 * CHW, PB = NF8 + 4 * CHW;   // first E4M3 and bf16 piece of the half
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    // one 16-byte unit (16 E4M3 channels of key m) per lane feeds two k-steps;
    // the reads run two units ahead of their conversions and MFMAs (a
    // sched_barrier keeps the order; -1% against the compiler's own placement)
    constexpr int NU = F8_K8 / 2 + (KQ - F8_K8);   // 16-byte units: E4M3 pairs, then bf16 k-steps
    auto rd = [&](int u) -> u32x4 {
      const int piece = u < F8_K8 / 2 ? P8 + 2 * u + G : PB + 2 * (u - F8_K8 / 2) + G;
      return *reinterpret_cast<const u32x4*>(stg + piece * (TS * 16) + kslot);
    };
    constexpr int RA = 2;
    u32x4 buf[RA];
#pragma unroll
    for (int u = 0; u < RA; ++u) buf[u] = rd(u);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const u32x4 w = buf[u % RA];
      if (u + RA < NU) buf[u % RA] = rd(u + RA);
      if (u < F8_K8 / 2) {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8((u32x2){w[0], w[1]}), qf[2 * u], sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8((u32x2){w[2], w[3]}), qf[2 * u + 1], sacc, 0, 0, 0);
      } else {
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w), qf[F8_K8 + (u - F8_K8 / 2)], sacc, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return sacc;
  };
  // PV over key half s: lane l's 8-byte transposed read of m-tile mo.  The
  // reads run three m-tiles ahead of the conversions and MFMAs (sched_barrier
  // keeps that order), so an LDS read's latency overlaps three MFMAs instead of
  // stalling each one; at occupancy 2 there is room for just these registers
  const int lam = l & 15, grp = (l >> 4) & 1;
  auto pv_half = [&](auto chc, const uint8_t* stg, int s, const bf16x8& pf) {
    constexpr int CHW = decltype(chc)::value;
    constexpr int P8 = F8_K8 * CHW, PB = NF8 + 4 * CHW;
    constexpr int M8 = F8_K8 / 2;                  // E4M3 m-tiles (32 channels each)
    const int slot8 = 16 * s + 8 * G;              // first of the 8 stage slots of this lane half
    const int pos8 = slot8 ^ (8 * grp);            // their positions in a piece of parity grp
    auto rd = [&](int mo) {                        // E4M3 pieces P8 + 2 mo + grp
      return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)(
          stg + ((P8 + 2 * mo + grp) * TS + pos8 + (lam >> 1)) * 16 + 8 * (lam & 1)));
    };
    v2i w1 = rd(0), w2 = rd(1), w3 = rd(2);
#pragma unroll
    for (int mo = 0; mo < M8; ++mo) {
      const v2i w = w1;
      w1 = w2;
      w2 = w3;
      if (mo + 3 < M8) w3 = rd(mo + 3);
      acc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8(__builtin_bit_cast(u32x2, w)), pf, acc[mo], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    {                                              // bf16 channels 448 + 32 ch + 16 grp + lam
      const int par = (lam >> 1) & 1;              // parity of the piece
      const int piece = PB + 2 * grp + par;
      const uint8_t* p0 = stg + (piece * TS + (slot8 ^ (8 * par)) + (lam >> 2)) * 16 + 8 * (lam & 1);
      const v4s t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p0));
      const v4s t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p0 + 4 * 16));
      const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1b = __builtin_bit_cast(u32x2, t1);
      acc[M8] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8((u32x4){w0[0], w0[1], w1b[0], w1b[1]}), pf,
                                                        acc[M8], 0, 0, 0);
    }
  };
  // channel of register r of m-tile mo: f8_chan(mo) + 8 (r / 4) + 4 G + r % 4
  auto f8_chan = [&](int mo) { return mo < F8_K8 / 2 ? 224 * ch + 32 * mo : (C - ROPE_DIMS) + 32 * ch; };

  // prologue: copies of tiles 0 and 1 in flight, their masks
  if (ntiles > 0) issue(0, s_stage);
  if (ntiles > 1) issue(1, s_stage + Cf::STAGE);
  if (ntiles > 0) masks(0, 0);
  if (ntiles > 1) masks(1, 1);
  const int partner = wv ^ 1;
  // the tile loop, compiled once per channel half (straight-line code for each)
  auto tile_loop = [&](auto chc) {
  constexpr int CHW = decltype(chc)::value;
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it % F8_NSTG;
    const uint8_t* stg = s_stage + buf * Cf::STAGE;
    wait_copies(it + 1 < ntiles ? my_dma : 0);      // this wave's copies of tile it have landed
    lds_barrier();                                   // A: tile it visible, stage of it-1 and s_x free
    if (it + 2 < ntiles) {
      const int nb = (it + 2) % F8_NSTG;
      issue(it + 2, s_stage + nb * Cf::STAGE);
      masks(it + 2, nb);
    }
    f32x16 sc = score_tile(chc, stg);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      *reinterpret_cast<f32x4*>(s_x + ((wv * 4 + rr) * 64 + l) * 4) =
          (f32x4){sc[4 * rr], sc[4 * rr + 1], sc[4 * rr + 2], sc[4 * rr + 3]};
    lds_barrier();                                   // B: partials of tile it
    // full scores: the channel-0 half plus the channel-1 half, in that order in
    // both waves of the pair, so that both get the same sums
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(s_x + ((partner * 4 + rr) * 64 + l) * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[4 * rr + j] = CHW == 0 ? sc[4 * rr + j] + o[j] : o[j] + sc[4 * rr + j];
    }
    if (!tile_full(it)) {
      const uint32_t mk = s_vmask[buf][qloc] >> (4 * G);
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = ((mk >> (8 * (r >> 2) + (r & 3))) & 1u) ? sc[r] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = max_halves(mx) * sl;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
      float alpha = 1.f;
      if (mx > m_run + 8.0f) {
        alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
        m_run = mx;
      }
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < MO; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
    }
    const float mneg = m_run == -INFINITY ? 0.f : -m_run;
    uint32_t pk[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      // v_exp_f32 directly: results below 2^-126 flush to zero, which leaves
      // the normalised output unchanged at fp32 resolution
      const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[r], sl, mneg));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[r + 1], sl, mneg));
      l_run += e0 + e1;
      pk[r >> 1] = __builtin_bit_cast(uint32_t, (bf16x2){(__bf16)e0, (__bf16)e1});
    }
    pv_half(chc, stg, 0, as_bf16x8((u32x4){pk[0], pk[1], pk[2], pk[3]}));
    pv_half(chc, stg, 1, as_bf16x8((u32x4){pk[4], pk[5], pk[6], pk[7]}));
  }
  };
  if (ch == 0) tile_loop(std::integral_constant<int, 0>());
  else tile_loop(std::integral_constant<int, 1>());

  l_run = sum_halves(l_run);
  // output rotation table in the stage (after a barrier: every wave is done with it)
  const int R = pl.max_splits == 1 ? a.rot_dims : 0;
  float* tcs = reinterpret_cast<float*>(s_stage);
  float* tsn = tcs + nq_blk * (R >> 1);
  if (R > 0) {
    lds_barrier();
    out_rot_table(tcs, tsn, nq_blk, pfirst, R, a.rot_theta);
    lds_barrier();
  }
  if (!qvalid) return;
  if (pl.max_splits == 1) {
    float f = m_run == -INFINITY ? 0.f : 1.f, den = l_run;
    if (a.sink) {
      const float z = a.sink[h] * LOG2E;
      const float M = fmaxf(m_run, z);
      f = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
      den = l_run * f + exp2f(z - M);
    }
    const float inv = den > 0.f ? f / den : 0.f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + ((b * a.nq + t) * a.nh + h) * C;
    const float* qcs = tcs + qloc * (R >> 1);
    const float* qsn = tsn + qloc * (R >> 1);
#pragma unroll
    for (int mo = 0; mo < MO; ++mo)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e0 = f8_chan(mo) + 8 * j + 4 * G;
        store4_bf16_rot(orow + e0, acc[mo][4 * j] * inv, acc[mo][4 * j + 1] * inv, acc[mo][4 * j + 2] * inv,
                        acc[mo][4 * j + 3] * inv, e0, C, R, qcs, qsn);
      }
  } else {
    const int64_t unit = blockIdx.x;
    const int64_t rows = Cf::R;
    // the unit's partial rows in fragment order (f8_frag_elem): each store is
    // 64 lanes x 8 contiguous bytes
    const PartialRow pr = partial_row(a, pl, gridDim.x, unit, split, rows, row, C);
    uint16_t* ob = pr.o - (int64_t)row * C;
    if (G == 0 && ch == 0) { pr.ml[0] = m_run; pr.ml[1] = l_run; }
#pragma unroll
    for (int mo = 0; mo < MO; ++mo)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store_partial4(ob + 4 * (((wv * MO + mo) * 4 + j) * 64 + l), acc[mo][4 * j], acc[mo][4 * j + 1],
                       acc[mo][4 * j + 2], acc[mo][4 * j + 3]);
  }
}

// ------------------------------------------------------------------ bf16 rows at c = 128
// The stage, copies and operand reads of attn_f8 for rows of 128 bf16
// channels (sixteen 16-byte pieces), with one wave holding all 128 channels
// of its 32 rows: Q^T (8 k-steps) and O^T (4 m-tiles) fit in registers, so
// every wave computes the full S^T itself and nothing is exchanged between
// waves.  S^T reads 8 bf16 channels of one key per lane and k-step straight
// from the stage (ds_read_b128; key j of a tile at slot kperm(j), odd pieces
// at position slot ^ 8), V^T comes from ds_read_b64_tr_b16 as in attn_f8's
// RoPE channels.  Per tile: [copies of tile it landed] barrier, copies of
// tile it + NST - 1, S^T, softmax, PV; block = 32 rows per wave, NRG waves.
//
// Occupancy: the kernel fits 168 registers without spills, so it is built
// for 3 waves per SIMD (unbounded, the compiler takes 232 and 2 waves; 3
// waves measured 28% faster on 128-row dense blocks).  NST stage buffers:
// 3 for 4 row groups (33 KB, 3 blocks per CU), 2 for fewer (25 KB, so that
// 6 blocks of 2 waves fit the 160 KB of LDS; 13% faster on the 64-head
// sparse blocks than 3 buffers at 4 blocks per CU).
template <int NRG, int NST>
__global__ __launch_bounds__(64 * NRG) __attribute__((amdgpu_waves_per_eu(3, 3)))
void attn_b16(AttnArgs a, PosTable pt, int b0, AttnPlan pl) {
  constexpr int C = 128;
  using Cf = AttnCfg<C, ROW_BF16, 1, NRG>;
  constexpr int KQ = Cf::KQ, MO = Cf::MO, RB = Cf::RB, NW = Cf::NW;   // 8, 4, 256, NRG
  static_assert(KQ == 8 && MO == 4 && RB == 256 && Cf::NF8 == 0, "c = 128, bf16 rows");
  static_assert(NST == 2 || NST == 3, "stage buffers");
  __shared__ __align__(16) uint8_t s_stage[NST * Cf::STAGE];
  __shared__ uint32_t s_vmask[NST][8];
  __shared__ int s_nvisq[8];
  __shared__ int s_sidx[SIDX_CAP];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, G = l >> 5, col = l & 31;
  const int64_t bl = blockIdx.x / pl.units_per_b, u = blockIdx.x % pl.units_per_b;
  const int64_t b = b0 + bl;
  const int64_t p0 = pt.q_pos0[bl], wpos0 = pt.win_pos0[bl];
  const UnitInfo ui = unit_info(a, pl, p0, u);
  const int64_t nsplit = pl.max_splits == 1 ? 1 : (ui.total + pl.chunk - 1) / pl.chunk;
  const int split = blockIdx.y;
  if (split > 0 && split >= nsplit) return;
  const int slot_lo = split * pl.chunk;
  const int slot_hi = (int)(pl.max_splits == 1 ? ui.total : (slot_lo + pl.chunk < ui.total ? slot_lo + pl.chunk : ui.total));
  const int ncomp = (int)ui.ncomp;
  const uint8_t* comp_base = reinterpret_cast<const uint8_t*>(a.kv_comp) + b * a.S * (int64_t)RB;
  const uint8_t* win_base = reinterpret_cast<const uint8_t*>(a.kv_win) + (b * a.W + (ui.wlo - wpos0)) * (int64_t)RB;
  static_assert(RB <= (int)sizeof(g_zero_row), "zero row shorter than a stored row");
  const uint8_t* dummy = g_zero_row;
  const int nq_blk = (int)(ui.tl - ui.t0 + 1);
  const int pfirst = (int)(p0 + ui.t0);
  const int ntiles = slot_hi > slot_lo ? (slot_hi - slot_lo + TS - 1) / TS : 0;

  if (threadIdx.x < 8) s_nvisq[threadIdx.x] = pl.dense ? (int)visible_count(pfirst + threadIdx.x, a.ratio, a.S) : (int)a.S;
  int bad_idx = 0;
  if (a.idx) {
    const int32_t* irow = a.idx + (b * a.nq + ui.t0) * a.k;
    const int n_i = (ncomp < slot_hi ? ncomp : slot_hi) - slot_lo;
    for (int i = threadIdx.x; i < n_i; i += Cf::NT) {
      const int e = irow[slot_lo + i];
      s_sidx[i] = e;
      bad_idx |= (e < 0 || e >= a.S) ? 1 : 0;
    }
  }
  const bool idx_ok = !__syncthreads_or(bad_idx);
  const int plast = (int)(p0 + ui.tl);
  const int nvis_first = pl.dense ? (int)visible_count(pfirst, a.ratio, a.S) : (int)a.S;

  const int row = 32 * wv + col;
  const int qloc = row / a.nh;
  const int h = row % a.nh;
  const int64_t t = ui.t0 + qloc;
  const bool qvalid = t <= ui.tl;
  const int64_t tq = qvalid ? t : ui.tl;

  // Q^T: k-step kk of lane half G takes channels 16 kk + 8 G .. + 8 (piece 2 kk + G)
  bf16x8 qf[KQ];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((b * a.nq + tq) * a.nh + h) * C;
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * G));
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): only tile copies are counted from here on
  }
  f32x16 acc[MO];
#pragma unroll
  for (int i = 0; i < MO; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl = pl.scale_log2;

  auto slot_src = [&](int s, int* pos, bool* win) -> const uint8_t* {
    if (s < ncomp) {
      *win = false;
      const int e = a.idx ? s_sidx[s - slot_lo] : s;
      *pos = e;
      if (e < 0 || e >= a.S) return nullptr;
      return comp_base + (int64_t)e * RB;
    }
    *win = true;
    *pos = (int)ui.wlo + (s - ncomp);
    return win_base + (int64_t)(s - ncomp) * RB;
  };
  // copies of tile `it`: lane l fills position l % 32 of a piece of parity G,
  // which holds slot (l % 32) ^ 8 G, that is key kperm((l % 32) ^ 8 G)
  const int kp = kperm((l & 31) ^ (8 * G));
  auto issue = [&](int it, uint8_t* stg) {
    const int s0 = slot_lo + it * TS;
    const uint8_t* rowp;
    if (s0 + TS <= ncomp && s0 + TS <= slot_hi && (!a.idx || idx_ok)) {
      const int e = a.idx ? s_sidx[s0 + kp - slot_lo] : s0 + kp;
      rowp = comp_base + (int64_t)e * RB;
    } else {
      const int slot = s0 + kp;
      int pos;
      bool win;
      rowp = slot < slot_hi ? slot_src(slot, &pos, &win) : nullptr;
      rowp = rowp ? rowp : dummy;
    }
    const uint8_t* base = rowp + 16 * G + 32 * wv;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)(stg + wv * 1024));
    DmaCopies<0, (Cf::NDMA + NW - 1) / NW, NW, Cf::NDMA>::run(base, lds0, wv);
  };
  // this wave's copies per tile: NDMA / NW (NDMA = 8 divides evenly for NW = 1, 2, 4)
  static_assert(Cf::NDMA % NW == 0, "copies per wave");
  constexpr int MYDMA = Cf::NDMA / NW;
  auto wait_copies = [&](bool one_more) {
    if (!one_more) __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0)
    else if constexpr (MYDMA == 8) __builtin_amdgcn_s_waitcnt(0x0F78);
    else if constexpr (MYDMA == 4) __builtin_amdgcn_s_waitcnt(0x0F74);
    else __builtin_amdgcn_s_waitcnt(0x0F72);
  };
  static_assert(MYDMA == 8 || MYDMA == 4 || MYDMA == 2, "vmcnt encodings below");
  auto tile_full = [&](int it) -> bool {
    const int s0 = slot_lo + it * TS, s1 = s0 + TS;
    if (s1 > slot_hi) return false;
    if (s0 < ncomp) {
      if (a.idx ? !idx_ok : (s1 < ncomp ? s1 : ncomp) > nvis_first) return false;
    }
    if (s1 > ncomp) {
      const int lo = (int)ui.wlo + ((s0 > ncomp ? s0 : ncomp) - ncomp), hi = (int)ui.wlo + (s1 - 1 - ncomp);
      if (hi > pfirst || lo < plast - a.n_win + 1) return false;
    }
    return true;
  };
  // per-query visibility bits of a tile that is not full, in key order (wave 0)
  auto masks = [&](int it, int buf) {
    if (wv != 0 || tile_full(it)) return;
    const int s0 = slot_lo + it * TS;
    uint32_t vbits = 0;
    const int slot = s0 + l;
    if (l < TS && slot < slot_hi) {
      int pos;
      bool win;
      if (slot_src(slot, &pos, &win)) {
        for (int q = 0; q < nq_blk; ++q) {
          const int pq = pfirst + q;
          const bool ok = win ? (pos <= pq && pos >= pq - a.n_win + 1) : (pos < s_nvisq[q]);
          vbits |= (ok ? 1u : 0u) << q;
        }
      }
    }
    for (int q = 0; q < nq_blk; ++q) {
      const uint32_t bal = (uint32_t)__ballot((vbits >> q) & 1u);
      if (l == 0) s_vmask[buf][q] = bal;
    }
  };

  typedef short v4s __attribute__((ext_vector_type(4)));
  // S^T: key m = l % 32 at stage slot kperm(m); k-step kk reads piece 2 kk + G
  // (parity G), the reads two k-steps ahead of their MFMAs
  const int kslot = (kperm(col) ^ (8 * G)) * 16;
  auto score_tile = [&](const uint8_t* stg) -> f32x16 {
    f32x16 sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    auto rd = [&](int kk) { return *reinterpret_cast<const u32x4*>(stg + (2 * kk + G) * (TS * 16) + kslot); };
    u32x4 buf[2] = {rd(0), rd(1)};
#pragma unroll
    for (int kk = 0; kk < KQ; ++kk) {
      const u32x4 w = buf[kk & 1];
      if (kk + 2 < KQ) buf[kk & 1] = rd(kk + 2);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(w), qf[kk], sacc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    return sacc;
  };
  // PV over key half s: m-tile mo holds channels 32 mo + 16 grp + lam; lane
  // half G takes the 8 slots 16 s + 8 G .. + 7 (keys of its P^T fragment)
  const int lam = l & 15, grp = (l >> 4) & 1;
  auto pv_half = [&](const uint8_t* stg, int s, const bf16x8& pf) {
    const int slot8 = 16 * s + 8 * G;
    const int par = (lam >> 1) & 1;                // parity of the piece
#pragma unroll
    for (int mo = 0; mo < MO; ++mo) {
      const int piece = 4 * mo + 2 * grp + par;
      const uint8_t* pp = stg + (piece * TS + (slot8 ^ (8 * par)) + (lam >> 2)) * 16 + 8 * (lam & 1);
      const v4s t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(pp));
      const v4s t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(pp + 4 * 16));
      const u32x2 w0 = __builtin_bit_cast(u32x2, t0), w1 = __builtin_bit_cast(u32x2, t1);
      acc[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8((u32x4){w0[0], w0[1], w1[0], w1[1]}), pf, acc[mo],
                                                        0, 0, 0);
    }
  };

  // prologue: copies of tiles 0 .. NST - 2 in flight, their masks
  for (int i = 0; i < NST - 1; ++i)
    if (i < ntiles) issue(i, s_stage + i * Cf::STAGE);
  for (int i = 0; i < NST - 1; ++i)
    if (i < ntiles) masks(i, i);
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it % NST;
    const uint8_t* stg = s_stage + buf * Cf::STAGE;
    wait_copies(NST == 3 && it + 1 < ntiles);       // this wave's copies of tile it have landed
    lds_barrier();                                   // tile it visible, stage of it-1 free
    if (it + NST - 1 < ntiles) {
      const int nb = (it + NST - 1) % NST;
      issue(it + NST - 1, s_stage + nb * Cf::STAGE);
      masks(it + NST - 1, nb);
    }
    f32x16 sc = score_tile(stg);
    if (!tile_full(it)) {
      const uint32_t mk = s_vmask[buf][qloc] >> (4 * G);
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[r] = ((mk >> (8 * (r >> 2) + (r & 3))) & 1u) ? sc[r] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    mx = max_halves(mx) * sl;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.0f) != 0) {
      float alpha = 1.f;
      if (mx > m_run + 8.0f) {
        alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - mx);
        m_run = mx;
      }
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < MO; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
    }
    const float mneg = m_run == -INFINITY ? 0.f : -m_run;
    uint32_t pk[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      // v_exp_f32 directly: results below 2^-126 flush to zero, which leaves
      // the normalised output unchanged at fp32 resolution
      const float e0 = __builtin_amdgcn_exp2f(fmaf(sc[r], sl, mneg));
      const float e1 = __builtin_amdgcn_exp2f(fmaf(sc[r + 1], sl, mneg));
      l_run += e0 + e1;
      pk[r >> 1] = __builtin_bit_cast(uint32_t, (bf16x2){(__bf16)e0, (__bf16)e1});
    }
    pv_half(stg, 0, as_bf16x8((u32x4){pk[0], pk[1], pk[2], pk[3]}));
    pv_half(stg, 1, as_bf16x8((u32x4){pk[4], pk[5], pk[6], pk[7]}));
  }

  l_run = sum_halves(l_run);
  // output rotation table in the stage (after a barrier: every wave is done with it)
  const int R = pl.max_splits == 1 ? a.rot_dims : 0;
  float* tcs = reinterpret_cast<float*>(s_stage);
  float* tsn = tcs + nq_blk * (R >> 1);
  if (R > 0) {
    lds_barrier();
    out_rot_table(tcs, tsn, nq_blk, pfirst, R, a.rot_theta);
    lds_barrier();
  }
  if (!qvalid) return;
  // register r of m-tile mo holds channel 32 mo + 8 (r/4) + 4 G + r%4 of this lane's row
  if (pl.max_splits == 1) {
    float f = m_run == -INFINITY ? 0.f : 1.f, den = l_run;
    if (a.sink) {
      const float z = a.sink[h] * LOG2E;
      const float M = fmaxf(m_run, z);
      f = m_run == -INFINITY ? 0.f : exp2f(m_run - M);
      den = l_run * f + exp2f(z - M);
    }
    const float inv = den > 0.f ? f / den : 0.f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(a.out) + ((b * a.nq + t) * a.nh + h) * C;
    const float* qcs = tcs + qloc * (R >> 1);
    const float* qsn = tsn + qloc * (R >> 1);
#pragma unroll
    for (int mo = 0; mo < MO; ++mo)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store4_bf16_rot(orow + 32 * mo + 8 * j + 4 * G, acc[mo][4 * j] * inv, acc[mo][4 * j + 1] * inv,
                        acc[mo][4 * j + 2] * inv, acc[mo][4 * j + 3] * inv, 32 * mo + 8 * j + 4 * G, C, R, qcs, qsn);
  } else {
    const int64_t unit = blockIdx.x;
    const int64_t rows = Cf::R;
    const PartialRow pr = partial_row(a, pl, gridDim.x, unit, split, rows, row, C);
    if (G == 0) { pr.ml[0] = m_run; pr.ml[1] = l_run; }
#pragma unroll
    for (int mo = 0; mo < MO; ++mo)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        store_partial4(pr.o + 32 * mo + 8 * j + 4 * G, acc[mo][4 * j], acc[mo][4 * j + 1], acc[mo][4 * j + 2],
                       acc[mo][4 * j + 3]);
  }
}

// Merge of the split partials, splits in increasing order (deterministic).
// A block takes 4 rows of one unit; each row's 64 threads own CPT = c / 64
// consecutive channels and read every split's bf16 partial for them with one
// vector load per split, all issued before the merge.
template <int CPT>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, PosTable pt, int b0, AttnPlan pl) {
  const int64_t unit = blockIdx.x;
  const int64_t bl = unit / pl.units_per_b, u = unit % pl.units_per_b;
  const int64_t b = b0 + bl;
  const UnitInfo ui = unit_info(a, pl, pt.q_pos0[bl], u);
  const int64_t nsplit = (ui.total + pl.chunk - 1) / pl.chunk;   // <= ATTN_MAX_SPLITS by the plan
  const int64_t rows = (int64_t)pl.qpw * a.nh;
  const int64_t r = (int64_t)blockIdx.y * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c = CPT * 64;
  if (r >= rows) return;
  const int qw = (int)(r / a.nh), h = (int)(r % a.nh);
  const int64_t t = ui.t0 + qw;
  if (t > ui.tl) return;
  const PartialRow pr = partial_row(a, pl, gridDim.x, unit, 0, rows, r, c);
  const float* ml = pr.ml;                                   // split s at + 2 s rows
  const uint16_t* ow = pr.o + lane * CPT;                    // split s at + s rows c
  // a split that saw no visible key (m = -inf, zero partial) gets weight 0
  constexpr int MS = ATTN_MAX_SPLITS;
  constexpr int NW = CPT / 2;                                // bf16 pairs per thread and split
  static_assert(NW == 4 || NW == 1, "channels per thread");
  float mv[MS], lv[MS];
  uint32_t ov[MS][NW];
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) {
    mv[sp] = -INFINITY;
    lv[sp] = 0.f;
#pragma unroll
    for (int j = 0; j < NW; ++j) ov[sp][j] = 0u;
    if (sp < nsplit) {
      mv[sp] = ml[sp * rows * 2];
      lv[sp] = ml[sp * rows * 2 + 1];
      const uint16_t* src = ow + sp * rows * (int64_t)c;
      if constexpr (NW == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(src);
        ov[sp][0] = v[0]; ov[sp][1] = v[1]; ov[sp][2] = v[2]; ov[sp][3] = v[3];
      } else {
        ov[sp][0] = *reinterpret_cast<const uint32_t*>(src);
      }
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) M = fmaxf(M, mv[sp]);
  const float z = a.sink ? a.sink[h] * LOG2E : -INFINITY;
  const float Mt = fmaxf(M, z);
  float den = a.sink ? exp2f(z - Mt) : 0.f;
  float o[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) o[j] = 0.f;
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) {
    if (sp >= nsplit) break;
    const float w = mv[sp] == -INFINITY ? 0.f : exp2f(mv[sp] - Mt);
    den = fmaf(lv[sp], w, den);
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      o[2 * q] = fmaf(bf16_to_f32(ov[sp][q] & 0xFFFFu), w, o[2 * q]);
      o[2 * q + 1] = fmaf(bf16_to_f32(ov[sp][q] >> 16), w, o[2 * q + 1]);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int64_t obase = ((b * a.nq + t) * a.nh + h) * c + lane * CPT;
  const int R = a.rot_dims;
#pragma unroll
  for (int j = 0; j < CPT; j += 2) {
    const int e = lane * CPT + j;
    uint32_t w2;
    if (R > 0 && e >= c - R) {
      float x0 = bf16_round(o[j] * inv), x1 = bf16_round(o[j + 1] * inv), cs, sn;
      rope_cs(-(pt.q_pos0[bl] + t), (e - (c - R)) >> 1, R, a.rot_theta, &cs, &sn);
      rope_pair(x0, x1, cs, sn);
      w2 = pack_bf16x2(x0, x1);
    } else {
      w2 = __builtin_bit_cast(uint32_t, (bf16x2){(__bf16)(o[j] * inv), (__bf16)(o[j + 1] * inv)});
    }
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.out) + obase + j) = w2;
  }
}

// attn_f8's split partials are stored in fragment order: 8-byte element
// e = ((w * 8 + mo) * 4 + j) * 64 + l of a (unit, split) holds the 4 channels
// that lane l of wave w kept in register group j of m-tile mo, that is
// channels f8_chan(mo) + 8 j + 4 (l / 32) .. + 3 of row 32 (w / 2) + l % 32,
// f8_chan(mo) = 224 ch + 32 mo (mo < 7) or 448 + 32 ch, ch = w % 2.
struct F8Elem {
  int row, chan;
};
__device__ __forceinline__ F8Elem f8_frag_elem(int e) {
  const int w = e >> 11, mo = (e >> 8) & 7, j = (e >> 6) & 3, l = e & 63;
  const int ch = w & 1;
  return {32 * (w >> 1) + (l & 31), (mo < 7 ? 224 * ch + 32 * mo : 448 + 32 * ch) + 8 * j + 4 * (l >> 5)};
}

// Merge of attn_f8's split partials (c = 512), splits in increasing order
// (deterministic): a thread takes one fragment element (4 channels of one
// row) of every split, all loads issued before the merge.
__global__ __launch_bounds__(256) void attn_combine_f8(AttnArgs a, PosTable pt, int b0, AttnPlan pl) {
  constexpr int C = 512;
  const int64_t unit = blockIdx.x;
  const int64_t bl = unit / pl.units_per_b, u = unit % pl.units_per_b;
  const int64_t b = b0 + bl;
  const UnitInfo ui = unit_info(a, pl, pt.q_pos0[bl], u);
  const int64_t nsplit = (ui.total + pl.chunk - 1) / pl.chunk;   // <= ATTN_MAX_SPLITS by the plan
  const int64_t rows = (int64_t)pl.qpw * a.nh;
  const int e = (int)blockIdx.y * 256 + (int)threadIdx.x;
  if (e >= rows * (C / 4)) return;
  const F8Elem fe = f8_frag_elem(e);
  const int qw = fe.row / a.nh, h = fe.row % a.nh;
  const int64_t t = ui.t0 + qw;
  if (t > ui.tl) return;
  const PartialRow pr = partial_row(a, pl, gridDim.x, unit, 0, rows, fe.row, C);
  const float* ml = pr.ml;                                        // split s at + 2 s rows
  const uint16_t* ob = pr.o - (int64_t)fe.row * C + 4 * e;        // split s at + s rows C
  constexpr int MS = ATTN_MAX_SPLITS;
  float mv[MS], lv[MS];
  u32x2 ov[MS];
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) {
    mv[sp] = -INFINITY;
    lv[sp] = 0.f;
    ov[sp] = (u32x2){0u, 0u};
    if (sp < nsplit) {
      mv[sp] = ml[sp * rows * 2];
      lv[sp] = ml[sp * rows * 2 + 1];
      ov[sp] = *reinterpret_cast<const u32x2*>(ob + sp * rows * (int64_t)C);
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) M = fmaxf(M, mv[sp]);
  const float z = a.sink ? a.sink[h] * LOG2E : -INFINITY;
  const float Mt = fmaxf(M, z);
  float den = a.sink ? exp2f(z - Mt) : 0.f;
  float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int sp = 0; sp < MS; ++sp) {
    if (sp >= nsplit) break;
    // a split that saw no visible key (m = -inf, zero partial) gets weight 0
    const float w = mv[sp] == -INFINITY ? 0.f : exp2f(mv[sp] - Mt);
    den = fmaf(lv[sp], w, den);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      o[2 * q] = fmaf(bf16_to_f32(ov[sp][q] & 0xFFFFu), w, o[2 * q]);
      o[2 * q + 1] = fmaf(bf16_to_f32(ov[sp][q] >> 16), w, o[2 * q + 1]);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + ((b * a.nq + t) * a.nh + h) * C + fe.chan;
  const int R = a.rot_dims;
  if (R > 0 && fe.chan >= C - R) {
    float x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = bf16_round(o[q] * inv);
#pragma unroll
    for (int q = 0; q < 4; q += 2) {
      float cs, sn;
      rope_cs(-(pt.q_pos0[bl] + t), (fe.chan + q - (C - R)) >> 1, R, a.rot_theta, &cs, &sn);
      rope_pair(x[q], x[q + 1], cs, sn);
    }
    *reinterpret_cast<u32x2*>(dst) = (u32x2){pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  } else {
    *reinterpret_cast<u32x2*>(dst) = (u32x2){__builtin_bit_cast(uint32_t, (bf16x2){(__bf16)(o[0] * inv), (__bf16)(o[1] * inv)}),
                                            __builtin_bit_cast(uint32_t, (bf16x2){(__bf16)(o[2] * inv), (__bf16)(o[3] * inv)})};
  }
}

// ------------------------------------------------------------------ launch
// The plan (path, rows per block, split) comes from attn_make_plan, the same
// function the argument checks sized the workspace with.

template <int C, int KVL, int CS, int NRG_MAX>
static void launch_mfma_c(const AttnArgs& a, dim3 grid, int nrg, const PosTable& pt, int b0, const AttnPlan& pl,
                          hipStream_t s) {
  switch (nrg) {
    case 1: hipLaunchKernelGGL((attn_mfma<C, KVL, CS, 1>), grid, dim3(64 * 1 * CS), 0, s, a, pt, b0, pl); break;
    case 2: hipLaunchKernelGGL((attn_mfma<C, KVL, CS, 2>), grid, dim3(64 * 2 * CS), 0, s, a, pt, b0, pl); break;
    default:
      hipLaunchKernelGGL((attn_mfma<C, KVL, CS, NRG_MAX>), grid, dim3(64 * NRG_MAX * CS), 0, s, a, pt, b0, pl);
      break;
  }
}

hipError_t launch_attn(const AttnArgs& a, const int64_t* q_pos0, const int64_t* win_pos0, const AttnLaunchPlan& lp,
                       hipStream_t s) {
  if (a.B <= 0 || a.nq <= 0) return hipSuccess;
  // the partials of a split launch must fit the workspace the checks accepted
  if (lp.ws_bytes > 0 && (a.ws == nullptr || a.ws_bytes < lp.ws_bytes)) return hipErrorInvalidValue;
  const AttnPlan& pl = lp.pl;
  for (int64_t b0 = 0; b0 < a.B; b0 += MAXB) {
    const int nb = (int)(a.B - b0 < MAXB ? a.B - b0 : MAXB);
    PosTable pt;
    for (int i = 0; i < nb; ++i) { pt.q_pos0[i] = q_pos0[b0 + i]; pt.win_pos0[i] = win_pos0 ? win_pos0[b0 + i] : 0; }
    if (lp.path != ATTN_GENERIC) {
      dim3 grid((unsigned)(nb * pl.units_per_b), (unsigned)pl.max_splits);
      if (lp.path == ATTN_F8) {
        if (lp.nrg == 1) hipLaunchKernelGGL(attn_f8<1>, grid, dim3(128), 0, s, a, pt, (int)b0, pl);
        else hipLaunchKernelGGL(attn_f8<2>, grid, dim3(256), 0, s, a, pt, (int)b0, pl);
      } else {
        if (a.kv_layout == ROW_FP8) launch_mfma_c<128, ROW_FP8, 1, 4>(a, grid, lp.nrg, pt, (int)b0, pl, s);
        else if (lp.nrg == 1) hipLaunchKernelGGL((attn_b16<1, 2>), grid, dim3(64), 0, s, a, pt, (int)b0, pl);
        else if (lp.nrg == 2) hipLaunchKernelGGL((attn_b16<2, 2>), grid, dim3(128), 0, s, a, pt, (int)b0, pl);
        else hipLaunchKernelGGL((attn_b16<4, 3>), grid, dim3(256), 0, s, a, pt, (int)b0, pl);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (pl.max_splits > 1) {
        const int rows = pl.qpw * a.nh;
        if (lp.path == ATTN_F8) {        // fragment-order partials: one thread per 4 channels of a row
          const dim3 cg((unsigned)(nb * pl.units_per_b), (unsigned)((rows * 128 + 255) / 256));
          hipLaunchKernelGGL(attn_combine_f8, cg, dim3(256), 0, s, a, pt, (int)b0, pl);
        } else {
          const dim3 cg((unsigned)(nb * pl.units_per_b), (unsigned)((rows + 3) / 4));
          hipLaunchKernelGGL(attn_combine<2>, cg, dim3(256), 0, s, a, pt, (int)b0, pl);
        }
      }
    } else {
      hipLaunchKernelGGL(attn_generic, dim3((unsigned)(nb * a.nq * a.nh)), dim3(256), 0, s, a, pt, (int)b0, pl);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dsv4
