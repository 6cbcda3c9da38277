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
// MFMA path (bf16 queries, BF16 or FP8+bf16-RoPE rows, c in {128, 512}, 64
// head rows per block): each wave owns 16 heads of one query.  A 32-key tile is
// gathered, decoded once to bf16 and written to LDS twice: row-major (keys) and
// transposed (values).  Scores are computed transposed, S^T = K Q^T, so the
// 16x16 MFMA output gives each lane the logits of ONE head; the online-softmax
// state, the rescaling and the P^T operand of O^T = V^T P^T are then lane-local.
// The running maximum is only raised when a tile exceeds it by 2^8 (exact in
// the final normalisation, and bf16 P stays well inside range).  Short key
// sets with few queries are split across blocks and merged in a fixed order.
#include "dsv4_common.h"
#include "dsv4_internal.h"

namespace dsv4 {

struct AttnPlan {
  int64_t units_per_b;   // query groups per batch entry
  int qpw;               // queries per group
  int chunk;             // key slots per split (multiple of 32)
  int max_splits;        // grid.y
  int dense;
  float scale_log2;
};

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
  for (int jj = 0; jj < 4; ++jj) {
    const int j = threadIdx.x + 256 * jj;
    if (j < c) store_act(a.out, a.q_dtype, qbase + j, o[jj] * inv);
  }
}

// ------------------------------------------------------------------ MFMA path
constexpr int TS = 32;       // key slots per tile
constexpr int VTP = TS + 4;  // padded transposed row

template <int C>
struct AttnLds {
  uint16_t Ks[TS * (C + 8)];
  uint16_t Vt[C * VTP];
  int64_t pos[TS];
  int win[TS];
};

template <int C, int KVL>
__global__ __launch_bounds__(256, 2) void attn_mfma(AttnArgs a, PosTable pt, int b0, AttnPlan pl) {
  constexpr int LDK = C + 8;
  constexpr int KK = C / 32;      // k-steps of S^T
  constexpr int MO = C / 16;      // O^T m-tiles
  __shared__ AttnLds<C> sm;
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, col = l & 15;
  const int wpq = a.nh / 16;               // waves per query
  const int qw = wv / wpq, hb = wv % wpq;
  const int64_t bl = blockIdx.x / pl.units_per_b, u = blockIdx.x % pl.units_per_b;
  const int64_t b = b0 + bl;
  const int64_t p0 = pt.q_pos0[bl], wpos0 = pt.win_pos0[bl];
  const UnitInfo ui = unit_info(a, pl, p0, u);
  const int64_t nsplit = pl.max_splits == 1 ? 1 : (ui.total + pl.chunk - 1) / pl.chunk;
  const int split = blockIdx.y;
  if (split > 0 && split >= nsplit) return;
  const int64_t slot_lo = (int64_t)split * pl.chunk;
  const int64_t slot_hi = pl.max_splits == 1 ? ui.total : (slot_lo + pl.chunk < ui.total ? slot_lo + pl.chunk : ui.total);
  const int rb = row_bytes(KVL, C);

  const int64_t t = ui.t0 + qw;
  const bool qvalid = t <= ui.tl;
  const int64_t tq = qvalid ? t : ui.tl;
  const int64_t p = p0 + tq;
  const int64_t nvis = pl.dense ? visible_count(p, a.ratio, a.S) : a.S;
  const int h = 16 * hb + col;             // the head this lane owns

  // Q^T fragments: lane holds q[h][32 kk + 8 g .. + 8]
  bf16x8 qf[KK];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + ((b * a.nq + tq) * a.nh + h) * C;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 32 * kk + 8 * g));
  }
  f32x4 acc[MO];
#pragma unroll
  for (int i = 0; i < MO; ++i) acc[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // loader mapping: 4 slots x 16 channels per thread
  const int kg = threadIdx.x & 7, cs = threadIdx.x >> 3;

  for (int64_t s0 = slot_lo; s0 < slot_hi; s0 += TS) {
    if (cs < C / 16) {
      uint32_t v[4][8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t slot = s0 + 4 * kg + j;
        int64_t pos = -1;
        bool win = false;
        const uint8_t* row = nullptr;
        if (slot < slot_hi) row = slot_row(a, b, ui.t0, ui, wpos0, slot, rb, &pos, &win);
        if (cs == 0) { sm.pos[4 * kg + j] = row ? pos : -1; sm.win[4 * kg + j] = win ? 1 : 0; }
        if (!row) {
#pragma unroll
          for (int d = 0; d < 8; ++d) v[j][d] = 0u;
        } else if (KVL == ROW_FP8 && 16 * cs < C - ROPE_DIMS) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(row + 16 * cs);
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            v[j][2 * d] = e4m3x2_to_bf16x2(w[d], false);
            v[j][2 * d + 1] = e4m3x2_to_bf16x2(w[d], true);
          }
        } else {
          const uint8_t* src = KVL == ROW_FP8 ? row + (C - ROPE_DIMS) + 2 * (16 * cs - (C - ROPE_DIMS))
                                              : row + 32 * cs;
          const u32x4 w0 = *reinterpret_cast<const u32x4*>(src);
          const u32x4 w1 = *reinterpret_cast<const u32x4*>(src + 16);
#pragma unroll
          for (int d = 0; d < 4; ++d) { v[j][d] = w0[d]; v[j][4 + d] = w1[d]; }
        }
        uint16_t* kd = sm.Ks + (4 * kg + j) * LDK + 16 * cs;
        *reinterpret_cast<u32x4*>(kd) = (u32x4){v[j][0], v[j][1], v[j][2], v[j][3]};
        *reinterpret_cast<u32x4*>(kd + 8) = (u32x4){v[j][4], v[j][5], v[j][6], v[j][7]};
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint32_t lo0 = (v[0][d] & 0xFFFFu) | (v[1][d] << 16);
        const uint32_t lo1 = (v[2][d] & 0xFFFFu) | (v[3][d] << 16);
        const uint32_t hi0 = (v[0][d] >> 16) | (v[1][d] & 0xFFFF0000u);
        const uint32_t hi1 = (v[2][d] >> 16) | (v[3][d] & 0xFFFF0000u);
        *reinterpret_cast<u32x2*>(sm.Vt + (16 * cs + 2 * d) * VTP + 4 * kg) = (u32x2){lo0, lo1};
        *reinterpret_cast<u32x2*>(sm.Vt + (16 * cs + 2 * d + 1) * VTP + 4 * kg) = (u32x2){hi0, hi1};
      }
    }
    __syncthreads();

    // S^T[key][head] for 32 keys (two 16-row tiles)
    f32x4 st[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      st[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 kf = as_bf16x8(*reinterpret_cast<const u32x4*>(sm.Ks + (16 * mt + col) * LDK + 32 * kk + 8 * g));
        st[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kk], st[mt], 0, 0, 0);
      }
    }
    float x[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int sl = 16 * mt + 4 * g + i;
        const bool ok = sm.pos[sl] >= 0 && slot_visible(sm.win[sl] != 0, sm.pos[sl], p, nvis, a.n_win);
        x[mt][i] = ok ? st[mt][i] * pl.scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, x[mt][i]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (tmax > m_run + 8.0f) {
      const float alpha = m_run == -INFINITY ? 0.f : exp2f(m_run - tmax);
      m_run = tmax;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < MO; ++i) acc[i] *= alpha;
    }
    float pr[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[mt][i] = (x[mt][i] == -INFINITY) ? 0.f : exp2f(x[mt][i] - m_run);
        l_run += pr[mt][i];
      }
    const u32x4 pw = {pack_bf16x2(pr[0][0], pr[0][1]), pack_bf16x2(pr[0][2], pr[0][3]),
                      pack_bf16x2(pr[1][0], pr[1][1]), pack_bf16x2(pr[1][2], pr[1][3])};
    const bf16x8 pf = as_bf16x8(pw);
#pragma unroll
    for (int mo = 0; mo < MO; ++mo) {
      const uint16_t* vr = sm.Vt + (16 * mo + col) * VTP;
      const u32x2 v0 = *reinterpret_cast<const u32x2*>(vr + 4 * g);
      const u32x2 v1 = *reinterpret_cast<const u32x2*>(vr + 16 + 4 * g);
      const bf16x8 vf = as_bf16x8((u32x4){v0[0], v0[1], v1[0], v1[1]});
      acc[mo] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, acc[mo], 0, 0, 0);
    }
    __syncthreads();
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
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
#pragma unroll
    for (int mo = 0; mo < MO; ++mo) {
      const u32x2 w = {pack_bf16x2(acc[mo][0] * inv, acc[mo][1] * inv), pack_bf16x2(acc[mo][2] * inv, acc[mo][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + 16 * mo + 4 * g) = w;
    }
  } else {
    // partials: [unit][split][qpw*nh] {m, l} and [unit][split][qpw*nh][C]
    const int64_t unit = blockIdx.x;
    const int64_t rows = (int64_t)pl.qpw * a.nh;
    const int64_t r = (int64_t)qw * a.nh + h;
    float* ml = reinterpret_cast<float*>(a.ws) + ((unit * pl.max_splits + split) * rows + r) * 2;
    float* ow = reinterpret_cast<float*>(a.ws) + (int64_t)gridDim.x * pl.max_splits * rows * 2 +
                ((unit * pl.max_splits + split) * rows + r) * C;
    if (g == 0) { ml[0] = m_run; ml[1] = l_run; }
#pragma unroll
    for (int mo = 0; mo < MO; ++mo)
      *reinterpret_cast<f32x4*>(ow + 16 * mo + 4 * g) = acc[mo];
  }
}

// merge of the split partials, splits in increasing order (deterministic)
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, PosTable pt, int b0, AttnPlan pl, int c) {
  const int64_t unit = blockIdx.x;
  const int64_t bl = unit / pl.units_per_b, u = unit % pl.units_per_b;
  const int64_t b = b0 + bl;
  const UnitInfo ui = unit_info(a, pl, pt.q_pos0[bl], u);
  const int64_t nsplit = (ui.total + pl.chunk - 1) / pl.chunk;
  const int64_t rows = (int64_t)pl.qpw * a.nh;
  const float* mlb = reinterpret_cast<const float*>(a.ws);
  const float* owb = mlb + (int64_t)gridDim.x * pl.max_splits * rows * 2;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const int qw = (int)(r / a.nh), h = (int)(r % a.nh);
    const int64_t t = ui.t0 + qw;
    if (t > ui.tl) continue;
    float M = -INFINITY;
    for (int64_t s = 0; s < nsplit; ++s) M = fmaxf(M, mlb[((unit * pl.max_splits + s) * rows + r) * 2]);
    const float z = a.sink ? a.sink[h] * LOG2E : -INFINITY;
    const float Mt = fmaxf(M, z);
    float den = a.sink ? exp2f(z - Mt) : 0.f;
    for (int64_t s = 0; s < nsplit; ++s) {
      const float ms = mlb[((unit * pl.max_splits + s) * rows + r) * 2];
      if (ms != -INFINITY) den += mlb[((unit * pl.max_splits + s) * rows + r) * 2 + 1] * exp2f(ms - Mt);
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int j = threadIdx.x; j < c; j += 256) {
      float o = 0.f;
      for (int64_t s = 0; s < nsplit; ++s) {
        const float ms = mlb[((unit * pl.max_splits + s) * rows + r) * 2];
        if (ms != -INFINITY) o = fmaf(owb[((unit * pl.max_splits + s) * rows + r) * c + j], exp2f(ms - Mt), o);
      }
      store_act(a.out, a.q_dtype, ((b * a.nq + t) * a.nh + h) * c + j, o * inv);
    }
  }
}

// ------------------------------------------------------------------ planning and launch
static bool attn_mfma_ok(const AttnArgs& a, bool dense) {
  if (a.q_dtype != ACT_BF16 || (a.kv_layout != ROW_BF16 && a.kv_layout != ROW_FP8)) return false;
  if (a.c != 128 && a.c != 512) return false;
  if (dense) return a.nh == 16 || a.nh == 32 || a.nh == 64;
  return a.nh == 64;
}

static AttnPlan make_plan(const AttnArgs& a, bool dense, int64_t max_keys) {
  AttnPlan pl;
  pl.dense = dense ? 1 : 0;
  pl.scale_log2 = a.scale * LOG2E;
  pl.qpw = dense ? 64 / a.nh : 1;
  if (pl.qpw < 1) pl.qpw = 1;
  pl.units_per_b = (a.nq + pl.qpw - 1) / pl.qpw;
  // split the keys only when a sequence has few query groups; the split size
  // depends on the sequence alone, so results do not depend on the batch
  if (pl.units_per_b >= 32) {
    pl.chunk = 1 << 30;
    pl.max_splits = 1;
  } else {
    pl.chunk = 64;
    int64_t ms = (max_keys + pl.chunk - 1) / pl.chunk;
    pl.max_splits = (int)(ms < 1 ? 1 : ms);
  }
  return pl;
}

size_t attn_workspace_bytes(int64_t B, int64_t nq, int nh, int c, int64_t max_keys, bool dense) {
  AttnArgs a = {};
  a.nq = nq; a.nh = nh; a.c = c; a.scale = 1.f;
  AttnPlan pl = make_plan(a, dense, max_keys);
  if (pl.max_splits == 1) return 0;
  const int64_t units = (B < MAXB ? B : MAXB) * pl.units_per_b;
  return (size_t)units * pl.max_splits * pl.qpw * nh * (c + 2) * sizeof(float);
}

hipError_t launch_attn(const AttnArgs& a, const int64_t* q_pos0, const int64_t* win_pos0, bool dense, hipStream_t s) {
  if (a.B <= 0 || a.nq <= 0) return hipSuccess;
  const bool mf = attn_mfma_ok(a, dense);
  // most key slots any group can have
  int64_t max_keys = 0;
  for (int64_t b = 0; b < a.B; ++b) {
    const int64_t pl_ = q_pos0[b] + a.nq - 1;
    const int64_t ncomp = dense ? visible_count(pl_, a.ratio, a.S) : a.k;
    const int64_t qpw = mf && dense ? 64 / a.nh : 1;
    const int64_t wl = a.n_win > 0 ? a.n_win + qpw - 1 : 0;
    max_keys = ncomp + wl > max_keys ? ncomp + wl : max_keys;
  }
  for (int64_t b0 = 0; b0 < a.B; b0 += MAXB) {
    const int nb = (int)(a.B - b0 < MAXB ? a.B - b0 : MAXB);
    PosTable pt;
    for (int i = 0; i < nb; ++i) { pt.q_pos0[i] = q_pos0[b0 + i]; pt.win_pos0[i] = win_pos0[b0 + i]; }
    if (mf) {
      AttnPlan pl = make_plan(a, dense, max_keys);
      dim3 grid((unsigned)(nb * pl.units_per_b), (unsigned)pl.max_splits);
      if (a.c == 512) {
        if (a.kv_layout == ROW_FP8) hipLaunchKernelGGL((attn_mfma<512, ROW_FP8>), grid, dim3(256), 0, s, a, pt, (int)b0, pl);
        else hipLaunchKernelGGL((attn_mfma<512, ROW_BF16>), grid, dim3(256), 0, s, a, pt, (int)b0, pl);
      } else {
        if (a.kv_layout == ROW_FP8) hipLaunchKernelGGL((attn_mfma<128, ROW_FP8>), grid, dim3(256), 0, s, a, pt, (int)b0, pl);
        else hipLaunchKernelGGL((attn_mfma<128, ROW_BF16>), grid, dim3(256), 0, s, a, pt, (int)b0, pl);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (pl.max_splits > 1) {
        const int rows = pl.qpw * a.nh;
        hipLaunchKernelGGL(attn_combine, dim3((unsigned)(nb * pl.units_per_b), (unsigned)(rows < 64 ? rows : 64)),
                           dim3(256), 0, s, a, pt, (int)b0, pl, a.c);
      }
    } else {
      AttnPlan pl = {};
      pl.dense = dense ? 1 : 0;
      pl.qpw = 1;
      pl.units_per_b = a.nq;
      pl.chunk = 1 << 30;
      pl.max_splits = 1;
      pl.scale_log2 = a.scale * LOG2E;
      hipLaunchKernelGGL(attn_generic, dim3((unsigned)(nb * a.nq * a.nh)), dim3(256), 0, s, a, pt, (int)b0, pl);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dsv4
