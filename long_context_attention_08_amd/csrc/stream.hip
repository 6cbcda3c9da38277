// Streaming compressors for decode and the mirrored sliding-window ring
// (DeepSeek-V4 digest, 模块 F: every compressed entry is persisted and a reused
// prefix computes only its incomplete trailing block again, and the
// uncompressed window rows are cached, checkpointed or recomputed; 模块 B eq 9-12
// and 模块 C eq 20-23 for the pooling; jsqmd blog 第一阶段 for the b-window).
//
// State of one sequence: a ring of R slots (R = 2m for CSA: the current block
// and the one before it, whose b-rows the next entry pools; R = m for HCA),
// slot x mod R holding the projected fp32 row [C^a | C^b | Z^a | Z^b] (CSA) or
// [C | Z] (HCA) of position x, tagged with x.
//
// A call runs two kernels:
//   1. the projection P = H W^T of the B * n_new new rows, split along d into
//      KS slices whose fp32 partials go to the workspace (KS depends on the
//      shapes only, so a row's sum does not depend on the batch);
//   2. one block per sequence walks its new tokens in order: the partials are
//      summed in slice order into the token's slot, its C^a / C row is
//      normalised, rotated and packed into the window ring, and a token that
//      completes block s pools entry s from the ring slots (tags checked: an
//      entry whose rows were never fed is written as NaN) and stores it,
//      normalised, rotated and packed, as cache row s.
#include "dsv4_common.h"
#include "dsv4_internal.h"

namespace dsv4 {

constexpr int SP_COLS = 64;            // projection: output columns per block (16 per wave)
constexpr int SP_ROWS = 64;            // projection: rows per block (four 16-row MFMA tiles)
constexpr int SU_THREADS = 256;        // update: threads per block, two channels each

// ---- slices of d for the projection partials (shapes only)
static void stream_split(int64_t NC, int64_t d, int* ks, int64_t* kslice) {
  const int64_t col_blocks = (NC + SP_COLS - 1) / SP_COLS;
  int64_t want = (256 + col_blocks - 1) / col_blocks;      // about 256 blocks for one row group
  const int64_t most = d / 256 > 1 ? d / 256 : 1;           // slices of at least 256
  if (want > most) want = most;
  if (want < 1) want = 1;
  int64_t sl = (d + want - 1) / want;
  sl = (sl + 31) / 32 * 32;
  *kslice = sl;
  *ks = (int)((d + sl - 1) / sl);
}

size_t stream_state_bytes(int overlap, int m, int c) {
  const int64_t R = overlap ? 2 * (int64_t)m : m;
  const int64_t nc = (overlap ? 4 : 2) * (int64_t)c;
  const size_t tags = (size_t)((R * 8 + 255) / 256 * 256);
  return ((tags + (size_t)(R * nc * 4)) + 255) / 256 * 256;
}

size_t stream_ws_bytes(int64_t rows, int overlap, int c, int64_t d) {
  const int64_t nc = (overlap ? 4 : 2) * (int64_t)c;
  int ks;
  int64_t sl;
  stream_split(nc, d, &ks, &sl);
  return (size_t)ks * (size_t)rows * (size_t)nc * sizeof(float);
}

// ---- 1. projection partials, bf16 rows on v_mfma_f32_16x16x32_bf16: lane l
// of a wave holds W row (16 columns) l % 16 and H row l % 16 of each 16-row
// tile, k-group l / 16 (8 values); its outputs are column l % 16, rows
// 4 (l / 16) .. + 3 of each tile
__global__ __launch_bounds__(256) void stream_proj_bf16(StreamArgs a, int64_t kslice, int64_t M) {
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t NC = a.nmat * (int64_t)a.c;
  const int64_t col = (int64_t)blockIdx.x * SP_COLS + wv * 16 + (l & 15);
  const int ks = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.z * SP_ROWS;
  const int64_t k_lo = ks * kslice, k_hi = k_lo + kslice < a.d ? k_lo + kslice : a.d;
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.W);
  const uint16_t* H = reinterpret_cast<const uint16_t*>(a.H);
  const uint16_t* wp = W + (col < NC ? col : 0) * a.d + 8 * (l >> 4);
  const uint16_t* hp[4];
  bool hok[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int64_t row = r0 + 16 * mt + (l & 15);
    hok[mt] = row < M;
    hp[mt] = H + (hok[mt] ? row : 0) * a.d + 8 * (l >> 4);
  }
  const bool cok = col < NC;
  f32x4 acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll 4
  for (int64_t k = k_lo; k < k_hi; k += 32) {
    const u32x4 w = cok ? *reinterpret_cast<const u32x4*>(wp + k) : z;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const u32x4 h = hok[mt] ? *reinterpret_cast<const u32x4*>(hp[mt] + k) : z;
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(h), as_bf16x8(w), acc[mt], 0, 0, 0);
    }
  }
  if (!cok) return;
  float* part = a.part + (int64_t)ks * M * NC;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = r0 + 16 * mt + 4 * (l >> 4) + i;
      if (row < M) part[row * NC + col] = acc[mt][i];
    }
}

// any dtype or shape: one thread per (row, column), fp32 sums over the slice
__global__ __launch_bounds__(256) void stream_proj_generic(StreamArgs a, int64_t kslice, int64_t M) {
  const int64_t NC = a.nmat * (int64_t)a.c;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= M * NC) return;
  const int64_t row = t / NC, col = t % NC;
  const int ks = blockIdx.y;
  const int64_t k_lo = ks * kslice, k_hi = k_lo + kslice < a.d ? k_lo + kslice : a.d;
  float acc = 0.f;
  for (int64_t k = k_lo; k < k_hi; ++k)
    acc = fmaf(load_act(a.H, a.act, row * a.d + k), load_act(a.W, a.act, col * a.d + k), acc);
  a.part[((int64_t)ks * M + row) * NC + col] = acc;
}

// ---- 2. per-sequence update
// block-wide sum of one value per thread
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wv = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < SU_THREADS / 64; ++w) s += red[w];
  return s;
}

// Normalise, rotate (position pos) and store channels 2t, 2t + 1 of a row,
// held by thread t (every thread of the block calls this; `act` marks the
// threads with t < c / 2).  nan: store the NaN marker of the layout instead.
__device__ void emit_pair(const StreamArgs& a, float v0, float v1, bool act, int64_t pos, bool nan,
                          uint8_t* row, uint8_t* scale_row, int layout, float* red) {
  const int t = threadIdx.x, c = a.c;
  const int j0 = 2 * t;
  if (a.norm) {
    const float ss = block_sum(act ? fmaf(v0, v0, v1 * v1) : 0.f, red);
    const float inv = 1.0f / sqrtf(ss / (float)c + a.eps);
    const float g0 = act && a.gamma ? a.gamma[j0] : 1.f, g1 = act && a.gamma ? a.gamma[j0 + 1] : 1.f;
    v0 *= inv * g0;
    v1 *= inv * g1;
  }
  if (act && a.rope_dims > 0 && j0 >= c - a.rope_dims) {
    float cs, sn;
    rope_cs(pos, (j0 - (c - a.rope_dims)) >> 1, a.rope_dims, a.theta, &cs, &sn);
    const float u = v0, w = v1;
    v0 = u * cs - w * sn;
    v1 = u * sn + w * cs;
  }
  if (layout == ROW_MXFP4) {
    // 16 threads (32 channels) per E8M0 block; every thread takes part in the shuffles
    float amax = act ? fmaxf(fabsf(v0), fabsf(v1)) : 0.f;
    for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    if (!act) return;
    const uint32_t E = mx_scale_code(amax);
    const float inv = ldexpf(1.0f, 127 - (int)E);
    const uint32_t c0 = E ? f32_to_e2m1(v0 * inv) : 0u, c1 = E ? f32_to_e2m1(v1 * inv) : 0u;
    row[t] = nan ? (uint8_t)0 : (uint8_t)(c0 | (c1 << 4));
    if ((t & 15) == 0) scale_row[j0 >> 5] = nan ? (uint8_t)0xFF : (uint8_t)E;
    return;
  }
  if (!act) return;
  if (layout == ROW_F32) {
    reinterpret_cast<float*>(row)[j0] = nan ? __builtin_nanf("") : v0;
    reinterpret_cast<float*>(row)[j0 + 1] = nan ? __builtin_nanf("") : v1;
  } else if (layout == ROW_BF16 || (layout == ROW_FP8 && j0 >= c - ROPE_DIMS)) {
    const uint32_t w = nan ? 0x7FC07FC0u : pack_bf16x2(v0, v1);
    uint8_t* p = layout == ROW_BF16 ? row + 4 * t : row + (c - ROPE_DIMS) + 2 * (j0 - (c - ROPE_DIMS));
    *reinterpret_cast<uint32_t*>(p) = w;
  } else {                                           // two E4M3 bytes
    const uint32_t w = nan ? 0x7F7Fu : (f32_to_e4m3(v0) | (f32_to_e4m3(v1) << 8));
    *reinterpret_cast<uint16_t*>(row + j0) = (uint16_t)w;
  }
}

__global__ __launch_bounds__(SU_THREADS) void stream_update(StreamArgs a, PosTable pt, int b0, int64_t M, int ks) {
  __shared__ float red[SU_THREADS / 64];
  const int bl = blockIdx.x;
  const int64_t b = b0 + bl;
  const int t = threadIdx.x, c = a.c, m = a.m;
  const int64_t NC = a.nmat * (int64_t)c;
  const int R = a.overlap ? 2 * m : m;
  uint8_t* sbase = reinterpret_cast<uint8_t*>(a.state) + b * (int64_t)a.state_bytes;
  int64_t* tags = reinterpret_cast<int64_t*>(sbase);
  float* srows = reinterpret_cast<float*>(sbase + (R * 8 + 255) / 256 * 256);
  const bool act = t < c / 2;
  const int j0 = 2 * t;
  const int crb = row_bytes(a.cache_layout, c), rrb = row_bytes(a.ring_layout, c);
  for (int64_t i = 0; i < a.n_new; ++i) {
    // the previous token's pooling may still read the slot (and tag) this one overwrites
    if (i > 0) __syncthreads();
    const int64_t x = pt.q_pos0[bl] + i;
    const int slot = (int)(x % R);
    const int64_t prow = b * a.n_new + i;                // row of the projection
    // the token's projected row, partials summed in slice order, into its slot
    float* dst = srows + (int64_t)slot * NC;
    float raw0 = 0.f, raw1 = 0.f;
    for (int64_t j = t; j < NC; j += SU_THREADS) {
      float v = 0.f;
      for (int k = 0; k < ks; ++k) v += a.part[((int64_t)k * M + prow) * NC + j];
      dst[j] = v;
    }
    if (act) {                                           // C^a / C channels 2t, 2t + 1, recomputed the same way
      for (int k = 0; k < ks; ++k) {
        raw0 += a.part[((int64_t)k * M + prow) * NC + j0];
        raw1 += a.part[((int64_t)k * M + prow) * NC + j0 + 1];
      }
    }
    if (t == 0) tags[slot] = x;
    // the slot is read back below (pooling) by other threads of this block:
    // one workgroup shares the CU's L1, so the barrier's fence suffices
    __syncthreads();
    if (a.ring) {
      const int64_t rr = x % a.ring_w;
      uint8_t* ring_b = reinterpret_cast<uint8_t*>(a.ring) + b * 2 * a.ring_w * (int64_t)rrb;
      emit_pair(a, raw0, raw1, act, x, false, ring_b + rr * rrb, nullptr, a.ring_layout, red);
      emit_pair(a, raw0, raw1, act, x, false, ring_b + (rr + a.ring_w) * rrb, nullptr, a.ring_layout, red);
    }
    if ((x + 1) % m != 0) continue;
    const int64_t s = (x + 1) / m - 1;                   // this token completes block s
    if (s < pt.win_pos0[bl] || s >= a.S || !a.cache) continue;
    // pool channels 2t, 2t + 1 (R1-R3 of the batch compressor)
    bool ok = true;
    for (int r = 0; r < m; ++r) {
      ok = ok && tags[(m * s + r) % R] == m * s + r;
      if (a.overlap && s >= 1) ok = ok && tags[(m * (s - 1) + r) % R] == m * (s - 1) + r;
    }
    float v[2] = {0.f, 0.f};
    if (act && ok) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = j0 + h;
        const int64_t zoff = a.overlap ? 2 * c : c;
        float mx = -INFINITY;
        for (int r = 0; r < m; ++r) {
          const float* ra = srows + (int64_t)((m * s + r) % R) * NC;
          mx = fmaxf(mx, ra[zoff + j] + a.bias[r * c + j]);
          if (a.overlap && s >= 1) {
            const float* rb = srows + (int64_t)((m * (s - 1) + r) % R) * NC;
            mx = fmaxf(mx, rb[3 * c + j] + a.bias[(m + r) * c + j]);
          }
        }
        float num = 0.f, den = 0.f;
        for (int r = 0; r < m; ++r) {
          const float* ra = srows + (int64_t)((m * s + r) % R) * NC;
          const float w = __expf(ra[zoff + j] + a.bias[r * c + j] - mx);
          num = fmaf(w, ra[j], num);
          den += w;
        }
        if (a.overlap && s >= 1)
          for (int r = 0; r < m; ++r) {
            const float* rb = srows + (int64_t)((m * (s - 1) + r) % R) * NC;
            const float w = __expf(rb[3 * c + j] + a.bias[(m + r) * c + j] - mx);
            num = fmaf(w, rb[c + j], num);
            den += w;
          }
        v[h] = num / den;
      }
    }
    uint8_t* crow = reinterpret_cast<uint8_t*>(a.cache) + (b * a.S + s) * (int64_t)crb;
    uint8_t* cscl = a.cache_scales ? a.cache_scales + (b * a.S + s) * (int64_t)(c / 32) : nullptr;
    emit_pair(a, v[0], v[1], act, m * (s + 1) - 1, !ok, crow, cscl, a.cache_layout, red);
  }
}

__global__ void stream_reset(uint8_t* state, int64_t B, int64_t state_bytes, int R) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= B * R) return;
  reinterpret_cast<int64_t*>(state + (t / R) * state_bytes)[t % R] = -1;
}

hipError_t launch_stream_reset(void* state, int64_t B, int overlap, int m, int c, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const int R = overlap ? 2 * m : m;
  const int64_t n = B * R;
  hipLaunchKernelGGL(stream_reset, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<uint8_t*>(state), B, (int64_t)stream_state_bytes(overlap, m, c), R);
  return hipGetLastError();
}

hipError_t launch_stream(const StreamArgs& a0, const int64_t* pos0, const int64_t* emit_from, hipStream_t s) {
  if (a0.B <= 0 || a0.n_new <= 0) return hipSuccess;
  StreamArgs a = a0;
  a.state_bytes = (int64_t)stream_state_bytes(a.overlap, a.m, a.c);
  const int64_t NC = a.nmat * (int64_t)a.c;
  const int64_t M = a.B * a.n_new;
  int ks;
  int64_t kslice;
  stream_split(NC, a.d, &ks, &kslice);
  const bool mfma = a.act == ACT_BF16 && a.d % 32 == 0;
  if (mfma) {
    const dim3 grid((unsigned)((NC + SP_COLS - 1) / SP_COLS), (unsigned)ks, (unsigned)((M + SP_ROWS - 1) / SP_ROWS));
    hipLaunchKernelGGL(stream_proj_bf16, grid, dim3(256), 0, s, a, kslice, M);
  } else {
    const dim3 grid((unsigned)((M * NC + 255) / 256), (unsigned)ks);
    hipLaunchKernelGGL(stream_proj_generic, grid, dim3(256), 0, s, a, kslice, M);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int64_t b0 = 0; b0 < a.B; b0 += MAXB) {
    const int nb = (int)(a.B - b0 < MAXB ? a.B - b0 : MAXB);
    PosTable pt;
    for (int i = 0; i < nb; ++i) {
      pt.q_pos0[i] = pos0[b0 + i];
      pt.win_pos0[i] = emit_from ? emit_from[b0 + i] : 0;
    }
    hipLaunchKernelGGL(stream_update, dim3((unsigned)nb), dim3(SU_THREADS), 0, s, a, pt, (int)b0, M, ks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dsv4
