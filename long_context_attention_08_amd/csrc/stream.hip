// Streaming compressors for decode and the mirrored sliding-window ring
// (DeepSeek-V4 digest, 模块 F: every compressed entry is persisted and a reused
// prefix computes only its incomplete trailing block again, and the
// uncompressed window rows are cached, checkpointed or recomputed; 模块 B eq 9-12
// and 模块 C eq 20-23 for the pooling; jsqmd blog 第一阶段 for the b-window).
//
// State of one sequence: per channel an online-softmax accumulator (running
// maximum, sum of weights, weighted sum) of the entry of the current block
// and, for CSA, one for the b-part of the next entry (the current block's
// b-rows), each tagged with its entry and the number of rows it holds.  An
// entry pools the same rows with the same weights as the batch compressor;
// only the order of the exponentials differs.
//
// A call runs two kernels:
//   1. the projection P = H W^T of the B * n_new new rows, split along d into
//      KS slices whose fp32 partials go to the workspace (KS depends on the
//      shapes only, so a row's sum does not depend on the batch);
//   2. one block per sequence walks its new tokens in order, thread t owning
//      channels 2t and 2t + 1 with the accumulators in registers: the
//      partials are summed in slice order, the C^a / C row is normalised,
//      rotated and packed into the window ring, the token's logits and values
//      enter the accumulators, and a token that completes block s stores entry
//      s (normalised, rotated, packed) as cache row s, or the layout's NaN if
//      the accumulator did not see every row of the entry.
#include "dsv4_common.h"
#include "dsv4_internal.h"

namespace dsv4 {

constexpr int SP_COLS = STREAM_SP_COLS;     // projection: output columns per block (16 per wave)
constexpr int SP_ROWS = 64;            // projection: rows per block (four 16-row MFMA tiles)
constexpr int SU_THREADS = 256;        // update: threads per block, two channels each

// state: [meta 256 B][mx | sum | wsum] x c of the current entry, and for CSA
// the same for the next entry's b-part
struct StreamMeta {
  int64_t a_entry, b_entry;     // entry the accumulator belongs to (-1: none)
  int32_t a_na, a_nb, b_cnt;    // a-rows and b-rows in it; b-rows in the next
  int32_t pad;
};
constexpr int SMETA = STREAM_META_BYTES;
static_assert(sizeof(StreamMeta) <= SMETA, "state header");

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

// Normalise and rotate channels 2t, 2t + 1 of a row, held by thread t (every
// thread of the block calls this; `act` marks the threads with t < c / 2);
// (cs, sn) is the rotation of this thread's pair at the row's position.
__device__ void prep_pair(const StreamArgs& a, float& v0, float& v1, bool act, float cs, float sn, float* red) {
  const int j0 = 2 * threadIdx.x, c = a.c;
  if (a.norm) {
    const float ss = block_sum(act ? fmaf(v0, v0, v1 * v1) : 0.f, red);
    const float inv = 1.0f / sqrtf(ss / (float)c + a.eps);
    const float g0 = act && a.gamma ? a.gamma[j0] : 1.f, g1 = act && a.gamma ? a.gamma[j0 + 1] : 1.f;
    v0 *= inv * g0;
    v1 *= inv * g1;
  }
  if (act && a.rope_dims > 0 && j0 >= c - a.rope_dims) {
    const float u = v0, w = v1;
    v0 = u * cs - w * sn;
    v1 = u * sn + w * cs;
  }
}

// Store channels 2t, 2t + 1 into a row in `layout` (every thread calls this:
// MXFP4 blocks reduce over 16 threads).  nan: the NaN marker of the layout.
__device__ void store_pair(const StreamArgs& a, float v0, float v1, bool act, bool nan, uint8_t* row,
                           uint8_t* scale_row, int layout) {
  const int t = threadIdx.x, c = a.c;
  const int j0 = 2 * t;
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

// online softmax: fold logit L with value v into (mx, sum, wsum)
__device__ __forceinline__ void acc_add(float& mx, float& sum, float& wsum, float L, float v) {
  if (L > mx) {
    const float sc = mx == -INFINITY ? 0.f : __expf(mx - L);
    sum = fmaf(sum, sc, 1.f);
    wsum = fmaf(wsum, sc, v);
    mx = L;
  } else {
    const float w = __expf(L - mx);
    sum += w;
    wsum = fmaf(w, v, wsum);
  }
}

__global__ __launch_bounds__(SU_THREADS) void stream_update(StreamArgs a, PosTable pt, int b0, int64_t M, int ks) {
  __shared__ float red[SU_THREADS / 64];
  const int bl = blockIdx.x;
  const int64_t b = b0 + bl;
  const int t = threadIdx.x, c = a.c, m = a.m;
  const int64_t NC = a.nmat * (int64_t)c;
  uint8_t* sbase = reinterpret_cast<uint8_t*>(a.state) + b * (int64_t)a.state_bytes;
  StreamMeta* meta = reinterpret_cast<StreamMeta*>(sbase);
  float* acc = reinterpret_cast<float*>(sbase + SMETA);       // [6 or 3][c]
  const bool act = t < c / 2;
  const int j0 = 2 * t;
  const int crb = row_bytes(a.cache_layout, c), rrb = row_bytes(a.ring_layout, c);
  // accumulators of channels j0, j0 + 1 (A: current entry, N: next entry's b-part)
  float amx[2], asum[2], aws[2], nmx[2], nsum[2], nws[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = act ? j0 + h : 0;
    amx[h] = acc[0 * c + j]; asum[h] = acc[1 * c + j]; aws[h] = acc[2 * c + j];
    nmx[h] = a.overlap ? acc[3 * c + j] : 0.f;
    nsum[h] = a.overlap ? acc[4 * c + j] : 0.f;
    nws[h] = a.overlap ? acc[5 * c + j] : 0.f;
  }
  StreamMeta md = *meta;                 // every thread keeps the same copy
  const float* Ba = a.bias;
  const float* Bb = a.bias + (int64_t)m * c;
  for (int64_t i = 0; i < a.n_new; ++i) {
    const int64_t x = pt.q_pos0[bl] + i;
    const int64_t s = x / m;
    const int r = (int)(x % m);
    const int64_t prow = b * a.n_new + i;                // row of the projection
    // the rotation of this thread's pair at position x: the window row's, and
    // the entry's when x completes a block (its newest token is x)
    float cs = 1.f, sn = 0.f;
    if (act && a.rope_dims > 0 && j0 >= c - a.rope_dims)
      rope_cs(x, (j0 - (c - a.rope_dims)) >> 1, a.rope_dims, a.theta, &cs, &sn);
    // the token's projected values of this thread's channels, partials summed in slice order
    float ca[2] = {0.f, 0.f}, cb[2] = {0.f, 0.f}, za[2] = {0.f, 0.f}, zb[2] = {0.f, 0.f};
    if (act) {
      const int64_t zoff = a.overlap ? 2 * c : c;
#pragma unroll 8
      for (int k = 0; k < ks; ++k) {
        const float* pr = a.part + ((int64_t)k * M + prow) * NC;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          ca[h] += pr[j0 + h];
          za[h] += pr[zoff + j0 + h];
          if (a.overlap) {
            cb[h] += pr[c + j0 + h];
            zb[h] += pr[3 * c + j0 + h];
          }
        }
      }
    }
    if (a.ring) {                                        // both mirrored rows, one preparation
      const int64_t rr = x % a.ring_w;
      uint8_t* ring_b = reinterpret_cast<uint8_t*>(a.ring) + b * 2 * a.ring_w * (int64_t)rrb;
      float w0 = ca[0], w1 = ca[1];
      prep_pair(a, w0, w1, act, cs, sn, red);
      store_pair(a, w0, w1, act, false, ring_b + rr * rrb, nullptr, a.ring_layout);
      store_pair(a, w0, w1, act, false, ring_b + (rr + a.ring_w) * rrb, nullptr, a.ring_layout);
    }
    // the current entry: a new block takes over the b-part gathered during the
    // previous one (CSA); a stream that starts inside a block starts empty
    if (r == 0 || md.a_entry != s) {
      const bool carry = a.overlap && r == 0 && md.b_entry == s;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        amx[h] = carry ? nmx[h] : -INFINITY;
        asum[h] = carry ? nsum[h] : 0.f;
        aws[h] = carry ? nws[h] : 0.f;
      }
      md.a_nb = carry ? md.b_cnt : 0;
      md.a_na = 0;
      md.a_entry = s;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (act) acc_add(amx[h], asum[h], aws[h], za[h] + Ba[r * c + j0 + h], ca[h]);
    md.a_na += 1;
    if (a.overlap) {                                     // b-rows of block s serve entry s + 1
      if (r == 0 || md.b_entry != s + 1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) { nmx[h] = -INFINITY; nsum[h] = 0.f; nws[h] = 0.f; }
        md.b_entry = s + 1;
        md.b_cnt = 0;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (act) acc_add(nmx[h], nsum[h], nws[h], zb[h] + Bb[r * c + j0 + h], cb[h]);
      md.b_cnt += 1;
    }
    if (r != m - 1) continue;
    // this token completes block s
    if (s < pt.win_pos0[bl] || s >= a.S || !a.cache) continue;
    const bool ok = md.a_na == m && (!a.overlap || s == 0 || md.a_nb == m);
    float v0 = ok ? aws[0] / asum[0] : 0.f, v1 = ok ? aws[1] / asum[1] : 0.f;
    uint8_t* crow = reinterpret_cast<uint8_t*>(a.cache) + (b * a.S + s) * (int64_t)crb;
    uint8_t* cscl = a.cache_scales ? a.cache_scales + (b * a.S + s) * (int64_t)(c / 32) : nullptr;
    prep_pair(a, v0, v1, act, cs, sn, red);             // position m (s + 1) - 1 == x
    store_pair(a, v0, v1, act, !ok, crow, cscl, a.cache_layout);
  }
  // the accumulators and the bookkeeping back to the state
  if (act) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = j0 + h;
      acc[0 * c + j] = amx[h]; acc[1 * c + j] = asum[h]; acc[2 * c + j] = aws[h];
      if (a.overlap) { acc[3 * c + j] = nmx[h]; acc[4 * c + j] = nsum[h]; acc[5 * c + j] = nws[h]; }
    }
  }
  if (t == 0) *meta = md;
}

__global__ void stream_reset(uint8_t* state, int64_t B, int64_t state_bytes) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  StreamMeta md;
  md.a_entry = -1; md.b_entry = -1;
  md.a_na = 0; md.a_nb = 0; md.b_cnt = 0; md.pad = 0;
  *reinterpret_cast<StreamMeta*>(state + b * state_bytes) = md;
}

hipError_t launch_stream_reset(void* state, int64_t B, int overlap, int m, int c, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(stream_reset, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s,
                     reinterpret_cast<uint8_t*>(state), B, (int64_t)stream_state_bytes(overlap, m, c));
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
