// Token-level KV compressors of CSA and HCA (DeepSeek-V4 digest, 模块 B eq 9-12
// and 模块 C eq 20-23; jsqmd blog 第一阶段).
//
// CSA entry i, channel j: per-channel softmax over the logits
//   Z^a[m i + r, j] + B^a[r, j]   and   Z^b[m (i-1) + r, j] + B^b[r, j]   (r < m)
// (the b-part is absent for absolute entry 0), then the weighted sum of the
// matching C^a / C^b values, with C^x = H W_x^T and Z^x = H W_x^T.
// HCA entry i: softmax over Z[m' i + r, j] + B[r, j], weighted sum of C.
//
// Two paths:
//   * generic: one thread per (entry, channel) computing its dot products in
//     fp32 -- any m, c, d, either activation dtype (small or odd shapes);
//   * MFMA (bf16, CSA m = 4 / HCA m' = 128, c % 32 == 0, d % 64 == 0): the
//     projection GEMM on v_mfma_f32_16x16x32_bf16 with the pooling softmax,
//     the window-row export and the storage packing fused in the epilogue, so
//     C and Z never touch HBM.
#include "dsv4_common.h"
#include "dsv4_internal.h"

namespace dsv4 {

// ------------------------------------------------------------------------
// shared epilogue: pack a pooled fp32 tile row (32 channels of one entry,
// channels [j0, j0+32)) into the output layout.  Called by a 32-lane group
// holding one channel each (lane32 = channel offset).
// ------------------------------------------------------------------------
__device__ __forceinline__ void pack32(float v, int lane32, uint8_t* row, uint8_t* scale_row,
                                       int layout, int c, int j0) {
  const int j = j0 + lane32;
  if (layout != ROW_MXFP4) {
    store_row_elem(row, layout, c, j, v);
    return;
  }
  float amax = fabsf(v);
  for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
  const uint32_t E = mx_scale_code(amax);
  const float inv = ldexpf(1.0f, 127 - (int)E);
  uint32_t code = E ? f32_to_e2m1(v * inv) : 0u;
  uint32_t partner = __shfl_xor(code, 1, 32);
  if ((lane32 & 1) == 0) row[j >> 1] = (uint8_t)(code | (partner << 4));
  if (lane32 == 0) scale_row[j0 >> 5] = (uint8_t)E;
}

// ------------------------------------------------------------------------
// generic path
// ------------------------------------------------------------------------
__device__ __forceinline__ float dot_row(const void* H, int act, int64_t hrow, const void* W,
                                         int64_t wrow, int64_t d) {
  float acc = 0.0f;
  if (act == ACT_F32) {
    const float* h = reinterpret_cast<const float*>(H) + hrow * d;
    const float* w = reinterpret_cast<const float*>(W) + wrow * d;
    for (int64_t k = 0; k < d; ++k) acc = fmaf(h[k], w[k], acc);
  } else {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(H) + hrow * d;
    const uint16_t* w = reinterpret_cast<const uint16_t*>(W) + wrow * d;
    for (int64_t k = 0; k < d; ++k) acc = fmaf(bf16_to_f32(h[k]), bf16_to_f32(w[k]), acc);
  }
  return acc;
}

// threads: (entry slot e in [0, ceil(n/m)), channel j); c % 32 == 0 is not
// required except for MXFP4 output (32 consecutive lanes = one block).
__global__ void csa_compress_generic(CompressArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int c = a.c, m = a.m;
  const int64_t n_slots = (a.n + m - 1) / m;
  const int64_t e = t / c;
  const int j = (int)(t % c);
  if (e >= n_slots) return;
  const int64_t a0 = a.n_left + (int64_t)m * e;     // H row of the first a-token
  const int rb = row_bytes(a.comp_layout, c);
  const int rrb = row_bytes(a.raw_layout, c);
  float La[64], Ca[64];
  float mx = -INFINITY;
  int na = 0;
  for (int r = 0; r < m; ++r) {
    const int64_t tok = (int64_t)m * e + r;
    if (tok >= a.n) break;
    Ca[r] = dot_row(a.H, a.act, a0 + r, a.W, j, a.d);
    if (a.raw) store_row_elem(reinterpret_cast<uint8_t*>(a.raw) + tok * rrb, a.raw_layout, c, j, Ca[r]);
    La[r] = dot_row(a.H, a.act, a0 + r, a.W, 2 * c + j, a.d) + a.bias[r * c + j];
    mx = fmaxf(mx, La[r]);
    ++na;
  }
  const bool complete = (na == m);
  const bool has_b = (a.block0 + e) >= 1;
  float Cb[64], Lb[64];
  if (complete && has_b) {
    for (int r = 0; r < m; ++r) {
      Cb[r] = dot_row(a.H, a.act, a0 - m + r, a.W, c + j, a.d);
      Lb[r] = dot_row(a.H, a.act, a0 - m + r, a.W, 3 * c + j, a.d) + a.bias[(m + r) * c + j];
      mx = fmaxf(mx, Lb[r]);
    }
  }
  float v = 0.0f;
  if (complete) {
    float num = 0.0f, den = 0.0f;
    for (int r = 0; r < m; ++r) {
      const float w = __expf(La[r] - mx);
      num = fmaf(w, Ca[r], num);
      den += w;
    }
    if (has_b)
      for (int r = 0; r < m; ++r) {
        const float w = __expf(Lb[r] - mx);
        num = fmaf(w, Cb[r], num);
        den += w;
      }
    v = num / den;
  }
  // full 32-lane groups must reach the MXFP4 shuffles: every lane of a
  // complete entry participates (entries are uniform across a block of 32
  // channels because c % 32 == 0 for MXFP4)
  if (!complete) return;
  uint8_t* row = reinterpret_cast<uint8_t*>(a.comp) + e * rb;
  if (a.comp_layout == ROW_MXFP4)
    pack32(v, j & 31, row, a.comp_scales + e * (c / 32), ROW_MXFP4, c, j & ~31);
  else
    store_row_elem(row, a.comp_layout, c, j, v);
}

__global__ void hca_compress_generic(CompressArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int c = a.c, m = a.m;
  const int64_t n_slots = (a.n + m - 1) / m;
  const int64_t e = t / c;
  const int j = (int)(t % c);
  if (e >= n_slots) return;
  const int rb = row_bytes(a.comp_layout, c);
  const int rrb = row_bytes(a.raw_layout, c);
  const bool complete = (int64_t)m * (e + 1) <= a.n;
  // two passes over the block: max of the logits, then the weighted sums
  float mx = -INFINITY;
  for (int r = 0; r < m; ++r) {
    const int64_t tok = (int64_t)m * e + r;
    if (tok >= a.n) break;
    const float C = dot_row(a.H, a.act, tok, a.W, j, a.d);
    if (a.raw) store_row_elem(reinterpret_cast<uint8_t*>(a.raw) + tok * rrb, a.raw_layout, c, j, C);
    if (complete) mx = fmaxf(mx, dot_row(a.H, a.act, tok, a.W, c + j, a.d) + a.bias[r * c + j]);
  }
  if (!complete) return;
  float num = 0.0f, den = 0.0f;
  for (int r = 0; r < m; ++r) {
    const int64_t tok = (int64_t)m * e + r;
    const float w = __expf(dot_row(a.H, a.act, tok, a.W, c + j, a.d) + a.bias[r * c + j] - mx);
    num = fmaf(w, dot_row(a.H, a.act, tok, a.W, j, a.d), num);
    den += w;
  }
  const float v = num / den;
  uint8_t* row = reinterpret_cast<uint8_t*>(a.comp) + e * rb;
  if (a.comp_layout == ROW_MXFP4)
    pack32(v, j & 31, row, a.comp_scales + e * (c / 32), ROW_MXFP4, c, j & ~31);
  else
    store_row_elem(row, a.comp_layout, c, j, v);
}

// ------------------------------------------------------------------------
// MFMA path (bf16)
// ------------------------------------------------------------------------
constexpr int KSTEP = 64;          // d elements staged per LDS round
constexpr int LDK = KSTEP + 8;     // padded LDS row (bf16 elements)

// Copy `rows` rows of KSTEP bf16 each (global row stride `ld` elements, first
// column k0) into LDS; rows with a negative or out-of-range global index are
// zero.  256 threads, 16-byte chunks.
__device__ __forceinline__ void stage_rows(uint16_t* lds, const uint16_t* g, int64_t row0,
                                           int rows, int64_t row_lo, int64_t row_hi,
                                           int64_t ld, int64_t k0) {
  constexpr int CH = KSTEP / 8;    // 16-byte chunks per row
  for (int i = threadIdx.x; i < rows * CH; i += 256) {
    const int r = i / CH, cc = i % CH;
    const int64_t gr = row0 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (gr >= row_lo && gr < row_hi)
      v = *reinterpret_cast<const u32x4*>(g + gr * ld + k0 + cc * 8);
    *reinterpret_cast<u32x4*>(lds + r * LDK + cc * 8) = v;
  }
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* lds, int row, int col) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(lds + row * LDK + col));
}

// CSA, m = 4.  Block: 64 tokens x 32 channels (16 entries); wave w owns
// tokens [16w, 16w+16) = entries [4w, 4w+4).  In the 16x16 MFMA output a lane
// holds 4 consecutive rows of one column, i.e. exactly the 4 a-tokens (or
// b-tokens) of one entry for one channel, so the pooling runs in registers.
__global__ __launch_bounds__(256) void csa_compress_mfma(CompressArgs a) {
  __shared__ uint16_t As[68 * LDK];    // tokens T0-4 .. T0+63
  __shared__ uint16_t Bs[128 * LDK];   // 4 matrices x 32 channels
  __shared__ float Ps[16][33];
  const int c = a.c;
  const int64_t T0 = (int64_t)blockIdx.x * 64;      // chunk-local token
  const int j0 = blockIdx.y * 32;
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, col = l & 15;
  const uint16_t* H = reinterpret_cast<const uint16_t*>(a.H);
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.W);

  f32x4 acc[4][2];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int h = 0; h < 2; ++h) acc[q][h] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < a.d; k0 += KSTEP) {
    // H rows: local token t sits at H row n_left + t; valid rows [0, n_left + n)
    stage_rows(As, H, a.n_left + T0 - 4, 68, 0, a.n_left + a.n, a.d, k0);
    for (int i = threadIdx.x; i < 128 * (KSTEP / 8); i += 256) {
      const int r = i / (KSTEP / 8), cc = i % (KSTEP / 8);
      const int q = r >> 5, jj = r & 31;
      const u32x4 v = *reinterpret_cast<const u32x4*>(W + (int64_t)(q * c + j0 + jj) * a.d + k0 + cc * 8);
      *reinterpret_cast<u32x4*>(Bs + r * LDK + cc * 8) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KSTEP; kk += 32) {
      const bf16x8 fa = lds_frag(As, 16 * wv + 4 + col, kk + 8 * g);   // a-tokens
      const bf16x8 fb = lds_frag(As, 16 * wv + col, kk + 8 * g);       // b-tokens (shifted by -m)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 fw = lds_frag(Bs, 32 * q + 16 * h + col, kk + 8 * g);
          acc[q][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16((q & 1) ? fb : fa, fw, acc[q][h], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  // epilogue: lane holds tokens T0 + 16w + 4g + i (i < 4) = entry e of channel j
  const int64_t e = blockIdx.x * 16 + 4 * wv + g;          // chunk-local entry
  const int64_t n_ent = a.n / 4;
  const bool has_b = (a.block0 + e) >= 1;
  const int rrb = row_bytes(a.raw_layout, c);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = j0 + 16 * h + col;
    float La[4], Lb[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      La[i] = acc[2][h][i] + a.bias[i * c + j];
      Lb[i] = acc[3][h][i] + a.bias[(4 + i) * c + j];
      mx = fmaxf(mx, La[i]);
      if (has_b) mx = fmaxf(mx, Lb[i]);
    }
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float w = __expf(La[i] - mx);
      num = fmaf(w, acc[0][h][i], num);
      den += w;
    }
    if (has_b) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float w = __expf(Lb[i] - mx);
        num = fmaf(w, acc[1][h][i], num);
        den += w;
      }
    }
    Ps[4 * wv + g][16 * h + col] = num / den;
    if (a.raw) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t tok = T0 + 16 * wv + 4 * g + i;
        if (tok < a.n)
          store_row_elem(reinterpret_cast<uint8_t*>(a.raw) + tok * rrb, a.raw_layout, c, j, acc[0][h][i]);
      }
    }
  }
  __syncthreads();
  // pack: 16 entries x 32 channels; a 32-lane group per entry, two passes
  const int rb = row_bytes(a.comp_layout, c);
  for (int pass = 0; pass < 2; ++pass) {
    const int el = pass * 8 + (threadIdx.x >> 5);
    const int64_t ee = blockIdx.x * 16 + el;
    if (ee < n_ent)   // uniform across the 32-lane group
      pack32(Ps[el][threadIdx.x & 31], threadIdx.x & 31,
             reinterpret_cast<uint8_t*>(a.comp) + ee * rb,
             a.comp_scales ? a.comp_scales + ee * (c / 32) : nullptr, a.comp_layout, c, j0);
  }
}

// HCA, m' = 128.  Block: one entry (128 tokens) x 32 channels; wave w owns
// tokens [32w, 32w+32) as two 16-row MFMA tiles.  The per-channel softmax
// over 128 rows reduces within lanes, across the 4 lane groups and across
// the 4 waves.
__global__ __launch_bounds__(256) void hca_compress_mfma(CompressArgs a) {
  __shared__ uint16_t As[128 * LDK];
  __shared__ uint16_t Bs[64 * LDK];
  __shared__ float red[4][32];
  __shared__ float red2[4][32];
  __shared__ float Ps[32];
  const int c = a.c;
  const int64_t T0 = (int64_t)blockIdx.x * 128;
  const int j0 = blockIdx.y * 32;
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63, g = l >> 4, col = l & 15;
  const uint16_t* H = reinterpret_cast<const uint16_t*>(a.H);
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.W);

  f32x4 acc[2][2][2];   // [mtile][KV/Z][channel half]
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[t][q][h] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int64_t k0 = 0; k0 < a.d; k0 += KSTEP) {
    stage_rows(As, H, T0, 128, 0, a.n, a.d, k0);
    for (int i = threadIdx.x; i < 64 * (KSTEP / 8); i += 256) {
      const int r = i / (KSTEP / 8), cc = i % (KSTEP / 8);
      const int q = r >> 5, jj = r & 31;
      const u32x4 v = *reinterpret_cast<const u32x4*>(W + (int64_t)(q * c + j0 + jj) * a.d + k0 + cc * 8);
      *reinterpret_cast<u32x4*>(Bs + r * LDK + cc * 8) = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KSTEP; kk += 32) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const bf16x8 fa = lds_frag(As, 32 * wv + 16 * t + col, kk + 8 * g);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            acc[t][q][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                fa, lds_frag(Bs, 32 * q + 16 * h + col, kk + 8 * g), acc[t][q][h], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  const bool complete = T0 + 128 <= a.n;
  const int rrb = row_bytes(a.raw_layout, c);
  float M[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int j = j0 + 16 * h + col;
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * wv + 16 * t + 4 * g + i;
        acc[t][1][h][i] += a.bias[r * c + j];          // logit Z + B
        mx = fmaxf(mx, acc[t][1][h][i]);
        if (a.raw && T0 + r < a.n)
          store_row_elem(reinterpret_cast<uint8_t*>(a.raw) + (T0 + r) * rrb, a.raw_layout, c, j,
                         acc[t][0][h][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = max_halves(mx);
    if (g == 0) red[wv][16 * h + col] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cc = 16 * h + col;
    M[h] = fmaxf(fmaxf(red[0][cc], red[1][cc]), fmaxf(red[2][cc], red[3][cc]));
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float w = __expf(acc[t][1][h][i] - M[h]);
        num = fmaf(w, acc[t][0][h][i], num);
        den += w;
      }
    num += __shfl_xor(num, 16);
    num = sum_halves(num);
    den += __shfl_xor(den, 16);
    den = sum_halves(den);
    __syncthreads();   // red is reused below
    if (g == 0) { red[wv][cc] = num; red2[wv][cc] = den; }
    __syncthreads();
    if (threadIdx.x < 16) {
      const int c2 = 16 * h + threadIdx.x;
      Ps[c2] = ((red[0][c2] + red[1][c2]) + (red[2][c2] + red[3][c2])) /
               ((red2[0][c2] + red2[1][c2]) + (red2[2][c2] + red2[3][c2]));
    }
  }
  __syncthreads();
  if (complete && threadIdx.x < 32) {
    const int rb = row_bytes(a.comp_layout, c);
    pack32(Ps[threadIdx.x], threadIdx.x, reinterpret_cast<uint8_t*>(a.comp) + blockIdx.x * rb,
           a.comp_scales ? a.comp_scales + blockIdx.x * (c / 32) : nullptr, a.comp_layout, c, j0);
  }
}

// ------------------------------------------------------------------------
// launchers
// ------------------------------------------------------------------------
static bool mfma_ok(const CompressArgs& a, int want_m) {
  return a.act == ACT_BF16 && a.m == want_m && a.c % 32 == 0 && a.d % KSTEP == 0 && a.n > 0;
}

// the pipelined path: c a multiple of 64; MXFP4 entries for CSA only
static bool gemm_path_ok(const CompressArgs& a, int want_m) {
  return mfma_ok(a, want_m) && a.c % 64 == 0 && (want_m == 4 || a.comp_layout != ROW_MXFP4) &&
         (!a.raw || a.raw_layout != ROW_MXFP4);
}

// ------------------------------------------------------------------------
// Pipelined MFMA path (bf16, c % 64 == 0)
// ------------------------------------------------------------------------
// Block: 64 MT tokens x 64 channels, four waves in 2 x 2; wave (wm, wn) holds
// tokens [32 MT wm, 32 MT (wm + 1)) of the block and channels j0 + 32 wn + [0, 32)
// in 32x32 tiles of v_mfma_f32_32x32x16_bf16: NT column tiles, one per matrix
// (CSA: C^a, C^b, Z^a, Z^b; HCA: C, Z), so a lane's column is one channel of
// every matrix, and its registers 4q .. 4q+3 of a tile are 4 consecutive
// tokens.  The b-matrices of CSA multiply the H rows 4 tokens earlier, so a
// lane holds an entry's four a-tokens next to the b-tokens of the block
// before and pools them in registers (MXFP4 rows: the 32 lanes of a lane half
// hold one entry's 32 channels, so the E8M0 block scale is a lane reduction);
// an HCA entry (MT = 4) is exactly one wave's 128 tokens, pooled within the
// lane (64 rows) and with its partner lane (the other 64).  MT = 4 for wide
// rows, MT = 1 (64-token blocks, more of them) for narrow ones.  H rows
// T0 - 32 .. T0 + 64 MT - 1 and the block's W rows travel
// global -> LDS by global_load_lds_dwordx4 into an XOR-swizzled layout (chunk
// j of row r at j ^ ((r >> 1) & 7): 16 consecutive 128-byte rows then fill
// the 64 LDS banks twice over in distinct 16-byte groups, so a 16-lane
// fragment read is conflict-free), two stages, one barrier per 64-wide k tile.
// Staged H rows outside the input are clamped copies that no entry uses.
constexpr int CG_K = 64;
template <bool HCA, int MT>
struct CgShape {
  static constexpr int NT = HCA ? 2 : 4;               // column tiles (matrices) per wave
  static constexpr int BM = 64 * MT;                   // tokens per block
  static constexpr int CG_AR = BM + 32;                // staged H rows: 32 before the tile, BM in it
  static constexpr int BN = 2 * 32 * NT;               // staged W rows
  static constexpr int ASZ = CG_AR * CG_K * 2, BSZ = BN * CG_K * 2;   // bytes of one stage
};

// One block's tile: tokens [bx BM, bx BM + BM) of the chunk, channels
// [64 by, 64 by + 64) of every matrix; s_a / s_b hold two stages each.
template <bool HCA, int MT>
__device__ __forceinline__ void compress_tile(const CompressArgs& a, int64_t bx, int by, uint8_t* s_a,
                                              uint8_t* s_b) {
  static_assert(!HCA || MT == 4, "an HCA entry is one wave's 128 tokens");
  using Sh = CgShape<HCA, MT>;
  constexpr int NT = Sh::NT, BM = Sh::BM, CG_AR = Sh::CG_AR, BN = Sh::BN, ASZ = Sh::ASZ, BSZ = Sh::BSZ;
  constexpr int CA = CG_AR / 32, CB = BN / 32;  // 1 KB copies per wave and k tile
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, G = l >> 5, col = l & 31;
  const int wm = wv >> 1, wn = wv & 1;
  const int c = a.c;
  const int64_t T0 = bx * BM;                      // chunk-local token of tile row 0
  const int j0 = by * 64;
  const uint16_t* H = reinterpret_cast<const uint16_t*>(a.H);
  const uint16_t* W = reinterpret_cast<const uint16_t*>(a.W);
  // copy k of a tile covers staged rows [8k, 8k + 8): lane L takes row 8k + L/8
  // and writes LDS chunk L % 8, which holds source chunk (L % 8) ^ ((row >> 1) & 7);
  // this wave's copies are k = wv + 4 i, so (row >> 1) & 7 = (4 wv + L/16) & 7
  const int crow = l >> 3, gch = (l & 7) ^ ((4 * wv + (crow >> 1)) & 7);
  const int64_t hrows = a.n_left + a.n;
  const uint16_t* pa[CA];
  const uint16_t* pb[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    int64_t hr = a.n_left + T0 - 32 + 8 * (wv + 4 * i) + crow;
    hr = hr < 0 ? 0 : (hr >= hrows ? hrows - 1 : hr);
    pa[i] = H + hr * a.d + 8 * gch;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int nb = 8 * (wv + 4 * i) + crow;       // W row: matrix t, channel j0 + 32 wn' + jj
    const int wnb = nb / (32 * NT), t = (nb / 32) % NT, jj = nb & 31;
    pb[i] = W + ((int64_t)t * c + j0 + 32 * wnb + jj) * a.d + 8 * gch;
  }
  const uint32_t la = lds_addr(s_a), lb = lds_addr(s_b);
  auto issue = [&](int kt, int st) {
    const int64_t k0 = (int64_t)kt * CG_K;
#pragma unroll
    for (int i = 0; i < CA; ++i) dma16<0>(pa[i] + k0, la + st * ASZ + 1024 * (wv + 4 * i));
#pragma unroll
    for (int i = 0; i < CB; ++i) dma16<0>(pb[i] + k0, lb + st * BSZ + 1024 * (wv + 4 * i));
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.f;

  // fragment rows: a-tokens at staged row (tile row + 32), b-tokens at (tile row + 28)
  const int ra = 32 * MT * wm + 32 + col, rbr = 32 * MT * wm + 28 + col;   // + 32 i
  const int swa = (ra >> 1) & 7, swb = (rbr >> 1) & 7;
  const int rw = 32 * NT * wn + col, sww = (rw >> 1) & 7;           // + 32 t
  const int nk = (int)(a.d / CG_K);
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0): this wave's copies of tile kt
    __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();                 // every copy landed; stage st ^ 1 is free
    if (kt + 1 < nk) issue(kt + 1, st ^ 1);
    const uint8_t* ta = s_a + st * ASZ;
    const uint8_t* tb = s_b + st * BSZ;
#pragma unroll
    for (int kk = 0; kk < CG_K / 16; ++kk) {
      const int cq = 2 * kk + G;
      bf16x8 fw[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t)
        fw[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(tb + (rw + 32 * t) * 128 + ((cq ^ sww) << 4)));
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const bf16x8 fa = as_bf16x8(*reinterpret_cast<const u32x4*>(ta + (ra + 32 * i) * 128 + ((cq ^ swa) << 4)));
        if constexpr (HCA) {
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, fw[t], acc[i][t], 0, 0, 0);
        } else {
          const bf16x8 fb = as_bf16x8(*reinterpret_cast<const u32x4*>(ta + (rbr + 32 * i) * 128 + ((cq ^ swb) << 4)));
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16((t & 1) ? fb : fa, fw[t], acc[i][t], 0, 0, 0);
        }
      }
    }
  }

  // epilogue: lane holds channel j of every matrix; register 4q + e of M tile i
  // is tile row 32 i + 8 q + 4 G + e of this wave's 128 tokens
  const int j = j0 + 32 * wn + col;
  const int rb = row_bytes(a.comp_layout, c), rrb = row_bytes(a.raw_layout, c);
  uint8_t* comp = reinterpret_cast<uint8_t*>(a.comp);
  uint8_t* raw = reinterpret_cast<uint8_t*>(a.raw);
  const int64_t tw = T0 + 32 * MT * wm;              // first token of this wave
  if (a.raw) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t tok = tw + 32 * i + 8 * (r >> 2) + 4 * G + (r & 3);
        if (tok < a.n) store_row_elem(raw + tok * rrb, a.raw_layout, c, j, acc[i][0][r]);
      }
  }
  if constexpr (HCA) {
    const int64_t e = tw / 128;                      // this wave's entry
    if (tw + 128 > a.n) return;                      // an incomplete block emits nothing
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * i + 8 * (r >> 2) + 4 * G + (r & 3);
        acc[i][1][r] += a.bias[row * c + j];          // logit Z + B
        mx = fmaxf(mx, acc[i][1][r]);
      }
    mx = max_halves(mx);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float w = __expf(acc[i][1][r] - mx);
        num = fmaf(w, acc[i][0][r], num);
        den += w;
      }
    num = sum_halves(num);
    den = sum_halves(den);
    if (G == 0) store_row_elem(comp + e * rb, a.comp_layout, c, j, num / den);
  } else {
    const int64_t n_ent = a.n / 4;
    float ba[4], bb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) { ba[e] = a.bias[e * c + j]; bb[e] = a.bias[(4 + e) * c + j]; }
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t ent = (tw + 32 * i + 8 * q + 4 * G) / 4;
        if (ent >= n_ent) continue;
        const bool has_b = a.block0 + ent >= 1;
        float La[4], Lb[4], mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          La[e] = acc[i][2][4 * q + e] + ba[e];
          Lb[e] = acc[i][3][4 * q + e] + bb[e];
          mx = fmaxf(mx, La[e]);
          if (has_b) mx = fmaxf(mx, Lb[e]);
        }
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float w = __expf(La[e] - mx);
          num = fmaf(w, acc[i][0][4 * q + e], num);
          den += w;
        }
        if (has_b)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float w = __expf(Lb[e] - mx);
            num = fmaf(w, acc[i][1][4 * q + e], num);
            den += w;
          }
        const float v = num / den;
        if (a.comp_layout == ROW_MXFP4) {
          // E8M0 block of channels j0 + 32 wn + [0, 32): the 32 lanes of this lane half
          float amax = fabsf(v);
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
          const uint32_t E = mx_scale_code(amax);
          const uint32_t code = E ? f32_to_e2m1(v * ldexpf(1.0f, 127 - (int)E)) : 0u;
          const uint32_t hi = __shfl_xor(code, 1);
          if ((col & 1) == 0) comp[ent * rb + (j >> 1)] = (uint8_t)(code | (hi << 4));
          if (col == 0) a.comp_scales[ent * (c / 32) + (j >> 5)] = (uint8_t)E;
        } else {
          store_row_elem(comp + ent * rb, a.comp_layout, c, j, v);
        }
      }
  }
}

template <bool HCA, int MT>
__global__ __launch_bounds__(256, 1) void compress_gemm(CompressArgs a) {
  using Sh = CgShape<HCA, MT>;
  __shared__ __align__(16) uint8_t s_a[2 * Sh::ASZ];
  __shared__ __align__(16) uint8_t s_b[2 * Sh::BSZ];
  compress_tile<HCA, MT>(a, blockIdx.x, blockIdx.y, s_a, s_b);
}

// The three compressors of a chunk in one launch, all over the same 256-token
// tiles of H: grid.y runs the 64-channel tiles of the CSA KV compressor
// (ny0), then of the indexer-key compressor (ny1), then of the HCA compressor.
__global__ __launch_bounds__(256, 1) void compress_fused(CompressArgs kv, CompressArgs ki, CompressArgs hca,
                                                         int ny0, int ny1) {
  using S4 = CgShape<false, 4>;
  static_assert(CgShape<true, 4>::ASZ <= S4::ASZ && CgShape<true, 4>::BSZ <= S4::BSZ, "stage sizes");
  __shared__ __align__(16) uint8_t s_a[2 * S4::ASZ];
  __shared__ __align__(16) uint8_t s_b[2 * S4::BSZ];
  const int y = blockIdx.y;
  if (y < ny0) compress_tile<false, 4>(kv, blockIdx.x, y, s_a, s_b);
  else if (y < ny0 + ny1) compress_tile<false, 4>(ki, blockIdx.x, y - ny0, s_a, s_b);
  else compress_tile<true, 4>(hca, blockIdx.x, y - ny0 - ny1, s_a, s_b);
}

hipError_t launch_csa_compress(const CompressArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  if (gemm_path_ok(a, 4) && a.c >= 256) {
    dim3 grid((unsigned)((a.n + 255) / 256), (unsigned)(a.c / 64));
    hipLaunchKernelGGL((compress_gemm<false, 4>), grid, dim3(256), 0, s, a);
  } else if (gemm_path_ok(a, 4)) {
    dim3 grid((unsigned)((a.n + 63) / 64), (unsigned)(a.c / 64));
    hipLaunchKernelGGL((compress_gemm<false, 1>), grid, dim3(256), 0, s, a);
  } else if (mfma_ok(a, 4)) {
    dim3 grid((unsigned)((a.n + 63) / 64), (unsigned)(a.c / 32));
    hipLaunchKernelGGL(csa_compress_mfma, grid, dim3(256), 0, s, a);
  } else {
    const int64_t slots = (a.n + a.m - 1) / a.m;
    const int64_t threads = slots * a.c;
    hipLaunchKernelGGL(csa_compress_generic, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// the fused path serves a chunk when every given compressor takes the
// pipelined MFMA path at 256-token tiles and all share n
bool compress_fused_ok(const CompressArgs* kv, const CompressArgs* ki, const CompressArgs* hca) {
  int64_t n = -1;
  for (const CompressArgs* a : {kv, ki, hca}) {
    if (!a) continue;
    if (!gemm_path_ok(*a, a == hca ? 128 : 4)) return false;
    if (n >= 0 && a->n != n) return false;
    n = a->n;
  }
  return n > 0;
}

hipError_t launch_compress_fused(const CompressArgs* kv, const CompressArgs* ki, const CompressArgs* hca,
                                 hipStream_t s) {
  const int ny0 = kv ? kv->c / 64 : 0, ny1 = ki ? ki->c / 64 : 0, ny2 = hca ? hca->c / 64 : 0;
  const int64_t n = kv ? kv->n : ki ? ki->n : hca->n;
  const CompressArgs none{};
  dim3 grid((unsigned)((n + 255) / 256), (unsigned)(ny0 + ny1 + ny2));
  hipLaunchKernelGGL(compress_fused, grid, dim3(256), 0, s, kv ? *kv : none, ki ? *ki : none, hca ? *hca : none,
                     ny0, ny1);
  return hipGetLastError();
}

hipError_t launch_hca_compress(const CompressArgs& a, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  if (gemm_path_ok(a, 128)) {
    dim3 grid((unsigned)((a.n + 255) / 256), (unsigned)(a.c / 64));
    hipLaunchKernelGGL((compress_gemm<true, 4>), grid, dim3(256), 0, s, a);
  } else if (mfma_ok(a, 128)) {
    dim3 grid((unsigned)((a.n + 127) / 128), (unsigned)(a.c / 32));
    hipLaunchKernelGGL(hca_compress_mfma, grid, dim3(256), 0, s, a);
  } else {
    const int64_t slots = (a.n + a.m - 1) / a.m;
    const int64_t threads = slots * a.c;
    hipLaunchKernelGGL(hca_compress_generic, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dsv4
