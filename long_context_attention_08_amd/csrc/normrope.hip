// Q/KV RMSNorm, partial RoPE and the output rotation (DeepSeek-V4 digest,
// 模块 D: each query head and the single KV head are RMS-normalised before core
// attention; RoPE acts on the last 64 dims of queries and KV entries only, and
// because an entry is key and value at once, the output's last 64 dims are
// rotated back by the query's position).
//
//   RMSNorm:  y = x / sqrt(mean(x^2) + eps) * gamma      (gamma NULL: 1)
//   RoPE:     pairs (c - R + 2j, c - R + 2j + 1), j < R/2, rotated by
//             pos * theta^(-2j/R)
//
// One wave per row, 8 consecutive elements per lane (rows of up to 512
// elements in one pass, longer rows in passes of 512).  Angles reach 2^20 rad,
// so the phase is formed and reduced in fp64; the rotation itself is fp32.
#include "dsv4_common.h"
#include "dsv4_internal.h"

namespace dsv4 {

constexpr int NR_THREADS = 256;
constexpr int NR_MAXC = 4096;          // widest row (8 passes of 512)
constexpr int NR_MAXR = 512;           // widest rotated block (R/2 <= 256 pairs)

__device__ __forceinline__ void load8(const void* p, int dtype, int64_t off, float (&x)[8]) {
  if (dtype == ACT_F32) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + off);
    const f32x4 b = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p) + off + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_to_f32(w[i] & 0xFFFFu); x[2 * i + 1] = bf16_to_f32(w[i] >> 16); }
  }
}

__device__ __forceinline__ void store8(void* p, int dtype, int64_t off, const float (&y)[8]) {
  if (dtype == ACT_F32) {
    float* q = reinterpret_cast<float*>(p) + off;
    *reinterpret_cast<f32x4*>(q) = (f32x4){y[0], y[1], y[2], y[3]};
    *reinterpret_cast<f32x4*>(q + 4) = (f32x4){y[4], y[5], y[6], y[7]};
  } else {
    *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p) + off) =
        (u32x4){pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
  }
}

// RMSNorm of one row held as NP passes of 8 elements per lane; returns 1/rms
template <int NP>
__device__ __forceinline__ float row_inv_rms(const float (&x)[NP][8], int c, int l, float eps) {
  float ss = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(x[p][i], x[p][i], ss);
  ss = wave_sum(ss);
  return 1.0f / sqrtf(ss / (float)c + eps);
}

// normalise (and rotate) one row in place; g holds this lane's gamma values,
// cs/sn[j] pair j's rotation
template <int NP>
__device__ __forceinline__ void norm_rope_row(float (&x)[NP][8], int c, int l, float eps, const float (&g)[NP][8],
                                              int R, const float* cs, const float* sn, bool norm) {
  const float inv = norm ? row_inv_rms<NP>(x, c, l, eps) : 1.0f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int e0 = 512 * p + 8 * l;
    if (e0 >= c) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[p][i] *= inv * g[p][i];
    if (e0 >= c - R) {
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const int j = (e0 + i - (c - R)) >> 1;
        rope_pair(x[p][i], x[p][i + 1], cs[j], sn[j]);
      }
    }
  }
}

// ---- queries: one block per (b, t); the rotation is shared by its heads
// a block takes QH heads of one query (grid.y splits the heads), or all of
// them for the output rotation
constexpr int QH = 16;
template <int NP>
__global__ __launch_bounds__(NR_THREADS) void q_norm_rope_k(QPrepArgs a, PosTable pt, int b0) {
  __shared__ float s_cs[NR_MAXR / 2], s_sn[NR_MAXR / 2];
  const int64_t bl = blockIdx.x / a.nq, t = blockIdx.x % a.nq;
  const int64_t pos = a.out_rot ? -(pt.q_pos0[bl] + t) : pt.q_pos0[bl] + t;
  for (int j = threadIdx.x; j < a.R / 2; j += NR_THREADS) rope_cs(pos, j, a.R, a.theta, &s_cs[j], &s_sn[j]);
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  float g[NP][8];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 512 * p + 8 * l + i;
      g[p][i] = (a.gamma && e < a.c) ? a.gamma[e] : 1.0f;
    }
  __syncthreads();
  const int64_t row0 = ((b0 + bl) * a.nq + t) * a.nh;
  const int hpb = a.out_rot ? a.nh : QH;         // heads per block
  const int hend = (int)(blockIdx.y + 1) * hpb < a.nh ? (int)(blockIdx.y + 1) * hpb : a.nh;
  // HB rows per wave at a time, their loads in flight together; the output
  // rotation reads and writes the rotated block only
  constexpr int HB = NP == 1 ? 4 : NP == 2 ? 2 : 1;
  constexpr int NW = NR_THREADS / 64;
  for (int h0 = (int)blockIdx.y * hpb + wv * HB; h0 < hend; h0 += NW * HB) {
    float x[HB][NP][8];
#pragma unroll
    for (int r = 0; r < HB; ++r) {
      const int64_t base = (row0 + (h0 + r < hend ? h0 + r : hend - 1)) * a.c;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int e0 = 512 * p + 8 * l;
        if (e0 < a.c && (!a.out_rot || e0 >= a.c - a.R)) load8(a.in, a.dtype, base + e0, x[r][p]);
        else
#pragma unroll
          for (int i = 0; i < 8; ++i) x[r][p][i] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < HB; ++r) {
      if (h0 + r >= hend) break;
      const int64_t base = (row0 + h0 + r) * a.c;
      norm_rope_row<NP>(x[r], a.c, l, a.eps, g, a.R, s_cs, s_sn, !a.out_rot);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int e0 = 512 * p + 8 * l;
        if (e0 < a.c && (!a.out_rot || e0 >= a.c - a.R)) store8(a.out, a.dtype, base + e0, x[r][p]);
      }
    }
  }
}

// ---- KV rows: one wave per row, row i of batch entry b at pos0[b] + stride i
template <int NP>
__global__ __launch_bounds__(NR_THREADS) void kv_norm_rope_k(KvPrepArgs a, PosTable pt, int b0, int nb) {
  const int wv = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * (NR_THREADS / 64) + wv;
  if (gw >= (int64_t)nb * a.n) return;
  const int64_t bl = gw / a.n, i = gw % a.n;
  const int64_t row = (b0 + bl) * a.n + i;
  const int64_t pos = pt.q_pos0[bl] + a.pos_stride * i;
  // pair j's rotation computed by lane j (and lane j + 64 k for wide blocks), handed out by shuffles
  constexpr int PPL = NR_MAXR / 2 / 64;       // pairs per lane
  float cl[PPL], sl[PPL];
#pragma unroll
  for (int k = 0; k < PPL; ++k) {
    const int j = l + 64 * k;
    cl[k] = 1.f; sl[k] = 0.f;
    if (j < a.R / 2) rope_cs(pos, j, a.R, a.theta, &cl[k], &sl[k]);
  }
  float x[NP][8];
  const int in_es = a.in_layout == ROW_F32 ? ACT_F32 : ACT_BF16;
  const uint8_t* src = reinterpret_cast<const uint8_t*>(a.in) + row * (int64_t)row_bytes(a.in_layout, a.c);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int e0 = 512 * p + 8 * l;
    if (e0 < a.c) load8(src, in_es, e0, x[p]);
    else
#pragma unroll
      for (int i2 = 0; i2 < 8; ++i2) x[p][i2] = 0.f;
  }
  const float inv = a.norm ? row_inv_rms<NP>(x, a.c, l, a.eps) : 1.0f;
  uint8_t* dst = reinterpret_cast<uint8_t*>(a.out) + row * (int64_t)row_bytes(a.out_layout, a.c);
  const int nf8 = a.c - ROPE_DIMS;              // E4M3 dims of an FP8 row
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int e0 = 512 * p + 8 * l;
    // shuffles are wave-wide: every lane takes part, the inactive ones discard
    float y[8];
#pragma unroll
    for (int i2 = 0; i2 < 8; ++i2) {
      const int e = e0 + i2 < a.c ? e0 + i2 : a.c - 1;
      y[i2] = x[p][i2] * inv * (a.norm && a.gamma ? a.gamma[e] : 1.0f);
    }
#pragma unroll
    for (int i2 = 0; i2 < 8; i2 += 2) {
      const int jr = (e0 + i2 - (a.c - a.R)) >> 1;          // pair index (negative: not rotated)
      const int jj = jr < 0 ? 0 : jr;
      float c = 1.f, s = 0.f;
#pragma unroll
      for (int k = 0; k < PPL; ++k) {
        const float ck = __shfl(cl[k], jj & 63), sk = __shfl(sl[k], jj & 63);
        if ((jj >> 6) == k) { c = ck; s = sk; }
      }
      if (jr >= 0 && e0 < a.c) {
        const float u = y[i2], v = y[i2 + 1];
        y[i2] = u * c - v * s;
        y[i2 + 1] = u * s + v * c;
      }
    }
    if (e0 >= a.c) continue;
    if (a.out_layout == ROW_F32 || a.out_layout == ROW_BF16) {
      store8(dst, a.out_layout == ROW_F32 ? ACT_F32 : ACT_BF16, e0, y);
    } else if (e0 < nf8) {                                   // 8 E4M3 bytes
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        w0 |= f32_to_e4m3(y[i2]) << (8 * i2);
        w1 |= f32_to_e4m3(y[4 + i2]) << (8 * i2);
      }
      *reinterpret_cast<u32x2*>(dst + e0) = (u32x2){w0, w1};
    } else {                                                 // 8 bf16 RoPE dims
      *reinterpret_cast<u32x4*>(dst + nf8 + 2 * (e0 - nf8)) =
          (u32x4){pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
    }
  }
}

hipError_t launch_q_prep(const QPrepArgs& a, const int64_t* q_pos0, hipStream_t s) {
  if (a.B <= 0 || a.nq <= 0) return hipSuccess;
  const int np = (a.c + 511) / 512;
  for (int64_t b0 = 0; b0 < a.B; b0 += MAXB) {
    const int nb = (int)(a.B - b0 < MAXB ? a.B - b0 : MAXB);
    PosTable pt;
    for (int i = 0; i < nb; ++i) { pt.q_pos0[i] = q_pos0[b0 + i]; pt.win_pos0[i] = 0; }
    // the output rotation moves little data per head: one block per query
    const dim3 grid((unsigned)(nb * a.nq), a.out_rot ? 1u : (unsigned)((a.nh + QH - 1) / QH));
    switch (np) {
      case 1: hipLaunchKernelGGL(q_norm_rope_k<1>, grid, dim3(NR_THREADS), 0, s, a, pt, (int)b0); break;
      case 2: hipLaunchKernelGGL(q_norm_rope_k<2>, grid, dim3(NR_THREADS), 0, s, a, pt, (int)b0); break;
      case 3: case 4: hipLaunchKernelGGL(q_norm_rope_k<4>, grid, dim3(NR_THREADS), 0, s, a, pt, (int)b0); break;
      default: hipLaunchKernelGGL(q_norm_rope_k<8>, grid, dim3(NR_THREADS), 0, s, a, pt, (int)b0); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_kv_prep(const KvPrepArgs& a, const int64_t* pos0, hipStream_t s) {
  if (a.B <= 0 || a.n <= 0) return hipSuccess;
  const int np = (a.c + 511) / 512;
  for (int64_t b0 = 0; b0 < a.B; b0 += MAXB) {
    const int nb = (int)(a.B - b0 < MAXB ? a.B - b0 : MAXB);
    PosTable pt;
    for (int i = 0; i < nb; ++i) { pt.q_pos0[i] = pos0[b0 + i]; pt.win_pos0[i] = 0; }
    const int64_t waves = (int64_t)nb * a.n;
    const dim3 grid((unsigned)((waves + NR_THREADS / 64 - 1) / (NR_THREADS / 64)));
    switch (np) {
      case 1: hipLaunchKernelGGL(kv_norm_rope_k<1>, grid, dim3(NR_THREADS), 0, s, a, pt, (int)b0, nb); break;
      case 2: hipLaunchKernelGGL(kv_norm_rope_k<2>, grid, dim3(NR_THREADS), 0, s, a, pt, (int)b0, nb); break;
      case 3: case 4: hipLaunchKernelGGL(kv_norm_rope_k<4>, grid, dim3(NR_THREADS), 0, s, a, pt, (int)b0, nb); break;
      default: hipLaunchKernelGGL(kv_norm_rope_k<8>, grid, dim3(NR_THREADS), 0, s, a, pt, (int)b0, nb); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dsv4
