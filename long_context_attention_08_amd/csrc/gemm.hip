// bf16 GEMM C = A B^T with fp32 accumulation, for the low-rank query path and
// the grouped output projection (DeepSeek-V4 digest, 模块 B: c^Q = h W^DQ,
// q = c^Q W^UQ, q^I = c^Q W^IUQ, w^I = h W^w; the n_h head outputs in g groups,
// each projected to d_g, then concatenated and projected to d).
//
// A [M, K] and B [N, K] are both K-contiguous (the [out, in] weight layout),
// C [M, N] row-major in bf16 or fp32; grid.z runs a batch with element strides.
// Block tile BM x BN x 64, four waves in 2 x 2, each wave (BM/2) x (BN/2) in
// 32x32 tiles of v_mfma_f32_32x32x16_bf16 (accumulators in AGPRs at 256 x 256).
// Tiles travel global -> LDS by global_load_lds_dwordx4 into an XOR-swizzled
// layout (16-byte chunk j of row r at chunk j ^ ((r >> 1) & 7): 16 consecutive
// 128-byte rows in distinct 16-byte groups of the 64 LDS banks), two stages, one
// block barrier per K tile: the copies of tile k+1 run under the MFMAs of tile
// k.  Rows past M or N read the last valid row; their results are not stored.
#include "dsv4_common.h"
#include "dsv4_internal.h"

namespace dsv4 {

constexpr int GK = 64;           // K per tile: 128 bytes of bf16 per row

template <int BM, int BN>
__global__ __launch_bounds__(256, 1) void gemm_nt(GemmArgs a, int tiles_n, int xcd_map, int GM) {
  constexpr int WM = BM / 2, WN = BN / 2, TM = WM / 32, TN = WN / 32;
  constexpr int ASZ = BM * GK * 2, BSZ = BN * GK * 2;      // bytes of one stage
  constexpr int CA = BM / 8 / 4, CB = BN / 8 / 4;           // 1 KB copies per wave and tile
  __shared__ __align__(16) uint8_t s_a[2 * ASZ];
  __shared__ __align__(16) uint8_t s_b[2 * BSZ];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63, G = l >> 5, col = l & 31;
  const int wm = wv >> 1, wn = wv & 1;
  // tile order: with xcd_map, the 8 XCDs (blocks are dealt round-robin) each
  // get a contiguous run of tile numbers; numbers run down groups of GM
  // tile-rows before moving right.  GM = 8 makes the blocks an XCD runs at once
  // a patch of about 8 x 4 tiles sharing both A and B tiles in L2 (long K);
  // GM = 1 is plain row order, whose C writes spread over more HBM channels
  // when K is short and the kernel is bound by writing C
  int64_t t = blockIdx.x;
  if (xcd_map) t = (t & 7) * (gridDim.x >> 3) + (t >> 3);
  const int64_t tiles_m = gridDim.x / tiles_n;
  const int64_t grp = t / (GM * tiles_n), first = grp * GM;
  const int64_t gm = tiles_m - first < GM ? tiles_m - first : GM;
  const int64_t in = t - grp * GM * tiles_n;
  const int64_t m0 = (first + in % gm) * BM, n0 = (in / gm) * BN;
  const uint16_t* A = reinterpret_cast<const uint16_t*>(a.A) + (int64_t)blockIdx.z * a.sA;
  const uint16_t* B = reinterpret_cast<const uint16_t*>(a.B) + (int64_t)blockIdx.z * a.sB;

  // copy q of a tile covers rows [8q, 8q + 8): lane L takes row 8q + L/8 and
  // writes LDS chunk L % 8, which holds global chunk (L % 8) ^ ((row >> 1) & 7);
  // this wave's copies are q = wv + 4 i, so (row >> 1) & 7 = (4 wv + L/16) & 7
  const int crow = l >> 3, gch = (l & 7) ^ ((4 * wv + (crow >> 1)) & 7);
  auto src_row = [](const uint16_t* X, int64_t r0, int64_t r, int64_t rows, int64_t ld) {
    const int64_t rr = r0 + r < rows ? r0 + r : rows - 1;
    return X + rr * ld;
  };
  // copy i of this wave reads row 8 (wv + 4 i) + crow: when the whole tile is
  // in range that is base + 32 i rows; at a ragged edge every row is clamped
  const bool fa = m0 + BM <= a.M, fb = n0 + BN <= a.N;
  const uint16_t* pa0 = src_row(A, m0, 8 * wv + crow, a.M, a.lda) + 8 * gch;
  const uint16_t* pb0 = src_row(B, n0, 8 * wv + crow, a.N, a.ldb) + 8 * gch;
  const uint32_t la = lds_addr(s_a), lb = lds_addr(s_b);
  auto issue = [&](int kt, int st) {
    const int64_t k0 = (int64_t)kt * GK;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const uint16_t* p = fa ? pa0 + 32 * i * a.lda : src_row(A, m0, 8 * (wv + 4 * i) + crow, a.M, a.lda) + 8 * gch;
      dma16<0>(p + k0, la + st * ASZ + 1024 * (wv + 4 * i));
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const uint16_t* p = fb ? pb0 + 32 * i * a.ldb : src_row(B, n0, 8 * (wv + 4 * i) + crow, a.N, a.ldb) + 8 * gch;
      dma16<0>(p + k0, lb + st * BSZ + 1024 * (wv + 4 * i));
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // fragment rows of this lane and their swizzle
  const int ra0 = wm * WM + col, rb0 = wn * WN + col;       // + 32 i / 32 j; (r >> 1) & 7 is (col >> 1) & 7
  const int sw = (col >> 1) & 7;
  const int nk = (int)(a.K / GK);
  issue(0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0): this wave's copies of tile kt
    __builtin_amdgcn_s_waitcnt(0xC07F);                       // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();                             // every copy landed; stage st ^ 1 is free
    if (kt + 1 < nk) issue(kt + 1, st ^ 1);
    const uint8_t* ta = s_a + st * ASZ;
    const uint8_t* tb = s_b + st * BSZ;
#pragma unroll
    for (int kk = 0; kk < GK / 16; ++kk) {
      const int ch = ((2 * kk + G) ^ sw) * 16;
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(ta + (ra0 + 32 * i) * 128 + ch));
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(tb + (rb0 + 32 * j) * 128 + ch));
      // the B tile is the MFMA's row operand: each accumulator is a 32 x 32
      // tile of C^T, so a lane ends up with 4 consecutive columns of C rows
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: lane holds row m = m0 + wm WM + 32 i + col and, in registers
  // 4q .. 4q+3, columns n0 + wn WN + 32 j + 8 q + 4 G .. + 3: one 8-byte (bf16)
  // or 16-byte (fp32) store each when the row is aligned and in range
  uint8_t* C = reinterpret_cast<uint8_t*>(a.C) + (int64_t)blockIdx.z * a.sC * (a.c_f32 ? 4 : 2);
  const bool vec = (a.ldc & 3) == 0 && ((uintptr_t)C & 15) == 0;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + wm * WM + 32 * i + col;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n = n0 + wn * WN + 32 * j + 8 * q + 4 * G;
        const f32x16& v = acc[i][j];
        if (vec && n + 3 < a.N) {
          if (a.c_f32)
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(C) + m * a.ldc + n) =
                (f32x4){v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
          else
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(C) + m * a.ldc + n) =
                (u32x2){pack_bf16x2(v[4 * q], v[4 * q + 1]), pack_bf16x2(v[4 * q + 2], v[4 * q + 3])};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (n + e >= a.N) break;
            if (a.c_f32) reinterpret_cast<float*>(C)[m * a.ldc + n + e] = v[4 * q + e];
            else reinterpret_cast<uint16_t*>(C)[m * a.ldc + n + e] = (uint16_t)f32_to_bf16(v[4 * q + e]);
          }
        }
      }
  }
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.batch <= 0) return hipSuccess;
  const int64_t big = ((a.M + 255) / 256) * ((a.N + 255) / 256) * a.batch;
  if (big >= 256) {
    const int tn = (int)((a.N + 255) / 256);
    const int64_t tiles = ((a.M + 255) / 256) * tn;
    hipLaunchKernelGGL((gemm_nt<256, 256>), dim3((unsigned)tiles, 1, (unsigned)a.batch), dim3(256), 0, s, a, tn,
                       tiles % 8 == 0 ? 1 : 0, a.K >= 4096 && tn >= 16 ? 8 : 1);
  } else {
    const int tn = (int)((a.N + 127) / 128);
    const int64_t tiles = ((a.M + 127) / 128) * tn;
    hipLaunchKernelGGL((gemm_nt<128, 128>), dim3((unsigned)tiles, 1, (unsigned)a.batch), dim3(256), 0, s, a, tn,
                       tiles % 8 == 0 ? 1 : 0, a.K >= 4096 && tn >= 16 ? 8 : 1);
  }
  return hipGetLastError();
}

}  // namespace dsv4
