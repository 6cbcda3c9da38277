// Device helpers shared by the gfx950 kernels of libdsv4attn: vector types,
// storage codecs (bf16, OCP E4M3, OCP E2M1/E8M0) and small wave utilities.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsv4_internal.h"

namespace dsv4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;

// ------------------------------------------------------------------ bf16

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// ------------------------------------------------------------------ OCP E4M3
// decode via the gfx950 conversion (OCP E4M3, exact into f32 and bf16)

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(byte, false)[0];
}

// Two E4M3 bytes (the low or high 16-bit word of w) -> two bf16 in one dword.
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi_word) {
  bf16x2 r = hi_word ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                     : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

// f32 -> E4M3, round to nearest even, saturating at +-448 (finite inputs).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  float a = fabsf(x);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);   // 8 -> 0x08, the smallest normal
  } else {
    uint32_t ua = __float_as_uint(a);
    ua += 0x7FFFFu + ((ua >> 20) & 1u);     // RNE at mantissa bit 20
    int e = (int)(ua >> 23) - 127;
    code = ((uint32_t)(e + 7) << 3) | ((ua >> 20) & 7u);
    if (e > 8 || code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// ------------------------------------------------------------------ OCP E2M1 / E8M0 (MXFP4)

// One MXFP4 byte (two E2M1 codes) times 2^(E-127) -> two bf16 (element 0 = low nibble).
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t byte_word, int byte_sel, float scale) {
  bf16x2 r;
  switch (byte_sel) {
    case 0: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(byte_word, scale, 0); break;
    case 1: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(byte_word, scale, 1); break;
    case 2: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(byte_word, scale, 2); break;
    default: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(byte_word, scale, 3); break;
  }
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t E) {
  return E == 0 ? 0x1p-127f : __uint_as_float(E << 23);
}

__device__ __forceinline__ float e2m1_to_f32(uint32_t nib) {
  const uint32_t mag = nib & 7u;
  float v = mag < 2 ? 0.5f * (float)mag : (mag < 4 ? 1.0f + 0.5f * (float)(mag - 2)
                                                   : (mag < 6 ? 2.0f + (float)(mag - 4) : (mag == 6 ? 4.0f : 6.0f)));
  return (nib & 8u) ? -v : v;
}

// y -> E2M1 code (sign bit 3), round to nearest even, saturating at 6.  The
// magnitude code counts the rounding boundaries |y| lies beyond; a boundary
// that is a tie belongs to the even code below or above it (branch-free).
__device__ __forceinline__ uint32_t f32_to_e2m1(float y) {
  const float a = fabsf(y);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return m | ((__float_as_uint(y) >> 28) & 8u);
}

// Shared scale exponent of an MXFP4 block from its largest magnitude:
// E8M0 code of 2^(floor(log2 amax) - 2); amax == 0 -> 0.
__device__ __forceinline__ uint32_t mx_scale_code(float amax) {
  if (!(amax > 0.0f)) return 0u;
  int ef = (int)(__float_as_uint(amax) >> 23);   // biased exponent of amax
  int E = ef - 2;
  return (uint32_t)(E < 0 ? 0 : (E > 254 ? 254 : E));
}

// E8M0 code of the MXFP8 (E4M3) block scale 2^(floor(log2 amax) - 8)
__device__ __forceinline__ uint32_t mx8_scale_code(float amax) {
  if (!(amax > 0.0f)) return 0u;
  int E = (int)(__float_as_uint(amax) >> 23) - 8;
  return (uint32_t)(E < 0 ? 0 : (E > 254 ? 254 : E));
}

// ------------------------------------------------------------------ global -> LDS copies

// 16-byte global -> LDS copy of every lane: lane l's bytes from gsrc + OFF land
// at LDS address lds_base + 16 l (lds_base wave-uniform).  The instruction's
// immediate offset is added to the LDS address as well as to the global one,
// so M0 is set to lds_base - OFF (one wait state between the M0 write and the
// copy that reads it).  Written as a three-instruction asm block (M0 set in the
// same block) so that the compiler does not track it: callers wait for these
// copies themselves (vmcnt) before reading the destination.  The instruction
// has no register results, so nothing is written back into VGPRs while it is
// in flight.
template <int OFF>
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_base) {
  static_assert(OFF >= 0 && OFF < 4096, "global offset is a 13-bit signed immediate");
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2"
               : : "v"(gsrc), "s"(lds_base - (uint32_t)OFF), "i"(OFF) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)(p);
}

// ------------------------------------------------------------------ generic row access

__host__ __device__ __forceinline__ int row_bytes(int layout, int c) {
  return layout == ROW_F32 ? 4 * c : layout == ROW_BF16 ? 2 * c : layout == ROW_FP8 ? c + ROPE_DIMS : c / 2;
}

// element j of a stored row (not MXFP4)
__device__ __forceinline__ float load_row_elem(const uint8_t* row, int layout, int c, int j) {
  if (layout == ROW_F32) return reinterpret_cast<const float*>(row)[j];
  if (layout == ROW_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[j]);
  // ROW_FP8: E4M3 dims then bf16 RoPE dims
  const int nf8 = c - ROPE_DIMS;
  if (j < nf8) return e4m3_to_f32(row[j]);
  return bf16_to_f32(reinterpret_cast<const uint16_t*>(row + nf8)[j - nf8]);
}

__device__ __forceinline__ float load_act(const void* p, int dtype, int64_t i) {
  return dtype == ACT_F32 ? reinterpret_cast<const float*>(p)[i]
                          : bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

__device__ __forceinline__ void store_act(void* p, int dtype, int64_t i, float v) {
  if (dtype == ACT_F32) reinterpret_cast<float*>(p)[i] = v;
  else reinterpret_cast<uint16_t*>(p)[i] = (uint16_t)f32_to_bf16(v);
}

// store element j of a row in `layout` (not MXFP4)
__device__ __forceinline__ void store_row_elem(uint8_t* row, int layout, int c, int j, float v) {
  if (layout == ROW_F32) { reinterpret_cast<float*>(row)[j] = v; return; }
  if (layout == ROW_BF16) { reinterpret_cast<uint16_t*>(row)[j] = (uint16_t)f32_to_bf16(v); return; }
  const int nf8 = c - ROPE_DIMS;
  if (j < nf8) row[j] = (uint8_t)f32_to_e4m3(v);
  else reinterpret_cast<uint16_t*>(row + nf8)[j - nf8] = (uint16_t)f32_to_bf16(v);
}

// RoPE rotation of one pair by the angle with cosine c and sine s, in one
// fixed rounding order (every rotation that must agree bit for bit with
// another, such as the output rotation fused into an attention store and the
// separate output-rotation call, goes through here)
__device__ __forceinline__ void rope_pair(float& x0, float& x1, float c, float s) {
  const float a = x0, b = x1;
  x0 = fmaf(a, c, -(b * s));
  x1 = fmaf(a, s, b * c);
}

// cos / sin of pos * theta^(-2j/R)
__device__ __forceinline__ void rope_cs(int64_t pos, int j, int R, float theta, float* c, float* s) {
  const double inv = exp2(-2.0 * (double)j / (double)R * log2((double)theta));
  double ang = (double)pos * inv;
  // reduce to [-pi, pi] in fp64 before the fp64 sincos
  const double twopi = 6.283185307179586476925286766559;
  ang -= twopi * rint(ang / twopi);
  double sd, cd;
  sincos(ang, &sd, &cd);
  *c = (float)cd;
  *s = (float)sd;
}

// ------------------------------------------------------------------ wave helpers

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// v combined with the value of lane l ^ 32, for every lane, by one
// v_permlane32_swap (a VALU exchange of the wave's halves, no LDS round trip).
// The swap leaves {v[l], v[l ^ 32]} in its two results, in an order that
// depends on the half; max and sum do not care, so the results equal those of
// an exchange through LDS bit for bit.
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ------------------------------------------------------------------ top-k order keys
// Order-preserving uint32 key of an fp32 score (-0.0 ties with +0.0), and the
// unique composite (key << 32 | ~index): "score descending, ties to the lower
// index" is plain descending order of the composite.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
  return ((uint64_t)key << 32) | (uint64_t)(~idx);
}

}  // namespace dsv4
