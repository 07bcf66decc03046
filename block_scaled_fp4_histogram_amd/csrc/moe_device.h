// Device helpers shared by the gfx950 kernels: number formats, MXFP8
// quantisation, MFMA wrappers and the register dequantisation of NVFP4 / NF3
// weight tiles.
#pragma once

#include "moe_common.h"

namespace moe {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ numerics

// Shared exponent of an MXFP8 block: E = floor(log2 amax) - 8, clamped to
// [-127, 127]; returns the E8M0 byte E + 127 and the multiplier 2^-E.
__device__ __forceinline__ uint32_t mx_scale(float amax, float *inv_scale) {
  const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFFu);   // amax >= 0
  const int E = max(ex - 135, -127);
  *inv_scale = __uint_as_float((uint32_t)(127 - E) << 23);
  return (uint32_t)(E + 127);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// E2M1 code (4 bits) -> fp32.
__device__ __forceinline__ float e2m1_f32(uint32_t c) {
  const uint32_t m = c & 7u;
  const uint32_t bits = (m < 2u) ? (m * 0x3F000000u) : ((m + 252u) << 22);
  return __uint_as_float(bits | ((c & 8u) << 28));
}

// E4M3 (fn) byte -> fp32 (NaN codes are out of contract).
__device__ __forceinline__ float e4m3_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (b & 0x80u) ? -v : v;
}

__device__ __forceinline__ float silu_clamped(float gate, float up, float limit, int has_limit) {
  if (has_limit) {
    gate = fminf(gate, limit);
    up = fminf(fmaxf(up, -limit), limit);
  }
  return gate / (1.0f + __expf(-gate)) * up;
}

// Two fp32 -> two E4M3 (fn) codes (bits 0-7, 8-15), nearest with ties to even,
// magnitudes above 448 saturating to 448.  The hardware conversion rounds to
// nearest even (subnormals included) but turns magnitudes above 464 into NaN,
// so inputs are clamped to +-448 first.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four scaled values -> one dword of E4M3 codes.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d, float inv) {
  return e4m3x2(a * inv, b * inv) | (e4m3x2(c * inv, d * inv) << 16);
}

// Quantise 32 fp32 values to MXFP8 (codes packed 4 per dword).
__device__ __forceinline__ uint32_t quant_block32(const float *v, uint32_t *codes) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; i++) amax = fmaxf(amax, fabsf(v[i]));
  float inv;
  const uint32_t sb = mx_scale(amax, &inv);
#pragma unroll
  for (int i = 0; i < 8; i++) codes[i] = e4m3x4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3], inv);
  return sb;
}

// MFMA operand of an FP4 weight tile (16 bytes per lane in the low 4 VGPRs).
__device__ __forceinline__ v8i fp4_operand(v4i a) { return v8i{a[0], a[1], a[2], a[3], 0, 0, 0, 0}; }

// Block-scaled MFMA: A = 16 rows x 128 k of E2M1 (scale sa), B = 128 k x 16 columns of E4M3 (scale sb).
__device__ __forceinline__ v4f mfma_fp4_fp8(v4i a, v8i b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fp4_operand(a), b, c, 4, 0, 0, sa, 0, sb);
}

// ------------------------------------------- W4A16 (NVFP4) / W3A16 (NF3)

// Weight tiles as for MXFP4 (lane l = row + 16*q holds 32 consecutive columns of
// its row; 16 bytes for NVFP4, 12 bytes = four 3-byte NF3 groups), scales 2
// bytes per lane (NVFP4, E4M3 per 16) or 1 byte (NF3, E4M3 per 32).  The bf16
// MFMA v_mfma_f32_16x16x32_bf16 takes 8 consecutive k per lane group; lane l
// feeds its 32 columns in 4 steps of 8, and the activation operand walks the
// same columns, so each step pairs the same k on both sides.

// 8 fp4 codes (one dword) x scale -> 8 bf16 (exact: E2M1 x E4M3 fits bf16).
__device__ __forceinline__ v8bf nvfp4_step(uint32_t w, float sc) {
  v4i r;
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const uint32_t byte = (w >> (8 * m)) & 0xFFu;
    const float lo = e2m1_f32(byte & 15u) * sc, hi = e2m1_f32(byte >> 4) * sc;
    r[m] = (int)__builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  return __builtin_bit_cast(v8bf, r);
}

// NF3 magnitudes |codebook| ascending; code c >= 4 is +mag[c-4], c < 4 is -mag[3-c].
__device__ __forceinline__ float nf3_val(uint32_t c, float m0, float m1, float m2, float m3) {
  const uint32_t mi = (c & 4u) ? (c & 3u) : (3u - (c & 3u));
  const float v = (mi & 2u) ? ((mi & 1u) ? m3 : m2) : ((mi & 1u) ? m1 : m0);
  return (c & 4u) ? v : -v;
}

// 8 NF3 codes (one 24-bit group) -> 8 bf16 (codebook x scale, rounded to bf16).
__device__ __forceinline__ v8bf nf3_step(uint32_t w24, float m0, float m1, float m2, float m3) {
  v4i r;
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const float lo = nf3_val((w24 >> (6 * m)) & 7u, m0, m1, m2, m3);
    const float hi = nf3_val((w24 >> (6 * m + 3)) & 7u, m0, m1, m2, m3);
    r[m] = (int)pack_bf16x2(lo, hi);
  }
  return __builtin_bit_cast(v8bf, r);
}

// Dequantised operand of one lane for k-step s (0..3) of a 128-column k-tile.
template <int WF>
struct A16Tile {
  uint32_t d[4];   // NVFP4: 4 dwords of codes; NF3: 3 dwords (12 bytes)
  uint32_t sc;     // scale byte(s)
  __device__ __forceinline__ void load(const uint8_t *data, const uint8_t *scales) {
    if (WF == W_NVFP4) {
      const v4i v = *(const v4i *)data;
      d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
      sc = *(const uint16_t *)scales;
    } else {
      const uint32_t *p = (const uint32_t *)data;
      d[0] = p[0]; d[1] = p[1]; d[2] = p[2]; d[3] = 0;
      sc = *scales;
    }
  }
  __device__ __forceinline__ void zero() { d[0] = d[1] = d[2] = d[3] = 0; sc = 0; }
  __device__ __forceinline__ v8bf step(int s) const {
    if (WF == W_NVFP4) {
      return nvfp4_step(d[s], e4m3_f32(s < 2 ? (sc & 0xFFu) : (sc >> 8)));
    } else {
      const float f = e4m3_f32(sc);
      // group s of 24 bits starts at bit 24*s of the 96-bit lane word
      const uint64_t lo = (uint64_t)d[0] | ((uint64_t)d[1] << 32);
      uint32_t w24;
      if (s == 0) w24 = (uint32_t)lo & 0xFFFFFFu;
      else if (s == 1) w24 = (uint32_t)(lo >> 24) & 0xFFFFFFu;
      else if (s == 2) w24 = (uint32_t)((lo >> 48) | ((uint64_t)d[2] << 16)) & 0xFFFFFFu;
      else w24 = d[2] >> 8;
      return nf3_step(w24, 0.1275f * f, 0.3563f * f, 0.6047f * f, f);
    }
  }
};

template <int WF>
struct FmtGeom {
  static constexpr int unit = (WF == W_NF3) ? 12 : 16;   // data bytes per (row, 32-col group)
  static constexpr int sunit = (WF == W_NVFP4) ? 2 : 1;  // scale bytes per (row, 32-col group)
};

__device__ __forceinline__ v4f mfma_bf16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}


// ------------------------------------------------ GEMM1 k-tile stages

// Operands of one 128-column k-tile of GEMM1 for one lane: the up and gate
// row tiles of two adjacent 16-column intermediate blocks, and the token's
// MXFP8 activation slice.
struct A8G1Stage {
  v4i A[4];
  int sa[4];
  v4i B0, B1;
  int sb;
};

__device__ __forceinline__ void a8g1_load(A8G1Stage &st, const uint8_t *wt, const uint8_t *sp, size_t rt_bytes,
                                          size_t rt_scales, int kt, const uint8_t *xrow, const uint8_t *xsrow,
                                          bool have, int g) {
#pragma unroll
  for (int q = 0; q < 4; q++) {
    st.A[q] = *(const v4i *)(wt + q * rt_bytes + (size_t)kt * 1024);
    st.sa[q] = sp[q * rt_scales + kt * 64];
  }
  if (have) {
    st.B0 = *(const v4i *)(xrow + kt * 128 + 16 * g);
    st.B1 = *(const v4i *)(xrow + kt * 128 + 64 + 16 * g);
    st.sb = xsrow[kt * 4 + g];
  } else {
    st.B0 = v4i{0, 0, 0, 0};
    st.B1 = v4i{0, 0, 0, 0};
    st.sb = 0;
  }
}

__device__ __forceinline__ void a8g1_compute(const A8G1Stage &st, v4f *acc) {
  const v8i bop = v8i{st.B0[0], st.B0[1], st.B0[2], st.B0[3], st.B1[0], st.B1[1], st.B1[2], st.B1[3]};
#pragma unroll
  for (int q = 0; q < 4; q++) acc[q] = mfma_fp4_fp8(st.A[q], bop, acc[q], st.sa[q], st.sb);
}

template <int WF>
struct A16G1Stage {
  A16Tile<WF> A[4];
  v4i B[4];
};

template <int WF>
__device__ __forceinline__ void a16g1_load(A16G1Stage<WF> &st, const uint8_t *wt, const uint8_t *sp, size_t rt_bytes,
                                           size_t rt_scales, int kt, const uint16_t *xrow, bool have, int g) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
#pragma unroll
  for (int q = 0; q < 4; q++) st.A[q].load(wt + q * rt_bytes + (size_t)kt * 64 * U, sp + q * rt_scales + kt * 64 * SU);
  if (have) {
    const v4i *xp = (const v4i *)(xrow + kt * 128 + 32 * g);
#pragma unroll
    for (int s = 0; s < 4; s++) st.B[s] = xp[s];
  } else {
#pragma unroll
    for (int s = 0; s < 4; s++) st.B[s] = v4i{0, 0, 0, 0};
  }
}

template <int WF>
__device__ __forceinline__ void a16g1_compute(const A16G1Stage<WF> &st, v4f *acc) {
#pragma unroll
  for (int s = 0; s < 4; s++) {
    const v8bf b = __builtin_bit_cast(v8bf, st.B[s]);
#pragma unroll
    for (int q = 0; q < 4; q++) acc[q] = mfma_bf16(st.A[q].step(s), b, acc[q]);
  }
}

}  // namespace moe
