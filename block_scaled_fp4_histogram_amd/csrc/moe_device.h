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
typedef float v2f __attribute__((ext_vector_type(2)));

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

// Two fp32 -> two bf16 (low, high half), nearest with ties to even, i.e.
// (u + 0x7FFF + bit 16 of u) >> 16 on each value's bits.  gfx950's
// v_cvt_pk_bf16_f32 gives exactly that for every finite input, denormals and
// overflow to infinity included (compared over all 2^32 bit patterns on the
// GPU), in one instruction for the pair.
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{lo, hi}, v2bf));
}

// E4M3 (fn) byte (the low byte of b) -> fp32, exact, by gfx950's FP8
// conversion (OCP E4M3: bias 7, subnormals m * 2^-9; NaN codes are out of
// contract).  One instruction and no branches, so a scale decoded once per
// loaded tile stays cheap next to the dequantisation it feeds.
__device__ __forceinline__ float e4m3_f32(uint32_t b) { return __builtin_amdgcn_cvt_f32_fp8((int)b, 0); }

// The same decode from the bit fields, with the subnormal case on a branch of
// its own.  The prefill W4A16/W3A16 k-loops keep this form: its control flow
// bounds the compiler's scheduling regions there, and with any branch-free
// decode their register use rises from about 245 to 300 VGPRs (one wave per
// SIMD instead of two), which measured 45 % slower.
__device__ __forceinline__ float e4m3_f32_branched(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (b & 0x80u) ? -v : v;
}

// Activation of one intermediate column from its GEMM1 pair.  act == ACT_SITU:
// both branches softly capped by tanh, silu(4 tanh(gate / 4)) * 25 tanh(up / 25)
// (vLLM "fused_moe/b12x" page: SiTU with beta 4 and linear beta 25, no limit).
// Otherwise the SwiGLU, with the limit clamps and the OAI alpha / beta.
__device__ __forceinline__ float silu_clamped(float gate, float up, float limit, int has_limit, float alpha,
                                              float beta, int act = ACT_SWIGLU) {
  // the sigmoid's reciprocal by v_rcp_f32 (1 ulp), not a correctly rounded
  // division (about ten instructions): the prefill epilogues run it for every
  // intermediate value
  if (act == ACT_SITU) {
    const float g = 4.0f * tanhf(0.25f * gate), u = 25.0f * tanhf(0.04f * up);
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
  }
  if (has_limit) {
    gate = fminf(gate, limit);
    up = fminf(fmaxf(up, -limit), limit);
  }
  // alpha = 1, beta = 0: silu(gate) * up; otherwise the OAI form gate * sigmoid(alpha gate) * (up + beta)
  return gate * __builtin_amdgcn_rcpf(1.0f + __expf(-alpha * gate)) * (up + beta);
}

// ReLU^2 without the gate multiply (vLLM "fused_moe/b12x" page, RELU2_NO_MUL):
// each GEMM1 output z gives its own intermediate column relu(z)^2.
__device__ __forceinline__ float relu2(float z) { return z > 0.f ? z * z : 0.f; }

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

// Quantise 32 bf16 values (4 x 16 bytes, element order) to MXFP8 without
// unpacking them first: the block maximum is the integer maximum of the bf16
// magnitude bits (same order as the values), then pairs are converted in place.
__device__ __forceinline__ uint32_t quant_block32_bf16(const v4i *x, uint32_t *codes) {
  uint32_t mbits = 0;
#pragma unroll
  for (int q = 0; q < 4; q++)
#pragma unroll
    for (int d = 0; d < 4; d++) {
      const uint32_t w = (uint32_t)x[q][d];
      mbits = max(mbits, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
    }
  float inv;
  const uint32_t sb = mx_scale(__uint_as_float(mbits << 16), &inv);
#pragma unroll
  for (int q = 0; q < 4; q++)
#pragma unroll
    for (int d = 0; d < 4; d += 2) {
      const uint32_t w0 = (uint32_t)x[q][d], w1 = (uint32_t)x[q][d + 1];
      codes[2 * q + d / 2] = e4m3x4(bf16_to_f32(w0 & 0xFFFFu), bf16_to_f32(w0 >> 16), bf16_to_f32(w1 & 0xFFFFu),
                                    bf16_to_f32(w1 >> 16), inv);
    }
  return sb;
}

// ------------------------------------------------------------ buffer loads
//
// Weight streams go through raw buffer loads: a wave-uniform 128-bit resource
// (base address, byte range) in scalar registers plus a 32-bit offset per lane,
// so no 64-bit per-lane address is formed.  Loads beyond the range return 0.
typedef int v3i __attribute__((ext_vector_type(3)));
extern "C" __device__ v4i moe_raw_buffer_load_v4i32(v4i rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.v4i32");
extern "C" __device__ v3i moe_raw_buffer_load_v3i32(v4i rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.v3i32");
extern "C" __device__ unsigned int moe_raw_buffer_load_i32(v4i rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.i32");
extern "C" __device__ unsigned short moe_raw_buffer_load_i16(v4i rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.i16");
extern "C" __device__ unsigned char moe_raw_buffer_load_i8(v4i rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.i8");

struct Buf {
  v4i r;
};

// Resource over [base, base + bytes); word 3 is the gfx9 default data format.
__device__ __forceinline__ Buf make_buf(const void *base, uint32_t bytes) {
  const uint64_t p = (uint64_t)base;
  Buf b;
  b.r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  b.r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  b.r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  b.r[3] = 0x00020000;
  return b;
}

__device__ __forceinline__ v4i buf_load16(const Buf &b, uint32_t voff, uint32_t soff) {
  return moe_raw_buffer_load_v4i32(b.r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ v3i buf_load12(const Buf &b, uint32_t voff, uint32_t soff) {
  return moe_raw_buffer_load_v3i32(b.r, (int)voff, (int)soff, 0);
}
// Non-temporal forms (the nt cache-policy bit) for streams read once, such as
// the decode kernels' weights: the caches do not keep their dead lines
// (decode layer at K = 7168: 48.6 -> 44.4 us).
constexpr int kNT = 2;
__device__ __forceinline__ v4i buf_load16_nt(const Buf &b, uint32_t voff, uint32_t soff) {
  return moe_raw_buffer_load_v4i32(b.r, (int)voff, (int)soff, kNT);
}
__device__ __forceinline__ v3i buf_load12_nt(const Buf &b, uint32_t voff, uint32_t soff) {
  return moe_raw_buffer_load_v3i32(b.r, (int)voff, (int)soff, kNT);
}
__device__ __forceinline__ uint32_t buf_load4(const Buf &b, uint32_t voff, uint32_t soff) {
  return moe_raw_buffer_load_i32(b.r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t buf_load2(const Buf &b, uint32_t voff, uint32_t soff) {
  return moe_raw_buffer_load_i16(b.r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t buf_load1(const Buf &b, uint32_t voff, uint32_t soff) {
  return moe_raw_buffer_load_i8(b.r, (int)voff, (int)soff, 0);
}

// Direct global -> LDS loads: lane i of the wave writes lds + i * bytes (the
// LDS address is wave-uniform).  They count in vmcnt like any vector load.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void dma16(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void *)lds, 4, 0, 0);
}

// s_waitcnt vmcnt(n), other counters untouched (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt lgkmcnt(0), other counters untouched.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

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

// 8 fp4 codes (one dword, element 2i in the low nibble of byte i) x scale -> 8
// bf16, exact (an E2M1 value times an E4M3 scale has at most 5 significant
// bits, so the fp32 product's upper half is the bf16 value).
// v_cvt_scalef32_pk_f32_fp4 decodes the two codes of one byte; its scale
// operand only contributes a power of two, so it is 1 here and the E4M3 scale
// is applied with an fp32 multiply.
__device__ __forceinline__ v8bf nvfp4_step(uint32_t w, float sc) {
  v4i r;
#pragma unroll
  for (int m = 0; m < 4; m++) {
    v2f f;
    if (m == 0) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    else if (m == 1) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    else if (m == 2) f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    else f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    const float lo = f[0] * sc, hi = f[1] * sc;
    r[m] = (int)__builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  return __builtin_bit_cast(v8bf, r);
}

// NF3 codes in tile layout.  A code c stands for +mag[c - 4] (c >= 4) or
// -mag[3 - c] (c < 4), mag ascending {0.1275, 0.3563, 0.6047, 1}.  The
// repacker rewrites each lane's 12 bytes (32 codes: 3 bits each, code e at bit
// 3e) as a sign bit and a 2-bit magnitude index per code, placed so that one
// shift and mask give a byte-permute selector and one shift gives the sign:
//   d0 / d1: magnitude indices of codes 0..15 / 16..31; for code e = 8 s + 2 m
//     + h (step s, pair m, half h) at bits 8 (s & 1) + 2 m + 16 h of d[s >> 1];
//   d2: sign of code e (1 = negative) at bit 15 - (4 s + m) + 16 h.
// The same number of bits as the packed codes, so no extra HBM traffic.
// t01 / t23: the bf16 magnitudes times the group's scale (rounded once),
// entries 0, 1 and 2, 3 in the low / high halves.
__device__ __forceinline__ void nf3_tables(float f, uint32_t &t01, uint32_t &t23) {
  t01 = pack_bf16x2(0.1275f * f, 0.3563f * f);
  t23 = pack_bf16x2(0.6047f * f, f);
}

// 8 codes of step s (dsel = d0 for s < 2, else d1) -> 8 bf16: per code pair a
// byte permute picks both magnitudes, then the two sign bits are or-ed in.
__device__ __forceinline__ v8bf nf3_step_rc(uint32_t dsel, uint32_t d2, int s, uint32_t t01, uint32_t t23) {
  v4i r;
#pragma unroll
  for (int m = 0; m < 4; m++) {
    const uint32_t x = (dsel >> (8 * (s & 1) + 2 * m)) & 0x00030003u;   // index of code 2m at bit 0, 2m+1 at bit 16
    const uint32_t sel = x * 0x0202u + 0x01000100u;                      // bytes 2i, 2i + 1 of each half's entry
    r[m] = (int)(__builtin_amdgcn_perm(t23, t01, sel) | ((d2 << (4 * s + m)) & 0x80008000u));
  }
  return __builtin_bit_cast(v8bf, r);
}

// ------------------------------------------- the same operands in fp16
//
// An NVFP4 weight value (E2M1 code times E4M3 scale: at most five significant
// bits, magnitudes 2^-10 .. 2688) and a scaled NF3 table entry (a bf16 value
// between about 2^-12 and 448) are exact in fp16 as they are in bf16.  In fp16
// the scale goes onto two values at once: v_cvt_scalef32_pk_f16_fp4 decodes a
// byte's two codes and one packed 16-bit multiply scales them, one instruction
// a value against two for bf16, for which gfx950 has no packed multiply.  The
// activations must then be fp16 too: a bf16 row is multiplied by the power of
// two 2^-e that puts its largest magnitude in [2^14, 2^15) and converted, which
// is exact for every element above 2^-28 of that maximum (bf16's 8 significant
// bits fit fp16's 11 wherever the scaled value is an fp16 normal); the sums are
// multiplied back by 2^e.  fp16 x fp16 products are exact in the MFMA's fp32 as
// bf16 products are, so only elements below 2^-28 of their row's largest
// round differently from the bf16 form.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v4f mfma_f16(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The two E4M3 scales in the low 16 bits of b as an fp16 pair (exact).
__device__ __forceinline__ v2h e4m3x2_h(uint32_t b) { return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false); }

// 8 fp4 codes (as for nvfp4_step) x scale sc -> 8 fp16, exact.
__device__ __forceinline__ v8h nvfp4_step_h(uint32_t w, _Float16 sc) {
  const v2h s2 = v2h{sc, sc};
  v4i r;
#pragma unroll
  for (int m = 0; m < 4; m++) {
    v2h f;
    if (m == 0) f = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    else if (m == 1) f = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    else if (m == 2) f = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    else f = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
    r[m] = __builtin_bit_cast(int, f * s2);
  }
  return __builtin_bit_cast(v8h, r);
}

// Two bf16 (low, high half) -> the same two values as fp16 where they are
// fp16 normals (the NF3 tables' entries are).
__device__ __forceinline__ uint32_t bf16x2_to_h2(uint32_t u) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(u << 16), __uint_as_float(u & 0xFFFF0000u)));
}

// nf3_tables with fp16 entries holding the same bf16-rounded products.
__device__ __forceinline__ void nf3_tables_h(float f, uint32_t &t01, uint32_t &t23) {
  nf3_tables(f, t01, t23);
  t01 = bf16x2_to_h2(t01);
  t23 = bf16x2_to_h2(t23);
}

// nf3_step_rc selects whole 16-bit entries and ORs in bit 15, the sign bit of
// fp16 as of bf16, so fp16 tables give the fp16 operand.
__device__ __forceinline__ v8h nf3_step_h(uint32_t dsel, uint32_t d2, int s, uint32_t t01, uint32_t t23) {
  return __builtin_bit_cast(v8h, nf3_step_rc(dsel, d2, s, t01, t23));
}

// Largest magnitude of eight bf16 (one 16-byte chunk), as fp32 bits.
__device__ __forceinline__ uint32_t bf16x8_amax(v4i x) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t u = (uint32_t)x[i] & 0x7FFF7FFFu;
    m = max(m, max(u & 0xFFFFu, u >> 16));
  }
  return m << 16;
}

// Maximum over the 16 lanes of each row of the wave (every lane gets it):
// rotations within the row by DPP, no LDS round trip.  All 16 lanes active.
__device__ __forceinline__ uint32_t row16_max(uint32_t m) {
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x128, 0xF, 0xF, false));   // row_ror:8
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x124, 0xF, 0xF, false));   // row_ror:4
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x122, 0xF, 0xF, false));   // row_ror:2
  m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x121, 0xF, 0xF, false));   // row_ror:1
  return m;
}

// The exponent e of a row whose largest magnitude has fp32 bits amax: the row
// is converted as values * 2^-e, its largest then in [2^14, 2^15) (for a zero
// or subnormal maximum, e = -141 keeps every value below 2^15).
__device__ __forceinline__ int h_row_exp(uint32_t amax) { return (int)((amax >> 23) & 0xFFu) - 141; }

// Two bf16 -> two fp16 of the values times 2^-e.
__device__ __forceinline__ uint32_t bf16x2_to_h(uint32_t u, int e) {
  const float lo = __builtin_amdgcn_ldexpf(__uint_as_float(u << 16), -e);
  const float hi = __builtin_amdgcn_ldexpf(__uint_as_float(u & 0xFFFF0000u), -e);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// Eight bf16 -> eight fp16 of the values times 2^-e.
__device__ __forceinline__ v4i bf16x8_to_h(v4i x, int e) {
  v4i r;
#pragma unroll
  for (int i = 0; i < 4; i++) r[i] = (int)bf16x2_to_h((uint32_t)x[i], e);
  return r;
}

// 2^d as an fp16 pair, for -24 <= d <= 0 (subnormal below 2^-14); 0 for d < -24.
__device__ __forceinline__ v2h pow2_h2(int d) {
  const uint32_t b = d >= -14 ? (uint32_t)(d + 15) << 10 : d >= -24 ? 1u << (d + 24) : 0u;
  return __builtin_bit_cast(v2h, b | (b << 16));
}

// Dequantised operand of one lane for k-step s (0..3) of a 128-column k-tile.
template <int WF>
struct A16Tile {
  uint32_t d[4];   // NVFP4: 4 dwords of codes; NF3: 3 dwords (12 bytes)
  uint32_t sc;     // scale byte(s)
  template <bool NT = false>   // NT: non-temporal data loads
  __device__ __forceinline__ void load(const uint8_t *data, const uint8_t *scales) {
    if (WF == W_NVFP4) {
      const v4i v = NT ? __builtin_nontemporal_load((const v4i *)data) : *(const v4i *)data;
      d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
      sc = *(const uint16_t *)scales;
    } else {
      const uint32_t *p = (const uint32_t *)data;
      if (NT) {
        d[0] = __builtin_nontemporal_load(p); d[1] = __builtin_nontemporal_load(p + 1); d[2] = __builtin_nontemporal_load(p + 2);
      } else {
        d[0] = p[0]; d[1] = p[1]; d[2] = p[2];
      }
      d[3] = 0;
      sc = *scales;
    }
  }
  // the same from buffer resources (data wb, scales sb) at lane offsets vd, vs
  // plus wave-uniform offsets sd, ss; NT: the data loads are non-temporal
  template <bool NT = false>
  __device__ __forceinline__ void load(const Buf &wb, uint32_t vd, uint32_t sd, const Buf &sb, uint32_t vs,
                                       uint32_t ss) {
    if (WF == W_NVFP4) {
      const v4i v = NT ? buf_load16_nt(wb, vd, sd) : buf_load16(wb, vd, sd);
      d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = v[3];
      sc = buf_load2(sb, vs, ss);
    } else {
      const v3i v = NT ? buf_load12_nt(wb, vd, sd) : buf_load12(wb, vd, sd);
      d[0] = v[0]; d[1] = v[1]; d[2] = v[2]; d[3] = 0;
      sc = buf_load1(sb, vs, ss);
    }
  }
  __device__ __forceinline__ void zero() { d[0] = d[1] = d[2] = d[3] = 0; sc = 0; }
  // The tile's decoded scales, computed once before its four steps: NVFP4 the
  // fp32 scales of columns 0..15 and 16..31 (as bits), NF3 the scaled
  // magnitude tables t01, t23.
  struct Deq {
    uint32_t u, v;
  };
  __device__ __forceinline__ Deq prep() const {
    Deq q;
    if (WF == W_NVFP4) {
      q.u = __float_as_uint(e4m3_f32(sc & 0xFFu));
      q.v = __float_as_uint(e4m3_f32((sc >> 8) & 0xFFu));
    } else {
      nf3_tables(e4m3_f32(sc & 0xFFu), q.u, q.v);
    }
    return q;
  }
  __device__ __forceinline__ v8bf step(int s, const Deq &q) const {
    if (WF == W_NVFP4) return nvfp4_step(d[s], __uint_as_float(s < 2 ? q.u : q.v));
    return nf3_step_rc(s < 2 ? d[0] : d[1], d[2], s, q.u, q.v);
  }
  // fp16 forms: NVFP4 u = both scales as an fp16 pair; NF3 fp16 tables
  __device__ __forceinline__ Deq prep_h() const {
    Deq q;
    if (WF == W_NVFP4) {
      q.u = __builtin_bit_cast(uint32_t, e4m3x2_h(sc));
      q.v = 0;
    } else {
      nf3_tables_h(e4m3_f32(sc & 0xFFu), q.u, q.v);
    }
    return q;
  }
  __device__ __forceinline__ v8h step_h(int s, const Deq &q) const {
    if (WF == W_NVFP4) {
      const v2h p = __builtin_bit_cast(v2h, q.u);
      return nvfp4_step_h(d[s], s < 2 ? p.x : p.y);
    }
    return nf3_step_h(s < 2 ? d[0] : d[1], d[2], s, q.u, q.v);
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


// ------------------------------------------------ tile schedule

struct TileInfo {
  int valid, e, p0, rows;
};

__device__ __forceinline__ TileInfo tile_info(const GemmArgs &a) {
  TileInfo ti;
  const int tbeg = a.tier_tiles[2 * a.tier], tend = a.tier_tiles[2 * a.tier + 1];
  const int tile = tbeg + (int)blockIdx.y;
  ti.valid = tile < tend;
  if (!ti.valid) return ti;
  const int u = a.tile_u[tile];
  ti.e = u - a.u_base;
  ti.p0 = a.off[u] + a.tile_row0[tile];
  ti.rows = min(a.tile_rows, a.off[u + 1] - ti.p0);
  return ti;
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
    st.A[q] = __builtin_nontemporal_load((const v4i *)(wt + q * rt_bytes + (size_t)kt * 1024));   // read once
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
  for (int q = 0; q < 4; q++)   // weights read once at the batch sizes this serves: non-temporal
    st.A[q].template load<true>(wt + q * rt_bytes + (size_t)kt * 64 * U, sp + q * rt_scales + kt * 64 * SU);
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
  typename A16Tile<WF>::Deq dq[4];
#pragma unroll
  for (int q = 0; q < 4; q++) dq[q] = st.A[q].prep();
#pragma unroll
  for (int s = 0; s < 4; s++) {
    const v8bf b = __builtin_bit_cast(v8bf, st.B[s]);
#pragma unroll
    for (int q = 0; q < 4; q++) acc[q] = mfma_bf16(st.A[q].step(s, dq[q]), b, acc[q]);
  }
}

}  // namespace moe
