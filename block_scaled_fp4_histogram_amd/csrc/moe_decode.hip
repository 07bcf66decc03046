// Decode-size layer: T <= 16 tokens and T * top_k <= 64 routes, two launches.
//
// At these sizes the layer streams the weights of ~35 distinct experts and does
// almost no arithmetic, so launches and idle lanes, not FLOPs, decide the time.
// Every workgroup therefore recomputes the routing itself from the <= 64 ids
// (one route per lane; wave ballots group the routes of each expert in order of
// first occurrence), and there is no separate planner, quantiser or combine:
//
//   k_dec_gemm1  grid (N/32 intermediate blocks, expert slots), 8 waves split K.
//                The token rows of the expert's routes are quantised to MXFP8
//                into LDS once per workgroup (W4A8) or read as bf16 (W4A16);
//                up/gate GEMMs, clamped SwiGLU and requantisation of h, stored
//                per route r = t*top_k + j.
//   k_dec_gemm2  grid (K/16 output row tiles), 8 waves split the experts.
//                Each wave runs the down GEMM of its experts for 16 output
//                columns and folds the router-weighted results into per-token
//                fp32 accumulators; the 8 waves are summed in a fixed order and
//                the bf16 output written.  No atomics: bit-stable run to run.
#include "moe_device.h"

namespace moe {

// Unified expert of route `lane` (experts of earlier tiers first), or -1.
__device__ __forceinline__ int dec_route_u(const DecArgs &a, int lane) {
  if (lane >= a.R) return -1;
  const int id = a.ids[lane];
  if (id < 0 || id >= a.E) return -1;
  const int e0 = a.tier[0].emap ? a.tier[0].emap[id] : id;
  if (e0 >= 0 && e0 < a.tier[0].E) return e0;
  if (a.n_tiers > 1) {
    const int e1 = a.tier[1].emap ? a.tier[1].emap[id] : id;
    if (e1 >= 0 && e1 < a.tier[1].E) return a.tier[0].E + e1;
  }
  return -1;
}

// Group d, in order of first occurrence, of the routes sharing one expert:
// its expert and the mask of its routes (bit r = route r).  Wave-uniform.
__device__ __forceinline__ bool dec_group(int u, int d, int *gu, unsigned long long *gm) {
  unsigned long long rem = __ballot(u >= 0);
  for (int i = 0; rem; i++) {
    const int leader = __ffsll(rem) - 1;
    const int lu = __shfl(u, leader);
    const unsigned long long m = __ballot(u == lu);
    if (i == d) {
      *gu = lu;
      *gm = m;
      return true;
    }
    rem &= ~m;
  }
  return false;
}

// Index of the n-th set bit of m (n from 0), or -1.
__device__ __forceinline__ int nth_bit(unsigned long long m, int n) {
  for (int i = 0; i < n && m; i++) m &= m - 1;
  return m ? __ffsll(m) - 1 : -1;
}

struct DecExpert {
  const uint8_t *w13, *s13, *w2, *s2;
  float g13, g2;
  int fmt, e;
};

__device__ __forceinline__ DecExpert dec_expert(const DecArgs &a, int u) {
  DecExpert x;
  const bool t1 = a.n_tiers > 1 && u >= a.tier[0].E;
  const DecTier &T = t1 ? a.tier[1] : a.tier[0];
  x.e = t1 ? u - a.tier[0].E : u;
  x.w13 = T.w13;
  x.s13 = T.s13;
  x.w2 = T.w2;
  x.s2 = T.s2;
  x.g13 = T.g13 ? T.g13[x.e] : 1.0f;
  x.g2 = T.g2 ? T.g2[x.e] : 1.0f;
  x.fmt = T.fmt;
  return x;
}

// Fixed-order sum over the 8 waves of the 16 GEMM1 accumulators, clamped
// SwiGLU; returns the 8 intermediate values of lane (route column c, group g):
// columns 32*hb + 16*s + 4*g + i for s, i.
__device__ __forceinline__ void dec_swiglu(const float *red, int l, float gs, float limit, int has_limit, float *h) {
#pragma unroll
  for (int s = 0; s < 2; s++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int iu = (2 * s) * 4 + i, ig = (2 * s + 1) * 4 + i;
      float up = 0.f, gate = 0.f;
#pragma unroll
      for (int w = 0; w < 8; w++) {
        up += red[(w * 16 + iu) * 64 + l];
        gate += red[(w * 16 + ig) * 64 + l];
      }
      h[s * 4 + i] = silu_clamped(gate * gs, up * gs, limit, has_limit);
    }
}

// ---------------------------------------------------------------- GEMM1, W4A8
__global__ __launch_bounds__(512) void k_dec_gemm1_a8(DecArgs a) {
  extern __shared__ __align__(16) uint8_t dsm[];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  int ud;
  unsigned long long md;
  if (!dec_group(dec_route_u(a, l), blockIdx.y, &ud, &md)) return;
  const DecExpert X = dec_expert(a, ud);
  const int K = a.K, N = a.N, nkt = K / 128, hb = blockIdx.x, kb32 = K / 32;
  const size_t rt_bytes = (size_t)16 * (K / 2), rt_scales = (size_t)16 * kb32;
  const uint8_t *wt = X.w13 + (size_t)X.e * (2 * N) * (K / 2) + (size_t)(4 * hb) * rt_bytes + l * 16;
  const uint8_t *st = X.s13 + (size_t)X.e * (2 * N) * kb32 + (size_t)(4 * hb) * rt_scales + l;
  const int xstride = K + 16;   // LDS row stride: rows land on different banks
  uint8_t *xq = dsm;
  uint8_t *xsc = dsm + (size_t)a.cpass * xstride;
  float *red = (float *)dsm;    // reused after the k-loop: [8 waves][16][64]
  const int ncols = __popcll(md);
  for (int p0 = 0; p0 < ncols; p0 += a.cpass) {
    const int ncol = min(a.cpass, ncols - p0);
    // first weight stage in flight while the token rows are quantised
    A8G1Stage s0, s1;
    const bool have = c < ncol;
    if (w < nkt) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        s0.A[q] = *(const v4i *)(wt + q * rt_bytes + (size_t)w * 1024);
        s0.sa[q] = st[q * rt_scales + w * 64];
      }
    }
    for (int i = tid; i < ncol * kb32; i += 512) {
      const int col = i / kb32, blk = i - col * kb32;
      const int t = nth_bit(md, p0 + col) / a.topk;
      const v4i *src = (const v4i *)(a.x + (size_t)t * K + blk * 32);
      float v[32];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const v4i x4 = src[q];
#pragma unroll
        for (int d = 0; d < 4; d++) {
          v[8 * q + 2 * d] = bf16_to_f32((uint32_t)x4[d] & 0xFFFFu);
          v[8 * q + 2 * d + 1] = bf16_to_f32((uint32_t)x4[d] >> 16);
        }
      }
      uint32_t codes[8];
      xsc[col * kb32 + blk] = (uint8_t)quant_block32(v, codes);
      v4i *dst = (v4i *)(xq + col * xstride + blk * 32);
      dst[0] = v4i{(int)codes[0], (int)codes[1], (int)codes[2], (int)codes[3]};
      dst[1] = v4i{(int)codes[4], (int)codes[5], (int)codes[6], (int)codes[7]};
    }
    __syncthreads();
    const uint8_t *xrow = xq + (have ? c : 0) * xstride;
    const uint8_t *xsrow = xsc + (have ? c : 0) * kb32;
    if (w < nkt) {
      if (have) {
        s0.B0 = *(const v4i *)(xrow + w * 128 + 16 * g);
        s0.B1 = *(const v4i *)(xrow + w * 128 + 64 + 16 * g);
        s0.sb = xsrow[w * 4 + g];
      } else {
        s0.B0 = s0.B1 = v4i{0, 0, 0, 0};
        s0.sb = 0;
      }
    }
    v4f acc[4];
#pragma unroll
    for (int q = 0; q < 4; q++) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int kt = w; kt < nkt; kt += 16) {
      if (kt + 8 < nkt) a8g1_load(s1, wt, st, rt_bytes, rt_scales, kt + 8, xrow, xsrow, have, g);
      a8g1_compute(s0, acc);
      if (kt + 16 < nkt) a8g1_load(s0, wt, st, rt_bytes, rt_scales, kt + 16, xrow, xsrow, have, g);
      if (kt + 8 < nkt) a8g1_compute(s1, acc);
    }
    __syncthreads();   // the staged rows are dead; LDS becomes the reduction buffer
#pragma unroll
    for (int q = 0; q < 4; q++)
#pragma unroll
      for (int i = 0; i < 4; i++) red[(w * 16 + q * 4 + i) * 64 + l] = acc[q][i];
    __syncthreads();
    if (w == 0) {
      float h[8];
      dec_swiglu(red, l, 1.0f, a.limit, a.has_limit, h);
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(h[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      float inv;
      const uint32_t sbyte = mx_scale(amax, &inv);
      if (have) {
        const size_t r = (size_t)nth_bit(md, p0 + c);
#pragma unroll
        for (int s = 0; s < 2; s++)
          *(uint32_t *)(a.hq + r * N + hb * 32 + 16 * s + 4 * g) =
              e4m3x4(h[s * 4], h[s * 4 + 1], h[s * 4 + 2], h[s * 4 + 3], inv);
        if (g == 0) a.hs[r * (N / 32) + hb] = (uint8_t)sbyte;
      }
    }
    __syncthreads();   // LDS is restaged by the next pass
  }
}

// ---------------------------------------------------- GEMM1, W4A16 / W3A16
template <int WF>
__device__ __forceinline__ void dec_gemm1_a16_body(const DecArgs &a, const DecExpert &X, unsigned long long md,
                                                   float *red) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int K = a.K, N = a.N, nkt = K / 128, groups = K / 32, hb = blockIdx.x;
  const size_t rt_bytes = (size_t)16 * groups * U, rt_scales = (size_t)16 * groups * SU;
  const uint8_t *wt = X.w13 + (size_t)X.e * (2 * N) * groups * U + (size_t)(4 * hb) * rt_bytes + l * U;
  const uint8_t *st = X.s13 + (size_t)X.e * (2 * N) * groups * SU + (size_t)(4 * hb) * rt_scales + l * SU;
  const int ncols = __popcll(md);
  for (int p0 = 0; p0 < ncols; p0 += 16) {
    const int r = (p0 + c < ncols) ? nth_bit(md, p0 + c) : -1;
    const bool have = r >= 0;
    const uint16_t *xrow = a.x + (size_t)(have ? r / a.topk : 0) * K;
    v4f acc[4];
#pragma unroll
    for (int q = 0; q < 4; q++) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    A16G1Stage<WF> s0, s1;
    if (w < nkt) a16g1_load(s0, wt, st, rt_bytes, rt_scales, w, xrow, have, g);
    for (int kt = w; kt < nkt; kt += 16) {
      if (kt + 8 < nkt) a16g1_load(s1, wt, st, rt_bytes, rt_scales, kt + 8, xrow, have, g);
      a16g1_compute(s0, acc);
      if (kt + 16 < nkt) a16g1_load(s0, wt, st, rt_bytes, rt_scales, kt + 16, xrow, have, g);
      if (kt + 8 < nkt) a16g1_compute(s1, acc);
    }
#pragma unroll
    for (int q = 0; q < 4; q++)
#pragma unroll
      for (int i = 0; i < 4; i++) red[(w * 16 + q * 4 + i) * 64 + l] = acc[q][i];
    __syncthreads();
    if (w == 0 && have) {
      float h[8];
      dec_swiglu(red, l, X.g13, a.limit, a.has_limit, h);
#pragma unroll
      for (int s = 0; s < 2; s++) {
        uint2 v;
        v.x = pack_bf16x2(h[s * 4], h[s * 4 + 1]);
        v.y = pack_bf16x2(h[s * 4 + 2], h[s * 4 + 3]);
        *(uint2 *)(a.hb + (size_t)r * N + hb * 32 + 16 * s + 4 * g) = v;
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(512) void k_dec_gemm1_a16(DecArgs a) {
  __shared__ float red[8 * 16 * 64];
  int ud;
  unsigned long long md;
  if (!dec_group(dec_route_u(a, threadIdx.x & 63), blockIdx.y, &ud, &md)) return;
  const DecExpert X = dec_expert(a, ud);
  if (X.fmt == W_NVFP4) dec_gemm1_a16_body<W_NVFP4>(a, X, md, red);
  else dec_gemm1_a16_body<W_NF3>(a, X, md, red);
}

// ---------------------------------------------------------------- GEMM2
//
// Lane (token t = l % 16, group g) accumulates output columns 16*rt + 4g .. +3
// of token t.  After the down GEMM of one expert for up to 16 of its routes
// (MFMA columns), each route's router-weighted result moves to the lane of its
// token by a lane shuffle; slots j of a token are visited in order.
__device__ __forceinline__ void dec_fold(const DecArgs &a, unsigned long long md, int p0, int c, int g, const v4f &acc,
                                         float wr, float *tok) {
  float val[4];
#pragma unroll
  for (int i = 0; i < 4; i++) val[i] = acc[i] * wr;
  for (int j = 0; j < a.topk; j++) {
    const int rr = c * a.topk + j;   // route of token c, slot j
    int src = 0;
    bool take = false;
    if (c < a.T && rr < 64 && ((md >> rr) & 1ull)) {
      const int col = __popcll(md & ((1ull << rr) - 1ull)) - p0;
      if (col >= 0 && col < 16) {
        src = col;
        take = true;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float v = __shfl(val[i], src + 16 * g);
      if (take) tok[i] += v;
    }
  }
}

__device__ __forceinline__ void dec_gemm2_a8_expert(const DecArgs &a, const DecExpert &X, unsigned long long md,
                                                    int rt, int l, float *tok) {
  const int c = l & 15, g = l >> 4, K = a.K, N = a.N, nkt = (N + 127) / 128;
  const size_t rt_bytes = (size_t)16 * (N / 2), rt_scales = (size_t)16 * (N / 32);
  const uint8_t *wt = X.w2 + (size_t)X.e * K * (N / 2) + (size_t)rt * rt_bytes + l * 16;
  const uint8_t *st = X.s2 + (size_t)X.e * K * (N / 32) + (size_t)rt * rt_scales + l;
  const int ncols = __popcll(md);
  for (int p0 = 0; p0 < ncols; p0 += 16) {
    const int r = (p0 + c < ncols) ? nth_bit(md, p0 + c) : -1;
    const bool have = r >= 0;
    const uint8_t *hrow = a.hq + (size_t)(have ? r : 0) * N;
    const uint8_t *hsrow = a.hs + (size_t)(have ? r : 0) * (N / 32);
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    for (int kt0 = 0; kt0 < nkt; kt0 += 8) {
      v4i A[8], B0[8], B1[8];
      int sa[8], sb[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int kt = kt0 + j, kb = kt * 128;
        A[j] = B0[j] = B1[j] = v4i{0, 0, 0, 0};
        sa[j] = sb[j] = 0;
        if (kt < nkt && kb + 32 * g < N) {
          A[j] = *(const v4i *)(wt + (size_t)kt * 1024);
          sa[j] = st[kt * 64];
        }
        if (have && kt < nkt) {
          if (kb + 16 * g < N) B0[j] = *(const v4i *)(hrow + kb + 16 * g);
          if (kb + 64 + 16 * g < N) B1[j] = *(const v4i *)(hrow + kb + 64 + 16 * g);
          if (kb + 32 * g < N) sb[j] = hsrow[kb / 32 + g];
        }
      }
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if (kt0 + j < nkt) {
          const v8i bop = v8i{B0[j][0], B0[j][1], B0[j][2], B0[j][3], B1[j][0], B1[j][1], B1[j][2], B1[j][3]};
          acc = mfma_fp4_fp8(A[j], bop, acc, sa[j], sb[j]);
        }
      }
    }
    dec_fold(a, md, p0, c, g, acc, have ? a.topk_w[r] * X.g2 : 0.f, tok);
  }
}

template <int WF>
__device__ __forceinline__ void dec_gemm2_a16_expert(const DecArgs &a, const DecExpert &X, unsigned long long md,
                                                     int rt, int l, float *tok) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  const int c = l & 15, g = l >> 4, K = a.K, N = a.N, nkt = (N + 127) / 128, groups = N / 32;
  const size_t rt_bytes = (size_t)16 * groups * U, rt_scales = (size_t)16 * groups * SU;
  const uint8_t *wt = X.w2 + (size_t)X.e * K * groups * U + (size_t)rt * rt_bytes + l * U;
  const uint8_t *st = X.s2 + (size_t)X.e * K * groups * SU + (size_t)rt * rt_scales + l * SU;
  const int ncols = __popcll(md);
  for (int p0 = 0; p0 < ncols; p0 += 16) {
    const int r = (p0 + c < ncols) ? nth_bit(md, p0 + c) : -1;
    const bool have = r >= 0;
    const uint16_t *hrow = a.hb + (size_t)(have ? r : 0) * N;
    v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
    for (int kt0 = 0; kt0 < nkt; kt0 += 4) {
      A16Tile<WF> A[4];
      v4i B[4][4];
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int kt = kt0 + j, kb = kt * 128;
        const bool inb = kt < nkt && kb + 32 * g < N;
        if (inb) A[j].load(wt + (size_t)kt * 64 * U, st + kt * 64 * SU);
        else A[j].zero();
#pragma unroll
        for (int s = 0; s < 4; s++) B[j][s] = v4i{0, 0, 0, 0};
        if (have && inb) {
          const v4i *hp = (const v4i *)(hrow + kb + 32 * g);
#pragma unroll
          for (int s = 0; s < 4; s++) B[j][s] = hp[s];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (kt0 + j < nkt) {
#pragma unroll
          for (int s = 0; s < 4; s++) acc = mfma_bf16(A[j].step(s), __builtin_bit_cast(v8bf, B[j][s]), acc);
        }
    }
    dec_fold(a, md, p0, c, g, acc, have ? a.topk_w[r] * X.g2 : 0.f, tok);
  }
}

template <bool A8>
__global__ __launch_bounds__(512) void k_dec_gemm2(DecArgs a) {
  __shared__ int gu_s[kDecodeMaxRoutes];
  __shared__ unsigned long long gm_s[kDecodeMaxRoutes];
  __shared__ int ng_s;
  __shared__ float tred[8][4][64];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  if (w == 0) {
    const int u = dec_route_u(a, l);
    unsigned long long rem = __ballot(u >= 0);
    int n = 0;
    while (rem) {
      const int leader = __ffsll(rem) - 1;
      const int lu = __shfl(u, leader);
      const unsigned long long m = __ballot(u == lu);
      if (l == 0) {
        gu_s[n] = lu;
        gm_s[n] = m;
      }
      n++;
      rem &= ~m;
    }
    if (l == 0) ng_s = n;
  }
  __syncthreads();
  const int ng = ng_s, rt = blockIdx.x;
  float tok[4] = {0.f, 0.f, 0.f, 0.f};
  for (int gi = w; gi < ng; gi += 8) {
    const DecExpert X = dec_expert(a, gu_s[gi]);
    const unsigned long long md = gm_s[gi];
    if (A8) dec_gemm2_a8_expert(a, X, md, rt, l, tok);
    else if (X.fmt == W_NVFP4) dec_gemm2_a16_expert<W_NVFP4>(a, X, md, rt, l, tok);
    else dec_gemm2_a16_expert<W_NF3>(a, X, md, rt, l, tok);
  }
#pragma unroll
  for (int i = 0; i < 4; i++) tred[w][i][l] = tok[i];
  __syncthreads();
  if (w == 0 && c < a.T) {
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      s[i] = 0.f;
#pragma unroll
      for (int v = 0; v < 8; v++) s[i] += tred[v][i][l];
    }
    uint2 o;
    o.x = pack_bf16x2(s[0], s[1]);
    o.y = pack_bf16x2(s[2], s[3]);
    *(uint2 *)(a.out + (size_t)c * a.K + rt * 16 + 4 * g) = o;
  }
}

int decode_cpass(int K) { return max(1, min(kDecodeMaxT, 61440 / (K + 16 + K / 32))); }

size_t decode_gemm1_lds(int K, int cpass) {
  const size_t stage = (size_t)cpass * (K + 16) + (size_t)cpass * (K / 32);
  const size_t red = (size_t)8 * 16 * 64 * sizeof(float);
  return ((stage > red ? stage : red) + 15) & ~(size_t)15;
}

hipError_t launch_decode(int a8, const DecArgs &a, hipStream_t s, hipEvent_t ev_mid) {
  if (a.R == 0) return hipSuccess;
  int U = a.tier[0].E + (a.n_tiers > 1 ? a.tier[1].E : 0);
  const dim3 g1(a.N / 32, (unsigned)min(a.R, U)), g2(a.K / 16), block(512);
  if (a8) {
    hipLaunchKernelGGL(k_dec_gemm1_a8, g1, block, decode_gemm1_lds(a.K, a.cpass), s, a);
  } else {
    hipLaunchKernelGGL(k_dec_gemm1_a16, g1, block, 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_mid) {
    e = hipEventRecord(ev_mid, s);
    if (e != hipSuccess) return e;
  }
  if (a8) hipLaunchKernelGGL(k_dec_gemm2<true>, g2, block, 0, s, a);
  else hipLaunchKernelGGL(k_dec_gemm2<false>, g2, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
