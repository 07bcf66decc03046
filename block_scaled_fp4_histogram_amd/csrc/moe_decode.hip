// Decode-size layer: T <= 16 tokens and T * top_k <= 64 routes, two launches.
//
// At these sizes the layer streams the weights of ~35 distinct experts and does
// almost no arithmetic, so launches and idle lanes, not FLOPs, decide the time.
// Every workgroup therefore recomputes the routing itself from the <= 64 ids
// (one route per lane; wave ballots group the routes of each expert in order of
// first occurrence), and there is no separate planner, quantiser or combine:
//
//   k_dec_gemm1  grid (N/32 intermediate blocks, expert slots), 4 waves split K.
//                The token rows of the expert's routes are quantised to MXFP8
//                into LDS once per workgroup (W4A8) or read as bf16 (W4A16);
//                up/gate GEMMs, clamped SwiGLU and requantisation of h, stored
//                per route r = t*top_k + j.  Block (0, 0) also publishes the
//                expert-group table the down GEMM reads.
//   k_dec_gemm2  grid (K/16 output row tiles), 8 waves.  The block's work is
//                the list of (expert group, 16-route pass, k-tile) items, split
//                evenly over the waves; each wave streams its items' weights
//                through a register ring and folds the router-weighted results
//                into per-token fp32 accumulators; the waves are summed in a
//                fixed order and the bf16 output written.  No atomics:
//                bit-stable run to run.  Every route's intermediate row is
//                staged in LDS by direct loads ahead of the ring.
#include <type_traits>

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

__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int lane) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, lane), hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), lane);
  return ((unsigned long long)hi << 32) | lo;
}

// Routes (lanes) whose expert equals this lane's, as a 64-bit mask (0 for a
// route without one): the AND over the 10 bits of the unified expert index
// (< kMaxExperts = 1024) of the lanes that agree on that bit.  Ten ballots, no
// per-route loop.
__device__ __forceinline__ unsigned long long dec_same(int u) {
  unsigned long long s = __ballot(u >= 0);
#pragma unroll
  for (int b = 0; b < 10; b++) {
    const bool bit = (u >> b) & 1;
    const unsigned long long m = __ballot(bit);
    s &= bit ? m : ~m;
  }
  return u >= 0 ? s : 0ull;
}

// Group d, in order of first occurrence, of the routes sharing one expert:
// its expert and the mask of its routes (bit r = route r).  Wave-uniform.
__device__ __forceinline__ bool dec_group(int u, int d, int *gu, unsigned long long *gm) {
  const int l = threadIdx.x & 63;
  const unsigned long long same = dec_same(u);
  unsigned long long f = __ballot(same != 0 && __ffsll(same) - 1 == l);   // first route of each expert
  if (d >= __popcll(f)) return false;
  int L = 0;   // position of the d-th set bit of f, by halving
#pragma unroll
  for (int width = 32; width >= 1; width >>= 1) {
    const int below = __popcll(f & ((1ull << width) - 1ull));
    if (d >= below) {
      d -= below;
      f >>= width;
      L += width;
    }
  }
  *gu = __builtin_amdgcn_readlane(u, L);
  *gm = readlane_u64(same, L);
  return true;
}

// Index of the n-th set bit of m (n from 0), or -1.
__device__ __forceinline__ int nth_bit(unsigned long long m, int n) {
  for (int i = 0; i < n && m; i++) m &= m - 1;
  return m ? __ffsll(m) - 1 : -1;
}

// Route of token t in pass p of a group with route mask md: the token's p-th
// slot on the group's expert, or -1.
__device__ __forceinline__ int dec_token_route(unsigned long long md, int p, int t, int T, int topk) {
  if (t >= T) return -1;
  const unsigned long long tm = topk >= 64 ? md : (md >> (t * topk)) & ((1ull << topk) - 1ull);
  const int j = nth_bit(tm, p);
  return j < 0 ? -1 : t * topk + j;
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

// Fixed-order sum over the NW waves of the 16 GEMM1 accumulators, wave w's
// times 2^ex[w] (its fp16 activation exponent for the lane's route; 0 for
// MXFP8), clamped SwiGLU; returns the 8 intermediate values of lane (route
// column c, group g): columns 32*hb + 16*s + 4*g + i for s, i.
template <int NW>
__device__ __forceinline__ void dec_swiglu(const float *red, int l, float gs, float limit, int has_limit, float alpha,
                                           float beta, int act, const int *ex, float *h) {
#pragma unroll
  for (int s = 0; s < 2; s++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int iu = (2 * s) * 4 + i, ig = (2 * s + 1) * 4 + i;
      float up = 0.f, gate = 0.f;
#pragma unroll 2
      for (int w = 0; w < NW; w++) {
        up += __builtin_amdgcn_ldexpf(red[(w * 16 + iu) * 64 + l], ex[w]);
        gate += __builtin_amdgcn_ldexpf(red[(w * 16 + ig) * 64 + l], ex[w]);
      }
      h[s * 4 + i] = silu_clamped(gate * gs, up * gs, limit, has_limit, alpha, beta, act);
    }
}

// ---------------------------------------------------------------- GEMM1
//
// One k-tile of weights for one lane: the up and gate row tiles of two
// adjacent 16-column intermediate blocks.  Activations are read from LDS at
// MFMA time, so only weights travel through registers and two k-tiles of them
// are kept in flight per wave.
struct A8W {
  v4i A[4];
  int sa[4];
};

// The expert's w13 data and scales as buffer resources; row tile q of the
// block starts at wave-uniform offsets w0 + q * wstep, s0 + q * sstep.
struct RowTiles {
  Buf wb, sb;
  uint32_t w0, wstep, s0, sstep;
};

// ok false (a k-tile past the reduction): the offsets fall outside the
// buffers' range, so the loads return zeros without memory traffic.
__device__ __forceinline__ void a8w_load(A8W &st, const RowTiles &rt, uint32_t l, int kt, bool ok) {
#pragma unroll
  for (int q = 0; q < 4; q++) {
    st.A[q] = buf_load16_nt(rt.wb, ok ? (uint32_t)kt * 1024u + l * 16u : 0x80000000u, rt.w0 + q * rt.wstep);
    st.sa[q] = buf_load1(rt.sb, ok ? (uint32_t)kt * 64u + l : 0x80000000u, rt.s0 + q * rt.sstep);
  }
}

// MXFP8 activations of route column c (LDS row xrow, scales xsrow) for k-tile kt.
__device__ __forceinline__ void a8w_mfma(const A8W &st, const uint8_t *xrow, const uint8_t *xsrow, bool have, int g,
                                         int kt, v4f *acc) {
  v4i B0 = v4i{0, 0, 0, 0}, B1 = v4i{0, 0, 0, 0};
  int sb = 0;
  if (have) {
    B0 = *(const v4i *)(xrow + kt * 128 + 16 * g);
    B1 = *(const v4i *)(xrow + kt * 128 + 64 + 16 * g);
    sb = xsrow[kt * 4 + g];
  }
  const v8i bop = v8i{B0[0], B0[1], B0[2], B0[3], B1[0], B1[1], B1[2], B1[3]};
#pragma unroll
  for (int q = 0; q < 4; q++) acc[q] = mfma_fp4_fp8(st.A[q], bop, acc[q], st.sa[q], sb);
}

template <int WF>
struct A16W {
  A16Tile<WF> A[4];
};

template <int WF>
__device__ __forceinline__ void a16w_load(A16W<WF> &st, const RowTiles &rt, uint32_t l, int kt, bool ok) {
  constexpr uint32_t U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
#pragma unroll
  for (int q = 0; q < 4; q++)
    st.A[q].template load<true>(rt.wb, ok ? (uint32_t)kt * 64u * U + l * U : 0x80000000u, rt.w0 + q * rt.wstep, rt.sb,
                 ok ? (uint32_t)kt * 64u * SU + l * SU : 0x80000000u, rt.s0 + q * rt.sstep);
}

// fp16 activations of route column c (LDS row xrow, scaled by its row's
// power of two) for k-tile kt; the weights are dequantised to fp16.
template <int WF>
__device__ __forceinline__ void a16w_mfma(const A16W<WF> &st, const uint16_t *xrow, bool have, int g, int kt,
                                          v4f *acc) {
  typename A16Tile<WF>::Deq dq[4];
#pragma unroll
  for (int q = 0; q < 4; q++) dq[q] = st.A[q].prep_h();
#pragma unroll
  for (int s = 0; s < 4; s++) {
    v4i b = v4i{0, 0, 0, 0};
    if (have) b = *(const v4i *)(xrow + kt * 128 + 32 * g + 8 * s);
    const v8h bb = __builtin_bit_cast(v8h, b);
#pragma unroll
    for (int q = 0; q < 4; q++) acc[q] = mfma_f16(st.A[q].step_h(s, dq[q]), bb, acc[q]);
  }
}

// Stage the activation rows of the pass's route columns into LDS: MXFP8 codes
// and scales (W4A8, the block's threads together), or (W4A16) fp16 rows.
// W4A16: wave w stages only the columns of its own k-tiles (w, w + NW, ...),
// the only ones it reads, as fp16 times 2^-e with e = h_row_exp of their
// largest magnitude (xe[w][col]), so no wave waits for another.
template <bool A8, int NW>
__device__ __forceinline__ void dec_stage_x(const DecArgs &a, unsigned long long md, int p0, int ncol, uint8_t *dsm,
                                            int (*xe)[kDecodeMaxT]) {
  const int K = a.K, kb32 = K / 32, tid = threadIdx.x;
  if (A8) {
    const int xstride = K + 16;
    uint8_t *xq = dsm, *xsc = dsm + (size_t)a.cpass * xstride;
#pragma unroll 1
    for (int i = tid; i < ncol * kb32; i += NW * 64) {
      const int col = i / kb32, blk = i - col * kb32;
      const int t = nth_bit(md, p0 + col) / a.topk;
      const v4i *src = (const v4i *)(a.x + (size_t)t * K + blk * 32);
      v4i x4[4];
#pragma unroll
      for (int q = 0; q < 4; q++) x4[q] = src[q];
      uint32_t codes[8];
      xsc[col * kb32 + blk] = (uint8_t)quant_block32_bf16(x4, codes);
      v4i *dst = (v4i *)(xq + col * xstride + blk * 32);
      dst[0] = v4i{(int)codes[0], (int)codes[1], (int)codes[2], (int)codes[3]};
      dst[1] = v4i{(int)codes[4], (int)codes[5], (int)codes[6], (int)codes[7]};
    }
  } else {
    constexpr int kB = 4;   // chunks of 8 loaded per lane at once
    const int w = tid >> 6, l = tid & 63, xstride = K + 8, nkt = K / 128;
    const int nq = ((nkt - w + NW - 1) / NW) * 16;   // 16-byte chunks of this wave's k-tiles in a row
    uint16_t *xb = (uint16_t *)dsm;
    for (int col = 0; col < ncol; col++) {
      const int t = nth_bit(md, p0 + col) / a.topk;
      const uint16_t *src = a.x + (size_t)t * K;
      uint16_t *dst = xb + col * xstride;
      uint32_t m = 0;
      for (int q0 = 0; q0 < nq; q0 += 64 * kB) {
        v4i v[kB];
#pragma unroll
        for (int j = 0; j < kB; j++) {   // chunk q: k-tile w + NW * (q / 16), chunk q % 16 of it
          const int q = q0 + l + 64 * j, e8 = ((q >> 4) * NW + w) * 128 + (q & 15) * 8;
          v[j] = q < nq ? *(const v4i *)(src + e8) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < kB; j++) {
          const int q = q0 + l + 64 * j, e8 = ((q >> 4) * NW + w) * 128 + (q & 15) * 8;
          if (q < nq) *(v4i *)(dst + e8) = v[j];
          m = max(m, bf16x8_amax(v[j]));
        }
      }
      m = row16_max(m);
      m = max(max((uint32_t)__builtin_amdgcn_readlane((int)m, 0), (uint32_t)__builtin_amdgcn_readlane((int)m, 16)),
              max((uint32_t)__builtin_amdgcn_readlane((int)m, 32), (uint32_t)__builtin_amdgcn_readlane((int)m, 48)));
      const int e = h_row_exp(m);
      for (int q = l; q < nq; q += 64) {
        v4i *p = (v4i *)(dst + ((q >> 4) * NW + w) * 128 + (q & 15) * 8);
        *p = bf16x8_to_h(*p, e);
      }
      if (l == 0) xe[w][col] = e;
    }
  }
}

template <bool A8, int WF, int NW>
__device__ __forceinline__ void dec_gemm1_body(const DecArgs &a, const DecExpert &X, unsigned long long md,
                                               uint8_t *dsm) {
  constexpr int U = A8 ? 16 : FmtGeom<WF>::unit, SU = A8 ? 1 : FmtGeom<WF>::sunit;
  typedef typename std::conditional<A8, A8W, A16W<WF>>::type Stage;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int K = a.K, N = a.N, N1 = a.N1, nkt = K / 128, groups = K / 32, hb = blockIdx.x;
  const size_t rt_bytes = (size_t)16 * groups * U, rt_scales = (size_t)16 * groups * SU;
  RowTiles rt;
  rt.wb = make_buf(X.w13 + (size_t)X.e * (2 * N1) * groups * U, (uint32_t)((size_t)(2 * N1) * groups * U));
  rt.sb = make_buf(X.s13 + (size_t)X.e * (2 * N1) * groups * SU, (uint32_t)((size_t)(2 * N1) * groups * SU));
  rt.w0 = (uint32_t)((size_t)(4 * hb) * rt_bytes);
  rt.wstep = (uint32_t)rt_bytes;
  rt.s0 = (uint32_t)((size_t)(4 * hb) * rt_scales);
  rt.sstep = (uint32_t)rt_scales;
  const uint32_t lu = (uint32_t)l;
  float *red = (float *)dsm;   // after the k-loop: [NW waves][16][64]
  __shared__ int xe[NW][kDecodeMaxT];   // W4A16: exponent of each wave's fp16 activation columns per route
  const int ncols = __popcll(md);
  for (int p0 = 0; p0 < ncols; p0 += a.cpass) {
    const int ncol = min(a.cpass, ncols - p0);
    const bool have = c < ncol;
    // weights are read once per layer: non-temporal loads (buf_load16_nt).
    // two k-tiles of weights in flight per wave: tiles w, w + NW, ... (three
    // measured 1.4 us slower for the NVFP4 up/gate GEMM at K = 6144 and level
    // for MXFP4: with every block resident, more requests only lengthen the
    // memory queues).  Every load is issued, past the last k-tile too (zeros,
    // no traffic): with loads under branches the compiler's wait before each
    // MFMA group drained nearly every load in flight, the newly issued k-tiles
    // included.
    Stage s0, s1;
    auto load = [&](Stage &st, int kt) {
      if constexpr (A8) a8w_load(st, rt, lu, kt, kt < nkt);
      else a16w_load<WF>(st, rt, lu, kt, kt < nkt);
    };
    load(s0, w);
    dec_stage_x<A8, NW>(a, md, p0, ncol, dsm, xe);
    if (A8) __syncthreads();   // W4A16: each wave reads only what it staged
    v4f acc[4];
#pragma unroll
    for (int q = 0; q < 4; q++) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
    const int cc = have ? c : 0;
    auto mfma = [&](const Stage &st, int kt) {
      if constexpr (A8) {
        const uint8_t *xrow = dsm + cc * (K + 16);
        const uint8_t *xsrow = dsm + (size_t)a.cpass * (K + 16) + cc * (K / 32);
        a8w_mfma(st, xrow, xsrow, have, g, kt, acc);
      } else {
        a16w_mfma<WF>(st, (const uint16_t *)dsm + cc * (K + 8), have, g, kt, acc);
      }
    };
    for (int kt = w; kt < nkt; kt += 2 * NW) {
      load(s1, kt + NW);
      mfma(s0, kt);
      load(s0, kt + 2 * NW);
      if (kt + NW < nkt) mfma(s1, kt + NW);
    }
    __syncthreads();   // the staged rows are dead; LDS becomes the reduction buffer
#pragma unroll
    for (int q = 0; q < 4; q++)
#pragma unroll
      for (int i = 0; i < 4; i++) red[(w * 16 + q * 4 + i) * 64 + l] = acc[q][i];
    __syncthreads();
    int ex[NW];   // the waves' activation exponents for the lane's column (fp16 rows only)
#pragma unroll
    for (int ww = 0; ww < NW; ww++) ex[ww] = (!A8 && have) ? xe[ww][c] : 0;
    if (!A8 && a.act == ACT_RELU2) {
      // ReLU^2 without the multiply: both halves' rows give their own columns,
      // each 32-column slice in fp16 with its exponent byte (as below)
      if (w == 0) {
        uint32_t mh[2] = {0u, 0u};
        uint2 o[2][2];   // [s][half], bf16
        const float gs = X.g13 * ((a.w_on_input && have) ? a.topk_w[nth_bit(md, p0 + c)] : 1.0f);
#pragma unroll
        for (int s = 0; s < 2; s++)
#pragma unroll
          for (int half = 0; half < 2; half++) {
            float z[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
              const int ir = (2 * s + half) * 4 + i;
              float v = 0.f;
#pragma unroll 2
              for (int ww = 0; ww < NW; ww++) v += __builtin_amdgcn_ldexpf(red[(ww * 16 + ir) * 64 + l], ex[ww]);
              z[i] = relu2(v * gs);
            }
            o[s][half].x = pack_bf16x2(z[0], z[1]);
            o[s][half].y = pack_bf16x2(z[2], z[3]);
            mh[half] = max(mh[half], bf16x8_amax(v4i{(int)o[s][half].x, (int)o[s][half].y, 0, 0}));
          }
#pragma unroll
        for (int half = 0; half < 2; half++) {
          uint32_t m = max(mh[half], (uint32_t)__shfl_xor((int)mh[half], 16));
          m = max(m, (uint32_t)__shfl_xor((int)m, 32));
          if (have) {
            const size_t r = (size_t)nth_bit(md, p0 + c);
            const int e = h_row_exp(m);
#pragma unroll
            for (int s = 0; s < 2; s++)
              *(uint2 *)(a.hb + r * N + half * N1 + hb * 32 + 16 * s + 4 * g) =
                  uint2{bf16x2_to_h(o[s][half].x, e), bf16x2_to_h(o[s][half].y, e)};
            if (g == 0) a.hs[r * hs_stride(N) + half * (N1 / 32) + hb] = (uint8_t)(m >> 23);
          }
        }
      }
    } else if (w == 0) {
      float h[8];
      // router weight on the input (W4A16 / W3A16): GEMM1 is linear, so it scales the accumulators
      const float gs = X.g13 * ((!A8 && a.w_on_input && have) ? a.topk_w[nth_bit(md, p0 + c)] : 1.0f);
      dec_swiglu<NW>(red, l, gs, a.limit, a.has_limit, a.alpha, a.beta, a.act, ex, h);
      if (A8) {
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
          if (g == 0) a.hs[r * hs_stride(N) + hb] = (uint8_t)sbyte;
        }
      } else {
        // the bf16-rounded values of each 32-column slice as fp16 times 2^-e,
        // e from the slice's largest magnitude, whose exponent byte is stored
        // for the down GEMM (which brings the slices of a row to one scale)
        uint2 v[2];
        uint32_t m = 0;
#pragma unroll
        for (int s = 0; s < 2; s++) {
          v[s].x = pack_bf16x2(h[s * 4], h[s * 4 + 1]);
          v[s].y = pack_bf16x2(h[s * 4 + 2], h[s * 4 + 3]);
          m = max(m, bf16x8_amax(v4i{(int)v[s].x, (int)v[s].y, 0, 0}));
        }
        m = max(m, (uint32_t)__shfl_xor((int)m, 16));
        m = max(m, (uint32_t)__shfl_xor((int)m, 32));
        if (have) {
          const size_t r = (size_t)nth_bit(md, p0 + c);
          const int e = h_row_exp(m);
#pragma unroll
          for (int s = 0; s < 2; s++)
            *(uint2 *)(a.hb + r * N + hb * 32 + 16 * s + 4 * g) = uint2{bf16x2_to_h(v[s].x, e), bf16x2_to_h(v[s].y, e)};
          if (g == 0) a.hs[r * hs_stride(N) + hb] = (uint8_t)(m >> 23);
        }
      }
    }
    __syncthreads();   // LDS is restaged by the next pass
  }
}

// grid (N/32 intermediate blocks, expert slots); the block's 4 waves split K.
// At decode sizes (~35 experts x N/32 blocks) every block is resident at once
// with up to 128 VGPRs per lane, so no block waits for a second round.
// The expert groups and the down GEMM's item offsets (passes of up to 16
// routes times its k-tiles), for the down kernel.
__device__ __forceinline__ void dec_write_groups(const DecArgs &a, int u) {
  const int l = threadIdx.x & 63, nkt2 = (a.N + 127) / 128;
  const unsigned long long same = dec_same(u);
  const bool first = same != 0 && __ffsll(same) - 1 == l;   // this lane opens a group
  const unsigned long long F = __ballot(first);
  // a group's index is the number of groups opened by lower lanes; its item
  // offset is the inclusive lane scan of the item counts minus its own.  One
  // store per table entry, all lanes at once (a store per group in a loop
  // queues behind the weight loads of the other blocks on the CU).  A group
  // runs one pass per slot a token has on its expert (the down GEMM's MFMA
  // columns are the batch's tokens), mostly one.
  const int n = __popcll(F & ((1ull << l) - 1ull));
  int np = 0;
  if (first) {
    const unsigned long long tmask = a.topk >= 64 ? ~0ull : (1ull << a.topk) - 1ull;
    for (int t = 0; t < a.T; t++) np = max(np, __popcll((same >> (t * a.topk)) & tmask));
  }
  const int mine = np * nkt2;
  int incl = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (l >= d) incl += v;
  }
  if (first) {
    a.groups->gu[n] = u;
    a.groups->gm[n] = same;
    a.groups->np[n] = np;
    a.groups->istart[n] = incl - mine;
  }
  if (l == 63) {
    a.groups->ng = __popcll(F);
    a.groups->nitems = incl;
  }
}

__global__ __launch_bounds__(256, 4) void k_dec_gemm1_a8(DecArgs a) {
  extern __shared__ __align__(16) uint8_t dsm[];
  int ud;
  unsigned long long md;
  const int u = dec_route_u(a, threadIdx.x & 63);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 64) dec_write_groups(a, u);
  if (!dec_group(u, blockIdx.y, &ud, &md)) return;
  dec_gemm1_body<true, W_MXFP4, 4>(a, dec_expert(a, ud), md, dsm);
}

__global__ __launch_bounds__(256, 4) void k_dec_gemm1_a16(DecArgs a) {
  extern __shared__ __align__(16) uint8_t dsm[];
  int ud;
  unsigned long long md;
  const int u = dec_route_u(a, threadIdx.x & 63);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < 64) dec_write_groups(a, u);
  if (dec2_a16_halves(a.N) == 2) {
    // the down GEMM's per-tile accumulators and counters of finished halves
    // start at zero: every block clears a slice
    const int nb = gridDim.x * gridDim.y, b = blockIdx.y * gridDim.x + blockIdx.x;
    const int n4 = a.K / 16 * 64;   // 256 floats per 16-row output tile, as float4
    for (int i = b * 256 + (int)threadIdx.x; i < n4; i += nb * 256) ((v4f *)a.dpart)[i] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int i = b * 256 + (int)threadIdx.x; i < a.K / 16; i += nb * 256) a.dcnt[i] = 0;
  }
  if (!dec_group(u, blockIdx.y, &ud, &md)) return;
  const DecExpert X = dec_expert(a, ud);
  if (X.fmt == W_NVFP4) dec_gemm1_body<false, W_NVFP4, 4>(a, X, md, dsm);
  else dec_gemm1_body<false, W_NF3, 4>(a, X, md, dsm);
}

// ---------------------------------------------------------------- GEMM2
//
// Lane (token t = l % 16, group g) accumulates output columns 16*rt + 4g .. +3
// of token t.  The MFMA columns are the batch's tokens (at most 16): in pass p
// of an expert group, column t multiplies the intermediate row of token t's
// p-th slot on that expert (zero where it has none), so at the end of a run of
// one (group, pass) the lane adds its router-weighted accumulator to its
// token sums directly; the group order fixes the order of each token's terms.

// W4A8 down GEMM, grid (K/16 output row tiles).  The block's work is the list
// of items (expert group, 16-route pass, k-tile of N) in group-major order; its
// waves take equal contiguous slices.  A wave streams its items through a ring
// of kG2Ring register slots: the weights of the next kG2Ring items are always
// in flight, so every wave keeps its share of HBM busy from the first
// instruction to the last.  Two slots are enough: with 448 blocks of 8 waves
// a deeper ring only lengthens the memory queues (measured at K = 7168:
// 2 slots 18.9 us, 3 19.6, 6 21.2, 12 24.2).  A wave folds its accumulator
// into per-token sums whenever a run of one (group, pass) ends; the waves'
// token sums are added in wave order.  The partition depends only on the ids:
// bit-stable run to run.
constexpr int kG2Ring = 2;
constexpr int kDecG2WavesA8 = 8;

// Position in the item list; the expert's weight streams (and format, global
// scale and this block's row-tile offsets) follow the group.
struct G2Iter {
  int rt;            // the block's 16-row output tile (set before g2_start)
  int item, grp, pass, kt, npass, fmt;
  float g2;
  unsigned long long md;
  Buf wb, sb;
  uint32_t w0, s0;   // this block's output row tile within the expert's data / scales
};

// The group table, one group per lane (loaded up front: a load here would be
// waited for behind the weight ring); g2v: the groups' global scales.
struct G2Tab {
  int gu, np;
  unsigned long long gm;
  float g2v;
};

__device__ __forceinline__ void g2_enter_group(G2Iter &it, const DecArgs &a, const G2Tab &tb) {
  const int gu = tb.gu;
  const float g2v = tb.g2v;
  it.md = readlane_u64(tb.gm, it.grp);
  it.npass = __builtin_amdgcn_readlane(tb.np, it.grp);
  const int u = __builtin_amdgcn_readlane(gu, it.grp);
  const bool t1 = a.n_tiers > 1 && u >= a.tier[0].E;
  const DecTier &T = t1 ? a.tier[1] : a.tier[0];
  const int e = t1 ? u - a.tier[0].E : u;
  const int groups = a.N / 32;
  it.fmt = __builtin_amdgcn_readfirstlane(T.fmt);
  const uint32_t U = it.fmt == W_NF3 ? 12u : 16u, SU = it.fmt == W_NVFP4 ? 2u : 1u;
  it.g2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g2v), it.grp));
  it.wb = make_buf(T.w2 + (size_t)e * a.K * groups * U, (uint32_t)((size_t)a.K * groups * U));
  it.sb = make_buf(T.s2 + (size_t)e * a.K * groups * SU, (uint32_t)((size_t)a.K * groups * SU));
  it.w0 = __builtin_amdgcn_readfirstlane((uint32_t)it.rt * 16u * (uint32_t)groups * U);
  it.s0 = __builtin_amdgcn_readfirstlane((uint32_t)it.rt * 16u * (uint32_t)groups * SU);
}

__device__ __forceinline__ void g2_start(G2Iter &it, const DecArgs &a, int item, int istart, int ng, int nkt,
                                         const G2Tab &tb) {
  const int l = threadIdx.x & 63;
  it.item = item;
  it.grp = max(0, __popcll(__ballot(l < ng && istart <= item)) - 1);
  const int rel = item - __builtin_amdgcn_readlane(istart, it.grp);
  it.pass = rel / nkt;
  it.kt = rel - it.pass * nkt;
  g2_enter_group(it, a, tb);
}

__device__ __forceinline__ void g2_next(G2Iter &it, const DecArgs &a, int ng, int nkt, const G2Tab &tb) {
  it.item++;
  if (++it.kt < nkt) return;
  it.kt = 0;
  if (++it.pass < it.npass) return;
  it.pass = 0;
  if (++it.grp < ng) g2_enter_group(it, a, tb);
}

__global__ __launch_bounds__(kDecG2WavesA8 * 64) void k_dec_gemm2_a8(DecArgs a) {
  extern __shared__ __align__(16) uint8_t dsm2[];
  __shared__ float tred[kDecG2WavesA8][4][64];
  __shared__ float wr_s[kDecodeMaxRoutes];
  __shared__ __align__(16) uint8_t zb[64];   // zero operand bytes for absent routes and columns past N
  // wave-uniform values are pinned to scalar registers: derived from them, the
  // item bounds and weight descriptors stay scalar through the ring's branches
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, c = l & 15, g = l >> 4;
  if (tid < 16) ((uint32_t *)zb)[tid] = 0u;
  const int K = a.K, N = a.N, nkt = (N + 127) / 128, rt = blockIdx.x;
  // expert groups (one per lane) and item offsets, from the up/gate kernel
  const DecGroups *G = a.groups;
  const int ng = __builtin_amdgcn_readfirstlane(G->ng), NI = __builtin_amdgcn_readfirstlane(G->nitems);
  int gu = G->gu[l], istart = G->istart[l], gnp = G->np[l];
  uint32_t gm_lo = (uint32_t)G->gm[l], gm_hi = (uint32_t)(G->gm[l] >> 32);
  float wv = tid < a.R ? a.topk_w[tid] : 0.f;
  // the table and router weights are complete here; re-defined by an empty
  // asm, their registers carry no pending load, so nothing after waits on them
  wait_vm<0>();
  asm volatile("" : "+v"(gu), "+v"(istart), "+v"(gnp), "+v"(gm_lo), "+v"(gm_hi), "+v"(wv));
  G2Tab tb;
  tb.gu = gu;
  tb.np = gnp;
  tb.gm = ((unsigned long long)gm_hi << 32) | gm_lo;
  tb.g2v = 1.0f;
  if (tid < a.R) wr_s[tid] = wv;
  const int per = (NI + kDecG2WavesA8 - 1) / kDecG2WavesA8;
  const int i0 = min(NI, w * per), i1 = min(NI, i0 + per);
  // ring of weight k-tiles; items past the slice load out of the buffer's range
  // (zero, no memory traffic) so every slot issues the same two loads
  v4i A[kG2Ring];
  int sa[kG2Ring];
  G2Iter is;
  is.rt = rt;
  if (i0 < i1) g2_start(is, a, i0, istart, ng, nkt, tb);
  else is.item = i1;
  auto issue = [&](int s) {
    const bool ok = is.item < i1 && is.kt * 128 + 32 * g < N;
    A[s] = buf_load16_nt(is.wb, ok ? (uint32_t)is.kt * 1024u + (uint32_t)l * 16u : 0x80000000u, is.w0);
    sa[s] = buf_load1(is.sb, ok ? (uint32_t)is.kt * 64u + (uint32_t)l : 0x80000000u, is.s0);
    if (is.item < i1) g2_next(is, a, ng, nkt, tb);
  };
  if (i0 >= i1) {   // no items: the ring's loads still need valid descriptors
    is.wb = make_buf(a.hq, 0);
    is.sb = is.wb;
    is.w0 = is.s0 = 0;
  }
  // every route's MXFP8 intermediate row and scales -> LDS by direct loads
  // (1 KB / 256-byte chunks; bytes past the rows read a valid dummy address),
  // issued ahead of the ring
  uint8_t *hq_s = dsm2, *hs_s = dsm2 + dec2_hq_bytes(a.R, N);
  {
    const int rs = N + 16, hss = hs_stride(N);
    for (int ch = w; ch * 1024 < dec2_hq_bytes(a.R, N); ch += kDecG2WavesA8) {
      const int pos = ch * 1024 + l * 16, row = pos / rs, col = pos - row * rs;
      dma16(row < a.R && col < N ? a.hq + (size_t)row * N + col : a.hq, hq_s + ch * 1024);
    }
    for (int ch = w; ch * 256 < dec2_hs_bytes(a.R, N); ch += kDecG2WavesA8) {
      const int pos = ch * 256 + l * 4;
      dma4(pos < a.R * hss ? a.hs + pos : a.hs, hs_s + ch * 256);
    }
  }
#pragma unroll
  for (int s = 0; s < kG2Ring; s++) issue(s);
  // the staged rows have landed once at most the ring's 2 kG2Ring loads are
  // outstanding; LDS stores done; then every wave's share is visible
  wait_vm<2 * kG2Ring>();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  float tok[4] = {0.f, 0.f, 0.f, 0.f};
  G2Iter ic;
  ic.rt = rt;
  if (i0 < i1) g2_start(ic, a, i0, istart, ng, nkt, tb);
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  int r = -1;
  for (int base = i0; base < i1; base += kG2Ring) {
#pragma unroll
    for (int s = 0; s < kG2Ring; s++) {
      if (base + s < i1) {
        if (s == 0 || ic.kt == 0 || base + s == i0)   // route of this lane's token in the current run
          r = dec_token_route(ic.md, ic.pass, c, a.T, a.topk);
        // absent routes and columns past N read zero bytes (zb) instead of branching
        const int kb = ic.kt * 128;
        const uint8_t *hrow = hq_s + (r >= 0 ? r : 0) * (N + 16);
        const v4i B0 = *(const v4i *)(r >= 0 && kb + 16 * g < N ? hrow + kb + 16 * g : zb);
        const v4i B1 = *(const v4i *)(r >= 0 && kb + 64 + 16 * g < N ? hrow + kb + 64 + 16 * g : zb);
        const int sbv = *(r >= 0 && kb + 32 * g < N ? hs_s + (r >= 0 ? r : 0) * hs_stride(N) + kb / 32 + g : zb);
        const v8i bop = v8i{B0[0], B0[1], B0[2], B0[3], B1[0], B1[1], B1[2], B1[3]};
        acc = mfma_fp4_fp8(A[s], bop, acc, sa[s], sbv);
        if (ic.kt == nkt - 1 || base + s + 1 == i1) {
          const float wgt = r >= 0 ? wr_s[r] : 0.f;
#pragma unroll
          for (int i = 0; i < 4; i++) tok[i] += acc[i] * wgt;
          acc = v4f{0.f, 0.f, 0.f, 0.f};
        }
        g2_next(ic, a, ng, nkt, tb);
      }
      issue(s);   // the item kG2Ring ahead (out of range past the slice)
    }
  }
#pragma unroll
  for (int i = 0; i < 4; i++) tred[w][i][l] = tok[i];
  __syncthreads();
  if (w == 0 && c < a.T) {
    float s4[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      s4[i] = 0.f;
#pragma unroll
      for (int v = 0; v < kDecG2WavesA8; v++) s4[i] += tred[v][i][l];
    }
    uint2 o;
    o.x = pack_bf16x2(s4[0], s4[1]);
    o.y = pack_bf16x2(s4[2], s4[3]);
    *(uint2 *)(a.out + (size_t)c * K + rt * 16 + 4 * g) = o;
  }
}

// W4A16 / W3A16 down GEMM, grid (K/16 output row tiles): the same item list,
// wave slices and weight ring as the W4A8 kernel (a slot: NVFP4 16 + 2 bytes
// or NF3 12 + 1 bytes a lane, per the group's tier); every route's bf16
// intermediate row is staged in LDS by direct loads and converted there to
// fp16 times a power of two per row.  Each item is four dequantise-and-multiply
// steps of 8 columns (fp16 MFMA).  WF: the format of
// every tier (one 16- or 12-byte load per slot), or 0 for two tiers of
// different formats (one load shape for both, below).
constexpr int kG2RingA16 = 2;   // as kG2Ring (NVFP4 at K = 6144: 2 slots 40.4 us, 6 42.3)

//
// Two blocks share each 16-row output tile when the reduction has two k-tiles
// or more: block half h takes k-tiles [kt0, kt0 + nkh) of every (group, pass)
// and stages only those columns of the intermediate rows, so a block needs
// half the LDS and three fit on a CU (with all columns, 384 blocks of about
// 66 KB at K = 6144 left half the CUs with twice the work of the others).
// Each half adds its fp32 token sums into the tile's accumulator with device
// atomics that return (so they have been performed once the wave has waited
// for them), then counts itself on the tile's counter; the half that counts
// second reads the sums back with atomics and writes the bf16 output.  No
// fence is needed, which matters: a device-scope fence writes back and
// invalidates the whole L2 of the XCD (measured: the down GEMM 2.3 times
// slower with one fence pair per block).  The accumulators and counters are
// zeroed by the up/gate kernel.  Two additions onto +0 give the same bits in
// either order, so the result is bit-stable run to run.
template <int WF>
__global__ __launch_bounds__(kDecG2WavesA8 * 64) void k_dec_gemm2_a16r(DecArgs a) {
  extern __shared__ __align__(16) uint8_t dsm2[];
  __shared__ float wr_s[kDecodeMaxRoutes];
  __shared__ __align__(16) float yb[kDecG2WavesA8][256];   // per-wave token sums
  __shared__ __align__(16) uint8_t zb[64];   // zero operand bytes for absent routes and columns past N
  __shared__ uint32_t rexb[kDecodeMaxRoutes];  // per route the largest exponent byte of its slices in this half
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, c = l & 15, g = l >> 4;
  if (tid < 16) ((uint32_t *)zb)[tid] = 0u;
  if (tid < kDecodeMaxRoutes) rexb[tid] = 0u;
  const int K = a.K, N = a.N, nkt = (N + 127) / 128;
  const int halves = dec2_a16_halves(N), rt = blockIdx.x / halves, h = blockIdx.x - rt * halves;
  const int nk0 = halves == 2 ? (nkt + 1) / 2 : nkt;   // k-tiles of half 0
  const int kt0 = h ? nk0 : 0, nkh = h ? nkt - nk0 : nk0;
  const int c0 = 128 * kt0, nh = min(N, 128 * (kt0 + nkh)) - c0;   // this half's intermediate columns
  const DecGroups *G = a.groups;
  // every group's item count is a multiple of nkt (passes x k-tiles): the
  // half's list keeps nkh of each pass's nkt k-tiles
  const int ng = __builtin_amdgcn_readfirstlane(G->ng),
            NI = __builtin_amdgcn_readfirstlane(G->nitems) / nkt * nkh;
  int gu = G->gu[l], istart = G->istart[l] / nkt * nkh, gnp = G->np[l];
  uint32_t gm_lo = (uint32_t)G->gm[l], gm_hi = (uint32_t)(G->gm[l] >> 32);
  float wv = tid < a.R ? (a.w_on_input ? 1.0f : a.topk_w[tid]) : 0.f;   // weight on the input: 1 here
  // the exponent bytes of the routes' 32-column slices in this half (written
  // by the up/gate kernel), one a thread; their maximum per route is the
  // exponent of its fp16 row here
  const int nsl = nh / 32, nsr = a.R * nsl;
  const float rsl = 1.0f / (float)nsl;   // route of slice entry i: exact for the sizes here
  int sr = 0;
  uint32_t sb8 = 0;
  if (tid < nsr) {
    sr = (int)(((float)tid + 0.5f) * rsl);
    sb8 = a.hs[(size_t)sr * hs_stride(N) + c0 / 32 + (tid - sr * nsl)];
  }
  float g2v = 1.0f;   // global scale of group l's expert
  if (l < ng) {
    const bool t1 = a.n_tiers > 1 && gu >= a.tier[0].E;
    const float *g2p = t1 ? a.tier[1].g2 : a.tier[0].g2;
    if (g2p) g2v = g2p[t1 ? gu - a.tier[0].E : gu];
  }
  // the table, router weights and scales are complete here; re-defined by an
  // empty asm, their registers carry no pending load
  wait_vm<0>();
  asm volatile("" : "+v"(gu), "+v"(istart), "+v"(gnp), "+v"(gm_lo), "+v"(gm_hi), "+v"(wv), "+v"(g2v), "+v"(sb8));
  G2Tab tb;
  tb.gu = gu;
  tb.np = gnp;
  tb.gm = ((unsigned long long)gm_hi << 32) | gm_lo;
  tb.g2v = g2v;
  if (tid < a.R) wr_s[tid] = wv;
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();   // rexb is zero
  if (tid < nsr) atomicMax(&rexb[sr], sb8);
  for (int i = tid + kDecG2WavesA8 * 64; i < nsr; i += kDecG2WavesA8 * 64) {
    const int r = (int)(((float)i + 0.5f) * rsl);
    atomicMax(&rexb[r], (uint32_t)a.hs[(size_t)r * hs_stride(N) + c0 / 32 + (i - r * nsl)]);
  }
  const int per = (NI + kDecG2WavesA8 - 1) / kDecG2WavesA8;
  const int i0 = min(NI, w * per), i1 = min(NI, i0 + per);
  v4i A16[kG2RingA16];   // NVFP4: the lane's 16 weight bytes
  v3i A3[kG2RingA16];    // otherwise: weight bytes 0..11 of the lane
  uint32_t A4[kG2RingA16], sa[kG2RingA16];
  G2Iter is;   // its kt runs over the half's k-tiles: k-tile kt0 + kt of the reduction
  is.rt = rt;
  if (i0 < i1) g2_start(is, a, i0, istart, ng, nkh, tb);
  else is.item = i1;
  if (i0 >= i1) {   // no items: the ring's loads still need valid descriptors
    is.wb = make_buf(a.hb, 0);
    is.sb = is.wb;
    is.w0 = is.s0 = 0;
    is.fmt = W_NVFP4;
    is.kt = 0;
  }
  // mixed tiers: one instruction shape for both formats (no branch: a loaded
  // value copied out of a branch would have to be waited for): 12 data bytes,
  // the 4th dword (NVFP4 only; NF3 loads out of range), and an aligned 16-bit
  // scale load (NVFP4: the lane's two E4M3 bytes; NF3: the pair holding its
  // byte).  One format: one data load of its width.
  // the k-tile's offset is wave-uniform, so it goes into the scalar offset
  auto issue = [&](int s) {
    const int kt = kt0 + is.kt;
    const bool ok = is.item < i1 && kt * 128 + 32 * g < N;
    const bool nv = WF == W_NVFP4 || (WF == 0 && is.fmt == W_NVFP4);
    const uint32_t U = nv ? 16u : 12u, SU = nv ? 2u : 1u;
    const uint32_t dv = ok ? (uint32_t)l * U : 0x80000000u, wo = is.w0 + (uint32_t)kt * 64u * U;
    if constexpr (WF == W_NVFP4) {
      A16[s] = buf_load16_nt(is.wb, dv, wo);
    } else {
      A3[s] = buf_load12_nt(is.wb, dv, wo);
      if constexpr (WF == 0) A4[s] = buf_load4(is.wb, nv && ok ? dv + 12u : 0x80000000u, wo);
    }
    sa[s] = buf_load2(is.sb, ok ? (nv ? (uint32_t)l * 2u : (uint32_t)(l & ~1)) : 0x80000000u,
                      is.s0 + (uint32_t)kt * 64u * SU);
    if (is.item < i1) g2_next(is, a, ng, nkh, tb);
  };
  // this half's columns of every route's intermediate row -> LDS (row stride
  // nh + 8 elements) at one scale per row.  The up/gate kernel wrote each
  // 32-column slice in fp16 times 2^-e_s of its own; each 8-column chunk is
  // loaded into registers ahead of the ring (with its slice's exponent byte),
  // multiplied by 2^(e_s - e) for its row's exponent e (the largest e_s of the
  // row in this half, so the factor is at most 1) and stored.  Chunks past the
  // rows load out of range (zeros, no traffic), so every round issues the same
  // loads.
  uint16_t *hb_s = (uint16_t *)dsm2;
  {
    constexpr int kCh = 4, NT = kDecG2WavesA8 * 64;
    const int n8 = nh / 8, nch = a.R * n8;
    const float rn = 1.0f / (float)n8;   // row of chunk i: exact for the sizes here
    const Buf hbuf = make_buf(a.hb, (uint32_t)((size_t)a.R * N * 2)), sbuf = make_buf(a.hs, (uint32_t)(a.R * hs_stride(N)));
    for (int base = 0; base < nch; base += kCh * NT) {
      v4i v[kCh];
      uint32_t eb[kCh];
#pragma unroll
      for (int j = 0; j < kCh; j++) {
        const int i = base + tid + j * NT, r = (int)(((float)i + 0.5f) * rn), c8 = i - r * n8;
        const bool ok = i < nch;
        v[j] = buf_load16(hbuf, ok ? (uint32_t)(r * N + c0 + 8 * c8) * 2u : 0x80000000u, 0);
        eb[j] = buf_load1(sbuf, ok ? (uint32_t)(r * hs_stride(N) + (c0 + 8 * c8) / 32) : 0x80000000u, 0);
      }
      if (base == 0) {
#pragma unroll
        for (int q = 0; q < kG2RingA16; q++) issue(q);
        // the routes' exponent bytes (rexb) are complete for every wave
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
      }
#pragma unroll
      for (int j = 0; j < kCh; j++) {
        const int i = base + tid + j * NT, r = (int)(((float)i + 0.5f) * rn), c8 = i - r * n8;
        if (i < nch) {
          const v2h f = pow2_h2((int)(eb[j] & 0xFFu) - (int)rexb[r]);
          v4i o;
#pragma unroll
          for (int d = 0; d < 4; d++) {
            const uint32_t u = (uint32_t)v[j][d];   // a copy: bit_cast reads objects, not vector elements
            o[d] = __builtin_bit_cast(int, __builtin_bit_cast(v2h, u) * f);
          }
          *(v4i *)(hb_s + r * (nh + 8) + 8 * c8) = o;
        }
      }
    }
    if (nch == 0) {
#pragma unroll
      for (int q = 0; q < kG2RingA16; q++) issue(q);
    }
  }
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  float tok[4] = {0.f, 0.f, 0.f, 0.f};
  G2Iter ic;
  ic.rt = rt;
  if (i0 < i1) g2_start(ic, a, i0, istart, ng, nkh, tb);
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  int r = -1, er = 0;
  for (int base = i0; base < i1; base += kG2RingA16) {
#pragma unroll
    for (int s = 0; s < kG2RingA16; s++) {
      if (base + s < i1) {
        if (s == 0 || ic.kt == 0 || base + s == i0) {   // route of this lane's token in the current run
          r = dec_token_route(ic.md, ic.pass, c, a.T, a.topk);
          er = r >= 0 ? (int)rexb[r] - 141 : 0;   // the row's exponent, h_row_exp of its byte
        }
        // absent routes and columns past N read zero bytes (zb) instead of branching
        const int kb = (kt0 + ic.kt) * 128 + 32 * g;
        const v4i *hp = (const v4i *)(r >= 0 && kb < N ? (const uint8_t *)(hb_s + r * (nh + 8) + (kb - c0)) : zb);
        v4i B[4];
#pragma unroll
        for (int st = 0; st < 4; st++) B[st] = hp[st];
        uint32_t d[4];
        if constexpr (WF == W_NVFP4) {
#pragma unroll
          for (int i = 0; i < 4; i++) d[i] = (uint32_t)A16[s][i];
        } else {
#pragma unroll
          for (int i = 0; i < 3; i++) d[i] = (uint32_t)A3[s][i];
          d[3] = WF == 0 ? A4[s] : 0u;
        }
        const uint32_t sc = sa[s];
        if (WF == W_NVFP4 || (WF == 0 && ic.fmt == W_NVFP4)) {
          const v2h sp = e4m3x2_h(sc);
#pragma unroll
          for (int st = 0; st < 4; st++)
            acc = mfma_f16(nvfp4_step_h(d[st], st < 2 ? sp.x : sp.y), __builtin_bit_cast(v8h, B[st]), acc);
        } else {
          uint32_t t01, t23;
          nf3_tables_h(e4m3_f32((l & 1) ? (sc >> 8) & 0xFFu : sc & 0xFFu), t01, t23);
#pragma unroll
          for (int st = 0; st < 4; st++)
            acc = mfma_f16(nf3_step_h(st < 2 ? d[0] : d[1], d[2], st, t01, t23), __builtin_bit_cast(v8h, B[st]), acc);
        }
        if (ic.kt == nkh - 1 || base + s + 1 == i1) {
          const float wgt = r >= 0 ? wr_s[r] * ic.g2 : 0.f;
#pragma unroll
          for (int i = 0; i < 4; i++) tok[i] += __builtin_amdgcn_ldexpf(acc[i], er) * wgt;
          acc = v4f{0.f, 0.f, 0.f, 0.f};
        }
        g2_next(ic, a, ng, nkh, tb);
      }
      issue(s);   // the item kG2RingA16 ahead (out of range past the slice)
    }
  }
  float *tw = &yb[w][0];   // this wave's token sums [4][64]
#pragma unroll
  for (int i = 0; i < 4; i++) tw[i * 64 + l] = tok[i];
  __syncthreads();
  if (w != 0) return;
  float s4[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    s4[i] = 0.f;
#pragma unroll
    for (int v = 0; v < kDecG2WavesA8; v++) s4[i] += yb[v][i * 64 + l];
  }
  if (halves == 2) {
    // token c, columns 4g .. 4g + 3 of the tile
    float *accp = a.dpart + (size_t)rt * 256 + c * 16 + 4 * g;
    float done = 0.f;
    if (c < a.T) {
#pragma unroll
      for (int i = 0; i < 4; i++)
        done += __hip_atomic_fetch_add(accp + i, s4[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("" ::"v"(done));   // the returned values are waited for here
    wait_vm<0>();
    int prev = 0;
    if (l == 0) prev = __hip_atomic_fetch_add(a.dcnt + rt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__shfl(prev, 0) == 0) return;   // the other half writes the output
    if (c < a.T) {
#pragma unroll
      for (int i = 0; i < 4; i++) s4[i] = __hip_atomic_fetch_add(accp + i, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (c < a.T) {
    uint2 o;
    o.x = pack_bf16x2(s4[0], s4[1]);
    o.y = pack_bf16x2(s4[2], s4[3]);
    *(uint2 *)(a.out + (size_t)c * K + rt * 16 + 4 * g) = o;
  }
}

int decode_cpass(int K, int a8) {
  const int row = a8 ? K + 16 + K / 32 : 2 * (K + 8);
  return max(1, min(kDecodeMaxT, kDecStageBytes / row));
}

size_t decode_gemm1_lds(int K, int cpass, int a8) {
  const size_t stage = a8 ? (size_t)cpass * (K + 16) + (size_t)cpass * (K / 32) : (size_t)cpass * 2 * (K + 8);
  const size_t red = (size_t)4 * 16 * 64 * sizeof(float);
  return ((stage > red ? stage : red) + 15) & ~(size_t)15;
}

hipError_t launch_decode(int a8, const DecArgs &a, hipStream_t s, hipEvent_t ev_mid) {
  if (a.R == 0) return hipSuccess;
  int U = a.tier[0].E + (a.n_tiers > 1 ? a.tier[1].E : 0);
  const dim3 g1(a.N1 / 32, (unsigned)min(a.R, U)), g2(a.K / 16);
  const size_t lds1 = decode_gemm1_lds(a.K, a.cpass, a8);
  if (a8) hipLaunchKernelGGL(k_dec_gemm1_a8, g1, dim3(256), lds1, s, a);
  else hipLaunchKernelGGL(k_dec_gemm1_a16, g1, dim3(256), lds1, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ev_mid) {
    e = hipEventRecord(ev_mid, s);
    if (e != hipSuccess) return e;
  }
  const size_t lds2 = a8 ? (size_t)dec2_hq_bytes(a.R, a.N) + dec2_hs_bytes(a.R, a.N) : 0;
  if (a8) hipLaunchKernelGGL(k_dec_gemm2_a8, g2, dim3(kDecG2WavesA8 * 64), lds2, s, a);
  else {
    const int f0 = a.tier[0].fmt, f1 = a.n_tiers > 1 ? a.tier[1].fmt : f0;
    const dim3 g2h(a.K / 16 * dec2_a16_halves(a.N));
    const size_t lds = (size_t)dec2_hb_bytes(a.R, min(dec2_a16_cols0(a.N), a.N));
    if (f0 == W_NVFP4 && f1 == W_NVFP4) hipLaunchKernelGGL(k_dec_gemm2_a16r<W_NVFP4>, g2h, dim3(kDecG2WavesA8 * 64), lds, s, a);
    else if (f0 == W_NF3 && f1 == W_NF3) hipLaunchKernelGGL(k_dec_gemm2_a16r<W_NF3>, g2h, dim3(kDecG2WavesA8 * 64), lds, s, a);
    else hipLaunchKernelGGL(k_dec_gemm2_a16r<0>, g2h, dim3(kDecG2WavesA8 * 64), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
