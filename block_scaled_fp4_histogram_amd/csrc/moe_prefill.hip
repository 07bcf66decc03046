// Prefill-size W4A8 GEMMs: tiles of 64 routes of one expert, operands staged
// through LDS and shared by a 2 x 2 grid of waves.
//
// Per 128-column k-tile a block stages 8 weight row tiles (8 x 1 KB of FP4 in
// MFMA lane order + 8 x 64 E8M0 bytes) and the 64 routes' MXFP8 activation
// slices (64 x 128 bytes + 64 x 4 scale bytes) into one of two LDS buffers
// while the waves multiply the other.  Wave (wr, wc) owns row tiles 4*wr..+3
// and routes 32*wc..+31: 8 block-scaled MFMAs per k-tile from 4 weight and 2
// activation operands.  Each weight byte is read from memory once per 64
// routes, each activation byte once per 64 (GEMM1) or 128 (GEMM2) outputs.
//
//   k_pf_gemm1_a8  grid (N/64 intermediate blocks, tiles): up/gate GEMMs over K,
//                  clamped SwiGLU and MXFP8 requantisation of 64 intermediate
//                  columns of 64 routes.
//   k_pf_gemm2_a8  grid (K/128 output blocks, tiles): down GEMM over N; the
//                  accumulators are transposed through LDS so each combine
//                  store (fp32 atomic or bf16 route-buffer write) covers
//                  consecutive output columns of one route.
#include "moe_device.h"

namespace moe {

constexpr int kPfRowTiles = 8;   // weight row tiles per block
constexpr int kPfBStride = 144;  // LDS bytes per activation row (128 + 16: rows on different banks)

struct PfStage {
  uint8_t A[kPfRowTiles][1024];
  uint8_t As[kPfRowTiles][64];
  uint8_t B[kPfTileRows][kPfBStride];
  uint8_t Bs[kPfTileRows][4];
};

union PfLds {
  PfStage st[2];
  float tr[kPfTileRows][132];   // GEMM2 epilogue: [route][128 columns + pad]
};

// Registers of one thread's share of a stage: 2 weight chunks, 1 scale dword,
// 2 activation chunks, 1 activation-scale dword.
struct PfRegs {
  v4i a[2], b[2];
  uint32_t as, bs;
};

// Global -> registers.  Weight chunk q = tid + 256 j: row tile q / 64, lane q % 64.
// Activation chunk q: route row q / 8, 16-byte part q % 8 (parts at or past
// n_valid_parts of a partial k-tile are zero).
__device__ __forceinline__ void pf_load(PfRegs &R, const Buf &wb, const Buf &sb, uint32_t w0, uint32_t wstep,
                                        uint32_t s0, uint32_t sstep, int kt, const Buf &xb, const Buf &xsb,
                                        const uint32_t *xrow_off, const uint32_t *xsrow_off, const bool *rvalid,
                                        int kbytes, int kscales, int tid) {
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const uint32_t q = tid + 256 * j, rt = q >> 6, ln = q & 63;
    // lanes of a 32-column group past the reduction length hold no data (partial k-tile)
    const bool in = (uint32_t)kt * 128 + 32 * (ln >> 4) < (uint32_t)kbytes;
    R.a[j] = in ? buf_load16(wb, (uint32_t)kt * 1024u + ln * 16u, w0 + rt * wstep) : v4i{0, 0, 0, 0};
  }
  if (tid < 128) {   // 8 row tiles x 64 scale bytes = 128 dwords (dword-aligned: K/2 and N/2 are multiples of 16)
    const uint32_t rt = tid >> 4, d = tid & 15;
    const bool in = (uint32_t)kt * 4 + (d >> 2) < (uint32_t)kscales;   // the 4 lanes of dword d share one group
    R.as = in ? buf_load4(sb, (uint32_t)kt * 64u + 4 * d, s0 + rt * sstep) : 0u;
  }
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int q = tid + 256 * j, part = q & 7;   // row q / 8 is the row of xrow_off[j]
    const bool in = rvalid[j] && kt * 128 + part * 16 < kbytes;
    R.b[j] = in ? buf_load16(xb, xrow_off[j] + (uint32_t)(kt * 128 + part * 16), 0) : v4i{0, 0, 0, 0};
  }
  if (tid < 64) {
    uint32_t v = 0;
    if (rvalid[2]) {
#pragma unroll
      for (int j = 0; j < 4; j++)
        if (kt * 4 + j < kscales) v |= buf_load1(xsb, xsrow_off[0] + (uint32_t)(kt * 4 + j), 0) << (8 * j);
    }
    R.bs = v;
  }
}

__device__ __forceinline__ void pf_store(PfStage &S, const PfRegs &R, int tid) {
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int q = tid + 256 * j;
    *(v4i *)&S.A[q >> 6][(q & 63) * 16] = R.a[j];
  }
  if (tid < 128) *(uint32_t *)&S.As[tid >> 4][(tid & 15) * 4] = R.as;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int q = tid + 256 * j;
    *(v4i *)&S.B[q >> 3][(q & 7) * 16] = R.b[j];
  }
  if (tid < 64) *(uint32_t *)&S.Bs[tid][0] = R.bs;
}

// 8 MFMAs of wave (wr, wc) on one staged k-tile.
__device__ __forceinline__ void pf_mfma(const PfStage &S, int wr, int wc, int l, v4f (*acc)[2]) {
  const int c = l & 15, g = l >> 4;
  v8i bop[2];
  int sb[2];
#pragma unroll
  for (int cb = 0; cb < 2; cb++) {
    const int row = 32 * wc + 16 * cb + c;
    const v4i b0 = *(const v4i *)&S.B[row][16 * g];
    const v4i b1 = *(const v4i *)&S.B[row][64 + 16 * g];
    bop[cb] = v8i{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    sb[cb] = S.Bs[row][g];
  }
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const v4i a = *(const v4i *)&S.A[4 * wr + q][l * 16];
    const int sa = S.As[4 * wr + q][l];
#pragma unroll
    for (int cb = 0; cb < 2; cb++) acc[q][cb] = mfma_fp4_fp8(a, bop[cb], acc[q][cb], sa, sb[cb]);
  }
}

// The k-loop shared by both GEMMs: double-buffered LDS stages, one barrier per
// k-tile.  kbytes / kscales: reduction length in bytes of activation / scales.
__device__ __forceinline__ void pf_kloop(PfLds &L, const Buf &wb, const Buf &sb, uint32_t w0, uint32_t wstep,
                                         uint32_t s0, uint32_t sstep, const Buf &xb, const Buf &xsb,
                                         const uint32_t *xrow_off, const uint32_t *xsrow_off, const bool *rvalid,
                                         int kbytes, int kscales, v4f (*acc)[2]) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, wr = w >> 1, wc = w & 1;
  const int nkt = (kbytes + 127) / 128;
  PfRegs R;
  pf_load(R, wb, sb, w0, wstep, s0, sstep, 0, xb, xsb, xrow_off, xsrow_off, rvalid, kbytes, kscales, tid);
  pf_store(L.st[0], R, tid);
  __syncthreads();
  for (int kt = 0; kt < nkt; kt++) {
    const bool more = kt + 1 < nkt;
    if (more) pf_load(R, wb, sb, w0, wstep, s0, sstep, kt + 1, xb, xsb, xrow_off, xsrow_off, rvalid, kbytes, kscales, tid);
    pf_mfma(L.st[kt & 1], wr, wc, l, acc);
    if (more) pf_store(L.st[(kt + 1) & 1], R, tid);
    __syncthreads();
  }
}

// ---------------------------------------------------------------- GEMM1
__global__ __launch_bounds__(256) void k_pf_gemm1_a8(GemmArgs a) {
  __shared__ PfLds L;
  const TileInfo ti = tile_info(a);
  if (!ti.valid) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4, wr = w >> 1, wc = w & 1;
  const int K = a.K, N = a.N, hb = blockIdx.x;
  const size_t rt_bytes = (size_t)16 * (K / 2), rt_scales = (size_t)16 * (K / 32);
  const Buf wb = make_buf(a.w13 + (size_t)ti.e * (2 * N) * (K / 2), (uint32_t)((size_t)(2 * N) * (K / 2)));
  const Buf sb = make_buf(a.s13 + (size_t)ti.e * (2 * N) * (K / 32), (uint32_t)((size_t)(2 * N) * (K / 32)));
  // activation rows of this thread's staging chunks (rows tid/8 and tid/8 + 32) and scale row (tid < 64)
  const int T = a.T;
  const Buf xb = make_buf(a.xq, (uint32_t)((size_t)T * K));
  const Buf xsb = make_buf(a.xs, (uint32_t)((size_t)T * (K / 32)));
  uint32_t xrow_off[2], xsrow_off[1];
  bool rvalid[3];
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int row = (tid + 256 * j) >> 3;
    rvalid[j] = row < ti.rows;
    const int t = rvalid[j] ? a.perm[ti.p0 + row] / a.topk : 0;
    xrow_off[j] = (uint32_t)((size_t)t * K);
  }
  {
    rvalid[2] = tid < 64 && tid < ti.rows;
    const int t = rvalid[2] ? a.perm[ti.p0 + tid] / a.topk : 0;
    xsrow_off[0] = (uint32_t)((size_t)t * (K / 32));
  }
  v4f acc[4][2];
#pragma unroll
  for (int q = 0; q < 4; q++)
#pragma unroll
    for (int cb = 0; cb < 2; cb++) acc[q][cb] = v4f{0.f, 0.f, 0.f, 0.f};
  pf_kloop(L, wb, sb, (uint32_t)((size_t)(8 * hb) * rt_bytes), (uint32_t)rt_bytes, (uint32_t)((size_t)(8 * hb) * rt_scales),
           (uint32_t)rt_scales, xb, xsb, xrow_off, xsrow_off, rvalid, K, K / 32, acc);
  // epilogue: row tiles 4wr + {0,1,2,3} = up/gate of intermediate blocks 4hb + 2wr + {0,1}
#pragma unroll
  for (int cb = 0; cb < 2; cb++) {
    float h[8];
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
      for (int i = 0; i < 4; i++) h[s * 4 + i] = silu_clamped(acc[2 * s + 1][cb][i], acc[2 * s][cb][i], a.limit, a.has_limit);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(h[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    float inv;
    const uint32_t sbyte = mx_scale(amax, &inv);
    const int row = 32 * wc + 16 * cb + c;
    if (row < ti.rows) {
      const size_t p = (size_t)(ti.p0 + row);
#pragma unroll
      for (int s = 0; s < 2; s++)
        *(uint32_t *)(a.hq + p * N + 64 * hb + 32 * wr + 16 * s + 4 * g) =
            e4m3x4(h[s * 4], h[s * 4 + 1], h[s * 4 + 2], h[s * 4 + 3], inv);
      if (g == 0) a.hs[p * hs_stride(N) + 2 * hb + wr] = (uint8_t)sbyte;
    }
  }
}

// ---------------------------------------------------------------- GEMM2
__global__ __launch_bounds__(256) void k_pf_gemm2_a8(GemmArgs a) {
  __shared__ PfLds L;
  const TileInfo ti = tile_info(a);
  if (!ti.valid) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4, wr = w >> 1, wc = w & 1;
  const int K = a.K, N = a.N, ob = blockIdx.x;   // output columns 128 ob .. +127 = w2 row tiles 8 ob .. +7
  const size_t rt_bytes = (size_t)16 * (N / 2), rt_scales = (size_t)16 * (N / 32);
  const Buf wb = make_buf(a.w2 + (size_t)ti.e * K * (N / 2), (uint32_t)((size_t)K * (N / 2)));
  const Buf sb = make_buf(a.s2 + (size_t)ti.e * K * (N / 32), (uint32_t)((size_t)K * (N / 32)));
  const Buf hb = make_buf(a.hq, (uint32_t)((size_t)(ti.p0 + ti.rows) * N));
  const Buf hsb = make_buf(a.hs, (uint32_t)((size_t)(ti.p0 + ti.rows) * hs_stride(N)));
  uint32_t hrow_off[2], hsrow_off[1];
  bool rvalid[3];
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int row = (tid + 256 * j) >> 3;
    rvalid[j] = row < ti.rows;
    hrow_off[j] = (uint32_t)((size_t)(ti.p0 + row) * N);
  }
  rvalid[2] = tid < 64 && tid < ti.rows;
  hsrow_off[0] = (uint32_t)((size_t)(ti.p0 + tid) * hs_stride(N));
  v4f acc[4][2];
#pragma unroll
  for (int q = 0; q < 4; q++)
#pragma unroll
    for (int cb = 0; cb < 2; cb++) acc[q][cb] = v4f{0.f, 0.f, 0.f, 0.f};
  pf_kloop(L, wb, sb, (uint32_t)((size_t)(8 * ob) * rt_bytes), (uint32_t)rt_bytes, (uint32_t)((size_t)(8 * ob) * rt_scales),
           (uint32_t)rt_scales, hb, hsb, hrow_off, hsrow_off, rvalid, N, N / 32, acc);
  // per-row route, token and router weight
  __shared__ int s_r[kPfTileRows];
  __shared__ float s_w[kPfTileRows];
  if (tid < ti.rows) {
    const int r = a.perm[ti.p0 + tid];
    s_r[tid] = r;
    s_w[tid] = a.topk_w[r];
  }
  // transpose: wave (wr, wc), lane (c, g): columns 64 wr + 16 q + 4 g + i of route 32 wc + 16 cb + c
#pragma unroll
  for (int q = 0; q < 4; q++)
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
      for (int i = 0; i < 4; i++) L.tr[32 * wc + 16 * cb + c][64 * wr + 16 * q + 4 * g + i] = acc[q][cb][i];
  __syncthreads();
  const size_t col0 = (size_t)128 * ob;
  if (a.deterministic) {
    // bf16 route buffer: 2 columns per thread, 64 routes x 64 column pairs
    for (int idx = tid; idx < kPfTileRows * 64; idx += 256) {
      const int row = idx >> 6, cp = idx & 63;
      if (row >= ti.rows) break;
      const int r = s_r[row];
      const float wgt = s_w[row];
      *(uint32_t *)(a.rb + (size_t)r * K + col0 + 2 * cp) = pack_bf16x2(wgt * L.tr[row][2 * cp], wgt * L.tr[row][2 * cp + 1]);
    }
  } else {
    // fp32 atomics: each wave instruction adds 64 consecutive columns of one route
    for (int idx = tid; idx < kPfTileRows * 128; idx += 256) {
      const int row = idx >> 7, col = idx & 127;
      if (row >= ti.rows) break;
      atomicAdd(a.out_acc + (size_t)(s_r[row] / a.topk) * K + col0 + col, s_w[row] * L.tr[row][col]);
    }
  }
}

hipError_t launch_pf_gemm1(const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pf_gemm1_a8, dim3(a.N / 64, grid_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pf_gemm2(const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pf_gemm2_a8, dim3(a.K / 128, grid_tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
