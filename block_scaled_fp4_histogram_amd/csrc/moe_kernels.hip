// gfx950 kernels of the routed MoE layer with block-scaled 4-bit expert weights.
//
// Three launch sequences by batch size (the host picks one per chunk):
//   * decode batches (<= 16 tokens, <= 64 routes): two kernels, see
//     moe_decode.hip;
//   * prefill batches (>= 128 tokens, N % 64 == 0): the route planner below,
//     then the 64-route-tile GEMMs of moe_prefill.hip, then the combine below;
//   * everything between: the route planner, the 16-route-tile GEMMs of this
//     file, then the combine.
// The planner and combine of the last two (one chunk of T tokens, R = T * top_k
// routes):
//   k_route      expert histogram, prefix offsets, stable route permutation and
//                the tile table (one block when R <= kRouteChunk; otherwise
//                count -> scan -> scatter); extra blocks of the one-block launch
//                or of the scan quantise x to MXFP8 and clear the fp32
//                accumulator.
//   k_gemm1_*    per (tile of 16 routes of one expert, 32 intermediate columns):
//                up and gate GEMMs over K, clamped SwiGLU, requantisation of h
//                (MXFP8 for W4A8, bf16 for W4A16/W3A16).
//   k_gemm2_*    per (tile, 64 output columns): down GEMM over N, router weight,
//                then fp32 atomics (atomic combine) or a bf16 per-slot route
//                buffer (deterministic combine).
//   k_cast / k_topk_sum   fp32 accumulator -> bf16, or fixed slot-order sum.
//
// Operand layouts of the block-scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4
// (A = 16 weight rows x 128 k, FP4; B = 128 k x 16 routes, FP8 E4M3), as
// measured on gfx950: an FP4 operand lane l holds row (l % 16) and the 32
// consecutive k of block (l / 16), element 2i in the low nibble of byte i; an
// FP8 operand lane l holds column (l % 16), bytes 0..15 at k = 16*(l/16) + j and
// bytes 16..31 at k = 64 + 16*(l/16) + j; lane l supplies the E8M0 scale of
// (row or column l % 16, 32-block l / 16); the accumulator lane l holds column
// l % 16, rows 4*(l/16) .. +3.
#include "moe_device.h"

namespace moe {

// ------------------------------------------------------------ route planner

__device__ __forceinline__ int resolve_u(int id, const RouteArgs &a) {
  if (id < 0 || id >= a.E) return -1;
  const int e0 = a.emap0 ? a.emap0[id] : id;
  if (e0 >= 0 && e0 < a.E0) return e0;
  if (a.n_tiers > 1) {
    const int e1 = a.emap1 ? a.emap1[id] : id;
    if (e1 >= 0 && e1 < a.E1) return a.E0 + e1;
  }
  return -1;
}

// Tile table of `rows` routes per tile from the per-expert counts: wave 1
// scans the tile counts (each lane owns a run of consecutive experts, runs
// combined with a wave prefix sum) into LDS tbeg[U+1]; after the barrier each
// thread writes whole tiles, finding a tile's expert by binary search over
// tbeg (one thread per expert would write a hot expert's ~60 tiles alone).
__device__ void write_tiles(const RouteArgs &a, int U, const int *cnt, int *tbeg, int rows, int32_t *tile_u,
                            int32_t *tile_row0, int32_t *tier_tiles) {
  const int tid = threadIdx.x;
  if (tid >= 64 && tid < 128) {
    const int lane = tid - 64, per = (U + 63) / 64, b = lane * per;
    int nt = 0;
    for (int i = 0; i < per; i++)
      if (b + i < U) nt += (cnt[b + i] + rows - 1) / rows;
    int it = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int vt = __shfl_up(it, d);
      if (lane >= d) it += vt;
    }
    int rt = it - nt;
    for (int i = 0; i < per; i++)
      if (b + i < U) {
        tbeg[b + i] = rt;
        rt += (cnt[b + i] + rows - 1) / rows;
      }
    if (lane == 63) tbeg[U] = it;
  }
  __syncthreads();
  const int ntiles = tbeg[U];
  for (int t = tid; t < ntiles; t += blockDim.x) {
    int lo = 0, hi = U - 1;   // the last u with tbeg[u] <= t (experts without routes have empty ranges)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (tbeg[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    tile_u[t] = lo;
    tile_row0[t] = (t - tbeg[lo]) * rows;
  }
  if (tid == 0) {
    tier_tiles[0] = 0;
    tier_tiles[1] = tbeg[a.E0];
    tier_tiles[2] = tbeg[a.E0];
    tier_tiles[3] = tbeg[U];
  }
}

// Offsets and tile table(s) from per-expert counts held in LDS cnt[U].  Wave 0
// scans the counts (each lane owns a run of consecutive experts, runs combined
// with a wave prefix sum); leaves the exclusive offsets in LDS off[U+1].
__device__ void finish_plan(const RouteArgs &a, int U, const int *cnt, int *off, int *tbeg) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int per = (U + 63) / 64, b = tid * per;
    int s = 0;
    for (int i = 0; i < per; i++)
      if (b + i < U) s += cnt[b + i];
    int is = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int vs = __shfl_up(is, d);
      if (tid >= d) is += vs;
    }
    int rs = is - s;
    for (int i = 0; i < per; i++)
      if (b + i < U) {
        off[b + i] = rs;
        rs += cnt[b + i];
      }
    if (tid == 63) off[U] = is;
  }
  write_tiles(a, U, cnt, tbeg, a.tile_rows, a.tile_u, a.tile_row0, a.tier_tiles);
  for (int u = tid; u <= U; u += blockDim.x) a.off[u] = off[u];
  for (int u = tid; u < U; u += blockDim.x) a.cnt[u] = cnt[u];
  if (a.tile_u2) {
    __syncthreads();   // tbeg is reused
    write_tiles(a, U, cnt, tbeg, a.tile_rows2, a.tile_u2, a.tile_row02, a.tier_tiles2);
  }
}

// Work fused into the route launches: MXFP8 quantisation of x (one thread per
// 32-element block) and clearing of the fp32 accumulator, part `part` of
// `nparts` equal slices (a launch's side blocks sb = 0 .. side_blocks - 1 take
// one part; with several chunks the histogram launch and the scan launch each
// take one, beside their latency-bound route work).
__device__ void route_side_work(const RouteArgs &a, int sb, int part, int nparts) {
  const long stride = (long)a.side_blocks * blockDim.x;
  const long i0 = (long)sb * blockDim.x + threadIdx.x;
  if (a.xq) {
    const long nall = (long)a.T * (a.K / 32), nblk = nall * (part + 1) / nparts;
    for (long i = nall * part / nparts + i0; i < nblk; i += stride) {
      const v4i *src = (const v4i *)(a.x + i * 32);
      v4i x4[4];
#pragma unroll
      for (int q = 0; q < 4; q++) x4[q] = src[q];
      uint32_t codes[8];
      const uint32_t s = quant_block32_bf16(x4, codes);   // the decode path's quantiser, bit for bit
      v4i *dst = (v4i *)(a.xq + i * 32);
      dst[0] = v4i{(int)codes[0], (int)codes[1], (int)codes[2], (int)codes[3]};
      dst[1] = v4i{(int)codes[4], (int)codes[5], (int)codes[6], (int)codes[7]};
      a.xs[i] = (uint8_t)s;
    }
  }
  if (a.zero_buf) {
    const long nall = a.zero_n / 4, n4 = nall * (part + 1) / nparts;
    for (long i = nall * part / nparts + i0; i < n4; i += stride) ((v4f *)a.zero_buf)[i] = v4f{0.f, 0.f, 0.f, 0.f};
  }
}

// One block per chunk of kRouteChunk routes (16 waves x 64).  Each route's
// rank among the routes of its expert with a smaller index is found with wave
// ballots (the lanes of one expert are found together; no LDS round trip in
// the loop), then the waves' counts are scanned per expert, so the permutation
// is a stable counting sort.  SINGLE: the grid has one route block, which also
// scans and scatters.
constexpr int kRouteWaves = 16, kRouteRounds = kRouteChunk / (64 * kRouteWaves);
static_assert(kRouteRounds == 1, "one 64-route round per wave");

template <bool SINGLE>
__global__ __launch_bounds__(64 * kRouteWaves) void k_route(RouteArgs a) {
  if ((int)blockIdx.x >= a.G) {
    route_side_work(a, blockIdx.x - a.G, 0, SINGLE ? 1 : 2);
    return;
  }
  __shared__ uint16_t whist[kRouteWaves][kMaxExperts];   // per wave: count, then exclusive prefix
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int tbeg[kMaxExperts + 1];
  const int U = a.E0 + a.E1;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  for (int u = tid; u < U; u += 64 * kRouteWaves)
#pragma unroll
    for (int v = 0; v < kRouteWaves; v++) whist[v][u] = 0;
  __syncthreads();
  const int b = blockIdx.x;
  const int r = b * kRouteChunk + w * 64 + lane;
  const int u = (r < a.R) ? resolve_u(a.ids[r], a) : -1;
  int rk = 0;
  {
    const unsigned long long ltmask = (1ull << lane) - 1ull;
    unsigned long long rem = __ballot(u >= 0);
    while (rem) {
      const int leader = __ffsll((unsigned long long)rem) - 1;
      const int lu = __shfl(u, leader);
      const unsigned long long m = __ballot(u == lu);
      if (u == lu) rk = __popcll(m & ltmask);
      if (lane == leader) whist[w][lu] = (uint16_t)__popcll(m);
      rem &= ~m;
    }
  }
  __syncthreads();
  // wave prefixes within the chunk; chunk totals
  for (int x = tid; x < U; x += 64 * kRouteWaves) {
    int run = 0;
#pragma unroll
    for (int v = 0; v < kRouteWaves; v++) {
      const int c = whist[v][x];
      whist[v][x] = (uint16_t)run;
      run += c;
    }
    if (SINGLE) cnt[x] = run;
    else a.chunk_hist[b * U + x] = run;
  }
  __syncthreads();
  if (u >= 0) rk += whist[w][u];
  if (!SINGLE) {
    if (r < a.R) {
      a.ru[r] = u;
      a.lrank[r] = rk;
    }
    return;
  }
  // single chunk: the chunk totals are the expert counts
  finish_plan(a, U, cnt, off, tbeg);
  __syncthreads();
  if (r < a.R) {
    if (u >= 0) {
      const int pos = off[u] + rk;
      a.perm[pos] = r;
      a.inv[r] = pos;
    } else {
      a.inv[r] = -1;
    }
  }
}

// Multi-chunk: per-expert scan over chunks, offsets, tile table.  One thread
// per expert; up to 32 chunk counts are read in one batch and kept in
// registers for the second pass (more chunks take further batches).  The
// launch's other blocks do the side work (quantising x, clearing the
// accumulator), which the scan's one latency-bound block then runs under
// instead of after (4096 tokens at K = 7168: planner 35 -> 25 us).
__global__ __launch_bounds__(1024) void k_route_scan(RouteArgs a) {
  if (blockIdx.x > 0) {
    route_side_work(a, blockIdx.x - 1, 1, 2);
    return;
  }
  __shared__ int cnt[kMaxExperts];
  __shared__ int off[kMaxExperts + 1];
  __shared__ int tbeg[kMaxExperts + 1];
  const int U = a.E0 + a.E1, u = threadIdx.x;
  constexpr int B = 32;
  int v[B];
  if (u < U) {
#pragma unroll
    for (int j = 0; j < B; j++) v[j] = j < a.G ? a.chunk_hist[j * U + u] : 0;
    int run = 0;
#pragma unroll
    for (int j = 0; j < B; j++) run += v[j];
    for (int b0 = B; b0 < a.G; b0 += B) {
      int x[B];
#pragma unroll
      for (int j = 0; j < B; j++) x[j] = b0 + j < a.G ? a.chunk_hist[(b0 + j) * U + u] : 0;
#pragma unroll
      for (int j = 0; j < B; j++) run += x[j];
    }
    cnt[u] = run;
  }
  __syncthreads();
  finish_plan(a, U, cnt, off, tbeg);
  __syncthreads();
  if (u < U) {
    int run = off[u];
#pragma unroll
    for (int j = 0; j < B; j++)
      if (j < a.G) {
        a.chunk_hist[j * U + u] = run;
        run += v[j];
      }
    for (int b0 = B; b0 < a.G; b0 += B) {
      int x[B];
#pragma unroll
      for (int j = 0; j < B; j++) x[j] = b0 + j < a.G ? a.chunk_hist[(b0 + j) * U + u] : 0;
#pragma unroll
      for (int j = 0; j < B; j++)
        if (b0 + j < a.G) {
          a.chunk_hist[(b0 + j) * U + u] = run;
          run += x[j];
        }
    }
  }
}

__global__ __launch_bounds__(256) void k_route_scatter(RouteArgs a) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= a.R) return;
  const int U = a.E0 + a.E1;
  const int u = a.ru[r];
  if (u < 0) {
    a.inv[r] = -1;
    return;
  }
  const int pos = a.chunk_hist[(r / kRouteChunk) * U + u] + a.lrank[r];
  a.perm[pos] = r;
  a.inv[r] = pos;
}

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
  if (a.G == 1) {
    hipLaunchKernelGGL(k_route<true>, dim3(1 + a.side_blocks), dim3(64 * kRouteWaves), 0, s, a);
  } else {
    hipLaunchKernelGGL(k_route<false>, dim3(a.G + a.side_blocks), dim3(64 * kRouteWaves), 0, s, a);
    hipLaunchKernelGGL(k_route_scan, dim3(1 + a.side_blocks), dim3(1024), 0, s, a);
    hipLaunchKernelGGL(k_route_scatter, dim3((a.R + 255) / 256), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ quantisers

// The MXFP8 quantiser every bf16 activation path runs (quant_block32_bf16).
__global__ __launch_bounds__(256) void k_quant_bf16(const uint16_t *x, long nblk, uint8_t *q, uint8_t *sc) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblk) return;
  v4i x4[4];
  for (int j = 0; j < 4; j++) x4[j] = ((const v4i *)(x + i * 32))[j];
  uint32_t codes[8];
  sc[i] = (uint8_t)quant_block32_bf16(x4, codes);
  for (int j = 0; j < 8; j++) ((uint32_t *)(q + i * 32))[j] = codes[j];
}

__global__ __launch_bounds__(256) void k_quant_f32(const float *h, long nblk, uint8_t *q, uint8_t *sc) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblk) return;
  float v[32];
  for (int j = 0; j < 32; j++) v[j] = h[i * 32 + j];
  uint32_t codes[8];
  sc[i] = (uint8_t)quant_block32(v, codes);
  for (int j = 0; j < 8; j++) ((uint32_t *)(q + i * 32))[j] = codes[j];
}

hipError_t launch_quant_bf16(const uint16_t *x, long rows, int cols, uint8_t *q, uint8_t *sc, hipStream_t s) {
  const long nblk = rows * (cols / 32);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_bf16, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s, x, nblk, q, sc);
  return hipGetLastError();
}

hipError_t launch_quant_f32(const float *h, long rows, int cols, uint8_t *q, uint8_t *sc, hipStream_t s) {
  const long nblk = rows * (cols / 32);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_f32, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, s, h, nblk, q, sc);
  return hipGetLastError();
}

// ------------------------------------------------------------ tile schedule

// -------------------------------------------------- W4A8 (MXFP4 x MXFP8)

// Weight tile layout (per expert, per matrix of R rows x Kd columns): row tiles
// of 16 rows; within a row tile, k-tiles of 128 columns, each stored lane-major
// (lane l = row + 16*q holds the 32 columns 128*kt + 32*q .. +31 of its row),
// 16 bytes per lane for FP4.  The last k-tile of a row tile may hold fewer
// 32-column groups (only its first 16*nq lanes exist).  Scales likewise, one
// byte per lane.  MXFP4 experts also keep second copies of the scales, for
// the prefill GEMMs, with the k-tiles of a row tile in mx_soff's order (a
// lane's bytes of four consecutive k-tiles in one dword).
// w13 row tiles interleave up and gate: tile 2j = up rows 16j..16j+15, tile
// 2j+1 = gate rows 16j..16j+15.

// grid: x = N/32 (intermediate column blocks), y = tiles; 4 waves split K
// (wave w takes k-tiles w, w+4, ...), loads double-buffered in registers.  At
// the batch sizes this sequence serves an expert mostly fills one tile, so its
// weights are read once: non-temporal loads (16 to 256 tokens at K = 7168:
// 11 to 12 % faster layers).
__global__ __launch_bounds__(256) void k_gemm1_a8(GemmArgs a) {
  const TileInfo ti = tile_info(a);
  if (!ti.valid) return;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 15, g = l >> 4;
  const int K = a.K, N = a.N, nkt = K / 128;
  const int hb = blockIdx.x;
  int t = -1;
  if (c < ti.rows) t = a.perm[ti.p0 + c] / a.topk;
  const bool have = t >= 0;
  const uint8_t *xrow = a.xq + (size_t)(have ? t : 0) * K;
  const uint8_t *xsrow = a.xs + (size_t)(have ? t : 0) * (K / 32);
  const size_t rt_bytes = (size_t)16 * (K / 2);
  const size_t rt_scales = (size_t)16 * (K / 32);
  const uint8_t *wt = a.w13 + (size_t)ti.e * (2 * N) * (K / 2) + (size_t)(4 * hb) * rt_bytes + l * 16;
  const uint8_t *st = a.s13 + (size_t)ti.e * (2 * N) * (K / 32) + (size_t)(4 * hb) * rt_scales + l;
  v4f acc[4];
#pragma unroll
  for (int q = 0; q < 4; q++) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
  A8G1Stage s0, s1;
  if (w < nkt) a8g1_load(s0, wt, st, rt_bytes, rt_scales, w, xrow, xsrow, have, g);
  for (int kt = w; kt < nkt; kt += 8) {
    if (kt + 4 < nkt) a8g1_load(s1, wt, st, rt_bytes, rt_scales, kt + 4, xrow, xsrow, have, g);
    a8g1_compute(s0, acc);
    if (kt + 8 < nkt) a8g1_load(s0, wt, st, rt_bytes, rt_scales, kt + 8, xrow, xsrow, have, g);
    if (kt + 4 < nkt) a8g1_compute(s1, acc);
  }
  __shared__ float red[4][16][64];
#pragma unroll
  for (int q = 0; q < 4; q++)
#pragma unroll
    for (int i = 0; i < 4; i++) red[w][q * 4 + i][l] = acc[q][i];
  __syncthreads();
  if (w != 0) return;
  float h[8];
#pragma unroll
  for (int s = 0; s < 2; s++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int iu = (2 * s) * 4 + i, ig = (2 * s + 1) * 4 + i;
      const float up = red[0][iu][l] + red[1][iu][l] + red[2][iu][l] + red[3][iu][l];
      const float gate = red[0][ig][l] + red[1][ig][l] + red[2][ig][l] + red[3][ig][l];
      h[s * 4 + i] = silu_clamped(gate, up, a.limit, a.has_limit, a.alpha, a.beta, a.act);
    }
  // MXFP8 block of 32 intermediate columns of route c: 8 values here x 4 lanes
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(h[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 16));
  amax = fmaxf(amax, __shfl_xor(amax, 32));
  float inv;
  const uint32_t sbyte = mx_scale(amax, &inv);
  if (c < ti.rows) {
    const size_t p = (size_t)(ti.p0 + c);
    const int n0 = hb * 32;
#pragma unroll
    for (int s = 0; s < 2; s++)
      *(uint32_t *)(a.hq + p * N + n0 + 16 * s + 4 * g) = e4m3x4(h[s * 4], h[s * 4 + 1], h[s * 4 + 2], h[s * 4 + 3], inv);
    if (g == 0) a.hs[p * hs_stride(N) + hb] = (uint8_t)sbyte;
  }
}

// Combine epilogue shared by the GEMM2 kernels: acc holds 4 output columns
// (f0 .. f0+3) of route column c.
__device__ __forceinline__ void combine_store(const GemmArgs &a, const TileInfo &ti, int c, int f0, v4f acc,
                                              float gscale) {
  if (c >= ti.rows) return;
  const int r = a.perm[ti.p0 + c];
  const float wgt = (a.w_on_input ? 1.0f : a.topk_w[r]) * gscale;
  if (a.deterministic) {
    uint2 v;
    v.x = pack_bf16x2(wgt * acc[0], wgt * acc[1]);
    v.y = pack_bf16x2(wgt * acc[2], wgt * acc[3]);
    *(uint2 *)(a.rb + (size_t)r * a.K + f0) = v;
  } else {
    float *o = a.out_acc + (size_t)(r / a.topk) * a.K + f0;
#pragma unroll
    for (int i = 0; i < 4; i++) atomicAdd(o + i, wgt * acc[i]);
  }
}

// grid: x = K/64 (output column blocks), y = tiles; wave w owns 16 columns.
// The reduction over N runs in batches of 4 k-tiles whose loads are all issued
// before the batch's MFMAs.
__global__ __launch_bounds__(256) void k_gemm2_a8(GemmArgs a) {
  const TileInfo ti = tile_info(a);
  if (!ti.valid) return;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 15, g = l >> 4;
  const int K = a.K, N = a.N, nkt = (N + 127) / 128;
  const int rt = blockIdx.x * 4 + w;
  const size_t rt_bytes = (size_t)16 * (N / 2);
  const size_t rt_scales = (size_t)16 * (N / 32);
  const uint8_t *wt = a.w2 + (size_t)ti.e * K * (N / 2) + (size_t)rt * rt_bytes + l * 16;
  const uint8_t *st = a.s2 + (size_t)ti.e * K * (N / 32) + (size_t)rt * rt_scales + l;
  const bool have = c < ti.rows;
  const uint8_t *hrow = a.hq + (size_t)(ti.p0 + (have ? c : 0)) * N;
  const uint8_t *hsrow = a.hs + (size_t)(ti.p0 + (have ? c : 0)) * hs_stride(N);
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  for (int kt0 = 0; kt0 < nkt; kt0 += 4) {
    v4i A[4], B0[4], B1[4];
    int sa[4], sb[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int kt = kt0 + j, kb = kt * 128;
      A[j] = B0[j] = B1[j] = v4i{0, 0, 0, 0};
      sa[j] = sb[j] = 0;
      if (kt < nkt && kb + 32 * g < N) {
        A[j] = __builtin_nontemporal_load((const v4i *)(wt + (size_t)kt * 1024));   // read once
        sa[j] = st[kt * 64];
      }
      if (have && kt < nkt) {
        if (kb + 16 * g < N) B0[j] = *(const v4i *)(hrow + kb + 16 * g);
        if (kb + 64 + 16 * g < N) B1[j] = *(const v4i *)(hrow + kb + 64 + 16 * g);
        if (kb + 32 * g < N) sb[j] = hsrow[kb / 32 + g];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const v8i bop = v8i{B0[j][0], B0[j][1], B0[j][2], B0[j][3], B1[j][0], B1[j][1], B1[j][2], B1[j][3]};
      acc = mfma_fp4_fp8(A[j], bop, acc, sa[j], sb[j]);
    }
  }
  combine_store(a, ti, c, rt * 16 + 4 * g, acc, 1.0f);
}

template <int WF>
__global__ __launch_bounds__(256) void k_gemm1_a16(GemmArgs a) {
  const TileInfo ti = tile_info(a);
  if (!ti.valid) return;
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 15, g = l >> 4;
  const int K = a.K, N = a.N, N1 = a.N1, nkt = K / 128, groups = K / 32;
  const int hb = blockIdx.x;
  int t = -1;
  if (c < ti.rows) t = a.perm[ti.p0 + c] / a.topk;
  const bool have = t >= 0;
  const uint16_t *xrow = a.xb + (size_t)(have ? t : 0) * K;
  const size_t rt_bytes = (size_t)16 * groups * U;
  const size_t rt_scales = (size_t)16 * groups * SU;
  const uint8_t *wt = a.w13 + (size_t)ti.e * (2 * N1) * groups * U + (size_t)(4 * hb) * rt_bytes + l * U;
  const uint8_t *st = a.s13 + (size_t)ti.e * (2 * N1) * groups * SU + (size_t)(4 * hb) * rt_scales + l * SU;
  v4f acc[4];
#pragma unroll
  for (int q = 0; q < 4; q++) acc[q] = v4f{0.f, 0.f, 0.f, 0.f};
  A16G1Stage<WF> s0, s1;
  if (w < nkt) a16g1_load(s0, wt, st, rt_bytes, rt_scales, w, xrow, have, g);
  for (int kt = w; kt < nkt; kt += 8) {
    if (kt + 4 < nkt) a16g1_load(s1, wt, st, rt_bytes, rt_scales, kt + 4, xrow, have, g);
    a16g1_compute(s0, acc);
    if (kt + 8 < nkt) a16g1_load(s0, wt, st, rt_bytes, rt_scales, kt + 8, xrow, have, g);
    if (kt + 4 < nkt) a16g1_compute(s1, acc);
  }
  __shared__ float red[4][16][64];
#pragma unroll
  for (int q = 0; q < 4; q++)
#pragma unroll
    for (int i = 0; i < 4; i++) red[w][q * 4 + i][l] = acc[q][i];
  __syncthreads();
  if (w != 0) return;
  if (c < ti.rows) {
    const size_t p = (size_t)(ti.p0 + c);
    // router weight on the input: GEMM1 is linear, so it scales the accumulators
    const float gs = (a.g13 ? a.g13[ti.e] : 1.0f) * (a.w_on_input ? a.topk_w[a.perm[p]] : 1.0f);
#pragma unroll
    for (int s = 0; s < 2; s++) {
      float h[4], h2[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int iu = (2 * s) * 4 + i, ig = (2 * s + 1) * 4 + i;
        const float up = (red[0][iu][l] + red[1][iu][l] + red[2][iu][l] + red[3][iu][l]) * gs;
        const float gate = (red[0][ig][l] + red[1][ig][l] + red[2][ig][l] + red[3][ig][l]) * gs;
        if (a.act == ACT_RELU2) {
          h[i] = relu2(up);
          h2[i] = relu2(gate);
        } else {
          h[i] = silu_clamped(gate, up, a.limit, a.has_limit, a.alpha, a.beta, a.act);
        }
      }
      uint2 v;
      v.x = pack_bf16x2(h[0], h[1]);
      v.y = pack_bf16x2(h[2], h[3]);
      *(uint2 *)(a.hb + p * N + hb * 32 + 16 * s + 4 * g) = v;
      if (a.act == ACT_RELU2) {   // the second half's rows: columns N1 + ...
        v.x = pack_bf16x2(h2[0], h2[1]);
        v.y = pack_bf16x2(h2[2], h2[3]);
        *(uint2 *)(a.hb + p * N + N1 + hb * 32 + 16 * s + 4 * g) = v;
      }
    }
  }
}

template <int WF>
__global__ __launch_bounds__(256) void k_gemm2_a16(GemmArgs a) {
  const TileInfo ti = tile_info(a);
  if (!ti.valid) return;
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63, c = l & 15, g = l >> 4;
  const int K = a.K, N = a.N, nkt = (N + 127) / 128, groups = N / 32;
  const int rt = blockIdx.x * 4 + w;
  const size_t rt_bytes = (size_t)16 * groups * U;
  const size_t rt_scales = (size_t)16 * groups * SU;
  const uint8_t *wt = a.w2 + (size_t)ti.e * K * groups * U + (size_t)rt * rt_bytes + l * U;
  const uint8_t *st = a.s2 + (size_t)ti.e * K * groups * SU + (size_t)rt * rt_scales + l * SU;
  const bool have = c < ti.rows;
  const uint16_t *hrow = a.hb + (size_t)(ti.p0 + (have ? c : 0)) * N;
  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
  for (int kt0 = 0; kt0 < nkt; kt0 += 2) {
    A16Tile<WF> A[2];
    v4i B[2][4];
#pragma unroll
    for (int j = 0; j < 2; j++) {
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
    for (int j = 0; j < 2; j++) {
      const typename A16Tile<WF>::Deq dq = A[j].prep();
#pragma unroll
      for (int s = 0; s < 4; s++) acc = mfma_bf16(A[j].step(s, dq), __builtin_bit_cast(v8bf, B[j][s]), acc);
    }
  }
  combine_store(a, ti, c, rt * 16 + 4 * g, acc, a.g2 ? a.g2[ti.e] : 1.0f);
}

hipError_t launch_gemm1(int wfmt, const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  const dim3 grid(a.N1 / 32, grid_tiles), block(256);
  if (wfmt == W_MXFP4) hipLaunchKernelGGL(k_gemm1_a8, grid, block, 0, s, a);
  else if (wfmt == W_NVFP4) hipLaunchKernelGGL(k_gemm1_a16<W_NVFP4>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_gemm1_a16<W_NF3>, grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gemm2(int wfmt, const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  const dim3 grid(a.K / 64, grid_tiles), block(256);
  if (wfmt == W_MXFP4) hipLaunchKernelGGL(k_gemm2_a8, grid, block, 0, s, a);
  else if (wfmt == W_NVFP4) hipLaunchKernelGGL(k_gemm2_a16<W_NVFP4>, grid, block, 0, s, a);
  else hipLaunchKernelGGL(k_gemm2_a16<W_NF3>, grid, block, 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ combine

// fp32 accumulator -> bf16, 8 values per thread.
__global__ __launch_bounds__(256) void k_cast(const float *acc, long n8, uint16_t *out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const v4f a = ((const v4f *)acc)[2 * i], b = ((const v4f *)acc)[2 * i + 1];
  uint4 o;
  o.x = pack_bf16x2(a[0], a[1]);
  o.y = pack_bf16x2(a[2], a[3]);
  o.z = pack_bf16x2(b[0], b[1]);
  o.w = pack_bf16x2(b[2], b[3]);
  ((uint4 *)out)[i] = o;
}

// out[t] = bf16(sum over valid slots j, in slot order, of rb[t*topk + j]); 8 columns per thread.
// All TK slot rows and their validity are requested before the first add (rows
// of invalid slots are in the buffer's range, just never written, and are
// masked), so each thread has one memory round trip instead of TK.  The route
// buffer is read once, by non-temporal loads that keep its dead lines from
// displacing other data in the caches (4096-token W4A8 prefill: this kernel
// 70.4 -> 61.3 us, and the next layer's route planner 29.5 -> 27.5 us).
template <int TK>
__global__ __launch_bounds__(256) void k_topk_sum(const uint16_t *rb, const int32_t *inv, int T, int K,
                                                  uint16_t *out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  const long per_row = K / 8;
  if (i >= (long)T * per_row) return;
  const long t = i / per_row, c8 = i % per_row;
  uint4 v[TK];
  int ok[TK];
#pragma unroll
  for (int j = 0; j < TK; j++) {
    const long r = t * TK + j;
    ok[j] = inv[r];
    const v4i q = __builtin_nontemporal_load((const v4i *)(rb + r * K + c8 * 8));
    v[j] = uint4{(uint32_t)q[0], (uint32_t)q[1], (uint32_t)q[2], (uint32_t)q[3]};
  }
  float s[8];
#pragma unroll
  for (int m = 0; m < 8; m++) s[m] = 0.f;
#pragma unroll
  for (int j = 0; j < TK; j++) {
    if (ok[j] < 0) continue;
    const uint32_t wv[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
    for (int m = 0; m < 4; m++) {
      s[2 * m] += bf16_to_f32(wv[m] & 0xFFFFu);
      s[2 * m + 1] += bf16_to_f32(wv[m] >> 16);
    }
  }
  uint4 o;
  o.x = pack_bf16x2(s[0], s[1]);
  o.y = pack_bf16x2(s[2], s[3]);
  o.z = pack_bf16x2(s[4], s[5]);
  o.w = pack_bf16x2(s[6], s[7]);
  *(uint4 *)(out + t * K + c8 * 8) = o;
}

template <int TK>
static void launch_topk_sum(dim3 grid, dim3 block, hipStream_t s, const uint16_t *rb, const int32_t *inv, int T, int K,
                            uint16_t *out) {
  hipLaunchKernelGGL(k_topk_sum<TK>, grid, block, 0, s, rb, inv, T, K, out);
}

hipError_t launch_finalize(int deterministic, const float *out_acc, const uint16_t *rb, const int32_t *inv, int T,
                           int K, int topk, uint16_t *out, hipStream_t s) {
  const long n8 = (long)T * K / 8;
  if (n8 == 0) return hipSuccess;
  const dim3 grid((unsigned)((n8 + 255) / 256)), block(256);
  if (deterministic) {
    typedef void (*Fn)(dim3, dim3, hipStream_t, const uint16_t *, const int32_t *, int, int, uint16_t *);
    static const Fn fns[16] = {launch_topk_sum<1>,  launch_topk_sum<2>,  launch_topk_sum<3>,  launch_topk_sum<4>,
                               launch_topk_sum<5>,  launch_topk_sum<6>,  launch_topk_sum<7>,  launch_topk_sum<8>,
                               launch_topk_sum<9>,  launch_topk_sum<10>, launch_topk_sum<11>, launch_topk_sum<12>,
                               launch_topk_sum<13>, launch_topk_sum<14>, launch_topk_sum<15>, launch_topk_sum<16>};
    if (topk < 1 || topk > 16) return hipErrorInvalidValue;
    fns[topk - 1](grid, block, s, rb, inv, T, K, out);
  } else {
    hipLaunchKernelGGL(k_cast, grid, block, 0, s, out_acc, n8, out);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------ EP id remap
//
// One expert-parallel rank's view of the router output (sglang moe_b12x_next.py,
// ep_remap / ep_remap_reference): lid = id - offset; a slot with lid in
// [0, num_local) keeps lid and its weight; every other slot (another rank's
// expert, padding) gets weight 0 and the lowest valid lid of its row, else of
// the batch, else 0, so that every slot names an expert the batch already
// streams.  One workgroup: a batch-wide minimum (wave reductions, then LDS
// across the waves), then one thread per row.  Ids are compared in 64 bits so
// that id - offset cannot wrap.
constexpr int kRemapThreads = 1024;

__device__ __forceinline__ bool remap_ok(int32_t id, long offset, long num_local, long *lid) {
  *lid = (long)id - offset;
  return *lid >= 0 && *lid < num_local;
}

__global__ __launch_bounds__(kRemapThreads) void k_ep_remap(const int32_t *ids, const float *w, long T, int topk,
                                                            long offset, long num_local, int32_t *out_ids,
                                                            float *out_w) {
  __shared__ int s_min[kRemapThreads / 64];
  const long R = T * topk;
  int best = INT32_MAX;
  for (long r = threadIdx.x; r < R; r += kRemapThreads) {
    long lid;
    if (remap_ok(ids[r], offset, num_local, &lid)) best = min(best, (int)lid);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) best = min(best, __shfl_xor(best, d));
  if ((threadIdx.x & 63) == 0) s_min[threadIdx.x >> 6] = best;
  __syncthreads();
  best = INT32_MAX;
#pragma unroll
  for (int i = 0; i < kRemapThreads / 64; i++) best = min(best, s_min[i]);
  const int fb = best < num_local ? best : 0;   // no local slot in the batch: expert 0
  for (long t = threadIdx.x; t < T; t += kRemapThreads) {
    const int32_t *row = ids + t * topk;
    int row_min = INT32_MAX;
    for (int j = 0; j < topk; j++) {
      long lid;
      if (remap_ok(row[j], offset, num_local, &lid)) row_min = min(row_min, (int)lid);
    }
    const int fill = row_min < num_local ? row_min : fb;
    for (int j = 0; j < topk; j++) {
      long lid;
      const bool ok = remap_ok(row[j], offset, num_local, &lid);
      out_ids[t * topk + j] = ok ? (int32_t)lid : fill;
      out_w[t * topk + j] = ok ? w[t * topk + j] : 0.0f;
    }
  }
}

hipError_t launch_ep_remap(const int32_t *ids, const float *w, long T, int topk, long offset, long num_local,
                           int32_t *out_ids, float *out_w, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_ep_remap, dim3(1), dim3(kRemapThreads), 0, s, ids, w, T, topk, offset, num_local, out_ids,
                     out_w);
  return hipGetLastError();
}

// ------------------------------------------------------------ repacker

// Position, in the checkpoint layout, of byte `o` of the tile layout (both
// within one expert).  See the weight tile layout above; mxs: MXFP4 scales,
// whose k-tiles are in mx_soff's order (one byte a lane).
__device__ __forceinline__ long ckpt_offset(long o, int unit, int rows, int groups, int pair, int gate_up, int mxs) {
  const long rt_size = (long)16 * groups * unit;
  const long rt = o / rt_size;
  const long in_rt = o % rt_size;
  long kt;
  int lane, b;
  if (mxs) {
    // the inverse of mx_soff (unit 1)
    const long nkf = groups / 4, g4 = nkf & ~3L;
    b = 0;
    if (in_rt < g4 * 64) {
      kt = 4 * (in_rt / 256) + (in_rt & 3);
      lane = (int)((in_rt & 255) >> 2);
    } else if (in_rt < nkf * 64) {
      const long r = nkf & 3, x = in_rt - g4 * 64;
      kt = g4 + x % r;
      lane = (int)(x / r);
    } else {
      kt = nkf;
      lane = (int)(in_rt - nkf * 64);
    }
  } else {
    kt = in_rt / (64L * unit);
    const long rem = in_rt % (64L * unit);
    lane = (int)(rem / unit);
    b = (int)(rem % unit);
  }
  const int r = lane & 15, q = lane >> 4;
  long row;
  if (pair) {
    const long j = rt >> 1;
    const int half = (int)(rt & 1);  // 0 = up, 1 = gate
    const long half_rows = rows / 2;
    const long start = (half == 0) == (gate_up == 0) ? 0 : half_rows;
    row = start + 16 * j + r;
  } else {
    row = 16 * rt + r;
  }
  return row * ((long)groups * unit) + (kt * 4 + q) * unit + b;
}

template <typename Word>
__global__ __launch_bounds__(256) void k_permute(const uint8_t *tmp, uint8_t *dst, long total_words, long exp_bytes,
                                                 int unit, int rows, int groups, int pair, int gate_up,
                                                 int to_tiles, int mxs) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total_words) return;
  const long o = i * (long)sizeof(Word);
  const long e = o / exp_bytes, in_e = o % exp_bytes;
  const long ck = e * exp_bytes + ckpt_offset(in_e, unit, rows, groups, pair, gate_up, mxs);
  if (to_tiles) *(Word *)(dst + o) = *(const Word *)(tmp + ck);
  else *(Word *)(dst + ck) = *(const Word *)(tmp + o);
}

// NF3 codes between the packed form (code e of a 12-byte unit at bit 3e of its
// 96 bits, little endian) and the kernels' sign / magnitude-index form (see
// nf3_step_rc).  Both hold the same 96 bits of information per unit; the
// rewrite is per unit, so it commutes with the tile permutation.
__global__ __launch_bounds__(256) void k_nf3_recode(uint32_t *w, long units, int to_kernel) {
  const long u = (long)blockIdx.x * 256 + threadIdx.x;
  if (u >= units) return;
  uint32_t *p = w + 3 * u;
  const uint32_t a0 = p[0], a1 = p[1], a2 = p[2];
  uint32_t b0 = 0, b1 = 0, b2 = 0;
  if (to_kernel) {
#pragma unroll
    for (int e = 0; e < 32; e++) {
      const int bit = 3 * e;
      uint32_t c;
      if (bit + 3 <= 32) c = (a0 >> bit) & 7u;
      else if (bit < 32) c = ((a0 >> bit) | (a1 << (32 - bit))) & 7u;
      else if (bit + 3 <= 64) c = (a1 >> (bit - 32)) & 7u;
      else if (bit < 64) c = ((a1 >> (bit - 32)) | (a2 << (64 - bit))) & 7u;
      else c = (a2 >> (bit - 64)) & 7u;
      const uint32_t neg = c < 4u ? 1u : 0u, idx = c < 4u ? 3u - c : c - 4u;
      const int s = e >> 3, m = (e >> 1) & 3, h = e & 1;
      const uint32_t ib = idx << (8 * (s & 1) + 2 * m + 16 * h);
      if (s < 2) b0 |= ib;
      else b1 |= ib;
      b2 |= neg << (15 - (4 * s + m) + 16 * h);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; e++) {
      const int s = e >> 3, m = (e >> 1) & 3, h = e & 1;
      const uint32_t idx = ((s < 2 ? a0 : a1) >> (8 * (s & 1) + 2 * m + 16 * h)) & 3u;
      const uint32_t neg = (a2 >> (15 - (4 * s + m) + 16 * h)) & 1u;
      const uint32_t c = neg ? 3u - idx : idx + 4u;
      const int bit = 3 * e;
      if (bit < 32) b0 |= c << bit;
      if (bit + 3 > 32 && bit < 64) b1 |= bit < 32 ? c >> (32 - bit) : c << (bit - 32);
      if (bit + 3 > 64) b2 |= bit < 64 ? c >> (64 - bit) : c << (bit - 64);
    }
  }
  p[0] = b0;
  p[1] = b1;
  p[2] = b2;
}

hipError_t launch_nf3_recode(uint8_t *w, long units, int to_kernel, hipStream_t s) {
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_nf3_recode, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, s, (uint32_t *)w, units,
                     to_kernel);
  return hipGetLastError();
}

hipError_t launch_permute(const uint8_t *tmp, uint8_t *dst, long ne, int unit, int rows, int groups, int pair,
                          int gate_up, int to_tiles, int mxs, hipStream_t s) {
  const long exp_bytes = (long)rows * groups * unit;
  const long bytes = ne * exp_bytes;
  if (bytes == 0) return hipSuccess;
  if (unit % 4 == 0) {
    const long words = bytes / 4;
    hipLaunchKernelGGL(k_permute<uint32_t>, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s, tmp, dst, words,
                       exp_bytes, unit, rows, groups, pair, gate_up, to_tiles, mxs);
  } else {
    hipLaunchKernelGGL(k_permute<uint8_t>, dim3((unsigned)((bytes + 255) / 256)), dim3(256), 0, s, tmp, dst, bytes,
                       exp_bytes, unit, rows, groups, pair, gate_up, to_tiles, mxs);
  }
  return hipGetLastError();
}

}  // namespace moe
