// Prefill-size W4A8 GEMMs: tiles of 64 routes of one expert, operands streamed
// into an LDS ring by direct global-to-LDS loads and shared by a 2 x 2 grid of
// waves.
//
// One ring stage holds one 128-column k-tile: 8 weight row tiles (8 x 1 KB of
// FP4 in MFMA lane order), the 64 routes' MXFP8 activation slices (8 blocks of
// 8 rows x 128 bytes, 16-byte chunks XOR-swizzled so that MFMA operand reads
// spread over the LDS banks) and the scales of both (As: 8 x 64 bytes, Bs:
// 64 x 4 bytes).  Every wave issues the same five loads per stage (two weight
// tiles, two activation blocks, one 256-byte scale chunk), so "all but the
// newest n stages have landed" is one s_waitcnt vmcnt(5 n) per wave followed
// by a barrier.  Each wave reads its operands of k-tile kt+1 from LDS while its
// MFMAs of k-tile kt run, and the ring keeps its other stages in flight.
//
// Wave (wr, wc) owns row tiles 4 wr .. +3 and routes 32 wc .. +31: 8 block-
// scaled MFMAs per k-tile.
//
// Blocks are numbered XCD-major: the hardware hands workgroup b to XCD b % 8,
// so logical work item (b % 8) * per + b / 8 puts a contiguous run of
// (tile, column block) items on each XCD, in order.  The up/gate GEMM orders
// items column-block-major: all tiles of a hot expert then run at once on one
// XCD against the same weight slab, which is read once, while the activations
// (tens of MB, re-read once per column block) stay in the last-level cache.
// The down GEMM orders them tile-major: the 56-odd column blocks of a tile
// share its activation rows in L2, and one expert's w2 (2 MB) stays in L2
// across its consecutive tiles.
//
//   k_pf_gemm1_a8  items (tile, 64-column intermediate block): up/gate GEMMs over
//                  K, clamped SwiGLU and MXFP8 requantisation of 64 intermediate
//                  columns of 64 routes.
//   k_pf_gemm2_a8  items (tile, 128-column output block): down GEMM over N with
//                  the activations as the MFMA's A operand, so each lane holds
//                  16 consecutive output columns' worth of one route per
//                  instruction; combine straight from the accumulators (fp32
//                  atomics, or bf16 route-buffer rows).
#include "moe_device.h"

namespace moe {

constexpr int kPfRowTiles = 8;   // weight row tiles per block
constexpr int kPfStages1 = 4;    // LDS ring depth (k-tiles), up/gate GEMM
constexpr int kPfStages2 = 3;    // down GEMM: short k-loops, more blocks per CU
constexpr int kPfLoadsPerStage = 5;

struct PfStage {
  uint8_t A[kPfRowTiles][1024];   // weight row tiles, MFMA lane order
  uint8_t B[8][1024];             // activation rows 8b .. 8b+7 of block b, swizzled 16-byte chunks
  uint8_t S[1024];                // As [8][64] | Bs [64][4] | spare
};

template <int ST>
struct __attribute__((aligned(16))) PfLds {
  PfStage st[ST];
};


// Wait until at most `stages` ring stages issued by this wave are in flight.
__device__ __forceinline__ void wait_stages(int stages) {
  if (stages >= 3) wait_vm<3 * kPfLoadsPerStage>();
  else if (stages == 2) wait_vm<2 * kPfLoadsPerStage>();
  else if (stages == 1) wait_vm<kPfLoadsPerStage>();
  else wait_vm<0>();
}

// LDS chunk (0..63) of activation row r8 = row % 8, 16-byte part p, inside its block.
__device__ __forceinline__ int pf_slot(int r8, int p) { return r8 * 8 + (p ^ r8); }

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// One block's work item: tile of the tier's tile table and column block.
struct PfWork {
  int valid, e, p0, rows, sub;
};

__device__ __forceinline__ PfWork pf_work(const GemmArgs &a, int nsub, bool sub_major) {
  PfWork w;
  const int tbeg = a.tier_tiles[2 * a.tier], tend = a.tier_tiles[2 * a.tier + 1];
  const int items = (tend - tbeg) * nsub, per = (items + 7) >> 3;
  const int b = blockIdx.x, slot = b >> 3, item = (b & 7) * per + slot;
  w.valid = slot < per && item < items;
  if (!w.valid) return w;
  const int ntiles = tend - tbeg;
  const int t = sub_major ? item % ntiles : item / nsub;
  w.sub = sub_major ? item / ntiles : item - t * nsub;
  const int u = a.tile_u[tbeg + t];
  w.e = u - a.u_base;
  w.p0 = a.off[u] + a.tile_row0[tbeg + t];
  w.rows = min(a.tile_rows, a.off[u + 1] - w.p0);
  return w;
}

struct PfSrc {
  const uint8_t *wbase, *sbase;   // row tile rt, k-tile kt: wbase + rt * wstep + kt * 1024 (scales: 64 per k-tile)
  size_t wstep, sstep;
  const uint8_t *brow[2];         // this lane's activation rows of its two B blocks
  const uint8_t *bsrow;           // activation scale row of route (lane)
  int kbytes;                     // reduction length (bytes of one activation row)
};

// The five loads of wave w for k-tile kt into stage S.  Lanes whose data lies
// past the reduction length (a partial last k-tile) load from a valid address
// instead; the MFMA step zeroes those activation bytes and both scales there.
__device__ __forceinline__ void pf_issue(PfStage &S, const PfSrc &src, int kt, int w, int l) {
#pragma unroll
  for (int j = 0; j < 2; j++) {   // weight row tiles 2w + j
    const int rt = 2 * w + j;
    const bool in = (kt * 4 + (l >> 4)) * 32 < src.kbytes;
    dma16(src.wbase + rt * src.wstep + (in ? (size_t)kt * 1024 + l * 16 : 0), &S.A[rt][0]);
  }
#pragma unroll
  for (int j = 0; j < 2; j++) {   // activation blocks 2w + j: lane l -> row l / 8, its chunk slot l
    const int r8 = l >> 3, part = (l & 7) ^ r8, off = kt * 128 + part * 16;
    dma16(src.brow[j] + (off < src.kbytes ? off : 0), &S.B[2 * w + j][0]);
  }
  if (w < 2) {   // As row tiles 4w .. 4w+3: lane l -> row tile 4w + l / 16, dword l % 16
    const int rt = 4 * w + (l >> 4), d = l & 15;
    const bool in = (kt * 4 + (d >> 2)) * 32 < src.kbytes;
    dma4(src.sbase + rt * src.sstep + (in ? (size_t)kt * 64 + 4 * d : 0), &S.S[256 * w]);
  } else {       // Bs (wave 3 fills the spare slot to keep the per-wave load count equal)
    dma4(src.bsrow + 4 * kt, &S.S[w == 2 ? 512 : 768]);
  }
}

// One wave's operands of a landed stage.  The LDS reads are issued by asm the
// compiler cannot see into: seen, each would make it wait for every direct-to-
// LDS load in flight (it cannot tell ring stages apart), emptying the ring at
// every k-tile.  pf_read issues them; pf_wait waits for them and, taking the
// registers as operands, keeps every use of them after the wait.
struct PfOps {
  v4i a[4];      // weight row tiles 4 wr + q
  v4i b[4];      // activation chunks: [cb] = columns 16 g .. of route block cb, [2 + cb] = columns 64 + 16 g ..
  int sa[4], sb[2];
};

__device__ __forceinline__ void pf_read(PfOps &o, const PfStage &S, int wr, int wc, int l) {
  const int c = l & 15, g = l >> 4, r8 = c & 7;
  const uint8_t *bblk = &S.B[4 * wc + (c >> 3)][0];
  const uint32_t va = lds_addr(&S.A[4 * wr][l * 16]), vb0 = lds_addr(bblk + pf_slot(r8, g) * 16),
                 vb1 = lds_addr(bblk + pf_slot(r8, 4 + g) * 16), vsa = lds_addr(&S.S[4 * wr * 64 + l]),
                 vsb = lds_addr(&S.S[512 + (32 * wc + c) * 4 + g]);
  asm volatile(
      "ds_read_b128 %0, %14\n"
      "ds_read_b128 %1, %14 offset:1024\n"
      "ds_read_b128 %2, %14 offset:2048\n"
      "ds_read_b128 %3, %14 offset:3072\n"
      "ds_read_b128 %4, %15\n"
      "ds_read_b128 %5, %15 offset:2048\n"
      "ds_read_b128 %6, %16\n"
      "ds_read_b128 %7, %16 offset:2048\n"
      "ds_read_u8 %8, %17\n"
      "ds_read_u8 %9, %17 offset:64\n"
      "ds_read_u8 %10, %17 offset:128\n"
      "ds_read_u8 %11, %17 offset:192\n"
      "ds_read_u8 %12, %18\n"
      "ds_read_u8 %13, %18 offset:64"
      : "=&v"(o.a[0]), "=&v"(o.a[1]), "=&v"(o.a[2]), "=&v"(o.a[3]), "=&v"(o.b[0]), "=&v"(o.b[1]), "=&v"(o.b[2]),
        "=&v"(o.b[3]), "=&v"(o.sa[0]), "=&v"(o.sa[1]), "=&v"(o.sa[2]), "=&v"(o.sa[3]), "=&v"(o.sb[0]), "=&v"(o.sb[1])
      : "v"(va), "v"(vb0), "v"(vb1), "v"(vsa), "v"(vsb)
      : "memory");
}

__device__ __forceinline__ void pf_wait(PfOps &o) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(o.a[0]), "+v"(o.a[1]), "+v"(o.a[2]), "+v"(o.a[3]), "+v"(o.b[0]), "+v"(o.b[1]), "+v"(o.b[2]),
                 "+v"(o.b[3]), "+v"(o.sa[0]), "+v"(o.sa[1]), "+v"(o.sa[2]), "+v"(o.sa[3]), "+v"(o.sb[0]), "+v"(o.sb[1])
               :
               : "memory");
}

// 8 MFMAs of one k-tile.  Past the reduction length (a partial last k-tile)
// the activation bytes are zeroed and both scales set to 2^-127, so the
// products there are exact zeros whatever the stage held.  SWAP: activations
// as the A operand (accumulator lane = output column, elements = 4 routes).
template <bool SWAP>
__device__ __forceinline__ void pf_mma(const PfOps &o, int kt, int kbytes, int l, v4f (*acc)[2]) {
  const int g = l >> 4;
  const bool in0 = kt * 128 + 16 * g < kbytes, in1 = kt * 128 + 64 + 16 * g < kbytes;
  const bool gin = (kt * 4 + g) * 32 < kbytes;   // 32-column group g of this k-tile exists
  v8i bop[2];
#pragma unroll
  for (int cb = 0; cb < 2; cb++) {
    const v4i b0 = in0 ? o.b[cb] : v4i{0, 0, 0, 0};
    const v4i b1 = in1 ? o.b[2 + cb] : v4i{0, 0, 0, 0};
    bop[cb] = v8i{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  }
#pragma unroll
  for (int q = 0; q < 4; q++)
#pragma unroll
    for (int cb = 0; cb < 2; cb++) {
      const int sa = gin ? o.sa[q] : 0, sb = gin ? o.sb[cb] : 0;
      if (SWAP)
        acc[q][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bop[cb], fp4_operand(o.a[q]), acc[q][cb], 0, 4,
                                                                      0, sb, 0, sa);
      else
        acc[q][cb] = mfma_fp4_fp8(o.a[q], bop[cb], acc[q][cb], sa, sb);
    }
}

// One k-tile: operands of kt are in `cur` (reads issued one k-tile earlier).
template <bool SWAP, int ST>
__device__ __forceinline__ void pf_step(PfLds<ST> &L, const PfSrc &src, int kt, int nkt, PfOps &cur, PfOps &nxt,
                                        v4f (*acc)[2]) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, wr = w >> 1, wc = w & 1;
  pf_wait(cur);
  wait_stages(min(ST - 2, nkt - 2 - kt));   // stage kt + 1 has landed
  __builtin_amdgcn_s_barrier();                   // ... for every wave, and no wave reads stage kt any more
  if (kt + ST < nkt) pf_issue(L.st[kt % ST], src, kt + ST, w, l);
  if (kt + 1 < nkt) pf_read(nxt, L.st[(kt + 1) % ST], wr, wc, l);
  pf_mma<SWAP>(cur, kt, src.kbytes, l, acc);
}

// The k-loop of both GEMMs.
template <bool SWAP, int ST>
__device__ __forceinline__ void pf_kloop(PfLds<ST> &L, const PfSrc &src, v4f (*acc)[2]) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, wr = w >> 1, wc = w & 1;
  const int nkt = (src.kbytes + 127) / 128;
#pragma unroll
  for (int s = 0; s < ST; s++)
    if (s < nkt) pf_issue(L.st[s], src, s, w, l);
  wait_stages(min(ST - 1, nkt - 1));   // stage 0 has landed
  __builtin_amdgcn_s_barrier();
  PfOps r0, r1;
  pf_read(r0, L.st[0], wr, wc, l);
  for (int kt = 0; kt + 1 < nkt; kt += 2) {
    pf_step<SWAP, ST>(L, src, kt, nkt, r0, r1, acc);
    pf_step<SWAP, ST>(L, src, kt + 1, nkt, r1, r0, acc);
  }
  if (nkt & 1) pf_step<SWAP, ST>(L, src, nkt - 1, nkt, r0, r1, acc);
}

__device__ __forceinline__ void zero_acc(v4f (*acc)[2]) {
#pragma unroll
  for (int q = 0; q < 4; q++)
#pragma unroll
    for (int cb = 0; cb < 2; cb++) acc[q][cb] = v4f{0.f, 0.f, 0.f, 0.f};
}

// ---------------------------------------------------------------- GEMM1
__global__ __launch_bounds__(256) void k_pf_gemm1_a8(GemmArgs a) {
  __shared__ PfLds<kPfStages1> L;
  const int K = a.K, N = a.N;
  const PfWork wk = pf_work(a, N / 64, true);
  if (!wk.valid) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4, wr = w >> 1, wc = w & 1;
  const int hb = wk.sub;
  PfSrc src;
  src.wstep = (size_t)16 * (K / 2);
  src.sstep = (size_t)16 * (K / 32);
  src.wbase = a.w13 + (size_t)wk.e * (2 * N) * (K / 2) + (size_t)(8 * hb) * src.wstep;
  src.sbase = a.s13 + (size_t)wk.e * (2 * N) * (K / 32) + (size_t)(8 * hb) * src.sstep;
  src.kbytes = K;
  // rows past the tile read route p0's token; their results are never stored
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int row = 8 * (2 * w + j) + (l >> 3);
    src.brow[j] = a.xq + (size_t)(a.perm[wk.p0 + (row < wk.rows ? row : 0)] / a.topk) * K;
  }
  src.bsrow = a.xs + (size_t)(a.perm[wk.p0 + (l < wk.rows ? l : 0)] / a.topk) * (K / 32);
  v4f acc[4][2];
  zero_acc(acc);
  pf_kloop<false, kPfStages1>(L, src, acc);
  // epilogue: row tiles 4wr + {0,1,2,3} = up/gate of intermediate blocks 4hb + 2wr + {0,1}
  const int hss = hs_stride(N);
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
    if (row < wk.rows) {
      const size_t p = (size_t)(wk.p0 + row);
#pragma unroll
      for (int s = 0; s < 2; s++)
        *(uint32_t *)(a.hq + p * N + 64 * hb + 32 * wr + 16 * s + 4 * g) =
            e4m3x4(h[s * 4], h[s * 4 + 1], h[s * 4 + 2], h[s * 4 + 3], inv);
      if (g == 0) a.hs[p * hss + 2 * hb + wr] = (uint8_t)sbyte;
    }
  }
}

// ---------------------------------------------------------------- GEMM2
__global__ __launch_bounds__(256) void k_pf_gemm2_a8(GemmArgs a) {
  __shared__ PfLds<kPfStages2> L;
  __shared__ int s_r[kPfTileRows];
  __shared__ float s_w[kPfTileRows];
  const int K = a.K, N = a.N;
  const PfWork wk = pf_work(a, K / 128, false);
  if (!wk.valid) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4, wr = w >> 1, wc = w & 1;
  const int ob = wk.sub;   // output columns 128 ob .. +127 = w2 row tiles 8 ob .. +7
  PfSrc src;
  src.wstep = (size_t)16 * (N / 2);
  src.sstep = (size_t)16 * (N / 32);
  src.wbase = a.w2 + (size_t)wk.e * K * (N / 2) + (size_t)(8 * ob) * src.wstep;
  src.sbase = a.s2 + (size_t)wk.e * K * (N / 32) + (size_t)(8 * ob) * src.sstep;
  src.kbytes = N;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int row = 8 * (2 * w + j) + (l >> 3);
    src.brow[j] = a.hq + (size_t)(wk.p0 + (row < wk.rows ? row : 0)) * N;
  }
  src.bsrow = a.hs + (size_t)(wk.p0 + (l < wk.rows ? l : 0)) * hs_stride(N);
  if (tid < wk.rows) {
    const int r = a.perm[wk.p0 + tid];
    s_r[tid] = r;
    s_w[tid] = a.topk_w[r];
  }
  v4f acc[4][2];
  zero_acc(acc);
  pf_kloop<true, kPfStages2>(L, src, acc);
  __syncthreads();   // s_r / s_w visible
  // acc[q][cb][i]: route 32 wc + 16 cb + 4 g + i, output column 128 ob + 64 wr + 16 q + c
  const size_t col = (size_t)128 * ob + 64 * wr + c;
  if (a.deterministic) {
    // bf16 route-buffer rows: lanes c, c ^ 1 swap one value so each writes two adjacent columns of one route
    const bool odd = c & 1;
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
      for (int ip = 0; ip < 2; ip++) {
        const int row = 32 * wc + 16 * cb + 4 * g + 2 * ip + (odd ? 1 : 0);
        const bool ok = row < wk.rows;
        const int r = ok ? s_r[row] : 0;
        const float wgt = ok ? s_w[row] : 0.f;
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const float mine = acc[q][cb][2 * ip + (odd ? 1 : 0)], give = acc[q][cb][2 * ip + (odd ? 0 : 1)];
          const float got = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(give), 0xB1, 0xF, 0xF, false));
          const float lo = odd ? got : mine, hi = odd ? mine : got;
          if (ok) *(uint32_t *)(a.rb + (size_t)r * K + col + 16 * q - (odd ? 1 : 0)) = pack_bf16x2(wgt * lo, wgt * hi);
        }
      }
  } else {
    // fp32 atomics: per instruction 4 routes x 16 consecutive columns
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = 32 * wc + 16 * cb + 4 * g + i;
        if (row < wk.rows) {
          float *dst = a.out_acc + (size_t)(s_r[row] / a.topk) * K + col;
          const float wgt = s_w[row];
#pragma unroll
          for (int q = 0; q < 4; q++) atomicAdd(dst + 16 * q, wgt * acc[q][cb][i]);
        }
      }
  }
}

static int pf_grid(int grid_tiles, int nsub) { return (grid_tiles * nsub + 7) / 8 * 8; }

hipError_t launch_pf_gemm1(const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pf_gemm1_a8, dim3(pf_grid(grid_tiles, a.N / 64)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pf_gemm2(const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pf_gemm2_a8, dim3(pf_grid(grid_tiles, a.K / 128)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
