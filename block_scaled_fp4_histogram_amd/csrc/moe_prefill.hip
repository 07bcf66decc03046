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

constexpr int kPfRT = 16;        // W4A8: weight row tiles per block (256 weight rows)
constexpr int kPfQ = 8;          // W4A8: row tiles per wave
constexpr int kPfStages = 3;     // W4A8: LDS ring depth (k-tiles)
constexpr int kPfLoadsPerStage = 8;

struct PfStage {
  uint8_t A[kPfRT][1024];         // weight row tiles, MFMA lane order
  uint8_t B[8][1024];             // activation rows 8b .. 8b+7 of block b, swizzled 16-byte chunks
  uint8_t S[2048];                // As [16][64] | Bs [64][4] | 3 spare 256-byte slots
};

struct __attribute__((aligned(16))) PfLds {
  PfStage st[kPfStages];
};

// Wait until at most `stages` ring stages issued by this wave are in flight.
__device__ __forceinline__ void wait_stages(int stages) {
  if (stages >= 2) wait_vm<2 * kPfLoadsPerStage>();
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
  int nrt;                        // row tiles of this block that exist (8 or 16); the rest repeat the last one
  const uint8_t *brow[2];         // this lane's activation rows of its two B blocks
  const uint8_t *bsrow;           // activation scale row of route (lane)
  int kbytes;                     // reduction length (bytes of one activation row)
};

// The eight loads of wave w for k-tile kt into stage S: weight row tiles 4w ..
// 4w+3, activation blocks 2w, 2w+1, the scales of row tiles 4w .. 4w+3, and the
// activation scales (wave 0; waves 1-3 fill spare slots to keep the per-wave
// load count equal).  Lanes whose data lies past the reduction length (a
// partial last k-tile) load from a valid address instead; the MFMA step zeroes
// those activation bytes and both scales there.
template <bool FULL>
__device__ __forceinline__ void pf_issue(PfStage &S, const PfSrc &src, int kt, int w, int l) {
  const bool in = FULL || (kt * 4 + (l >> 4)) * 32 < src.kbytes;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int rt = 4 * w + j, rs = min(rt, src.nrt - 1);
    dma16(src.wbase + rs * src.wstep + (in ? (size_t)kt * 1024 + l * 16 : 0), &S.A[rt][0]);
  }
#pragma unroll
  for (int j = 0; j < 2; j++) {   // activation blocks 2w + j: lane l -> row l / 8, its chunk slot l
    const int r8 = l >> 3, part = (l & 7) ^ r8, off = kt * 128 + part * 16;
    dma16(src.brow[j] + (FULL || off < src.kbytes ? off : 0), &S.B[2 * w + j][0]);
  }
  {   // As row tiles 4w .. 4w+3: lane l -> row tile 4w + l / 16, dword l % 16
    const int rs = min(4 * w + (l >> 4), src.nrt - 1), d = l & 15;
    const bool ins = FULL || (kt * 4 + (d >> 2)) * 32 < src.kbytes;
    dma4(src.sbase + rs * src.sstep + (ins ? (size_t)kt * 64 + 4 * d : 0), &S.S[256 * w]);
  }
  dma4(src.bsrow + 4 * kt, &S.S[w == 0 ? 1024 : 1024 + 256 * w]);
}

// One wave's operands of a landed stage.  The LDS reads are issued by asm the
// compiler cannot see into: seen, each would make it wait for every direct-to-
// LDS load in flight (it cannot tell ring stages apart), emptying the ring at
// every k-tile.  pf_read issues them and waits for them in one statement.
struct PfOps {
  v4i a[kPfQ];   // weight row tiles 8 wr + q
  v4i b[4];      // activation chunks: [cb] = columns 16 g .. of route block cb, [2 + cb] = columns 64 + 16 g ..
  int sa[kPfQ], sb[2];
};

__device__ __forceinline__ void pf_read(PfOps &o, const PfStage &S, int wr, int wc, int l) {
  const int c = l & 15, g = l >> 4, r8 = c & 7;
  const uint8_t *bblk = &S.B[4 * wc + (c >> 3)][0];
  const uint32_t va = lds_addr(&S.A[kPfQ * wr][l * 16]), vb0 = lds_addr(bblk + pf_slot(r8, g) * 16),
                 vb1 = lds_addr(bblk + pf_slot(r8, 4 + g) * 16), vsa = lds_addr(&S.S[kPfQ * wr * 64 + l]),
                 vsb = lds_addr(&S.S[1024 + (32 * wc + c) * 4 + g]);
  // the wait is part of the same statement: between an LDS read and its wait
  // the compiler could copy the register it loads (it cannot know the value
  // is still in flight)
  asm volatile(
      "ds_read_b128 %8, %23\n"
      "ds_read_b128 %9, %23 offset:2048\n"
      "ds_read_b128 %10, %24\n"
      "ds_read_b128 %11, %24 offset:2048\n"
      "ds_read_u8 %20, %26\n"
      "ds_read_u8 %21, %26 offset:64\n"
      "ds_read_u8 %12, %25\n"
      "ds_read_u8 %13, %25 offset:64\n"
      "ds_read_u8 %14, %25 offset:128\n"
      "ds_read_u8 %15, %25 offset:192\n"
      "ds_read_u8 %16, %25 offset:256\n"
      "ds_read_u8 %17, %25 offset:320\n"
      "ds_read_u8 %18, %25 offset:384\n"
      "ds_read_u8 %19, %25 offset:448\n"
      "ds_read_b128 %0, %22\n"
      "ds_read_b128 %1, %22 offset:1024\n"
      "ds_read_b128 %2, %22 offset:2048\n"
      "ds_read_b128 %3, %22 offset:3072\n"
      "ds_read_b128 %4, %22 offset:4096\n"
      "ds_read_b128 %5, %22 offset:5120\n"
      "ds_read_b128 %6, %22 offset:6144\n"
      "ds_read_b128 %7, %22 offset:7168\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o.a[0]), "=&v"(o.a[1]), "=&v"(o.a[2]), "=&v"(o.a[3]), "=&v"(o.a[4]), "=&v"(o.a[5]), "=&v"(o.a[6]),
        "=&v"(o.a[7]), "=&v"(o.b[0]), "=&v"(o.b[1]), "=&v"(o.b[2]), "=&v"(o.b[3]), "=&v"(o.sa[0]), "=&v"(o.sa[1]),
        "=&v"(o.sa[2]), "=&v"(o.sa[3]), "=&v"(o.sa[4]), "=&v"(o.sa[5]), "=&v"(o.sa[6]), "=&v"(o.sa[7]),
        "=&v"(o.sb[0]), "=&v"(o.sb[1])
      : "v"(va), "v"(vb0), "v"(vb1), "v"(vsa), "v"(vsb)
      : "memory");
}

// 16 MFMAs of one k-tile, two per weight row tile.  Past the reduction length (a partial last k-tile; FULL: none) the activation
// bytes are zeroed and both scales set to 2^-127, so the products there are
// exact zeros whatever the stage held.  SWAP: activations as the A operand
// (accumulator lane = output column, elements = 4 routes).
template <bool SWAP, bool FULL, int Q>
__device__ __forceinline__ void pf_mma_q(const PfOps &o, bool gin, const v8i (&bop)[2], v4f (*acc)[2]) {
#pragma unroll
  for (int cb = 0; cb < 2; cb++) {
    const int sa = (FULL || gin) ? o.sa[Q] : 0, sb = (FULL || gin) ? o.sb[cb] : 0;
    if (SWAP)
      acc[Q][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bop[cb], fp4_operand(o.a[Q]), acc[Q][cb], 0, 4, 0,
                                                                    sb, 0, sa);
    else
      acc[Q][cb] = mfma_fp4_fp8(o.a[Q], bop[cb], acc[Q][cb], sa, sb);
  }
}

template <bool SWAP, bool FULL>
__device__ __forceinline__ void pf_mma(const PfOps &o, int kt, int kbytes, int l, v4f (*acc)[2]) {
  const int g = l >> 4;
  const bool in0 = FULL || kt * 128 + 16 * g < kbytes, in1 = FULL || kt * 128 + 64 + 16 * g < kbytes;
  const bool gin = FULL || (kt * 4 + g) * 32 < kbytes;   // 32-column group g of this k-tile exists
  v8i bop[2];
#pragma unroll
  for (int cb = 0; cb < 2; cb++) {
    const v4i b0 = in0 ? o.b[cb] : v4i{0, 0, 0, 0};
    const v4i b1 = in1 ? o.b[2 + cb] : v4i{0, 0, 0, 0};
    bop[cb] = v8i{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  }
  pf_mma_q<SWAP, FULL, 0>(o, gin, bop, acc);
  pf_mma_q<SWAP, FULL, 1>(o, gin, bop, acc);
  pf_mma_q<SWAP, FULL, 2>(o, gin, bop, acc);
  pf_mma_q<SWAP, FULL, 3>(o, gin, bop, acc);
  pf_mma_q<SWAP, FULL, 4>(o, gin, bop, acc);
  pf_mma_q<SWAP, FULL, 5>(o, gin, bop, acc);
  pf_mma_q<SWAP, FULL, 6>(o, gin, bop, acc);
  pf_mma_q<SWAP, FULL, 7>(o, gin, bop, acc);
}

// One k-tile: wait until stage kt has landed for every wave (every wave is
// then also done with stage kt - 1), refill stage kt - 1's slot with k-tile
// kt + kPfStages - 1, read this wave's operands of stage kt, multiply.
template <bool SWAP>
__device__ __forceinline__ void pf_step(PfLds &L, const PfSrc &src, int kt, int nkt, v4f (*acc)[2]) {
  constexpr int ST = kPfStages;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, wr = w >> 1, wc = w & 1;
  wait_stages(min(ST - 2, nkt - 1 - kt));   // stage kt has landed
  __builtin_amdgcn_s_barrier();
  const int kn = kt + ST - 1;
  if (kn < nkt) {
    if ((kn + 1) * 128 <= src.kbytes) pf_issue<true>(L.st[kn % ST], src, kn, w, l);
    else pf_issue<false>(L.st[kn % ST], src, kn, w, l);
  }
  PfOps o;
  pf_read(o, L.st[kt % ST], wr, wc, l);
  if ((kt + 1) * 128 <= src.kbytes) pf_mma<SWAP, true>(o, kt, src.kbytes, l, acc);
  else pf_mma<SWAP, false>(o, kt, src.kbytes, l, acc);
}

// The k-loop of both GEMMs.
template <bool SWAP>
__device__ __forceinline__ void pf_kloop(PfLds &L, const PfSrc &src, v4f (*acc)[2]) {
  constexpr int ST = kPfStages;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int nkt = (src.kbytes + 127) / 128;
#pragma unroll
  for (int s = 0; s < ST - 1; s++)
    if (s < nkt) pf_issue<false>(L.st[s], src, s, w, l);
  for (int kt = 0; kt < nkt; kt++) pf_step<SWAP>(L, src, kt, nkt, acc);
}

template <int Q>
__device__ __forceinline__ void zero_acc(v4f (*acc)[2]) {
#pragma unroll
  for (int q = 0; q < Q; q++)
#pragma unroll
    for (int cb = 0; cb < 2; cb++) acc[q][cb] = v4f{0.f, 0.f, 0.f, 0.f};
}

// Down-GEMM combine from accumulators in the swapped layout: acc[q][cb][i] is
// route 32 wc + 16 cb + 4 g + i (tile row; cb < CB), output column col + 16 q; s_r, s_w
// hold each tile row's route and its router weight (times the expert's global
// scale).  Deterministic mode writes bf16 route-buffer rows (lanes c, c ^ 1
// swap one value so each stores two adjacent columns of one route); atomic mode
// adds fp32 into the token accumulator, 4 routes x 16 consecutive columns per
// instruction.
template <int Q, int CB>
__device__ __forceinline__ void pf_combine(const GemmArgs &a, const PfWork &wk, v4f (*acc)[CB], const int *s_r,
                                           const float *s_w, size_t col, int wc, int c, int g) {
  const int K = a.K;
  if (a.deterministic) {
    const bool odd = c & 1;
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int ip = 0; ip < 2; ip++) {
        const int row = 32 * wc + 16 * cb + 4 * g + 2 * ip + (odd ? 1 : 0);
        const bool ok = row < wk.rows;
        const int r = ok ? s_r[row] : 0;
        const float wgt = ok ? s_w[row] : 0.f;
#pragma unroll
        for (int q = 0; q < Q; q++) {
          const float mine = acc[q][cb][2 * ip + (odd ? 1 : 0)], give = acc[q][cb][2 * ip + (odd ? 0 : 1)];
          const float got = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(give), 0xB1, 0xF, 0xF, false));
          const float lo = odd ? got : mine, hi = odd ? mine : got;
          if (ok) *(uint32_t *)(a.rb + (size_t)r * K + col + 16 * q - (odd ? 1 : 0)) = pack_bf16x2(wgt * lo, wgt * hi);
        }
      }
  } else {
#pragma unroll
    for (int cb = 0; cb < CB; cb++)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int row = 32 * wc + 16 * cb + 4 * g + i;
        if (row < wk.rows) {
          float *dst = a.out_acc + (size_t)(s_r[row] / a.topk) * K + col;
          const float wgt = s_w[row];
#pragma unroll
          for (int q = 0; q < Q; q++) atomicAdd(dst + 16 * q, wgt * acc[q][cb][i]);
        }
      }
  }
}

// ---------------------------------------------------------------- GEMM1
// Block: 16 row tiles of w13 = up and gate of 128 intermediate columns (the
// last block of an N % 128 == 64 layer holds 8).
__global__ __launch_bounds__(256) void k_pf_gemm1_a8(GemmArgs a) {
  __shared__ PfLds L;
  const int K = a.K, N = a.N;
  const PfWork wk = pf_work(a, (N + 127) / 128, true);
  if (!wk.valid) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4, wr = w >> 1, wc = w & 1;
  const int hb = wk.sub;
  PfSrc src;
  src.wstep = (size_t)16 * (K / 2);
  src.sstep = (size_t)16 * (K / 32);
  src.wbase = a.w13 + (size_t)wk.e * (2 * N) * (K / 2) + (size_t)(kPfRT * hb) * src.wstep;
  src.sbase = a.s13 + (size_t)wk.e * (2 * N) * (K / 32) + (size_t)(kPfRT * hb) * src.sstep;
  src.nrt = min(kPfRT, N / 8 - kPfRT * hb);
  src.kbytes = K;
  // rows past the tile read route p0's token; their results are never stored
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int row = 8 * (2 * w + j) + (l >> 3);
    src.brow[j] = a.xq + (size_t)(a.perm[wk.p0 + (row < wk.rows ? row : 0)] / a.topk) * K;
  }
  src.bsrow = a.xs + (size_t)(a.perm[wk.p0 + (l < wk.rows ? l : 0)] / a.topk) * (K / 32);
  v4f acc[kPfQ][2];
  zero_acc<kPfQ>(acc);
  pf_kloop<false>(L, src, acc);
  if (kPfQ * wr >= src.nrt) return;   // the missing half of a partial block
  // epilogue: row tiles 8 wr + q, q = 2 s + {0, 1}: up / gate of intermediate
  // columns 128 hb + 64 wr + 16 s .. +15; MXFP8 groups of two 16-column blocks
  const int hss = hs_stride(N);
#pragma unroll
  for (int cb = 0; cb < 2; cb++) {
    const int row = 32 * wc + 16 * cb + c;
#pragma unroll
    for (int pp = 0; pp < 2; pp++) {
      float h[8];
#pragma unroll
      for (int s = 0; s < 2; s++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int q = 2 * (2 * pp + s);
          h[s * 4 + i] = silu_clamped(acc[q + 1][cb][i], acc[q][cb][i], a.limit, a.has_limit);
        }
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(h[i]));
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      float inv;
      const uint32_t sbyte = mx_scale(amax, &inv);
      if (row < wk.rows) {
        const size_t p = (size_t)(wk.p0 + row);
        const size_t c0 = (size_t)128 * hb + 64 * wr + 32 * pp;
#pragma unroll
        for (int s = 0; s < 2; s++)
          *(uint32_t *)(a.hq + p * N + c0 + 16 * s + 4 * g) = e4m3x4(h[s * 4], h[s * 4 + 1], h[s * 4 + 2], h[s * 4 + 3], inv);
        if (g == 0) a.hs[p * hss + c0 / 32] = (uint8_t)sbyte;
      }
    }
  }
}

// ---------------------------------------------------------------- GEMM2
// Block: 16 row tiles of w2 = 256 output columns.
__global__ __launch_bounds__(256) void k_pf_gemm2_a8(GemmArgs a) {
  __shared__ PfLds L;
  __shared__ int s_r[kPfTileRows];
  __shared__ float s_w[kPfTileRows];
  const int K = a.K, N = a.N;
  const PfWork wk = pf_work(a, K / 256, false);
  if (!wk.valid) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4, wr = w >> 1, wc = w & 1;
  const int ob = wk.sub;
  PfSrc src;
  src.wstep = (size_t)16 * (N / 2);
  src.sstep = (size_t)16 * (N / 32);
  src.wbase = a.w2 + (size_t)wk.e * K * (N / 2) + (size_t)(kPfRT * ob) * src.wstep;
  src.sbase = a.s2 + (size_t)wk.e * K * (N / 32) + (size_t)(kPfRT * ob) * src.sstep;
  src.nrt = kPfRT;
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
  v4f acc[kPfQ][2];
  zero_acc<kPfQ>(acc);
  pf_kloop<true>(L, src, acc);
  __syncthreads();   // s_r / s_w visible
  pf_combine<kPfQ, 2>(a, wk, acc, s_r, s_w, (size_t)256 * ob + 128 * wr + c, wc, c, g);
}

static int pf_grid(int grid_tiles, int nsub) { return (grid_tiles * nsub + 7) / 8 * 8; }

hipError_t launch_pf_gemm1(const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pf_gemm1_a8, dim3(pf_grid(grid_tiles, (a.N + 127) / 128)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pf_gemm2(const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pf_gemm2_a8, dim3(pf_grid(grid_tiles, a.K / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ================================================================ W4A16 / W3A16
//
// The same 64-route tiles and LDS ring for NVFP4 and NF3 experts with bf16
// activations.  A ring stage holds 8 weight row tiles of one 128-column k-tile
// in MFMA lane order (16 / 12 bytes and 2 / 1 scale bytes per lane) and the 64
// routes' bf16 activation slices (256 bytes each, 16-byte chunks XOR-swizzled
// by row % 16).  Wave w owns row tiles 2w, 2w + 1 against all 64 routes, so
// each weight element is dequantised once per tile, one 8-column step at a
// time (E2M1 x E4M3, or NF3 codebook x E4M3, to bf16; exact for E2M1), and
// feeds 4 bf16 MFMAs: 4 steps x 2 row tiles x 4 route blocks per k-tile.
namespace {

constexpr int kPf16Stages = 3;

// Direct-to-LDS loads of one wave per stage: NVFP4 2 weight tiles (16 bytes a
// lane) + 1 scale chunk + 4 activation chunks; NF3 6 dword loads for 2 weight
// tiles (768 bytes each) + 1 scale chunk + 4 activation chunks.  Loads narrower
// than a dword are not used: they would leave 4-byte lane slots in LDS.
template <int WF>
struct Pf16Loads {
  static constexpr int n = (WF == W_NVFP4) ? 7 : 11;
};

template <int WF>
struct Pf16Stage {
  static constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  uint8_t A[8][64 * U];
  uint8_t AS[8][64 * SU];
  uint8_t spare[256];   // NF3: landing slot of the scale loads of waves 2, 3
  uint8_t B[kPfTileRows][256];
};

template <int WF>
struct __attribute__((aligned(16))) Pf16Lds {
  Pf16Stage<WF> st[kPf16Stages];
};

template <int WF>
__device__ __forceinline__ void wait16_stages(int stages) {
  constexpr int n = Pf16Loads<WF>::n;
  if (stages >= 2) wait_vm<2 * n>();
  else if (stages == 1) wait_vm<n>();
  else wait_vm<0>();
}

struct Pf16Src {
  const uint8_t *wbase, *sbase;   // row tile rt, k-tile kt: wbase + rt * wstep + kt * 64 U (scales: 64 SU)
  size_t wstep, sstep;
  const uint16_t *brow[4];        // this lane's activation rows of its four B chunks
  int kcols;                      // reduction length (columns)
};

// The loads of wave w for k-tile kt: weight row tiles 2w, 2w+1 (NVFP4: one
// 16-byte load each; NF3: three dword loads of 256 bytes each), one dword load
// of scales (NVFP4: row tiles 2w, 2w+1; NF3: waves 0, 1 row tiles 4w .. 4w+3,
// waves 2, 3 a spare slot), activation chunks 4w .. 4w+3 (1 KB each: 4 routes x
// 256 bytes; lane l -> route 4j + l/16, LDS slot l % 16 holding global chunk
// slot ^ route%16).  Lanes past the reduction length load from a valid address.
template <int WF, bool FULL>
__device__ __forceinline__ void pf16_issue(Pf16Stage<WF> &S, const Pf16Src &src, int kt, int w, int l) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  if constexpr (WF == W_NVFP4) {
    const bool in = FULL || kt * 128 + 32 * (l >> 4) < src.kcols;
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int rt = 2 * w + j;
      dma16(src.wbase + rt * src.wstep + (in ? (size_t)kt * 64 * U + l * U : 0), &S.A[rt][0]);
    }
    // dword d of row tile 2w + l/32 holds the scales of MFMA lanes 2d, 2d + 1
    const int rt = 2 * w + (l >> 5), d = l & 31;
    const bool ins = FULL || kt * 128 + 32 * ((2 * d) >> 4) < src.kcols;
    dma4(src.sbase + rt * src.sstep + (ins ? (size_t)kt * 64 * SU + 4 * d : 0), &S.AS[2 * w][0]);
  } else {
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int rt = 2 * w + j;
#pragma unroll
      for (int m = 0; m < 3; m++) {   // bytes 256 m + 4 l of the row tile's 768-byte k-tile: MFMA lane (256 m + 4 l) / 12
        const int lane = (256 * m + 4 * l) / 12;
        const bool in = FULL || kt * 128 + 32 * (lane >> 4) < src.kcols;
        dma4(src.wbase + rt * src.wstep + (in ? (size_t)kt * 64 * U + 256 * m + 4 * l : 0), &S.A[rt][256 * m]);
      }
    }
    if (w < 2) {   // dword d of row tile 4w + l/16 holds the scales of MFMA lanes 4d .. 4d + 3
      const int rt = 4 * w + (l >> 4), d = l & 15;
      const bool ins = FULL || kt * 128 + 32 * ((4 * d) >> 4) < src.kcols;
      dma4(src.sbase + rt * src.sstep + (ins ? (size_t)kt * 64 * SU + 4 * d : 0), &S.AS[4 * w][0]);
    } else {
      dma4(src.sbase, &S.spare[0]);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int r = 4 * (4 * w + j) + (l >> 4), cg = (l & 15) ^ (r & 15), col = kt * 128 + 8 * cg;
    dma16(src.brow[j] + (FULL || col < src.kcols ? col : 0), &S.B[4 * (4 * w + j)][0]);
  }
}

// One wave's operands of a landed stage: its 2 weight row tiles (2w, 2w + 1)
// and all 64 routes' activation chunks (4 steps x 4 route blocks).
template <int WF>
struct Pf16Ops {
  uint32_t a[2][4];   // row tile q: NVFP4 4 dwords, NF3 3 dwords (+1 unused)
  int sc[2];
  v4i b[4][4];        // step s, route block cb
};

// LDS reads of one wave's operands (asm: invisible to the compiler's
// direct-to-LDS bookkeeping, as for the W4A8 kernels).  The wait is part of
// each statement: between an LDS read and its wait the compiler could copy the
// register it loads.
template <int WF>
__device__ __forceinline__ void pf16_read(Pf16Ops<WF> &o, const Pf16Stage<WF> &S, int w, int l) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  const int c = l & 15, g = l >> 4;
  const uint32_t va = lds_addr(&S.A[2 * w][l * U]), vs = lds_addr(&S.AS[2 * w][l * SU]);
  const uint8_t *brow = &S.B[c][0];   // + 16 rows (4096 bytes) per route block
  uint32_t vb[4];
#pragma unroll
  for (int s = 0; s < 4; s++) vb[s] = lds_addr(brow + 16 * ((4 * g + s) ^ c));
#define PF16_READ_B                               \
  "ds_read_b128 %0, %[b0]\n"                      \
  "ds_read_b128 %1, %[b0] offset:4096\n"          \
  "ds_read_b128 %2, %[b0] offset:8192\n"          \
  "ds_read_b128 %3, %[b0] offset:12288\n"         \
  "ds_read_b128 %4, %[b1]\n"                      \
  "ds_read_b128 %5, %[b1] offset:4096\n"          \
  "ds_read_b128 %6, %[b1] offset:8192\n"          \
  "ds_read_b128 %7, %[b1] offset:12288\n"         \
  "ds_read_b128 %8, %[b2]\n"                      \
  "ds_read_b128 %9, %[b2] offset:4096\n"          \
  "ds_read_b128 %10, %[b2] offset:8192\n"         \
  "ds_read_b128 %11, %[b2] offset:12288\n"        \
  "ds_read_b128 %12, %[b3]\n"                     \
  "ds_read_b128 %13, %[b3] offset:4096\n"         \
  "ds_read_b128 %14, %[b3] offset:8192\n"         \
  "ds_read_b128 %15, %[b3] offset:12288\n"
#define PF16_B_OUT                                                                                             \
  "=&v"(o.b[0][0]), "=&v"(o.b[0][1]), "=&v"(o.b[0][2]), "=&v"(o.b[0][3]), "=&v"(o.b[1][0]), "=&v"(o.b[1][1]), \
      "=&v"(o.b[1][2]), "=&v"(o.b[1][3]), "=&v"(o.b[2][0]), "=&v"(o.b[2][1]), "=&v"(o.b[2][2]),                 \
      "=&v"(o.b[2][3]), "=&v"(o.b[3][0]), "=&v"(o.b[3][1]), "=&v"(o.b[3][2]), "=&v"(o.b[3][3])
  if constexpr (WF == W_NVFP4) {
    v4i a0, a1;
    asm volatile(PF16_READ_B
                 "ds_read_b128 %16, %[va]\n"
                 "ds_read_b128 %17, %[va] offset:1024\n"
                 "ds_read_u16 %18, %[vs]\n"
                 "ds_read_u16 %19, %[vs] offset:128\n"
                 "s_waitcnt lgkmcnt(0)"
                 : PF16_B_OUT, "=&v"(a0), "=&v"(a1), "=&v"(o.sc[0]), "=&v"(o.sc[1])
                 : [b0] "v"(vb[0]), [b1] "v"(vb[1]), [b2] "v"(vb[2]), [b3] "v"(vb[3]), [va] "v"(va), [vs] "v"(vs)
                 : "memory");
#pragma unroll
    for (int d = 0; d < 4; d++) {
      o.a[0][d] = (uint32_t)a0[d];
      o.a[1][d] = (uint32_t)a1[d];
    }
  } else {
    // 12-byte lanes are only 4-byte aligned: three dword reads per row tile
    asm volatile(PF16_READ_B
                 "ds_read_b32 %16, %[va]\n"
                 "ds_read_b32 %17, %[va] offset:4\n"
                 "ds_read_b32 %18, %[va] offset:8\n"
                 "ds_read_b32 %19, %[va] offset:768\n"
                 "ds_read_b32 %20, %[va] offset:772\n"
                 "ds_read_b32 %21, %[va] offset:776\n"
                 "ds_read_u8 %22, %[vs]\n"
                 "ds_read_u8 %23, %[vs] offset:64\n"
                 "s_waitcnt lgkmcnt(0)"
                 : PF16_B_OUT, "=&v"(o.a[0][0]), "=&v"(o.a[0][1]), "=&v"(o.a[0][2]), "=&v"(o.a[1][0]),
                   "=&v"(o.a[1][1]), "=&v"(o.a[1][2]), "=&v"(o.sc[0]), "=&v"(o.sc[1])
                 : [b0] "v"(vb[0]), [b1] "v"(vb[1]), [b2] "v"(vb[2]), [b3] "v"(vb[3]), [va] "v"(va), [vs] "v"(vs)
                 : "memory");
    o.a[0][3] = o.a[1][3] = 0;
  }
#undef PF16_READ_B
#undef PF16_B_OUT
}

// 8 bf16 MFMAs of step S of a k-tile (2 row tiles x 4 route blocks); each
// dequantised weight operand feeds 4 MFMAs.  Columns past the reduction
// length: scale 0 (weights 0) and activations 0.  SWAP: activations as the A
// operand.
template <int WF, bool SWAP, bool FULL, int S>
__device__ __forceinline__ void pf16_mma_step(const Pf16Ops<WF> &o, bool gin, const float (&slo)[2], const float (&shi)[2],
                                              const uint32_t (&t01)[2], const uint32_t (&t23)[2], v4f (*acc)[4]) {
  v8bf bop[4];
#pragma unroll
  for (int cb = 0; cb < 4; cb++) bop[cb] = __builtin_bit_cast(v8bf, (FULL || gin) ? o.b[S][cb] : v4i{0, 0, 0, 0});
#pragma unroll
  for (int q = 0; q < 2; q++) {
    v8bf aop;
    if constexpr (WF == W_NVFP4) aop = nvfp4_step(o.a[q][S], S < 2 ? slo[q] : shi[q]);
    else aop = nf3_step_rc(S < 2 ? o.a[q][0] : o.a[q][1], o.a[q][2], S, t01[q], t23[q]);
#pragma unroll
    for (int cb = 0; cb < 4; cb++) acc[q][cb] = SWAP ? mfma_bf16(bop[cb], aop, acc[q][cb]) : mfma_bf16(aop, bop[cb], acc[q][cb]);
  }
}

// One k-tile: the scales are decoded once per row tile (NF3: its scaled
// magnitude table).
template <int WF, bool SWAP, bool FULL>
__device__ __forceinline__ void pf16_mma(const Pf16Ops<WF> &o, int kt, int kcols, int l, v4f (*acc)[4]) {
  const int g = l >> 4;
  const bool gin = FULL || kt * 128 + 32 * g < kcols;
  float slo[2] = {0.f, 0.f}, shi[2] = {0.f, 0.f};
  uint32_t t01[2] = {0u, 0u}, t23[2] = {0u, 0u};
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const uint32_t sc = gin ? (uint32_t)o.sc[q] : 0u;
    if constexpr (WF == W_NVFP4) {
      slo[q] = e4m3_f32(sc & 0xFFu);
      shi[q] = e4m3_f32((sc >> 8) & 0xFFu);
    } else {
      nf3_tables(e4m3_f32(sc & 0xFFu), t01[q], t23[q]);
    }
  }
  pf16_mma_step<WF, SWAP, FULL, 0>(o, gin, slo, shi, t01, t23, acc);
  pf16_mma_step<WF, SWAP, FULL, 1>(o, gin, slo, shi, t01, t23, acc);
  pf16_mma_step<WF, SWAP, FULL, 2>(o, gin, slo, shi, t01, t23, acc);
  pf16_mma_step<WF, SWAP, FULL, 3>(o, gin, slo, shi, t01, t23, acc);
}

// One k-tile of the ring: after the barrier that proves stage kt landed for
// every wave (and that every wave is done with stage kt - 1, whose slot then
// takes stage kt + ST - 1), stage kt is read.
template <int WF, bool SWAP>
__device__ __forceinline__ void pf16_step(Pf16Lds<WF> &L, const Pf16Src &src, int kt, int nkt, int w,
                                          v4f (*acc)[4]) {
  constexpr int ST = kPf16Stages;
  const int l = threadIdx.x & 63;
  wait16_stages<WF>(min(ST - 2, nkt - 1 - kt));   // stage kt has landed
  __builtin_amdgcn_s_barrier();
  const int kn = kt + ST - 1;
  if (kn < nkt) {
    if ((kn + 1) * 128 <= src.kcols) pf16_issue<WF, true>(L.st[kn % ST], src, kn, w, l);
    else pf16_issue<WF, false>(L.st[kn % ST], src, kn, w, l);
  }
  Pf16Ops<WF> o;
  pf16_read<WF>(o, L.st[kt % ST], w, l);
  if ((kt + 1) * 128 <= src.kcols) pf16_mma<WF, SWAP, true>(o, kt, src.kcols, l, acc);
  else pf16_mma<WF, SWAP, false>(o, kt, src.kcols, l, acc);
}

// w: the wave index, wave-uniform (scalar), so stage and weight addresses stay scalar.
template <int WF, bool SWAP>
__device__ __forceinline__ void pf16_kloop(Pf16Lds<WF> &L, const Pf16Src &src, int w, v4f (*acc)[4]) {
  constexpr int ST = kPf16Stages;
  const int l = threadIdx.x & 63;
  const int nkt = (src.kcols + 127) / 128;
#pragma unroll
  for (int s = 0; s < ST - 1; s++)
    if (s < nkt) pf16_issue<WF, false>(L.st[s], src, s, w, l);
  for (int kt = 0; kt < nkt; kt++) pf16_step<WF, SWAP>(L, src, kt, nkt, w, acc);
}

}  // namespace

// ---------------------------------------------------------------- GEMM1 (A16)
template <int WF>
__global__ __launch_bounds__(256) void k_pf_gemm1_a16(GemmArgs a) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  __shared__ Pf16Lds<WF> L;
  const int K = a.K, N = a.N;
  const PfWork wk = pf_work(a, N / 64, true);
  if (!wk.valid) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int hb = wk.sub, groups = K / 32;
  Pf16Src src;
  src.wstep = (size_t)16 * groups * U;
  src.sstep = (size_t)16 * groups * SU;
  src.wbase = a.w13 + (size_t)wk.e * (2 * N) * groups * U + (size_t)(8 * hb) * src.wstep;
  src.sbase = a.s13 + (size_t)wk.e * (2 * N) * groups * SU + (size_t)(8 * hb) * src.sstep;
  src.kcols = K;
  // rows past the tile read route p0's token; their results are never stored
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int row = 4 * (4 * w + j) + (l >> 4);
    src.brow[j] = a.xb + (size_t)(a.perm[wk.p0 + (row < wk.rows ? row : 0)] / a.topk) * K;
  }
  v4f acc[2][4];
#pragma unroll
  for (int q = 0; q < 2; q++)
#pragma unroll
    for (int cb = 0; cb < 4; cb++) acc[q][cb] = v4f{0.f, 0.f, 0.f, 0.f};
  pf16_kloop<WF, false>(L, src, wu, acc);
  // epilogue: row tiles 2w (up) and 2w + 1 (gate) = intermediate columns 64 hb + 16 w .. +15
  const float gs = a.g13 ? a.g13[wk.e] : 1.0f;
#pragma unroll
  for (int cb = 0; cb < 4; cb++) {
    const int row = 16 * cb + c;
    if (row < wk.rows) {
      const size_t p = (size_t)(wk.p0 + row);
      float h[4];
#pragma unroll
      for (int i = 0; i < 4; i++) h[i] = silu_clamped(acc[1][cb][i] * gs, acc[0][cb][i] * gs, a.limit, a.has_limit);
      uint2 v;
      v.x = pack_bf16x2(h[0], h[1]);
      v.y = pack_bf16x2(h[2], h[3]);
      *(uint2 *)(a.hb + p * N + 64 * hb + 16 * w + 4 * g) = v;
    }
  }
}

// ---------------------------------------------------------------- GEMM2 (A16)
template <int WF>
__global__ __launch_bounds__(256) void k_pf_gemm2_a16(GemmArgs a) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  __shared__ Pf16Lds<WF> L;
  __shared__ int s_r[kPfTileRows];
  __shared__ float s_w[kPfTileRows];
  const int K = a.K, N = a.N;
  const PfWork wk = pf_work(a, K / 128, false);
  if (!wk.valid) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int ob = wk.sub, groups = N / 32;   // output columns 128 ob .. +127 = w2 row tiles 8 ob .. +7
  Pf16Src src;
  src.wstep = (size_t)16 * groups * U;
  src.sstep = (size_t)16 * groups * SU;
  src.wbase = a.w2 + (size_t)wk.e * K * groups * U + (size_t)(8 * ob) * src.wstep;
  src.sbase = a.s2 + (size_t)wk.e * K * groups * SU + (size_t)(8 * ob) * src.sstep;
  src.kcols = N;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int row = 4 * (4 * w + j) + (l >> 4);
    src.brow[j] = a.hb + (size_t)(wk.p0 + (row < wk.rows ? row : 0)) * N;
  }
  if (tid < wk.rows) {
    const int r = a.perm[wk.p0 + tid];
    s_r[tid] = r;
    s_w[tid] = a.topk_w[r] * (a.g2 ? a.g2[wk.e] : 1.0f);
  }
  v4f acc[2][4];
#pragma unroll
  for (int q = 0; q < 2; q++)
#pragma unroll
    for (int cb = 0; cb < 4; cb++) acc[q][cb] = v4f{0.f, 0.f, 0.f, 0.f};
  pf16_kloop<WF, true>(L, src, wu, acc);
  __syncthreads();   // s_r / s_w visible
  // acc[q][cb][i]: route 16 cb + 4 g + i, output column 128 ob + 32 w + 16 q + c
  pf_combine<2, 4>(a, wk, acc, s_r, s_w, (size_t)128 * ob + 32 * w + c, 0, c, g);
}

template <int WF>
static hipError_t launch_pf_a16(const GemmArgs &a, int grid_tiles, hipStream_t s, bool second) {
  if (second) hipLaunchKernelGGL(k_pf_gemm2_a16<WF>, dim3(pf_grid(grid_tiles, a.K / 128)), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_pf_gemm1_a16<WF>, dim3(pf_grid(grid_tiles, a.N / 64)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pf16_gemm1(int wfmt, const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  return wfmt == W_NVFP4 ? launch_pf_a16<W_NVFP4>(a, grid_tiles, s, false) : launch_pf_a16<W_NF3>(a, grid_tiles, s, false);
}

hipError_t launch_pf16_gemm2(int wfmt, const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  return wfmt == W_NVFP4 ? launch_pf_a16<W_NVFP4>(a, grid_tiles, s, true) : launch_pf_a16<W_NF3>(a, grid_tiles, s, true);
}

}  // namespace moe
