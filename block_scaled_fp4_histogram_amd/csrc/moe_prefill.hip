// Prefill-size GEMMs: tiles of 64 routes of one expert.
//
// W4A8 (MXFP4 weights x MXFP8 activations).  A block of 4 waves holds 16
// weight row tiles (256 weight rows) against the tile's 64 routes; wave w owns
// row tiles 4w .. 4w+3 against all 64 routes, 16 block-scaled MFMAs per
// 128-column k-tile.  The weights and their scale dwords stream by buffer
// loads into a 3-deep register ring of each wave (no LDS); the activations are
// shared, so they go through a 3-stage LDS ring by direct global-to-LDS loads:
// one stage holds the 64 routes' MXFP8 slices of one k-tile (8 blocks of 8
// rows x 128 bytes, 16-byte chunks XOR-swizzled so that MFMA operand reads
// spread over the LDS banks) and their scales (64 x 4 bytes); each wave loads
// two of the blocks.  Every wave issues the same eleven loads per stage, so
// "all but the newest n stages have landed" is one s_waitcnt vmcnt(11 n) per
// wave followed by a barrier; the activations are read from LDS at the
// k-tile that uses them.
//
// Blocks are numbered XCD-major: the hardware hands workgroup b to XCD b % 8,
// so logical work item (b % 8) * per + b / 8 puts a contiguous run of items on
// each XCD, in order.  All prefill GEMMs order items tile-major: the column
// blocks of one tile run together on one XCD and share its activation rows in
// L2, and an expert's weights stay in L2 across its consecutive tiles.  (The
// up/gate GEMM ran column-block-major first, all tiles of an expert against
// one weight slab at once; its 64 resident blocks per XCD then each streamed
// private activation rows, about 530 KB of L2 fills per k-step against about
// 190 KB tile-major, and it measured 3 % slower; the W4A16 / W3A16 up/gate
// GEMM, whose bf16 activations are twice the bytes, 1-2 % slower.)
//
//   k_pf_gemm1_a8  items (tile, 128-column intermediate block = 8 up and 8
//                  gate row tiles): up/gate GEMMs over K, clamped SwiGLU and
//                  MXFP8 requantisation of 128 intermediate columns of 64 routes.
//   k_pf_gemm2_a8  items (tile, 256-column output block): down GEMM over N with
//                  the activations as the MFMA's A operand, so each lane holds
//                  16 consecutive output columns' worth of one route per
//                  instruction; combine straight from the accumulators (fp32
//                  atomics, or bf16 route-buffer rows).
//
// W4A16 / W3A16 (NVFP4 or NF3 weights x bf16 activations): see that section.
#include "moe_device.h"

namespace moe {

constexpr int kPfRT = 16;        // W4A8: weight row tiles per block (256 weight rows)
constexpr int kPfQ = 4;          // W4A8: row tiles per wave
constexpr int kPfStages = 3;     // W4A8: ring depth (k-tiles), LDS and registers
// vector-memory operations of one wave per stage: 4 weight tiles, 4 weight
// scale dwords, 2 activation blocks, 1 activation scale chunk (or a spare)
constexpr int kPfLoads = 11;

struct PfStage {
  uint8_t B[8][1024];             // activation rows 8b .. 8b+7 of block b, swizzled 16-byte chunks
  uint8_t S[1024];                // Bs [64][4] | 3 spare 256-byte slots
};

struct __attribute__((aligned(16))) PfLds {
  PfStage st[kPfStages];
};
// the deterministic combine stages 4 waves x 16 routes x (32 Q + 16) bytes in stage 0
static_assert(sizeof(PfStage) >= 4 * 16 * (32 * kPfQ + 16), "combine staging fits one ring stage");

// Wait until at most `stages` ring stages issued by this wave are in flight.
__device__ __forceinline__ void wait_stages(int stages) {
  if (stages >= 2) wait_vm<2 * kPfLoads>();
  else if (stages == 1) wait_vm<kPfLoads>();
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
  int single;   // the expert's routes fit this one tile: its weights are read once per column block
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
  w.single = a.off[u + 1] - a.off[u] <= a.tile_rows;
  return w;
}

struct PfSrc {
  Buf wb, sb;                     // the block's weight row tiles / their scales (nrt tiles)
  uint32_t wstep, sstep;          // bytes per row tile (data / scales)
  int nrt;                        // row tiles of this block that exist (8 or 16)
  const uint8_t *brow[2];         // this lane's activation rows of its two B blocks
  const uint8_t *bsrow;           // activation scale row of route (lane)
  int kbytes;                     // reduction length (bytes of one activation row)
  int nrb;                        // 16-route blocks holding routes of the tile (the rest are padding)
};

// A wave's weight operands of one k-tile: row tiles 4w + q, and the aligned
// scale dword holding this lane's byte (a narrower load would be zero-extended
// where the ring is carried round the loop, which makes the compiler wait for
// every load in flight there).  The scales are the prefill copies, in
// mx_soff's order: within a run of four whole k-tiles that dword holds the
// lane's bytes of all four, at bit 8 * (kt % 4) (pf_scale_shift).
struct PfW {
  v4i a[kPfQ];
  uint32_t sa[kPfQ];
};

// Weight and scale loads of wave w for k-tile kt.  Lanes whose 32-column group
// lies past the reduction length, and row tiles past the block's last one,
// read past the buffer's range: zeros, and no memory traffic.
// NT: non-temporal weight loads, for up/gate tiles whose expert's weights are
// read once per column block (the 64-route kernel on the 1024-token rung:
// 546 -> 517 us with them), not for the tiles of hot experts, which share
// weight lines in L2 (with them for every tile the 128-route kernel measured
// 268 -> 281 us at the Zipf-skewed 4096-token batch, the 64-route one
// 577 -> 669 us).  The 128-route kernel takes them for blocks whose expert
// fits the one tile (that batch: 271 -> 262 us), the 64-route one always.
// REUSE: kt lies inside a run of four whole k-tiles, past its first, and prev
// is the landed slot of k-tile kt - 1, whose scale dword holds this k-tile's
// bytes too: it is copied and no scale load is issued (for callers that wait
// for every load).
template <bool NT = false, bool REUSE = false>
__device__ __forceinline__ void pf_load_w(PfW &r, const PfSrc &src, int kt, int w, int l, const PfW *prev = nullptr) {
  const bool in = (kt * 4 + (l >> 4)) * 32 < src.kbytes;
  const uint32_t sv = mx_soff(kt, l, src.kbytes >> 7) & ~3u;
#pragma unroll
  for (int q = 0; q < kPfQ; q++) {
    const int rt = 4 * w + q;
    const bool ok = in && rt < src.nrt;
    const uint32_t so = rt < src.nrt ? (uint32_t)rt : 0u;
    const uint32_t vo = ok ? (uint32_t)(kt * 1024 + l * 16) : 0x80000000u;
    r.a[q] = NT ? buf_load16_nt(src.wb, vo, so * src.wstep) : buf_load16(src.wb, vo, so * src.wstep);
    if constexpr (REUSE) r.sa[q] = prev->sa[q];
    else r.sa[q] = buf_load4(src.sb, ok ? sv : 0x80000000u, so * src.sstep);
  }
}

// Bit position of lane l's scale byte of k-tile kt in its slot's dword.
__device__ __forceinline__ int pf_scale_shift(int kt, int l, int kbytes) {
  return 8 * (int)(mx_soff(kt, l, kbytes >> 7) & 3u);
}

// The shared loads of wave w for k-tile kt into stage S: activation blocks 2w,
// 2w+1 (lane l -> row l / 8, its chunk slot l) and the activation scales (wave
// 0; waves 1-3 fill spare slots to keep the per-wave load count equal).  Lanes
// past the reduction length load column 0; the MFMA step zeroes those bytes.
__device__ __forceinline__ void pf_issue_b(PfStage &S, const PfSrc &src, int kt, int w, int l) {
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int r8 = l >> 3, part = (l & 7) ^ r8, off = kt * 128 + part * 16;
    dma16(src.brow[j] + (off < src.kbytes ? off : 0), &S.B[2 * w + j][0]);
  }
  const int nkt = (src.kbytes + 127) / 128;
  dma4(src.bsrow + 4 * min(kt, nkt - 1), &S.S[256 * w]);   // a stage past the end re-reads the last one
}

// The 64 routes' activations of a landed stage: b[cb][h] = columns 64 h +
// 16 g .. of route 16 cb + c, sb[cb] its scale of 32-column group g.  Read
// with asm (invisible to the compiler's direct-to-LDS bookkeeping, which would
// otherwise wait for every ring stage in flight) and waited for in the same
// statement (a wait in a later statement would let the compiler copy
// registers still in flight).
// B0: the first of the 8 activation blocks (8 rows each) of the 64 routes read;
// S0: their scales, 4 bytes a route.
__device__ __forceinline__ void pf_read_b_at(v4i (&b)[4][2], int (&sb)[4], const uint8_t (*B0)[1024],
                                             const uint8_t *S0, int l) {
  const int c = l & 15, g = l >> 4, r8 = c & 7;
  const uint8_t *blk = &B0[c >> 3][0];   // + 2 KB per route block
  const uint32_t vb0 = lds_addr(blk + pf_slot(r8, g) * 16), vb1 = lds_addr(blk + pf_slot(r8, 4 + g) * 16),
                 vsb = lds_addr(&S0[c * 4 + g]);   // + 64 bytes per route block
  asm volatile(
      "ds_read_b128 %0, %12\n"
      "ds_read_b128 %1, %13\n"
      "ds_read_b128 %2, %12 offset:2048\n"
      "ds_read_b128 %3, %13 offset:2048\n"
      "ds_read_b128 %4, %12 offset:4096\n"
      "ds_read_b128 %5, %13 offset:4096\n"
      "ds_read_b128 %6, %12 offset:6144\n"
      "ds_read_b128 %7, %13 offset:6144\n"
      "ds_read_u8 %8, %14\n"
      "ds_read_u8 %9, %14 offset:64\n"
      "ds_read_u8 %10, %14 offset:128\n"
      "ds_read_u8 %11, %14 offset:192\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(b[0][0]), "=&v"(b[0][1]), "=&v"(b[1][0]), "=&v"(b[1][1]), "=&v"(b[2][0]), "=&v"(b[2][1]),
        "=&v"(b[3][0]), "=&v"(b[3][1]), "=&v"(sb[0]), "=&v"(sb[1]), "=&v"(sb[2]), "=&v"(sb[3])
      : "v"(vb0), "v"(vb1), "v"(vsb)
      : "memory");
}

__device__ __forceinline__ void pf_read_b(v4i (&b)[4][2], int (&sb)[4], const PfStage &S, int l) {
  pf_read_b_at(b, sb, S.B, S.S, l);
}

// 16 block-scaled MFMAs of one k-tile (4 row tiles x 4 route blocks).  Past
// the reduction length (a partial last k-tile; FULL: none) the activation
// bytes are zeroed and both scales set to 2^-127, so the products there are
// exact zeros.  SWAP: activations as the A operand (accumulator lane = output
// column, elements = 4 routes).
template <bool SWAP, bool FULL>
__device__ __forceinline__ void pf_mma(const PfW &wt, const v4i (&b)[4][2], const int (&sb)[4], int kt, int kbytes,
                                       int nrb, int l, v4f (*acc)[4], const uint32_t *sa_src = nullptr) {
  const int g = l >> 4;
  const bool in0 = FULL || kt * 128 + 16 * g < kbytes, in1 = FULL || kt * 128 + 64 + 16 * g < kbytes;
  const bool gin = FULL || (kt * 4 + g) * 32 < kbytes;   // 32-column group g of this k-tile exists
  v8i bop[4];
#pragma unroll
  for (int cb = 0; cb < 4; cb++) {
    const v4i b0 = in0 ? b[cb][0] : v4i{0, 0, 0, 0};
    const v4i b1 = in1 ? b[cb][1] : v4i{0, 0, 0, 0};
    bop[cb] = v8i{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
  }
  // route blocks past the tile's last route hold padding: their MFMAs are skipped,
  // one branch per route block (4 MFMAs)
  int sa[kPfQ];
  const uint32_t *sap = sa_src ? sa_src : wt.sa;
  const int sh = pf_scale_shift(kt, l, kbytes);
#pragma unroll
  for (int q = 0; q < kPfQ; q++) sa[q] = gin ? (int)(sap[q] >> sh) : 0;   // the MFMA takes the low byte
#pragma unroll
  for (int cb = 0; cb < 4; cb++) {
    if (cb < nrb) {
      const int sbv = gin ? sb[cb] : 0;
#pragma unroll
      for (int q = 0; q < kPfQ; q++) {
        if (SWAP)
          acc[q][cb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bop[cb], fp4_operand(wt.a[q]), acc[q][cb], 0,
                                                                        4, 0, sbv, 0, sa[q]);
        else
          acc[q][cb] = mfma_fp4_fp8(wt.a[q], bop[cb], acc[q][cb], sa[q], sbv);
      }
    }
  }
}

// One k-tile (R = kt % ST).  After the barrier that proves stage kt landed for
// every wave (and that every wave is done with stage kt - 1), k-tile
// kt + ST - 1 is issued: its activations into stage kt - 1's LDS slot, its
// weights into the register set that held k-tile kt - 1.  Then stage kt is
// read and multiplied with register set R.  WAITN: loads allowed in flight at
// the wait (kPfLoads when k-tile kt + 1 exists, else 0; -1: decided at run
// time); ISSUE: whether k-tile kt + ST - 1 exists (-1: at run time).  Where
// both are known at compile time the compiler's own bookkeeping of the ring
// registers stays exact.  Waves without weight rows (the missing half of a
// partial block) still load and pass the barriers, but skip the MFMAs.
template <bool SWAP, int R, int WAITN, int ISSUE, bool NT>
__device__ __forceinline__ void pf_step(PfLds &L, const PfSrc &src, PfW (&ring)[kPfStages], int kt, int nkt, int w,
                                        bool active, v4f (*acc)[4]) {
  constexpr int ST = kPfStages;
  const int l = threadIdx.x & 63;
  if constexpr (WAITN == kPfLoads) wait_vm<kPfLoads>();
  else if constexpr (WAITN == 0) wait_vm<0>();
  else wait_stages(min(ST - 2, nkt - 1 - kt));   // stage kt has landed
  __builtin_amdgcn_s_barrier();
  const int kn = kt + ST - 1;
  if (ISSUE == 1 || (ISSUE == -1 && kn < nkt)) {
    // one branch-free load sequence keeps the compiler's waits exact
    pf_load_w<NT>(ring[(R + ST - 1) % ST], src, kn, w, l);
    pf_issue_b(L.st[kn % ST], src, kn, w, l);
  }
  v4i b[4][2];
  int sb[4];
  pf_read_b(b, sb, L.st[kt % ST], l);
  if (active) {
    // raised issue priority while this wave has MFMAs ready: the arbiter then
    // feeds the matrix core from it while the SIMD's other wave waits on memory
    __builtin_amdgcn_s_setprio(1);
    // a step that issues k-tile kt + ST - 1 is not the last one, so its k-tile
    // is whole: known at compile time, the partial-tile variant and the
    // accumulator copies where the two variants meet drop out of the loop
    if (ISSUE == 1 || (kt + 1) * 128 <= src.kbytes) pf_mma<SWAP, true>(ring[R], b, sb, kt, src.kbytes, src.nrb, l, acc);
    else pf_mma<SWAP, false>(ring[R], b, sb, kt, src.kbytes, src.nrb, l, acc);
    __builtin_amdgcn_s_setprio(0);
  }
}

// The k-loop of both GEMMs: whole ring turns while every step is steady, then
// at most ST + 1 closing steps.  w: the wave index, wave-uniform (scalar).
template <bool SWAP, bool NT = false>
__device__ __forceinline__ void pf_kloop(PfLds &L, const PfSrc &src, int w, v4f (*acc)[4]) {
  constexpr int ST = kPfStages;
  static_assert(ST == 3, "the k-loop is unrolled by the ring depth");
  const int l = threadIdx.x & 63;
  const int nkt = (src.kbytes + 127) / 128;
  const bool active = kPfQ * w < src.nrt;
  PfW ring[ST];
  // stages 0 .. ST - 2 are issued even past the last k-tile (weights then load
  // as zeros without traffic, activations from column 0): a fixed load count
  // keeps the compiler's bookkeeping of the ring registers exact
#pragma unroll
  for (int s = 0; s < ST - 1; s++) {
    pf_load_w<NT>(ring[s], src, s, w, l);
    pf_issue_b(L.st[s], src, s, w, l);
  }
  int kt = 0;
  for (; kt + 2 * ST - 1 <= nkt; kt += ST) {   // k-tiles kt .. kt + 2 steady: kt + 2 + ST - 1 < nkt
    pf_step<SWAP, 0, kPfLoads, 1, NT>(L, src, ring, kt, nkt, w, active, acc);
    pf_step<SWAP, 1, kPfLoads, 1, NT>(L, src, ring, kt + 1, nkt, w, active, acc);
    pf_step<SWAP, 2, kPfLoads, 1, NT>(L, src, ring, kt + 2, nkt, w, active, acc);
  }
  if (kt < nkt) pf_step<SWAP, 0, -1, -1, NT>(L, src, ring, kt, nkt, w, active, acc);
  if (kt + 1 < nkt) pf_step<SWAP, 1, -1, -1, NT>(L, src, ring, kt + 1, nkt, w, active, acc);
  if (kt + 2 < nkt) pf_step<SWAP, 2, -1, -1, NT>(L, src, ring, kt + 2, nkt, w, active, acc);
  if (kt + 3 < nkt) pf_step<SWAP, 0, -1, -1, NT>(L, src, ring, kt + 3, nkt, w, active, acc);
  if (kt + 4 < nkt) pf_step<SWAP, 1, -1, -1, NT>(L, src, ring, kt + 4, nkt, w, active, acc);
}

template <int Q, int CB>
__device__ __forceinline__ void zero_acc(v4f (*acc)[CB]) {
#pragma unroll
  for (int q = 0; q < Q; q++)
#pragma unroll
    for (int cb = 0; cb < CB; cb++) acc[q][cb] = v4f{0.f, 0.f, 0.f, 0.f};
}

// Down-GEMM combine from accumulators in the swapped layout: acc[q][cb][i] is
// route 32 wc + 16 cb + 4 g + i (tile row; cb < CB), output column col + 16 q; s_r, s_w
// hold each tile row's route and its router weight (times the expert's global
// scale).  Deterministic mode writes bf16 route-buffer rows through LDS
// (pf_store_rb; wc = 0); atomic mode adds fp32 into the token accumulator, 4
// routes x 16 consecutive columns per instruction.
//
// The deterministic combine through LDS (lds: 16 x (32 Q + 16) bytes per
// wave, free after the k-loop's last barrier): for each block of 16 routes the
// wave stages its slice (16 Q columns, bf16, router weight applied) in its
// own region and writes it back as 16-byte chunks, whole 32 Q-byte row
// segments per route, in a quarter of the store instructions that writing the
// 4-byte pairs directly takes (each of those covers eight rows 32 bytes apart).
// A wave's LDS reads and writes are done in order, so no wait or barrier is
// needed between the two phases or before the next block overwrites them.
// SE: the sums are of fp16 rows scaled by 2^-s_e[route]; they are multiplied
// back by 2^s_e before the router weight.
template <int Q, int CB, bool SE = false>
__device__ __forceinline__ void pf_store_rb(const GemmArgs &a, const PfWork &wk, v4f (*acc)[CB], const int *s_r,
                                            const float *s_w, size_t col0, int c, int g, uint8_t *lds,
                                            const int *s_e = nullptr) {
  constexpr int RB = 32 * Q, RS = RB + 16, CH = RB / 16;   // row bytes, LDS row stride, 16-byte chunks a row
  const int l = threadIdx.x & 63;
  uint8_t *lw = lds + (threadIdx.x >> 6) * 16 * RS;
  const bool odd = c & 1;   // lanes c, c ^ 1 swap one value: each then holds two adjacent columns of one route
#pragma unroll
  for (int cb = 0; cb < CB; cb++) {
#pragma unroll
    for (int ip = 0; ip < 2; ip++) {
      const int rl = 4 * g + 2 * ip + (odd ? 1 : 0), row = 16 * cb + rl;
      const float wgt = row < wk.rows ? s_w[row] : 0.f;
      const int er = (SE && row < wk.rows) ? s_e[row] : 0;
#pragma unroll
      for (int q = 0; q < Q; q++) {
        // even lane: lo = its a0, hi = the odd partner's a0; odd lane: lo = the
        // even partner's a1, hi = its a1 (selects on two named elements: an
        // element index that depends on the lane compiles to a 4-way chain)
        const float a0 = acc[q][cb][2 * ip], a1 = acc[q][cb][2 * ip + 1];
        const float give = odd ? a0 : a1;
        const float got = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(give), 0xB1, 0xF, 0xF, false));
        float lo = odd ? got : a0, hi = odd ? a1 : got;
        if constexpr (SE) {
          lo = __builtin_amdgcn_ldexpf(lo, er);
          hi = __builtin_amdgcn_ldexpf(hi, er);
        }
        *(uint32_t *)(lw + rl * RS + 2 * ((c & ~1) + 16 * q)) = pack_bf16x2(wgt * lo, wgt * hi);
      }
    }
#pragma unroll
    for (int j = 0; j < Q / 2; j++) {
      const int idx = l + 64 * j, rl = idx / CH, ch = idx - rl * CH, row = 16 * cb + rl;
      const v4i v = *(const v4i *)(lw + rl * RS + 16 * ch);
      if (row < wk.rows) *(v4i *)(a.rb + (size_t)s_r[row] * a.K + col0 + 8 * ch) = v;
    }
  }
}

template <int Q, int CB>
__device__ __forceinline__ void pf_combine(const GemmArgs &a, const PfWork &wk, v4f (*acc)[CB], const int *s_r,
                                           const float *s_w, size_t col, int wc, int c, int g, uint8_t *lds) {
  const int K = a.K;
  if (a.deterministic) {
    pf_store_rb<Q, CB>(a, wk, acc, s_r, s_w, col - c, c, g, lds);
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
// last block of an N % 128 == 64 layer holds 8).  Wave w: row tiles 4w .. 4w+3
// = up and gate of intermediate columns 128 hb + 32 w .. +31 (one MXFP8 group).
__global__ __launch_bounds__(256, 2) void k_pf_gemm1_a8(GemmArgs a) {
  __shared__ PfLds L;
  const int K = a.K, N = a.N;
  const PfWork wk = pf_work(a, (N + 127) / 128, false);
  if (!wk.valid) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int hb = wk.sub;
  PfSrc src;
  src.wstep = (uint32_t)(16 * (K / 2));
  src.sstep = (uint32_t)(16 * (K / 32));
  src.nrt = min(kPfRT, N / 8 - kPfRT * hb);
  src.wb = make_buf(a.w13 + (size_t)wk.e * (2 * N) * (K / 2) + (size_t)(kPfRT * hb) * src.wstep, src.nrt * src.wstep);
  src.sb = make_buf(a.s13 + (size_t)wk.e * (2 * N) * (K / 32) + (size_t)(kPfRT * hb) * src.sstep,
                    src.nrt * src.sstep);
  src.kbytes = K;
  // rows past the tile read route p0's token; their results are never stored
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int row = 8 * (2 * w + j) + (l >> 3);
    src.brow[j] = a.xq + (size_t)(a.perm[wk.p0 + (row < wk.rows ? row : 0)] / a.topk) * K;
  }
  src.bsrow = a.xs + (size_t)(a.perm[wk.p0 + (l < wk.rows ? l : 0)] / a.topk) * (K / 32);
  src.nrb = 4;   // every route block (skipping padding here costs registers this kernel does not have)
  v4f acc[kPfQ][4];
  zero_acc<kPfQ, 4>(acc);
  // non-temporal weights for every tile: the ladder runs this kernel where experts
  // average under 32 routes, mostly one tile each (choosing per block, as the
  // 128-route kernel does, makes this kernel spill and measured slower: 1024-token
  // rung 568 vs 516 us)
  pf_kloop<false, true>(L, src, wu, acc);
  if (kPfQ * w >= src.nrt) return;   // the missing half of a partial block
  // epilogue: row tiles 4w + 2s (up) and 4w + 2s + 1 (gate) = intermediate
  // columns 128 hb + 32 w + 16 s .. +15; their 32 columns form one MXFP8 group
  const int hss = hs_stride(N);
  const size_t c0 = (size_t)128 * hb + 32 * w;
#pragma unroll
  for (int cb = 0; cb < 4; cb++) {
    const int row = 16 * cb + c;
    float h[8];
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
      for (int i = 0; i < 4; i++) h[s * 4 + i] = silu_clamped(acc[2 * s + 1][cb][i], acc[2 * s][cb][i], a.limit, a.has_limit, a.alpha, a.beta, a.act);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(h[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    float inv;
    const uint32_t sbyte = mx_scale(amax, &inv);
    if (row < wk.rows) {
      const size_t p = (size_t)(wk.p0 + row);
#pragma unroll
      for (int s = 0; s < 2; s++)
        *(uint32_t *)(a.hq + p * N + c0 + 16 * s + 4 * g) = e4m3x4(h[s * 4], h[s * 4 + 1], h[s * 4 + 2], h[s * 4 + 3], inv);
      if (g == 0) a.hs[p * hss + c0 / 32] = (uint8_t)sbyte;
    }
  }
}

// ------------------------------------------------ GEMM1, 128-route tiles
// The same block of 16 weight row tiles (256 weight rows) against a tile of 128
// routes: each wave owns row tiles 4w .. 4w+3 against all 128 routes, 32
// block-scaled MFMAs per k-tile between two barriers, and each weight row tile
// streamed from L2 serves twice the routes of a 64-route tile (at the 4096-token
// prefill with Zipf-skewed loads, 299 weight passes instead of 485).  The
// activations of a k-tile (16 blocks of 8 routes, 16.5 KB) go through a 2-deep
// LDS ring, the weights through a 2-deep register ring: one k-tile of 32 MFMAs
// per wave covers the next one's loads.  The routes are read from LDS in two
// halves of 64 (the second skipped in tiles of at most 64 routes), and the MFMAs
// of 16-route blocks past the tile's last route are skipped.
constexpr int kPwStages = 2;
// Activation scales: every route's whole scale row (K / 32 bytes) is staged in
// LDS once per block, rows kPwXsRow bytes apart (68 dwords: the 16 routes a
// read touches fall in 16 different banks).  Per-k-tile scale loads would each
// touch one 128-byte line per route, a third of the lines a step requests.
constexpr int kPwXsRow = 272;
constexpr int kPwMaxK = kPwXsRow * 32;   // largest reduction the staged rows hold

struct PwStage {
  uint8_t B[16][1024];            // activation rows 8b .. 8b+7 of block b, swizzled 16-byte chunks
};

struct __attribute__((aligned(16))) PwLds {
  PwStage st[kPwStages];
  uint8_t XS[kPfWideRows * kPwXsRow];   // the tile's 128 activation scale rows
};

struct PwSrc {
  PfSrc w;                        // weights (wb, sb, wstep, sstep, nrt, kbytes)
  const uint8_t *xq;              // MXFP8 activations (uniform base)
  uint32_t brow[4];               // byte offsets of this lane's activation rows of its four B blocks
};

// Activation blocks 4w .. 4w+3 of k-tile kt into stage S (lane l -> row l / 8
// of its block, chunk slot l).  The reduction is whole k-tiles (K % 256 == 0).
__device__ __forceinline__ void pw_issue_b(PwStage &S, const PwSrc &src, int kt, int w, int l) {
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int r8 = l >> 3, part = (l & 7) ^ r8;
    dma16(src.xq + (src.brow[j] + (uint32_t)(kt * 128 + part * 16)), &S.B[4 * w + j][0]);
  }
}

// Every route's scale row into XS by direct 16-byte loads: wave w fills the
// 1 KB chunks w, w + 4, ... (chunk q of the flat XS holds part q % 17 of row
// q / 17; parts past the row's K / 32 bytes re-read part 0, padding nothing
// reads).  Rows past the tile read route p0's token.
__device__ __forceinline__ void pw_stage_scales(PwLds &L, const GemmArgs &a, const PfWork &wk, int w, int l) {
  constexpr int kParts = kPwXsRow / 16, kChunks = kPfWideRows * kParts / 64;
  const int row_bytes = a.K / 32;
  for (int i = w; i < kChunks; i += 4) {
    const int q = i * 64 + l, r = q / kParts, part = q - r * kParts;
    const int tok = a.perm[wk.p0 + (r < wk.rows ? r : 0)] / a.topk;
    dma16(a.xs + (size_t)tok * row_bytes + (part * 16 < row_bytes ? part * 16 : 0), &L.XS[i * 1024]);
  }
}

// The 64 routes of half H of a landed stage (as pf_read_b_at) and their scales
// of k-tile kt from XS: vxs = XS + c * kPwXsRow + g, offsets per 16-route block.
template <int H>
__device__ __forceinline__ void pw_read_b(v4i (&b)[4][2], int (&sb)[4], const PwStage &S, uint32_t vxs, int kt,
                                          int l) {
  const int c = l & 15, g = l >> 4, r8 = c & 7;
  const uint8_t *blk = &S.B[8 * H + (c >> 3)][0];   // + 2 KB per route block
  const uint32_t vb0 = lds_addr(blk + pf_slot(r8, g) * 16), vb1 = lds_addr(blk + pf_slot(r8, 4 + g) * 16),
                 vsb = vxs + (uint32_t)(4 * kt);
  constexpr int R16 = 16 * kPwXsRow, O = 64 * H * kPwXsRow;   // bytes per 16 routes; half H's first route
  asm volatile(
      "ds_read_b128 %0, %12\n"
      "ds_read_b128 %1, %13\n"
      "ds_read_b128 %2, %12 offset:2048\n"
      "ds_read_b128 %3, %13 offset:2048\n"
      "ds_read_b128 %4, %12 offset:4096\n"
      "ds_read_b128 %5, %13 offset:4096\n"
      "ds_read_b128 %6, %12 offset:6144\n"
      "ds_read_b128 %7, %13 offset:6144\n"
      "ds_read_u8 %8, %14 offset:%c15\n"
      "ds_read_u8 %9, %14 offset:%c16\n"
      "ds_read_u8 %10, %14 offset:%c17\n"
      "ds_read_u8 %11, %14 offset:%c18\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(b[0][0]), "=&v"(b[0][1]), "=&v"(b[1][0]), "=&v"(b[1][1]), "=&v"(b[2][0]), "=&v"(b[2][1]),
        "=&v"(b[3][0]), "=&v"(b[3][1]), "=&v"(sb[0]), "=&v"(sb[1]), "=&v"(sb[2]), "=&v"(sb[3])
      : "v"(vb0), "v"(vb1), "v"(vsb), "i"(O), "i"(O + R16), "i"(O + 2 * R16), "i"(O + 3 * R16)
      : "memory");
}

// 16 MFMAs of one half (routes 64 h .. 64 h + 63) of a k-tile: the half's
// 16-route blocks cb with 4 h + cb < nrb.
template <int H>
__device__ __forceinline__ void pw_mma(const PfW &wt, const v4i (&b)[4][2], const int (&sb)[4], int nrb, int sh,
                                       v4f (*acc)[8]) {
#pragma unroll
  for (int cb = 0; cb < 4; cb++) {
    if (4 * H + cb < nrb) {
      const v8i bop = v8i{b[cb][0][0], b[cb][0][1], b[cb][0][2], b[cb][0][3],
                          b[cb][1][0], b[cb][1][1], b[cb][1][2], b[cb][1][3]};
#pragma unroll
      for (int q = 0; q < kPfQ; q++)
        acc[q][4 * H + cb] = mfma_fp4_fp8(wt.a[q], bop, acc[q][4 * H + cb], (int)(wt.sa[q] >> sh), sb[cb]);
    }
  }
}

// One k-tile (R = kt % 2): wait for stage kt (the only one in flight), barrier
// (every wave is also done with stage kt - 1), issue k-tile kt + 1 into the
// slots kt - 1 held (ISSUE), then both halves of stage kt.
// REUSE: k-tile kt + 1 lies inside a run of four whole k-tiles, past its first.
template <int R, bool ISSUE, bool NT, bool REUSE = false>
__device__ __forceinline__ void pw_step(PwLds &L, const PwSrc &src, PfW (&ring)[kPwStages], int kt, int w,
                                        bool active, int nrb, uint32_t vxs, v4f (*acc)[8]) {
  const int l = threadIdx.x & 63;
  wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  if (ISSUE) {
    pf_load_w<NT, REUSE>(ring[R ^ 1], src.w, kt + 1, w, l, &ring[R]);
    pw_issue_b(L.st[R ^ 1], src, kt + 1, w, l);
  }
  if (active) {
    v4i b[4][2];
    int sb[4];
    const int sh = pf_scale_shift(kt, l, src.w.kbytes);
    pw_read_b<0>(b, sb, L.st[R], vxs, kt, l);
    __builtin_amdgcn_s_setprio(1);
    pw_mma<0>(ring[R], b, sb, nrb, sh, acc);
    __builtin_amdgcn_s_setprio(0);
    if (nrb > 4) {
      pw_read_b<1>(b, sb, L.st[R], vxs, kt, l);
      __builtin_amdgcn_s_setprio(1);
      pw_mma<1>(ring[R], b, sb, nrb, sh, acc);
      __builtin_amdgcn_s_setprio(0);
    }
  }
}

// The k-loop; NT: non-temporal weight loads.
template <bool NT>
__device__ __forceinline__ void pw_kloop(PwLds &L, const PwSrc &src, int nkt, int wu, bool active, int nrb,
                                         uint32_t vxs, v4f (*acc)[8]) {
  const int l = threadIdx.x & 63;
  PfW ring[kPwStages];
  pf_load_w<NT>(ring[0], src.w, 0, wu, l);
  pw_issue_b(L.st[0], src, 0, wu, l);
  int kt = 0;
  // runs of four k-tiles: one scale load each
  for (; kt + 4 < nkt; kt += 4) {
    pw_step<0, true, NT, true>(L, src, ring, kt, wu, active, nrb, vxs, acc);
    pw_step<1, true, NT, true>(L, src, ring, kt + 1, wu, active, nrb, vxs, acc);
    pw_step<0, true, NT, true>(L, src, ring, kt + 2, wu, active, nrb, vxs, acc);
    pw_step<1, true, NT>(L, src, ring, kt + 3, wu, active, nrb, vxs, acc);
  }
  for (; kt + 2 < nkt; kt += 2) {
    pw_step<0, true, NT>(L, src, ring, kt, wu, active, nrb, vxs, acc);
    pw_step<1, true, NT>(L, src, ring, kt + 1, wu, active, nrb, vxs, acc);
  }
  pw_step<0, true, NT>(L, src, ring, kt, wu, active, nrb, vxs, acc);
  pw_step<1, false, NT>(L, src, ring, kt + 1, wu, active, nrb, vxs, acc);
}

// Block: 16 row tiles of w13 = up and gate of 128 intermediate columns (8 in
// the last block of an N % 128 == 64 layer) against a tile of up to 128 routes.
__global__ __launch_bounds__(256, 2) void k_pf_gemm1_a8w(GemmArgs a) {
  __shared__ PwLds L;
  const int K = a.K, N = a.N;
  const PfWork wk = pf_work(a, (N + 127) / 128, false);
  if (!wk.valid) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int hb = wk.sub;
  PwSrc src;
  src.w.wstep = (uint32_t)(16 * (K / 2));
  src.w.sstep = (uint32_t)(16 * (K / 32));
  src.w.nrt = min(kPfRT, N / 8 - kPfRT * hb);
  src.w.wb = make_buf(a.w13 + (size_t)wk.e * (2 * N) * (K / 2) + (size_t)(kPfRT * hb) * src.w.wstep,
                      src.w.nrt * src.w.wstep);
  src.w.sb = make_buf(a.s13 + (size_t)wk.e * (2 * N) * (K / 32) + (size_t)(kPfRT * hb) * src.w.sstep,
                      src.w.nrt * src.w.sstep);
  src.w.kbytes = K;
  // rows past the tile read route p0's token; their results are never stored
  // 32-bit byte offsets: the host runs this kernel only for chunks with T * K < 2^32
  src.xq = a.xq;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int row = 8 * (4 * w + j) + (l >> 3);
    src.brow[j] = (uint32_t)(a.perm[wk.p0 + (row < wk.rows ? row : 0)] / a.topk) * (uint32_t)K;
  }
  const int nrb = __builtin_amdgcn_readfirstlane((wk.rows + 15) / 16);
  const bool active = kPfQ * w < src.w.nrt;
  v4f acc[kPfQ][8];
  zero_acc<kPfQ, 8>(acc);
  const int nkt = K / 128;   // even: K % 256 == 0
  pw_stage_scales(L, a, wk, wu, l);   // landed by the first step's wait
  const uint32_t vxs = lds_addr(&L.XS[c * kPwXsRow + g]);
  if (wk.single) pw_kloop<true>(L, src, nkt, wu, active, nrb, vxs, acc);
  else pw_kloop<false>(L, src, nkt, wu, active, nrb, vxs, acc);
  if (!active) return;   // the missing half of a partial block
  // epilogue: row tiles 4w + 2s (up) and 4w + 2s + 1 (gate) = intermediate
  // columns 128 hb + 32 w + 16 s .. +15; their 32 columns form one MXFP8 group
  const int hss = hs_stride(N);
  const size_t c0 = (size_t)128 * hb + 32 * w;
#pragma unroll
  for (int cb = 0; cb < 8; cb++) {
    if (cb >= nrb) break;
    const int row = 16 * cb + c;
    float h[8];
#pragma unroll
    for (int s = 0; s < 2; s++)
#pragma unroll
      for (int i = 0; i < 4; i++)
        h[s * 4 + i] = silu_clamped(acc[2 * s + 1][cb][i], acc[2 * s][cb][i], a.limit, a.has_limit, a.alpha, a.beta,
                                    a.act);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(h[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16));
    amax = fmaxf(amax, __shfl_xor(amax, 32));
    float inv;
    const uint32_t sbyte = mx_scale(amax, &inv);
    if (row < wk.rows) {
      const size_t p = (size_t)(wk.p0 + row);
#pragma unroll
      for (int s = 0; s < 2; s++)
        *(uint32_t *)(a.hq + p * N + c0 + 16 * s + 4 * g) = e4m3x4(h[s * 4], h[s * 4 + 1], h[s * 4 + 2], h[s * 4 + 3], inv);
      if (g == 0) a.hs[p * hss + c0 / 32] = (uint8_t)sbyte;
    }
  }
}

// ---------------------------------------------------------------- GEMM2
// Block: 16 row tiles of w2 = 256 output columns; wave w: output columns
// 256 ob + 64 w .. +63 of all 64 routes.
struct PfG2 {
  PfSrc src;
  PfWork wk;
  int ob;
};

__device__ __forceinline__ bool pf_g2_setup(const GemmArgs &a, PfG2 &g2, int *s_r, float *s_w) {
  const int K = a.K, N = a.N, tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  g2.wk = pf_work(a, K / 256, false);
  if (!g2.wk.valid) return false;
  const PfWork &wk = g2.wk;
  g2.ob = wk.sub;
  PfSrc &src = g2.src;
  src.wstep = (uint32_t)(16 * (N / 2));
  src.sstep = (uint32_t)(16 * (N / 32));
  src.nrt = kPfRT;
  src.wb = make_buf(a.w2 + (size_t)wk.e * K * (N / 2) + (size_t)(kPfRT * g2.ob) * src.wstep, kPfRT * src.wstep);
  src.sb = make_buf(a.s2 + (size_t)wk.e * K * (N / 32) + (size_t)(kPfRT * g2.ob) * src.sstep, kPfRT * src.sstep);
  src.kbytes = N;
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int row = 8 * (2 * w + j) + (l >> 3);
    src.brow[j] = a.hq + (size_t)(wk.p0 + (row < wk.rows ? row : 0)) * N;
  }
  src.bsrow = a.hs + (size_t)(wk.p0 + (l < wk.rows ? l : 0)) * hs_stride(N);
  src.nrb = __builtin_amdgcn_readfirstlane((wk.rows + 15) / 16);
  if (tid < wk.rows) {
    const int r = a.perm[wk.p0 + tid];
    s_r[tid] = r;
    s_w[tid] = a.topk_w[r];
  }
  return true;
}

__global__ __launch_bounds__(256, 2) void k_pf_gemm2_a8(GemmArgs a) {
  __shared__ PfLds L;
  __shared__ int s_r[kPfTileRows];
  __shared__ float s_w[kPfTileRows];
  PfG2 g2;
  if (!pf_g2_setup(a, g2, s_r, s_w)) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  v4f acc[kPfQ][4];
  zero_acc<kPfQ, 4>(acc);
  pf_kloop<true>(L, g2.src, wu, acc);
  __syncthreads();   // s_r / s_w visible; every wave is done with the ring's LDS
  // acc[q][cb][i]: route 16 cb + 4 g + i, output column 256 ob + 64 w + 16 q + c
  pf_combine<kPfQ, 4>(a, g2.wk, acc, s_r, s_w, (size_t)256 * g2.ob + 64 * w + c, 0, c, g, (uint8_t *)&L);
}

// The same for a short reduction (N <= 128 NKT): every k-tile's weights and
// activations are requested up front (one memory round trip per block instead
// of one per ring turn), then consumed in order as each stage lands.
template <int NKT>
struct PfShortLds {
  PfStage st[NKT];
};

template <int NKT>
__global__ __launch_bounds__(256, 2) void k_pf_gemm2_a8_short(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) PfShortLds<NKT> L;
  __shared__ int s_r[kPfTileRows];
  __shared__ float s_w[kPfTileRows];
  PfG2 g2;
  if (!pf_g2_setup(a, g2, s_r, s_w)) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const PfSrc &src = g2.src;
  PfW wt[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; kt++) {
    pf_load_w(wt[kt], src, kt, wu, l);
    pf_issue_b(L.st[kt], src, kt, wu, l);
  }
  v4f acc[kPfQ][4];
  zero_acc<kPfQ, 4>(acc);
#pragma unroll
  for (int kt = 0; kt < NKT; kt++) {
    // stage kt has landed once the kPfLoads loads of each later stage are all
    // that may still be in flight (loads complete in order)
    if constexpr (true) {
      switch (NKT - 1 - kt) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<kPfLoads>(); break;
        case 2: wait_vm<2 * kPfLoads>(); break;
        case 3: wait_vm<3 * kPfLoads>(); break;
        default: wait_vm<4 * kPfLoads>(); break;
      }
    }
    __builtin_amdgcn_s_barrier();
    v4i b[4][2];
    int sb[4];
    pf_read_b(b, sb, L.st[kt], l);
    __builtin_amdgcn_s_setprio(1);
    // only the last k-tile can be partial (NKT = N / 128 rounded up)
    if (kt < NKT - 1 || (kt + 1) * 128 <= src.kbytes) pf_mma<true, true>(wt[kt], b, sb, kt, src.kbytes, src.nrb, l, acc);
    else pf_mma<true, false>(wt[kt], b, sb, kt, src.kbytes, src.nrb, l, acc);
    __builtin_amdgcn_s_setprio(0);
  }
  __syncthreads();   // s_r / s_w visible; every wave is done with the ring's LDS
  pf_combine<kPfQ, 4>(a, g2.wk, acc, s_r, s_w, (size_t)256 * g2.ob + 64 * w + c, 0, c, g, (uint8_t *)&L);
}

// ------------------------------------ GEMM2, resident intermediate rows
// The down GEMM of the route-buffer combine as blocks of (64-route tile, run
// of a.obg 256-column output blocks).  The tile's MXFP8 intermediate rows and
// scales (all NKT k-tiles of N <= 128 NKT) go into LDS once per block, in the
// stage layout of the other W4A8 kernels; each wave then streams its weights
// through a register ring of NKT k-tiles that runs on across the output
// blocks of the run, so the next block's weights are in flight while the
// current one is multiplied and its route-buffer rows are stored.  A block of
// one output block paid the intermediate rows' load, the perm lookups and the
// ring's first round trip for five k-tiles of MFMAs; here it pays them once
// per run.  The LDS rows are read-only after the first barrier and the
// combine stages through per-wave regions, so the loop has no barrier.
template <int NKT>
struct PfResLds {
  PfStage st[NKT];
  uint8_t rb[4 * 16 * (32 * kPfQ + 16)];   // per-wave route-buffer staging (pf_store_rb)
};

// Weight and scale loads of row tiles rt0 .. rt0 + 3 (wave-uniform) for
// k-tile kt.  vd / vs: the lane's byte offsets inside a k-tile's data / scales
// (l * 16 and l & ~3), or past the buffer's range (zeros without memory
// traffic) for loads past the run or lanes past the reduction length; the
// k-tile's own offset goes into the scalar offset, so one lane offset serves
// every k-tile.
// son: the scale loads are in range.  skip: this k-tile's scale bytes are in
// the dword of its run's first k-tile, which the caller keeps: no scale load
// (pf_res_loads counts the loads of a slot).
template <bool NT = false>   // NT: non-temporal weight loads
__device__ __forceinline__ void pf_load_w_rt(PfW &r, const PfSrc &src, uint32_t rt0, int kt, uint32_t vd, bool son,
                                             bool skip, int l) {
  const uint32_t vs = son ? (mx_soff(kt, l, src.kbytes >> 7) & ~3u) : 0x80000000u;
#pragma unroll
  for (int q = 0; q < kPfQ; q++) {
    const uint32_t so = (rt0 + q) * src.wstep + (uint32_t)kt * 1024u;
    r.a[q] = NT ? buf_load16_nt(src.wb, vd, so) : buf_load16(src.wb, vd, so);
    if (!skip) r.sa[q] = buf_load4(src.sb, vs, (rt0 + q) * src.sstep);
  }
}

// Loads of ring slot kt (kt < 0: of every slot) for a reduction of NKF whole
// k-tiles in NKT: the weights, and the scales outside a run's later k-tiles.
template <int NKT, int NKF>
__host__ __device__ constexpr int pf_res_loads(int kt) {
  if (kt >= 0) return kPfQ * ((kt < (NKF & ~3) && (kt & 3) != 0) ? 1 : 2);
  int n = 0;
  for (int k = 0; k < NKT; k++) n += pf_res_loads<NKT, NKF>(k);
  return n;
}

// One block's work.
// NT: non-temporal weight loads, for blocks whose expert fits its one 64-route
// tile (its weights are then read once; every tile non-temporal measured
// 198 -> 211 us at the Zipf-skewed 4096-token batch, this choice 189.5 -> 185.0).
template <int NKT, bool LASTFULL, bool NT>
__device__ __forceinline__ void pf_res_body(PfResLds<NKT> &L, const GemmArgs &a, const PfWork &wk, int *s_r,
                                            float *s_w) {
  const int K = a.K, N = a.N, nob = K / 256, obg = a.obg;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int ob0 = wk.sub * obg, ob1 = min(nob, ob0 + obg);
  PfSrc src;
  src.wstep = (uint32_t)(16 * (N / 2));
  src.sstep = (uint32_t)(16 * (N / 32));
  src.nrt = kPfRT;
  src.wb = make_buf(a.w2 + (size_t)wk.e * K * (N / 2), (uint32_t)((size_t)K * (N / 2)));
  src.sb = make_buf(a.s2 + (size_t)wk.e * K * (N / 32), (uint32_t)((size_t)K * (N / 32)));
  src.kbytes = N;
  src.nrb = __builtin_amdgcn_readfirstlane((wk.rows + 15) / 16);
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
  // the tile's intermediate rows (every k-tile), then the first output block's weights
#pragma unroll
  for (int kt = 0; kt < NKT; kt++) pf_issue_b(L.st[kt], src, kt, wu, l);
  // lane offsets inside a k-tile.  The lanes of a partial last k-tile past N
  // load the next row tile's bytes (or zeros past the expert): E2M1 codes are
  // finite, and the MFMA step zeroes their activations and scales.
  const uint32_t kOut = 0x80000000u, vd = (uint32_t)(l * 16);
  // whole k-tiles of the reduction; those in runs of four (scale bytes of a
  // run in one dword a lane: loaded with the run's first k-tile)
  constexpr int NKF = LASTFULL ? NKT : NKT - 1, G4 = NKF & ~3;
  PfW ring[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; kt++)
    pf_load_w_rt<NT>(ring[kt], src, (uint32_t)(16 * ob0 + 4 * wu), kt, vd, true, kt < G4 && (kt & 3) != 0, l);
  // the rows have landed once only the weight loads may be in flight; then
  // every wave's share (and s_r / s_w) is visible
  wait_vm<pf_res_loads<NKT, NKF>(-1)>();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  for (int ob = ob0; ob < ob1; ob++) {
    // the epilogue's route rows and weights are re-read from LDS in each pass: hoisted out
    // of the loop as addresses, they would stay live in registers next to the ring and spill
    asm volatile("" ::: "memory");
    const bool next = ob + 1 < ob1;
    const uint32_t rtn = (uint32_t)(16 * (next ? ob + 1 : ob) + 4 * wu);
    const uint32_t nd = next ? vd : kOut;
    v4f acc[kPfQ][4];
    zero_acc<kPfQ, 4>(acc);
    uint32_t srun[kPfQ];   // this output block's scale dwords of the current run of four k-tiles
#pragma unroll
    for (int kt = 0; kt < NKT; kt++) {
      // slot kt holds this block's k-tile kt once at most the loads of the NKT - 1
      // slots issued after it are in flight (stores in between only add to the count)
      constexpr int TOT = pf_res_loads<NKT, NKF>(-1);
      if (kt < G4 && (kt & 3) != 0) wait_vm<TOT - kPfQ>();
      else wait_vm<TOT - 2 * kPfQ>();
      v4i b[4][2];
      int sb[4];
      pf_read_b(b, sb, L.st[kt], l);
      const bool run = kt < G4;
      if (run && (kt & 3) == 0) {
#pragma unroll
        for (int q = 0; q < kPfQ; q++) srun[q] = ring[kt].sa[q];   // kept past the slot's reload
      }
      __builtin_amdgcn_s_setprio(1);
      if (kt < NKT - 1 || LASTFULL) pf_mma<true, true>(ring[kt], b, sb, kt, N, src.nrb, l, acc, run ? srun : nullptr);
      else pf_mma<true, false>(ring[kt], b, sb, kt, N, src.nrb, l, acc, run ? srun : nullptr);
      __builtin_amdgcn_s_setprio(0);
      // the next output block's k-tile kt into the slot the MFMAs above read; issued after
      // them (hoisted above, the loads would need a second register set and spill), and no
      // step is interleaved with the next for the same reason
      __builtin_amdgcn_sched_barrier(0);
      pf_load_w_rt<NT>(ring[kt], src, rtn, kt, nd, next, run && (kt & 3) != 0, l);
      __builtin_amdgcn_sched_barrier(0);
    }
    // acc[q][cb][i]: route 16 cb + 4 g + i, output column 256 ob + 64 w + 16 q + c
    pf_store_rb<kPfQ, 4>(a, wk, acc, s_r, s_w, (size_t)256 * ob + 64 * w, c, g, L.rb);
  }
}

template <int NKT, bool LASTFULL>
__global__ __launch_bounds__(256, 2) void k_pf_gemm2_a8_res(GemmArgs a) {
  __shared__ PfResLds<NKT> L;
  __shared__ int s_r[kPfTileRows];
  __shared__ float s_w[kPfTileRows];
  const int nob = a.K / 256;
  const PfWork wk = pf_work(a, (nob + a.obg - 1) / a.obg, false);
  if (!wk.valid) return;
  if (wk.single) pf_res_body<NKT, LASTFULL, true>(L, a, wk, s_r, s_w);
  else pf_res_body<NKT, LASTFULL, false>(L, a, wk, s_r, s_w);
}

static int pf_grid(int grid_tiles, int nsub) { return (grid_tiles * nsub + 7) / 8 * 8; }

hipError_t launch_pf_gemm1(const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  if (a.tile_rows == kPfWideRows)
    hipLaunchKernelGGL(k_pf_gemm1_a8w, dim3(pf_grid(grid_tiles, (a.N + 127) / 128)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_pf_gemm1_a8, dim3(pf_grid(grid_tiles, (a.N + 127) / 128)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int NKT>
static void launch_pf_gemm2_res(const GemmArgs &a, dim3 grid, hipStream_t s) {
  if (a.N == 128 * NKT) hipLaunchKernelGGL((k_pf_gemm2_a8_res<NKT, true>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((k_pf_gemm2_a8_res<NKT, false>), grid, dim3(256), 0, s, a);
}

hipError_t launch_pf_gemm2(const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  const int nkt = (a.N + 127) / 128;
  if (a.deterministic && a.obg > 0 && nkt <= 5) {   // the route-buffer combine: resident intermediate rows
    const dim3 grid(pf_grid(grid_tiles, (a.K / 256 + a.obg - 1) / a.obg));
    switch (nkt) {
      case 1: launch_pf_gemm2_res<1>(a, grid, s); break;
      case 2: launch_pf_gemm2_res<2>(a, grid, s); break;
      case 3: launch_pf_gemm2_res<3>(a, grid, s); break;
      case 4: launch_pf_gemm2_res<4>(a, grid, s); break;
      default: launch_pf_gemm2_res<5>(a, grid, s); break;
    }
    return hipGetLastError();
  }
  const dim3 grid(pf_grid(grid_tiles, a.K / 256)), block(256);
  switch ((a.N + 127) / 128) {
    case 1: hipLaunchKernelGGL(k_pf_gemm2_a8_short<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_pf_gemm2_a8_short<2>, grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL(k_pf_gemm2_a8_short<3>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_pf_gemm2_a8_short<4>, grid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL(k_pf_gemm2_a8_short<5>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(k_pf_gemm2_a8, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

// ================================================================ W4A16 / W3A16
//
// The same 64-route tiles for NVFP4 and NF3 experts with bf16 activations.
// Wave w owns weight row tiles 2w, 2w + 1 against all 64 routes, so each
// weight element is dequantised once per tile, one 8-column step at a time
// (E2M1 x E4M3, or NF3 codebook x E4M3, to bf16; exact for E2M1), and feeds 4
// bf16 MFMAs: 4 steps x 2 row tiles x 4 route blocks per k-tile.  A wave's
// weights are used by that wave only, so they skip LDS: buffer loads put each
// k-tile's weight and scale bytes (16 / 12 and 2 / 1 per lane, MFMA lane
// order) straight into a ring of kPf16Stages register sets.  The activations
// are shared by the four waves and go through an LDS ring of the same depth:
// a stage holds the 64 routes' bf16 slices of one 128-column k-tile (256 bytes
// each, 16-byte chunks XOR-swizzled by route (pf16_slot)) loaded directly to LDS.
namespace {

constexpr int kPf16Stages = 3;
// vector-memory operations of one wave per stage: 2 weight tiles, 2 scale
// loads, 4 activation chunks (both formats)
constexpr int kPf16Loads = 8;

struct Pf16Stage {
  uint8_t B[kPfTileRows][256];
};

struct __attribute__((aligned(16))) Pf16Lds {
  Pf16Stage st[kPf16Stages];
};

__device__ __forceinline__ void wait16_stages(int stages) {
  if (stages >= 2) wait_vm<2 * kPf16Loads>();
  else if (stages == 1) wait_vm<kPf16Loads>();
  else wait_vm<0>();
}

struct Pf16Src {
  Buf wb, sb;                  // the block's 8 weight row tiles / their scales
  uint32_t wstep, sstep;       // bytes per row tile (data / scales)
  const uint16_t *brow[4];     // this lane's activation rows of its four B chunks
  int kcols;                   // reduction length (columns)
};

// A wave's weight operands of one k-tile: row tiles 2w + q.  The scales come
// as the aligned dword holding this lane's 2 (NVFP4) or 1 (NF3) bytes: a
// narrower load would be zero-extended where the ring is carried round the
// loop, which makes the compiler wait for every load in flight there.
struct Pf16W {
  uint32_t a[2][4];   // NVFP4 4 dwords, NF3 3 dwords (+1 zero)
  uint32_t sc[2];
};

// This lane's scale bits (low 16 for NVFP4, low 8 for NF3) in its scale dword.
template <int WF>
__device__ __forceinline__ uint32_t pf16_scale(uint32_t dw, int l) {
  return WF == W_NVFP4 ? dw >> (16 * (l & 1)) : dw >> (8 * (l & 3));
}

// Weight and scale loads of wave w for k-tile kt.  Lanes whose 32-column group
// lies past the reduction length read past the buffer's range: zeros, and no
// memory traffic.
// The weight data goes through non-temporal loads (hybrid prefill at 2048
// tokens: 632.5 -> 626.6 us; level at the NVFP4 one; the W4A8 kernels, whose
// hot experts' tiles share weight lines, measured slower with them).
template <int WF>
__device__ __forceinline__ void pf16_load_w(Pf16W &r, const Pf16Src &src, int kt, int w, int l) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  const bool in = kt * 128 + 32 * (l >> 4) < src.kcols;
  const uint32_t vd = in ? (uint32_t)(kt * 64 * U + l * U) : 0x80000000u;
  const uint32_t vs = in ? (uint32_t)(kt * 64 * SU + ((l * SU) & ~3)) : 0x80000000u;
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const uint32_t rt = (uint32_t)(2 * w + q);
    if constexpr (WF == W_NVFP4) {
      const v4i v = buf_load16_nt(src.wb, vd, rt * src.wstep);
      r.a[q][0] = v[0]; r.a[q][1] = v[1]; r.a[q][2] = v[2]; r.a[q][3] = v[3];
      r.sc[q] = buf_load4(src.sb, vs, rt * src.sstep);
    } else {
      const v3i v = buf_load12_nt(src.wb, vd, rt * src.wstep);
      r.a[q][0] = v[0]; r.a[q][1] = v[1]; r.a[q][2] = v[2]; r.a[q][3] = 0;
      r.sc[q] = buf_load4(src.sb, vs, rt * src.sstep);
    }
  }
}

// LDS slot of 16-byte chunk k (8 bf16 columns) of a route row (256 bytes, one
// k-tile), and its inverse: XOR-swizzled by route % 16 so that the 16 routes a
// read touches spread over the banks, and bit 3 flipped for chunks 4..7 and
// 12..15, so that the two 16-lane quarters of a read (chunk groups g and g ^ 1)
// fall in different halves of the row.  (Swizzled by the route alone, the
// 16-bit up/gate GEMM's reads took 3.8e7 bank-conflict cycles at the 2048-token
// NVFP4 prefill, about 4 a read; with the bit flipped, none.)
__device__ __forceinline__ int pf16_slot(int k, int r) { return (k ^ (r & 15)) ^ (((k >> 2) & 1) << 3); }
__device__ __forceinline__ int pf16_chunk(int slot, int r) {
  const int y = slot ^ (r & 15);
  return y ^ (((y >> 2) & 1) << 3);
}

// Activation chunks 4w .. 4w+3 of k-tile kt (1 KB each: 4 routes x 256 bytes;
// lane l -> route 4j + l/16, LDS slot l % 16 holding the chunk pf16_chunk
// gives).  Lanes past the reduction length load column 0.
__device__ __forceinline__ void pf16_issue_b(Pf16Stage &S, const Pf16Src &src, int kt, int w, int l) {
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int r = 4 * (4 * w + j) + (l >> 4), cg = pf16_chunk(l & 15, r), col = kt * 128 + 8 * cg;
    dma16(src.brow[j] + (col < src.kcols ? col : 0), &S.B[4 * (4 * w + j)][0]);
  }
}

// The 64 routes' activations of a landed stage, read and waited for in one
// asm statement (invisible to the compiler's direct-to-LDS bookkeeping; a
// wait in a later statement would let the compiler copy registers still in
// flight).  b[s][cb]: step s, route block cb.
__device__ __forceinline__ void pf16_read_b(v4i (&b)[4][4], const Pf16Stage &S, int l) {
  const int c = l & 15, g = l >> 4;
  const uint8_t *brow = &S.B[c][0];   // + 16 rows (4096 bytes) per route block
  uint32_t vb[4];
#pragma unroll
  for (int s = 0; s < 4; s++) vb[s] = lds_addr(brow + 16 * pf16_slot(4 * g + s, c));
  asm volatile(
      "ds_read_b128 %0, %16\n"
      "ds_read_b128 %1, %16 offset:4096\n"
      "ds_read_b128 %2, %16 offset:8192\n"
      "ds_read_b128 %3, %16 offset:12288\n"
      "ds_read_b128 %4, %17\n"
      "ds_read_b128 %5, %17 offset:4096\n"
      "ds_read_b128 %6, %17 offset:8192\n"
      "ds_read_b128 %7, %17 offset:12288\n"
      "ds_read_b128 %8, %18\n"
      "ds_read_b128 %9, %18 offset:4096\n"
      "ds_read_b128 %10, %18 offset:8192\n"
      "ds_read_b128 %11, %18 offset:12288\n"
      "ds_read_b128 %12, %19\n"
      "ds_read_b128 %13, %19 offset:4096\n"
      "ds_read_b128 %14, %19 offset:8192\n"
      "ds_read_b128 %15, %19 offset:12288\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(b[0][0]), "=&v"(b[0][1]), "=&v"(b[0][2]), "=&v"(b[0][3]), "=&v"(b[1][0]), "=&v"(b[1][1]),
        "=&v"(b[1][2]), "=&v"(b[1][3]), "=&v"(b[2][0]), "=&v"(b[2][1]), "=&v"(b[2][2]), "=&v"(b[2][3]),
        "=&v"(b[3][0]), "=&v"(b[3][1]), "=&v"(b[3][2]), "=&v"(b[3][3])
      : "v"(vb[0]), "v"(vb[1]), "v"(vb[2]), "v"(vb[3])
      : "memory");
}

// 32 bf16 MFMAs of one k-tile (4 steps x 2 row tiles x 4 route blocks); each
// dequantised weight operand feeds 4 MFMAs.  Scales are decoded once per row
// tile (NF3: its scaled magnitude table).  Columns past the reduction length
// (FULL: none): the weights there are zero (their scales load as 0) and the
// activations are zeroed.  SWAP: activations as the A operand.
// CVT: decode the scales with the one-instruction E4M3 convert (kernels with
// the registers for it; in the 64-route ring kernels it raised the schedule to
// about 300 VGPRs).  H: fp16 activations and fp16 weight operands (fp16 MFMA).
template <int WF, bool SWAP, bool FULL, bool CVT = false, bool H = false>
__device__ __forceinline__ void pf16_mma(const Pf16W &wt, const v4i (&b)[4][4], int kt, int kcols, int l,
                                         v4f (*acc)[4]) {
  const bool gin = FULL || kt * 128 + 32 * (l >> 4) < kcols;
  if constexpr (H) {
    v2h sp[2];
    uint32_t t01[2] = {0u, 0u}, t23[2] = {0u, 0u};
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const uint32_t sc = pf16_scale<WF>(wt.sc[q], l);
      if constexpr (WF == W_NVFP4) sp[q] = e4m3x2_h(sc & 0xFFFFu);
      else nf3_tables_h(e4m3_f32(sc & 0xFFu), t01[q], t23[q]);
    }
#pragma unroll
    for (int s = 0; s < 4; s++) {
      v8h bop[4];
#pragma unroll
      for (int cb = 0; cb < 4; cb++) bop[cb] = __builtin_bit_cast(v8h, gin ? b[s][cb] : v4i{0, 0, 0, 0});
#pragma unroll
      for (int q = 0; q < 2; q++) {
        v8h aop;
        if constexpr (WF == W_NVFP4) aop = nvfp4_step_h(wt.a[q][s], s < 2 ? sp[q].x : sp[q].y);
        else aop = nf3_step_h(s < 2 ? wt.a[q][0] : wt.a[q][1], wt.a[q][2], s, t01[q], t23[q]);
#pragma unroll
        for (int cb = 0; cb < 4; cb++)
          acc[q][cb] = SWAP ? mfma_f16(bop[cb], aop, acc[q][cb]) : mfma_f16(aop, bop[cb], acc[q][cb]);
      }
    }
    return;
  }
  float slo[2] = {0.f, 0.f}, shi[2] = {0.f, 0.f};
  uint32_t t01[2] = {0u, 0u}, t23[2] = {0u, 0u};
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const uint32_t sc = pf16_scale<WF>(wt.sc[q], l);
    if constexpr (WF == W_NVFP4) {
      slo[q] = CVT ? e4m3_f32(sc & 0xFFu) : e4m3_f32_branched(sc & 0xFFu);
      shi[q] = CVT ? e4m3_f32((sc >> 8) & 0xFFu) : e4m3_f32_branched((sc >> 8) & 0xFFu);
    } else {
      nf3_tables(CVT ? e4m3_f32(sc & 0xFFu) : e4m3_f32_branched(sc & 0xFFu), t01[q], t23[q]);
    }
  }
#pragma unroll
  for (int s = 0; s < 4; s++) {
    v8bf bop[4];
#pragma unroll
    for (int cb = 0; cb < 4; cb++) bop[cb] = __builtin_bit_cast(v8bf, gin ? b[s][cb] : v4i{0, 0, 0, 0});
#pragma unroll
    for (int q = 0; q < 2; q++) {
      v8bf aop;
      if constexpr (WF == W_NVFP4) aop = nvfp4_step(wt.a[q][s], s < 2 ? slo[q] : shi[q]);
      else aop = nf3_step_rc(s < 2 ? wt.a[q][0] : wt.a[q][1], wt.a[q][2], s, t01[q], t23[q]);
#pragma unroll
      for (int cb = 0; cb < 4; cb++)
        acc[q][cb] = SWAP ? mfma_bf16(bop[cb], aop, acc[q][cb]) : mfma_bf16(aop, bop[cb], acc[q][cb]);
    }
  }
}

// One k-tile (R = kt % ST).  After the barrier that proves stage kt landed for
// every wave (and that every wave is done with stage kt - 1), k-tile
// kt + ST - 1 is issued: its activations into stage kt - 1's LDS slot, its
// weights into the register set that held k-tile kt - 1.  Then stage kt is
// read and multiplied with register set R.  WAITN: loads allowed in flight at
// the wait (kPf16Loads when k-tile kt + 1 exists, else 0; -1: decided at run
// time); ISSUE: whether k-tile kt + ST - 1 exists (-1: at run time).  Where
// both are known at compile time the compiler's own bookkeeping of the ring
// registers stays exact; at run time it falls back to full waits.
template <int WF, bool SWAP, int R, int WAITN, int ISSUE>
__device__ __forceinline__ void pf16_step(Pf16Lds &L, const Pf16Src &src, Pf16W (&ring)[kPf16Stages], int kt,
                                          int nkt, int w, v4f (*acc)[4]) {
  constexpr int ST = kPf16Stages;
  const int l = threadIdx.x & 63;
  if constexpr (WAITN == kPf16Loads) wait_vm<kPf16Loads>();
  else if constexpr (WAITN == 0) wait_vm<0>();
  else wait16_stages(min(ST - 2, nkt - 1 - kt));   // stage kt has landed
  __builtin_amdgcn_s_barrier();
  const int kn = kt + ST - 1;
  if (ISSUE == 1 || (ISSUE == -1 && kn < nkt)) {
    // one branch-free load sequence: two paths of loads here would make the
    // compiler's bookkeeping of the ring registers conservative (a full wait)
    pf16_load_w<WF>(ring[(R + ST - 1) % ST], src, kn, w, l);
    pf16_issue_b(L.st[kn % ST], src, kn, w, l);
  }
  v4i b[4][4];
  pf16_read_b(b, L.st[kt % ST], l);
  // raised issue priority around the MFMAs as for the W4A8 kernels (measured:
  // faster for the up/gate GEMM, slower for the down GEMM's short k-loops)
  if (!SWAP) __builtin_amdgcn_s_setprio(1);
  // (the run-time check is kept in the steady loop too: its compile-time form,
  // as in pf_step, measured 2 % slower here)
  if ((kt + 1) * 128 <= src.kcols) pf16_mma<WF, SWAP, true>(ring[R], b, kt, src.kcols, l, acc);
  else pf16_mma<WF, SWAP, false>(ring[R], b, kt, src.kcols, l, acc);
  if (!SWAP) __builtin_amdgcn_s_setprio(0);
}

// A k-loop of exactly NKT k-tiles (NKT <= 4), straight-line.
template <int WF, bool SWAP, int NKT>
__device__ __forceinline__ void pf16_kloop_fixed(Pf16Lds &L, const Pf16Src &src, Pf16W (&ring)[kPf16Stages], int w,
                                                 v4f (*acc)[4]) {
  constexpr int ST = kPf16Stages;
  static_assert(NKT >= 1 && NKT <= 4, "short k-loops");
  pf16_step<WF, SWAP, 0, (1 < NKT) ? kPf16Loads : 0, (ST - 1 < NKT) ? 1 : 0>(L, src, ring, 0, NKT, w, acc);
  if constexpr (NKT > 1)
    pf16_step<WF, SWAP, 1, (2 < NKT) ? kPf16Loads : 0, (ST < NKT) ? 1 : 0>(L, src, ring, 1, NKT, w, acc);
  if constexpr (NKT > 2)
    pf16_step<WF, SWAP, 2, (3 < NKT) ? kPf16Loads : 0, (ST + 1 < NKT) ? 1 : 0>(L, src, ring, 2, NKT, w, acc);
  if constexpr (NKT > 3)
    pf16_step<WF, SWAP, 0, (4 < NKT) ? kPf16Loads : 0, (ST + 2 < NKT) ? 1 : 0>(L, src, ring, 3, NKT, w, acc);
}

// w: the wave index, wave-uniform (scalar), so stage and weight offsets stay
// scalar.  Short reductions run a straight-line loop; long ones whole ring
// turns while every step is steady, then at most ST + 1 closing steps.
template <int WF, bool SWAP>
__device__ __forceinline__ void pf16_kloop(Pf16Lds &L, const Pf16Src &src, int w, v4f (*acc)[4]) {
  constexpr int ST = kPf16Stages;
  static_assert(ST == 3, "the k-loop is unrolled by the ring depth");
  const int l = threadIdx.x & 63;
  const int nkt = (src.kcols + 127) / 128;
  Pf16W ring[ST];
  // stages 0 .. ST - 2 are issued even past the last k-tile (weights then load
  // as zeros without traffic, activations from column 0): a fixed load count
  // keeps the compiler's bookkeeping of the ring registers exact
#pragma unroll
  for (int s = 0; s < ST - 1; s++) {
    pf16_load_w<WF>(ring[s], src, s, w, l);
    pf16_issue_b(L.st[s], src, s, w, l);
  }
  if (nkt <= 4) {
    if (nkt == 4) pf16_kloop_fixed<WF, SWAP, 4>(L, src, ring, w, acc);
    else if (nkt == 3) pf16_kloop_fixed<WF, SWAP, 3>(L, src, ring, w, acc);
    else if (nkt == 2) pf16_kloop_fixed<WF, SWAP, 2>(L, src, ring, w, acc);
    else pf16_kloop_fixed<WF, SWAP, 1>(L, src, ring, w, acc);
    return;
  }
  int kt = 0;
  for (; kt + 2 * ST - 1 <= nkt; kt += ST) {   // k-tiles kt .. kt + 2 steady: kt + 2 + ST - 1 < nkt
    pf16_step<WF, SWAP, 0, kPf16Loads, 1>(L, src, ring, kt, nkt, w, acc);
    pf16_step<WF, SWAP, 1, kPf16Loads, 1>(L, src, ring, kt + 1, nkt, w, acc);
    pf16_step<WF, SWAP, 2, kPf16Loads, 1>(L, src, ring, kt + 2, nkt, w, acc);
  }
  if (kt < nkt) pf16_step<WF, SWAP, 0, -1, -1>(L, src, ring, kt, nkt, w, acc);
  if (kt + 1 < nkt) pf16_step<WF, SWAP, 1, -1, -1>(L, src, ring, kt + 1, nkt, w, acc);
  if (kt + 2 < nkt) pf16_step<WF, SWAP, 2, -1, -1>(L, src, ring, kt + 2, nkt, w, acc);
  if (kt + 3 < nkt) pf16_step<WF, SWAP, 0, -1, -1>(L, src, ring, kt + 3, nkt, w, acc);
  if (kt + 4 < nkt) pf16_step<WF, SWAP, 1, -1, -1>(L, src, ring, kt + 4, nkt, w, acc);
}

}  // namespace

// ---------------------------------------------------------------- GEMM1 (A16)
// One tier's expert tensors.
struct PfTier {
  const uint8_t *w13, *s13, *w2, *s2;
  const float *g13, *g2;
};

__device__ __forceinline__ PfTier pf_tier(const GemmArgs &a, int tier) {
  PfTier t;
  t.w13 = tier ? a.w13b : a.w13;
  t.s13 = tier ? a.s13b : a.s13;
  t.w2 = tier ? a.w2b : a.w2;
  t.s2 = tier ? a.s2b : a.s2;
  t.g13 = tier ? a.g13b : a.g13;
  t.g2 = tier ? a.g2b : a.g2;
  return t;
}

// Work item of a launch that covers both tiers: tier 0's items, then tier 1's,
// each in its own order (as pf_work), all numbered XCD-major together.
__device__ __forceinline__ PfWork pf_work_tiers(const GemmArgs &a, int nsub, bool sub_major, int *tier) {
  PfWork w;
  const int n0 = a.tier_tiles[1] - a.tier_tiles[0], n1 = a.tier_tiles[3] - a.tier_tiles[2];
  const int items0 = n0 * nsub, items = items0 + n1 * nsub, per = (items + 7) >> 3;
  const int b = blockIdx.x, slot = b >> 3, item = (b & 7) * per + slot;
  w.valid = slot < per && item < items;
  if (!w.valid) return w;
  const int t1 = item >= items0 ? 1 : 0, local = t1 ? item - items0 : item, ntiles = t1 ? n1 : n0;
  const int tbeg = a.tier_tiles[2 * t1];
  const int t = sub_major ? local % ntiles : local / nsub;
  w.sub = sub_major ? local / ntiles : local - t * nsub;
  const int u = a.tile_u[tbeg + t];
  w.e = u - (t1 ? a.u_base_b : 0);
  w.p0 = a.off[u] + a.tile_row0[tbeg + t];
  w.rows = min(a.tile_rows, a.off[u + 1] - w.p0);
  w.single = a.off[u + 1] - a.off[u] <= a.tile_rows;
  *tier = t1;
  return w;
}

// Block: w13 row tiles 8 hb .. +7 = up and gate of intermediate columns 64 hb .. +63.
template <int WF>
__device__ __forceinline__ void pf16_gemm1_body(const GemmArgs &a, const PfWork &wk, const PfTier &T, Pf16Lds &L) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  const int K = a.K, N = a.N, N1 = a.N1;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int hb = wk.sub, groups = K / 32;
  Pf16Src src;
  src.wstep = (uint32_t)(16 * groups * U);
  src.sstep = (uint32_t)(16 * groups * SU);
  src.wb = make_buf(T.w13 + (size_t)wk.e * (2 * N1) * groups * U + (size_t)(8 * hb) * src.wstep, 8 * src.wstep);
  src.sb = make_buf(T.s13 + (size_t)wk.e * (2 * N1) * groups * SU + (size_t)(8 * hb) * src.sstep, 8 * src.sstep);
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
  const float g13 = T.g13 ? T.g13[wk.e] : 1.0f;
#pragma unroll
  for (int cb = 0; cb < 4; cb++) {
    const int row = 16 * cb + c;
    if (row < wk.rows) {
      const size_t p = (size_t)(wk.p0 + row);
      // router weight on the input: GEMM1 is linear, so it scales the accumulators
      const float gs = g13 * (a.w_on_input ? a.topk_w[a.perm[p]] : 1.0f);
      uint2 v;
      if (a.act == ACT_RELU2) {
        // ReLU^2 without the multiply: the up and gate halves' rows give columns n and N1 + n
#pragma unroll
        for (int half = 0; half < 2; half++) {
          v.x = pack_bf16x2(relu2(acc[half][cb][0] * gs), relu2(acc[half][cb][1] * gs));
          v.y = pack_bf16x2(relu2(acc[half][cb][2] * gs), relu2(acc[half][cb][3] * gs));
          *(uint2 *)(a.hb + p * N + half * N1 + 64 * hb + 16 * w + 4 * g) = v;
        }
        continue;
      }
      float h[4];
#pragma unroll
      for (int i = 0; i < 4; i++) h[i] = silu_clamped(acc[1][cb][i] * gs, acc[0][cb][i] * gs, a.limit, a.has_limit, a.alpha, a.beta, a.act);
      v.x = pack_bf16x2(h[0], h[1]);
      v.y = pack_bf16x2(h[2], h[3]);
      *(uint2 *)(a.hb + p * N + 64 * hb + 16 * w + 4 * g) = v;
    }
  }
}

template <int WF>
__global__ __launch_bounds__(256) void k_pf_gemm1_a16(GemmArgs a) {
  __shared__ Pf16Lds L;
  const PfWork wk = pf_work(a, a.N1 / 64, false);
  if (!wk.valid) return;
  pf16_gemm1_body<WF>(a, wk, pf_tier(a, 0), L);
}

// Both tiers in one launch: each block runs its tier's format.
__global__ __launch_bounds__(256) void k_pf_gemm1_a16_tiers(GemmArgs a) {
  __shared__ Pf16Lds L;
  int tier = 0;
  const PfWork wk = pf_work_tiers(a, a.N1 / 64, false, &tier);
  if (!wk.valid) return;
  const PfTier T = pf_tier(a, tier);
  if ((tier ? a.fmt_b : a.fmt_a) == W_NVFP4) pf16_gemm1_body<W_NVFP4>(a, wk, T, L);
  else pf16_gemm1_body<W_NF3>(a, wk, T, L);
}

// ------------------------------------------ GEMM1 (A16), 128-route tiles
// The W4A16 / W3A16 up/gate GEMM on the up/gate table of 128-route tiles: the
// same block of 8 weight row tiles (up and gate of 64 intermediate columns,
// row tiles 2w, 2w + 1 for wave w) against up to 128 routes.  Each wave
// dequantises its two row tiles' k-tile once and feeds the operands to the
// MFMAs of both 64-route halves, half the dequantisation per MFMA of 64-route
// tiles; where every expert's routes fit one tile (the 2048-token NVFP4
// prefill: at most 95 routes an expert) each expert's weights are streamed
// once instead of once per 64-route tile, and the MFMAs of 16-route blocks
// holding only padding are skipped.  Activations: a 2-stage LDS ring of 32 KB
// stages (128 routes x 256 bytes of a bf16 k-tile, 16-byte chunks swizzled by
// route as on 64-route tiles); weights: a 2-deep register ring; one
// k-tile of lookahead (two blocks per CU).  K % 256 == 0 (every plan's).
constexpr int kPw16Stages = 2;

struct Pw16Stage {
  uint8_t B[kPfWideRows][256];
};

struct __attribute__((aligned(16))) Pw16Lds {
  Pw16Stage st[kPw16Stages];
};

struct Pw16Src {
  Pf16Src w;                      // the block's weight row tiles (wb, sb, wstep, sstep, kcols)
  const uint8_t *xb;              // bf16 activations (uniform base)
  uint32_t brow[8];               // byte offsets of this lane's activation rows of its 8 chunks
};

// Activation chunks 8w .. 8w+7 of k-tile kt (1 KB each: 4 routes x 256 bytes;
// lane l -> route 4 (8w + j) + l / 16, LDS slot l % 16 holding the chunk
// pf16_chunk gives).
__device__ __forceinline__ void pw16_issue_b(Pw16Stage &S, const Pw16Src &src, int kt, int w, int l) {
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int r = 4 * (8 * w + j) + (l >> 4), cg = pf16_chunk(l & 15, r);
    dma16(src.xb + (src.brow[j] + (uint32_t)(kt * 256 + 16 * cg)), &S.B[4 * (8 * w + j)][0]);
  }
}

// The wave's two row tiles of one k-tile as bf16 MFMA operands: aop[q][s] =
// 8 columns of step s (scales decoded once per row tile).
template <int WF>
__device__ __forceinline__ void pw16_deq(const Pf16W &wt, int l, v8bf (&aop)[2][4]) {
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const uint32_t sc = pf16_scale<WF>(wt.sc[q], l);
    if constexpr (WF == W_NVFP4) {
      const float slo = e4m3_f32(sc & 0xFFu), shi = e4m3_f32((sc >> 8) & 0xFFu);
#pragma unroll
      for (int st = 0; st < 4; st++) aop[q][st] = nvfp4_step(wt.a[q][st], st < 2 ? slo : shi);
    } else {
      uint32_t t01, t23;
      nf3_tables(e4m3_f32(sc & 0xFFu), t01, t23);
#pragma unroll
      for (int st = 0; st < 4; st++) aop[q][st] = nf3_step_rc(st < 2 ? wt.a[q][0] : wt.a[q][1], wt.a[q][2], st, t01, t23);
    }
  }
}

// The MFMAs of half H (routes 64 H .. 64 H + 63) of a k-tile; route blocks
// past the tile's last route are skipped, one branch per block (8 MFMAs).
template <int H>
__device__ __forceinline__ void pw16_mma(const v8bf (&aop)[2][4], const v4i (&b)[4][4], int nrb, v4f (*acc)[8]) {
#pragma unroll
  for (int cb = 0; cb < 4; cb++) {
    if (4 * H + cb < nrb) {
#pragma unroll
      for (int st = 0; st < 4; st++) {
        const v8bf bop = __builtin_bit_cast(v8bf, b[st][cb]);
#pragma unroll
        for (int q = 0; q < 2; q++) acc[q][4 * H + cb] = mfma_bf16(aop[q][st], bop, acc[q][4 * H + cb]);
      }
    }
  }
}

// One k-tile (R = kt % 2): wait for stage kt (the only one in flight), barrier
// (every wave is also done with stage kt - 1), issue k-tile kt + 1 into the
// slots kt - 1 held (ISSUE), dequantise, then both halves of stage kt.
template <int WF, int R, bool ISSUE>
__device__ __forceinline__ void pw16_step(Pw16Lds &L, const Pw16Src &src, Pf16W (&ring)[kPw16Stages], int kt, int w,
                                          int nrb, v4f (*acc)[8]) {
  const int l = threadIdx.x & 63;
  wait_vm<0>();
  __builtin_amdgcn_s_barrier();
  if (ISSUE) {
    pf16_load_w<WF>(ring[R ^ 1], src.w, kt + 1, w, l);
    pw16_issue_b(L.st[R ^ 1], src, kt + 1, w, l);
  }
  v8bf aop[2][4];
  pw16_deq<WF>(ring[R], l, aop);
  v4i b[4][4];
  pf16_read_b(b, *(const Pf16Stage *)&L.st[R].B[0][0], l);
  __builtin_amdgcn_s_setprio(1);
  pw16_mma<0>(aop, b, nrb, acc);
  __builtin_amdgcn_s_setprio(0);
  if (nrb > 4) {
    pf16_read_b(b, *(const Pf16Stage *)&L.st[R].B[64][0], l);
    __builtin_amdgcn_s_setprio(1);
    pw16_mma<1>(aop, b, nrb, acc);
    __builtin_amdgcn_s_setprio(0);
  }
}

template <int WF>
__device__ __forceinline__ void pw16_gemm1_body(const GemmArgs &a, const PfWork &wk, const PfTier &T, Pw16Lds &L) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  const int K = a.K, N = a.N, N1 = a.N1;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int hb = wk.sub, groups = K / 32;
  Pw16Src src;
  src.w.wstep = (uint32_t)(16 * groups * U);
  src.w.sstep = (uint32_t)(16 * groups * SU);
  src.w.wb = make_buf(T.w13 + (size_t)wk.e * (2 * N1) * groups * U + (size_t)(8 * hb) * src.w.wstep, 8 * src.w.wstep);
  src.w.sb = make_buf(T.s13 + (size_t)wk.e * (2 * N1) * groups * SU + (size_t)(8 * hb) * src.w.sstep, 8 * src.w.sstep);
  src.w.kcols = K;
  src.xb = (const uint8_t *)a.xb;
  // rows past the tile read route p0's token; their results are never stored.
  // 32-bit byte offsets: the host runs this kernel only for chunks with 2 T K < 2^32
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int row = 4 * (8 * w + j) + (l >> 4);
    src.brow[j] = (uint32_t)(a.perm[wk.p0 + (row < wk.rows ? row : 0)] / a.topk) * (uint32_t)(2 * K);
  }
  const int nrb = __builtin_amdgcn_readfirstlane((wk.rows + 15) / 16);
  v4f acc[2][8];
  zero_acc<2, 8>(acc);
  const int nkt = K / 128;
  Pf16W ring[kPw16Stages];
  pf16_load_w<WF>(ring[0], src.w, 0, wu, l);
  pw16_issue_b(L.st[0], src, 0, wu, l);
  // an even number of k-tiles: K % 256 == 0
  int kt = 0;
  for (; kt + 2 < nkt; kt += 2) {
    pw16_step<WF, 0, true>(L, src, ring, kt, wu, nrb, acc);
    pw16_step<WF, 1, true>(L, src, ring, kt + 1, wu, nrb, acc);
  }
  pw16_step<WF, 0, true>(L, src, ring, kt, wu, nrb, acc);
  pw16_step<WF, 1, false>(L, src, ring, kt + 1, wu, nrb, acc);
  // epilogue: row tiles 2w (up) and 2w + 1 (gate) = intermediate columns 64 hb + 16 w .. +15;
  // acc[q][cb][i]: route 16 cb + c, column 16 w + 4 g + i
  const float g13 = T.g13 ? T.g13[wk.e] : 1.0f;
#pragma unroll
  for (int cb = 0; cb < 8; cb++) {
    if (cb >= nrb) break;
    const int row = 16 * cb + c;
    if (row < wk.rows) {
      const size_t p = (size_t)(wk.p0 + row);
      // router weight on the input: GEMM1 is linear, so it scales the accumulators
      const float gs = g13 * (a.w_on_input ? a.topk_w[a.perm[p]] : 1.0f);
      uint2 v;
      if (a.act == ACT_RELU2) {
        // ReLU^2 without the multiply: the up and gate halves' rows give columns n and N1 + n
#pragma unroll
        for (int half = 0; half < 2; half++) {
          v.x = pack_bf16x2(relu2(acc[half][cb][0] * gs), relu2(acc[half][cb][1] * gs));
          v.y = pack_bf16x2(relu2(acc[half][cb][2] * gs), relu2(acc[half][cb][3] * gs));
          *(uint2 *)(a.hb + p * N + half * N1 + 64 * hb + 16 * w + 4 * g) = v;
        }
        continue;
      }
      float h[4];
#pragma unroll
      for (int i = 0; i < 4; i++)
        h[i] = silu_clamped(acc[1][cb][i] * gs, acc[0][cb][i] * gs, a.limit, a.has_limit, a.alpha, a.beta, a.act);
      v.x = pack_bf16x2(h[0], h[1]);
      v.y = pack_bf16x2(h[2], h[3]);
      *(uint2 *)(a.hb + p * N + 64 * hb + 16 * w + 4 * g) = v;
    }
  }
}

template <int WF>
__global__ __launch_bounds__(256, 2) void k_pf_gemm1_a16w(GemmArgs a) {
  __shared__ Pw16Lds L;
  const PfWork wk = pf_work(a, a.N1 / 64, false);
  if (!wk.valid) return;
  pw16_gemm1_body<WF>(a, wk, pf_tier(a, 0), L);
}

__global__ __launch_bounds__(256, 2) void k_pf_gemm1_a16w_tiers(GemmArgs a) {
  __shared__ Pw16Lds L;
  int tier = 0;
  const PfWork wk = pf_work_tiers(a, a.N1 / 64, false, &tier);
  if (!wk.valid) return;
  const PfTier T = pf_tier(a, tier);
  if ((tier ? a.fmt_b : a.fmt_a) == W_NVFP4) pw16_gemm1_body<W_NVFP4>(a, wk, T, L);
  else pw16_gemm1_body<W_NF3>(a, wk, T, L);
}

// ---------------------------------------------------------------- GEMM2 (A16)
// Block: w2 row tiles 8 ob .. +7 = output columns 128 ob .. +127.
template <int WF>
__device__ __forceinline__ void pf16_gemm2_body(const GemmArgs &a, const PfWork &wk, const PfTier &T, Pf16Lds &L,
                                                int *s_r, float *s_w) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  const int K = a.K, N = a.N;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int ob = wk.sub, groups = N / 32;
  Pf16Src src;
  src.wstep = (uint32_t)(16 * groups * U);
  src.sstep = (uint32_t)(16 * groups * SU);
  src.wb = make_buf(T.w2 + (size_t)wk.e * K * groups * U + (size_t)(8 * ob) * src.wstep, 8 * src.wstep);
  src.sb = make_buf(T.s2 + (size_t)wk.e * K * groups * SU + (size_t)(8 * ob) * src.sstep, 8 * src.sstep);
  src.kcols = N;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int row = 4 * (4 * w + j) + (l >> 4);
    src.brow[j] = a.hb + (size_t)(wk.p0 + (row < wk.rows ? row : 0)) * N;
  }
  if (tid < wk.rows) {
    const int r = a.perm[wk.p0 + tid];
    s_r[tid] = r;
    s_w[tid] = (a.w_on_input ? 1.0f : a.topk_w[r]) * (T.g2 ? T.g2[wk.e] : 1.0f);
  }
  v4f acc[2][4];
#pragma unroll
  for (int q = 0; q < 2; q++)
#pragma unroll
    for (int cb = 0; cb < 4; cb++) acc[q][cb] = v4f{0.f, 0.f, 0.f, 0.f};
  pf16_kloop<WF, true>(L, src, wu, acc);
  __syncthreads();   // s_r / s_w visible; every wave is done with the ring's LDS
  // acc[q][cb][i]: route 16 cb + 4 g + i, output column 128 ob + 32 w + 16 q + c
  pf_combine<2, 4>(a, wk, acc, s_r, s_w, (size_t)128 * ob + 32 * w + c, 0, c, g, (uint8_t *)&L);
}

template <int WF>
__global__ __launch_bounds__(256) void k_pf_gemm2_a16(GemmArgs a) {
  __shared__ Pf16Lds L;
  __shared__ int s_r[kPfTileRows];
  __shared__ float s_w[kPfTileRows];
  const PfWork wk = pf_work(a, a.K / 128, false);
  if (!wk.valid) return;
  pf16_gemm2_body<WF>(a, wk, pf_tier(a, 0), L, s_r, s_w);
}

__global__ __launch_bounds__(256) void k_pf_gemm2_a16_tiers(GemmArgs a) {
  __shared__ Pf16Lds L;
  __shared__ int s_r[kPfTileRows];
  __shared__ float s_w[kPfTileRows];
  int tier = 0;
  const PfWork wk = pf_work_tiers(a, a.K / 128, false, &tier);
  if (!wk.valid) return;
  const PfTier T = pf_tier(a, tier);
  if ((tier ? a.fmt_b : a.fmt_a) == W_NVFP4) pf16_gemm2_body<W_NVFP4>(a, wk, T, L, s_r, s_w);
  else pf16_gemm2_body<W_NF3>(a, wk, T, L, s_r, s_w);
}

// ------------------------ GEMM2 (A16), resident intermediate rows
// The route-buffer combine's down GEMM as blocks of (64-route tile, run of
// a.obg 128-column output blocks), as the W4A8 one: the tile's bf16
// intermediate rows (all NKT k-tiles of N <= 128 NKT, 16 KB each) go into LDS
// once (NVFP4 tiles then convert them to fp16, below, and multiply in fp16:
// NVFP4 prefill at 2048 tokens, down GEMM 211 -> 196 us), and each wave streams its two weight row tiles of every output block
// of the run through a register ring of NKT k-tiles, so the next block's
// weights are in flight while the current one is multiplied and stored.  (One
// block per output block paid the rows' load, the perm lookups and the ring's
// first round trip for four k-tiles at N = 512.)
template <int NKT>
struct Pf16ResLds {
  Pf16Stage st[NKT];
  uint8_t rb[4 * 16 * (32 * 2 + 16)];   // per-wave route-buffer staging (pf_store_rb)
  int re[kPfTileRows];                   // each route's fp16 row exponent
};

// Weight and scale loads of row tiles rt0, rt0 + 1 (wave-uniform) for k-tile
// kt; vd / vs: the lane's offsets inside a k-tile's data / scales, or past the
// buffer's range (zeros, no traffic).  The k-tile's own offset is scalar.
template <int WF>
__device__ __forceinline__ void pf16_load_w_rt(Pf16W &r, const Pf16Src &src, uint32_t rt0, int kt, uint32_t vd,
                                               uint32_t vs) {
  constexpr uint32_t U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
#pragma unroll
  for (int q = 0; q < 2; q++) {
    const uint32_t so = (rt0 + q) * src.wstep + (uint32_t)kt * 64u * U, ss = (rt0 + q) * src.sstep + (uint32_t)kt * 64u * SU;
    if constexpr (WF == W_NVFP4) {
      const v4i v = buf_load16_nt(src.wb, vd, so);
      r.a[q][0] = v[0]; r.a[q][1] = v[1]; r.a[q][2] = v[2]; r.a[q][3] = v[3];
    } else {
      const v3i v = buf_load12_nt(src.wb, vd, so);
      r.a[q][0] = v[0]; r.a[q][1] = v[1]; r.a[q][2] = v[2]; r.a[q][3] = 0;
    }
    r.sc[q] = buf_load4(src.sb, vs, ss);
  }
}

template <int WF, int NKT, bool LASTFULL>
__device__ __forceinline__ void pf16_gemm2_res_body(const GemmArgs &a, const PfWork &wk, const PfTier &T,
                                                    Pf16ResLds<NKT> &L, int *s_r, float *s_w) {
  constexpr int U = FmtGeom<WF>::unit, SU = FmtGeom<WF>::sunit;
  constexpr bool H = WF == W_NVFP4;   // fp16 operands (one packed multiply a value pair in the decode)
  const int K = a.K, N = a.N, nob = K / 128, groups = N / 32;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, g = l >> 4;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int ob0 = wk.sub * a.obg, ob1 = min(nob, ob0 + a.obg);
  Pf16Src src;
  src.wstep = (uint32_t)(16 * groups * U);
  src.sstep = (uint32_t)(16 * groups * SU);
  src.wb = make_buf(T.w2 + (size_t)wk.e * K * groups * U, (uint32_t)((size_t)K * groups * U));
  src.sb = make_buf(T.s2 + (size_t)wk.e * K * groups * SU, (uint32_t)((size_t)K * groups * SU));
  src.kcols = N;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int row = 4 * (4 * w + j) + (l >> 4);
    src.brow[j] = a.hb + (size_t)(wk.p0 + (row < wk.rows ? row : 0)) * N;
  }
  if (tid < wk.rows) {
    const int r = a.perm[wk.p0 + tid];
    s_r[tid] = r;
    s_w[tid] = (a.w_on_input ? 1.0f : a.topk_w[r]) * (T.g2 ? T.g2[wk.e] : 1.0f);
  }
  // the tile's intermediate rows (every k-tile), then the first output block's weights
#pragma unroll
  for (int kt = 0; kt < NKT; kt++) pf16_issue_b(L.st[kt], src, kt, wu, l);
  // lane offsets: a whole k-tile, and the partial last one (lanes past N load
  // zeros: their scales then decode to 0, so no garbage code meets a zeroed input)
  const uint32_t kOut = 0x80000000u, vd = (uint32_t)(l * U), vs = (uint32_t)((l * SU) & ~3);
  const bool lin = LASTFULL || (NKT - 1) * 128 + 32 * g < N;
  const uint32_t vdl = lin ? vd : kOut, vsl = lin ? vs : kOut;
  Pf16W ring[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; kt++)
    pf16_load_w_rt<WF>(ring[kt], src, (uint32_t)(8 * ob0 + 2 * wu), kt, kt < NKT - 1 ? vd : vdl, kt < NKT - 1 ? vs : vsl);
  // the rows have landed once only the weight loads may be in flight; then
  // every wave's share (and s_r / s_w) is visible
  wait_vm<4 * NKT>();
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  // NVFP4 (H): the staged bf16 rows in place as fp16 times 2^-e, e from each
  // route's largest magnitude (h_row_exp; L.re for the epilogue).  Threads
  // 4r .. 4r + 3 take route r's chunks, a quarter of every k-tile's 16 slots
  // each, and meet by DPP; the slot order is rotated by r so that the 16 lanes
  // of a read cover all 16 slots (no bank conflicts).  Chunks past N hold a
  // copy of the row's first columns (harmless).  NF3 tiles stay bf16: their
  // table decode costs the same in either type.
  if constexpr (H) {
    const int r = tid >> 2, qq = tid & 3;
    uint32_t m = 0;
#pragma unroll
    for (int kt = 0; kt < NKT; kt++)
#pragma unroll
      for (int j = 0; j < 4; j++) m = max(m, bf16x8_amax(*(const v4i *)&L.st[kt].B[r][16 * (4 * qq + ((j + r) & 3))]));
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    const int e = h_row_exp(m);
#pragma unroll
    for (int kt = 0; kt < NKT; kt++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        v4i *p = (v4i *)&L.st[kt].B[r][16 * (4 * qq + ((j + r) & 3))];
        *p = bf16x8_to_h(*p, e);
      }
    if (qq == 0) L.re[r] = e;
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
  }
  for (int ob = ob0; ob < ob1; ob++) {
    asm volatile("" ::: "memory");   // keep the epilogue's LDS reads in the epilogue
    const bool next = ob + 1 < ob1;
    const uint32_t rtn = (uint32_t)(8 * (next ? ob + 1 : ob) + 2 * wu);
    const uint32_t nd = next ? vd : kOut, ns = next ? vs : kOut, ndl = next ? vdl : kOut, nsl = next ? vsl : kOut;
    v4f acc[2][4];
    zero_acc<2, 4>(acc);
#pragma unroll
    for (int kt = 0; kt < NKT; kt++) {
      wait_vm<4 * (NKT - 1)>();   // slot kt has landed (the NKT - 1 later slots may be in flight)
      v4i b[4][4];
      pf16_read_b(b, L.st[kt], l);
      if (kt < NKT - 1 || LASTFULL) pf16_mma<WF, true, true, true, H>(ring[kt], b, kt, N, l, acc);
      else pf16_mma<WF, true, false, true, H>(ring[kt], b, kt, N, l, acc);
      __builtin_amdgcn_sched_barrier(0);
      pf16_load_w_rt<WF>(ring[kt], src, rtn, kt, kt < NKT - 1 ? nd : ndl, kt < NKT - 1 ? ns : nsl);
      __builtin_amdgcn_sched_barrier(0);
    }
    // acc[q][cb][i]: route 16 cb + 4 g + i, output column 128 ob + 32 w + 16 q + c
    pf_store_rb<2, 4, H>(a, wk, acc, s_r, s_w, (size_t)128 * ob + 32 * w, c, g, L.rb, L.re);
  }
}

template <int WF, int NKT, bool LASTFULL>
__global__ __launch_bounds__(256, 2) void k_pf_gemm2_a16_res(GemmArgs a) {
  __shared__ Pf16ResLds<NKT> L;
  __shared__ int s_r[kPfTileRows];
  __shared__ float s_w[kPfTileRows];
  const PfWork wk = pf_work(a, (a.K / 128 + a.obg - 1) / a.obg, false);
  if (!wk.valid) return;
  pf16_gemm2_res_body<WF, NKT, LASTFULL>(a, wk, pf_tier(a, 0), L, s_r, s_w);
}

template <int NKT, bool LASTFULL>
__global__ __launch_bounds__(256, 2) void k_pf_gemm2_a16_res_tiers(GemmArgs a) {
  __shared__ Pf16ResLds<NKT> L;
  __shared__ int s_r[kPfTileRows];
  __shared__ float s_w[kPfTileRows];
  int tier = 0;
  const PfWork wk = pf_work_tiers(a, (a.K / 128 + a.obg - 1) / a.obg, false, &tier);
  if (!wk.valid) return;
  const PfTier T = pf_tier(a, tier);
  if ((tier ? a.fmt_b : a.fmt_a) == W_NVFP4) pf16_gemm2_res_body<W_NVFP4, NKT, LASTFULL>(a, wk, T, L, s_r, s_w);
  else pf16_gemm2_res_body<W_NF3, NKT, LASTFULL>(a, wk, T, L, s_r, s_w);
}

// The resident down GEMM for the route-buffer combine at N <= 512 (NKT <= 4);
// false where it does not apply.
template <int WF, int NKT>
static void launch_pf16_res_n(const GemmArgs &a, dim3 grid, hipStream_t s, bool tiers) {
  if (tiers) {
    if (a.N == 128 * NKT) hipLaunchKernelGGL((k_pf_gemm2_a16_res_tiers<NKT, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_pf_gemm2_a16_res_tiers<NKT, false>), grid, dim3(256), 0, s, a);
  } else {
    if (a.N == 128 * NKT) hipLaunchKernelGGL((k_pf_gemm2_a16_res<WF, NKT, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_pf_gemm2_a16_res<WF, NKT, false>), grid, dim3(256), 0, s, a);
  }
}

template <int WF>
static bool launch_pf16_res(const GemmArgs &a, int grid_tiles, hipStream_t s, bool tiers) {
  const int nkt = (a.N + 127) / 128;
  if (!a.deterministic || a.obg <= 0 || nkt > 4) return false;
  const dim3 grid(pf_grid(grid_tiles, (a.K / 128 + a.obg - 1) / a.obg));
  switch (nkt) {
    case 1: launch_pf16_res_n<WF, 1>(a, grid, s, tiers); break;
    case 2: launch_pf16_res_n<WF, 2>(a, grid, s, tiers); break;
    case 3: launch_pf16_res_n<WF, 3>(a, grid, s, tiers); break;
    default: launch_pf16_res_n<WF, 4>(a, grid, s, tiers); break;
  }
  return true;
}

template <int WF>
static hipError_t launch_pf_a16(const GemmArgs &a, int grid_tiles, hipStream_t s, bool second) {
  if (second && launch_pf16_res<WF>(a, grid_tiles, s, false)) return hipGetLastError();
  if (second) hipLaunchKernelGGL(k_pf_gemm2_a16<WF>, dim3(pf_grid(grid_tiles, a.K / 128)), dim3(256), 0, s, a);
  else if (a.tile_rows == kPfWideRows)
    hipLaunchKernelGGL(k_pf_gemm1_a16w<WF>, dim3(pf_grid(grid_tiles, a.N1 / 64)), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_pf_gemm1_a16<WF>, dim3(pf_grid(grid_tiles, a.N1 / 64)), dim3(256), 0, s, a);
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

// grid_tiles: an upper bound on both tiers' tiles together.
hipError_t launch_pf16_gemm1_tiers(const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  if (a.tile_rows == kPfWideRows)
    hipLaunchKernelGGL(k_pf_gemm1_a16w_tiers, dim3(pf_grid(grid_tiles, a.N1 / 64)), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_pf_gemm1_a16_tiers, dim3(pf_grid(grid_tiles, a.N1 / 64)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pf16_gemm2_tiers(const GemmArgs &a, int grid_tiles, hipStream_t s) {
  if (grid_tiles <= 0) return hipSuccess;
  if (launch_pf16_res<W_NVFP4>(a, grid_tiles, s, true)) return hipGetLastError();
  hipLaunchKernelGGL(k_pf_gemm2_a16_tiers, dim3(pf_grid(grid_tiles, a.K / 128)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
