// Internal declarations shared by the C-ABI host code and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kTileRows = 16;        // routes of one tile of the general GEMM kernels
constexpr int kPfTileRows = 64;      // routes of one tile of the prefill kernels
constexpr int kPfWideRows = 128;     // routes of one tile of the prefill W4A8 up/gate kernel
constexpr int kPfWideMaxK = 8704;    // largest K it takes (it stages the tile's activation scale rows in LDS)
constexpr int kPfResSlots = 512;     // resident blocks of the prefill W4A8 down GEMM (2 per CU)
constexpr int kPrefillMinT = 512;    // smallest batch the ladder runs with the prefill kernels (16-bit activations)
constexpr int kPrefillMinTA8 = 256;  // the same for W4A8
constexpr int kWideMinRoutes = 32;   // routes an expert averages from which the ladder takes 128-route up/gate tiles
constexpr int kRouteChunk = 1024;    // routes handled by one route-planner block
constexpr int kMaxExperts = 1024;    // experts of all tiers together (LDS histogram size)
constexpr int kMaxTiers = 2;

enum WFmt { W_MXFP4 = 1, W_NVFP4 = 2, W_NF3 = 3 };
// activation forms of the GEMM1 epilogue (MOE_ACT_* of the C ABI)
enum Act { ACT_SWIGLU = 0, ACT_SITU = 1, ACT_RELU2 = 2 };

// Bytes per row of the MXFP8 intermediate's scales: N/32 rounded up to a
// multiple of 4, so every row starts 4-byte aligned.
__host__ __device__ constexpr int hs_stride(int N) { return (N / 32 + 3) & ~3; }

// Prefill copies of the MXFP4 scales: the bytes of one 16-row tile (E8M0, one per lane and k-tile; nkf =
// the whole 128-column k-tiles of the reduction, a partial last one after
// them): whole k-tiles in runs of four with each lane's four bytes in one
// dword (lane-major), so that a wave loads the scales of four consecutive
// k-tiles at once; whole k-tiles after the last run lane-major with as many
// bytes a lane as there are of them; a partial last k-tile a byte a lane (its
// first 16 * (32-column groups) lanes).  Byte offset of lane l of k-tile kt:
__host__ __device__ constexpr uint32_t mx_soff(int kt, int l, int nkf) {
  return kt < (nkf & ~3) ? (uint32_t)((kt >> 2) * 256 + l * 4 + (kt & 3))
         : kt < nkf      ? (uint32_t)((nkf & ~3) * 64 + l * (nkf & 3) + (kt & 3))
                         : (uint32_t)(nkf * 64 + l);
}

// LDS budget of the decode up/gate GEMM's staged token rows: six MXFP8 rows
// at K = 7168 (one pass for every expert of an 8-token batch at top-6), and
// three blocks per CU.
constexpr int kDecStageBytes = 45056;

// Dynamic LDS of the W4A8 decode down GEMM: every route's MXFP8 row (stride
// N + 16) rounded up to whole 1 KB direct-load chunks, then the scale rows
// (stride hs_stride(N)) rounded up to whole 256-byte chunks.
__host__ __device__ constexpr int dec2_hq_bytes(int R, int N) { return (R * (N + 16) + 1023) & ~1023; }
__host__ __device__ constexpr int dec2_hs_bytes(int R, int N) { return (R * hs_stride(N) + 255) & ~255; }
// W4A16: every route's bf16 intermediate row (stride 2 N + 16 bytes) in whole 1 KB chunks.
__host__ __device__ constexpr int dec2_hb_bytes(int R, int N) { return (R * (2 * N + 16) + 1023) & ~1023; }
constexpr int kDec2MaxLds = 73728;   // dynamic LDS bound of the decode down GEMM (two blocks per CU)

// Route planner: ids -> per-expert counts, offsets, stable permutation, tile table.
struct RouteArgs {
  const int32_t *ids;
  int R, topk, E;                    // routes, slots per token, global id range
  int n_tiers;
  const int32_t *emap0, *emap1;      // NULL = identity
  int E0, E1;                        // experts per tier; U = E0 + E1
  int G;                             // route blocks (ceil(R / kRouteChunk))
  int tile_rows;                     // routes per GEMM tile
  int max_tiles;
  int32_t *ru, *lrank, *chunk_hist;  // per-route expert / in-chunk rank; [G][U] counts
  int32_t *cnt, *off, *perm, *inv;
  int32_t *tile_u, *tile_row0, *tier_tiles;
  // optional second tile table of tile_rows2 routes per tile (NULL: none)
  int tile_rows2;
  int32_t *tile_u2, *tile_row02, *tier_tiles2;
  // work fused into the same launch by extra blocks
  const uint16_t *x;                 // bf16 [T, K] (MXFP8 quantisation when xq != NULL)
  int T, K;
  uint8_t *xq, *xs;
  float *zero_buf;                   // fp32 accumulator to clear (atomic combine)
  long zero_n;
  int side_blocks;
};

// GEMM launches (one tier at a time).
struct GemmArgs {
  const int32_t *tile_u, *tile_row0, *tier_tiles;
  int tier, u_base, tile_rows;
  const int32_t *off, *perm;
  int topk, K, N;
  const uint8_t *w13, *s13, *w2, *s2;
  const float *g13, *g2;
  const uint8_t *xq, *xs;            // MXFP8 activations (A8)
  const uint16_t *xb;                // bf16 activations (A16)
  uint8_t *hq, *hs;                  // MXFP8 intermediate (A8), [Rcap, N] / [Rcap, N/32]
  uint16_t *hb;                      // bf16 intermediate (A16), [Rcap, N]
  float limit;
  int has_limit;
  const float *topk_w;
  float *out_acc;                    // fp32 [T, K] (atomic combine)
  uint16_t *rb;                      // bf16 [R, K] route buffer (deterministic combine)
  int deterministic;
  int T;                             // tokens of the chunk (rows of x / the accumulator)
  int w_on_input;                    // router weight scales GEMM1 (W4A16 / W3A16), not the GEMM2 result
  float alpha, beta;                 // SwiGLU form: gate * sigmoid(alpha gate) * (up + beta)
  int act;                           // Act: SwiGLU (limit, alpha, beta), SiTU or ReLU^2 without the multiply
  // column pairs of GEMM1: N, or N / 2 for ReLU^2 without the multiply, whose w13
  // of N rows runs as an [up; gate] w13 of N / 2 pairs (h columns n and N / 2 + n)
  int N1;
  // both tiers in one launch (prefill W4A16 / W3A16): the fields above are tier 0,
  // these tier 1, whose experts follow tier 0's in the unified index (u_base_b)
  const uint8_t *w13b, *s13b, *w2b, *s2b;
  const float *g13b, *g2b;
  int fmt_a, fmt_b, u_base_b;
  // prefill W4A8 down GEMM with the route-buffer combine: 256-column output blocks per block (0: one)
  int obg;
};

// Decode-size batches (T <= kDecodeMaxT tokens, T * top_k <= 64 routes): two
// launches, routing recomputed in each workgroup from the ids.
constexpr int kDecodeMaxT = 16;
constexpr int kDecodeMaxRoutes = 64;

struct DecTier {
  const uint8_t *w13, *s13, *w2, *s2;
  const float *g13, *g2;
  const int32_t *emap;
  int fmt, E;
};

// Expert groups of a decode batch (routes sharing an expert, in order of first
// occurrence) with their pass counts (the most slots one token has on the
// group's expert) and the first item of each in the down GEMM's item list;
// written by the up/gate kernel, read by the down kernel.
struct DecGroups {
  int ng, nitems;
  int gu[kDecodeMaxRoutes];
  int istart[kDecodeMaxRoutes];
  int np[kDecodeMaxRoutes];
  unsigned long long gm[kDecodeMaxRoutes];
};

struct DecArgs {
  const int32_t *ids;
  const float *topk_w;
  const uint16_t *x;                 // bf16 [T, K]
  int T, R, topk, E, K, N, n_tiers;
  DecTier tier[kMaxTiers];
  float limit;
  int has_limit;
  int cpass;                         // token rows per LDS staging pass (MXFP8 x)
  uint8_t *hq, *hs;                  // MXFP8 intermediate per route r: [R, N], [R, N/32]; W4A16: hs the
                                     // exponent byte of each 32-column slice of hb
  uint16_t *hb;                      // W4A16 intermediate per route r: [R, N], each 32-column slice the
                                     // bf16-rounded values in fp16 times 2^-e of its own (from its byte)
  uint16_t *out;                     // bf16 [T, K]
  DecGroups *groups;                 // scratch
  int w_on_input;                    // router weight scales GEMM1 (W4A16 / W3A16), not the GEMM2 result
  float alpha, beta;                 // SwiGLU form: gate * sigmoid(alpha gate) * (up + beta)
  int act;                           // Act: SwiGLU (limit, alpha, beta), SiTU or ReLU^2 without the multiply
  int N1;                            // column pairs of GEMM1 (as GemmArgs::N1)
  // W4A16 / W3A16 down GEMM split over two blocks per output row tile (scratch):
  float *dpart;                      // [K/16][16 tokens][16 columns] fp32 token sums, both halves added
  int *dcnt;                         // [K/16] halves finished; both zeroed by the up/gate kernel
};

// The W4A16 / W3A16 decode down GEMM runs two blocks per 16-row output tile,
// one per half of the reduction's k-tiles, when there are two k-tiles or more.
__host__ __device__ constexpr int dec2_a16_halves(int N) { return (N + 127) / 128 >= 2 ? 2 : 1; }
// intermediate columns of half 0 (the wider one)
__host__ __device__ constexpr int dec2_a16_cols0(int N) {
  return dec2_a16_halves(N) == 1 ? N : ((((N + 127) / 128) + 1) / 2) * 128;
}

// Sets the calling thread's moe_last_error message; returns code.
int set_error(int code, const char *msg);

int decode_cpass(int K, int a8);
size_t decode_gemm1_lds(int K, int cpass, int a8);
hipError_t launch_decode(int a8, const DecArgs &a, hipStream_t s, hipEvent_t ev_mid);

hipError_t launch_route(const RouteArgs &a, hipStream_t s);
hipError_t launch_gemm1(int wfmt, const GemmArgs &a, int grid_tiles, hipStream_t s);
hipError_t launch_gemm2(int wfmt, const GemmArgs &a, int grid_tiles, hipStream_t s);
// Prefill kernels (64-route tiles, LDS-staged operands); W4A8 and N % 64 == 0.
hipError_t launch_pf_gemm1(const GemmArgs &a, int grid_tiles, hipStream_t s);
hipError_t launch_pf_gemm2(const GemmArgs &a, int grid_tiles, hipStream_t s);
hipError_t launch_pf16_gemm1(int wfmt, const GemmArgs &a, int grid_tiles, hipStream_t s);
hipError_t launch_pf16_gemm2(int wfmt, const GemmArgs &a, int grid_tiles, hipStream_t s);
hipError_t launch_pf16_gemm1_tiers(const GemmArgs &a, int grid_tiles, hipStream_t s);
hipError_t launch_pf16_gemm2_tiers(const GemmArgs &a, int grid_tiles, hipStream_t s);
hipError_t launch_finalize(int deterministic, const float *out_acc, const uint16_t *rb, const int32_t *inv,
                           int T, int K, int topk, uint16_t *out, hipStream_t s);
hipError_t launch_ep_remap(const int32_t *ids, const float *w, long T, int topk, long offset, long num_local,
                           int32_t *out_ids, float *out_w, hipStream_t s);
hipError_t launch_quant_bf16(const uint16_t *x, long rows, int cols, uint8_t *q, uint8_t *sc, hipStream_t s);
hipError_t launch_quant_f32(const float *h, long rows, int cols, uint8_t *q, uint8_t *sc, hipStream_t s);

// In-place layout change of one weight tensor, experts [e0, e0+ne) staged in tmp.
//   unit   bytes per (row, 32-column group): 16 (fp4 data), 12 (NF3 data),
//          1 (E8M0 / E4M3-per-32 scales), 2 (E4M3-per-16 scales)
//   rows   rows per expert (2N for w13, K for w2); groups = columns / 32
//   pair   1 for w13: row tiles interleave up and gate halves
//   gate_up 1 when the checkpoint stacks w13 as [gate; up]
//   to_tiles 1 = checkpoint -> tile layout, 0 = back
//   mxs    1: the k-tiles of a row tile in mx_soff's order (the prefill copies of MXFP4 scales)
hipError_t launch_nf3_recode(uint8_t *w, long units, int to_kernel, hipStream_t s);
hipError_t launch_permute(const uint8_t *tmp, uint8_t *dst, long ne, int unit, int rows, int groups, int pair,
                          int gate_up, int to_tiles, int mxs, hipStream_t s);

}  // namespace moe
