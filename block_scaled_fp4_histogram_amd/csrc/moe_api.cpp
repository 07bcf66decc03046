// C ABI of the routed MoE layer (declared in include/moe.h): plans, the
// capacity ladder, scratch carving, argument validation, in-place weight
// preparation and the launch sequence of one layer.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <vector>

#include "moe.h"
#include "moe_common.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

}  // namespace

namespace moe {
// The calling thread's error message, for entry points in other source files.
int set_error(int code, const char *msg) { return fail(code, "%s", msg); }
}  // namespace moe

namespace {

#define HIP_TRY(expr)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(MOE_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

constexpr int kStageEvents = 5;  // before route, after route / gemm1 / gemm2 / combine
constexpr uint32_t kPlanMagic = 0x4D4F4550u;     // "MOEP"
constexpr uint32_t kExpertsMagic = 0x4D4F4558u;  // "MOEX"

// Capacity ladder rungs (tokens per launch): exact small decode batches, then
// powers of two up to the plan's max_tokens (sglang moe_b12x_next.py: exact
// decode/verify capacities plus a bounded prefill ladder; a batch runs at the
// smallest capacity >= its size, larger batches in chunks of the top one).
const int kLadder[] = {1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16, 24, 32, 48, 64, 96, 128, 256, 512, 1024, 2048,
                       4096, 8192, 16384};

}  // namespace

struct moe_plan_s {
  uint32_t magic;
  int E, K, N, topk;
  float limit;
  int has_limit;
  int afmt, w13_layout, max_tokens;
  int w_on_input = 0;     // router weight applied to GEMM1's input (W4A16 / W3A16 only)
  float alpha = 1.f, beta = 0.f;   // SwiGLU form gate * sigmoid(alpha gate) * (up + beta)
  int act = MOE_ACT_SWIGLU;        // activation form of the GEMM1 epilogue
  std::vector<int> caps;  // ascending; caps.back() == chunk
  std::vector<int> seq;   // per rung: the launch sequence it is pinned to (MOE_SEQ_*), 0 = the ladder's choice
  std::vector<int> comb;  // per rung: the combine of deterministic = 0 runs (MOE_COMBINE_*), 0 = the ladder's
  // optional stage timing: kStageEvents events per recorded run
  std::vector<hipEvent_t> events;
  int timing_runs_max = 0, timing_runs = 0;
};

struct moe_experts_s {
  uint32_t magic;
  int K, N, w13_layout;   // geometry the buffers were prepared for
  int w13_rows;           // 2N, or N for ReLU^2 without the multiply
  int wfmt, E;
  uint8_t *w13, *s13, *w2, *s2;
  uint8_t *s13g, *s2g;   // MXFP4, prepared: the scales in mx_soff's order for the prefill GEMMs (owned)
  const float *g13, *g2;
  int prepared;
};

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool plan_ok(const moe_plan_s *p) { return p && p->magic == kPlanMagic; }

// Rows of w13 and column pairs of GEMM1 under the plan's activation: ReLU^2
// without the multiply has a w13 of N rows, run as an [up; gate] w13 of N / 2
// pairs whose two halves give h columns n and N / 2 + n.
int w13_rows(const moe_plan_s *p) { return p->act == MOE_ACT_RELU2_NO_MUL ? p->N : 2 * p->N; }
int gemm1_pairs(const moe_plan_s *p) { return p->act == MOE_ACT_RELU2_NO_MUL ? p->N / 2 : p->N; }

int cap_for(const moe_plan_s *p, int T) {
  for (int c : p->caps)
    if (c >= T) return c;
  return p->caps.back();
}

int rung_of(const moe_plan_s *p, int T) {
  for (size_t i = 0; i < p->caps.size(); i++)
    if (p->caps[i] >= T) return (int)i;
  return (int)p->caps.size() - 1;
}

size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

int seq_for(const moe_plan_s *p, int T);

// Whether runs at the rung of `cap` tokens combine through the per-slot route
// buffer and the top-k sum (always in deterministic mode) rather than fp32
// atomics into an accumulator.  The ladder's choice for deterministic = 0: the
// route buffer with the prefill kernels, whose atomic adds all execute
// memory-side on this GPU (a 4096-token W4A8 prefill layer measured 903 us with
// atomics against 602 us through the route buffer), and with the W4A8 general
// kernels from 256 tokens (per-rung race: 456 vs 483 us at 256 tokens, 482 vs
// 600 us at 512; below 256 the two are within 2 %); atomics otherwise.  A
// chunked batch's chunks all follow the rung of its first chunk.
constexpr int kRbGeneralMinTA8 = 256;
bool route_buffer(const moe_plan_s *p, int cap, int deterministic) {
  if (deterministic) return true;
  const int pinned = p->comb[rung_of(p, cap)];
  if (pinned) return pinned == MOE_COMBINE_ROUTE_BUFFER;
  const int seq = seq_for(p, cap);
  if (seq == MOE_SEQ_PREFILL || seq == MOE_SEQ_PREFILL_NARROW) return true;
  return seq == MOE_SEQ_GENERAL && p->afmt == MOE_A_MXFP8 && cap >= kRbGeneralMinTA8;
}

// Carving of the scratch arena for one chunk of `cap` tokens.
struct Layout {
  size_t ru, lrank, inv, perm, cnt, off, chunk_hist, tile_u, tile_row0, tier_tiles, tile_u2, tile_row02, tier_tiles2;
  size_t xq, xs, hq, hs, hb, acc, rb, dpart, dcnt;
  size_t total;
  int R, G, max_tiles, max_tiles2;
};

Layout layout(const moe_plan_s *p, int cap, int deterministic) {
  Layout L;
  memset(&L, 0, sizeof L);
  const size_t R = (size_t)cap * p->topk;
  const int U = moe::kMaxExperts;
  L.R = (int)R;
  L.G = (int)((R + moe::kRouteChunk - 1) / moe::kRouteChunk);
  L.max_tiles = (int)((R + moe::kTileRows - 1) / moe::kTileRows + std::min<size_t>(U, R));
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = al256(o + bytes);
    return at;
  };
  L.ru = take(4 * R);
  L.lrank = take(4 * R);
  L.inv = take(4 * R);
  L.perm = take(4 * R);
  L.cnt = take(4 * (size_t)U);
  L.off = take(4 * (size_t)(U + 1));
  L.chunk_hist = take(4 * (size_t)L.G * U);
  L.tile_u = take(4 * (size_t)L.max_tiles);
  L.tile_row0 = take(4 * (size_t)L.max_tiles);
  L.tier_tiles = take(4 * 2 * moe::kMaxTiers);
  // the prefill up/gate GEMM's table of 128-route tiles
  L.max_tiles2 = (int)((R + moe::kPfWideRows - 1) / moe::kPfWideRows + std::min<size_t>(U, R));
  L.tile_u2 = take(4 * (size_t)L.max_tiles2);
  L.tile_row02 = take(4 * (size_t)L.max_tiles2);
  L.tier_tiles2 = take(4 * 2 * moe::kMaxTiers);
  if (p->afmt == MOE_A_MXFP8) {
    L.xq = take((size_t)cap * p->K);
    L.xs = take((size_t)cap * (p->K / 32));
    L.hq = take(R * p->N);
    L.hs = take(R * moe::hs_stride(p->N));
  } else {
    L.hb = take(2 * R * p->N);
    // per route and 32-column slice of hb, the exponent byte of its largest
    // magnitude: the decode down GEMM's fp16 row scale
    L.hs = take(R * moe::hs_stride(p->N));
    // the decode down GEMM's two halves per 16-row output tile meet here: carved at
    // every capacity, since the last chunk of a batch above the top capacity can be
    // decode-sized whatever the capacity the arena was sized for
    L.dpart = take((size_t)(p->K / 16) * 256 * sizeof(float));
    L.dcnt = take(4 * (size_t)(p->K / 16));
  }
  if (route_buffer(p, cap, deterministic)) L.rb = take(2 * R * p->K);
  else L.acc = take(4 * (size_t)cap * p->K);
  L.total = o;
  return L;
}

int check_tiers(const moe_plan_s *p, const moe_tier *tiers, int n_tiers) {
  if (!tiers || n_tiers < 1 || n_tiers > moe::kMaxTiers) return fail(MOE_EINVAL, "n_tiers must be 1 or 2");
  int U = 0;
  for (int i = 0; i < n_tiers; i++) {
    const moe_experts_s *x = tiers[i].experts;
    if (!x || x->magic != kExpertsMagic) return fail(MOE_EINVAL, "tier %d: null or invalid experts handle", i);
    if (!x->prepared) return fail(MOE_ENOTPREPARED, "tier %d: experts are not prepared (checkpoint layout)", i);
    if (x->K != p->K || x->N != p->N || x->w13_layout != p->w13_layout || x->w13_rows != w13_rows(p))
      return fail(MOE_ENOTPREPARED,
                  "tier %d: experts prepared for K=%d N=%d layout=%d w13 rows=%d, plan has K=%d N=%d layout=%d w13 "
                  "rows=%d",
                  i, x->K, x->N, x->w13_layout, x->w13_rows, p->K, p->N, p->w13_layout, w13_rows(p));
    const int want_a = (x->wfmt == MOE_W_MXFP4) ? MOE_A_MXFP8 : MOE_A_BF16;
    if (want_a != p->afmt) return fail(MOE_EUNSUPPORTED, "tier %d: weight format %d does not run with activation format %d", i, x->wfmt, p->afmt);
    if (tiers[i].expert_map && !aligned(tiers[i].expert_map, 4)) return fail(MOE_EINVAL, "tier %d: misaligned expert_map", i);
    if (!tiers[i].expert_map && x->E > p->E) return fail(MOE_EINVAL, "tier %d: %d experts exceed the id range %d without a map", i, x->E, p->E);
    U += x->E;
  }
  if (U > moe::kMaxExperts) return fail(MOE_EUNSUPPORTED, "tiers hold %d experts; at most %d", U, moe::kMaxExperts);
  return MOE_OK;
}

// Decode-size batch: the two-launch path (routing inside each workgroup).
int run_decode(const moe_plan_s *p, const moe_tier *tiers, int n_tiers, const uint16_t *x, const int32_t *ids,
               const float *wts, uint16_t *out, int T, const Layout &L, uint8_t *scratch, hipStream_t s,
               const hipEvent_t *ev) {
  moe::DecArgs da;
  memset(&da, 0, sizeof da);
  da.ids = ids;
  da.topk_w = wts;
  da.x = x;
  da.T = T;
  da.R = T * p->topk;
  da.topk = p->topk;
  da.E = p->E;
  da.K = p->K;
  da.N = p->N;
  da.n_tiers = n_tiers;
  for (int i = 0; i < n_tiers; i++) {
    const moe_experts_s *xp = tiers[i].experts;
    da.tier[i].w13 = xp->w13;
    da.tier[i].s13 = xp->s13;
    da.tier[i].w2 = xp->w2;
    da.tier[i].s2 = xp->s2;
    da.tier[i].g13 = xp->g13;
    da.tier[i].g2 = xp->g2;
    da.tier[i].emap = tiers[i].expert_map;
    da.tier[i].fmt = xp->wfmt;
    da.tier[i].E = xp->E;
  }
  da.limit = p->limit;
  da.has_limit = p->has_limit;
  da.w_on_input = p->w_on_input;
  da.alpha = p->alpha;
  da.beta = p->beta;
  da.act = p->act;
  da.N1 = gemm1_pairs(p);
  da.cpass = moe::decode_cpass(p->K, p->afmt == MOE_A_MXFP8);
  da.hq = scratch + L.hq;
  da.hs = scratch + L.hs;
  da.hb = (uint16_t *)(scratch + L.hb);
  da.out = out;
  static_assert(sizeof(moe::DecGroups) <= 4 * moe::kMaxExperts, "the group table fits the planner's count table");
  da.groups = (moe::DecGroups *)(scratch + L.cnt);   // the planner's count table is free on this path
  da.dpart = L.dpart ? (float *)(scratch + L.dpart) : nullptr;
  da.dcnt = L.dcnt ? (int *)(scratch + L.dcnt) : nullptr;
  if (p->afmt != MOE_A_MXFP8 && moe::dec2_a16_halves(p->N) == 2 && (!da.dpart || !da.dcnt))
    return fail(MOE_EINVAL, "decode down GEMM: the scratch layout lacks its per-tile accumulators (capacity %d)", T);
  if (ev) {
    HIP_TRY(hipEventRecord(ev[0], s));
    HIP_TRY(hipEventRecord(ev[1], s));
  }
  HIP_TRY(moe::launch_decode(p->afmt == MOE_A_MXFP8, da, s, ev ? ev[2] : nullptr));
  if (ev) {
    HIP_TRY(hipEventRecord(ev[3], s));
    HIP_TRY(hipEventRecord(ev[4], s));
  }
  return MOE_OK;
}

bool use_decode(const moe_plan_s *p, int T) {
  // the decode GEMM1 stages at least one token row in its LDS budget, and the
  // down GEMM all routes' rows of the intermediate
  const bool a8 = p->afmt == MOE_A_MXFP8;
  const long row = a8 ? (long)p->K + 16 + p->K / 32 : 2L * (p->K + 8);
  const long lds2 = a8 ? (long)moe::dec2_hq_bytes(T * p->topk, p->N) + moe::dec2_hs_bytes(T * p->topk, p->N)
                       : (long)moe::dec2_hb_bytes(T * p->topk, p->N);
  const bool lds_ok = row <= moe::kDecStageBytes && lds2 <= moe::kDec2MaxLds;
  return T <= moe::kDecodeMaxT && T * p->topk <= moe::kDecodeMaxRoutes && lds_ok;
}

// Launch sequences: which ones a rung of `cap` tokens may take, the capacity
// ladder's own choice for a chunk of T tokens, and the one a chunk runs with.
bool seq_eligible(const moe_plan_s *p, int cap, int seq) {
  switch (seq) {
    case MOE_SEQ_DECODE: return use_decode(p, cap);   // then also for every chunk of <= cap tokens
    case MOE_SEQ_GENERAL: return true;
    // PREFILL_NARROW: PREFILL with the up/gate GEMM on 64-route tiles as well
    case MOE_SEQ_PREFILL:
    case MOE_SEQ_PREFILL_NARROW: return gemm1_pairs(p) % 64 == 0 && p->N % 64 == 0;
    default: return false;
  }
}

// The ladder's own choice, from the per-rung race on uniform routing (one
// MI355X, both geometries of the pages, atomic and deterministic combine): the
// 64-route-tile kernels overtake the 16-route ones from 256 tokens for W4A8
// (deterministic: 448 vs 465 us) and from 512 for W4A16 / W3A16 (421 vs 569).
// The W4A8 up/gate GEMM's 128-route tiles overtake its 64-route ones once an
// expert averages 32 routes (below that they are mostly padding: at 1024
// tokens, 16 routes an expert at E = 384, top-6, the 64-route tiles lead by
// 2 %, at 2048 the 128-route ones by 1.5 %, at the Zipf-skewed 4096-token
// batch by 4 %); the 16-bit one, whose 128-route tiles also halve its
// dequantisation per MFMA, leads from 512 tokens (16 routes an expert).
int ladder_seq(const moe_plan_s *p, int T) {
  if (use_decode(p, T)) return MOE_SEQ_DECODE;
  const bool a8 = p->afmt == MOE_A_MXFP8;
  if (T < (a8 ? moe::kPrefillMinTA8 : moe::kPrefillMinT) || !seq_eligible(p, T, MOE_SEQ_PREFILL))
    return MOE_SEQ_GENERAL;
  if (!a8) return MOE_SEQ_PREFILL;
  return (long)T * p->topk >= (long)moe::kWideMinRoutes * p->E ? MOE_SEQ_PREFILL : MOE_SEQ_PREFILL_NARROW;
}

int seq_for(const moe_plan_s *p, int T) {
  const int pinned = p->seq[rung_of(p, T)];
  return pinned ? pinned : ladder_seq(p, T);
}

// Everything one chunk needs after validation.  deterministic: combine through
// the route buffer and the top-k sum (1) or fp32 atomics (0).
int run_chunk(const moe_plan_s *p, const moe_tier *tiers, int n_tiers, const uint16_t *x, const int32_t *ids,
              const float *wts, uint16_t *out, int T, int deterministic, const Layout &L, uint8_t *scratch,
              hipStream_t s, bool route_only, bool prefill, const hipEvent_t *ev = nullptr,
              bool narrow = false) {
  if (ev) HIP_TRY(hipEventRecord(ev[0], s));
  const int R = T * p->topk;
  auto I32 = [&](size_t o) { return (int32_t *)(scratch + o); };
  moe::RouteArgs ra;
  memset(&ra, 0, sizeof ra);
  ra.ids = ids;
  ra.R = R;
  ra.topk = p->topk;
  ra.E = p->E;
  ra.n_tiers = n_tiers;
  ra.emap0 = tiers[0].expert_map;
  ra.E0 = tiers[0].experts->E;
  ra.emap1 = n_tiers > 1 ? tiers[1].expert_map : nullptr;
  ra.E1 = n_tiers > 1 ? tiers[1].experts->E : 0;
  ra.G = (R + moe::kRouteChunk - 1) / moe::kRouteChunk;
  ra.max_tiles = L.max_tiles;
  // prefill kernels: 64-route tiles (N % 64 == 0); general kernels: 16-route tiles
  ra.tile_rows = prefill ? moe::kPfTileRows : moe::kTileRows;
  ra.ru = I32(L.ru);
  ra.lrank = I32(L.lrank);
  ra.chunk_hist = I32(L.chunk_hist);
  ra.cnt = I32(L.cnt);
  ra.off = I32(L.off);
  ra.perm = I32(L.perm);
  ra.inv = I32(L.inv);
  ra.tile_u = I32(L.tile_u);
  ra.tile_row0 = I32(L.tile_row0);
  ra.tier_tiles = I32(L.tier_tiles);
  // 128-route tiles for the up/gate GEMM: its activation offsets are 32-bit, and
  // the W4A8 one stages every route's whole scale row in LDS (K <= 8704)
  const bool wide = prefill && !narrow &&
                    (p->afmt == MOE_A_MXFP8 ? (uint64_t)T * p->K < (1ull << 32) && p->K <= moe::kPfWideMaxK
                                            : (uint64_t)2 * T * p->K < (1ull << 32));
  if (wide) {
    ra.tile_rows2 = moe::kPfWideRows;
    ra.tile_u2 = I32(L.tile_u2);
    ra.tile_row02 = I32(L.tile_row02);
    ra.tier_tiles2 = I32(L.tier_tiles2);
  }
  ra.x = x;
  ra.T = T;
  ra.K = p->K;
  long side_work = 0;
  if (!route_only) {
    if (p->afmt == MOE_A_MXFP8) {
      ra.xq = scratch + L.xq;
      ra.xs = scratch + L.xs;
      side_work = std::max(side_work, (long)T * (p->K / 32));
    }
    if (!deterministic) {
      ra.zero_buf = (float *)(scratch + L.acc);
      ra.zero_n = (long)T * p->K;
      side_work = std::max(side_work, ra.zero_n / 4);
    }
  }
  ra.side_blocks = (int)std::min<long>((side_work + 1023) / 1024, 512);   // blocks of 1024 threads
  HIP_TRY(moe::launch_route(ra, s));
  if (route_only) return MOE_OK;
  if (ev) HIP_TRY(hipEventRecord(ev[1], s));

  moe::GemmArgs ga;
  memset(&ga, 0, sizeof ga);
  ga.tile_rows = ra.tile_rows;
  ga.T = T;
  ga.tile_u = I32(L.tile_u);
  ga.tile_row0 = I32(L.tile_row0);
  ga.tier_tiles = I32(L.tier_tiles);
  ga.off = I32(L.off);
  ga.perm = I32(L.perm);
  ga.topk = p->topk;
  ga.K = p->K;
  ga.N = p->N;
  ga.xq = scratch + L.xq;
  ga.xs = scratch + L.xs;
  ga.xb = x;
  ga.hq = scratch + L.hq;
  ga.hs = scratch + L.hs;
  ga.hb = (uint16_t *)(scratch + L.hb);
  ga.limit = p->limit;
  ga.has_limit = p->has_limit;
  ga.w_on_input = p->w_on_input;
  ga.alpha = p->alpha;
  ga.beta = p->beta;
  ga.act = p->act;
  ga.N1 = gemm1_pairs(p);
  ga.topk_w = wts;
  ga.out_acc = (float *)(scratch + L.acc);
  ga.rb = (uint16_t *)(scratch + L.rb);
  ga.deterministic = deterministic;
  const int row_tiles = (R + ra.tile_rows - 1) / ra.tile_rows;
  // the route-buffer down GEMM's runs of 256-column output blocks per block: as
  // long as possible while the (tile, run) items still fill every resident slot,
  // and at least two runs a tile (at K = 7168 and 4096 tokens, 2 runs of 14:
  // 182 us; runs of 10, 7, 4, 2: 187, 185, 189, 200 us; one run of 28 leaves
  // CUs idle: 187 us)
  {
    // output blocks of 256 columns (W4A8) or 128 (16-bit activations)
    const int nob = p->afmt == MOE_A_MXFP8 ? p->K / 256 : p->K / 128, tiles = std::max(1, R / moe::kPfTileRows);
    const int runs = std::min(nob, std::max(2, (moe::kPfResSlots + tiles - 1) / tiles));
    ga.obg = (nob + runs - 1) / runs;
  }
  // prefill with two W4A16 / W3A16 tiers: one launch per GEMM covers both tiers,
  // so their weight streams share the machine instead of running back to back
  const bool tiers_together = prefill && n_tiers == 2 && tiers[0].experts->wfmt != MOE_W_MXFP4 &&
                              tiers[1].experts->wfmt != MOE_W_MXFP4;
  if (tiers_together) {
    const moe_experts_s *xa = tiers[0].experts, *xb = tiers[1].experts;
    ga.tier = 0;
    ga.u_base = 0;
    ga.w13 = xa->w13;
    ga.s13 = xa->s13;
    ga.w2 = xa->w2;
    ga.s2 = xa->s2;
    ga.g13 = xa->g13;
    ga.g2 = xa->g2;
    ga.fmt_a = xa->wfmt;
    ga.w13b = xb->w13;
    ga.s13b = xb->s13;
    ga.w2b = xb->w2;
    ga.s2b = xb->s2;
    ga.g13b = xb->g13;
    ga.g2b = xb->g2;
    ga.fmt_b = xb->wfmt;
    ga.u_base_b = xa->E;
    const int grid_tiles = row_tiles + std::min(xa->E + xb->E, R);
    if (wide) {
      moe::GemmArgs gw = ga;
      gw.tile_rows = moe::kPfWideRows;
      gw.tile_u = I32(L.tile_u2);
      gw.tile_row0 = I32(L.tile_row02);
      gw.tier_tiles = I32(L.tier_tiles2);
      HIP_TRY(moe::launch_pf16_gemm1_tiers(
          gw, (R + moe::kPfWideRows - 1) / moe::kPfWideRows + std::min(xa->E + xb->E, R), s));
    } else {
      HIP_TRY(moe::launch_pf16_gemm1_tiers(ga, grid_tiles, s));
    }
    if (ev) HIP_TRY(hipEventRecord(ev[2], s));
    HIP_TRY(moe::launch_pf16_gemm2_tiers(ga, grid_tiles, s));
    if (ev) HIP_TRY(hipEventRecord(ev[3], s));
    HIP_TRY(moe::launch_finalize(deterministic, ga.out_acc, ga.rb, I32(L.inv), T, p->K, p->topk, out, s));
    if (ev) HIP_TRY(hipEventRecord(ev[4], s));
    return MOE_OK;
  }
  int u_base = 0;
  for (int i = 0; i < n_tiers; i++) {
    const moe_experts_s *xp = tiers[i].experts;
    ga.tier = i;
    ga.u_base = u_base;
    ga.w13 = xp->w13;
    ga.s13 = prefill && xp->wfmt == MOE_W_MXFP4 ? xp->s13g : xp->s13;
    ga.w2 = xp->w2;
    ga.s2 = xp->s2;
    ga.g13 = xp->g13;
    ga.g2 = xp->g2;
    const int grid_tiles = row_tiles + std::min(xp->E, R);
    if (wide) {
      moe::GemmArgs gw = ga;
      gw.tile_rows = moe::kPfWideRows;
      gw.tile_u = I32(L.tile_u2);
      gw.tile_row0 = I32(L.tile_row02);
      gw.tier_tiles = I32(L.tier_tiles2);
      const int wtiles = (R + moe::kPfWideRows - 1) / moe::kPfWideRows + std::min(xp->E, R);
      if (xp->wfmt == MOE_W_MXFP4) HIP_TRY(moe::launch_pf_gemm1(gw, wtiles, s));
      else HIP_TRY(moe::launch_pf16_gemm1(xp->wfmt, gw, wtiles, s));
    } else if (prefill && xp->wfmt == MOE_W_MXFP4) HIP_TRY(moe::launch_pf_gemm1(ga, grid_tiles, s));
    else if (prefill) HIP_TRY(moe::launch_pf16_gemm1(xp->wfmt, ga, grid_tiles, s));
    else HIP_TRY(moe::launch_gemm1(xp->wfmt, ga, grid_tiles, s));
    u_base += xp->E;
  }
  if (ev) HIP_TRY(hipEventRecord(ev[2], s));
  u_base = 0;
  for (int i = 0; i < n_tiers; i++) {
    const moe_experts_s *xp = tiers[i].experts;
    ga.tier = i;
    ga.u_base = u_base;
    ga.w13 = xp->w13;
    ga.s13 = xp->s13;
    ga.w2 = xp->w2;
    ga.s2 = prefill && xp->wfmt == MOE_W_MXFP4 ? xp->s2g : xp->s2;
    ga.g13 = xp->g13;
    ga.g2 = xp->g2;
    const int grid_tiles = row_tiles + std::min(xp->E, R);
    if (prefill && xp->wfmt == MOE_W_MXFP4) HIP_TRY(moe::launch_pf_gemm2(ga, grid_tiles, s));
    else if (prefill) HIP_TRY(moe::launch_pf16_gemm2(xp->wfmt, ga, grid_tiles, s));
    else HIP_TRY(moe::launch_gemm2(xp->wfmt, ga, grid_tiles, s));
    u_base += xp->E;
  }
  if (ev) HIP_TRY(hipEventRecord(ev[3], s));
  HIP_TRY(moe::launch_finalize(deterministic, ga.out_acc, ga.rb, I32(L.inv), T, p->K, p->topk, out, s));
  if (ev) HIP_TRY(hipEventRecord(ev[4], s));
  return MOE_OK;
}

// Bytes per (row, 32-column group) of the data and scale tensors of a format.
void fmt_units(int wfmt, int *unit, int *sunit) {
  *unit = (wfmt == MOE_W_NF3) ? 12 : 16;
  *sunit = (wfmt == MOE_W_NVFP4) ? 2 : 1;
}

void free_prefill_scales(moe_experts_s *x) {
  for (uint8_t **p : {&x->s13g, &x->s2g}) {
    if (*p) (void)hipFree(*p);
    *p = nullptr;
  }
}

// Rewrite the four tensors between checkpoint and tile layout, a batch of
// experts at a time through a temporary device buffer.  Packing MXFP4 experts
// also writes the prefill copies of the scales (x->s13g, x->s2g, allocated
// here; their entries come before those that repack the scales themselves,
// so they read the checkpoint layout); unpacking frees them.
int permute_all(moe_experts_s *x, int to_tiles, hipStream_t s) {
  int unit, sunit;
  fmt_units(x->wfmt, &unit, &sunit);
  const bool mx = x->wfmt == MOE_W_MXFP4 && to_tiles;
  if (mx && !x->s13g) HIP_TRY(hipMalloc(&x->s13g, (size_t)x->E * x->w13_rows * (x->K / 32)));
  if (mx && !x->s2g) HIP_TRY(hipMalloc(&x->s2g, (size_t)x->E * x->K * (x->N / 32)));
  struct T {
    uint8_t *buf, *dst;   // dst: where the permuted bytes go (null: back into buf)
    int unit, rows, groups, pair, mxs;
  } tensors[6] = {{x->w13, nullptr, unit, x->w13_rows, x->K / 32, 1, 0},
                  {x->s13, mx ? x->s13g : nullptr, sunit, x->w13_rows, x->K / 32, 1, 1},
                  {x->s13, nullptr, sunit, x->w13_rows, x->K / 32, 1, 0},
                  {x->w2, nullptr, unit, x->K, x->N / 32, 0, 0},
                  {x->s2, mx ? x->s2g : nullptr, sunit, x->K, x->N / 32, 0, 1},
                  {x->s2, nullptr, sunit, x->K, x->N / 32, 0, 0}};
  size_t max_exp = 0;
  for (auto &t : tensors) max_exp = std::max(max_exp, (size_t)t.rows * t.groups * t.unit);
  const size_t budget = (size_t)256 << 20;
  const long batch = std::max<long>(1, std::min<long>(x->E, (long)(budget / max_exp)));
  // NF3 codes: unpacking leaves the kernels' sign / index form before the permutation
  if (x->wfmt == MOE_W_NF3 && !to_tiles) {
    HIP_TRY(moe::launch_nf3_recode(x->w13, (long)x->E * x->w13_rows * (x->K / 32), 0, s));
    HIP_TRY(moe::launch_nf3_recode(x->w2, (long)x->E * x->K * (x->N / 32), 0, s));
  }
  uint8_t *tmp = nullptr;
  HIP_TRY(hipMalloc(&tmp, batch * max_exp));
  int rc = MOE_OK;
  for (auto &t : tensors) {
    if (t.mxs && !t.dst) continue;   // no prefill copy (not MXFP4, or unpacking)
    const size_t exp_bytes = (size_t)t.rows * t.groups * t.unit;
    for (long e0 = 0; e0 < x->E && rc == MOE_OK; e0 += batch) {
      const long ne = std::min<long>(batch, x->E - e0);
      uint8_t *base = t.buf + e0 * exp_bytes;
      hipError_t e = hipMemcpyAsync(tmp, base, ne * exp_bytes, hipMemcpyDeviceToDevice, s);
      if (e == hipSuccess)
        e = moe::launch_permute(tmp, t.dst ? t.dst + e0 * exp_bytes : base, ne, t.unit, t.rows, t.groups, t.pair,
                                x->w13_layout == MOE_W13_GATE_UP, to_tiles, t.mxs, s);
      if (e != hipSuccess) rc = fail(MOE_EHIP, "weight permute: %s", hipGetErrorString(e));
    }
  }
  // NF3 codes: packing ends in the kernels' sign / index form
  if (rc == MOE_OK && x->wfmt == MOE_W_NF3 && to_tiles) {
    hipError_t e1 = moe::launch_nf3_recode(x->w13, (long)x->E * x->w13_rows * (x->K / 32), 1, s);
    if (e1 == hipSuccess) e1 = moe::launch_nf3_recode(x->w2, (long)x->E * x->K * (x->N / 32), 1, s);
    if (e1 != hipSuccess) rc = fail(MOE_EHIP, "nf3 recode: %s", hipGetErrorString(e1));
  }
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess && rc == MOE_OK) rc = fail(MOE_EHIP, "weight permute sync: %s", hipGetErrorString(e));
  (void)hipFree(tmp);
  if (rc != MOE_OK || !to_tiles) free_prefill_scales(x);
  return rc;
}

// T tokens in chunks of `cap` (the capacity the scratch layout L was carved
// for), each chunk on its rung's launch sequence.
int run_batch(const moe_plan_s *p, const moe_tier *tiers, int n_tiers, const void *x, const int32_t *ids,
              const float *wts, void *out, int T, int deterministic, int cap, const Layout &L, uint8_t *scratch,
              hipStream_t s, const hipEvent_t *ev = nullptr) {
  for (int t0 = 0; t0 < T; t0 += cap) {
    const int tc = std::min(cap, T - t0);
    const uint16_t *xc = (const uint16_t *)x + (size_t)t0 * p->K;
    const int32_t *idc = ids + (size_t)t0 * p->topk;
    const float *wc = wts + (size_t)t0 * p->topk;
    uint16_t *oc = (uint16_t *)out + (size_t)t0 * p->K;
    const int seq = seq_for(p, tc);
    const int rb = route_buffer(p, cap, deterministic) ? 1 : 0;   // the combine the arena was carved for
    const bool prefill = seq == MOE_SEQ_PREFILL || seq == MOE_SEQ_PREFILL_NARROW;
    const int rc = seq == MOE_SEQ_DECODE
                       ? run_decode(p, tiers, n_tiers, xc, idc, wc, oc, tc, L, scratch, s, ev)
                       : run_chunk(p, tiers, n_tiers, xc, idc, wc, oc, tc, rb, L, scratch, s, false, prefill, ev,
                                   seq == MOE_SEQ_PREFILL_NARROW);
    if (rc != MOE_OK) return rc;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

const char *moe_last_error(void) { return g_last_error.c_str(); }

int moe_plan(int E, int K, int N, int top_k, float swiglu_limit, int act_format, int w13_layout, int max_tokens,
             moe_plan_t *out) {
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  *out = nullptr;
  if (E < 1 || E > moe::kMaxExperts) return fail(MOE_EUNSUPPORTED, "E=%d outside [1, %d]", E, moe::kMaxExperts);
  if (K < 256 || K % 256) return fail(MOE_EUNSUPPORTED, "K=%d must be a positive multiple of 256", K);
  if (N < 32 || N % 32) return fail(MOE_EUNSUPPORTED, "N=%d must be a positive multiple of 32", N);
  if (top_k < 1 || top_k > 16) return fail(MOE_EINVAL, "top_k=%d outside [1, 16]", top_k);
  if (act_format != MOE_A_MXFP8 && act_format != MOE_A_BF16) return fail(MOE_EUNSUPPORTED, "act_format=%d", act_format);
  if (w13_layout != MOE_W13_UP_GATE && w13_layout != MOE_W13_GATE_UP) return fail(MOE_EINVAL, "w13_layout=%d", w13_layout);
  if (max_tokens < 1 || (long)max_tokens * top_k > (1L << 24)) return fail(MOE_EINVAL, "max_tokens=%d", max_tokens);
  moe_plan_s *p = new moe_plan_s();
  p->magic = kPlanMagic;
  p->E = E;
  p->K = K;
  p->N = N;
  p->topk = top_k;
  p->has_limit = !(isnan(swiglu_limit) || swiglu_limit <= 0.f);
  p->limit = p->has_limit ? swiglu_limit : 0.f;
  p->afmt = act_format;
  p->w13_layout = w13_layout;
  p->max_tokens = max_tokens;
  for (int c : kLadder)
    if (c < max_tokens) p->caps.push_back(c);
  p->caps.push_back(max_tokens);
  p->seq.assign(p->caps.size(), 0);
  p->comb.assign(p->caps.size(), 0);
  *out = p;
  return MOE_OK;
}

void moe_plan_destroy(moe_plan_t plan) {
  if (plan && plan->magic == kPlanMagic) {
    for (hipEvent_t e : plan->events) (void)hipEventDestroy(e);
    plan->magic = 0;
    delete plan;
  }
}

int moe_plan_set_router_weight_on_input(moe_plan_t plan, int enable) {
  if (!plan_ok(plan)) return fail(MOE_EINVAL, "invalid plan");
  if (enable && plan->afmt != MOE_A_BF16)
    return fail(MOE_EUNSUPPORTED, "router weight on the input needs bf16 activations (W4A16 / W3A16)");
  plan->w_on_input = enable ? 1 : 0;
  return MOE_OK;
}

int moe_plan_set_swiglu_oai(moe_plan_t plan, float alpha, float beta) {
  if (!plan_ok(plan)) return fail(MOE_EINVAL, "invalid plan");
  if (!std::isfinite(alpha) || !std::isfinite(beta)) return fail(MOE_EINVAL, "alpha and beta must be finite");
  const bool plain = alpha == 1.f && beta == 0.f;
  if (!plain && plan->afmt != MOE_A_BF16)
    return fail(MOE_EUNSUPPORTED, "the alpha/beta SwiGLU form needs bf16 activations (W4A16 / W3A16)");
  if (!plain && plan->act != MOE_ACT_SWIGLU) return fail(MOE_EUNSUPPORTED, "alpha and beta belong to the SwiGLU");
  plan->alpha = alpha;
  plan->beta = beta;
  return MOE_OK;
}

int moe_plan_set_activation(moe_plan_t plan, int act) {
  if (!plan_ok(plan)) return fail(MOE_EINVAL, "invalid plan");
  if (act != MOE_ACT_SWIGLU && act != MOE_ACT_SITU && act != MOE_ACT_RELU2_NO_MUL)
    return fail(MOE_EUNSUPPORTED, "activation %d", act);
  if (act != MOE_ACT_SWIGLU && (plan->has_limit || plan->alpha != 1.f || plan->beta != 0.f))
    return fail(MOE_EUNSUPPORTED, "SiTU and ReLU^2 take no swiglu limit, alpha or beta");
  if (act == MOE_ACT_RELU2_NO_MUL) {
    if (plan->afmt != MOE_A_BF16)
      return fail(MOE_EUNSUPPORTED, "ReLU^2 without the multiply needs bf16 activations (W4A16 / W3A16)");
    if (plan->N % 64) return fail(MOE_EUNSUPPORTED, "ReLU^2 without the multiply needs N %% 64 == 0");
    if (plan->w13_layout != MOE_W13_UP_GATE)
      return fail(MOE_EUNSUPPORTED, "ReLU^2 without the multiply has no gate half: w13 layout must be the default");
  }
  plan->act = act;
  // pins a rung can no longer take go back to the ladder's choice
  for (size_t r = 0; r < plan->caps.size(); r++)
    if (plan->seq[r] && !seq_eligible(plan, plan->caps[r], plan->seq[r])) plan->seq[r] = 0;
  return MOE_OK;
}

int moe_plan_enable_stage_timing(moe_plan_t plan, int max_runs) {
  if (!plan_ok(plan)) return fail(MOE_EINVAL, "invalid plan");
  if (max_runs < 0 || max_runs > 100000) return fail(MOE_EINVAL, "max_runs=%d", max_runs);
  for (hipEvent_t e : plan->events) (void)hipEventDestroy(e);
  plan->events.clear();
  plan->timing_runs = plan->timing_runs_max = 0;
  for (long i = 0; i < (long)max_runs * kStageEvents; i++) {
    // timing only: no system-scope fence (cache write-back and invalidate) at
    // each stage boundary, which would lengthen the stages it separates
    hipEvent_t e;
    HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
    plan->events.push_back(e);
  }
  plan->timing_runs_max = max_runs;
  return MOE_OK;
}

int moe_plan_stage_times(moe_plan_t plan, float *ms, int n, int *runs) {
  if (!plan_ok(plan)) return fail(MOE_EINVAL, "invalid plan");
  if (!ms || n < kStageEvents - 1) return fail(MOE_EINVAL, "need room for %d stages", kStageEvents - 1);
  for (int i = 0; i < n; i++) ms[i] = 0.f;
  for (int r = 0; r < plan->timing_runs; r++) {
    const hipEvent_t *ev = &plan->events[(size_t)r * kStageEvents];
    HIP_TRY(hipEventSynchronize(ev[kStageEvents - 1]));
    for (int i = 0; i + 1 < kStageEvents; i++) {
      float t = 0.f;
      HIP_TRY(hipEventElapsedTime(&t, ev[i], ev[i + 1]));
      ms[i] += t;
    }
  }
  if (runs) *runs = plan->timing_runs;
  plan->timing_runs = 0;
  return MOE_OK;
}

int moe_plan_capacity(moe_plan_t plan, int T, int *tile_rows) {
  if (!plan_ok(plan) || T < 0) return 0;
  const int cap = cap_for(plan, std::max(T, 1));
  if (tile_rows) {
    // the sequence a chunk of that capacity takes: decode (no route tiles), prefill, general
    const int seq = seq_for(plan, std::min(std::max(T, 1), cap));
    *tile_rows = seq == MOE_SEQ_DECODE                                           ? 0
                 : seq == MOE_SEQ_PREFILL || seq == MOE_SEQ_PREFILL_NARROW ? moe::kPfTileRows
                                                                           : moe::kTileRows;
  }
  return cap;
}

int moe_plan_set_sequence(moe_plan_t plan, int tokens, int seq) {
  if (!plan_ok(plan)) return fail(MOE_EINVAL, "invalid plan");
  if (tokens < 1) return fail(MOE_EINVAL, "tokens=%d", tokens);
  const int r = rung_of(plan, tokens), cap = plan->caps[r];
  if (seq == MOE_SEQ_AUTO) {
    plan->seq[r] = 0;
    return MOE_OK;
  }
  if (seq != MOE_SEQ_DECODE && seq != MOE_SEQ_GENERAL && seq != MOE_SEQ_PREFILL && seq != MOE_SEQ_PREFILL_NARROW)
    return fail(MOE_EINVAL, "sequence %d", seq);
  if (!seq_eligible(plan, cap, seq))
    return fail(MOE_EUNSUPPORTED, "sequence %d cannot run the %d-token capacity of this plan", seq, cap);
  plan->seq[r] = seq;
  return MOE_OK;
}

int moe_plan_set_combine(moe_plan_t plan, int tokens, int combine) {
  if (!plan_ok(plan)) return fail(MOE_EINVAL, "invalid plan");
  if (tokens < 1) return fail(MOE_EINVAL, "tokens=%d", tokens);
  if (combine != MOE_COMBINE_AUTO && combine != MOE_COMBINE_ATOMIC && combine != MOE_COMBINE_ROUTE_BUFFER)
    return fail(MOE_EINVAL, "combine %d", combine);
  plan->comb[rung_of(plan, tokens)] = combine;
  return MOE_OK;
}

int moe_plan_combine(moe_plan_t plan, int tokens) {
  if (!plan_ok(plan) || tokens < 1) return 0;
  const int cap = cap_for(plan, std::min(tokens, plan->caps.back()));
  return route_buffer(plan, cap, 0) ? MOE_COMBINE_ROUTE_BUFFER : MOE_COMBINE_ATOMIC;
}

int moe_plan_sequence(moe_plan_t plan, int tokens) {
  if (!plan_ok(plan) || tokens < 1) return 0;
  return seq_for(plan, std::min(tokens, plan->caps.back()));
}

// ---------------------------------------------------------------- tuning

namespace {

// Seeded synthetic batch for the race (splitmix64): x ~ sum of four uniforms
// (mean 0, variance 1/3) as bf16, each token's top_k distinct ids uniform over
// [0, E), positive router weights summing to 1.
uint64_t mix64(uint64_t &st) {
  uint64_t z = (st += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

double unit01(uint64_t &st) { return (double)(mix64(st) >> 11) * (1.0 / 9007199254740992.0); }

void tuning_batch(const moe_plan_s *p, int T, uint64_t seed, std::vector<uint16_t> &x, std::vector<int32_t> &ids,
                  std::vector<float> &w) {
  uint64_t st = seed;
  x.resize((size_t)T * p->K);
  for (auto &v : x) {
    const float f = (float)(unit01(st) + unit01(st) + unit01(st) + unit01(st) - 2.0);
    uint32_t b;
    memcpy(&b, &f, 4);
    v = (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
  }
  ids.resize((size_t)T * p->topk);
  w.resize(ids.size());
  const int k = std::min(p->topk, p->E);
  for (int t = 0; t < T; t++) {
    double sum = 0.0;
    for (int j = 0; j < p->topk; j++) {
      int e = -1;
      if (j < k) {
        bool dup = true;
        while (dup) {
          e = (int)(mix64(st) % (uint64_t)p->E);
          dup = false;
          for (int i = 0; i < j; i++) dup = dup || ids[(size_t)t * p->topk + i] == e;
        }
      }
      ids[(size_t)t * p->topk + j] = e;
      w[(size_t)t * p->topk + j] = (float)(0.05 + unit01(st));
      sum += w[(size_t)t * p->topk + j];
    }
    for (int j = 0; j < p->topk; j++) w[(size_t)t * p->topk + j] = (float)(w[(size_t)t * p->topk + j] / sum);
  }
}

// Device buffers of one race, freed on every path.
struct TuneBuffers {
  void *x = nullptr, *ids = nullptr, *w = nullptr, *out = nullptr, *scratch = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  ~TuneBuffers() {
    for (void *q : {x, ids, w, out, scratch})
      if (q) (void)hipFree(q);
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
  }
};

extern "C++" std::string geometry_key(const moe_plan_s *p) {
  char buf[128];
  snprintf(buf, sizeof buf, "E=%d K=%d N=%d topk=%d afmt=%d max_tokens=%d", p->E, p->K, p->N, p->topk, p->afmt,
           p->max_tokens);
  return buf;
}

}  // namespace

static int check_run_args(moe_plan_t p, const moe_tier *tiers, int n_tiers, const void *x, const int32_t *ids,
                          const float *wts, void *out, int T, void *scratch) {
  if (!plan_ok(p)) return fail(MOE_EINVAL, "invalid plan");
  if (T < 0) return fail(MOE_EINVAL, "T=%d", T);
  int rc = check_tiers(p, tiers, n_tiers);
  if (rc != MOE_OK) return rc;
  if (T == 0) return MOE_OK;
  if (!x || !ids || !wts || !out || !scratch) return fail(MOE_EINVAL, "null tensor pointer");
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(ids, 4) || !aligned(wts, 4) || !aligned(scratch, 256))
    return fail(MOE_EINVAL, "x/out need 16-byte, ids/weights 4-byte, scratch 256-byte alignment");
  return MOE_OK;
}

namespace {

// One race at the rung of `cap` tokens on a batch of T tokens already on the device:
// every launch sequence the rung can take, and for deterministic = 0 both combines
// of the planner-based sequences; pins the fastest.  us_out[kRaceSlots]: median
// microseconds of DECODE, GENERAL-atomic, GENERAL-route buffer, PREFILL-atomic,
// PREFILL-route buffer, PREFILL_NARROW-atomic, PREFILL_NARROW-route buffer (NaN
// where not raced; deterministic runs fill the route-buffer slots).
constexpr int kRaceSlots = 7;

int race_rung(moe_plan_s *plan, const moe_tier *tiers, int n_tiers, const void *x, const int32_t *ids,
              const float *wts, int T, int deterministic, int reps, hipStream_t s, float *us_out) {
  const int r = rung_of(plan, T), cap = plan->caps[r];
  struct Cand {
    int seq, comb;
  };
  const Cand cands[kRaceSlots] = {{MOE_SEQ_DECODE, 0},
                                  {MOE_SEQ_GENERAL, MOE_COMBINE_ATOMIC},
                                  {MOE_SEQ_GENERAL, MOE_COMBINE_ROUTE_BUFFER},
                                  {MOE_SEQ_PREFILL, MOE_COMBINE_ATOMIC},
                                  {MOE_SEQ_PREFILL, MOE_COMBINE_ROUTE_BUFFER},
                                  {MOE_SEQ_PREFILL_NARROW, MOE_COMBINE_ATOMIC},
                                  {MOE_SEQ_PREFILL_NARROW, MOE_COMBINE_ROUTE_BUFFER}};
  struct Restore {   // the rung's previous pins come back if the race stops early
    moe_plan_s *p;
    int r, seq, comb;
    bool armed;
    ~Restore() {
      if (armed) {
        p->seq[r] = seq;
        p->comb[r] = comb;
      }
    }
  } restore{plan, r, plan->seq[r], plan->comb[r], true};
  // one arena large enough for either combine
  plan->comb[r] = MOE_COMBINE_ROUTE_BUFFER;
  const size_t bytes_rb = layout(plan, cap, deterministic).total;
  plan->comb[r] = MOE_COMBINE_ATOMIC;
  const size_t bytes_at = layout(plan, cap, deterministic).total;
  TuneBuffers B;
  HIP_TRY(hipMalloc(&B.out, (size_t)T * plan->K * 2));
  HIP_TRY(hipMalloc(&B.scratch, std::max(bytes_rb, bytes_at)));
  HIP_TRY(hipEventCreate(&B.e0));
  HIP_TRY(hipEventCreate(&B.e1));
  int best = -1;
  float best_us = 0.f;
  for (int k = 0; k < kRaceSlots; k++) {
    float us = NAN;
    const Cand c = cands[k];
    const bool combine_matters = c.seq != MOE_SEQ_DECODE && !deterministic;
    const bool eligible = seq_eligible(plan, cap, c.seq) &&
                          (combine_matters || c.comb == 0 || c.comb == MOE_COMBINE_ROUTE_BUFFER);
    if (eligible) {
      plan->seq[r] = c.seq;
      plan->comb[r] = combine_matters ? c.comb : 0;
      const Layout L = layout(plan, cap, deterministic);
      std::vector<float> t;
      int rc = MOE_OK;
      for (int it = 0; it < reps + 2 && rc == MOE_OK; it++) {
        HIP_TRY(hipEventRecord(B.e0, s));
        rc = run_batch(plan, tiers, n_tiers, x, ids, wts, B.out, T, deterministic, cap, L, (uint8_t *)B.scratch, s);
        HIP_TRY(hipEventRecord(B.e1, s));
        HIP_TRY(hipEventSynchronize(B.e1));
        float ms = 0.f;
        HIP_TRY(hipEventElapsedTime(&ms, B.e0, B.e1));
        if (it >= 2) t.push_back(1000.f * ms);   // two warm-up runs
      }
      if (rc != MOE_OK) return rc;
      std::sort(t.begin(), t.end());
      us = t[t.size() / 2];
      if (best < 0 || us < best_us) {
        best = k;
        best_us = us;
      }
    }
    if (us_out) us_out[k] = us;
  }
  plan->seq[r] = cands[best].seq;
  plan->comb[r] = (cands[best].seq != MOE_SEQ_DECODE && !deterministic) ? cands[best].comb : restore.comb;
  restore.armed = false;
  return MOE_OK;
}

}  // namespace

int moe_plan_autotune(moe_plan_t plan, const moe_tier *tiers, int n_tiers, const int *tokens, int n, int deterministic,
                      int reps, void *stream, float *us_out) {
  if (!plan_ok(plan)) return fail(MOE_EINVAL, "invalid plan");
  int rc = check_tiers(plan, tiers, n_tiers);
  if (rc != MOE_OK) return rc;
  if (!tokens || n < 1 || reps < 1) return fail(MOE_EINVAL, "tokens, n and reps must be given");
  hipStream_t s = (hipStream_t)stream;
  for (int i = 0; i < n; i++) {
    if (tokens[i] < 1) return fail(MOE_EINVAL, "tokens[%d]=%d", i, tokens[i]);
    const int cap = plan->caps[rung_of(plan, std::min(tokens[i], plan->caps.back()))];
    std::vector<uint16_t> hx;
    std::vector<int32_t> hids;
    std::vector<float> hw;
    tuning_batch(plan, cap, 0x6D6F6521ull + (uint64_t)cap, hx, hids, hw);
    TuneBuffers B;
    HIP_TRY(hipMalloc(&B.x, hx.size() * 2));
    HIP_TRY(hipMalloc(&B.ids, hids.size() * 4));
    HIP_TRY(hipMalloc(&B.w, hw.size() * 4));
    HIP_TRY(hipMemcpy(B.x, hx.data(), hx.size() * 2, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(B.ids, hids.data(), hids.size() * 4, hipMemcpyHostToDevice));
    HIP_TRY(hipMemcpy(B.w, hw.data(), hw.size() * 4, hipMemcpyHostToDevice));
    rc = race_rung(plan, tiers, n_tiers, B.x, (const int32_t *)B.ids, (const float *)B.w, cap,
                   deterministic ? 1 : 0, reps, s, us_out ? us_out + (size_t)kRaceSlots * i : nullptr);
    if (rc != MOE_OK) return rc;
  }
  return MOE_OK;
}

int moe_plan_autotune_batch(moe_plan_t plan, const moe_tier *tiers, int n_tiers, const void *x,
                            const int32_t *topk_ids, const float *topk_weights, int T, int deterministic, int reps,
                            void *stream, float *us_out) {
  if (!plan_ok(plan)) return fail(MOE_EINVAL, "invalid plan");
  const int rc = check_tiers(plan, tiers, n_tiers);
  if (rc != MOE_OK) return rc;
  if (!x || !topk_ids || !topk_weights) return fail(MOE_EINVAL, "null tensor pointer");
  if (!aligned(x, 16) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4))
    return fail(MOE_EINVAL, "x needs 16-byte, ids/weights 4-byte alignment");
  if (T < 1 || T > plan->max_tokens) return fail(MOE_EINVAL, "T=%d outside [1, max_tokens=%d]", T, plan->max_tokens);
  if (reps < 1) return fail(MOE_EINVAL, "reps=%d", reps);
  return race_rung(plan, tiers, n_tiers, x, topk_ids, topk_weights, T, deterministic ? 1 : 0, reps,
                   (hipStream_t)stream, us_out);
}

int moe_plan_save_tuning(moe_plan_t plan, const char *path) {
  if (!plan_ok(plan) || !path) return fail(MOE_EINVAL, "invalid plan or path");
  const std::string key = geometry_key(plan);
  std::vector<std::string> keep;
  if (FILE *f = fopen(path, "r")) {   // lines of other geometries stay
    char line[512];
    while (fgets(line, sizeof line, f)) {
      std::string l(line);
      if (l.compare(0, 4, "moe ") == 0 && l.find(" " + key + " cap=") == std::string::npos) keep.push_back(l);
    }
    fclose(f);
  }
  FILE *f = fopen(path, "w");
  if (!f) return fail(MOE_EINVAL, "cannot write %s", path);
  for (auto &l : keep) fputs(l.c_str(), f);
  for (size_t r = 0; r < plan->caps.size(); r++)
    if (plan->seq[r] || plan->comb[r])
      fprintf(f, "moe v2 %s cap=%d seq=%d comb=%d\n", key.c_str(), plan->caps[r], plan->seq[r], plan->comb[r]);
  const bool ok = fclose(f) == 0;
  return ok ? MOE_OK : fail(MOE_EINVAL, "cannot write %s", path);
}

int moe_plan_load_tuning(moe_plan_t plan, const char *path) {
  if (!plan_ok(plan) || !path) return fail(MOE_EINVAL, "invalid plan or path");
  FILE *f = fopen(path, "r");
  if (!f) return fail(MOE_EINVAL, "cannot read %s", path);
  const std::string key = geometry_key(plan) + " cap=";
  const std::string v1 = "moe v1 " + key, v2 = "moe v2 " + key;
  char line[512];
  int applied = 0;
  while (fgets(line, sizeof line, f)) {
    int cap = 0, seq = 0, comb = 0;
    if (strncmp(line, v2.c_str(), v2.size()) == 0) {
      if (sscanf(line + v2.size(), "%d seq=%d comb=%d", &cap, &seq, &comb) != 3) continue;
    } else if (strncmp(line, v1.c_str(), v1.size()) == 0) {   // sequence pins only
      if (sscanf(line + v1.size(), "%d seq=%d", &cap, &seq) != 2) continue;
    } else {
      continue;
    }
    const int r = rung_of(plan, cap);
    if (plan->caps[r] != cap || (seq && !seq_eligible(plan, cap, seq)) || comb < 0 ||
        comb > MOE_COMBINE_ROUTE_BUFFER)
      continue;   // stale or foreign entry
    plan->seq[r] = seq;
    plan->comb[r] = comb;
    applied++;
  }
  fclose(f);
  return applied;
}

size_t moe_scratch_bytes(moe_plan_t plan, int tokens, int deterministic) {
  if (!plan_ok(plan) || tokens < 0) return 0;
  const int cap = cap_for(plan, std::max(1, std::min(tokens, plan->max_tokens)));
  return layout(plan, cap, deterministic ? 1 : 0).total;
}

int moe_prepare_weights(moe_plan_t plan, int weight_format, int num_experts, void *w13, void *s13, const float *g13,
                        void *w2, void *s2, const float *g2, void *stream, moe_experts_t *out) {
  if (!out) return fail(MOE_EINVAL, "out is NULL");
  *out = nullptr;
  if (!plan_ok(plan)) return fail(MOE_EINVAL, "invalid plan");
  if (weight_format != MOE_W_MXFP4 && weight_format != MOE_W_NVFP4 && weight_format != MOE_W_NF3)
    return fail(MOE_EUNSUPPORTED, "weight_format=%d", weight_format);
  const int want_a = (weight_format == MOE_W_MXFP4) ? MOE_A_MXFP8 : MOE_A_BF16;
  if (want_a != plan->afmt)
    return fail(MOE_EUNSUPPORTED, "weight format %d needs activation format %d, plan has %d", weight_format, want_a,
                plan->afmt);
  if (num_experts < 1 || num_experts > moe::kMaxExperts) return fail(MOE_EINVAL, "num_experts=%d", num_experts);
  if (!w13 || !s13 || !w2 || !s2) return fail(MOE_EINVAL, "null weight pointer");
  if (!aligned(w13, 16) || !aligned(w2, 16) || !aligned(s13, 4) || !aligned(s2, 4))
    return fail(MOE_EINVAL, "weights must be 16-byte aligned, scales 4-byte aligned");
  if ((g13 && !aligned(g13, 4)) || (g2 && !aligned(g2, 4))) return fail(MOE_EINVAL, "misaligned global scales");
  if (weight_format != MOE_W_NVFP4 && (g13 || g2)) return fail(MOE_EINVAL, "global scales are NVFP4-only");
  moe_experts_s *x = new moe_experts_s();
  x->magic = kExpertsMagic;
  x->K = plan->K;
  x->N = plan->N;
  x->w13_layout = plan->w13_layout;
  x->w13_rows = w13_rows(plan);
  x->wfmt = weight_format;
  x->E = num_experts;
  x->w13 = (uint8_t *)w13;
  x->s13 = (uint8_t *)s13;
  x->w2 = (uint8_t *)w2;
  x->s2 = (uint8_t *)s2;
  x->s13g = x->s2g = nullptr;
  x->g13 = g13;
  x->g2 = g2;
  x->prepared = 0;
  const int rc = permute_all(x, 1, (hipStream_t)stream);
  if (rc != MOE_OK) {
    x->magic = 0;
    free_prefill_scales(x);
    delete x;
    return rc;
  }
  x->prepared = 1;
  *out = x;
  return MOE_OK;
}

int moe_unpack_weights(moe_experts_t x, void *stream) {
  if (!x || x->magic != kExpertsMagic) return fail(MOE_EINVAL, "invalid experts handle");
  if (!x->prepared) return fail(MOE_ENOTPREPARED, "experts are already in checkpoint layout");
  const int rc = permute_all(x, 0, (hipStream_t)stream);
  if (rc == MOE_OK) x->prepared = 0;
  return rc;
}

void moe_experts_destroy(moe_experts_t x) {
  if (x && x->magic == kExpertsMagic) {
    x->magic = 0;
    free_prefill_scales(x);
    delete x;
  }
}

int moe_run(moe_plan_t p, const moe_tier *tiers, int n_tiers, const void *x, const int32_t *ids,
            const float *wts, void *out, int T, int deterministic, void *scratch, size_t scratch_bytes,
            void *stream) {
  int rc = check_run_args(p, tiers, n_tiers, x, ids, wts, out, T, scratch);
  if (rc != MOE_OK || T == 0) return rc;
  deterministic = deterministic ? 1 : 0;
  const int chunk = p->caps.back();
  const int cap = cap_for(p, std::min(T, chunk));
  const Layout L = layout(p, cap, deterministic);
  if (scratch_bytes < L.total)
    return fail(MOE_ESCRATCH, "scratch of %zu bytes; %zu needed for %d tokens", scratch_bytes, L.total, T);
  hipStream_t s = (hipStream_t)stream;
  // stage timing covers single-chunk runs only
  const hipEvent_t *ev = nullptr;
  if (p->timing_runs < p->timing_runs_max && T <= cap) {
    ev = &p->events[(size_t)p->timing_runs * kStageEvents];
    p->timing_runs++;
  }
  return run_batch(p, tiers, n_tiers, x, ids, wts, out, T, deterministic, cap, L, (uint8_t *)scratch, s, ev);
}

int moe_debug_route(moe_plan_t p, const moe_tier *tiers, int n_tiers, const int32_t *ids, int T, void *scratch,
                    size_t scratch_bytes, int32_t *cnt, int32_t *off, int32_t *perm, int32_t *inv, void *stream) {
  if (!plan_ok(p)) return fail(MOE_EINVAL, "invalid plan");
  int rc = check_tiers(p, tiers, n_tiers);
  if (rc != MOE_OK) return rc;
  if (T < 1 || T > p->max_tokens) return fail(MOE_EINVAL, "T=%d outside [1, max_tokens=%d]", T, p->max_tokens);
  if (!ids || !scratch || !cnt || !off || !perm || !inv) return fail(MOE_EINVAL, "null pointer");
  if (!aligned(scratch, 256)) return fail(MOE_EINVAL, "scratch needs 256-byte alignment");
  const int cap = cap_for(p, T);
  const Layout L = layout(p, cap, 1);
  if (scratch_bytes < L.total) return fail(MOE_ESCRATCH, "scratch of %zu bytes; %zu needed", scratch_bytes, L.total);
  hipStream_t s = (hipStream_t)stream;
  rc = run_chunk(p, tiers, n_tiers, nullptr, ids, nullptr, nullptr, T, 1, L, (uint8_t *)scratch, s, true, false);
  if (rc != MOE_OK) return rc;
  int U = 0;
  for (int i = 0; i < n_tiers; i++) U += tiers[i].experts->E;
  const size_t R = (size_t)T * p->topk;
  uint8_t *sc = (uint8_t *)scratch;
  HIP_TRY(hipMemcpyAsync(cnt, sc + L.cnt, 4 * (size_t)U, hipMemcpyDeviceToDevice, s));
  HIP_TRY(hipMemcpyAsync(off, sc + L.off, 4 * (size_t)(U + 1), hipMemcpyDeviceToDevice, s));
  HIP_TRY(hipMemcpyAsync(perm, sc + L.perm, 4 * R, hipMemcpyDeviceToDevice, s));
  HIP_TRY(hipMemcpyAsync(inv, sc + L.inv, 4 * R, hipMemcpyDeviceToDevice, s));
  return MOE_OK;
}

int moe_ep_remap(const int32_t *topk_ids, const float *topk_weights, int T, int top_k, long long offset,
                 int num_local, int32_t *out_ids, float *out_weights, void *stream) {
  if (T < 0) return fail(MOE_EINVAL, "T=%d", T);
  if (top_k < 1 || top_k > 64) return fail(MOE_EINVAL, "top_k=%d outside [1, 64]", top_k);
  if (num_local < 1) return fail(MOE_EINVAL, "num_local=%d", num_local);
  if (T == 0) return MOE_OK;
  if (!topk_ids || !topk_weights || !out_ids || !out_weights) return fail(MOE_EINVAL, "null pointer");
  if (!aligned(topk_ids, 4) || !aligned(topk_weights, 4) || !aligned(out_ids, 4) || !aligned(out_weights, 4))
    return fail(MOE_EINVAL, "ids and weights need 4-byte alignment");
  HIP_TRY(moe::launch_ep_remap(topk_ids, topk_weights, T, top_k, (long)offset, num_local, out_ids, out_weights,
                               (hipStream_t)stream));
  return MOE_OK;
}

int moe_debug_quant_mxfp8_bf16(const void *x, int rows, int cols, uint8_t *q, uint8_t *scales, void *stream) {
  if (rows < 0 || cols < 32 || cols % 32) return fail(MOE_EINVAL, "cols must be a positive multiple of 32");
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scales || !aligned(x, 16) || !aligned(q, 16)) return fail(MOE_EINVAL, "null or misaligned pointer");
  HIP_TRY(moe::launch_quant_bf16((const uint16_t *)x, rows, cols, q, scales, (hipStream_t)stream));
  return MOE_OK;
}

int moe_debug_quant_mxfp8_f32(const float *h, int rows, int cols, uint8_t *q, uint8_t *scales, void *stream) {
  if (rows < 0 || cols < 32 || cols % 32) return fail(MOE_EINVAL, "cols must be a positive multiple of 32");
  if (rows == 0) return MOE_OK;
  if (!h || !q || !scales || !aligned(h, 16) || !aligned(q, 16)) return fail(MOE_EINVAL, "null or misaligned pointer");
  HIP_TRY(moe::launch_quant_f32(h, rows, cols, q, scales, (hipStream_t)stream));
  return MOE_OK;
}

}  // extern "C"
