/*
 * CPU oracle for the routed mixture-of-experts layer with block-scaled 4-bit
 * expert weights.  TEST INFRASTRUCTURE ONLY: it is loaded by the test suite,
 * by the package's smoke check and by the benchmark's CPU-baseline leg, never
 * by the product path.  It shares no code, table or constant with the HIP
 * library: every format is decoded here from its definition.
 *
 * Plain and slow on purpose: one routed token at a time, weights decoded
 * element by element, dot products accumulated in double precision in
 * ascending index order.  Quantisation decisions are taken on fp32 values,
 * the precision the GPU kernels take them in.
 *
 * Sources (the pages are the sglang adapter "moe_b12x_next.py", the vLLM
 * loader "hybrid_loader.py" and the vLLM "B12xExperts" API page):
 *  - E8M0 block scale = 2^(byte-127): hybrid_loader.py, _fp8_ne_transform._deq.
 *  - E2M1 code and the MXFP4 checkpoint layout (two codes per byte, one E8M0
 *    scale per 32 along K): moe_b12x_next.py, module docstring and
 *    _convert_layer; the 16-value E2M1 table is the OCP MX format.
 *  - NVFP4 (E2M1 x E4M3 per 16 x fp32 global): hybrid_loader.py, _deq_nv and
 *    create_weights.
 *  - NF3 (3-bit codebook index, 8 codes in 3 little-endian bytes, E4M3 per
 *    32): hybrid_loader.py, _NF3_VALS and _unpack_nf3.
 *  - w13 stacked [up; gate]: moe_b12x_next.py, module docstring.
 *  - reference forward (per expert: x W13^T split, silu(gate)*up, W2, weight
 *    by router weight, sum into the token): hybrid_loader.py, _apply_ref.
 *  - ids outside [0,E) (CUDA-graph padding -1) contribute nothing:
 *    moe_b12x_next.py, module docstring (_DIRECT_IDS).
 *  - SwiGLU limit: B12xExperts._swiglu_params (the clamp's form is not printed;
 *    this file takes gate <- min(gate, L), up <- clamp(up, -L, L)).
 *  - SwiGLU-OAI alpha and beta: the same method returns them for the
 *    swigluoai activation only, and _supports_activation / the W4A8 check
 *    refuse that activation with quantised activations.  The activation's
 *    formula is not printed; this file takes gate * sigmoid(alpha gate) *
 *    (up + beta) after the clamps (alpha = 1, beta = 0 is the plain SwiGLU).
 *  - SiTU and ReLU^2 without the gate multiply: the same page lists them among
 *    the supported activations (_supports_activation; the W4A8 check allows
 *    SiLU and SiTU only; the support check takes SiTU with beta 4 and linear
 *    beta 25 only; _swiglu_params gives neither a limit).  Their formulas are
 *    not printed.  This file takes SiTU as the SwiGLU with both branches
 *    softly capped by tanh, silu(b tanh(gate / b)) * (bl tanh(up / bl)) with
 *    b = 4, bl = 25, and ReLU^2 without the multiply as relu(z)^2 on a w13 of
 *    N rows (no gate half).
 *  - EP id remap (moe_b12x_next.py, ep_remap / ep_remap_reference): local id
 *    = global id - offset when that lies in [0, num_local); every other slot
 *    takes weight 0 and the row's lowest local id (else the batch's lowest,
 *    else 0).
 *  - MXFP8 activations (E4M3 codes + E8M0 scale per 32): moe_b12x_next.py,
 *    module docstring ("in-kernel MXFP8 activations"); the scale rule is the
 *    OCP MX one, E = floor(log2 amax) - emax(E4M3 = 8), codes saturate.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_FMT_MXFP4 1
#define ORC_FMT_NVFP4 2
#define ORC_FMT_NF3 3

/* ---------------------------------------------------------------- decode */

/* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa. */
double orc_e2m1(unsigned code) {
  unsigned e = (code >> 1) & 3u, m = code & 1u;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, (int)e - 1);
  return (code & 8u) ? -v : v;
}

/* E8M0: a bare biased exponent, 2^(b-127); 0xFF is NaN. */
double orc_e8m0(unsigned b) {
  if ((b & 0xFFu) == 0xFFu) return NAN;
  return ldexp(1.0, (int)(b & 0xFFu) - 127);
}

/* E4M3 (fn variant): bias 7, subnormals m/8 * 2^-6, S.1111.111 is NaN, no inf. */
double orc_e4m3(unsigned b) {
  unsigned s = (b >> 7) & 1u, e = (b >> 3) & 15u, m = b & 7u;
  double v;
  if (e == 15 && m == 7) return NAN;
  v = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, (int)e - 7);
  return s ? -v : v;
}

/* NF3 codebook, the decimals printed on the page, in fp32. */
static const float orc_nf3_book[8] = {-1.0f, -0.6047f, -0.3563f, -0.1275f,
                                      0.1275f, 0.3563f, 0.6047f, 1.0f};
double orc_nf3(unsigned code) { return (double)orc_nf3_book[code & 7u]; }

/* bf16 <-> double.  bf16 is the upper half of an fp32. */
double orc_bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest bf16 (ties to even), returned as bits. */
uint16_t orc_bf16_from_double(double d) {
  float f;
  uint32_t u;
  int ex;
  double r;
  if (isnan(d)) return 0x7FC0;
  if (d == 0.0) return signbit(d) ? 0x8000 : 0x0000;
  frexp(d, &ex); /* |d| = f * 2^ex, f in [0.5, 1): 8 significant bits -> spacing 2^(ex-8) */
  if (ex - 8 < -133) ex = -133 + 8; /* bf16 subnormal spacing is 2^-133 */
  r = nearbyint(ldexp(d, 8 - ex));  /* default rounding mode: ties to even */
  r = ldexp(r, ex - 8);
  if (fabs(r) > 3.3895313892515355e38) return signbit(d) ? 0xFF80 : 0x7F80; /* overflow -> inf */
  f = (float)r; /* exact: r has at most 8 significant bits */
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

/* ---------------------------------------------------- E4M3 / MXFP8 encode */

static double orc_e4m3_pos[127]; /* values of codes 0x00..0x7E, ascending */
static int orc_tables_ready = 0;

__attribute__((constructor)) static void orc_init_tables(void) {
  int c;
  if (orc_tables_ready) return;
  for (c = 0; c < 127; c++) orc_e4m3_pos[c] = orc_e4m3((unsigned)c);
  orc_tables_ready = 1;
}

/* Nearest E4M3 code to v (ties to the even code), magnitudes above 448 saturate
   to 448.  Binary search over the ascending code values. */
unsigned orc_e4m3_encode(double v) {
  unsigned sign = signbit(v) ? 0x80u : 0u;
  double a = fabs(v);
  int lo = 0, hi = 126, c;
  if (isnan(v)) return 0x7Fu;
  if (a >= orc_e4m3_pos[126]) return sign | 126u;
  while (hi - lo > 1) { /* invariant: pos[lo] <= a < pos[hi] */
    int mid = (lo + hi) / 2;
    if (orc_e4m3_pos[mid] <= a) lo = mid; else hi = mid;
  }
  {
    double dlo = a - orc_e4m3_pos[lo], dhi = orc_e4m3_pos[hi] - a;
    if (dlo < dhi) c = lo;
    else if (dhi < dlo) c = hi;
    else c = (lo % 2 == 0) ? lo : hi;
  }
  return sign | (unsigned)c;
}

/* MXFP8 of one block of 32 fp32 values: shared exponent E = floor(log2 amax) - 8
   clamped to [-127, 127] (amax = 0 gives E = -127), scale byte E + 127,
   q_i = nearest E4M3 of v_i * 2^-E with saturation. */
static void orc_mxfp8_block(const float *v, uint8_t *q, uint8_t *scale) {
  double amax = 0.0;
  int i, E, ex;
  for (i = 0; i < 32; i++) if (fabs((double)v[i]) > amax) amax = fabs((double)v[i]);
  if (amax == 0.0) {
    E = -127;
  } else {
    frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5,1) -> floor(log2 amax) = ex - 1 */
    E = ex - 1 - 8;
    if (E < -127) E = -127;
    if (E > 127) E = 127;
  }
  *scale = (uint8_t)(E + 127);
  for (i = 0; i < 32; i++) q[i] = (uint8_t)orc_e4m3_encode(ldexp((double)v[i], -E));
}

/* Row-major [rows, cols] fp32 -> codes [rows, cols] and scales [rows, cols/32]. */
int orc_mxfp8_quantize_f32(const float *v, long rows, long cols, uint8_t *q, uint8_t *s) {
  long r, b;
  if (cols % 32) return -1;
  for (r = 0; r < rows; r++)
    for (b = 0; b < cols / 32; b++)
      orc_mxfp8_block(v + r * cols + b * 32, q + r * cols + b * 32, s + r * (cols / 32) + b);
  return 0;
}

int orc_mxfp8_quantize_bf16(const uint16_t *x, long rows, long cols, uint8_t *q, uint8_t *s) {
  long r, b;
  int i;
  float blk[32];
  if (cols % 32) return -1;
  for (r = 0; r < rows; r++)
    for (b = 0; b < cols / 32; b++) {
      for (i = 0; i < 32; i++) blk[i] = (float)orc_bf16_to_double(x[r * cols + b * 32 + i]);
      orc_mxfp8_block(blk, q + r * cols + b * 32, s + r * (cols / 32) + b);
    }
  return 0;
}

/* ---------------------------------------------------------- weight rows */

/* Decode row `row` of a checkpoint weight matrix with `cols` logical columns into
   out[cols] (double).  g is the per-tensor global (NVFP4; 1 otherwise). */
static void orc_decode_row(int fmt, const uint8_t *w, const uint8_t *s, double g, long row, long cols,
                           double *out) {
  long c;
  if (fmt == ORC_FMT_MXFP4) {
    const uint8_t *wr = w + row * (cols / 2), *sr = s + row * (cols / 32);
    for (c = 0; c < cols; c++) {
      unsigned byte = wr[c / 2], code = (c % 2 == 0) ? (byte & 15u) : (byte >> 4);
      out[c] = orc_e2m1(code) * orc_e8m0(sr[c / 32]);
    }
  } else if (fmt == ORC_FMT_NVFP4) {
    const uint8_t *wr = w + row * (cols / 2), *sr = s + row * (cols / 16);
    for (c = 0; c < cols; c++) {
      unsigned byte = wr[c / 2], code = (c % 2 == 0) ? (byte & 15u) : (byte >> 4);
      out[c] = orc_e2m1(code) * orc_e4m3(sr[c / 16]) * g;
    }
  } else { /* NF3: 8 codes per 3 bytes, code i = bits 3i..3i+2 of b0 | b1<<8 | b2<<16 */
    const uint8_t *wr = w + row * (cols / 8 * 3), *sr = s + row * (cols / 32);
    for (c = 0; c < cols; c++) {
      const uint8_t *grp = wr + (c / 8) * 3;
      uint32_t w24 = (uint32_t)grp[0] | ((uint32_t)grp[1] << 8) | ((uint32_t)grp[2] << 16);
      unsigned code = (w24 >> (3 * (c % 8))) & 7u;
      out[c] = orc_nf3(code) * orc_e4m3(sr[c / 32]);
    }
  }
}

/* Dequantise whole [rows, cols] matrices (for tests). */
int orc_dequant(int fmt, const uint8_t *w, const uint8_t *s, double g, long rows, long cols, double *out) {
  long r;
  if (fmt < 1 || fmt > 3 || cols % 32) return -1;
  for (r = 0; r < rows; r++) orc_decode_row(fmt, w, s, g, r, cols, out + r * cols);
  return 0;
}

/* -------------------------------------------------------------- routing */

typedef struct {
  int fmt;              /* ORC_FMT_* */
  int E;                /* experts held by this tier */
  const int32_t *emap;  /* [E_global]: global id -> local id or -1; NULL = identity */
  const uint8_t *w13, *s13;
  const float *g13;     /* [E] NVFP4 globals, NULL = 1 */
  const uint8_t *w2, *s2;
  const float *g2;
} orc_tier;

/* Which tier and local expert a global id goes to; -1 when no tier holds it. */
static int orc_resolve(int32_t id, int E_global, int n_tiers, const orc_tier *tiers, int *local) {
  int i;
  if (id < 0 || id >= E_global) return -1;
  for (i = 0; i < n_tiers; i++) {
    int32_t e = tiers[i].emap ? tiers[i].emap[id] : id;
    if (e >= 0 && e < tiers[i].E) { *local = e; return i; }
  }
  return -1;
}

/* Route planner's plain definition.  Experts of all tiers form one index space
   u = (experts of earlier tiers) + local id.  cnt[u] = routes to u; off = exclusive
   prefix sum (U+1 entries); perm lists the valid route indices r = t*k + j in
   (u ascending, r ascending) order -- a stable counting sort; inv[r] is r's
   position in perm, or -1 for a skipped slot.  Returns the valid route count. */
long orc_route(const int32_t *ids, long T, int topk, int E_global, int n_tiers, const orc_tier *tiers,
               int32_t *cnt, int32_t *off, int32_t *perm, int32_t *inv) {
  long R = T * topk, r, U = 0, u, nvalid = 0;
  int i, base[8];
  int32_t *fill;
  if (n_tiers < 1 || n_tiers > 8) return -1;
  for (i = 0; i < n_tiers; i++) {
    if (tiers[i].E < 1) return -1;
    base[i] = (int)U;
    U += tiers[i].E;
  }
  if (U < 1 || U > (1L << 24)) return -1;
  for (u = 0; u < U; u++) cnt[u] = 0;
  for (r = 0; r < R; r++) {
    int local, t = orc_resolve(ids[r], E_global, n_tiers, tiers, &local);
    if (t >= 0) cnt[base[t] + local]++;
  }
  off[0] = 0;
  for (u = 0; u < U; u++) off[u + 1] = off[u] + cnt[u];
  fill = (int32_t *)calloc((size_t)U, sizeof(int32_t));
  if (!fill) return -1;
  for (r = 0; r < R; r++) {
    int local, t = orc_resolve(ids[r], E_global, n_tiers, tiers, &local);
    if (t < 0) { inv[r] = -1; continue; }
    u = base[t] + local;
    perm[off[u] + fill[u]] = (int32_t)r;
    inv[r] = off[u] + fill[u];
    fill[u]++;
    nvalid++;
  }
  free(fill);
  return nvalid;
}

/* ------------------------------------------------------------ activation */

#define ORC_ACT_SWIGLU 0      /* silu(gate) * up after the limit clamps; alpha / beta: OAI form */
#define ORC_ACT_SITU 1        /* silu(4 tanh(gate/4)) * 25 tanh(up/25) */
#define ORC_ACT_RELU2_NO_MUL 2 /* relu(z)^2 on a w13 of N rows */

/* The activation of one intermediate column.  SwiGLU: when limit is not NaN,
   gate <- min(gate, limit) and up <- clamp(up, -limit, limit) first, then
   gate * sigmoid(alpha gate) * (up + beta) (alpha = 1, beta = 0: silu(gate) * up).
   SiTU: both branches softly capped, silu(4 tanh(gate/4)) * (25 tanh(up/25)).
   ReLU^2 without the multiply: relu(up)^2 (gate unused). */
double orc_act(int act, double gate, double up, double limit, double alpha, double beta) {
  if (act == ORC_ACT_RELU2_NO_MUL) return up > 0.0 ? up * up : 0.0;
  if (act == ORC_ACT_SITU) {
    double g = 4.0 * tanh(gate / 4.0), u = 25.0 * tanh(up / 25.0);
    return g / (1.0 + exp(-g)) * u;
  }
  if (!isnan(limit)) {
    if (gate > limit) gate = limit;
    if (up > limit) up = limit;
    if (up < -limit) up = -limit;
  }
  return gate / (1.0 + exp(-alpha * gate)) * (up + beta);
}

/* ------------------------------------------------------------- EP remap */

/* Expert-parallel id remap of one batch [T, k]: lid = id - offset.  A slot whose
   lid lies in [0, num_local) keeps lid and its weight; every other slot (another
   rank's expert, padding) gets weight 0 and a fill id: the lowest valid lid of
   its row, else the lowest valid lid of the batch, else 0.  Ids are compared in
   64-bit so that id - offset cannot wrap. */
int orc_ep_remap(const int32_t *ids, const float *w, long T, int topk, long offset, long num_local,
                 int32_t *out_ids, float *out_w) {
  long t, j, best = -1;
  if (T < 0 || topk < 1 || num_local < 1) return -1;
  for (t = 0; t < T * topk; t++) {
    long lid = (long)ids[t] - offset;
    if (lid >= 0 && lid < num_local && (best < 0 || lid < best)) best = lid;
  }
  for (t = 0; t < T; t++) {
    long row_min = -1, fill;
    for (j = 0; j < topk; j++) {
      long lid = (long)ids[t * topk + j] - offset;
      if (lid >= 0 && lid < num_local && (row_min < 0 || lid < row_min)) row_min = lid;
    }
    fill = row_min >= 0 ? row_min : (best >= 0 ? best : 0);
    for (j = 0; j < topk; j++) {
      long lid = (long)ids[t * topk + j] - offset;
      int ok = lid >= 0 && lid < num_local;
      out_ids[t * topk + j] = (int32_t)(ok ? lid : fill);
      out_w[t * topk + j] = ok ? w[t * topk + j] : 0.0f;
    }
  }
  return 0;
}

/* ---------------------------------------------------------------- layer */

/* One routed token through its expert: returns y[K] (double) for activation xh[K]. */
static void orc_expert(const orc_tier *tier, int e, int K, int N, int act, double limit, double alpha,
                       double beta, int gate_up, const double *xh, double *y, double *rowbuf, double *h) {
  int n, c, k;
  int a8 = tier->fmt == ORC_FMT_MXFP4;
  double g13 = tier->g13 ? (double)tier->g13[e] : 1.0, g2 = tier->g2 ? (double)tier->g2[e] : 1.0;
  long w13_row_bytes = (tier->fmt == ORC_FMT_NF3) ? (long)K / 8 * 3 : (long)K / 2;
  long s13_row_bytes = (tier->fmt == ORC_FMT_NVFP4) ? (long)K / 16 : (long)K / 32;
  long w2_row_bytes = (tier->fmt == ORC_FMT_NF3) ? (long)N / 8 * 3 : (long)N / 2;
  long s2_row_bytes = (tier->fmt == ORC_FMT_NVFP4) ? (long)N / 16 : (long)N / 32;
  /* w13 holds 2N rows ([up; gate] or [gate; up]), N rows for ReLU^2 without the multiply */
  int w13_rows = (act == ORC_ACT_RELU2_NO_MUL) ? N : 2 * N;
  const uint8_t *w13 = tier->w13 + (size_t)e * w13_rows * w13_row_bytes;
  const uint8_t *s13 = tier->s13 + (size_t)e * w13_rows * s13_row_bytes;
  const uint8_t *w2 = tier->w2 + (size_t)e * K * w2_row_bytes;
  const uint8_t *s2 = tier->s2 + (size_t)e * K * s2_row_bytes;
  float hf[32];
  uint8_t q[32], sc;

  /* GEMM1 + activation (orc_act); ReLU^2 without the multiply has no gate row */
  for (n = 0; n < N; n++) {
    double up = 0.0, gate = 0.0;
    int up_row = (act == ORC_ACT_RELU2_NO_MUL) ? n : (gate_up ? N + n : n), gate_row = gate_up ? n : N + n;
    orc_decode_row(tier->fmt, w13, s13, g13, up_row, K, rowbuf);
    for (k = 0; k < K; k++) up += rowbuf[k] * xh[k];
    if (act != ORC_ACT_RELU2_NO_MUL) {
      orc_decode_row(tier->fmt, w13, s13, g13, gate_row, K, rowbuf);
      for (k = 0; k < K; k++) gate += rowbuf[k] * xh[k];
    }
    h[n] = orc_act(act, gate, up, limit, alpha, beta);
  }
  /* requantiser between the GEMMs: MXFP8 on fp32 h (A8), bf16 (A16) */
  if (a8) {
    for (n = 0; n < N; n += 32) {
      for (c = 0; c < 32; c++) hf[c] = (float)h[n + c];
      orc_mxfp8_block(hf, q, &sc);
      for (c = 0; c < 32; c++) h[n + c] = orc_e4m3(q[c]) * orc_e8m0(sc);
    }
  } else {
    for (n = 0; n < N; n++) h[n] = orc_bf16_to_double(orc_bf16_from_double(h[n]));
  }
  /* GEMM2 */
  for (c = 0; c < K; c++) {
    double acc = 0.0;
    orc_decode_row(tier->fmt, w2, s2, g2, c, N, rowbuf);
    for (n = 0; n < N; n++) acc += rowbuf[n] * h[n];
    y[c] = acc;
  }
}

/*
 * The layer, for the token rows listed in rows[0..nrows) (pass rows = NULL and
 * nrows = T for all of them).  For each listed token t:
 *   acc[c] = sum over slots j = 0..k-1 with a valid id of w[t,j] * y_j[c],
 * in slot order, then out = bf16(acc).  A row with no valid slot is exactly 0.
 * Activation path follows the weight format: MXFP4 quantises x and h to MXFP8
 * (W4A8); NVFP4 and NF3 keep x in bf16 and round h to bf16 (W4A16 / W3A16).
 * limit: NaN = no clamp.  alpha, beta: the activation's form (1, 0 = SwiGLU;
 * other values 16-bit activation formats only).  gate_up = 1 when w13 is
 * stacked [gate; up].
 * acc [nrows, K] and out [nrows, K] are written.  Returns 0, or -1 on bad args.
 */
int orc_moe_act(int E_global, int K, int N, int topk, double limit, int gate_up, int n_tiers,
                const orc_tier *tiers, const uint16_t *x, const int32_t *ids, const float *wts, long T,
                const int32_t *rows, long nrows, double *acc, uint16_t *out, int weight_on_input, double alpha,
                double beta, int act) {
  long i;
  int bad = 0, tt;
  if (K % 32 || N % 32 || topk < 1 || n_tiers < 1 || n_tiers > 8) return -1;
  if (act < ORC_ACT_SWIGLU || act > ORC_ACT_RELU2_NO_MUL) return -1;
  /* SiTU and ReLU^2 take no limit, alpha or beta (vLLM "fused_moe/b12x" page, _swiglu_params) */
  if (act != ORC_ACT_SWIGLU && (!isnan(limit) || alpha != 1.0 || beta != 0.0)) return -1;
  /* the router weight on the input, the OAI form and ReLU^2 exist for the 16-bit activation
     path only (same page: process_weights_after_loading, the W4A8 activation check) */
  if (weight_on_input || alpha != 1.0 || beta != 0.0 || act == ORC_ACT_RELU2_NO_MUL)
    for (tt = 0; tt < n_tiers; tt++)
      if (tiers[tt].fmt == ORC_FMT_MXFP4) return -1;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (i = 0; i < nrows; i++) {
    long t = rows ? rows[i] : i;
    double *xh = (double *)malloc(sizeof(double) * K), *y = (double *)malloc(sizeof(double) * K);
    double *rowbuf = (double *)malloc(sizeof(double) * (K > N ? K : N));
    double *h = (double *)malloc(sizeof(double) * N);
    double *a = acc + i * K;
    int j, c, have_a8 = 0, have_a16 = 0;
    double *xa8 = (double *)malloc(sizeof(double) * K);
    double *xw = (double *)malloc(sizeof(double) * K);
    if (!xh || !y || !rowbuf || !h || !xa8 || !xw || t < 0 || t >= T) {
      bad = 1;
    } else {
      uint8_t q[32], sc;
      float blk[32];
      for (c = 0; c < K; c++) a[c] = 0.0;
      for (j = 0; j < topk; j++) {
        int local, tt = orc_resolve(ids[t * topk + j], E_global, n_tiers, tiers, &local);
        const double *xin;
        if (tt < 0) continue;
        if (tiers[tt].fmt == ORC_FMT_MXFP4) {
          if (!have_a8) { /* MXFP8 fake-quantised activation, once per token */
            int b;
            for (b = 0; b < K; b += 32) {
              for (c = 0; c < 32; c++) blk[c] = (float)orc_bf16_to_double(x[t * K + b + c]);
              orc_mxfp8_block(blk, q, &sc);
              for (c = 0; c < 32; c++) xa8[b + c] = orc_e4m3(q[c]) * orc_e8m0(sc);
            }
            have_a8 = 1;
          }
          xin = xa8;
        } else {
          if (!have_a16) {
            for (c = 0; c < K; c++) xh[c] = orc_bf16_to_double(x[t * K + c]);
            have_a16 = 1;
          }
          xin = xh;
        }
        if (weight_on_input) {
          /* the slot's copy of the token is scaled before GEMM1; its result enters with weight 1 */
          for (c = 0; c < K; c++) xw[c] = (double)wts[t * topk + j] * xin[c];
          orc_expert(&tiers[tt], local, K, N, act, limit, alpha, beta, gate_up, xw, y, rowbuf, h);
          for (c = 0; c < K; c++) a[c] += y[c];
        } else {
          orc_expert(&tiers[tt], local, K, N, act, limit, alpha, beta, gate_up, xin, y, rowbuf, h);
          for (c = 0; c < K; c++) a[c] += (double)wts[t * topk + j] * y[c];
        }
      }
      for (c = 0; c < K; c++) out[i * K + c] = orc_bf16_from_double(a[c]);
    }
    free(xh); free(y); free(rowbuf); free(h); free(xa8); free(xw);
  }
  return bad ? -1 : 0;
}

int orc_moe_ex(int E_global, int K, int N, int topk, double limit, int gate_up, int n_tiers,
               const orc_tier *tiers, const uint16_t *x, const int32_t *ids, const float *wts, long T,
               const int32_t *rows, long nrows, double *acc, uint16_t *out, int weight_on_input, double alpha,
               double beta) {
  return orc_moe_act(E_global, K, N, topk, limit, gate_up, n_tiers, tiers, x, ids, wts, T, rows, nrows, acc, out,
                     weight_on_input, alpha, beta, ORC_ACT_SWIGLU);
}

int orc_moe(int E_global, int K, int N, int topk, double limit, int gate_up, int n_tiers,
            const orc_tier *tiers, const uint16_t *x, const int32_t *ids, const float *wts, long T,
            const int32_t *rows, long nrows, double *acc, uint16_t *out) {
  return orc_moe_ex(E_global, K, N, topk, limit, gate_up, n_tiers, tiers, x, ids, wts, T, rows, nrows, acc, out,
                    0, 1.0, 0.0);
}

/* Threads an OpenMP build will use (1 without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
