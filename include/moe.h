/*
 * moe.h -- C ABI of the routed mixture-of-experts layer with block-scaled
 * 4-bit expert weights, for AMD MI355X (gfx950).
 *
 * What the layer computes (vLLM "hybrid_loader.py", _apply_ref; sglang
 * "moe_b12x_next.py", module docstring): for each token t and each of its
 * top_k slots j whose expert id e = topk_ids[t,j] lies in [0, E),
 *     z   = W13[e] . x_t                 (w13 stacked [up; gate])
 *     h   = silu(min(gate, L)) * clamp(up, -L, L)   (L = swiglu_limit)
 *     y   = W2[e] . h
 *     out[t] += topk_weights[t,j] * y
 * Ids outside [0, E), including the CUDA-graph padding id -1, contribute
 * nothing; a row with no valid slot is written as zeros (moe_b12x_next.py,
 * module docstring on direct ids).
 *
 * Weight formats (checkpoint layouts, all row-major and contiguous):
 *   MOE_W_MXFP4: w13 u8 [E, 2N, K/2] (two E2M1 codes per byte, element 2i in
 *                the low nibble), s13 E8M0 [E, 2N, K/32], w2 u8 [E, K, N/2],
 *                s2 E8M0 [E, K, N/32]   (moe_b12x_next.py, _convert_layer).
 *                Activations are quantised to MXFP8 (E4M3 + E8M0 per 32) in
 *                the layer, before each GEMM (W4A8).
 *   MOE_W_NVFP4: as MXFP4 but E4M3 scales per 16 (s13 [E, 2N, K/16], s2
 *                [E, K, N/16]) and one fp32 global per expert per tensor
 *                (g13 [E], g2 [E]) (hybrid_loader.py, create_weights, _deq_nv).
 *                bf16 activations (W4A16).
 *   MOE_W_NF3:   3-bit indices into {-1, -0.6047, -0.3563, -0.1275, 0.1275,
 *                0.3563, 0.6047, 1}, 8 codes per 3 little-endian bytes
 *                (w13 [E, 2N, K/8*3], w2 [E, K, N/8*3]), E4M3 scales per 32
 *                (hybrid_loader.py, _NF3_VALS, _unpack_nf3). bf16 activations.
 *
 * Conventions.  Every tensor pointer passed to moe_prepare_weights, moe_run
 * and the moe_debug_* calls is a DEVICE pointer.  Streams are hipStream_t
 * passed as void* (NULL = the null stream).  moe_run is stream-ordered: it
 * does not allocate, free or synchronise, so it may be captured in a HIP
 * graph once plan and weights are prepared.  Functions return a moe_status;
 * nothing throws.  moe_last_error() gives a message for the calling thread's
 * most recent failure.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,          /* null / misaligned pointer, bad size or argument */
  MOE_EUNSUPPORTED = -2,    /* shape or format combination the kernels do not cover */
  MOE_ENOTPREPARED = -3,    /* experts not prepared, or prepared for another plan */
  MOE_ESCRATCH = -4,        /* scratch buffer smaller than moe_scratch_bytes() */
  MOE_EHIP = -5             /* a HIP runtime call failed */
} moe_status;

typedef enum { MOE_W_MXFP4 = 1, MOE_W_NVFP4 = 2, MOE_W_NF3 = 3 } moe_wfmt;
typedef enum { MOE_A_MXFP8 = 1, MOE_A_BF16 = 2 } moe_afmt;
typedef enum { MOE_W13_UP_GATE = 0, MOE_W13_GATE_UP = 1 } moe_w13_layout;
/* Activation forms of the GEMM1 epilogue (vLLM "fused_moe/b12x" page,
 * _supports_activation and _swiglu_params): the SwiGLU (with the plan's limit
 * and the optional OAI alpha / beta), SiTU (beta 4, linear beta 25, no limit)
 * and ReLU^2 without the gate multiply (no limit; w13 holds N rows, not 2N). */
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_SITU = 1, MOE_ACT_RELU2_NO_MUL = 2 } moe_activation;
/* Launch sequences of one chunk (the capacity ladder's choice unless a rung is
 * pinned): DECODE = two kernels, no route planner (T <= 16, T * top_k <= 64);
 * GENERAL = planner + 16-route-tile GEMMs + combine (any batch); PREFILL =
 * planner + 64-route-tile GEMMs + combine (N % 64 == 0), the up/gate GEMM on
 * 128-route tiles; PREFILL_NARROW = PREFILL with 64-route up/gate tiles (a tile
 * height for the race). */
typedef enum {
  MOE_SEQ_AUTO = 0,
  MOE_SEQ_DECODE = 1,
  MOE_SEQ_GENERAL = 2,
  MOE_SEQ_PREFILL = 3,
  MOE_SEQ_PREFILL_NARROW = 4
} moe_sequence;
/* How runs with deterministic = 0 combine the k slots of a token (the
 * GENERAL and PREFILL sequences; DECODE folds them in its down GEMM either
 * way): ATOMIC = fp32 atomic adds into an accumulator, then one bf16 cast;
 * ROUTE_BUFFER = the deterministic combine (per-slot bf16 route buffer and a
 * slot-order top-k sum).  AUTO = the capacity ladder's choice: ROUTE_BUFFER on
 * the PREFILL sequence, ATOMIC on GENERAL. */
typedef enum { MOE_COMBINE_AUTO = 0, MOE_COMBINE_ATOMIC = 1, MOE_COMBINE_ROUTE_BUFFER = 2 } moe_combine;

typedef struct moe_plan_s *moe_plan_t;       /* one layer geometry (host memory only) */
typedef struct moe_experts_s *moe_experts_t; /* one layer's (or tier's) prepared weights */

/* One group of experts taking part in a moe_run.  expert_map (device, int32
 * [E], may be NULL = identity) maps a global expert id to this tier's local
 * id, or -1 when the id belongs elsewhere (hybrid_loader.py, the per-tier
 * expert maps of the hybrid runtime: each tier sees only its own experts, under
 * local ids, and skips the rest).  A global id is served by the first tier
 * whose map accepts it. */
typedef struct {
  moe_experts_t experts;
  const int32_t *expert_map;
} moe_tier;

/*
 * moe_plan -- plan one layer geometry (sglang moe_b12x_next.py: plans are per
 * geometry (experts, K, N, top-k, swiglu limit) and shared by every layer of
 * that geometry).
 *   E            global expert id range [0, E) of topk_ids (1 .. 1024; all tiers together
 *                hold at most 1024 experts)
 *   K            hidden size (GEMM1 reduction, output width); multiple of 256
 *   N            intermediate size of this rank's slice; multiple of 32
 *   top_k        slots per token (1 .. 16)
 *   swiglu_limit clamp L of the SwiGLU; NaN or <= 0 = no clamp
 *   act_format   MOE_A_MXFP8 (for MXFP4 experts) or MOE_A_BF16 (NVFP4 / NF3)
 *   w13_layout   MOE_W13_UP_GATE (default) or MOE_W13_GATE_UP
 *   max_tokens   largest T one launch handles; larger batches run in chunks
 *                of the largest capacity (moe_b12x_next.py, _Geometry.forward)
 * Host only.  *out receives a plan owned by the caller (moe_plan_destroy).
 */
int moe_plan(int E, int K, int N, int top_k, float swiglu_limit, int act_format, int w13_layout,
             int max_tokens, moe_plan_t *out);
void moe_plan_destroy(moe_plan_t plan);

/* Bytes of device scratch one moe_run of `tokens` tokens needs under `plan`
 * (tokens above the top capacity are sized for one chunk).  The arena is
 * carved into 256-byte aligned pieces.  Host only; 0 on a bad plan. */
size_t moe_scratch_bytes(moe_plan_t plan, int tokens, int deterministic);

/*
 * moe_prepare_weights -- repack one layer's checkpoint tensors IN PLACE into
 * the tile layout the kernels stream (moe_b12x_next.py, _convert_layer: the
 * checkpoint storage is reused, a second copy would double expert memory).
 *   weight_format  MOE_W_MXFP4 / MOE_W_NVFP4 / MOE_W_NF3 (must fit the plan's
 *                  act_format)
 *   num_experts    experts held in these tensors (this tier's local ids)
 *   w13,s13,w2,s2  device buffers in the checkpoint layout above; they are
 *                  rewritten in place and afterwards hold the tile layout
 *   g13, g2        device fp32 [num_experts] globals (NVFP4; NULL = 1.0)
 * The returned handle borrows the buffers (the caller keeps ownership and must
 * keep them alive).  For MXFP4 experts the handle also owns second copies of
 * s13 and s2 (device buffers of their sizes, 1/16 of w13 and w2), ordered for
 * the prefill GEMMs, which read a lane's scales of four k-tiles in one load;
 * moe_unpack_weights and moe_experts_destroy free them.  moe_experts_destroy
 * releases the handle and those copies, never the caller's buffers.  Prepare
 * allocates a temporary device buffer and synchronises `stream`; it is not
 * for graph capture.
 */
int moe_prepare_weights(moe_plan_t plan, int weight_format, int num_experts, void *w13, void *s13,
                        const float *g13, void *w2, void *s2, const float *g2, void *stream,
                        moe_experts_t *out);
/* Undo moe_prepare_weights: rewrite the buffers back to the checkpoint layout
 * in place.  The handle becomes unprepared (moe_run refuses it). */
int moe_unpack_weights(moe_experts_t experts, void *stream);
void moe_experts_destroy(moe_experts_t experts);

/*
 * moe_run -- the layer.
 *   tiers, n_tiers  1 or 2 groups of prepared experts (2 = hybrid: NVFP4 and
 *                   NF3 tiers, both through the 16-bit-activation path)
 *   x               bf16 [T, K] row-major.  16-bit-activation layers multiply
 *                   in bf16, except the decode-size launches and the NVFP4
 *                   route-buffer down GEMM, which multiply in fp16 on rows
 *                   scaled by a power of two each (exact for every element at
 *                   or above 2^-28 of its row's largest magnitude)
 *   topk_ids        int32 [T, top_k]; ids outside [0, E) are skipped
 *   topk_weights    fp32 [T, top_k]
 *   out             bf16 [T, K], fully overwritten
 *   T               tokens (0 = no-op)
 *   deterministic   0: per-route results are added into an fp32 accumulator
 *                   with atomics (run-to-run order may vary);
 *                   1: per-slot route buffer + fixed-order top-k sum,
 *                   bit-stable run to run (moe_b12x_next.py, DETERMINISTIC).
 *                   With 0, a rung whose combine is ROUTE_BUFFER (the
 *                   ladder's choice on the PREFILL sequences, and on W4A8
 *                   GENERAL rungs from 256 tokens when pinned there; see
 *                   moe_plan_set_combine) combines as 1 does.
 *                   Decode-size batches (<= 16 tokens, <= 64 routes) run two
 *                   kernels that fold each token's slots in slot order in
 *                   either mode (bit-stable); with 16-bit activations the down
 *                   GEMM adds two halves of each output tile into a zeroed
 *                   fp32 accumulator with atomics, which is order-independent
 *                   for two terms, so that stays bit-stable too.
 *   scratch         device buffer of >= moe_scratch_bytes(plan, T, deterministic)
 * Stream-ordered, no allocation, no synchronisation.
 */
int moe_run(moe_plan_t plan, const moe_tier *tiers, int n_tiers, const void *x, const int32_t *topk_ids,
            const float *topk_weights, void *out, int T, int deterministic, void *scratch,
            size_t scratch_bytes, void *stream);

/*
 * moe_run_noalloc -- moe_run with the scratch arena taken from a static device
 * array of the library instead of a caller buffer.  For callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.
 *   Arguments as moe_run, without scratch / scratch_bytes.
 *   The array holds 64 MiB per GPU (held from the library's load until the
 *   process ends); a batch whose moe_scratch_bytes(plan, T, deterministic)
 *   exceeds it is refused with MOE_ESCRATCH (e.g. 4096 tokens at K = 7168;
 *   the 8-token decode batch needs about 0.3 MiB).
 *   The first call on each device looks up that device's copy of the array
 *   (make it outside graph capture, e.g. with T = 0); later calls allocate,
 *   free and synchronise nothing.  Nothing in the array needs to start at zero.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 *   (two streams or two host threads) race.
 */
int moe_run_noalloc(moe_plan_t plan, const moe_tier *tiers, int n_tiers, const void *x, const int32_t *topk_ids,
                    const float *topk_weights, void *out, int T, int deterministic, void *stream);

/* Message of the calling thread's most recent failure ("" if none). */
const char *moe_last_error(void);

/* Capacity the plan runs a batch of T tokens at (0 on a bad plan), and the
 * route rows of the tiles its launch sequence uses: 0 for the decode sequence
 * (no route planner, no tiles), 64 for prefill, 16 for the general kernels.
 * Host only; used by tests and benches. */
int moe_plan_capacity(moe_plan_t plan, int T, int *tile_rows);

/* Per-capacity tuning (sglang "moe_b12x_next.py", module docstring and
 * _Geometry: each capacity of the ladder gets its own execution plan, raced
 * once per geometry and persisted, instead of a fixed heuristic).
 *
 * moe_plan_set_sequence pins the rung a batch of `tokens` runs at to one
 * launch sequence (MOE_SEQ_AUTO: back to the ladder's choice).  A sequence
 * the rung cannot take (DECODE above 16 tokens or 64 routes, PREFILL with
 * N % 64 != 0) is MOE_EUNSUPPORTED.  moe_plan_sequence returns the sequence a
 * batch of `tokens` runs with now (0 on a bad plan).  Host only.
 *
 * moe_plan_set_combine pins the combine of deterministic = 0 runs at the rung
 * of `tokens` (moe_combine; AUTO: back to the ladder's choice);
 * moe_plan_combine returns the one such a batch uses now (ATOMIC or
 * ROUTE_BUFFER; 0 on a bad plan).  The scratch a run needs follows the pin
 * (moe_scratch_bytes), so pin before sizing the arena.  Host only.
 *
 * moe_plan_autotune races, at the rung of each listed batch size, every launch
 * sequence the rung can take (so the route-tile height: 16 GENERAL, 64 / 128
 * PREFILL, 64 PREFILL_NARROW) and, for deterministic = 0, both combines of the
 * planner-based sequences, on a seeded synthetic batch of the rung's full
 * size with the caller's prepared experts (`reps` timed runs after two warm-up
 * runs, median), and pins the rung's sequence and combine to the fastest.
 * us_out (NULL or [n][7]) receives the median microseconds of DECODE,
 * GENERAL-atomic, GENERAL-route buffer, PREFILL-atomic, PREFILL-route buffer,
 * PREFILL_NARROW-atomic and PREFILL_NARROW-route buffer, NaN where not raced
 * (deterministic races fill the route-buffer entries).
 * moe_plan_autotune_batch races the rung of T on the caller's own batch
 * instead (device x [T, K] bf16, topk_ids, topk_weights; T <= max_tokens;
 * us_out NULL or [7]): the workload's routing, e.g. skewed expert loads,
 * decides.  Both allocate and synchronise (a tuning session,
 * not part of the layer): call them before graph capture.
 *
 * moe_plan_save_tuning writes the plan's pinned rungs to a text file, one line
 * per rung keyed by the geometry (E, K, N, top_k, act_format, max_tokens),
 * keeping other geometries' lines already in the file.  moe_plan_load_tuning
 * pins the rungs of the lines matching this plan's geometry and returns how
 * many it applied (entries a rung cannot take are skipped), or MOE_EINVAL when
 * the file cannot be read. */
int moe_plan_set_sequence(moe_plan_t plan, int tokens, int seq);
int moe_plan_sequence(moe_plan_t plan, int tokens);
int moe_plan_set_combine(moe_plan_t plan, int tokens, int combine);
int moe_plan_combine(moe_plan_t plan, int tokens);
int moe_plan_autotune(moe_plan_t plan, const moe_tier *tiers, int n_tiers, const int *tokens, int n, int deterministic,
                      int reps, void *stream, float *us_out);
int moe_plan_autotune_batch(moe_plan_t plan, const moe_tier *tiers, int n_tiers, const void *x,
                            const int32_t *topk_ids, const float *topk_weights, int T, int deterministic, int reps,
                            void *stream, float *us_out);
int moe_plan_save_tuning(moe_plan_t plan, const char *path);
int moe_plan_load_tuning(moe_plan_t plan, const char *path);

/* Apply each slot's router weight to that slot's copy of the token before
 * GEMM1 instead of to its GEMM2 result (vLLM "fused_moe/b12x" page,
 * process_weights_after_loading: apply_router_weight_on_input, W4A16 only):
 *     out[t] += W2[e] . act(W13[e] . (w[t,j] x_t)).
 * GEMM1 is linear, so the kernels scale its fp32 accumulators by w.  Only for
 * plans with MOE_A_BF16 activations: MOE_EUNSUPPORTED otherwise.  enable = 0
 * restores the default (weight on the GEMM2 result).  Host only. */
int moe_plan_set_router_weight_on_input(moe_plan_t plan, int enable);

/* The SwiGLU-OAI activation form (vLLM "fused_moe/b12x" page, _swiglu_params:
 * a limit plus alpha and beta for swigluoai): after the limit clamps,
 *     h = gate * sigmoid(alpha * gate) * (up + beta).
 * alpha = 1, beta = 0 (the default) is the plain clamped SwiGLU.  Other values
 * only for MOE_A_BF16 plans (the page refuses this activation with W4A8):
 * MOE_EUNSUPPORTED otherwise; non-finite values: MOE_EINVAL.  Host only. */
int moe_plan_set_swiglu_oai(moe_plan_t plan, float alpha, float beta);

/*
 * moe_ep_remap -- one expert-parallel rank's view of the router output
 * (sglang "moe_b12x_next.py", ep_remap / ep_remap_reference: the step before
 * the layer when the experts are sharded over ranks).  For each slot,
 * lid = topk_ids[t,j] - offset (computed in 64 bits, so no id wraps):
 *   lid in [0, num_local)  -> out_ids = lid, out_weights = topk_weights[t,j];
 *   otherwise (an expert of another rank, padding)
 *                          -> out_weights = 0 and out_ids = the lowest valid
 *                             lid of row t, else the lowest of the batch,
 *                             else 0,
 * so every slot names an expert whose weights the batch already streams and a
 * zero weight makes the slot add nothing.
 *   topk_ids      device int32 [T, top_k], contiguous (global ids)
 *   topk_weights  device fp32 [T, top_k], contiguous
 *   out_ids       device int32 [T, top_k] (local ids, for a plan with E = num_local)
 *   out_weights   device fp32 [T, top_k]; may not alias the inputs
 *   top_k 1 .. 64, num_local >= 1; T = 0 is a no-op.
 * One kernel on `stream`, no allocation, no synchronisation (graph-capturable).
 * Returns MOE_EINVAL for bad sizes or null / misaligned pointers, MOE_EHIP if
 * the launch fails.  The caller owns every buffer.
 */
int moe_ep_remap(const int32_t *topk_ids, const float *topk_weights, int T, int top_k, long long offset,
                 int num_local, int32_t *out_ids, float *out_weights, void *stream);

/* The activation form of the plan (moe_activation); set it before preparing
 * experts for the plan (the w13 row count follows it).
 *   MOE_ACT_SITU: both branches softly capped by tanh,
 *     h = silu(4 tanh(gate / 4)) * 25 tanh(up / 25)
 *   (vLLM "fused_moe/b12x" page: SiTU is taken only with beta 4 and linear beta
 *   25, without a limit, and is one of the two activations W4A8 runs; the page
 *   does not print the formula, this is the reading taken).  Any activation
 *   format.
 *   MOE_ACT_RELU2_NO_MUL: h[n] = relu(z[n])^2 for z = W13 . x with a w13 of N
 *   rows ([E, N, K] codes and scales in the checkpoint layout; the same page
 *   lists RELU2_NO_MUL and runs it without a gate multiply).  bf16 activations
 *   only (the page refuses it with W4A8), N % 64 == 0, the default w13 layout;
 *   the PREFILL sequence needs N % 128 == 0.
 * MOE_EUNSUPPORTED on a plan with a swiglu limit or OAI alpha / beta for the
 * other forms, for the cases above, or for an unknown form.  Host only. */
int moe_plan_set_activation(moe_plan_t plan, int act);

/* ---- instrumentation ------------------------------------------------- */

/* Stage timing for benchmarks: after this call, each moe_run under `plan`
 * records a HIP event on its stream before the route planner and after each
 * stage (route, gemm1, gemm2, combine), for up to max_runs runs (later runs
 * record nothing).  Events are created here, not in moe_run.  max_runs = 0
 * turns timing off and frees the events.  Returns a moe_status. */
int moe_plan_enable_stage_timing(moe_plan_t plan, int max_runs);
/* Waits for the recorded runs and writes the summed milliseconds of each
 * stage (ms[0] route, ms[1] gemm1, ms[2] gemm2, ms[3] combine; n >= 4) over
 * the recorded runs; *runs receives their count.  Resets the run counter. */
int moe_plan_stage_times(moe_plan_t plan, float *ms, int n, int *runs);

/* ---- stage entry points, for the bit-exact stage tests ---------------- */

/*
 * moe_debug_route -- the route planner alone (expert histogram, prefix-sum
 * offsets, stable token permutation).  Experts of all tiers form one index
 * space u = (experts of earlier tiers) + local id.
 *   cnt  int32 [U], off int32 [U+1], perm int32 [T*top_k] (first off[U]
 *   entries are the valid route indices r = t*top_k + j sorted by (u, r)),
 *   inv  int32 [T*top_k] (position of r in perm, or -1 for a skipped slot).
 * Uses `scratch` like moe_run (capacity of T tokens, T <= max_tokens).
 */
int moe_debug_route(moe_plan_t plan, const moe_tier *tiers, int n_tiers, const int32_t *topk_ids, int T,
                    void *scratch, size_t scratch_bytes, int32_t *cnt, int32_t *off, int32_t *perm,
                    int32_t *inv, void *stream);

/* MXFP8 quantiser alone: rows x cols (cols % 32 == 0) of bf16 or fp32 ->
 * E4M3 codes u8 [rows, cols] + E8M0 scales u8 [rows, cols/32].  The bf16 one
 * runs the block quantiser every bf16-activation path of moe_run uses (x in
 * the route launch and in the decode up/gate kernel); the fp32 one the
 * requantiser's arithmetic on the intermediate. */
int moe_debug_quant_mxfp8_bf16(const void *x, int rows, int cols, uint8_t *q, uint8_t *scales, void *stream);
int moe_debug_quant_mxfp8_f32(const float *h, int rows, int cols, uint8_t *q, uint8_t *scales, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
