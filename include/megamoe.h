/*
 * megamoe.h -- C ABI of the MI355X (gfx950) routed-expert path.
 *
 * The library computes, on one GPU with every expert local, the fused
 * Mega-MoE expert path defined on the Ascend CANN "mega_moe" operator page
 * (Formula; Computation Process): EP Dispatch -> Linear1 -> SwiGLU ->
 * Linear2 -> Token Combine,
 *
 *     y_i = sum_k G[i,k] * ( SwiGLU( x_i . W1[E[i,k]] ) . W2[E[i,k]] ),
 *     SwiGLU(h) = SiLU(h[:, :I]) * h[:, I:],  SiLU(z) = z / (1 + e^-z),
 *
 * with the dispatch metadata of the DeepEP "Metadata System" notes (Count ->
 * Prefix Sum -> Scatter into a BLOCK_M-padded pool that keeps the
 * (token, top-k slot) identity of every row, sections 1, 3 and 4).
 *
 * Symbols: T = num_tokens, H = hidden, I = intermediate_hidden,
 * E = num_experts, K = num_topk, S = num_shared_experts (0 or 1),
 * P = plan.pool_rows.
 *
 * Shared expert (DeepGEMM MegaMoE page, section 6 "Optional Shared
 * Experts"): with S = 1 every active token also goes through one always-local
 * SwiGLU FFN, expert index E in the weight arrays, whose output is added
 * after the K routed contributions (combine slot K) with weight 1:
 *     y_i = sum_k G[i,k] * FFN_{E[i,k]}(x_i) + FFN_E(x_i).
 * Internally a token then has K + S slots; route r = i*(K+S) + k names slot
 * k of token i, k = K being the shared expert's.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked "device" point to device memory on the current HIP
 *   device; the caller allocates and owns every buffer, including the
 *   workspace.  The library never allocates, frees or synchronises device
 *   memory and never reads device data on the host.
 * - Every compute entry point is asynchronous on `stream` (a hipStream_t
 *   passed as void*; NULL = the null stream).  A return of MM_OK means the
 *   kernels were enqueued; their errors surface on the stream.
 * - All tensors are dense, contiguous and row-major.
 * - Argument checks happen on the host before any HIP call: a NULL
 *   pointer, a misaligned pointer (every pointer must be 16-byte aligned)
 *   or a plan whose checksum does not match returns MM_ERR_INVALID_ARG and
 *   enqueues nothing.
 * - Route ids (topk_ids) must be in [0, E) and distinct within a token, as
 *   the Parameters table of the operator page requires; an id < 0 marks a
 *   masked route (DeepEP notes, section 5.2): it is skipped, counted for no
 *   expert and contributes 0.  An id >= E is skipped the same way and sets
 *   MM_DEVERR_BAD_EXPERT in the workspace error word (mm_read_device_error);
 *   duplicated ids are not detected and give undefined results.
 * - x_active_mask (operator page, Parameters: whether a token takes part in
 *   the layer's communication): device int8 [T] or NULL (every token
 *   active).  A token whose entry is 0 dispatches no route (routed or
 *   shared), is counted for no expert, and its row of y is 0.
 * - Workspace counters are reset by the library at the start of every
 *   call; the caller never clears them.
 * - Calls that share a workspace or intermediate buffers must be ordered
 *   on one stream; overlapping calls on the same buffers race.
 * - Results are deterministic: the top-k sum runs in slot order k = 0..K+S-1
 *   in float32 (operator page, "Deterministic Computation"), and a route's
 *   result depends on its own pool row alone, not on where in its expert's
 *   range the dispatch placed it.  (Setting MM_MAX_SPLIT above 1 for the
 *   bf16 or fp8 use case, a tuning knob, gives that up: a K-split tile
 *   rounds its float32 sums differently.)
 */
#ifndef MEGAMOE_H
#define MEGAMOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mm_status {
  MM_OK = 0,
  MM_ERR_INVALID_ARG = 1, /* NULL / misaligned pointer, bad dimension, bad plan */
  MM_ERR_UNSUPPORTED = 2, /* use case or output dtype not supported */
  MM_ERR_WORKSPACE = 3,   /* workspace smaller than the plan requires */
  MM_ERR_HIP = 4          /* a HIP launch or event call failed */
} mm_status;

/* Use cases of the operator page's use-case table (Computation Process).
 * A16W16: bf16 activations and weights.
 * A8W8_FP8: OCP float8 e4m3fn activations and weights with float32 scales
 *   (per-token for X, per output channel for W, per row for the SwiGLU
 *   output), by the A8W8 formulas with Qmax = 448.
 * A8W8_INT8: symmetric int8 in [-127, 127] with the same scales, Qmax = 127,
 *   exact int32 accumulation.
 * MXFP8: the A8W8-FP use case (operator page, A8W8-FP Quantization Use
 *   Case): e4m3 activations and weights, each group of 32 values along the
 *   contraction dimension with one FLOAT8_E8M0 scale (MX per-group
 *   quantisation: shared exponent floor(log2 max|v|) - 8, elements rounded
 *   to nearest even and saturated); X is quantised per token in Dispatch and
 *   the SwiGLU output per row in the Linear1 epilogue, both by the library.
 * MXFP4: the FP8 x FP4 path of the DeepGEMM MegaMoE page (section 1): the
 *   same MX-FP8 activations with MX-FP4 (e2m1) weights.
 * The MX use cases take weights as element codes with E8M0 scales
 * [E+S][N][K_in/32] (per output column, per group of 32 along the input
 * dimension: S1 [E+S][2I][H/32], S2 [E+S][H][I/32]) and hold at most 512
 * experts (E + S). */
typedef enum mm_usecase {
  MM_A16W16 = 0, MM_A8W8_FP8 = 1, MM_A8W8_INT8 = 2, MM_MXFP8 = 3, MM_MXFP4 = 4
} mm_usecase;

/* dtype of y: bf16 (the operator's output dtype) or float32 (the same
 * float32 value before its final round-to-nearest-even to bf16). */
typedef enum mm_out_dtype { MM_OUT_BF16 = 0, MM_OUT_F32 = 1 } mm_out_dtype;

typedef struct mm_problem {
  int64_t num_tokens;          /* T >= 1 */
  int64_t hidden;              /* H, multiple of 256 */
  int64_t intermediate_hidden; /* I, multiple of 128 */
  int64_t num_experts;         /* E in [1, 1024] */
  int64_t num_topk;            /* K in [1, min(E, 64)] */
  int32_t usecase;             /* mm_usecase */
  int32_t y_dtype;             /* mm_out_dtype */
  /* The operator's activation_clamp (mega_moe, Parameters): with
   * clamp_activation = 1, every element of Linear1's output H (gate and up
   * halves, after A8W8 dequantisation) is clamped to [-activation_clamp,
   * activation_clamp] before SwiGLU; activation_clamp must then be >= 0 (not
   * NaN).  clamp_activation = 0 (a zeroed struct) is the operator's None: no
   * clamp, activation_clamp ignored.  Other values: MM_ERR_INVALID_ARG. */
  int32_t clamp_activation;
  float activation_clamp;
  /* S: 0, or 1 for one shared expert (index E of the weight arrays, which
   * then hold E + 1 experts); K + S <= 64 and E + S <= 1024. */
  int32_t num_shared_experts;
  int32_t reserved0;          /* must be 0 */
} mm_problem;

/* A plan is plain host data filled by mm_plan_create.  Callers read the
 * sizes from it and pass it back unchanged to every entry point. */
typedef struct mm_plan {
  mm_problem prob;
  int32_t block_m;            /* BLOCK_M: pool rows per expert are padded to a multiple */
  int32_t tile_l1;            /* internal tile configuration of Linear1 */
  int32_t tile_l2;            /* internal tile configuration of Linear2 */
  int32_t gate_up_group;      /* gate/up interleave group of the prepared W1 */
  int64_t pool_rows;          /* P = capacity of the padded pool, a multiple of block_m */
  int64_t x_pool_bytes;       /* P * H * elem(usecase) */
  int64_t a_pool_bytes;       /* P * I * elem(usecase) */
  int64_t x_pool_scale_bytes; /* A8W8: P * 4 (float32); MX: P * H/32 (E8M0); A16W16: 0 */
  int64_t a_pool_scale_bytes; /* A8W8: P * 4 (float32); MX: P * I/32 (E8M0); A16W16: 0 */
  int64_t w1_bytes;           /* (E+S) * H * 2I * elem(usecase) (formula and prepared; e2m1: half a byte) */
  int64_t w2_bytes;           /* (E+S) * I * H * elem(usecase) */
  int64_t workspace_bytes;    /* scratch of the three-call path */
  int64_t fused_workspace_bytes; /* scratch of mega_moe (holds the pool too) */
  uint64_t checksum;          /* guards against a modified plan (covers every other byte) */
  int64_t reserved[8];        /* internal choices of the plan (workspace layout); do not modify */
} mm_plan;

/* Elements: bf16 = 2 bytes, e4m3fn / int8 = 1 byte, e2m1 = half a byte
 * (two per byte, the even index in the low nibble). */

/*
 * mm_plan_create -- validate a problem and choose BLOCK_M and tiles.
 * Host only, no HIP call.  BLOCK_M follows the expected rows per expert,
 * T*K/E (DeepGEMM MegaMoE page, section 3.3 shape heuristic): small loads
 * take a small BLOCK_M.  P = R + (E+S)*(BLOCK_M-1) rounded up to BLOCK_M,
 * with R = T*(K+S) routes: enough for any routing.
 * Errors: MM_ERR_INVALID_ARG for NULL pointers or dimensions outside the
 * ranges stated in mm_problem; MM_ERR_UNSUPPORTED for an unknown use case
 * or output dtype.
 */
mm_status mm_plan_create(const mm_problem* problem, mm_plan* plan);

/*
 * mm_prepare_weights -- one-time relayout of the expert weights into the
 * layout the GEMM kernels stream (DeepGEMM MegaMoE page, section 3.2: done
 * once by the caller before repeated launches; not part of the timed path).
 *   w1     device [E+S][H][2I]  formula layout of the operator page (Formula);
 *                               e2m1: [E+S][H][I] bytes, packed along 2I
 *   w2     device [E+S][I][H]   formula layout; e2m1: [E+S][I][H/2] bytes
 *   w1_out device [E+S][2I][H] K-contiguous rows (e2m1: packed along H); row n of expert e holds the
 *                             W1 column c(n) with gate and up columns
 *                             interleaved in groups of g = gate_up_group:
 *                             c(n) = (n/2g)*g + n%g            if n%2g <  g
 *                                    I + (n/2g)*g + n%g - g    otherwise
 *   w2_out device [E+S][H][I] K-contiguous (transposed; e2m1: packed along I)
 * Scales stay in formula layout ([E+S][2I] and [E+S][H], or the MX
 * [E+S][N][K_in/32] bytes).  Buffers must not
 * overlap.
 */
mm_status mm_prepare_weights(const mm_plan* plan, const void* w1, const void* w2,
                             void* w1_out, void* w2_out, void* stream);

/*
 * mm_dispatch_layout -- EP Dispatch: steps route read, count, claim +
 * prefix, scatter + gather, and (A8W8) per-token activation quantisation.
 * Operator page, Computation Process, EP Dispatch (and for A8W8 the
 * quantisation "before Dispatch": s_i = max|X[i,:]|/Qmax, q_i = round(X[i,:]/s_i));
 * DeepEP notes sections 3.2-3.5 (count in LDS, one claim atomic, scatter,
 * pool block offsets).
 *   topk_ids       device int32 [T][K]
 *   x_active_mask  device int8 [T] or NULL (see the conventions above)
 *   x              device bf16  [T][H]
 *   expert_counts  device int32 [E+S]  out: N_e (the operator's expert_token_nums;
 *                                      entry E: the shared expert's count)
 *   expert_offsets device int32 [E+S+1] out: padded exclusive prefix,
 *                                      off[e+1] = off[e] + BLOCK_M*ceil(N_e/BLOCK_M)
 *   pool_src       device int32 [P]    out: route i*(K+S)+k of pool row p, -1 on padding
 *   route_to_pool  device int32 [T*(K+S)] out: pool row of each route, -1 if skipped
 *   x_pool         device [P][H]       out: row p = x_i (bf16) or q_i (A8W8);
 *                                      padding rows are unspecified
 *   x_pool_scale   device, out: s_i of row p, f32 [P] (A8W8), or the E8M0
 *                                      scales of row p's groups of 32, [P][H/32] (MX);
 *                                      plan.x_pool_scale_bytes; may be NULL for A16W16
 *   workspace      device, plan.workspace_bytes
 * The order of the rows of one expert inside its pool range is unspecified
 * (the operator page stacks them "in any fixed order").
 */
mm_status mm_dispatch_layout(const mm_plan* plan, const int32_t* topk_ids, const int8_t* x_active_mask,
                             const void* x,
                             int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* pool_src, int32_t* route_to_pool,
                             void* x_pool, void* x_pool_scale,
                             void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * mm_grouped_l1_swiglu -- Linear1 per expert + SwiGLU (+ A8W8 row requant).
 * Operator page, Expert Compute steps 1-2: H_e = X_e . W1[e] (A8W8:
 * C = Q_e . W1q[e] in int32 / fp32, H_e = (C * s^W1_e) * s^X_e), then
 * A_e = SiLU(H_e[:, :I]) * H_e[:, I:]; for A8W8 step 3's requantisation
 * s^A_i = max|A_e[i,:]|/Qmax, A^q = round(A_e / s^A_i).
 *   expert_offsets, expert_counts  as written by mm_dispatch_layout
 *   x_pool, x_pool_scale           as written by mm_dispatch_layout
 *   w1        device, prepared by mm_prepare_weights
 *   w1_scale  device f32 [E+S][2I] formula order (A8W8), E8M0 [E+S][2I][H/32]
 *             (MX), NULL for A16W16
 *   a_pool    device [P][I] out: bf16 A (A16W16) or its int8 / e4m3 codes
 *   a_pool_scale device out: s^A f32 [P] (A8W8), or A's E8M0 group scales
 *             [P][I/32] (MX: A = Q_MX(SwiGLU(H)) per row, made in the Linear1
 *             epilogue); may be NULL for A16W16
 */
mm_status mm_grouped_l1_swiglu(const mm_plan* plan, const int32_t* expert_offsets,
                               const int32_t* expert_counts, const void* x_pool,
                               const void* x_pool_scale, const void* w1, const void* w1_scale,
                               void* a_pool, void* a_pool_scale,
                               void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * mm_grouped_l2_combine -- Linear2 per expert, gate weighting, Token Combine.
 * Operator page, Expert Compute step 3 (Y_e = A_e . W2[e]; A8W8:
 * Y_e = (D * s^W2_e) * s^A_e) and Token Combine
 * (y_i = sum_k G[i,k] * Y_{e_ik}[row(i,k)], stacked in token order; a
 * shared-expert slot has weight 1).  Each weighted contribution is stored in
 * float32 for A16W16 and in bf16 for the A8W8 use cases (whose y is bf16,
 * as the DeepGEMM page's combine slots are, section 4 step 7); the K + S
 * contributions of a token are summed in float32 in slot order.
 *   pool_src, route_to_pool        as written by mm_dispatch_layout
 *   a_pool, a_pool_scale           as written by mm_grouped_l1_swiglu
 *   w2        device, prepared by mm_prepare_weights
 *   w2_scale  device f32 [E+S][H] (A8W8), E8M0 [E+S][H][I/32] (MX), NULL for A16W16
 *   topk_weights device f32 [T][K]
 *   y         device [T][H] out, bf16 or f32 per plan.prob.y_dtype
 */
mm_status mm_grouped_l2_combine(const mm_plan* plan, const int32_t* expert_offsets,
                                const int32_t* expert_counts, const int32_t* pool_src,
                                const int32_t* route_to_pool, const void* a_pool,
                                const void* a_pool_scale, const void* w2, const void* w2_scale,
                                const float* topk_weights, void* y,
                                void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * mega_moe -- the whole path in one call: Dispatch, Linear1, SwiGLU,
 * Linear2, Combine (operator page, Function and Prototype: returns y and
 * expert_token_nums).  Every intermediate lives in the workspace.
 * It runs as one persistent kernel (one workgroup per compute unit, the
 * whole grid resident at once) after a small pre-pass that clears the
 * counters and stores the kernel's arguments in the workspace: the
 * phases count, scatter, gather, Linear1, (A8W8) requantisation, Linear2
 * and combine follow each other inside the kernel, separated by grid-wide
 * barriers.  The results are bitwise those of the three-call path.
 * Device-side conditions (an expert id >= E, a barrier that timed out) are
 * recorded in the workspace error word, see mm_read_device_error.  A device
 * that cannot hold one workgroup per compute unit makes the call fail with
 * MM_ERR_HIP before anything runs.
 * Co-residency: the grid barriers need every workgroup of the grid running
 * at once.  Work on other streams that holds compute units only delays the
 * late workgroups, but if it holds them longer than the barriers' bounded
 * wait (about a second), the barrier gives up: the call has already
 * returned MM_OK, y is then unspecified, and only the error word
 * (MM_DEVERR_BARRIER_TIMEOUT) reports it.  Callers that share the GPU with
 * long-running concurrent kernels must read the error word, or make the plan
 * with the environment variable MM_COOPERATIVE=1 set: the fused kernel is
 * then launched cooperatively, so the runtime starts it only once the whole
 * grid can be resident (some microseconds more per call).  A plan made with
 * MM_DEP=1 set replaces the barriers between Linear1, the requantisation and
 * Linear2 by per-M-block completion counters (same results, bit for bit;
 * off by default: not faster on the measured layers).  Its waits are bounded
 * the same way and report the same error bit.  The GEMM tiles of the fused
 * kernel are claimed from per-XCD counters (faster workgroups and XCDs take
 * more tiles; same results); MM_STATIC_TILES=1 at plan time restores a fixed
 * round robin.
 *   x              device bf16 [T][H]
 *   topk_ids       device int32 [T][K]
 *   topk_weights   device f32 [T][K]
 *   x_active_mask  device int8 [T] or NULL
 *   w1, w2         device, prepared by mm_prepare_weights
 *   w1_scale, w2_scale  device, as for the grouped entry points; NULL for A16W16
 *   y              device [T][H] out (bf16 or f32 per plan)
 *   expert_token_nums device int32 [E] out: N_e of the routed experts
 *   workspace      device, plan.fused_workspace_bytes
 */
mm_status mega_moe(const mm_plan* plan, const void* x, const int32_t* topk_ids,
                   const float* topk_weights, const int8_t* x_active_mask,
                   const void* w1, const void* w1_scale,
                   const void* w2, const void* w2_scale, void* y, int32_t* expert_token_nums,
                   void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * mega_moe_noalloc -- mega_moe for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, semantics and results as mega_moe
 * (bit for bit), without the workspace argument: the workspace is a static
 * device array of the library, 96 MiB, one per GPU the library runs on,
 * held until the process ends.  Allocates nothing and frees nothing.
 * Plans whose fused_workspace_bytes exceed 96 MiB get MM_ERR_WORKSPACE
 * (the DeepSeek-V3-shape layer, hidden 7168, intermediate 2048, 32 experts,
 * top-8, fits up to 128 tokens in every use case).  Every call on a GPU
 * shares that GPU's array and leaves its contents behind (the call clears
 * its counters itself): calls that overlap on one GPU, on any streams, race.
 * mm_read_device_error and mm_debug_fused_layout read this array when
 * passed a NULL workspace.
 */
mm_status mega_moe_noalloc(const mm_plan* plan, const void* x, const int32_t* topk_ids,
                           const float* topk_weights, const int8_t* x_active_mask,
                           const void* w1, const void* w1_scale, const void* w2, const void* w2_scale,
                           void* y, int32_t* expert_token_nums, void* stream);

/* Bits of the device error word. */
typedef enum mm_device_error {
  MM_DEVERR_NONE = 0,
  MM_DEVERR_BAD_EXPERT = 1,      /* a route named an expert id >= E (skipped like a masked route) */
  MM_DEVERR_BARRIER_TIMEOUT = 2, /* a wait inside a kernel gave up (a grid barrier of mega_moe, or a GEMM
                                    waiting for another workgroup's partial sums of a split tile);
                                    y is unspecified */
  MM_DEVERR_BAD_OFFSETS = 4      /* a GEMM got offsets/counts that do not describe a padded pool
                                    of at most P rows: it ran no tile (its outputs are unspecified) */
} mm_device_error;

/*
 * mm_read_device_error -- copies the error word of this workspace into
 * *host_out, asynchronously on `stream`: read it after the stream has
 * synchronised.  mega_moe and mm_dispatch_layout clear the word when they
 * start; the two GEMM entry points only add bits to it.  Diagnostics only.
 *   workspace  the workspace passed to that call (NULL: mega_moe_noalloc's)
 *   host_out   host int32, receives an OR of mm_device_error bits
 */
mm_status mm_read_device_error(const mm_plan* plan, const void* workspace, int32_t* host_out, void* stream);

/*
 * mm_debug_raw_accumulators -- the GEMM accumulators before any scaling:
 * for A8W8_INT8 the int32 sums, for checking that the products are exact
 * (operator page, A8W8-INT: C = Q_e . W1[e] and D = A^int8 . W2[e] in Z_32);
 * for A8W8_FP8 the float32 sums of the e4m3 code products, as int32 bit
 * patterns, for measuring how far the e4m3 MFMA's sums are from the exact
 * ones (Linear1 in the mode mega_moe uses: exact bf16 MFMA or e4m3 MFMA).
 * Runs the same mainloop, tile shape and tail-tile K split as the entry
 * points with an epilogue that stores the raw accumulators (other use
 * cases: MM_ERR_UNSUPPORTED).
 *   which = 1: c_out int32 [P][2I], column order of the formula (gate then up),
 *              from x_pool and the prepared w1;
 *   which = 2: c_out int32 [P][H] from a_pool and the prepared w2.
 *   workspace  device, plan.workspace_bytes (partial sums of split tiles)
 * Padding rows of c_out are unspecified.
 */
mm_status mm_debug_raw_accumulators(const mm_plan* plan, int which, const int32_t* expert_offsets,
                                    const int32_t* expert_counts, const void* act_pool,
                                    const void* w_prepared, int32_t* c_out,
                                    void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * mm_debug_fused_layout -- copies the dispatch metadata that the last
 * mega_moe call on `workspace` built inside it (DeepEP notes, sections 1
 * and 3.5: the padded per-expert offsets and the (token, slot) identity of
 * every pool row), asynchronously on `stream`, so that it can be checked
 * like mm_dispatch_layout's outputs (workspace NULL: the last
 * mega_moe_noalloc call's).  Diagnostics only.
 *   offsets_out        device int32 [E+S+1]
 *   pool_src_out       device int32 [P]
 *   route_to_pool_out  device int32 [T*(K+S)]
 */
mm_status mm_debug_fused_layout(const mm_plan* plan, const void* workspace, int32_t* offsets_out,
                                int32_t* pool_src_out, int32_t* route_to_pool_out, void* stream);

/*
 * mm_read_kernel_clock -- the clock sample of the last mega_moe call on
 * `workspace`: its workgroup 0 reads the shader-clock counter (s_memtime)
 * and the constant 100 MHz counter (s_memrealtime) when it starts and when
 * it is done.  host_out[0], [1]: shader clocks at start and end; [2], [3]:
 * 100 MHz ticks at start and end, so the mean shader clock over the run is
 * 100 MHz * (out[1] - out[0]) / (out[3] - out[2]).  Copied asynchronously on
 * `stream`; read it after the stream has synchronised.  Diagnostics only.
 */
mm_status mm_read_kernel_clock(const mm_plan* plan, const void* workspace, uint64_t* host_out, void* stream);

/* Kernel timing (diagnostics).  While enabled, every kernel the library
 * launches is bracketed by two HIP events on its stream; mm_trace_collect
 * waits for them and returns, per kernel id, the number of launches and
 * the summed duration in milliseconds, then clears the record. */
typedef enum mm_kernel_id {
  MM_K_ZERO = 0, MM_K_COUNT = 1, MM_K_SCATTER = 2, MM_K_GATHER = 3,
  MM_K_L1 = 4, MM_K_REQUANT = 5, MM_K_L2 = 6, MM_K_COMBINE = 7, MM_K_PREPARE = 8,
  MM_K_MEGA = 9,                 /* the fused persistent kernel of mega_moe */
  MM_K_COUNT_IDS = 10
} mm_kernel_id;

mm_status mm_trace_enable(int on);
mm_status mm_trace_collect(int32_t* launches /* [MM_K_COUNT_IDS] */,
                           double* total_ms /* [MM_K_COUNT_IDS] */);
const char* mm_kernel_name(int kernel_id);

const char* mm_status_string(mm_status s);

#ifdef __cplusplus
}
#endif
#endif /* MEGAMOE_H */
