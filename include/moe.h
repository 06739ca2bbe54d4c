/*
 * moe.h -- C ABI of a single-GPU (MI355X, gfx950) Mixture-of-Experts layer:
 *          route -> capacity-limited dispatch -> expert FFN -> weighted combine,
 *          plus a counters-only ledger.
 *
 * Pages cited (by title):
 *   [EP47] "47. MoE Expert Parallel | MoE 专家并行" (llm-algo-leetcode, ch. 47)
 *   [EP46] "46. MoE Expert Parallel | MoE 专家并行" (llm-algo-leetcode, ch. 46)
 *   [EPC]  "专家并行（Expert Parallelism）" (tier6-model)
 *   [DSV3] "MoE大模型专家并行与动态路由优化——从DeepSeek-V3到生产级推理架构"
 *
 * Conventions for every entry point
 *   - All tensors are dense, row-major, on the device, allocated and owned by
 *     the caller.  The library never allocates device memory and keeps no
 *     state between calls; it is safe to call from several host threads on
 *     different streams with different workspaces.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every entry point
 *     except moe_ledger only enqueues work and returns; moe_ledger waits for
 *     the stream (it copies the counters back to the host).
 *   - Floating-point activations and weights are MOE_BF16 (bfloat16) or
 *     MOE_F32 as cfg->dtype says; logits, gates, biases, expert outputs and
 *     the layer output are always fp32.
 *   - bf16 tensors and the dispatched buffer must be 16-byte aligned; on the
 *     bf16 path h and F must be multiples of 64 (else MOE_ERR_UNSUPPORTED).
 *   - Host-detectable errors (NULL pointers, sizes, K > E, capacity < 0,
 *     workspace too small, owner rank >= n_ep) return before anything is
 *     enqueued.  An expert id outside [0, E) inside a caller-built topk_idx is
 *     detected on the device: dispatch drops such a route and moe_ledger
 *     reports MOE_ERR_EXPERT_ID.  No exception crosses the ABI.
 *   - Sizes: T tokens, h hidden size, E experts, K experts per token, F FFN
 *     width, A = T*K routes, cap = capacity, R_max = min(A, E*cap) rows.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* NULL pointer, negative size, K > E, cf <= 0 ... */
  MOE_ERR_EXPERT_ID = 2,    /* device-detected expert id outside [0, E)       */
  MOE_ERR_SHAPE = 3,        /* inconsistent sizes (e.g. workspace too small)  */
  MOE_ERR_HIP = 4,          /* a HIP runtime call or kernel launch failed      */
  MOE_ERR_UNSUPPORTED = 5   /* valid, but outside what the kernels implement  */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Shape of one MoE layer invocation.  T may be 0 (an empty batch is valid
 * and yields a zero ledger, [EP46] empty-route contract). */
typedef struct moe_cfg {
  int32_t T;        /* tokens                                     */
  int32_t h;        /* hidden size (model dim)                    */
  int32_t E;        /* experts, 1..1024                           */
  int32_t K;        /* experts per token, 1..min(E, 32)           */
  int32_t F;        /* expert FFN width                           */
  int32_t dtype;    /* moe_dtype of x, W_g, W1, W2 and H          */
  double capacity_factor;  /* > 0                                  */
} moe_cfg;

/* Counters of one routed batch ([EP47] route ledger, [EP46] ledger and
 * dispatch-locality summaries, [DSV3] 3.2 load-balance terms).  Byte counts
 * use bytes_per_elem = 4 (MOE_F32) or 2 (MOE_BF16). */
typedef struct moe_ledger_t {
  int64_t total_tokens;          /* T                                         */
  int64_t total_routes;          /* A = T*K                                   */
  int64_t num_experts;           /* E                                         */
  int64_t capacity;              /* the capacity passed in                    */
  int64_t accepted_routes;       /* R = routes with route_row >= 0            */
  int64_t overflow;              /* sum_e max(load_e - capacity, 0)           */
  int64_t max_load;              /* max_e load_e                              */
  int64_t invalid_routes;        /* ids outside [0, E) (then status != OK)    */
  int64_t logical_route_bytes;   /* A*h*bytes (= the pages' dispatch_bytes)   */
  int64_t all_to_all_bytes;      /* 2 * logical_route_bytes                   */
  int64_t accepted_route_bytes;  /* R*h*bytes                                 */
  int64_t local_routes;          /* all routes with src_rank == owner_rank    */
  int64_t cross_rank_routes;     /* all routes with src_rank != owner_rank    */
  int64_t cross_rank_dispatch_bytes;   /* cross_rank_routes*h*bytes           */
  int64_t cross_rank_roundtrip_bytes;  /* 2 * cross_rank_dispatch_bytes       */
  int64_t accepted_local_routes;       /* same split over accepted routes     */
  int64_t accepted_cross_rank_routes;
  int64_t accepted_cross_rank_dispatch_bytes;
  int64_t accepted_cross_rank_roundtrip_bytes;
  int64_t n_ep;                  /* logical expert-parallel ranks             */
  double balance_ratio;          /* max load / (A/E), 0.0 when A == 0         */
  double local_hit_ratio;        /* local_routes / A, 0.0 when A == 0         */
  double accepted_local_hit_ratio;
  double pair_bytes_uniform;     /* logical_route_bytes / n_ep ([EPC])        */
  double l_aux;                  /* alpha * sum_i f_i P_i                     */
  double l_aux_norm;             /* alpha * E/K * sum_i f_i P_i               */
  double alpha;
  double load_var_over_mean;     /* unbiased variance of loads / mean load    */
  int32_t imbalanced;            /* 1 when max/mean load > 2                  */
  int32_t status;                /* MOE_OK or MOE_ERR_EXPERT_ID               */
} moe_ledger_t;

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(int status);

/* ceil((A / E) * capacity_factor) evaluated in IEEE double; 0 when A == 0;
 * -1 for E <= 0, A < 0 or capacity_factor not > 0.
 * [EP47] Step 3 (capacity), [EP46] TODO 1.  Pure host function. */
int64_t moe_capacity(int64_t A, int32_t E, double capacity_factor);

/* R_max = min(T*K, E*capacity): rows of the dispatched buffers. */
int64_t moe_max_rows(const moe_cfg* cfg, int64_t capacity);

/* Bytes of device workspace every call below needs for `cfg` (any n_ep up
 * to 64).  The same workspace may be reused by successive calls on one
 * stream; its contents need no initialisation. */
size_t moe_workspace_bytes(const moe_cfg* cfg);

/* Router: logits = x W_g^T (+ logit_bias), then per token the K largest
 * logits (descending; equal logits -> lower expert id) and the softmax over
 * those K ([DSV3] section 一 g = Softmax(TopK(W_g x)); 3.1 TopKGate).
 *   x          [T, h]  dtype      token activations, or NULL: then `logits`
 *                                 is an INPUT and the product is skipped
 *   w_gate     [E, h]  dtype      router weight (ignored when x == NULL)
 *   logit_bias [E]     fp32|NULL  added to every token's logits before the
 *                                 top-k; the softmax uses the biased logits
 *   logits     [T, E]  fp32       written (x != NULL) or read (x == NULL);
 *                                 always WITHOUT the bias
 *   topk_idx   [T, K]  int32      expert ids, slot 0 = largest
 *   topk_gate  [T, K]  fp32       softmax weights, each row sums to 1
 *   expert_load [E]    int32|NULL pre-capacity histogram of topk_idx
 * ws (16-byte aligned, may be NULL): for long batches or many experts the
 * bf16 product splits h into ranges whose fp32 partial products are kept
 * there and added in range order; with no (or too small a) workspace the
 * product runs unsplit, slower but equally valid.  Logits are not NaN. */
int moe_route(const moe_cfg* cfg, const void* x, const void* w_gate,
              const float* logit_bias, float* logits, int32_t* topk_idx,
              float* topk_gate, int32_t* expert_load, void* ws, size_t ws_bytes,
              void* stream);

/* FP8 (OCP E4M3) dispatch payload ([DSV3] 4.3: quantise the bf16 hidden
 * states to FP8 before the all-to-all, dequantise after it).  bf16 only.
 *
 * moe_fp8_scale: scale[0] = bf16(max|x| / 448) over the whole [T, h] tensor
 *   x (stored as the fp32 value of that bf16; 0 for all-zero x).  Uses the
 *   workspace (moe_workspace_bytes).  Asynchronous.
 * moe_dispatch_fp8: moe_dispatch whose gather sends E4M3 codes: x_disp_q
 *   [R_max, h] uint8 receives code(bf16(x / scale)) (ties to even; zero codes
 *   when scale == 0) of each accepted row; every other output as in
 *   moe_dispatch.  x and x_disp_q 16-byte aligned.
 * moe_fp8_dequantize: the receiver, x_disp[r] = bf16(value(code) * scale)
 *   for the R = expert_offsets[E] accepted rows (read on the device); rows
 *   >= R are left untouched.  Its output feeds moe_expert_ffn*.
 * All three return MOE_ERR_UNSUPPORTED for fp32 configurations. */
int moe_fp8_scale(const moe_cfg* cfg, const void* x, float* scale, void* ws,
                  size_t ws_bytes, void* stream);
int moe_dispatch_fp8(const moe_cfg* cfg, const void* x, const float* scale,
                     const int32_t* topk_idx, int64_t capacity, int32_t* expert_offsets,
                     int32_t* route_rank, int32_t* route_row, int32_t* row_token,
                     uint8_t* x_disp_q, int32_t* expert_load, void* ws, size_t ws_bytes,
                     void* stream);
int moe_fp8_dequantize(const moe_cfg* cfg, int64_t capacity, const uint8_t* x_disp_q,
                       const float* scale, const int32_t* expert_offsets, void* x_disp,
                       void* stream);

/* The expert FFN on the FP8 dispatch payload ([DSV3] 4.3: the receiver
 * dequantises the E4M3 hidden states before its experts): the H and Y of
 * moe_expert_ffn (packed == 0) or moe_expert_ffn_packed (packed != 0) on
 * x_disp[r] = bf16(value(x_disp_q[r]) * scale), with that dequantisation done
 * by the first GEMM as it stages its activations (no bf16 copy of the rows
 * is written).  x_disp_q [R_max, h] uint8 from moe_dispatch_fp8, scale the
 * device fp32 from moe_fp8_scale; the other arguments as for moe_expert_ffn.
 * bf16 only; MOE_ERR_UNSUPPORTED also where the first GEMM's rows per
 * expert (min(capacity, ceil(T*K/E))) reach 384 while F is not a multiple of
 * 128 (a shape whose kernel reads bf16 activations only), unless the weights
 * are packed and those rows reach 512. */
int moe_expert_ffn_fp8(const moe_cfg* cfg, int64_t capacity, const uint8_t* x_disp_q,
                       const float* scale, const int32_t* expert_offsets, const void* w1,
                       const float* b1, const void* w2, const float* b2, void* h_buf, float* y,
                       int32_t packed, void* stream);

/* Aux-loss-free balancing: one step of the expert-bias rule of [DSV3]
 * section 八 (DeepSeekV3Gate), bias += alpha * (mean_count - count), where
 * count[e] = tokens whose largest bias-adjusted logit is expert e.
 *   topk_idx    [T, K] int32  routing made by moe_route with
 *                             logit_bias = expert_bias (slot 0 = argmax of
 *                             the adjusted logits); ids outside [0, E) are
 *                             not counted
 *   expert_bias [E] fp32      updated in place (device memory)
 *   alpha                     step size (the page uses 0.1); finite
 *   counts      [E] int32|NULL  the per-expert counts used
 * In fp32 with one rounding per operation and no fused multiply-add:
 * mean = sum(count) / E, then per expert bias + alpha * (mean - count).
 * Asynchronous on `stream`; one workgroup. */
int moe_bias_update(const moe_cfg* cfg, const int32_t* topk_idx, float* expert_bias,
                    float alpha, int32_t* counts, void* stream);

/* Capacity-limited dispatch ([DSV3] 3.3 capacity loop; [EPC] Dispatch).
 * Routes are taken in (token, k-slot) order; the first `capacity` routes of
 * each expert are accepted and the rest dropped.  Accepted routes are packed
 * per expert (experts in id order, tokens in order inside an expert):
 *   expert_offsets [E+1] int32   exclusive prefix of min(load_e, capacity)
 *   route_rank     [T,K] int32   routes to the same expert before this one
 *                                (-1 for an invalid id)
 *   route_row      [T,K] int32   offset[e] + rank if rank < capacity, else -1
 *   row_token      [R_max] int32 token of each accepted row (rows >= R are
 *                                left untouched)
 *   x_disp         [R_max, h] dtype  x_disp[row] = x[row_token[row]] (rows
 *                                    >= R are left untouched); or NULL:
 *                                    routing metadata only (x may then be
 *                                    NULL), for moe_expert_ffn_rows
 *   expert_load    [E] int32|NULL    pre-capacity load of each expert
 * ws: at least moe_workspace_bytes(cfg) bytes.
 * Dropless variant: any capacity >= T accepts every route (a token's K
 * experts are distinct, so no expert receives more than T routes); then
 * R = T*K and R_max = T*K.  This is the dispatch that aux-loss-free
 * balancing (moe_bias_update) pairs with ([DSV3] 3.3, section 八). */
int moe_dispatch(const moe_cfg* cfg, const void* x, const int32_t* topk_idx,
                 int64_t capacity, int32_t* expert_offsets, int32_t* route_rank,
                 int32_t* route_row, int32_t* row_token, void* x_disp,
                 int32_t* expert_load, void* ws, size_t ws_bytes, void* stream);

/* moe_dispatch for callers that cannot allocate memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same arguments and results as moe_dispatch, without the workspace: the
 * dispatch's scratch (the per-block expert counts, ceil(T*K/1024) * (E+1)
 * int32) lives in a static device array of MOE_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends.  Allocates
 * nothing (no hipMalloc, no allocating library call).  Returns
 * MOE_ERR_UNSUPPORTED, before enqueuing anything, when that scratch would
 * exceed the array: ceil(T*K/1024) * (E+1) * 4 bytes, rounded up to 256,
 * above MOE_NOALLOC_SCRATCH_BYTES (4 MiB), e.g. more than 1,047,552 routes at
 * E = 1024 or 16,518,144 at E = 64.  Every call on one
 * GPU shares the array: calls that overlap on one GPU (on different streams
 * or host threads) race on it and may give wrong results; calls in order on
 * one stream are safe.  `stream` must belong to the current device. */
#define MOE_NOALLOC_SCRATCH_BYTES (4 << 20)
int moe_dispatch_noalloc(const moe_cfg* cfg, const void* x, const int32_t* topk_idx,
                         int64_t capacity, int32_t* expert_offsets, int32_t* route_rank,
                         int32_t* route_row, int32_t* row_token, void* x_disp,
                         int32_t* expert_load, void* stream);

/* Expert FFN over ragged expert segments ([DSV3] section 一
 * FFN(x) = W2 GELU(W1 x + b1) + b2, GELU in its tanh form):
 * for each expert e and row r in [offset[e], offset[e+1]):
 *   H[r] = GELU_tanh(W1[e] x_disp[r] + b1[e])   stored as dtype (bf16 RNE)
 *   Y[r] = W2[e] H[r] + b2[e]                    fp32
 *   x_disp [R_max, h] dtype;  w1 [E, F, h] dtype;  b1 [E, F] fp32
 *   w2 [E, h, F] dtype;  b2 [E, h] fp32;  h_buf [R_max, F] dtype (scratch,
 *   holds H afterwards);  y [R_max, h] fp32.  Rows >= R are not written.
 * `capacity` bounds R_max and every expert's segment, offset[e+1] -
 * offset[e] <= capacity (the same value given to moe_dispatch, whose
 * offsets satisfy it). */
int moe_expert_ffn(const moe_cfg* cfg, int64_t capacity, const void* x_disp,
                   const int32_t* expert_offsets, const void* w1, const float* b1,
                   const void* w2, const float* b2, void* h_buf, float* y,
                   void* stream);

/* The same expert FFN on weights in the packed fragment layout produced by
 * moe_pack_expert_weights (bf16 only).  Expert weights are static, so a
 * server packs them once at load time; the packed layout lets every wave
 * read its MFMA operands as contiguous 1 KB loads.  Arguments and results
 * are those of moe_expert_ffn. */
int moe_expert_ffn_packed(const moe_cfg* cfg, int64_t capacity, const void* x_disp,
                          const int32_t* expert_offsets, const void* w1_packed,
                          const float* b1, const void* w2_packed, const float* b2,
                          void* h_buf, float* y, void* stream);

/* Repack row-major expert weights (bf16) into the fragment layout:
 * for expert e, 32-row tile t, 64-wide k-chunk c, one 4096-byte block at
 * index (e * (N/32) + t) * (K/64) + c, whose 16-byte quad (64*q + l) holds
 * W[e][32t + l%32][64c + 32*(l/32) + 8q .. +7]  (l = 0..63, q = 0..3).
 * w1 [E, F, h] -> w1_packed (N = F, K = h); w2 [E, h, F] -> w2_packed
 * (N = h, K = F); same byte size as the input.  Either pair may be NULL.
 * Output buffers must not alias the inputs.  Asynchronous on `stream`. */
int moe_pack_expert_weights(const moe_cfg* cfg, const void* w1, const void* w2,
                            void* w1_packed, void* w2_packed, void* stream);

/* The expert FFN reading its rows from the token matrix: the same H and Y as
 * moe_expert_ffn (packed == 0) or moe_expert_ffn_packed (packed != 0) on
 * x_disp[r] = x[row_token[r]] ([EPC] Dispatch; [DSV3] section 一 FFN), with
 * that gather done by the first GEMM's own loads where its rows are few (a
 * few hundred per expert or less), and otherwise by a row copy into y's
 * storage that the first GEMM reads before the second writes y.  Pairs with
 * moe_dispatch(x_disp = NULL), which then moves no row.
 *   x [T, h] dtype (16-byte aligned); row_token [R_max] int32 from
 *   moe_dispatch (its first R entries must lie in [0, T): they are used as
 *   row indices of x without a check); the other arguments as for
 *   moe_expert_ffn.  y's storage may serve as staging for the rows. */
int moe_expert_ffn_rows(const moe_cfg* cfg, int64_t capacity, const void* x,
                        const int32_t* row_token, const int32_t* expert_offsets,
                        const void* w1, const float* b1, const void* w2, const float* b2,
                        void* h_buf, float* y, int32_t packed, void* stream);

/* Weighted combine in original token order, without atomics ([EP46]
 * combine_expert_outputs; [EPC] Combine):
 *   out[t] = sum over k = 0..K-1 with route_row[t,k] >= 0 of
 *            topk_gate[t,k] * y[route_row[t,k]]       (fp32, k ascending)
 * A token whose routes were all dropped gets zeros.  out [T, h] fp32. */
int moe_combine(const moe_cfg* cfg, const float* y, const int32_t* route_row,
                const float* topk_gate, float* out, void* stream);

/* Counters-only ledger ([EP47] summarize, [EP46] summarize + dispatch
 * locality, [DSV3] 2.2 placement and 3.2 auxiliary-loss terms).
 *   topk_idx [T,K] int32, topk_gate [T,K] fp32, route_row [T,K] int32 (from
 *   moe_dispatch), src_rank [T] int32 (token's source rank), owner_rank [E]
 *   int32 (expert's rank, e.g. e % n_ep), n_ep in 1..64, alpha (0.01 on the
 *   page).  Host outputs (each may be NULL except `out`): loads [E] int64,
 *   f [E] and P [E] double (f_i = load_i / T, P_i = sum_t g_{t,i} / T),
 *   pair_routes [n_ep*n_ep] int64 (accepted routes from source rank i to
 *   owner rank j, row-major).
 * Synchronises `stream`.  Returns MOE_ERR_EXPERT_ID (with `out` filled) when
 * topk_idx holds an id outside [0, E). */
int moe_ledger(const moe_cfg* cfg, const int32_t* topk_idx, const float* topk_gate,
               const int32_t* route_row, int64_t capacity, const int32_t* src_rank,
               const int32_t* owner_rank, int32_t n_ep, double alpha,
               moe_ledger_t* out, int64_t* loads, double* f, double* P,
               int64_t* pair_routes, void* ws, size_t ws_bytes, void* stream);

/* The same ledger in two halves, so that a serving loop (or a captured HIP
 * graph) never waits on the host:
 *   moe_ledger_launch  enqueues the counting kernels, whose compact counters
 *                      end up in `host_stage` (caller's host memory of
 *                      moe_ledger_stage_bytes(cfg, n_ep) bytes).  Page-locked
 *                      memory mapped into the device address space (what
 *                      hipHostMalloc returns) is written by the kernels
 *                      themselves; any other host memory receives an
 *                      asynchronous copy enqueued after them;
 *   moe_ledger_finalize, once that copy has completed (stream or event
 *                      synchronisation by the caller), turns the stage into
 *                      the same outputs as moe_ledger.  Pure host function.
 * The workspace must not be reused by another call before the copy is done.
 * moe_ledger_stage_bytes returns 0 for invalid arguments. */
size_t moe_ledger_stage_bytes(const moe_cfg* cfg, int32_t n_ep);
int moe_ledger_launch(const moe_cfg* cfg, const int32_t* topk_idx, const float* topk_gate,
                      const int32_t* route_row, const int32_t* src_rank,
                      const int32_t* owner_rank, int32_t n_ep, void* host_stage,
                      size_t stage_bytes, void* ws, size_t ws_bytes, void* stream);
/* moe_ledger_finalize returns MOE_ERR_SHAPE, and leaves every output
 * unwritten, for a stage that holds no completed ledger (its part count is
 * outside 1..4: zeroed, torn or never written).  Otherwise its statuses are
 * moe_ledger's, with `out` filled: MOE_OK, MOE_ERR_EXPERT_ID for ids outside
 * [0, E), MOE_ERR_INVALID_ARG for source or owner ranks outside [0, n_ep)
 * (out->status then holds the same code); argument errors (NULL pointers,
 * capacity < 0, n_ep outside 1..64) return MOE_ERR_INVALID_ARG with `out`
 * unwritten, so a caller tells the two apart by out->status. */
int moe_ledger_finalize(const moe_cfg* cfg, int64_t capacity, int32_t n_ep, double alpha,
                        const void* host_stage, moe_ledger_t* out, int64_t* loads,
                        double* f, double* P, int64_t* pair_routes);

/* moe_combine and moe_ledger_launch of the same routes in one call ([EP46]
 * combine_expert_outputs and summarize; [EPC] Combine; [EP47] summarize):
 * the arguments of both, the same `out`, and a `host_stage` that
 * moe_ledger_finalize decodes to the same ledger once the stream has passed
 * the call (its part count and byte layout may differ from
 * moe_ledger_launch's).  Up to 4096 routes (T*K) both run in ONE launch, the ledger's
 * workgroups (one per 1024 routes, each writing its own integer partials
 * into the stage, which moe_ledger_finalize adds) beside the combine's;
 * above that it enqueues the two calls' kernels in turn.  The
 * workspace is the ledger's (moe_workspace_bytes) and must not be reused
 * before the stage copy is done, as for moe_ledger_launch. */
int moe_combine_ledger(const moe_cfg* cfg, const float* y, const int32_t* route_row,
                       const float* topk_gate, float* out, const int32_t* topk_idx,
                       const int32_t* src_rank, const int32_t* owner_rank, int32_t n_ep,
                       void* host_stage, size_t stage_bytes, void* ws, size_t ws_bytes,
                       void* stream);

/* Joint parallel-plan decision over one ledger ([EP46] TODO 3, joint
 * decision; thresholds default to that page's):
 *   MOE_PLAN_ACCEPT  no overflow, balance_ratio <= 1.2 and cross-rank share
 *                    <= 0.5;
 *   MOE_PLAN_TUNE    overflow / total_routes <= 0.25, balance_ratio <= 1.8 and
 *                    cross-rank share <= 0.9;
 *   MOE_PLAN_REJECT  otherwise, and for an empty batch.
 * balance_ratio enters the comparisons rounded to 3 decimals (ties to even,
 * as Python's round(x, 3)), the value that page's summary stores.
 * The cross-rank share is cross_rank_routes / (local_routes +
 * cross_rank_routes) (all routes) when use_locality != 0, else 0.
 * thresholds: NULL, or 5 doubles in the order above (accept balance, accept
 * cross share, tune overflow share, tune balance, tune cross share).
 * Pure host function; returns -1 for a NULL ledger. */
enum { MOE_PLAN_ACCEPT = 0, MOE_PLAN_TUNE = 1, MOE_PLAN_REJECT = 2 };
int moe_recommend_plan(const moe_ledger_t* ledger, const double* thresholds,
                       int32_t use_locality);

/* Locality-aware expert placement ([EP46] Step 3: a more local placement of
 * the experts cuts cross-rank dispatch, watching whether the per-rank load
 * gets skewed; [DSV3] 2.2: uniform placement of E / N experts per device,
 * topology-aware placement matched on an affinity matrix by the Hungarian
 * algorithm).
 *
 * moe_expert_rank_affinity: affinity [E, n_ep] int32 (device) = routes to
 *   expert e from tokens of source rank r, over all routes (route_row NULL)
 *   or over the accepted ones (route_row[t,k] >= 0).  Ids outside [0, E) and
 *   ranks outside [0, n_ep) are not counted (moe_ledger reports them).
 *   Asynchronous on `stream`; the matrix is cleared by the call itself.
 * moe_place_experts: pure host function.  owner [E] int32 = the expert ->
 *   rank map with E / n_ep experts per rank that maximises the routes kept
 *   local, sum_e affinity[e][owner[e]] (affinity: host [E, n_ep] int32,
 *   non-negative).  An exact assignment (O(E^3) integer Hungarian method);
 *   when several maps reach the maximum, one of them.  E must be a multiple
 *   of n_ep (else MOE_ERR_INVALID_ARG). */
int moe_expert_rank_affinity(const moe_cfg* cfg, const int32_t* topk_idx,
                             const int32_t* route_row, const int32_t* src_rank, int32_t n_ep,
                             int32_t* affinity, void* stream);
int moe_place_experts(const int32_t* affinity, int32_t E, int32_t n_ep, int32_t* owner);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
