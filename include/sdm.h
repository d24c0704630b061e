/*
 * sdm.h -- C ABI of the Sparse Delta Memory (SDM) layer on MI355X (gfx950): the forward
 * path (selection pass and recurrent sparse scan), its variants, the scan's training
 * backward and a slot-update monitor.
 *
 * The method (no published code; defined by these pages):
 *   [rainbus]  "稀疏增量记忆：通过稀疏性扩展线性RNN的状态 / Sparse Delta Memory: Scaling
 *              the State of Linear RNNs through Sparsity", paper.rainbus.top, method
 *              paragraph (steps 1-4 with their formulas);
 *   [analysis] "用稀疏内存把线性RNN的状态放大1000倍：Meta SDM 在 8B 规模反超 Full
 *              Attention", ai-paper-analysis.pages.dev, sections "步骤 1" .. "步骤 4",
 *              Figure 2, and the section on the learned initial state M0;
 *   [163]      m.163.com article on arXiv 2607.07386, section 二 (outer-sum product-key
 *              addressing, forget + delta write, weighted sparse read).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer (allocated by the caller, e.g. as a
 *    torch tensor) unless stated otherwise; `dims` and `sel` structs live in host
 *    memory.  The library never allocates or frees device memory and is reentrant
 *    across streams.  Its global state: the host-side record of SDM_FLAG_TIMING (HIP
 *    events, created on first use), and the fixed device array that only
 *    sdm_forward_noalloc uses as its workspace (with its per-device address).
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is enqueued on it
 *    asynchronously; no call synchronises the host, allocates, or copies through
 *    pageable memory, so calls may be captured into a HIP graph.
 *  - Every argument is validated BEFORE anything is enqueued: a call that returns a
 *    nonzero status has enqueued nothing and left every output untouched.  Faults
 *    inside kernels surface at the caller's next synchronisation.  A launch error
 *    reported by the runtime right after a launch returns SDM_ERR_HIP.
 *  - Device pointers must be 16-byte aligned (SDM_ERR_ALIGN).
 *  - Layouts are row-major and contiguous.  Per-token tensors are [B, T, H, ...];
 *    the state is [B, H, N, d_v] fp32 (bf16 with SDM_FLAG_STATE_BF16) with N = n*n
 *    slots; slot id = i*n + j where i indexes the first half-score vector and j the
 *    second.
 *  - B*T == 0 is a valid empty call: SDM_OK, nothing enqueued.
 *  - NaN or Inf inputs propagate per IEEE in the arithmetic; the selection order of
 *    NaN scores is unspecified.
 */
#ifndef SDM_H
#define SDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SDM_API __attribute__((visibility("default")))
#else
#define SDM_API
#endif

#define SDM_ABI_VERSION 4

/* status codes */
#define SDM_OK 0
#define SDM_ERR_NULL (-1)        /* a required pointer is NULL */
#define SDM_ERR_SHAPE (-2)       /* inconsistent or out-of-range sizes */
#define SDM_ERR_DTYPE (-3)       /* unknown in_dtype or gate_act */
#define SDM_ERR_ALIGN (-4)       /* a device pointer is not 16-byte aligned */
#define SDM_ERR_WORKSPACE (-5)   /* workspace missing or smaller than sdm_workspace_bytes */
#define SDM_ERR_UNSUPPORTED (-6) /* valid for the method but outside this build's limits */
#define SDM_ERR_HIP (-7)         /* the HIP runtime reported a launch error */

/* element type of x and W_proj */
#define SDM_DTYPE_F32 0
#define SDM_DTYPE_BF16 1

/* activation of the output-gate vector */
#define SDM_GATE_NONE 0
#define SDM_GATE_SIGMOID 1
#define SDM_GATE_SILU 2

/* entry selector for sdm_workspace_bytes */
#define SDM_ENTRY_SELECT 0
#define SDM_ENTRY_SCAN 1
#define SDM_ENTRY_FORWARD 2
#define SDM_ENTRY_SCAN_BACKWARD 3
#define SDM_ENTRY_SCAN_TRAIN 4
#define SDM_ENTRY_SELECT_FROM_SCORES 5
#define SDM_ENTRY_SELECT_BACKWARD 6

/* scan schedule flags (sdm_dims.flags) */
#define SDM_FLAG_SCAN_DIRECT 1    /* one workgroup per (b,h), tokens in lock-step */
#define SDM_FLAG_SCAN_STREAM 2    /* slot-owner lane groups fed by per-group streams,
                                     a walk's groups split over workgroups */
#define SDM_FLAG_SCAN_TWO_PHASE 4 /* slot-owner writes, then token-major reads of the
                                     slots each workgroup owns */
/* Without a schedule flag, sdm_scan and sdm_forward run the per-slot rule on the
   two-phase schedule from 16 tokens, and on the direct one below that or from 512
   walks (B H: the lock-step workgroups then fill the chip twice over). */
/* instrumentation flag (sdm_dims.flags, may be combined with one schedule flag):
   every kernel launch of the call is bracketed by a pair of HIP events recorded on
   the call's stream; sdm_timing_read returns the durations.  Results are the same
   with and without it. */
#define SDM_FLAG_TIMING 8
/* variant flag (sdm_dims.flags): the write's error term is the key-weighted
   prediction of the whole write set, M[i] <- aM[i] + b k_i (v - sum_j k_j aM[j]),
   i.e. Gated DeltaNet's delta rule restricted to the selected slots (the form the
   pages say the layer reduces to when every slot is selected with a dense key:
   ai-paper-analysis.pages.dev, section "与 GDN 的关系"; m.163.com article on
   arXiv 2607.07386, section 二).  It needs every row of a token's write set before
   any is written, so it runs the direct schedule (each walk split over 16- or
   32-column slices of the state, which evolve independently under the rule) or the
   chunk schedule (SDM_FLAG_SCAN_CHUNK, its default from 64 tokens with an fp32
   state while B H d_v / 16 <= 1024: beyond that many (walk, slice) workgroups the
   sliced direct walk is faster); combined with SDM_FLAG_SCAN_STREAM or
   SDM_FLAG_SCAN_TWO_PHASE it is SDM_ERR_UNSUPPORTED. */
#define SDM_FLAG_DELTA_GDN 16
/* storage flag (sdm_dims.flags; sdm_scan and sdm_forward): the state buffer holds
   bf16 values.  The arithmetic stays fp32; each written row element is rounded to
   the nearest bf16 (ties to even) when stored, and later accesses of the token run
   see that stored value.  Half the state bytes of the fp32 layout move per slot
   access.  Not a step of the pages: they keep the live state in full precision and
   quantise only training checkpoints (to fp8 or int4, for long fine-tuning runs:
   ai-paper-analysis.pages.dev, section "训练效率"; m.163.com article on arXiv
   2607.07386, section 八).  Every schedule and both write rules support it. */
#define SDM_FLAG_STATE_BF16 32
/* storage flag (sdm_dims.flags; sdm_scan and sdm_forward): the state buffer holds
   fp8, B*H*N*d_v*33/32 bytes -- a codes plane [B, H, N, d_v] of OCP E4M3 bytes (the
   encoding of SDM_FLAG_LOG_FP8's codes), then an exponent plane [B, H, N, d_v / 32]
   of E8M0 bytes, one per 32-column block of a row.  Element = value(code) *
   2^(s - 127).  The arithmetic stays fp32; each written row is requantised block by
   block: e = the least exponent >= -127 with absmax <= 448 * 2^e (read off the fp32
   absmax's bits: its exponent - 8, plus 1 when its significand exceeds 1.75), then
   each element's nearest E4M3 value of x * 2^-e (ties to even; the scaling is exact
   and never saturates).  About a quarter of the fp32 bytes per slot access.  Not a
   step of the pages (see SDM_FLAG_STATE_BF16).  The per-slot rule on the two-phase
   and direct schedules with d_v >= 32; SDM_ERR_UNSUPPORTED with SDM_FLAG_DELTA_GDN,
   SDM_FLAG_SCAN_STREAM or SDM_FLAG_SCAN_CHUNK, d_v < 32, and in the training and
   shared-M0 entries; SDM_ERR_SHAPE with SDM_FLAG_STATE_BF16. */
#define SDM_FLAG_STATE_FP8 512
/* write-log format flags (sdm_dims.flags; sdm_scan_train / sdm_scan_backward only,
   at most one): the training checkpoints quantised as the pages do for long
   fine-tuning (fp8 or int4: m.163.com article on arXiv 2607.07386, section 八;
   ai-paper-analysis.pages.dev, section "训练效率").  One absmax per logged row of d_v
   values, the codes decided in fp32:
     SDM_FLAG_LOG_FP8   v = x * (448 / absmax), nearest OCP E4M3 value (ties to even,
                        saturating at 448); one byte per element
     SDM_FLAG_LOG_INT4  v = x * (7 / absmax), nearest integer (ties to even) in
                        [-7, 7]; two per byte, low nibble first
   Decoded as value * (absmax / 448) or code * (absmax / 7).  The backward then
   computes with, and restores, the decoded rows: the initial state comes back only
   as closely as the format holds it. */
#define SDM_FLAG_LOG_FP8 64
#define SDM_FLAG_LOG_INT4 128
/* schedule flag (sdm_dims.flags; sdm_scan, sdm_forward and their shared-M0 forms):
   the chunkwise-parallel form of the scan that the m.163.com article on arXiv
   2607.07386 (section 八, training paragraph) and the paper.rainbus.top summary (the
   novelty paragraph: chunk-wise parallelism through the WY representation)
   describe.  Tokens are cut into chunks of 32; inside a chunk every output follows
   from the chunk-start state and the tokens' pairwise sparse inner products (a
   two-pointer merge over the ascending slot lists), with a unit lower-triangular
   solve for the SDM_FLAG_DELTA_GDN rule; the state is carried from chunk to chunk.
   The same results as the other schedules up to fp32 rounding order (the decays of
   a chunk are summed as logarithms, each floored at -80).  Needs each token's write
   and read ids ascending (the selection's order), fp32 state (with
   SDM_FLAG_STATE_BF16 it is SDM_ERR_UNSUPPORTED) and a workspace.  sdm_scan_train
   takes it with an fp32 log (the last writer of each slot in a chunk also logs the
   row every earlier writer of the chunk replaced); with SDM_FLAG_LOG_FP8 or
   SDM_FLAG_LOG_INT4 it is SDM_ERR_UNSUPPORTED. */
#define SDM_FLAG_SCAN_CHUNK 256

/* Limits of this build (SDM_ERR_UNSUPPORTED beyond them). */
#define SDM_MAX_COUNT 128   /* W and R */
#define SDM_MAX_HALF 1024   /* n = sqrt(N) */

/*
 * Sizes of one SDM layer.
 *   B, T      batch and tokens per sequence (tokens are b*T + t)
 *   d_model   width of x
 *   H         heads; each head owns one memory of N = n*n slots of d_v floats per
 *             batch entry ([analysis] Figure 2; M_t in R^{N x d_v})
 *   n         half-score length sqrt(N); the pre-index vectors are in R^{2n}
 *             ([rainbus] step 1: W_k, W_q in R^{d x 2 sqrt(N)})
 *   W, R      write and read slots per token and head (top-W / top-R);
 *             1 <= W, R <= min(N, SDM_MAX_COUNT)
 *   d_v       value width; one of 16, 32, 64, 128, 256
 *   in_dtype  SDM_DTYPE_F32 or SDM_DTYPE_BF16 (x and W_proj); d_model % 8 == 0
 *   gate_act  activation of the output gate vector (SDM_GATE_*)
 *   eps       RMSNorm epsilon (>= 0)
 *   flags     0, or one SDM_FLAG_SCAN_* bit to force a scan schedule (all schedules
 *             compute the same recurrence; by default the library picks by shape),
 *             optionally OR-ed with SDM_FLAG_TIMING, SDM_FLAG_DELTA_GDN,
 *             SDM_FLAG_STATE_BF16 and one SDM_FLAG_LOG_* bit (each flag's comment
 *             names the entries it applies to; other entries ignore it)
 */
typedef struct sdm_dims {
  int64_t B, T, d_model;
  int32_t H, n, W, R, d_v;
  int32_t in_dtype;
  int32_t gate_act;
  float eps;
  int32_t flags;
} sdm_dims;

/*
 * Products of the selection pass, [B, T, H, ...] each (caller-allocated):
 *   idx_w [.., W] int32  write slot ids, ascending          ([rainbus] step 1, I_w)
 *   wt_w  [.., W] fp32   sparse key values k^(i), aligned   ([analysis] "步骤 2")
 *   idx_r [.., R] int32  read slot ids, ascending           (I_r)
 *   wt_r  [.., R] fp32   sparse query values q^(i)
 *   v     [.., d_v]      value v_t
 *   gate  [.., d_v]      activated output-gate vector
 *   alpha [..]           forget gate exp(-A softplus(W_a x + b_dt))  ([rainbus] step 2)
 *   beta  [..]           input gate sigma(W_b x)
 *   scores[.., 4n]       nullable: fp32 half-scores (write half 1 | write half 2 |
 *                        read half 1 | read half 2)
 * The weights are the softmax of the selected outer-sum scores; ties in score are
 * broken by the lower slot id.
 */
typedef struct sdm_sel {
  int32_t* idx_w;
  float* wt_w;
  int32_t* idx_r;
  float* wt_r;
  float* v;
  float* gate;
  float* alpha;
  float* beta;
  float* scores;
} sdm_sel;

/* SDM_ABI_VERSION of the built library. */
SDM_API int32_t sdm_abi_version(void);

/* Static human-readable text of a status code (never NULL). */
SDM_API const char* sdm_status_string(int32_t status);

/*
 * Device workspace, in bytes, that `entry` (SDM_ENTRY_*) needs for these sizes;
 * 0 when none is needed or the sizes are invalid.  The workspace is scratch owned by
 * the caller: its contents on entry do not matter and are undefined on return.
 */
SDM_API size_t sdm_workspace_bytes(const sdm_dims* dims, int32_t entry);

/*
 * Selection pass (parallel over tokens): [rainbus] steps 1-2 (projections, the
 * outer-sum product-key selection of top-W write and top-R read slots, gates) and
 * [analysis] "步骤 1".
 *   x       [B*T, d_model]  in_dtype
 *   w_proj  [H*P, d_model]  in_dtype, P = 4n + 2 d_v + 2; per head the P rows
 *           produce, in order: write half 1 (n), write half 2 (n), read half 1 (n),
 *           read half 2 (n), v (d_v), gate pre-activation (d_v), a (1), b (1)
 *   A, b_dt [H] fp32        forget-gate scale and bias per head
 *   out     every field but `scores` required; `scores` may be NULL
 *   ws      >= sdm_workspace_bytes(dims, SDM_ENTRY_SELECT) bytes (may be NULL if 0)
 * The projection accumulates in fp32 on matrix cores; the outer sums of the two fp32
 * half-scores are formed in fp64 (exact) before ranking.
 */
SDM_API int32_t sdm_select(const sdm_dims* dims, const void* x, const void* w_proj, const float* A,
                   const float* b_dt, const sdm_sel* out, void* ws, size_t ws_bytes,
                   void* stream);

/*
 * Selection from given half-scores (diagnostic entry, same ranking as sdm_select):
 * [rainbus] step 1 (top-W / top-R of the outer sums, softmax weights).
 *   scores [B, T, H, 4n] fp32 -> idx_w/wt_w [B,T,H,W], idx_r/wt_r [B,T,H,R].
 *   ws     >= sdm_workspace_bytes(dims, SDM_ENTRY_SELECT_FROM_SCORES) bytes (may be
 *          NULL if 0; this build needs none: the ranking runs in registers and LDS)
 * Given identical scores, the ids are bit-identical to the fp64 brute-force top-W.
 */
SDM_API int32_t sdm_select_from_scores(const sdm_dims* dims, const float* scores, int32_t* idx_w,
                                       float* wt_w, int32_t* idx_r, float* wt_r, void* ws,
                                       size_t ws_bytes, void* stream);

/*
 * Recurrent sparse scan: [rainbus] steps 2-4 without the head-mixing projection.
 * For each (b, h), tokens t = 0..T-1 in order:
 *   for each write slot i (weight k):  c = beta_t * k;
 *       M[i] <- (1 - c) * (alpha_t * M[i]) + c * v_t       (the pages' gated delta
 *       rule Mtilde + beta k (v - Mtilde), Mtilde = alpha M, rearranged so that c = 1
 *       stores v_t exactly and alpha = 1, c = 0 leaves M[i] unchanged)
 *   y_t = sum_{i in I_r} q^(i) M[i]          (after this token's writes)
 *   out_t = y_t / sqrt(mean(y_t^2) + eps) * norm_w[h] * gate_t
 * Slots never selected for writing are never written (bit-identical on return).
 *   in      pass-(a) products (every field but `scores` required)
 *   norm_w  [H, d_v] fp32 RMSNorm weight, or NULL for ones
 *   state   [B, H, N, d_v] fp32 (bf16 with SDM_FLAG_STATE_BF16; fp8 planes with
 *           SDM_FLAG_STATE_FP8), IN/OUT: M_0 on entry
 *           (e.g. a learned initial state,
 *           [analysis] section on M0), M_T on return.  Calling with T tokens equals
 *           calling on consecutive token chunks with the same state buffer.
 *   out     [B, T, H, d_v] fp32
 *   y_raw   [B, T, H, d_v] fp32 or NULL: the read vector before normalisation
 *   ws      >= sdm_workspace_bytes(dims, SDM_ENTRY_SCAN) bytes
 */
SDM_API int32_t sdm_scan(const sdm_dims* dims, const sdm_sel* in, const float* norm_w, void* state,
                 float* out, float* y_raw, void* ws, size_t ws_bytes, void* stream);

/*
 * Whole forward path: sdm_select followed by sdm_scan, with the pass-(a) products
 * kept in the workspace (or in `debug` when given, which must then hold every field;
 * `debug->scores` may be NULL).  Arguments as in those two calls.
 *   ws >= sdm_workspace_bytes(dims, SDM_ENTRY_FORWARD) bytes
 */
SDM_API int32_t sdm_forward(const sdm_dims* dims, const void* x, const void* w_proj, const float* A,
                    const float* b_dt, const float* norm_w, void* state, float* out,
                    const sdm_sel* debug, void* ws, size_t ws_bytes, void* stream);

/*
 * sdm_forward without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops (a decode step), harnesses
 * that forbid allocation.  The workspace is one fixed array of
 * SDM_NOALLOC_SCRATCH_BYTES per GPU, part of the library's device code (each GPU the
 * library runs on holds it until the process ends).  The call allocates nothing and
 * frees nothing.  Arguments and results as in sdm_forward (no `debug` products).
 *  - Sizes whose sdm_workspace_bytes(dims, SDM_ENTRY_FORWARD) exceed
 *    SDM_NOALLOC_SCRATCH_BYTES: SDM_ERR_WORKSPACE, nothing enqueued.  (The decode
 *    workload's step, 256 sequences x 1 token, N = 65536, W = R = 64, d_v = 128,
 *    needs about 6 MiB.)
 *  - SDM_FLAG_TIMING is not accepted here (SDM_ERR_UNSUPPORTED): its record creates
 *    HIP events.
 *  - Every call on one GPU uses that GPU's single array: calls that overlap in time
 *    on one GPU (two streams, two threads) race and give undefined results.  Calls
 *    ordered on one stream are fine; the array's contents between calls do not
 *    matter.
 *  - The first call on each device looks up the array's device address
 *    (hipGetSymbolAddress, with that device current); make that first call outside
 *    graph capture.  SDM_ERR_HIP if the lookup fails.
 */
#define SDM_NOALLOC_SCRATCH_BYTES 67108864 /* 64 MiB */
SDM_API int32_t sdm_forward_noalloc(const sdm_dims* dims, const void* x, const void* w_proj,
                                    const float* A, const float* b_dt, const float* norm_w,
                                    void* state, float* out, void* stream);

/*
 * Training (the m.163.com article on arXiv 2607.07386, section 八, memory-efficiency
 * paragraph: the sparse update is applied in place and undone in backward, keeping
 * the N x d state plus the T x W x d rows the writes overwrote).
 *
 * sdm_scan_train: sdm_scan that also records the write log.
 *   log     OUT: log[b][t][h][k] = the state row idx_w[..][k] just before token t's
 *           write: [B, T, H, W, d_v] fp32, or uint8 codes ([.., d_v] with
 *           SDM_FLAG_LOG_FP8, [.., d_v / 2] with SDM_FLAG_LOG_INT4)
 *   log_scale [B, T, H, W] fp32 OUT: each logged row's absmax (quantised formats;
 *           may be NULL for fp32)
 *   y_raw   required here (the backward needs it)
 *   ws      >= sdm_workspace_bytes(dims, SDM_ENTRY_SCAN_TRAIN) bytes (may be NULL
 *           if 0)
 *   Schedules: a schedule flag picks one (SDM_FLAG_SCAN_DIRECT, _STREAM, _TWO_PHASE
 *   or _CHUNK, the last with an fp32 log only); without one, the per-slot rule takes
 *   the two-phase schedule from 256 tokens and the direct one below that or from 512
 *   walks (B H).  On the
 *   slot-owner (stream, two-phase) schedules, and for the key-weighted rule on the
 *   direct one, a quantised log is staged in fp32 in the workspace (token chunks
 *   bounded near 2 GiB, and 256 MiB) and encoded after each chunk's walk.  State,
 *   y_raw and out equal sdm_scan's on the same schedule (bit for bit on the direct
 *   and chunk schedules, up to fp32 summation order on the slot-owner ones).  The
 *   log and its scales equal those of every per-slot schedule but the chunk one bit
 *   for bit; the chunk schedule's rows (each a fold of the chunk's earlier writes)
 *   and the key-weighted rule's equal the others up to fp32 rounding order.  fp32
 *   state only (SDM_FLAG_STATE_BF16 and SDM_FLAG_STATE_FP8 give
 *   SDM_ERR_UNSUPPORTED).  The key-weighted rule (SDM_FLAG_DELTA_GDN) takes the
 *   schedule sdm_scan would (the chunk one from 64 tokens while B H d_v / 16 <=
 *   1024) with an fp32 log, else the direct one; with SDM_FLAG_SCAN_STREAM or
 *   _TWO_PHASE it is SDM_ERR_UNSUPPORTED.
 *
 * sdm_scan_backward: gradients of that call, walking the tokens in reverse (per
 * token: the norm and gate, the read, then the write, whose overwritten rows are
 * restored from the log).
 *   state   [B, H, N, d_v] IN: the state sdm_scan_train returned; OUT: the state it
 *           started from, bit for bit (with a quantised log: the decoded rows)
 *   d_state [B, H, N, d_v] IN: gradient of the final state (zeros if the loss does
 *           not see it); OUT: gradient of the initial state
 *   y_raw, log, log_scale   as sdm_scan_train wrote them (same flags); d_out
 *           [B, T, H, d_v] gradient of out
 *   grads   outputs, overwritten: d_wt_w [B,T,H,W], d_wt_r [B,T,H,R], d_v and d_gate
 *           [B,T,H,d_v], d_alpha and d_beta [B,T,H]; d_norm_w [H, d_v] (summed over
 *           the batch) or NULL
 *   ws      >= sdm_workspace_bytes(dims, SDM_ENTRY_SCAN_BACKWARD) bytes
 * Schedules: the slot-owner walk from 256 tokens while B H < 512 (or with
 * SDM_FLAG_SCAN_STREAM or SDM_FLAG_SCAN_TWO_PHASE, which both select it): slot-owner
 * lane groups walk the accesses of each slot in reverse, any log format;
 * else (or with SDM_FLAG_SCAN_DIRECT) one workgroup per (b, h), tokens in
 * lock-step; SDM_FLAG_SCAN_CHUNK picks by length as no flag does.  The log of any
 * forward schedule serves any backward one.  The key-weighted rule
 * (SDM_FLAG_DELTA_GDN) undoes its write per token with m the logged rows,
 * m~ = alpha m, e = v - sum k m~, G = dL/dM rows: d_v = beta sum k G = de,
 * dm~ = G - k de, d_k = beta <G, e> - <de, m~>, d_beta = sum k <G, e>,
 * d_alpha = sum <dm~, m>, dL/dm = alpha dm~ (the dot products over d_v summed from
 * per-slice shares in slice order).  With SDM_FLAG_SCAN_CHUNK, or from 256 tokens
 * while B H d_v / 16 <= 256 (one workgroup per CU; beyond that the sliced walk is
 * faster), with an fp32 log and W, R <= 64, it walks chunks of 32 tokens in reverse (the m.163.com
 * article on arXiv 2607.07386, section 八): per chunk de solves the transposed
 * triangular system of the forward's chunk form, de = Tm^T h with
 * h_u = sum_{t >= u} A_{t,u} dy_t + sum_j k_{u,j} G_j(u, end] dL/dM_end[j], and then each
 * slot the chunk touches is walked back on its own (needs ascending ids, as the
 * chunk forward).  Otherwise (or with SDM_FLAG_SCAN_DIRECT) one workgroup per
 * (b, h, column slice) walks the tokens in reverse.
 * Every sum runs in a fixed order, so results are bit-reproducible, except d_v on
 * the stream schedule (summed with float atomics: reproducible up to fp32 summation
 * order).  Other flags as for sdm_scan_train.
 */
typedef struct sdm_scan_grads {
  float* d_wt_w;
  float* d_wt_r;
  float* d_v;
  float* d_gate;
  float* d_alpha;
  float* d_beta;
  float* d_norm_w;  /* nullable */
} sdm_scan_grads;

SDM_API int32_t sdm_scan_train(const sdm_dims* dims, const sdm_sel* in, const float* norm_w,
                               float* state, float* out, float* y_raw, void* log,
                               float* log_scale, void* ws, size_t ws_bytes, void* stream);
SDM_API int32_t sdm_scan_backward(const sdm_dims* dims, const sdm_sel* in, const float* norm_w,
                                  float* state, float* d_state, const float* y_raw,
                                  const void* log, const float* log_scale, const float* d_out,
                                  const sdm_scan_grads* grads, void* ws, size_t ws_bytes,
                                  void* stream);

/*
 * Backward of the selection pass (training): [rainbus] steps 1, 2 and 4 differentiated
 * down to the projection output Y = x W_proj^T.  The selected slot sets are piecewise
 * constant in the scores, so the gradient reaches the half-scores only through the
 * softmax weights of the selected slots ([analysis] "步骤 2": k^(i), q^(i) are the
 * normalised scores of the selected slots).  Per (token, head):
 *   ds_k = w_k (dw_k - sum_l w_l dw_l) for the selected slots k (id i_k n + j_k);
 *   dY[half 1, i] = sum_{k: i_k = i} ds_k, dY[half 2, j] = sum_{k: j_k = j} ds_k (per role);
 *   dY[v] = d_v;  dY[gate] = d_gate g (1 - g) (sigmoid), d_gate s (1 + p (1 - s)) with
 *   s = sigmoid(p) (SiLU, p the gate's pre-activation), or d_gate (no activation);
 *   dY[a] = d_alpha (-A alpha sigmoid(a + b_dt));  dY[b] = d_beta beta (1 - beta);
 *   d_A = sum over tokens of d_alpha (-softplus(a + b_dt) alpha);  d_b_dt = sum of dY[a].
 * The forget pre-gate a (and with SiLU the gate's pre-activations) is recomputed from
 * x and W_proj in fp32.  The remaining
 * gradients are plain GEMMs of dY for the caller: dx = dY W_proj, dW_proj = dY^T x.
 *   fwd      the forward's products: idx_w, wt_w, idx_r, wt_r, alpha, beta, gate
 *            (v and scores unused)
 *   x, w_proj, A, b_dt   as given to sdm_select
 *   g        incoming gradients [B, T, H, ...]: d_wt_w [.., W], d_wt_r [.., R], d_v and
 *            d_gate [.., d_v] (d_gate of the activated gate), d_alpha, d_beta [..]
 *            (as sdm_scan_backward returns them)
 *   d_y      [B*T, H*P] fp32 OUT, overwritten: per head the P columns in W_proj's row
 *            order (write half 1 | write half 2 | read half 1 | read half 2 | v | gate |
 *            a | b)
 *   d_A, d_b_dt  [H] fp32 OUT, overwritten (summed over every token of the call)
 *   ws       >= sdm_workspace_bytes(dims, SDM_ENTRY_SELECT_BACKWARD) bytes
 * Ids must lie in [0, N) (as sdm_select returns them).
 * Deterministic: sums over repeated half indices run in slot order, the other
 * reductions in fixed trees; results are reproducible bit for bit.
 */
typedef struct sdm_select_grads {
  const float* d_wt_w;
  const float* d_wt_r;
  const float* d_v;
  const float* d_gate;
  const float* d_alpha;
  const float* d_beta;
} sdm_select_grads;

SDM_API int32_t sdm_select_backward(const sdm_dims* dims, const sdm_sel* fwd, const void* x,
                                    const void* w_proj, const float* A, const float* b_dt,
                                    const sdm_select_grads* g, float* d_y, float* d_A,
                                    float* d_b_dt, void* ws, size_t ws_bytes, void* stream);

/*
 * Shared learned initial state, copied into a sequence's store on first touch.  M0 is
 * one parameter of the layer, the same for every sequence ([analysis] section on the
 * learned M0; m.163.com article on arXiv 2607.07386, section 三), so a batch need not
 * carry B copies of it: the store holds only the rows each sequence has touched.
 * The effective state of (b, h) slot i is state[b][h][i] if bit i of touched[b][h] is
 * set, else m0[h][i].  Results equal sdm_scan / sdm_forward run on the effective state
 * (bit for bit: the same kernels run on the same values).
 *   m0       [H, N, d_v] fp32 (bf16 with SDM_FLAG_STATE_BF16), read only
 *   state    [B, H, N, d_v] same type, IN/OUT: only rows whose bit is set are read; the
 *            call writes rows it touches and no others
 *   touched  [B, H, ceil(N/32)] uint32 bitmaps (bit i of word i/32), IN/OUT: the call
 *            sets the bit of every slot it reads or writes.  All zero starts every
 *            sequence from M0 without initialising `state`.
 * Other arguments as in sdm_scan / sdm_forward (same workspace sizes).  Ids must lie
 * in [0, N) (as sdm_select returns them).
 */
SDM_API int32_t sdm_scan_shared_m0(const sdm_dims* dims, const sdm_sel* in, const float* norm_w,
                                   const void* m0, void* state, uint32_t* touched, float* out,
                                   float* y_raw, void* ws, size_t ws_bytes, void* stream);
SDM_API int32_t sdm_forward_shared_m0(const sdm_dims* dims, const void* x, const void* w_proj,
                                      const float* A, const float* b_dt, const float* norm_w,
                                      const void* m0, void* state, uint32_t* touched, float* out,
                                      void* ws, size_t ws_bytes, void* stream);

/*
 * Slot-update histogram (monitoring; not a step of the layer): the papers.ananclaw.com
 * summary (engineering-risks section, risk 3) watches how often each slot is updated
 * to catch writes collapsing onto a few slots.
 *   idx_w   [B, T, H, W] int32 write ids, as sdm_select returns them
 *   counts  [H, N] int32, IN/OUT: counts[h][i] += the number of (b, t) whose write set
 *           of head h holds slot i.  It accumulates over calls (clear it to start
 *           over); a count wraps past 2^31 - 1.  Ids outside [0, N) are not counted.
 * Exact: integer adds, independent of their order.
 */
SDM_API int32_t sdm_slot_histogram(const sdm_dims* dims, const int32_t* idx_w, int32_t* counts,
                                   void* stream);

/*
 * Kernel durations recorded by calls made with SDM_FLAG_TIMING (instrumentation;
 * not a step of the method).  Fills out[0..k) with the oldest k records (k <= max),
 * waiting for each to complete, removes them from the record and returns k; 0 when
 * nothing is recorded.  `name` points to a static string naming the kernel.  The
 * record is process-wide and holds at most 65536 launches (older ones are dropped).
 * Returns SDM_ERR_NULL if out is NULL with max > 0, SDM_ERR_HIP if an event query
 * fails.
 */
typedef struct sdm_kernel_time {
  const char* name;
  float ms;
} sdm_kernel_time;
SDM_API int32_t sdm_timing_read(sdm_kernel_time* out, int32_t max);

#ifdef __cplusplus
}
#endif

#endif /* SDM_H */
