/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE expert layer.
 *
 * The layer (UniEP article, "UniEP: Unified Expert-Parallel MoE MegaKernel for
 * LLM Training", section 1.1 and Figure 1) is: a gate scores every expert for
 * every token, top-k picks the experts, the tokens are dispatched into
 * expert-contiguous rows, each expert runs a SwiGLU FFN (grouped GEMM, SiLU
 * gate product, second grouped GEMM back to the model dim), and the results
 * are weighted by the gate scores and summed (combine).  The backward mirrors
 * it; weight gradients are a transposed grouped GEMM over each expert's rows.
 * The SwiGLU form and its backward split (input-gradient part "B",
 * weight-gradient part "W") follow the GraphPP article, sections 2 and 5.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer, allocated and owned by the
 *    caller.  The library never allocates, frees, copies to the host or
 *    synchronises the host inside a call; every call is asynchronous on
 *    `stream` (a hipStream_t passed as void*; NULL = the null stream).
 *  - Row-major, contiguous, 16-byte aligned.  `dtype` (moe_dims.dtype) is
 *    the storage type of x, weights, activations and activation gradients
 *    (MOE_F32 or MOE_BF16, bf16 = upper 16 bits of an IEEE float32).
 *    Router logits, gate weights, their gradients and weight gradients are
 *    always float32.  Indices and counts are int32.
 *  - Shapes: T tokens, H model dim, E routed experts, K experts per token,
 *    I expert intermediate dim, Ns = n_shared shared experts of intermediate
 *    dim I_shared (the kernels support I_shared == I; other values are
 *    rejected with MOE_EUNSUPPORTED; ignored when Ns = 0).
 *    R = T*K routed rows.  "All rows" RA = R + Ns*T: rows [0, R) are the
 *    routed rows in slot order, rows [R + s*T, R + (s+1)*T) are shared
 *    expert s applied to tokens 0..T-1.
 *  - Weights: W1, W3 [E, H, I] (gate and up projection, y = x @ W), W2
 *    [E, I, H] (down projection); shared weights Ws1, Ws3 [Ns, H, I],
 *    Ws2 [Ns, I, H].  This orientation is the one in which the weight
 *    gradient of the down projection is h^T @ dy (GraphPP, section 5.1).
 *  - Results are deterministic: the same inputs give the same output bits
 *    on every run, whatever the stream, the launch shape or the order in
 *    which the GPU happens to run the work.  No floating-point atomics are
 *    used anywhere.  Inputs must be finite.
 *  - Every call returns a moe_status.  On error nothing has been launched
 *    and moe_last_error() gives a message (thread-local).
 *  - Validation (else MOE_EINVAL / MOE_EUNSUPPORTED): T >= 1,
 *    1 <= K <= E <= 256, H and I positive multiples of 8, 0 <= Ns <= 8,
 *    I_shared == I when Ns > 0, R + Ns*T < 2^31; non-null, 16-byte aligned
 *    pointers for every buffer the call uses.  Element offsets are computed
 *    in 64 bits, so buffers larger than 2^31 elements are fine.
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
  MOE_EINVAL = 1,       /* bad argument (null pointer, bad shape)            */
  MOE_EUNSUPPORTED = 2, /* shape/dtype outside what the kernels support       */
  MOE_EWORKSPACE = 3,   /* workspace missing or smaller than moe_workspace_bytes */
  MOE_EHIP = 4,         /* a HIP runtime call failed (see moe_last_error)     */
  MOE_ETIMEOUT = 5      /* a bounded wait inside a kernel gave up (moe_sync_status) */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef struct {
  int32_t T;        /* tokens                                */
  int32_t H;        /* model (hidden) dim                    */
  int32_t E;        /* routed experts                        */
  int32_t K;        /* experts per token (top-k)             */
  int32_t I;        /* expert FFN intermediate dim           */
  int32_t n_shared; /* shared experts (weight 1, all tokens) */
  int32_t I_shared; /* shared experts' intermediate dim      */
  int32_t dtype;    /* moe_dtype                             */
} moe_dims;

/* Caches device properties (CU count) for `device` and reads the debug
 * settings listed under moe_sync_status from the environment.  No other call
 * reads the environment: without moe_init the debug settings keep their
 * defaults (waits bounded at 20 s, normal schedule, one persistent worker per
 * CU), and every call initialises the device properties lazily.  May be
 * called again (e.g. after changing a debug setting); the settings are global
 * to the process.  Returns MOE_EINVAL for a device index outside [0, 64). */
int moe_init(int device);

/* Human-readable name of a status code; never NULL. */
const char* moe_status_str(int status);

/* Detail of the last error returned on this thread ("" if none). */
const char* moe_last_error(void);

/* Synchronises `stream` (the host waits for its work) and reports what the
 * kernels recorded while running.  The persistent kernels' waits (combine
 * tasks on their row tiles, split-tail owners on their helpers, the
 * one-launch backward on its first phase) always end by construction; each
 * is also bounded in time (20 s, or MOE_WAIT_LIMIT_US microseconds from the
 * environment as moe_init read it), and one that gives up records it on the
 * device and lets the kernel run to its end with invalid results.  Callers
 * that need valid results check this after their work (a timed-out step must
 * not be reported as a result).
 * Returns MOE_ETIMEOUT if any wait gave up since the last call (then clears
 * the record), MOE_EHIP if the stream reports a HIP error, MOE_OK otherwise.
 * The record is kept per device (the current one), not per stream: a wait
 * that gave up in work on another stream of the device is reported too.
 * Debug settings, read by moe_init only:
 *  MOE_DEBUG_UNREACHABLE_WAITS=1 makes every such wait target one more than
 *    can happen, to exercise this path;
 *  MOE_DEBUG_PERTURB_SEED=n (n > 0) makes the persistent GEMM launches claim
 *    their whole tiles in a seeded order and sleep a seeded time before every
 *    claim; results are bit-identical to the normal schedule (slower; for
 *    determinism tests);
 *  MOE_FUSED_WORKERS=n (n > 0) launches n persistent workers in the fused
 *    calls instead of one per CU (results do not depend on it). */
int moe_sync_status(void* stream);

/* Schedule knobs of the grouped GEMMs and fused kernels (the auto-tuning
 * space; UniEP article, section 3 of its table of contents: optimisation
 * space, analytical performance model).  None of them changes the arithmetic
 * of any output element -- only which tiles run together and how the fused
 * kernels cut their row tasks -- so every choice gives the same output bits.
 * The down projection and the input gradient, whose tail tiles are split
 * along k, keep fixed bands. */
typedef struct {
  int32_t band_up;         /* row tiles per band of a large group: gate/up projection */
  int32_t band_act;        /* the same for the activation gradient                    */
  int32_t small_group;     /* a group of at most this many row tiles is one band      */
  int32_t band_wgrad_up;   /* H blocks per band of the dW1/dW3 GEMM                   */
  int32_t band_wgrad_down; /* I blocks per band of the dW2 GEMM                       */
  int32_t combine_tokens;  /* tokens per combine task of moe_ffn_combine              */
  int32_t copy_tokens;     /* tokens per x_perm copy task of moe_dispatch_ffn          */
  int32_t copy_in_tiles;   /* 1: moe_dispatch_ffn writes x_perm from the gathered rows its
                              GEMM tiles hold in LDS (no copy tasks), 0: copy tasks      */
} moe_tuning;

/* The knobs every call with these dims uses: the library's choice for the
 * shape (an analytical model of the operand traffic beyond L2 for the band
 * heights; a cache-footprint rule for copy_in_tiles; measured defaults for
 * the others), with any override from the
 * MOE_TUNE environment variable as moe_init read it ("key=value,..." with the
 * field names above; band heights 1..64, task sizes 1..1024, copy_in_tiles
 * 0..1; moe_init returns MOE_EINVAL for anything else).  Errors: MOE_EINVAL
 * (NULL), bad dims. */
int moe_get_tuning(const moe_dims* d, moe_tuning* out);

/* The band model's prediction behind moe_get_tuning: operand bytes fetched
 * from beyond L2 per flop of the GEMM that `knob` schedules ("band_up": the
 * gate/up projection, "band_act": the activation gradient, "small_group":
 * both, summed) with the knob at `value` and the others as chosen.  Returns
 * a negative value for other knobs (the model does not cover them), for bad
 * dims or a value outside 1..64. */
double moe_tuning_predict(const moe_dims* d, const char* knob, int value);

/* Bytes of device workspace the calls that take `ws` need for these dims
 * (route scratch, tile tables, readiness flags, task cursors).  The same
 * workspace may be reused by consecutive calls on one stream; calls that
 * overlap in time need separate workspaces. */
size_t moe_workspace_bytes(const moe_dims* d);

/* ------------------------------------------------------------------ forward */

/* Route (UniEP section 1.1 gate + top-k; section 2.2 Algorithm 1, one rank).
 *  logits   [T, E] f32 in
 *  topk_idx [T, K] i32 out: K distinct experts per token by descending logit;
 *           equal logits go to the lower expert id; -0.0 equals +0.0.
 *  topk_w   [T, K] f32 out: softmax over the K selected logits (sums to 1).
 *  counts   [E]    i32 out: rows per expert (histogram of topk_idx).
 *  offsets  [E+1]  i32 out: exclusive prefix sum of counts; offsets[E] = R.
 *  slot     [T, K] i32 out: row of (t, k) in the expert-contiguous layout =
 *           offsets[e] + number of earlier (t', k') pairs, in t-major k-minor
 *           order, routed to the same expert (a stable sort by expert).
 *  slot_src [R]    i32 out: the token whose row lands in each slot.
 * No atomics decide any slot; the map is a pure function of topk_idx. */
int moe_route(const moe_dims* d, const float* logits, int32_t* topk_idx, float* topk_w,
              int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* slot_src,
              void* ws, size_t ws_bytes, void* stream);

/* moe_route for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same outputs, bit for bit, with the routing scratch taken from a fixed
 * 1 MiB device array of the library instead of a caller workspace.  The
 * array exists once per device and lives until the process ends; moe_init
 * looks up its address (else the first call on the device does).  Limit:
 * ceil(T / 64) * E <= 131072 (e.g. T = 131072 tokens with E <= 64), else
 * MOE_EUNSUPPORTED before anything is launched.  Calls that overlap in time on
 * one device share the array and race: order them on one stream.  Allocates
 * nothing, frees nothing, does not synchronise.  Arguments and errors as for
 * moe_route otherwise. */
int moe_route_noalloc(const moe_dims* d, const float* logits, int32_t* topk_idx, float* topk_w,
                      int32_t* counts, int32_t* offsets, int32_t* slot, int32_t* slot_src,
                      void* stream);

/* Algorithm 1 with G explicit ranks (UniEP section 2.2, "deterministic token
 * mapping"): rank r holds the contiguous tokens [floor(T r / G),
 * floor(T (r+1) / G)), 1 <= G <= T.  Every rank counts its own (token, k)
 * pairs per expert; the counts form a [G, E] table (what an all-gather of the
 * per-rank histograms gives every rank); the base offset of rank r in expert
 * e is the expert's start plus the counts of lower ranks; a pair's slot is
 * its rank's base plus its stable position among its rank's pairs of that
 * expert.  This is the multi-rank form of the map moe_route builds, and the
 * slots are identical to it for every G.
 *  topk_idx    [T, K] i32 in (as moe_route writes it; ids outside [0, E) are
 *              skipped: they get no slot and are not counted)
 *  rank_counts [G, E] i32 out: pairs of rank r routed to expert e
 *  rank_base   [G, E] i32 out: first slot of rank r's pairs in expert e
 *  counts [E], offsets [E+1], slot [T, K], slot_src [R] i32 out: as moe_route
 *  ws: device workspace of at least moe_route_ranks_workspace_bytes(d, G)
 *      bytes (it depends on G; moe_workspace_bytes does not cover it)
 * Errors: MOE_EINVAL for G outside [1, T] or a NULL array; MOE_EWORKSPACE. */
size_t moe_route_ranks_workspace_bytes(const moe_dims* d, int G);
int moe_route_ranks(const moe_dims* d, const int32_t* topk_idx, int G, int32_t* rank_counts,
                    int32_t* rank_base, int32_t* counts, int32_t* offsets, int32_t* slot,
                    int32_t* slot_src, void* ws, size_t ws_bytes, void* stream);

/* Dispatch (UniEP 1.1 "scatter"; padding-free layout of section 1.2):
 *  x_perm[slot[t,k]] = x[t];  x [T, H] in, x_perm [R, H] out (bit copy). */
int moe_dispatch(const moe_dims* d, const void* x, const int32_t* slot, void* x_perm, void* stream);

/* Expert FFN, first half (grouped GEMM + SwiGLU; GraphPP 5.1 forward):
 * for every routed row r of expert e (rows offsets[e]..offsets[e+1]) and
 * every shared row:  a = x_r W1_e, b = x_r W3_e, h = silu(a) * b
 * (float32 accumulation; h formed from the unrounded a and b).
 *  x_perm [R, H], x [T, H] (shared rows read x directly; may be NULL if Ns=0)
 *  ab [RA, 2I] out: a in columns [0, I), b in [I, 2I) (saved for backward)
 *  h  [RA, I]  out. */
int moe_expert_ffn_up(const moe_dims* d, const void* x_perm, const void* x, const int32_t* offsets,
                      const void* w1, const void* w3, const void* ws1, const void* ws3, void* ab,
                      void* h, void* ws, size_t ws_bytes, void* stream);

/* Expert FFN, second half (second grouped GEMM): y_r = h_r W2_e.
 *  h [RA, I] in, y [RA, H] out (routed rows then shared rows). */
int moe_expert_ffn_down(const moe_dims* d, const void* h, const int32_t* offsets, const void* w2,
                        const void* ws2, void* y, void* ws, size_t ws_bytes, void* stream);

/* Both halves in order (up then down). */
int moe_expert_ffn(const moe_dims* d, const void* x_perm, const void* x, const int32_t* offsets,
                   const void* w1, const void* w3, const void* w2, const void* ws1,
                   const void* ws3, const void* ws2, void* ab, void* h, void* y, void* ws,
                   size_t ws_bytes, void* stream);

/* Combine (UniEP 1.1): out[t] = sum_{k=0..K-1} w[t,k] y[slot[t,k]]
 *                               + sum_{s=0..Ns-1} y[R + s*T + t],
 * float32 accumulation in exactly that order, one rounding to dtype.
 *  y [RA, H] in, out [T, H] out. */
int moe_combine(const moe_dims* d, const void* y, const int32_t* slot, const float* topk_w,
                void* out, void* stream);

/* Fused Dispatch+GroupGEMM (UniEP section 2.1/2.2 MegaKernel): one persistent
 * launch whose workers claim tasks from atomic cursors.  The GEMM tiles of
 * moe_expert_ffn_up come first; each reads its routed rows straight from the
 * token rows x through slot_src as it loads its A operand, so no tile waits
 * for a gather.  Then copy tasks write the expert-contiguous rows x_perm
 * (which the backward reads) token by token: each token row of x is read once
 * and written to its K rows slot[t, 0..K-1].  slot_src [R] and slot [T, K]
 * are moe_route's outputs for the same routing.
 * Outputs (x_perm, ab, h) are bit-identical to moe_dispatch followed by
 * moe_expert_ffn_up.  f32, bf16 with T*H*2 bytes above 2^31 - 64 KiB (the
 * kernel's per-lane byte offsets into x are 32-bit), or K > 64 (its copy tasks
 * hold at most 64 pairs per token): a plain gather, then moe_expert_ffn_up,
 * with the same results. */
int moe_dispatch_ffn(const moe_dims* d, const void* x, const int32_t* slot_src,
                     const int32_t* slot, const int32_t* offsets, const void* w1, const void* w3,
                     const void* ws1, const void* ws3, void* x_perm, void* ab, void* h, void* ws,
                     size_t ws_bytes, void* stream);

/* Fused GroupGEMM+Combine (UniEP section 2.1 second MegaKernel): the GEMM
 * tiles of moe_expert_ffn_down, then combine tasks that wait on per-row-tile
 * completion counters.  y and out are bit-identical to moe_expert_ffn_down
 * followed by moe_combine.  f32 or K > 64: those two plain launches. */
int moe_ffn_combine(const moe_dims* d, const void* h, const int32_t* offsets, const void* w2,
                    const void* ws2, const int32_t* slot, const float* topk_w, void* y, void* out,
                    void* ws, size_t ws_bytes, void* stream);

/* ----------------------------------------------------------------- backward */

/* Combine backward: dy[slot[t,k]] = w[t,k] dout[t] (rounded to dtype);
 * dtopk_w[t,k] = <dout[t], y[slot[t,k]]> (float32, fixed reduction order).
 *  dout [T, H], y [RA, H] in; dy [R, H], dtopk_w [T, K] out. */
int moe_combine_bwd(const moe_dims* d, const void* dout, const void* y, const int32_t* slot,
                    const float* topk_w, void* dy, float* dtopk_w, void* stream);

/* Expert FFN input-gradient part ("B", GraphPP section 2 / 5.1):
 *  dh = dy_r W2_e^T;  da = dh b sig(a) (1 + a (1 - sig(a)));  db = dh silu(a)
 *  (a, b = the saved values in ab);  dx_r = da W1_e^T + db W3_e^T (one sum).
 * A shared expert's output gradient is dout itself (weight 1).
 *  dy [R, H], dout [T, H] (NULL ok if Ns=0), ab [RA, 2I] in;
 *  dab [RA, 2I] out (da then db), dx_rows [RA, H] out. */
int moe_expert_ffn_bwd_data(const moe_dims* d, const void* dy, const void* dout,
                            const int32_t* offsets, const void* w1, const void* w3,
                            const void* w2, const void* ws1, const void* ws3, const void* ws2,
                            const void* ab, void* dab, void* dx_rows, void* ws, size_t ws_bytes,
                            void* stream);

/* The two GEMMs of moe_expert_ffn_bwd_data, callable on their own:
 *  _act:   dh = dy_r W2_e^T, then da/db from the saved a, b -> dab [RA, 2I]
 *          (reads dy [R,H], dout [T,H] for shared rows, ab [RA,2I]);
 *  _input: dx_r = da W1_e^T + db W3_e^T -> dx_rows [RA, H] (reads dab). */
int moe_expert_ffn_bwd_act(const moe_dims* d, const void* dy, const void* dout,
                           const int32_t* offsets, const void* w2, const void* ws2,
                           const void* ab, void* dab, void* ws, size_t ws_bytes, void* stream);
int moe_expert_ffn_bwd_input(const moe_dims* d, const void* dab, const int32_t* offsets,
                             const void* w1, const void* w3, const void* ws1, const void* ws3,
                             void* dx_rows, void* ws, size_t ws_bytes, void* stream);

/* Expert FFN weight-gradient part ("W"): transposed grouped GEMM summing over
 * each expert's rows in slot order (UniEP 1.1), one owner per output tile:
 *  dW1_e = X_e^T dA_e, dW3_e = X_e^T dB_e, dW2_e = H_e^T dY_e  (float32 out;
 *  an expert with no rows gets exact zeros).  Shared experts use X = x,
 *  dY = dout.  x_perm [R,H], x [T,H], h [RA,I], dy [R,H], dout [T,H],
 *  dab [RA,2I] in; dw1, dw3 [E,H,I], dw2 [E,I,H], dws1, dws3 [Ns,H,I],
 *  dws2 [Ns,I,H] out (the shared ones may be NULL if Ns = 0). */
int moe_expert_ffn_bwd_weight(const moe_dims* d, const void* x_perm, const void* x,
                              const void* h, const void* dy, const void* dout, const void* dab,
                              const int32_t* offsets, float* dw1, float* dw3, float* dw2,
                              float* dws1, float* dws3, float* dws2, void* ws, size_t ws_bytes,
                              void* stream);

/* The two GEMMs of moe_expert_ffn_bwd_weight, callable on their own:
 *  _gate_up: dW1_e = X_e^T dA_e and dW3_e = X_e^T dB_e (one pass over X);
 *  _down:    dW2_e = H_e^T dY_e. */
int moe_expert_ffn_bwd_weight_gate_up(const moe_dims* d, const void* x_perm, const void* x,
                                      const void* dab, const int32_t* offsets, float* dw1,
                                      float* dw3, float* dws1, float* dws3, void* ws,
                                      size_t ws_bytes, void* stream);
int moe_expert_ffn_bwd_weight_down(const moe_dims* d, const void* h, const void* dy,
                                   const void* dout, const int32_t* offsets, float* dw2,
                                   float* dws2, void* ws, size_t ws_bytes, void* stream);

/* The whole expert-FFN backward, B and W, in one persistent launch, with the
 * weight-gradient GEMMs scheduled into the gaps of the input-gradient chain
 * (zero-bubble "B/W" split, GraphPP section 2 / 5.1: W needs only operands
 * that already exist, so it fills bubbles).  Phases of tiles, each one
 * filling the tail of the one before: dh -> dab (B), dW2 (W), dx_rows from dab
 * (B), dW1/dW3 from dab (W).  Outputs are bit-identical to
 * moe_expert_ffn_bwd_data followed by moe_expert_ffn_bwd_weight, for any
 * number of workers.  Arguments: the union of those two calls (same layouts
 * and ownership); dab is written and read back inside the call.  f32 runs the
 * two plain calls.  Errors as for the two calls. */
int moe_expert_ffn_bwd(const moe_dims* d, const void* dy, const void* dout,
                       const int32_t* offsets, const void* w1, const void* w3, const void* w2,
                       const void* ws1, const void* ws3, const void* ws2, const void* ab,
                       const void* x_perm, const void* x, const void* h, void* dab,
                       void* dx_rows, float* dw1, float* dw3, float* dw2, float* dws1,
                       float* dws3, float* dws2, void* ws, size_t ws_bytes, void* stream);

/* Dispatch backward: dx[t] = sum_k dx_rows[slot[t,k]] + sum_s dx_rows[R+s*T+t]
 * (float32 accumulation in that order, one rounding).
 *  dx_rows [RA, H] in, dx [T, H] out. */
int moe_dispatch_bwd(const moe_dims* d, const void* dx_rows, const int32_t* slot, void* dx,
                     void* stream);

/* Route backward (softmax over the selected logits):
 *  dlogits[t, e_k] = w_k (dw_k - sum_j w_j dw_j), 0 for unselected experts.
 *  dtopk_w, topk_w [T,K] f32, topk_idx [T,K] in; dlogits [T,E] f32 out. */
int moe_route_bwd(const moe_dims* d, const float* dtopk_w, const float* topk_w,
                  const int32_t* topk_idx, float* dlogits, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
