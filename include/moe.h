/*
 * moe.h -- C ABI of the pooled-wave capacity-dispatch MoE branch (forward),
 * for AMD Instinct MI355X (gfx950).
 *
 * The branch, as the pages describe it (lamjinlab.com, "Marin начинает
 * открытое обучение MoE-модели с 535 млрд параметров", section 2, "how the
 * sparse model is organised"; ranhao.site, "Marin 535B-A23B ...", sections 2.2
 * and 3.2):
 *
 *   z      = x W_lat^T                      latent compression d_model -> d_latent
 *   logits = z W_r^T                        router scores (fp32)
 *   top-k  by fl32(logit + bias), ties -> lower expert index
 *   gates  = softmax of the k selected raw logits (bias excluded)
 *   dispatch into one fixed pool per destination (a group of E/P experts),
 *            per wave of ceil(T/W) tokens, the expert id packed with the row;
 *            sender cap ceil(1.10 * expected rows per pool), receiver cap
 *            ceil(1.15 * expected rows per expert); overflow dropped, counted
 *   experts  o = (silu(u W_g^T) * (u W_u^T)) W_d^T per receiver-kept row
 *   combine  y_lat[t] = sum_j g[t,j] * o[t,j] over kept rows (no renormalising)
 *   y      = y_lat W_up^T + sum_s SwiGLU_s(x)   up-projection + shared experts
 *
 * On one device the P destinations are virtual: pools are blocks of one
 * buffer and the transport between sender and receiver is the identity.
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are device memory owned by the caller; the
 *     library never allocates, frees, or keeps them.  Pointers marked (host)
 *     are read during the call only.  A buffer whose size in the plan is 0
 *     (the pools, expert outputs and their gradients when the sender
 *     capacity is 0; bank_rows when the receiver capacity is 0) may be NULL.
 *   - Matrices are row-major.  Weights are [out, in] (the torch.nn.Linear
 *     layout): y = x W^T, so every contraction reads both operands along
 *     their contiguous dimension.
 *   - `dtype` selects the element type of activations, weights, pools and
 *     outputs: MOE_F32 (fp32) or MOE_BF16 (bf16, fp32 accumulation).  Router
 *     logits, bias and gates are always fp32; indices int32; counters int64.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously; no call synchronises the host.  Counters stay on the
 *     device.
 *   - Errors: every argument is validated on the host before anything is
 *     enqueued; on error nothing is enqueued and a moe_status != MOE_OK is
 *     returned.  MOE_ERR_HIP reports a launch failure (hipGetLastError).
 *     The library never aborts.  Inputs must be finite (NaN behaviour is
 *     unspecified).
 *   - Results are bitwise reproducible run to run.
 *   - Calls on one stream are ordered; calls that share buffers on different
 *     streams race.
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
  MOE_ERR_INVALID_ARG = 1, /* null pointer, inconsistent or out-of-range size */
  MOE_ERR_UNSUPPORTED = 2, /* valid but not handled (alignment of a width) */
  MOE_ERR_WORKSPACE = 3,   /* workspace too small or misaligned */
  MOE_ERR_HIP = 4          /* a kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Shape of one branch call. */
typedef struct {
  int64_t T;            /* tokens in the call (>= 0, T * top_k < 2^31) */
  int32_t d_model;      /* D: width of x and y                          */
  int32_t d_latent;     /* L: latent width, the width of a pool row     */
  int32_t n_experts;    /* E: routed experts (<= 1024)                  */
  int32_t n_pools;      /* P: destinations; E % P == 0, E/P experts each */
  int32_t top_k;        /* k: assignments per token, 1 <= k <= 64; routing
                           (moe_route, moe_forward) also needs k <= E    */
  int32_t d_ff;         /* F: routed expert intermediate width          */
  int32_t n_shared;     /* S: always-on shared experts (>= 0)           */
  int32_t d_ff_shared;  /* Fs: shared expert intermediate width         */
  int32_t n_waves;      /* W: waves, contiguous token chunks of ceil(T/W) */
  /* capacity factors as exact rationals: sender num/den (1.10 = 11/10),
     receiver num/den (1.15 = 23/20) */
  int32_t send_cap_num, send_cap_den;
  int32_t recv_cap_num, recv_cap_den;
  /* explicit capacities in rows; 0 = derive from the factors */
  int64_t cap_send_rows;
  int64_t cap_recv_rows;
  int32_t dtype;        /* moe_dtype */
  int32_t reserved;     /* must be 0 */
} moe_config;

/* Derived sizes (host-only, pure).  All byte sizes are multiples of 256. */
typedef struct {
  int64_t tokens_per_wave;   /* Tw = ceil(T / W)                                   */
  int64_t cap_send;          /* C_send = ceil(send_factor * Tw * k / P): rows per (wave, pool) */
  int64_t cap_recv;          /* C_recv = ceil(recv_factor * Tw * k / E): rows per (wave, expert) */
  int64_t experts_per_pool;  /* E / P                                              */
  int64_t elem_bytes;        /* 4 (f32) or 2 (bf16)                                */
  int64_t row_bytes;         /* L * elem_bytes: one pool row                       */
  int64_t pool_block_bytes;  /* one (wave, pool) block: C_send rows, then the int32 id column */
  int64_t ids_offset;        /* byte offset of the id column inside a block       */
  int64_t pools_bytes;       /* W * P * pool_block_bytes                           */
  int64_t expert_out_bytes;  /* W * P * C_send * row_bytes ([W][P][C_send][L])     */
  int64_t max_expert_rows;   /* W * C_recv: most rows one expert can receive       */
  int64_t dispatch_ws_bytes; /* workspace of moe_dispatch                          */
  int64_t experts_ws_bytes;  /* workspace of moe_experts                           */
  int64_t forward_ws_bytes;  /* workspace of moe_forward (covers every tap left NULL) */
  /* dropless ragged variant (moe_*_dropless) */
  int64_t dropless_rows;              /* T * k: rows of xs and expert_out               */
  int64_t dropless_dispatch_ws_bytes; /* workspace of moe_dispatch_dropless             */
  int64_t dropless_experts_ws_bytes;  /* workspace of moe_experts_dropless              */
  int64_t dropless_forward_ws_bytes;  /* workspace of moe_forward_dropless (taps NULL)  */
  /* backward of the routed path (moe_*_backward) */
  int64_t backward_rows;              /* padded expert-major rows the backward works in */
  int64_t experts_bwd_ws_bytes;       /* workspace of moe_experts_backward              */
  int64_t backward_ws_bytes;          /* workspace of moe_backward_routed               */
  int64_t dropless_backward_rows;     /* the same for the dropless variant (*_dropless) */
  int64_t dropless_experts_bwd_ws_bytes; /* workspace of moe_experts_backward_dropless  */
  int64_t dropless_backward_ws_bytes; /* workspace of moe_backward_dropless             */
} moe_plan;

/* Weights of one branch (device pointers, element type = dtype unless noted). */
typedef struct {
  const void* w_latent;     /* [L][D]                   */
  const void* w_router;     /* [E][L]                   */
  const float* router_bias; /* [E] fp32 (selection only) */
  const void* w_gate;       /* [E][F][L]                */
  const void* w_up;         /* [E][F][L]                */
  const void* w_down;       /* [E][L][F]                */
  const void* w_up_proj;    /* [D][L]                   */
  const void* ws_gate;      /* [S][Fs][D]               */
  const void* ws_up;        /* [S][Fs][D]               */
  const void* ws_down;      /* [S][D][Fs]               */
} moe_weights;

/* Optional taps of moe_forward (device pointers, each may be NULL).  A
   non-NULL tap is used as the buffer of that intermediate instead of
   workspace, so reading it costs no copy. */
typedef struct {
  float* logits;          /* [T][E] fp32                     */
  int32_t* topk_idx;      /* [T][k]                          */
  float* gates;           /* [T][k]                          */
  int32_t* pool_slot;     /* [T][k], -1 = sender-dropped     */
  int32_t* recv_slot;     /* [T][k], -1 = dropped            */
  int32_t* pool_count;    /* [W][P]                          */
  int32_t* expert_count;  /* [W][E]                          */
  int32_t* bank_rows;     /* [W][E][C_recv]                  */
  void* z;                /* [T][L]                          */
  void* pools;            /* pools_bytes                     */
  void* expert_out;       /* expert_out_bytes                */
  void* y_latent;         /* [T][L]                          */
} moe_taps;

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status s);

/* Library version, major * 10000 + minor * 100 + patch. */
int32_t moe_version(void);

/* Fill *plan from *cfg (host only, no device work).
   Capacities follow the pages' factors (lamjinlab.com section 2: sender
   factor 1.10 bounds the rows one source sends to one destination, receiver
   factor 1.15 bounds the rows of one local expert; ranhao.site section 3.2:
   the receive buffer is the expected rows in that wave times 1.15), rounded
   up, in exact integer arithmetic.
   Errors: MOE_ERR_INVALID_ARG (null pointer, a size out of range, E % P != 0,
   W < 1, a factor with den <= 0 or num < 0), MOE_ERR_UNSUPPORTED
   (d_model, d_latent, d_ff or d_ff_shared not a multiple of 64 or above
   2^20, E > 1024, k > 64, n_shared > 3, n_waves > 65535, an index that would
   not fit in int32, a bf16 operand buffer of 4 GiB or more, a grouped GEMM
   of more than 2^23 - 8 tiles). */
moe_status moe_make_plan(const moe_config* cfg, moe_plan* plan);

/* Router selection (ranhao.site section 2.2: top-8 routing with a balancing
   bias that takes no gradient; lamjinlab.com section 2: 8 of 384 experts).
   logits  (device) [T][E] fp32
   bias    (device) [E] fp32, or NULL for zero bias
   topk_idx (device, out) [T][k] int32: experts by fl32(logit + bias)
           descending, equal scores by lower index (-0 == +0)
   gates   (device, out) [T][k] fp32: softmax over the k selected raw logits
   Only T, n_experts and top_k of *cfg are read (and validated):
   1 <= top_k <= n_experts (MOE_ERR_INVALID_ARG), n_experts <= 1024 and
   top_k <= 64 (MOE_ERR_UNSUPPORTED). */
moe_status moe_route(const moe_config* cfg, const float* logits,
                     const float* bias, int32_t* topk_idx, float* gates,
                     void* stream);

/* Router balancing-bias update (ranhao.site section 2.2: the top-8 router
   is a histogram-based quantile router; its bias is zero-mean, computed for
   the next step, a heuristic that balances expert selection, outside the
   gradient).  The page gives no formula; the rule computed here is:
     1. per expert e, lo_e / hi_e = min / max of its logit over the T tokens;
     2. an n_bins equal-width histogram of the column over [lo_e, hi_e]: the
        bin of v is 0 if v == lo_e, else min(n_bins - 1, trunc(p)) with
        p = fl32(fl32(v - lo_e) * scale_e), scale_e = fl32 of the fp64
        quotient n_bins / (hi_e - lo_e) (0 for a constant column);
     3. Q_e = the quantile of level 1 - k/E read off the histogram by linear
        interpolation inside the first bin j whose cumulative count C_j
        satisfies C_j * E >= (E - k) * T:
          Q_e = lo_e + (j + (r - C_{j-1}) / h_j) * (hi_e - lo_e) / n_bins,
        r = (E - k) * T / E, each operation rounded in fp64;
     4. bias_next[e] = mean(Q) - Q_e, rounded to fp32 (zero-mean).
   Adding bias_next to the next step's logits before top-k moves every
   expert's 1 - k/E quantile onto the common mean, so each expert's logit
   clears a common threshold on about a k/E share of the tokens.
   logits    (device) [T][E] fp32, finite; ranges narrower than about
             n_bins * 2^-126 meet fp32 denormals and are not supported
   n_bins    1 <= n_bins <= 1024
   bias_next (device, out) [E] fp32
   hist      (device, out) [E][n_bins] int32 counts, or NULL
   lohi      (device, out) [E][2] fp32 {lo_e, hi_e}, or NULL
   ws        (device) >= moe_router_bias_ws_bytes(cfg, n_bins) bytes,
             256-byte aligned; nothing in it needs clearing.  Calls that
             share a workspace must not overlap (one stream does that)
   Only T, n_experts and top_k of *cfg are read: T >= 1 and 1 <= top_k <=
   n_experts (MOE_ERR_INVALID_ARG), n_experts <= 1024 (MOE_ERR_UNSUPPORTED).
   Null logits or bias_next: MOE_ERR_INVALID_ARG; a null, misaligned or
   short workspace: MOE_ERR_WORKSPACE.
   The result is bitwise reproducible: counts are integers and every sum has
   a fixed order. */
moe_status moe_router_bias_ws_bytes(const moe_config* cfg, int32_t n_bins, size_t* bytes);
moe_status moe_router_bias_update(const moe_config* cfg, const float* logits, int32_t n_bins,
                                  float* bias_next, int32_t* hist, float* lohi, void* ws,
                                  size_t ws_bytes, void* stream);

/* moe_router_bias_update recording stage_events (n_events >= 5 hipEvent_t,
   created by the caller) on the stream around its 4 launches: 0 per-chunk
   ranges, 1 per-chunk histograms, 2 quantiles, 3 the mean and the bias. */
int32_t moe_router_bias_stage_count(void);
moe_status moe_router_bias_update_profiled(const moe_config* cfg, const float* logits,
                                           int32_t n_bins, float* bias_next, int32_t* hist,
                                           float* lohi, void* ws, size_t ws_bytes, void* stream,
                                           void* const* stage_events, int32_t n_events);

/* Sender pooling and receiver binning (lamjinlab.com section 2: one fixed
   pool per receiving destination rather than one buffer per expert, three
   waves of identical array shapes, expert ids packed into the payload,
   overflow past either fixed buffer dropped and counted separately).
   topk_idx  (device) [T][k] int32, 0 <= e < E; an id outside [0, E) takes
             no slot and is counted as a sender drop
   z         (device) [T][L] dtype: the rows to send
   pools     (device, out) pools_bytes: for wave w and pool p the block at
             (w*P + p) * pool_block_bytes holds C_send rows of L elements,
             then C_send int32 expert ids at ids_offset (-1 = empty slot).
             Slot s of a block holds the s-th row the wave sent to that pool
             in (token, j) order.  Rows of empty slots are not written.
   pool_slot (device, out) [T][k]: pool slot of the assignment, -1 if the
             sender cap dropped it
   recv_slot (device, out) [T][k]: receiver slot, -1 if either cap dropped it
   bank_rows (device, out) [W][E][C_recv]: pool slot of the r-th row binned
             to expert e, found by the receiver from the id column alone;
             entries r >= expert_count[w][e] are not written
   pool_count (device, out) [W][P]: occupied slots = min(C_send, demand)
   expert_count (device, out) [W][E]: rows binned to e (<= C_recv)
   counts    (device, out) int64[3]: {kept, sender_dropped, receiver_dropped},
             kept + sender_dropped + receiver_dropped = T * k
   ws        (device) at least dispatch_ws_bytes, 256-byte aligned. */
moe_status moe_dispatch(const moe_config* cfg, const int32_t* topk_idx,
                        const void* z, void* pools, int32_t* pool_slot,
                        int32_t* recv_slot, int32_t* bank_rows,
                        int32_t* pool_count, int32_t* expert_count,
                        int64_t* counts, void* ws, size_t ws_bytes,
                        void* stream);

/* moe_dispatch for callers that cannot allocate device memory: code under
   HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
   The same work and the same results as moe_dispatch, with its scratch (the
   dispatch_ws_bytes moe_dispatch takes as ws) in a library-owned device
   array of moe_dispatch_noalloc_scratch_bytes() = 4 MiB instead of a
   workspace argument; the call allocates nothing.  Each GPU the library
   runs on holds its own copy of the array until the process ends.  Every
   call on one GPU shares that GPU's copy: calls that overlap on one GPU (on
   different streams, or from different host threads) race and must be
   serialised by the caller.  All other arguments as in moe_dispatch.
   Errors: as moe_dispatch; MOE_ERR_WORKSPACE when the shape's
   dispatch_ws_bytes exceeds the array; MOE_ERR_HIP when the array's device
   address cannot be obtained. */
moe_status moe_dispatch_noalloc(const moe_config* cfg, const int32_t* topk_idx,
                                const void* z, void* pools, int32_t* pool_slot,
                                int32_t* recv_slot, int32_t* bank_rows,
                                int32_t* pool_count, int32_t* expert_count,
                                int64_t* counts, void* stream);

/* Bytes of moe_dispatch_noalloc's scratch array (per GPU). */
int64_t moe_dispatch_noalloc_scratch_bytes(void);

/* Routed experts over the received pool blocks (ranhao.site section 2.2:
   384 routed experts of width 3072; SwiGLU, no biases).  For every expert e,
   the rows of all waves binned to it form one group:
   o = (silu(u W_g[e]^T) * (u W_u[e]^T)) W_d[e]^T, written to expert_out at
   the row's own (wave, pool, slot): [W][P][C_send][L].  Rows of empty or
   receiver-dropped slots are not written.
   pools, bank_rows, expert_count: as produced by moe_dispatch (device);
             counts are clamped to [0, C_recv] and slots to [0, C_send)
   w_gate, w_up (device) [E][F][L]; w_down (device) [E][L][F]
   ws (device) at least experts_ws_bytes, 256-byte aligned. */
moe_status moe_experts(const moe_config* cfg, const void* pools,
                       const int32_t* bank_rows, const int32_t* expert_count,
                       const void* w_gate, const void* w_up,
                       const void* w_down, void* expert_out, void* ws,
                       size_t ws_bytes, void* stream);

/* Gate-weighted combine (lamjinlab.com section 4: dropped assignments do
   not remove the token, the shared experts still process it).
   y_latent[t] = sum over j with recv_slot[t][j] >= 0 of
                 gates[t][j] * expert_out[w(t)][pool(topk_idx[t][j])][pool_slot[t][j]]
   with fp32 accumulation; dropped assignments add nothing and the gates are
   not renormalised.  w(t) = t / Tw.  An assignment whose expert id is not in
   [0, E) or whose pool slot is not in [0, C_send) adds nothing.  All pointers device; y_latent [T][L]
   dtype (out). */
moe_status moe_combine(const moe_config* cfg, const void* expert_out,
                       const int32_t* topk_idx, const int32_t* pool_slot,
                       const int32_t* recv_slot, const float* gates,
                       void* y_latent, void* stream);

/* The whole branch (lamjinlab.com section 2; ranhao.site section 2.2):
   x (device) [T][D]; y (device, out) [T][D]; w (host struct of device
   pointers); taps (host struct, may be NULL); counts (device, out, may be
   NULL) int64[3] as in moe_dispatch; ws (device) at least forward_ws_bytes,
   256-byte aligned.  If n_shared == 0 the shared weights may be NULL.
   Needs top_k <= E (MOE_ERR_INVALID_ARG) and E % 4 == 0
   (MOE_ERR_UNSUPPORTED). */
moe_status moe_forward(const moe_config* cfg, const moe_weights* w,
                       const void* x, void* y, const moe_taps* taps,
                       int64_t* counts, void* ws, size_t ws_bytes,
                       void* stream);

/* Number of stages of moe_forward, in launch order: 0 latent GEMM, 1 router
   GEMM, 2 top-k and gates, 3 slot assignment, 4 row scatter into the pools,
   5 receiver binning, 6 expert row lists, 7 expert gate/up GEMM, 8 expert
   down GEMM, 9 combine, 10 shared-expert gate/up GEMM, 11 output GEMM
   (up-projection plus shared down-projections). */
int32_t moe_forward_stage_count(void);

/* moe_forward that also records stage_events[0] on `stream` before stage 0
   and stage_events[i + 1] after stage i, for i < n_events - 1 (events past
   the stage count are not recorded).  stage_events are hipEvent_t handles
   created by the caller.  Same results as moe_forward.  Errors as
   moe_forward, plus MOE_ERR_INVALID_ARG for n_events < 0 or a NULL event. */
moe_status moe_forward_profiled(const moe_config* cfg, const moe_weights* w,
                                const void* x, void* y, const moe_taps* taps,
                                int64_t* counts, void* ws, size_t ws_bytes,
                                void* stream, void* const* stage_events,
                                int32_t n_events);

/* ------------------------------------------------------------------------
 * Dropless ragged variant (lamjinlab.com section 4 and ranhao.site section
 * 3.3: the fallback that keeps every routed assignment, a ragged all-to-all
 * in place of the fixed capped pools; the production run switched to it).
 * No caps, no pools, no waves: the T*k assignments are ordered by expert,
 * stably in (token, j) order, expert e's rows form the contiguous range
 * [expert_offsets[e], expert_offsets[e+1]) of xs and of expert_out, and the
 * grouped GEMM runs over these variable-size groups.  The result equals the
 * capped branch with caps large enough for every row.  bf16 only
 * (MOE_ERR_UNSUPPORTED for MOE_F32).  n_pools, n_waves and the caps of *cfg
 * are validated as for moe_make_plan but otherwise unused.
 * ---------------------------------------------------------------------- */

/* Optional taps of moe_forward_dropless (device pointers, each may be NULL). */
typedef struct {
  float* logits;           /* [T][E] fp32                              */
  int32_t* topk_idx;       /* [T][k]                                   */
  float* gates;            /* [T][k]                                   */
  int32_t* row_of;         /* [T][k]: row of the assignment in xs      */
  int32_t* expert_offsets; /* [E + 1]                                  */
  void* z;                 /* [T][L]                                   */
  void* xs;                /* [T*k][L] rows ordered by expert          */
  void* expert_out;        /* [T*k][L]                                 */
  void* y_latent;          /* [T][L]                                   */
} moe_dropless_taps;

/* Order the assignments by expert and copy their rows.
   topk_idx (device) [T][k]; an id outside [0, E) takes no row (row_of -1)
   and is counted in counts[1]
   z        (device) [T][L] bf16
   xs       (device, out) [T*k][L] bf16: row r holds z[t] of the assignment
            (t, j) with row_of[t][j] == r; rows past expert_offsets[E] are
            not written
   row_of   (device, out) [T][k] int32
   expert_offsets (device, out) [E + 1] int32, expert_offsets[0] = 0
   counts   (device, out, may be NULL) int64[3]: {kept, invalid ids, 0}
   ws       (device) at least dropless_dispatch_ws_bytes, 256-byte aligned. */
moe_status moe_dispatch_dropless(const moe_config* cfg, const int32_t* topk_idx, const void* z,
                                 void* xs, int32_t* row_of, int32_t* expert_offsets,
                                 int64_t* counts, void* ws, size_t ws_bytes, void* stream);

/* Grouped SwiGLU over the variable-size groups: for every expert e and row r
   of its range, expert_out[r] = (silu(xs[r] W_g[e]^T) * (xs[r] W_u[e]^T))
   W_d[e]^T.  xs, expert_out (device) [T*k][L] bf16; expert_offsets (device)
   [E + 1], non-decreasing with expert_offsets[E] <= T*k (not checked on the
   device); weights as in moe_experts.  ws (device) at least
   dropless_experts_ws_bytes, 256-byte aligned. */
moe_status moe_experts_dropless(const moe_config* cfg, const void* xs,
                                const int32_t* expert_offsets, const void* w_gate,
                                const void* w_up, const void* w_down, void* expert_out, void* ws,
                                size_t ws_bytes, void* stream);

/* y_latent[t] = sum over j with row_of[t][j] >= 0 of
   gates[t][j] * expert_out[row_of[t][j]], fp32 accumulation in j order.
   All pointers device; y_latent [T][L] bf16 (out). */
moe_status moe_combine_dropless(const moe_config* cfg, const void* expert_out,
                                const int32_t* row_of, const float* gates, void* y_latent,
                                void* stream);

/* The whole branch without caps: as moe_forward, with the ragged dispatch,
   grouped experts and combine above.  taps (host struct, may be NULL);
   counts (device, out, may be NULL) as in moe_dispatch_dropless; ws (device)
   at least dropless_forward_ws_bytes, 256-byte aligned. */
moe_status moe_forward_dropless(const moe_config* cfg, const moe_weights* w, const void* x, void* y,
                                const moe_dropless_taps* taps, int64_t* counts, void* ws,
                                size_t ws_bytes, void* stream);

/* Number of stages of moe_forward_dropless, in launch order: 0 latent GEMM,
   1 router GEMM, 2 top-k and gates, 3 expert sort, 4 row scatter, 5 tile
   lists, 6 expert gate/up GEMM, 7 expert down GEMM, 8 combine, 9
   shared-expert gate/up GEMM, 10 output GEMM. */
int32_t moe_forward_dropless_stage_count(void);

/* moe_forward_dropless recording stage_events as moe_forward_profiled does. */
moe_status moe_forward_dropless_profiled(const moe_config* cfg, const moe_weights* w,
                                         const void* x, void* y, const moe_dropless_taps* taps,
                                         int64_t* counts, void* ws, size_t ws_bytes, void* stream,
                                         void* const* stage_events, int32_t n_events);

/* ------------------------------------------------------------------------
 * Backward of the routed path (training).  The pages train this branch
 * (lamjinlab.com section 2) and print no backward pass; these entry points
 * are the derivative of the forward above for a fixed routing, one per
 * forward step, each the transpose of its forward:
 *   combine   -> d_gates[t][j] = <dy_latent[t], o[t][j]> and the row
 *                gradient g[t][j] * dy_latent[t] at o's pool slot
 *   experts   -> per expert, with a = u W_g^T, b = u W_u^T recomputed:
 *                dh = do W_d, da = dh * b * silu'(a), db = dh * silu(a),
 *                du = da W_g + db W_u (dgrad), dW_d = do^T (silu(a) * b),
 *                dW_g = da^T u, dW_u = db^T u (wgrad, summed over the
 *                expert's rows of every wave)
 *   dispatch  -> dz[t] = sum over receiver-kept j of du at (t, j)'s slot
 *   route     -> d_logits through the softmax over the k selected logits
 * Unselected experts and the balancing bias get no gradient (ranhao.site
 * section 2.2: the bias is a heuristic outside the gradient); dropped
 * assignments get nothing (lamjinlab.com section 4).  bf16 activations and
 * weights with fp32 accumulation; d_gates and d_logits fp32; weight
 * gradients bf16 in the weights' [out, in] layout, each the full fp32 sum
 * over the expert's rows rounded once.  bf16 only, d_latent and d_ff
 * multiples of 256 (else MOE_ERR_UNSUPPORTED).  All pointers device unless
 * noted.  Buffers, counts and slots are those of the forward call whose
 * gradient is taken (moe_taps gives them).
 * ------------------------------------------------------------------------ */

/* Transpose of moe_combine.  dy_latent [T][L]; d_gates (out) [T][k] fp32
   (0 for a dropped assignment); d_expert_out (out) expert_out_bytes: row
   gates[t][j] * dy_latent[t] at the (wave, pool, slot) each kept (t, j)
   read in the forward; other rows are not written. */
moe_status moe_combine_backward(const moe_config* cfg, const void* expert_out,
                                const int32_t* topk_idx, const int32_t* pool_slot,
                                const int32_t* recv_slot, const float* gates,
                                const void* dy_latent, float* d_gates,
                                void* d_expert_out, void* stream);

/* Transpose of moe_experts.  pools, bank_rows, expert_count: the forward's;
   d_expert_out: from moe_combine_backward; d_pool_rows (out)
   expert_out_bytes: du of every kept row at its (wave, pool, slot), other
   rows not written; dw_gate, dw_up (out) [E][F][L], dw_down (out) [E][L][F]
   bf16, written whole (zero for an expert without rows).  ws at least
   experts_bwd_ws_bytes, 256-byte aligned. */
moe_status moe_experts_backward(const moe_config* cfg, const void* pools,
                                const int32_t* bank_rows, const int32_t* expert_count,
                                const void* w_gate, const void* w_up, const void* w_down,
                                const void* d_expert_out, void* d_pool_rows,
                                void* dw_gate, void* dw_up, void* dw_down, void* ws,
                                size_t ws_bytes, void* stream);

/* Transpose of moe_dispatch: dz (out) [T][L] bf16, dz[t] = the fp32 sum of
   the d_pool_rows rows of t's receiver-kept assignments, in j order (zero
   for a token with none). */
moe_status moe_dispatch_backward(const moe_config* cfg, const int32_t* topk_idx,
                                 const int32_t* pool_slot, const int32_t* recv_slot,
                                 const void* d_pool_rows, void* dz, void* stream);

/* Transpose of the gate softmax of moe_route: d_logits (out) [T][E] fp32,
   d_logits[t][topk_idx[t][j]] = g_j (dg_j - sum_i g_i dg_i), 0 elsewhere.
   Only T, n_experts and top_k of *cfg are read. */
moe_status moe_route_backward(const moe_config* cfg, const int32_t* topk_idx,
                              const float* gates, const float* d_gates,
                              float* d_logits, void* stream);

/* The four in order: saved (host struct) names the forward's topk_idx,
   gates, pool_slot, recv_slot, expert_count, bank_rows, pools and
   expert_out (all required); w supplies w_gate, w_up, w_down.  dz, d_logits,
   dw_* as above; ws at least backward_ws_bytes, 256-byte aligned. */
moe_status moe_backward_routed(const moe_config* cfg, const moe_weights* w,
                               const moe_taps* saved, const void* dy_latent, void* dz,
                               float* d_logits, void* dw_gate, void* dw_up, void* dw_down,
                               void* ws, size_t ws_bytes, void* stream);

/* Stages of moe_backward_routed, in launch order: 0 combine backward,
   1 padded expert layout and tile lists, 2 row gathers, 3 dh GEMM, 4 gate/up
   recompute GEMM with the SwiGLU backward, 5 du GEMM, 6 dW_down, 7 dW_gate,
   8 dW_up, 9 dispatch backward, 10 route backward. */
int32_t moe_backward_routed_stage_count(void);

/* moe_backward_routed recording stage_events as moe_forward_profiled does. */
moe_status moe_backward_routed_profiled(const moe_config* cfg, const moe_weights* w,
                                        const moe_taps* saved, const void* dy_latent, void* dz,
                                        float* d_logits, void* dw_gate, void* dw_up,
                                        void* dw_down, void* ws, size_t ws_bytes, void* stream,
                                        void* const* stage_events, int32_t n_events);

/* Backward of the dropless variant: the same transposes over its
   expert-ordered rows (every assignment kept).  The experts' backward takes
   xs and expert_offsets from moe_dispatch_dropless; the stages of
   moe_backward_dropless are those of moe_backward_routed. */

/* d_gates[t][j] = <dy_latent[t], expert_out[row_of[t][j]]> (0 where
   row_of < 0); d_expert_out (out) [T*k][L]: gates[t][j] * dy_latent[t] at
   row row_of[t][j]; rows without an assignment are not written. */
moe_status moe_combine_backward_dropless(const moe_config* cfg, const void* expert_out,
                                         const int32_t* row_of, const float* gates,
                                         const void* dy_latent, float* d_gates,
                                         void* d_expert_out, void* stream);

/* d_xs (out) [T*k][L]: du of every row below expert_offsets[E]; dw_* (out)
   as in moe_experts_backward.  ws at least dropless_experts_bwd_ws_bytes,
   256-byte aligned. */
moe_status moe_experts_backward_dropless(const moe_config* cfg, const void* xs,
                                         const int32_t* expert_offsets, const void* w_gate,
                                         const void* w_up, const void* w_down,
                                         const void* d_expert_out, void* d_xs, void* dw_gate,
                                         void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                                         void* stream);

/* dz (out) [T][L]: dz[t] = sum over j with row_of[t][j] >= 0 of
   d_xs[row_of[t][j]], fp32 accumulation in j order. */
moe_status moe_dispatch_backward_dropless(const moe_config* cfg, const int32_t* row_of,
                                          const void* d_xs, void* dz, void* stream);

/* The chain (combine, experts, dispatch, route backward): saved (host
   struct) names the dropless forward's topk_idx, gates, row_of,
   expert_offsets, xs and expert_out (all required).  ws at least
   dropless_backward_ws_bytes, 256-byte aligned. */
moe_status moe_backward_dropless(const moe_config* cfg, const moe_weights* w,
                                 const moe_dropless_taps* saved, const void* dy_latent, void* dz,
                                 float* d_logits, void* dw_gate, void* dw_up, void* dw_down,
                                 void* ws, size_t ws_bytes, void* stream);

/* moe_backward_dropless recording stage_events as moe_forward_profiled does. */
moe_status moe_backward_dropless_profiled(const moe_config* cfg, const moe_weights* w,
                                          const moe_dropless_taps* saved, const void* dy_latent,
                                          void* dz, float* d_logits, void* dw_gate, void* dw_up,
                                          void* dw_down, void* ws, size_t ws_bytes, void* stream,
                                          void* const* stage_events, int32_t n_events);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
