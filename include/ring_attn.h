/*
 * ring_attn.h -- C ABI of the ring-attention rank-share library (gfx950).
 *
 * One rank's share of ring attention: the rank's local query shard attends,
 * step by step in ring order, to the D key/value blocks that pass around the
 * ring; each step is a flash-attention forward that yields a partial output
 * and a per-row log-sum-exp, and the partials are folded into a running
 * (out, lse) by the log-sum-exp merge.  The backward pass accumulates dQ, dK
 * and dV over the same steps.  On one GPU every block is already resident in
 * device memory and is read in ring order; there is no communication.
 *
 * Sources (web pages on ring attention, cited by title and section):
 *   - instagit.com, "How to Implement Ring Attention for Long Sequences in
 *     Nanotron": "Forward Pass Implementation" (per-step flash forward, the
 *     merge, the causal rule step <= rank), "Backward Pass and Gradient
 *     Accumulation", "Numerically-Stable Output Fusion", "Calling the Ring
 *     Attention Function Directly" (bshd tensors, cu_seqlens, the
 *     1/sqrt(head_dim) default scale, the returned (out, softmax_lse)).
 *   - ai360xpert.com, "Ring Attention": "Sequence sharding and the ring
 *     topology", "Online softmax across ring steps", "Watch Out For" (causal
 *     masks use global positions).
 *   - skillfed.io, "ring-flash-attn": basic, zigzag, stripe and llama3-style
 *     variants, in batch and varlen (packed) form.
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-allocated device memory, contiguous, 16-byte
 *     aligned.  The library never frees or reallocates them.
 *   - Host pointers are read during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     device work is enqueued on it; calls return without synchronising.
 *   - The first call for a shape builds its plan: host work, one hipMalloc
 *     and an upload that the host waits for (on a stream of the library's
 *     own, so not behind work queued on `stream`).  Later calls for that shape
 *     enqueue kernels only (no allocation, no memset, no copy), so they can
 *     be captured into a HIP graph and replayed; a call made while `stream`
 *     is being captured never builds a plan (RA_E_NO_PLAN).  The plans live
 *     in a cache of at most ring_attn_plan_cache_limit() plans (32 by
 *     default), least recently used first out; every packed-layout
 *     cu_seqlens is its own shape.  Evicted plans are freed in batches of the
 *     cache limit (the release waits for the device once per batch), and
 *     ring_attn_clear_cache() frees them all; either invalidates any captured
 *     graph that used those plans.
 *   - Return value: 0 on success, a negative RA_E_* code on failure.  All
 *     argument validation happens before any device work is enqueued, so a
 *     failing call leaves every buffer untouched.  Nothing is printed and no
 *     C++ exception crosses the ABI.  ring_attn_strerror() names each code.
 *   - Thread safety: calls may come from several threads.  The library's
 *     mutable globals are each mutex-guarded: the cache of per-shape plans
 *     (step schedule and tile lists uploaded to device memory it owns; a call
 *     keeps its plan alive until it returns, even if another thread evicts
 *     it or clears the cache meanwhile); a bounded host-side memo of dS store
 *     sizes; and the optional per-kernel timing state.  Calls that use the
 *     same workspace or output buffers on different streams at the same time
 *     race, as any kernels do.
 */
#ifndef RING_ATTN_H
#define RING_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Which global tokens each rank (and each KV block) holds.  N = seqlen,
 * D = world, S = N / D local rows.  Local order is increasing global order.
 *   RA_BASIC       rank r holds [r*S, (r+1)*S)          ("Ring Attention",
 *                  "Sequence sharding and the ring topology").
 *   RA_ZIGZAG      2D chunks of c = N/(2D); rank r holds chunk r, then chunk
 *                  2D-1-r ("ring-flash-attn": the compute-balanced variant).
 *   RA_STRIPE      token t belongs to rank t mod D (stripe width 1).
 *   RA_VARLEN_RING packed documents; every document (length a multiple of D)
 *                  is cut into D equal parts and rank r holds part r of each.
 *   RA_LLAMA3      query shard as RA_BASIC over the packed stream; the KV is
 *                  the gathered stream (all N tokens, global order), attended
 *                  in a single step with per-document causal masking.
 *   RA_VARLEN_ZIGZAG packed documents, RA_ZIGZAG applied inside each one:
 *                  every document (length a multiple of 2D) is cut into 2D
 *                  chunks and rank r holds chunks r and 2D-1-r of each, in
 *                  document order ("ring-flash-attn": every variant in batch
 *                  and varlen form).
 *   RA_VARLEN_STRIPE packed documents, RA_STRIPE applied inside each one:
 *                  token a+i of a document starting at a (length a multiple
 *                  of D) belongs to rank i mod D.
 * KV block j of the ring layouts is exactly what rank j holds. */
typedef enum {
    RA_BASIC = 0,
    RA_ZIGZAG = 1,
    RA_STRIPE = 2,
    RA_VARLEN_RING = 3,
    RA_LLAMA3 = 4,
    RA_VARLEN_ZIGZAG = 5,
    RA_VARLEN_STRIPE = 6
} ra_layout;

/* Element type of q, k, v, out and dout.  Accumulation is always fp32. */
typedef enum { RA_F32 = 0, RA_BF16 = 1 } ra_dtype;

/* How the forward folds the per-step partials ("Numerically-Stable Output
 * Fusion"; "Online softmax across ring steps").
 *   RA_MERGE_FUSED      bf16: ONE kernel launch walks every active ring step
 *                       of each query tile and folds each step's partial into
 *                       the running result in registers (running max, sum and
 *                       unnormalised output: the log-sum-exp merge without a
 *                       round trip through memory); no workspace.  fp32 inputs
 *                       (or more than 2048 steps, or more than 2^20 64-key
 *                       tiles per block) use RA_MERGE_STEPWISE instead.
 *   RA_MERGE_SEPARATE   each step's kernel writes its partial (out_j, lse_j);
 *                       the standalone merge kernel (ring_attn_lse_merge)
 *                       folds it in; a final kernel casts the result.
 *   RA_MERGE_STEPWISE   one launch per step; each merges its partial into the
 *                       running fp32 result in its epilogue and the last one
 *                       writes out. */
typedef enum { RA_MERGE_FUSED = 0, RA_MERGE_SEPARATE = 1, RA_MERGE_STEPWISE = 2 } ra_merge_mode;

typedef struct ring_attn_desc {
    int32_t batch;         /* B (must be 1 for the packed layouts)   */
    int32_t heads_q;       /* Hq                                               */
    int32_t heads_kv;      /* Hkv; Hq % Hkv == 0; q head h uses kv head h*Hkv/Hq */
    int32_t head_dim;      /* d: 64 or 128                                     */
    int64_t seqlen;        /* N: global length (total packed tokens if varlen) */
    int32_t world;         /* D >= 1                                           */
    int32_t rank;          /* r in [0, D)                                      */
    int32_t causal;        /* 0 or 1: key u visible to query t iff u <= t      */
    int32_t layout;        /* ra_layout                                        */
    int32_t dtype;         /* ra_dtype                                         */
    float softmax_scale;   /* <= 0 selects 1/sqrt(head_dim); NaN or +-inf is
                            * RA_E_ARG                                         */
    int32_t n_seqs;        /* number of packed documents (varlen layouts), else 0 */
    int32_t merge_mode;    /* ra_merge_mode                                    */
    int32_t window_left;   /* sliding window: key u visible to query t only if */
    int32_t window_right;  /* t-left <= u <= t+right (global positions); -1 on
                            * a side leaves that side unbounded, so (-1, -1) is
                            * plain attention.  Values below -1 are RA_E_ARG.
                            * ("Ring Attention for Long Sequences in Nanotron":
                            * the window_size argument of the call interface,
                            * (-1, -1) = unbounded.)  Combined with the causal
                            * and document rules by AND.                       */
} ring_attn_desc;

/* Error codes. */
#define RA_OK                 0
#define RA_E_NULL            -1  /* a required pointer is NULL                 */
#define RA_E_SHAPE           -2  /* batch/heads/seqlen out of range            */
#define RA_E_WORLD           -3  /* world < 1 or rank not in [0, world)        */
#define RA_E_DIVISIBILITY    -4  /* N % D != 0 (N % 2D for both zigzags)       */
#define RA_E_CU_SEQLENS      -5  /* cu_seqlens not 0 .. N non-decreasing, or a
                                    document length not a multiple of D
                                    (varlen ring, varlen stripe) or of 2D
                                    (varlen zigzag)                            */
#define RA_E_HEADS           -6  /* heads_q % heads_kv != 0                    */
#define RA_E_UNSUPPORTED     -7  /* no kernel for this head_dim/dtype/mode     */
#define RA_E_WORKSPACE       -8  /* workspace NULL or smaller than required    */
#define RA_E_LAYOUT          -9  /* unknown layout, or batch != 1 for varlen   */
#define RA_E_HIP            -10  /* the HIP runtime reported an error          */
#define RA_E_ARG            -11  /* another argument out of range              */
#define RA_E_NO_PLAN        -12  /* shape never planned, and no plan can be built
                                   * here (ring_attn_bwd_noalloc, or a call
                                   * made during graph capture)               */
#define RA_E_SCRATCH        -13  /* ring_attn_bwd_noalloc: scratch too small   */

/* Shapes (all row-major, last dimension fastest):
 *   S   = N / D local rows;  Skv = S for ring layouts, N for RA_LLAMA3;
 *   nb  = D for ring layouts, 1 for RA_LLAMA3.
 *   q, out, dout : [B, S, Hq, d]      rank-local rows in local order
 *   k, v         : [nb, B, Skv, Hkv, d] block-major: block j = what rank j holds
 *   lse          : fp32 [B, Hq, S]    natural log of the sum of exp(scaled scores)
 *   dq           : fp32 [B, S, Hq, d]
 *   dk, dv       : fp32, shaped like k and v
 *   cu_seqlens   : host int32 [n_seqs + 1] in global packed coordinates
 *                  (packed layouts RA_VARLEN_RING, RA_LLAMA3, RA_VARLEN_ZIGZAG
 *                  and RA_VARLEN_STRIPE only; NULL otherwise). */

/* Bytes of device workspace ring_attn_fwd (is_bwd = 0) or ring_attn_bwd
 * (is_bwd = 1) needs for this descriptor; negative RA_E_* if the descriptor is
 * invalid (cu_seqlens is not inspected).  Forward: 0 for the one-launch
 * RA_MERGE_FUSED path, else the fp32 running output (plus one partial in
 * RA_MERGE_SEPARATE mode).  Backward: two per-row fp32
 * arrays of B * Hq * S_pad floats (the lse in base 2 and -Delta, Delta =
 * rowsum(dout * out)) and an fp32 dQ accumulator of B * Hq * S_pad * d floats
 * (S_pad = S rounded up to 256; each part starts on a 256-byte boundary). */
int64_t ring_attn_workspace_bytes(const ring_attn_desc* desc, int is_bwd);

/* Extra backward workspace, in bytes, that lets ring_attn_bwd keep dS (the
 * softmax gradient P (dP - Delta), bf16) from the dK/dV pass and build dQ
 * from it instead of recomputing S and dP ("Backward Pass and Gradient
 * Accumulation": dQ, dK and dV all follow from dS; keeping it trades 2 bytes
 * per visible tile element of HBM traffic for two of the three dQ
 * products).  It is B * Hq * (tiles of the busiest step) * 16 KiB, where a
 * tile is 64 query rows x 128 keys with at least one visible pair; exact for
 * the given cu_seqlens (NULL unless the layout is packed).  Host only.
 * Returns a negative RA_E_* for an invalid descriptor. */
int64_t ring_attn_bwd_ds_bytes(const ring_attn_desc* desc, const int32_t* cu_seqlens);

/* Extra forward workspace, in bytes, that lets the one-launch RA_MERGE_FUSED
 * bf16 forward split long query-tile lists across CUs.  With more work items
 * (batch x q heads x 256-row query tiles) than CUs, the forward runs one
 * work-group per CU over a balanced list of items; a list much longer than
 * the others can be cut into parts run on different CUs, each part's
 * normalised partial and lse written to the workspace and the parts folded
 * by the log-sum-exp merge of "Numerically-Stable Output Fusion" (a second,
 * small kernel).  The parts never outnumber the CUs, so the bound is
 * (CUs of the current device, rounded down to a multiple of 8) x 256 rows x
 * (head_dim + 1) x 4 bytes; 0 for other dtypes and merge modes.  A smaller
 * workspace is accepted: the lists then run whole.  Host only (queries the
 * current device); negative RA_E_* for an invalid descriptor, RA_E_HIP when
 * no device can be queried. */
int64_t ring_attn_fwd_split_bytes(const ring_attn_desc* desc);

/* Forward of the rank share ("Forward Pass Implementation"): for s = 0..D-1
 * the block j = (rank - s) mod D is attended if at least one (query, key) pair
 * of the step is visible (under a causal basic layout exactly the steps with
 * s <= rank), each step's partial is merged into the running result, and the
 * result is written as out (dtype of q) and lse (fp32).  A row with no
 * visible key gets out = 0 and lse = -inf.  Workspace: at least
 * ring_attn_workspace_bytes(desc, 0) bytes of device memory; with
 * ring_attn_fwd_split_bytes(desc) bytes beyond that, long query-tile lists
 * may be split across CUs (the results then differ from an unsplit run only
 * by the rounding of the merge).  Its contents need not be initialised and
 * are garbage afterwards. */
int ring_attn_fwd(const ring_attn_desc* desc, const void* q, const void* k,
                  const void* v, const int32_t* cu_seqlens, void* out, float* lse,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Backward of the rank share ("Backward Pass and Gradient Accumulation") for
 * the loss sum(dout * out), given the out and lse that ring_attn_fwd returned.
 * dq is OVERWRITTEN (it belongs to this rank).  dk and dv are ACCUMULATED
 * (+=): this rank's contribution to every block is added, so calling the
 * backward for every rank on zeroed dk/dv yields the full gradient, as the
 * gradient accumulators travelling around the ring would.  Requires
 * dtype == RA_BF16.  Workspace: at least ring_attn_workspace_bytes(desc, 1)
 * bytes.  Bytes beyond that hold the dS tile store: with E extra bytes and
 * F = ring_attn_bwd_ds_bytes(desc, cu_seqlens), the kv heads are processed
 * min(heads_kv, floor(E / (F / heads_kv))) at a time and dQ is built from the
 * stored dS (same results up to summation order, less work); with less than
 * F / heads_kv extra bytes, dQ recomputes S and dP.  The contents need no
 * initialisation and are garbage afterwards. */
int ring_attn_bwd(const ring_attn_desc* desc, const void* dout, const void* q,
                  const void* k, const void* v, const void* out, const float* lse,
                  const int32_t* cu_seqlens, float* dq, float* dk, float* dv,
                  void* workspace, size_t workspace_bytes, void* stream);

/* ring_attn_bwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving or training loops, harnesses that forbid
 * hipMalloc): the same backward, with its workspace in a static device array
 * of ring_attn_noalloc_scratch_bytes() bytes (64 MiB) that the library holds
 * on every GPU it runs on until the process ends.  It calls no hipMalloc,
 * hipFree or other allocating routine, and never builds a plan: the shape's
 * plan must already be cached by an ordinary call (ring_attn_fwd or
 * ring_attn_bwd with the same descriptor and cu_seqlens), else RA_E_NO_PLAN.
 * A descriptor whose minimum backward workspace exceeds the array is
 * RA_E_SCRATCH; what the array holds beyond that minimum serves as the dS
 * tile store (kv heads in passes, or dQ by recomputation when none fits).
 * All calls on one GPU share its array: calls that overlap in time on one GPU
 * (other streams, other threads) race.  The array's contents are garbage
 * between calls and need no clearing.  Arguments and results as for
 * ring_attn_bwd. */
int ring_attn_bwd_noalloc(const ring_attn_desc* desc, const void* dout, const void* q,
                          const void* k, const void* v, const void* out, const float* lse,
                          const int32_t* cu_seqlens, float* dq, float* dk, float* dv,
                          void* stream);

/* Bytes of the static scratch array ring_attn_bwd_noalloc uses (per GPU). */
int64_t ring_attn_noalloc_scratch_bytes(void);

/* Log-sum-exp merge ("Numerically-Stable Output Fusion"), standalone.  Folds a
 * partial (out_j, lse_j) into the running (out, lse) in place:
 *   M = max(lse, lse_j); lse' = M + ln(e^(lse-M) + e^(lse_j-M));
 *   out' = e^(lse-lse') out + e^(lse_j-lse') out_j.
 * A partial with lse = -inf is the identity; two empty inputs stay (0, -inf).
 * out, out_j: fp32 [batch, seqlen, heads, head_dim]; lse, lse_j: fp32
 * [batch, heads, seqlen].  head_dim: any positive multiple of 4 (RA_E_SHAPE
 * otherwise).  Each row is merged by lanes of a single wave, so rows of any
 * length are safe to update in place. */
int ring_attn_lse_merge(float* out, float* lse, const float* out_j, const float* lse_j,
                        int32_t batch, int64_t seqlen, int32_t heads, int32_t head_dim,
                        void* stream);

/* Host only (no device work).  Global token index of each of the S local rows
 * of `rank` (pos_out: int64 [S]) or of each of the Skv rows of KV block
 * `block` (pos_out: int64 [Skv]).  Use these to shard global tensors. */
int ring_attn_positions(const ring_attn_desc* desc, const int32_t* cu_seqlens,
                        int32_t rank, int64_t* pos_out);
int ring_attn_kv_positions(const ring_attn_desc* desc, const int32_t* cu_seqlens,
                           int32_t block, int64_t* pos_out);

/* Host only.  The ring schedule of desc->rank: for each step s (nb entries),
 * the block it holds and its number of visible (query row, key) pairs per
 * (batch, q head); a step with 0 pairs is skipped by the forward and backward.
 * block_out: int32 [nb]; pairs_out: int64 [nb]; *n_steps receives nb. */
int ring_attn_schedule(const ring_attn_desc* desc, const int32_t* cu_seqlens,
                       int32_t* block_out, int64_t* pairs_out, int32_t* n_steps);

/* Host only.  Classification of the (query tile, key tile) pairs of step
 * `step` for tiles of tile_q query rows and tile_k keys: kinds_out is int8
 * [ceil(S/tile_q) * ceil(Skv/tile_k)], row-major by query tile, with
 * 0 = no visible pair, 1 = some pairs visible, 2 = every pair visible. */
int ring_attn_tile_kinds(const ring_attn_desc* desc, const int32_t* cu_seqlens,
                         int32_t step, int32_t tile_q, int32_t tile_k, int8_t* kinds_out);

/* Per-kernel timing with HIP events recorded on the launching stream around
 * every kernel the library enqueues (off by default).  ring_attn_timing_read
 * synchronises on the recorded events and reports, for the kernel class
 * `name` ("fwd_step", "lse_merge", "finalize", "bwd_pre", "bwd_step" (dK/dV),
 * "bwd_dq" (dQ recomputing S and dP), "bwd_dq_ds" (dQ from stored dS),
 * "bwd_post"), the
 * number of launches and their summed duration in milliseconds since the
 * last reset.  ring_attn_timing_enable(0) disables and resets. */
int ring_attn_timing_enable(int enable);
int ring_attn_timing_read(const char* name, int64_t* launches, double* total_ms);

/* Free every cached plan and every evicted one not yet released (and their
 * device memory on every device), waiting for the device first.  A plan that
 * a call in flight holds is freed when that call returns. */
int ring_attn_clear_cache(void);

/* Host only.  Sets the most plans the cache keeps (>= 1; RA_E_ARG otherwise),
 * evicting the least recently used ones beyond it; returns the previous
 * limit.  Evicted plans wait, up to as many again, for their batched
 * release. */
int ring_attn_plan_cache_limit(int32_t max_plans);

/* Host only.  Number of cached plans and the device bytes they hold (evicted
 * plans awaiting release are not counted). */
int ring_attn_plan_cache_info(int64_t* n_plans, int64_t* device_bytes);

const char* ring_attn_strerror(int code);

/* ABI version, currently 1. */
int ring_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RING_ATTN_H */
