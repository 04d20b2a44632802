/*
 * libkda — recurrent Kimi Delta Attention (KDA) training recurrence on AMD
 * Instinct MI355X (gfx950).  C ABI.
 *
 * What is computed (FlashInfer page "flashinfer.kda_backward.recurrent_kda_
 * backward", description; page "flashinfer.kda_training.recurrent_kda_training_
 * forward", parameter list).  For every sequence n and value head h, with the
 * q/k head hq = h / (Hv/Hqk), a 128x128 FP32 value-first state S[v][k] starts
 * at initial_state[n][h] and, token by token,
 *
 *     qn = q / sqrt(|q|^2 + 1e-6),   kn = k / sqrt(|k|^2 + 1e-6)
 *     alpha = exp(-5 * sigmoid(exp(A_log[h]) * (g + dt_bias[h][:])))   (per key)
 *     beta  = sigmoid(beta_logit)
 *     S <- S diag(alpha);   S <- S + beta (v - S kn) kn^T;   o = S qn / sqrt(128)
 *
 * o is stored in BF16 and the last S in FP32.  The backward returns the
 * gradients of <do, o> + <dfinal_state, S_final> with respect to the raw
 * inputs, in the order dq, dk, dv, dg, dbeta, dA_log, ddt_bias, dinitial_state
 * (page "flashinfer.kda_backward.recurrent_kda_backward", description).
 *
 * Tensor contract (page "flashinfer.kda_training.recurrent_kda_training_
 * forward", parameters; page "flashinfer.kda_training", paragraphs 3-4).  All
 * tensors are dense, row-major and contiguous, in device memory unless noted:
 *     q, k, dq, dk            BF16  [B][T][Hqk][128]
 *     v, g, o, do, dv, dg     BF16  [B][T][Hv][128]
 *     beta, dbeta             BF16  [B][T][Hv]       (raw logits)
 *     A_log, dA_log           FP32  [Hv]
 *     dt_bias, ddt_bias       FP32  [Hv][128]
 *     initial_state, final_state, dfinal_state, dinitial_state
 *                             FP32  [N][Hv][128][128]   (value-first: [v][k])
 * Fixed layout: N = B, every batch row is one sequence of T tokens, and both
 * cu_seqlens pointers are NULL.  Packed layout: B = 1, sequence n occupies
 * tokens [cu[n], cu[n+1]) of the single row; cu_seqlens (device, INT64 [N+1])
 * and its trusted host mirror cu_seqlens_host (INT64 [N+1]) are both given.
 * Every sequence is non-empty; lengths need not be multiples of 16.  Hv must
 * be a multiple of Hqk.  scale is 1/sqrt(128) and lower_bound is -5.
 *
 * Ownership.  The caller owns every buffer: inputs, outputs, the forward
 * context and the backward workspace.  The library keeps a cache of small
 * device-side schedules keyed by device and sequence lengths (as the pages
 * cache their longest-first order per unchanged offsets), and a host-side
 * record of each context's producing call for the backward's checks.  The
 * cache holds at most 1024 schedules.  When a call needs a new one and the
 * cache is full, the least recently used quarter of the schedules that no
 * call holds and no captured graph uses is freed.  That call first waits on
 * the host for the launches that last read them.  The context records keep
 * the last 4096 contexts filled; a backward on a context forgotten since
 * returns KDA_ERR_CTX_MISMATCH.
 *
 * Errors.  Every entry point returns a kda_status.  All argument checks run on
 * the host before any launch; nothing is launched when a check fails.  A HIP
 * failure after launches began returns KDA_ERR_HIP; kda_last_error() gives
 * the text of the last failure on the calling thread.  Launches are
 * asynchronous on the given stream (a hipStream_t; NULL is the null stream).
 * No entry point synchronises the device, except the schedule eviction above.
 *
 * Stream capture.  kda_fwd and kda_bwd may be recorded into a HIP graph: under
 * capture they enqueue kernel launches only (no allocation, copy, memset or
 * event wait).  That needs the schedule for the call's sequence lengths to be
 * cached already and known to be on the device: make one call with the same
 * lengths outside capture, let it complete, then make a second one outside
 * capture (it observes the upload as finished); otherwise a call under
 * capture returns KDA_ERR_CAPTURE before touching the stream.  A captured
 * graph keeps using the cached schedule, which lives until the process ends.
 */
#ifndef LIBKDA_H
#define LIBKDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128
#define KDA_VERSION 1
/* Size of the static device scratch of kda_fwd_noalloc (per device). */
#define KDA_NOALLOC_SCRATCH_BYTES (4u << 20)

typedef enum {
    KDA_OK = 0,
    KDA_ERR_NULL_ARG = 1,       /* a required pointer is NULL */
    KDA_ERR_SHAPE = 2,          /* B, T, heads, N out of range or inconsistent */
    KDA_ERR_GROUPING = 3,       /* Hv is not a multiple of Hqk */
    KDA_ERR_SEQLENS = 4,        /* cu_seqlens_host not 0 < ... strictly increasing ... = T */
    KDA_ERR_SCALE = 5,          /* scale is neither 0 nor 1/sqrt(128) */
    KDA_ERR_LOWER_BOUND = 6,    /* lower_bound is not -5 */
    KDA_ERR_OVERLAP = 7,        /* an output overlaps an input, the context or another output */
    KDA_ERR_CTX_SIZE = 8,       /* context smaller than kda_fwd_ctx_bytes() */
    KDA_ERR_CTX_MISMATCH = 9,   /* context not produced by a matching kda_fwd */
    KDA_ERR_WORKSPACE_SIZE = 10,/* workspace smaller than kda_bwd_workspace_bytes() */
    KDA_ERR_ROUTE = 11,         /* unknown route or checkpoint interval */
    KDA_ERR_HIP = 12,           /* a HIP runtime call failed */
    KDA_ERR_CAPTURE = 13        /* called under stream capture before the schedule
                                   for these lengths was made and had reached the
                                   device in an earlier call outside capture */
} kda_status;

typedef enum {
    KDA_ROUTE_AUTO = 0,      /* library chooses (see kda_plan_query) */
    KDA_ROUTE_CHUNK = 1,     /* chunked MFMA kernel */
    KDA_ROUTE_ROWSPLIT = 2,  /* per-token FP32 kernel, state rows split across workgroups */
    KDA_ROUTE_SEGMENTS = 3,  /* training forward with the tape context only: the chunked
                                kernel over all tape segments at once.  Each segment's
                                end state is affine in its start state (S_in P + Q); P
                                and Q of every segment are formed in parallel, chained
                                into the tape, and every segment is rerun for o.  The
                                context is larger by 3 states per segment and head
                                (P, Q and P transposed, which the backward chains
                                with).
                                AUTO takes it when 2 x segments x Hv <= 768 and the
                                longest sequence spans more than 4 tape segments (4 or
                                more when KDA_ROUTE_CHUNK_SPLIT does not apply).  Without
                                a context the plain chunked kernel runs. */
    KDA_ROUTE_CHUNK_SPLIT = 4 /* training forward (tape context or none): the chunk form
                                with each task's 128 value columns split over two
                                workgroups (the state path is column-local).  In each,
                                four waves run the state path while four others prepare
                                the next four chunks' state-independent work (prologue,
                                16x16 algebra), so with fewer tasks than compute units
                                a task's chain of chunks is shorter.  Its tape equals
                                KDA_ROUTE_CHUNK's to rounding; same backward.  AUTO
                                takes it when 2 x tasks <= 256 and route 3 is not
                                taken. */
} kda_route;

/* What the training forward saves for the backward.  TAPE: the FP32 state
 * every checkpoint_every tokens; the backward rebuilds each segment's chunk
 * states from it (small context, a rebuild pass in the backward).  RECORDS:
 * every chunk's start state (BF16), U (BF16) and T, Akk, Aqk (FP32), about
 * 39 KiB per 16 tokens and value head; with more than 256 tasks (sequences
 * x value heads; not on the segment-parallel route, which is for few tasks)
 * the start state only of every other chunk, with what steps
 * it to the next one (that chunk's U and Kt, BF16, and exp(gC)), about
 * 27 KiB.  The backward reruns no forward recurrence (page
 * "flashinfer.kda_training", paragraph 5), at the cost of a larger context
 * and a forward that writes it.  RECORDS needs the chunked route. */
typedef enum {
    KDA_CONTEXT_TAPE = 0,
    KDA_CONTEXT_RECORDS = 1
} kda_context;

/* Precision of the chunked kernels' state path.  The chunk form predicts the
 * state against each chunk's keys with BF16 MFMA operands (Kg S0^T, Tb Y, Akk);
 * under decay that rounding is forgotten within a few tokens, but a channel
 * whose decay is weak keeps it, and the FP32 state drifts past 1e-3.  AUTO
 * runs a chunk with BF16 hi/lo pairs on those operands too (three products
 * each, FP32-accurate) when some channel keeps more than exp(-2) of its state
 * over the chunk (page "flashinfer.kda_training", paragraph 1: the chunked
 * routes' public final state comes from a recurrence kept in full precision;
 * here per chunk, and only where the decay makes it matter); FULL runs every
 * chunk that way; FAST none (final states can then miss 1e-3 on weakly
 * decaying inputs).  The row-split route is FP32 throughout and ignores this. */
typedef enum {
    KDA_PRECISION_AUTO = 0,
    KDA_PRECISION_FULL = 1,
    KDA_PRECISION_FAST = 2
} kda_precision;

/* Order in which the (sequence, value head) tasks are dispatched.  Each task
 * is owned by one workgroup, so the results do not depend on it.
 * LONGEST_FIRST: longest sequence first (page "flashinfer.kda.recurrent_kda",
 * parameter cu_seqlens), so that a long task does not start last and run
 * alone; SEQUENCE: sequence order (for measuring what longest-first buys). */
typedef enum {
    KDA_SCHEDULE_LONGEST_FIRST = 0,
    KDA_SCHEDULE_SEQUENCE = 1
} kda_schedule;

/* One call's shape.  All fields are read by value; the struct is not kept. */
typedef struct {
    int32_t B;                       /* physical batch (1 when packed) */
    int32_t T;                       /* tokens per batch row */
    int32_t Hqk;                     /* q/k heads */
    int32_t Hv;                      /* value heads, a multiple of Hqk */
    int32_t N;                       /* sequences: B (fixed) or len(cu_seqlens)-1 (packed) */
    const int64_t* cu_seqlens;       /* device INT64 [N+1], or NULL for fixed layout */
    const int64_t* cu_seqlens_host;  /* host INT64 [N+1] mirror, NULL iff cu_seqlens is NULL */
    float scale;                     /* 0 selects 1/sqrt(128); any other value must equal it */
    float lower_bound;               /* must be -5 */
    int32_t route;                   /* kda_route; AUTO unless testing a route */
    int32_t checkpoint_every;        /* tape interval in tokens; 0 selects 256; a multiple of 16 */
    int32_t context;                 /* kda_context: what the forward saves for the backward */
    int32_t precision;               /* kda_precision; AUTO unless testing */
    int32_t schedule;                /* kda_schedule; LONGEST_FIRST unless measuring */
} kda_problem;

/* Library version (KDA_VERSION). */
int kda_version(void);

/* Static text for a status code. */
const char* kda_status_string(kda_status status);

/* Text of the last failure on this thread ("" if none). */
const char* kda_last_error(void);

/* Bytes the forward context needs: with KDA_CONTEXT_TAPE the FP32 state tape
 * saved for the backward (one [Hv][128][128] slab per sequence and per
 * interval boundary strictly inside the sequence), with KDA_CONTEXT_RECORDS
 * the records of every 16-token chunk (an even number per sequence) and value
 * head; plus alignment.  Validates the problem. */
kda_status kda_fwd_ctx_bytes(const kda_problem* p, size_t* bytes);

/* Bytes the backward workspace needs (with KDA_CONTEXT_TAPE the chunk
 * records rebuilt from the tape; BF16 dq/dk partial sums when value heads
 * share a q/k head; FP32 parameter partial sums).  Validates the problem. */
kda_status kda_bwd_workspace_bytes(const kda_problem* p, size_t* bytes);

/* Host planning only (no device access): the route the forward would take,
 * the number of (sequence, value head) tasks, and optionally the task order
 * (longest sequence first; each entry is n * Hv + h) into order[0..cap).
 * Used by tests of the scheduler.  Page "flashinfer.kda.recurrent_kda",
 * parameter cu_seqlens: longer sequences are scheduled first. */
kda_status kda_plan_query(const kda_problem* p, int32_t* route, int64_t* num_tasks,
                          int32_t* order, int64_t cap);

/* Training forward (page "flashinfer.kda_training.recurrent_kda_training_
 * forward").  Writes o and final_state, and, when ctx is not NULL, the state
 * tape that kda_bwd consumes.  ctx may be NULL (ctx_bytes 0) when no backward
 * will follow.  Outputs must not overlap inputs, ctx or each other
 * ("flashinfer.kda_training", paragraph 1).  Asynchronous on `stream`. */
kda_status kda_fwd(const kda_problem* p,
                   const void* q, const void* k, const void* v, const void* g,
                   const void* beta, const float* A_log, const float* dt_bias,
                   const float* initial_state,
                   void* o, float* final_state,
                   void* ctx, size_t ctx_bytes, void* stream);

/* kda_fwd for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, checks, kernels and results as kda_fwd, but the schedule (task
 * order, sequence and tape offsets, segment list) goes into a static device
 * array of KDA_NOALLOC_SCRATCH_BYTES per device instead of library-allocated
 * memory, written by small kernel launches on `stream` that carry it as
 * arguments (no hipMalloc or hipFree, no pinned host memory, no memset or
 * copy; the schedule is assembled in a static host buffer, and only the
 * argument checks and the ordering use small C++ heap allocations, as in
 * kda_fwd).  A problem whose schedule needs more than
 * that (about 900k (sequence, value head) tasks) is refused with
 * KDA_ERR_WORKSPACE_SIZE before any device work.  Every call on a device
 * shares that device's array and overwrites it: calls that overlap on one
 * device (other streams or threads) race, so serialise them.  The context it
 * fills is accepted by kda_bwd like kda_fwd's. */
kda_status kda_fwd_noalloc(const kda_problem* p,
                           const void* q, const void* k, const void* v, const void* g,
                           const void* beta, const float* A_log, const float* dt_bias,
                           const float* initial_state,
                           void* o, float* final_state,
                           void* ctx, size_t ctx_bytes, void* stream);

/* Training backward (pages "flashinfer.kda_backward.recurrent_kda_backward"
 * and "flashinfer.kda_training", paragraph 5).  Takes the same problem and
 * input pointers as the kda_fwd that filled ctx (checked against the host
 * record of that call, together with the device and the stream: a context is
 * used on the stream that created it; any route may consume the tape, except
 * that the segment-parallel backward needs a segment-parallel forward), the
 * adjoints d_o and dfinal_state, and
 * writes the eight gradients.  dq/dk sum over the value heads that share a
 * q/k head; dA_log/ddt_bias sum over all sequences and tokens.  The
 * workspace is caller-owned scratch of kda_bwd_workspace_bytes() bytes.
 * Inputs must not have changed since the forward.  Asynchronous. */
kda_status kda_bwd(const kda_problem* p,
                   const void* q, const void* k, const void* v, const void* g,
                   const void* beta, const float* A_log, const float* dt_bias,
                   const float* initial_state,
                   const void* ctx, size_t ctx_bytes,
                   const void* d_o, const float* dfinal_state,
                   void* dq, void* dk, void* dv, void* dg, void* dbeta,
                   float* dA_log, float* ddt_bias, float* dinitial_state,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Inference forward (page "flashinfer.kda.recurrent_kda"): decode (one
 * token per sequence) and prefill on a BF16 state pool updated in place.
 * The shape fields mean what they mean in kda_problem.  The options follow
 * the page's parameters:
 *   use_qk_l2norm       nonzero: L2-normalise q and k (epsilon 1e-6);
 *                       zero: use them as given;
 *   use_gate_in_kernel  nonzero: per-channel decay
 *                       exp(lower_bound * sigmoid(exp(A_log) * (g + dt_bias)))
 *                       (A_log required, dt_bias NULL counts as zero);
 *                       zero: g is the log-space decay, applied as exp(g)
 *                       (A_log and dt_bias unused, may be NULL);
 *   lower_bound         with use_gate_in_kernel a finite negative value; 0
 *                       (unset) is refused, as the page's softplus form is
 *                       not implemented;
 *   beta_is_logit       nonzero: beta = sigmoid(input); zero: used as given.
 * scale: 0 selects 1/sqrt(128), otherwise any finite positive value.
 * The state pool is BF16 [pool_slots][Hv][128][128], value-first ([v][k]).
 * Sequence n starts from slot state_indices[n] (slot n when state_indices is
 * NULL, which needs pool_slots >= N) and its final state is rounded to BF16
 * and written back to that slot; other slots are not touched.  The indices
 * must be distinct and in [0, pool_slots): they are checked on the host
 * mirror state_indices_host (given iff state_indices is).
 * Layout: q, k [B][T][Hqk][128], v, g [B][T][Hv][128], beta [B][T][Hv] BF16;
 * A_log FP32 [Hv], dt_bias FP32 [Hv][128]; o BF16 [B][T][Hv][128].  The state
 * runs in FP32 between the pool's load and store.
 * route: KDA_ROUTE_ROWSPLIT (2) runs the token-serial kernel, exact for any
 * gate; KDA_ROUTE_CHUNK (1) runs the chunked MFMA kernel, which needs every
 * per-token log-decay to be >= -5, so it is accepted only for the in-kernel
 * gate with lower_bound >= -5 (a log-space gate given as is has no bound the
 * host can check; KDA_ERR_ROUTE); KDA_ROUTE_AUTO (0) takes the chunked kernel
 * for the in-kernel gate with lower_bound >= -5 when some sequence is longer
 * than one token, else the token-serial one.
 * State checkpoints (parameters state_checkpoints, checkpoint_cu_starts,
 * checkpoint_every_n_tokens): with checkpoint_every = E > 0 (a multiple of
 * 16), sequence n stores ceil(L_n / E) BF16 states [Hv][128][128] into rows
 * checkpoint_cu_starts[n] ... of state_checkpoints ([checkpoint_rows][Hv]
 * [128][128]): row j holds the state before token j*E, so the first is the
 * initial state.  The starts are device INT64 [N+1] with a host mirror that
 * is checked (first 0, each count ceil(L_n / E), last <= checkpoint_rows).
 * The kernels read the device copy; a row it places outside
 * [0, checkpoint_rows) is not stored.
 * With E = 0 the four checkpoint fields must be NULL / 0.
 * Speculative decode (parameters num_spec_tokens, num_accepted_tokens,
 * ssm_state_indices [N, 1+S]): with num_spec_tokens = S > 0 every sequence
 * has exactly 1+S tokens and state_indices holds 1+S distinct slots per
 * sequence (row-major [N][1+S]).  The initial state is read from slot
 * state_indices[n][a-1], a = num_accepted_tokens[n] clamped to [1, 1+S]
 * (a = 1 when num_accepted_tokens is NULL), and the state after token s is
 * written to slot state_indices[n][s].  Always the token-serial kernel; no
 * checkpoints.
 * Read-only source pool (parameters initial_state_source,
 * initial_state_indices): when state_source is given, sequence n starts from
 * slot source_indices[n] of that BF16 pool [source_slots][Hv][128][128]
 * instead of its slot in the state pool; the final (or per-token) states
 * still go to the state pool.  Source slots may repeat; they are checked on
 * the host mirror.
 * Asynchronous; capturable under the same condition as kda_fwd. */
typedef struct {
    int32_t B;
    int32_t T;
    int32_t Hqk;
    int32_t Hv;
    int32_t N;
    const int64_t* cu_seqlens;          /* device INT64 [N+1], or NULL for fixed layout */
    const int64_t* cu_seqlens_host;     /* host INT64 [N+1] mirror, NULL iff cu_seqlens is NULL */
    float scale;
    int32_t use_qk_l2norm;
    int32_t use_gate_in_kernel;
    float lower_bound;
    int32_t beta_is_logit;
    int32_t route;
    int64_t pool_slots;
    const int32_t* state_indices;       /* device INT32 [N], or NULL */
    const int32_t* state_indices_host;  /* host INT32 [N] mirror, NULL iff state_indices is NULL */
    int32_t checkpoint_every;           /* E: 0 (none) or a positive multiple of 16 */
    void* state_checkpoints;            /* BF16 [checkpoint_rows][Hv][128][128], or NULL */
    int64_t checkpoint_rows;
    const int64_t* checkpoint_cu_starts;       /* device INT64 [N+1], or NULL */
    const int64_t* checkpoint_cu_starts_host;  /* host mirror */
    int32_t num_spec_tokens;            /* S: 0 (plain decode / prefill) or > 0 */
    const int32_t* num_accepted_tokens; /* device INT32 [N], or NULL */
    const void* state_source;           /* BF16 [source_slots][Hv][128][128], or NULL */
    int64_t source_slots;
    const int32_t* source_indices;      /* device INT32 [N], with state_source */
    const int32_t* source_indices_host; /* host mirror */
} kda_infer_problem;

kda_status kda_infer(const kda_infer_problem* p,
                     const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const float* A_log, const float* dt_bias,
                     void* state_pool, void* o, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBKDA_H */
