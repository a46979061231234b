/*
 * loglin.h -- C ABI of the MI355X (gfx950) log-linear Mamba-2 forward.
 *
 * Operation (log-linear attention write-up, yoousoft.com/industry/3746,
 * section "special structure: tree partition", matrix form; section
 * "log-linear generalisation of Mamba-2"): for every batch b and head h,
 *
 *     O = (C B^T  (.)  M^H) X,
 *     M^H[t,s] = prod_{r=s+1..t} a_r * lambda[t, level(t,s)]  for s <= t, else 0,
 *     level(t,s) = 0 if s == t else 1 + floor(log2(t XOR s))   (Fenwick level),
 *
 * with C as the query, B as the key and X as the value (state space
 * duality section of the biyoush.com article on Transformers, RNNs and
 * Mamba-2).  Heads share B/C in consecutive groups: group(h) = h / (H/G).
 * No skip term, no dt scaling of X, no output gate.
 *
 * The work is split into chunks of `chunk` tokens (efficient training
 * algorithm section): a dense intra-chunk block for levels 0..log2(chunk),
 * and, for every higher level, chunk states combined by a Fenwick-ordered
 * scan and read back by one output pass fused across levels.
 *
 * Layouts (all row-major, innermost dimension last, densely packed):
 *   X      [batch, seqlen, nheads,  headdim]   io dtype
 *   B, C   [batch, seqlen, ngroups, dstate ]   io dtype
 *   log_a  [batch, seqlen, nheads]             float32, log of the decay a_t
 *   lambda [batch, seqlen, nheads,  nlevels]   io dtype, weight of level l
 *                                              for query position t
 *   out    [batch, seqlen, nheads,  headdim]   io dtype (bf16: round to
 *                                              nearest even from fp32)
 * Accumulation is fp32 for both io dtypes.  Levels >= ceil(log2 seqlen)+1
 * are ignored.
 *
 * Ownership: every pointer argument except `dims`/`opts` is a device
 * pointer owned by the caller.  The library keeps no pointer after a call
 * returns, allocates no device memory and has no global mutable state; it
 * is safe to call from several host threads on different streams.  (The
 * one exception is loglin_fwd_noalloc below, which uses a fixed scratch
 * array of the library instead of a caller's workspace.)
 *
 * Asynchrony: loglin_fwd only enqueues kernels on `stream` (a hipStream_t,
 * NULL = the default stream) and returns.  Device faults surface at the
 * caller's next synchronisation.  Results are deterministic: no atomics,
 * repeated calls on the same inputs are bit-identical.
 *
 * Errors: functions returning int return LOGLIN_OK (0) or a negative
 * LOGLIN_ERR_* code.  Every argument check runs on the host before any HIP
 * call, so an invalid call touches no device state.
 */
#ifndef LOGLIN_H_
#define LOGLIN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOGLIN_VERSION 1

typedef enum {
  LOGLIN_F32 = 0,
  LOGLIN_BF16 = 1
} loglin_dtype;

enum {
  LOGLIN_OK = 0,
  LOGLIN_ERR_NULL = -1,        /* a required pointer is NULL */
  LOGLIN_ERR_DIM = -2,         /* a dimension is <= 0 or too large */
  LOGLIN_ERR_CHUNK = -3,       /* chunk is not 16, 32 or 64 */
  LOGLIN_ERR_SEQ_CHUNK = -4,   /* seqlen is not a multiple of chunk */
  LOGLIN_ERR_GROUPS = -5,      /* nheads is not a multiple of ngroups */
  LOGLIN_ERR_LEVELS = -6,      /* nlevels < ceil(log2 seqlen) + 1 */
  LOGLIN_ERR_DTYPE = -7,       /* io_dtype is not a loglin_dtype */
  LOGLIN_ERR_WORKSPACE = -8,   /* workspace NULL or smaller than required */
  LOGLIN_ERR_ALIGN = -9,       /* a pointer is not 16-byte aligned */
  LOGLIN_ERR_SHAPE = -10,      /* (headdim, dstate) not supported */
  LOGLIN_ERR_HIP = -11,        /* a HIP call failed */
  LOGLIN_ERR_OPTS = -12,       /* an option is out of range */
  LOGLIN_ERR_SCRATCH = -13     /* workspace larger than loglin_fwd_noalloc's array */
};

/* Problem sizes.  headdim = P (value dim), dstate = N (state dim),
 * nlevels = L (weights per token and head).  Supported: headdim in
 * {16, 32, 64}; dstate in {32, 64, 128}, plus 16 for LOGLIN_F32.
 * Bounds of the 32-bit index arithmetic and the launch grids (else
 * LOGLIN_ERR_DIM): seqlen <= 2^30, nheads <= 4096, nlevels <= 64,
 * batch * nheads <= 65535, batch * nheads * (seqlen / chunk) <= 2^30, and
 * at most 2^16 segments of 2^seg_log2 chunks (seqlen / chunk <= 2^19 at the
 * default depth of 8 chunks per segment). */
typedef struct {
  int64_t batch;
  int64_t seqlen;
  int64_t nheads;
  int64_t ngroups;
  int64_t headdim;
  int64_t dstate;
  int64_t nlevels;
  int32_t io_dtype; /* loglin_dtype */
  int32_t reserved; /* must be 0 */
} loglin_dims;

/* Number of timing points loglin_fwd_ex records when opts->stage_events is
 * set: before the chunk-state pass, before the level scan, before the
 * output pass, and after it. */
#define LOGLIN_NUM_STAGES 3

/* Optional knobs; pass NULL for defaults. */
typedef struct {
  /* log2 of the chunks per segment: the state pass reduces each segment to
   * one state and the output pass keeps the levels inside a segment on
   * chip.  -1 lets the library choose (min(3, ceil(log2(seqlen/chunk)))).
   * Valid: 0 <= seg_log2 <= min(3, ceil(log2(seqlen/chunk))). */
  int32_t seg_log2;
  /* Heads served by one work-group of the output pass.  2: two heads of the
   * same group share the group's B and C rows and the scores C B^T; needs
   * bf16, headdim 64 and an even number of heads per group (nheads /
   * ngroups), else LOGLIN_ERR_OPTS.  0 or 1: one head (the default). */
  int32_t heads_per_block;
  /* NULL, or LOGLIN_NUM_STAGES + 1 events (hipEvent_t) recorded on
   * `stream` at the stage boundaries, for per-pass timing. */
  void* const* stage_events;
  /* Levels the output includes: bit l set keeps level l (0 = all levels).
   * The excluded levels' terms are skipped, not computed and zeroed, so a
   * pass per level ("naive", unfused) can be timed against the fused one. */
  uint64_t level_mask;
} loglin_opts;

/* Bytes of device workspace loglin_fwd needs for these sizes (may be 0).
 * Returns 0 as well when the arguments are invalid; loglin_fwd then
 * reports the error. */
size_t loglin_workspace_bytes(const loglin_dims* dims, int chunk);
size_t loglin_workspace_bytes_ex(const loglin_dims* dims, int chunk,
                                 const loglin_opts* opts);

/* Enqueue the forward pass.  X, B, C, log_a, lambda, out and workspace are
 * device pointers, 16-byte aligned; `out` must not alias an input.  The
 * workspace (at least loglin_workspace_bytes bytes, contents ignored on
 * entry) must not be used by other work until the call's kernels finish. */
int loglin_fwd(const void* X, const void* B, const void* C,
               const float* log_a, const void* lambda, int chunk, void* out,
               const loglin_dims* dims, void* workspace,
               size_t workspace_bytes, void* stream);

int loglin_fwd_ex(const void* X, const void* B, const void* C,
                  const float* log_a, const void* lambda, int chunk,
                  void* out, const loglin_dims* dims, void* workspace,
                  size_t workspace_bytes, void* stream,
                  const loglin_opts* opts);

/* Host-only argument check: the same checks loglin_fwd runs first.
 * Pointers are only tested for NULL and alignment, never dereferenced. */
int loglin_validate(const void* X, const void* B, const void* C,
                    const float* log_a, const void* lambda, int chunk,
                    const void* out, const loglin_dims* dims,
                    const void* workspace, size_t workspace_bytes,
                    const loglin_opts* opts);

/* Static description of an error code (never NULL). */
const char* loglin_strerror(int code);

/* Segment depth (log2 chunks per segment) the library would use; negative
 * error code on invalid arguments.  Host only. */
int loglin_plan_seg_log2(const loglin_dims* dims, int chunk,
                         const loglin_opts* opts);

/* ---- Forward without allocation -----------------------------------------
 *
 * For callers that cannot allocate device memory or pass a workspace:
 * code under HIP graph or stream capture, tight serving loops, and hosts
 * that forbid allocation while a step runs.  loglin_fwd_noalloc computes
 * exactly what loglin_fwd computes (the same kernels; outputs are
 * bit-identical) with its workspace in a fixed array of device memory of
 * LOGLIN_NOALLOC_SCRATCH_MIB MiB that the library holds, one copy per GPU,
 * from the first call on that GPU until the process ends.  That covers
 * loglin_workspace_bytes up to 192 MiB: the 32K-token, 48-head, P=64,
 * N=128 bf16 workload needs about 101 MB.  Larger problems return
 * LOGLIN_ERR_SCRATCH (checked on the host before any HIP call, like every
 * other argument error); loglin_noalloc_scratch_bytes gives the limit.
 *
 * The call makes no device allocation.  Its first call on a GPU looks up
 * the array's address on that GPU (hipGetSymbolAddress); later calls reuse
 * it.  The array belongs to the current device: `stream` must be a stream
 * of the current device (or NULL).  Every call on a GPU shares that GPU's
 * array, whose contents the forward never needs cleared: calls whose
 * kernels overlap on one GPU (different streams, or host threads without
 * ordering) race on it and must be serialised by the caller.  Other
 * arguments, layouts and errors as for loglin_fwd. */
#define LOGLIN_NOALLOC_SCRATCH_MIB 192

size_t loglin_noalloc_scratch_bytes(void);

int loglin_fwd_noalloc(const void* X, const void* B, const void* C,
                       const float* log_a, const void* lambda, int chunk,
                       void* out, const loglin_dims* dims, void* stream);

/* ---- One-token decode (Fenwick recurrence) -------------------------------
 *
 * Operation (log-linear attention write-up, section "log-linear attention"
 * and "special structure: tree partition"): decoding keeps one N x P state
 * per Fenwick bucket of the prefix, O(log T) of them.  Step t (t = 0, 1, ...)
 * merges the buckets of levels 0..z into level z+1 (z = trailing zeros of
 * t, t > 0), decays every older bucket by a_t, starts level 0 with
 * B_t X_t^T and returns, for every batch entry and head,
 *
 *     out_t = sum_l lambda[t, l] S_l^T C_t,
 *
 * which equals row t of loglin_fwd's output for the same inputs.
 *
 * dims: as for loglin_fwd, with seqlen the number of positions the state
 * can hold (steps t = 0 .. seqlen - 1) and nlevels >= ceil(log2 seqlen) + 1.
 * Layouts (row-major, one token):
 *   X      [batch, nheads, headdim]    io dtype
 *   B, C   [batch, ngroups, dstate]    io dtype
 *   log_a  [batch, nheads]             float32
 *   lambda [batch, nheads, nlevels]    io dtype
 *   out    [batch, nheads, headdim]    io dtype
 * state: loglin_decode_state_bytes bytes of device memory owned by the
 * caller, 256-byte aligned, reused across the steps of one sequence
 * (batch).  Step 0 initialises it (no clearing needed); steps must run in
 * order t = 0, 1, 2, ... on one stream.  Other pointers: device pointers,
 * `out` 16-byte aligned, the inputs aligned to their element size.  Errors
 * as for loglin_fwd; t outside [0, seqlen) is LOGLIN_ERR_DIM. */
size_t loglin_decode_state_bytes(const loglin_dims* dims);

int loglin_decode_step(void* state, int64_t t, const void* X, const void* B,
                       const void* C, const float* log_a, const void* lambda,
                       void* out, const loglin_dims* dims, void* stream);

/* ---- Backward pass -------------------------------------------------------
 *
 * Operation: the gradients of loglin_fwd's O = (C B^T ⊙ M^H) X (log-linear
 * attention write-up, sections "special structure: tree partition" and
 * "efficient training algorithm"; the write-up names the backward pass but
 * prints no formula, so these are the calculus of that definition) for an
 * upstream gradient dO, with S = C B^T, D = dO X^T and M = M^H:
 *
 *     dX_s = sum_t (M ⊙ S)[t, s] dO_t        dB_s = sum_t (M ⊙ D)[t, s] C_t
 *     dC_t = sum_s (M ⊙ D)[t, s] B_s         dlambda[t, l] = dO_t . Y_t^(l)
 *     dlog_a_r = sum over t >= r, s < r of (M ⊙ S ⊙ D)[t, s]
 *
 * where Y^(l) is the output with lambda one-hot on level l; dB and dC sum
 * over the heads of each group.
 *
 * Inputs as for loglin_fwd (same dims, chunk and layouts), plus
 *   dO      [batch, seqlen, nheads, headdim]   io dtype
 * Outputs (written, not accumulated):
 *   dX      [batch, seqlen, nheads, headdim]   io dtype
 *   dB, dC  [batch, seqlen, ngroups, dstate]   io dtype
 *   dlog_a  [batch, seqlen, nheads]            float32
 *   dlambda [batch, seqlen, nheads, nlevels]   io dtype (0 on levels
 *                                              >= ceil(log2 seqlen) + 1)
 * All pointers are device pointers owned by the caller, 16-byte aligned;
 * outputs must not alias inputs or each other.  Accumulation is fp32 and
 * every output is written once, by one thread (no atomics): repeated calls
 * are bit-identical.
 *
 * Supported: bf16 with chunk 32 or 64, headdim 32 or 64, dstate 32..128;
 * float32 with chunk 16..64 and the forward's (headdim, dstate) pairs
 * except headdim 64 with dstate 128 at chunk 64 (LDS); otherwise
 * LOGLIN_ERR_SHAPE.  Size bounds as for loglin_fwd (seqlen <= 2^30, at most
 * 2^19 chunks), else LOGLIN_ERR_DIM.
 * Errors as for loglin_fwd, all
 * checked on the host before any HIP call.  The workspace (at least
 * loglin_bwd_workspace_bytes bytes, 256-byte aligned, contents ignored on
 * entry) must not be used by other work until the call's kernels finish. */
size_t loglin_bwd_workspace_bytes(const loglin_dims* dims, int chunk);

int loglin_bwd(const void* X, const void* B, const void* C,
               const float* log_a, const void* lambda, const void* dO,
               int chunk, void* dX, void* dB, void* dC, float* dlog_a,
               void* dlambda, const loglin_dims* dims, void* workspace,
               size_t workspace_bytes, void* stream);

/* ---- Log-linear gated DeltaNet forward -----------------------------------
 *
 * Operation (log-linear attention write-up, section "log-linear
 * generalisation of Mamba-2 and gated DeltaNet": each model keeps its own
 * transition and composes its attention mask with the log-linear mask):
 * gated DeltaNet's transition A_t = alpha_t (I - beta_t k_t k_t^T) acts on
 * every Fenwick level state, the token enters level 0 as beta_t k_t v_t^T,
 * and o_t = sum_l lambda[t, l] S_t^(l)^T q_t.  Equivalently, per batch and
 * head, O = (G ⊙ M^H) V with
 *   G[t, s] = beta_s (prod_{r=s+1..t} alpha_r) q_t^T H_t ... H_{s+1} k_s,
 *   H_r = I - beta_r k_r k_r^T,  M^H[t, s] = lambda[t, bit_length(t xor s)].
 *
 * dims: ngroups must equal nheads (one query and key per head); dstate N
 * is the key dimension (16, 32, 64 or 128), headdim P the value dimension
 * (16, 32 or 64); seqlen a multiple of 32 and at most 2^20; nlevels >=
 * ceil(log2 seqlen) + 1.  Layouts (row-major, contiguous):
 *   q, k      [batch, seqlen, nheads, dstate]   io dtype
 *   v, out    [batch, seqlen, nheads, headdim]  io dtype
 *   log_alpha [batch, seqlen, nheads]           float32 (alpha = exp)
 *   beta      [batch, seqlen, nheads]           float32
 *   lambda    [batch, seqlen, nheads, nlevels]  io dtype
 * All device pointers, 16-byte aligned, owned by the caller; `out` must not
 * alias an input.  The workspace (at least loglin_gdn_workspace_bytes
 * bytes, 256-byte aligned, contents ignored on entry; about 48 KB per
 * head and 32 tokens at key dim 128, value dim 64) holds the per-chunk
 * operands between the chunk-parallel pass and the level pass and must not
 * be used by other work until the call's kernels finish.  Accumulation is
 * fp32; repeated calls are bit-identical.  Keys are used as given (the
 * delta rule is stable for unit-norm keys and beta in [0, 2]).  Errors as
 * for loglin_fwd, checked on the host before any HIP call. */
size_t loglin_gdn_workspace_bytes(const loglin_dims* dims);

int loglin_gdn_fwd(const void* q, const void* k, const void* v,
                   const float* log_alpha, const float* beta,
                   const void* lambda, void* out, const loglin_dims* dims,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Event helpers for callers that time stages without linking HIP
 * themselves.  *event receives a hipEvent_t with timing enabled. */
int loglin_event_create(void** event);
int loglin_event_destroy(void* event);
int loglin_event_elapsed_ms(void* start, void* stop, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* LOGLIN_H_ */
