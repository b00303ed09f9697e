/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA library: the Kimi Delta Attention
 * chunked forward and the one-token paged decode.
 *
 * What is computed.  For each sequence n, value head h and token t (query/key
 * head hq = h / (Hv / Hqk): contiguous groups of Hv / Hqk value heads share one
 * query/key head), with K = V = 128:
 *
 *   qn = q / sqrt(sum(q^2) + 1e-6),  kn likewise       (when use_qk_l2norm)
 *   b  = sigmoid(beta)                                   (beta is a logit)
 *   S  = (I - b kn kn^T) diag(exp(g)) S + b kn v^T       (S is K x V)
 *   o  = scale * S^T qn                                  (after the write)
 *
 * g is a natural-log decay per key channel, expected in [-5, 0] per token
 * (the default lower bound of the gate); results for larger |g| are
 * unspecified.  States cross this interface "V-first": a state buffer
 * [.., 128 (V), 128 (K)] holds S[k][v] at element [v][k].
 *
 * Sources (pages, by title):
 *  - "mate.kda" (MATE 0.2.5): chunk_kda's argument set, shapes and checks
 *    (D = 128, GVA divisibility, beta shape, dtype equality, default scale
 *    128^-0.5, optional initial/final state, varlen cu_seqlens with B = 1);
 *    gated_delta_rule_decode's V-first state pool [pool, HV, V, K], the in
 *    place final state, and state_indices smaller than the pool size.
 *  - "vllm.models.kimi_k3.amd.ops.kda_chunk": fused_kda_chunk's paged state
 *    (state_cache / state_indices / has_initial_state replacing the initial
 *    and final state), the caller-owned group workspace, and 64-token chunks
 *    that restart at every sequence start.
 *  - "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify" (KdaTcVerify):
 *    the L2-norm epsilon, the sigmoid of the raw beta, and a null slot that
 *    produces zero output without touching the state.
 *
 * Conventions shared by every entry point.
 *  - Pointers marked (device) are HIP device pointers on the current device;
 *    (host) pointers are read before the call returns.  All tensors are
 *    dense, row-major and contiguous, and every tensor starts on a 16-byte
 *    boundary (KDA_ERR_ARG otherwise); beta, A_log and index arrays are exempt.
 *  - The library allocates nothing.  Every buffer, the workspace included,
 *    is owned by the caller and must outlive the queued work.
 *  - Arguments are checked on the host before anything is queued.  On an
 *    error nothing is launched, nothing is written, and a status other than
 *    KDA_OK comes back; kda_last_error() then holds a message for the
 *    calling thread.  Values that live in device memory (cu_seqlens,
 *    state_indices, has_initial_state) cannot be checked without a sync and
 *    are the caller's contract, as stated per field.
 *  - Work is queued asynchronously on `stream` (a hipStream_t; NULL = the
 *    default stream).  A launch failure returns KDA_ERR_HIP.
 *  - Outputs must not overlap inputs.  The only buffer updated in place is
 *    the paged state cache.
 *  - Calls are reentrant; two calls may run concurrently on different
 *    streams as long as they share no output, cache row or workspace.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128   /* K = V = 128, the only head size (chunk_kda's D) */
#define KDA_CHUNK 64       /* tokens per chunk of the chunked form */

/* Element type of q, k, v, g, beta and out (one type for all of them). */
typedef enum kda_dtype {
  KDA_F32 = 0,   /* fp32 inputs; MFMA operands carried as split bf16 pairs */
  KDA_BF16 = 1,  /* bf16 inputs; bf16 MFMA with fp32 accumulation */
  KDA_F16 = 2    /* fp16 inputs; the chunked forward runs them on its fp32
                    kernels (widened exactly, split MFMA operands) */
} kda_dtype;

typedef enum kda_status {
  KDA_OK = 0,
  KDA_ERR_SHAPE = 1,       /* inconsistent sizes (chunk_kda raises ValueError) */
  KDA_ERR_DTYPE = 2,       /* unsupported element type (TypeError) */
  KDA_ERR_UNSUPPORTED = 3, /* a valid request this library does not serve */
  KDA_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  KDA_ERR_HIP = 5,         /* the HIP runtime refused a launch */
  KDA_ERR_ARG = 6          /* a required pointer is NULL, or a bad struct */
} kda_status;

/* Execution plan of the chunked forward. */
typedef enum kda_path {
  KDA_PATH_AUTO = 0,    /* the library picks (today KDA_PATH_FUSED) */
  KDA_PATH_STAGED = 1,  /* prep -> wy -> walk, intermediates in the workspace */
  KDA_PATH_FUSED = 2,   /* prep folded into the WY kernel (one pass over q, k,
                           g) -> walk; same intermediates, same results */
  KDA_PATH_ONCHIP = 3   /* bf16 only: the intra-chunk stage is recomputed
                           inside the walk per chunk, in LDS; HBM carries only
                           inputs, outputs and states, and the workspace holds
                           only the chunk table and the group-scan planes */
} kda_path;

/*
 * kda_chunk_args -- the chunked forward (chunk_kda's problem statement).
 *
 * Token layout: varlen, T_tot = total_tokens rows.  Sequence n owns rows
 * [cu_seqlens[n], cu_seqlens[n+1]).  With cu_seqlens == NULL the batch is
 * dense: num_seqs sequences of total_tokens / num_seqs rows each.
 */
typedef struct kda_chunk_args {
  size_t struct_size;          /* = sizeof(kda_chunk_args) */
  const void *q;               /* (device) [T_tot, Hqk, 128] dtype */
  const void *k;               /* (device) [T_tot, Hqk, 128] dtype */
  const void *v;               /* (device) [T_tot, Hv, 128] dtype */
  const void *g;               /* (device) [T_tot, Hv, 128] dtype, log-decay <= 0 */
  const void *beta;            /* (device) [T_tot, Hv] dtype, logits */
  int32_t dtype;               /* kda_dtype: KDA_F32, KDA_BF16 or KDA_F16 */
  int32_t num_seqs;            /* N >= 0 */
  int64_t total_tokens;        /* T_tot >= 0; KDA_ERR_UNSUPPORTED above 2^31 - 1, or when
                                  (T_tot / 64 + num_seqs) * hv is */
  const int32_t *cu_seqlens;   /* (device) [N+1] non-decreasing, cu[0] = 0,
                                  cu[N] = T_tot; or NULL (dense) */
  int32_t hqk, hv;             /* heads; hv % hqk == 0 */
  float scale;                 /* output scale (128^-0.5 is the usual value) */
  int32_t use_qk_l2norm;       /* 1: L2-normalise q and k in the kernels */
  /* dense state mode (both optional, fp32, V-first) */
  const void *initial_state;   /* (device) [N, Hv, 128, 128] of state_dtype, or
                                  NULL (= zero) */
  void *final_state;           /* (device) [N, Hv, 128, 128] of state_dtype, or NULL */
  /* paged state mode (replaces initial_state / final_state) */
  float *state_cache;          /* (device) [num_slots, Hv, 128, 128] or NULL */
  const int32_t *state_indices;     /* (device) [N]; row per sequence, distinct;
                                       < 0 = no state I/O for that sequence */
  const uint8_t *has_initial_state; /* (device) [N]; 0 = start from zero */
  int32_t num_slots;           /* rows of state_cache (> every index used) */
  void *out;                   /* (device) [T_tot, Hv, 128] dtype */
  void *workspace;             /* (device) >= kda_chunk_fwd_workspace_size() */
  size_t workspace_bytes;
  int32_t path;                /* kda_path */
  int32_t groups;              /* chunk groups per sequence: 0 = auto, 1 = none,
                                  >= 2 = that many (the parallel group scan) */
  int32_t walk_waves;          /* waves per walk workgroup: 0 = auto, else 2, 4
                                  or 8 (a tuning knob; results do not change) */
  void **stage_events;         /* optional hipEvent_t[num_stage_events], recorded
                                  on `stream` at the stage boundaries below
                                  (profiling); NULL = none, and a NULL entry skips
                                  its boundary.  The caller owns them. */
  int32_t num_stage_events;
  void *stream;                /* hipStream_t or NULL */
  /* Gate parameters (optional; both or neither).  With them, g holds a raw
     gate and the log-decay of a step is
       lower_bound * sigmoid(exp(A_log[h]) * (g + dt_bias[h][c]))
     (the activation of KdaTcVerify, page
     "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify"; chunk_kda of page
     "mate.kda" takes A_log, dt_bias and lower_bound = -5 by default).
     lower_bound must lie in [-5, 0] (KDA_ERR_UNSUPPORTED otherwise), which
     keeps every step log-decay in the [-5, 0] range stated above. */
  const float *A_log;          /* (device) [Hv] fp32, or NULL */
  const void *dt_bias;         /* (device) [Hv, 128] of dt_bias_dtype, or NULL */
  int32_t dt_bias_dtype;       /* KDA_F32 or KDA_BF16 */
  float lower_bound;
  /* Mid-prefill state snapshots (optional; fused_kda_chunk's checkpoint
     arguments on page "vllm.models.kimi_k3.amd.ops.kda_chunk").  For a
     sequence n with 0 < checkpoint_offsets[n] <= its length and a multiple of
     64, the state after its first checkpoint_offsets[n] tokens is written
     (V-first) to row checkpoint_state_indices[n] of checkpoint_state (row n
     when the index array is NULL).  A 0, unaligned or too large offset, a row
     outside [0, checkpoint_rows), and a sequence with a null state slot in
     paged mode skip the snapshot (the row is left as it is). */
  float *checkpoint_state;     /* (device) [checkpoint_rows, Hv, 128, 128] fp32 or NULL */
  const int32_t *checkpoint_offsets;       /* (device) [N]; with checkpoint_state */
  const int32_t *checkpoint_state_indices; /* (device) [N] or NULL */
  int32_t checkpoint_rows;
  /* Storage of initial_state / final_state, or of the paged state_cache:
     KDA_F32 (0) or the input dtype (chunk_kda's rule on page "mate.kda": the
     states are fp32 or of q's dtype, both alike), and not fp16
     (KDA_ERR_UNSUPPORTED).  A bf16 start state is widened exactly; the final
     state is rounded to nearest even.  The checkpoint rows are always fp32. */
  int32_t state_dtype;
  /* Input strides (optional), in elements between consecutive tokens of
     q, k, v, g and beta; 0 means dense (hqk*128 for q and k, hv*128 for v
     and g, hv for beta).  Heads stay 128 elements apart inside a token (1
     for beta).  This serves views into a wider fused projection output,
     whose beta and g slices keep the projection's row stride and whose q
     may be a band view (fused_kda_prologue, page
     "vllm.models.kimi_k3.amd.ops.kda_chunk").  A nonzero stride is at least
     the dense one and at most 2^24; for q, k, v and g it also keeps every
     token row 16-byte aligned (a multiple of 16 bytes). */
  int64_t q_stride, k_stride, v_stride, g_stride, beta_stride;
  /* Elements between consecutive slots of the paged state pool (0: dense,
     hv*128*128).  Pools whose slots are padded to a cache page pass the
     padded stride (KdaTcVerify's state layout, page
     "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify"): at least
     hv*128*128 and a multiple of 8 elements. */
  int64_t state_slot_stride;
  /* Planning hint (optional): the longest sequence's token count, or 0 when
     unknown (cu_seqlens lives on the device).  It only steers the choice of
     chunk groups and walk width; results do not depend on it.  Without it a
     varlen batch is planned as if its sequences were equally long. */
  int64_t max_seqlen;
} kda_chunk_args;

/* Stage boundaries of kda_chunk_fwd (indices into stage_events).  Event i is
 * recorded when stage i ends; KDA_EV_BEGIN precedes the first kernel.  With
 * groups > 1 the walk runs as pass one, compose and pass two; with groups == 1
 * the compose and pass-two events are recorded right after the walk. */
enum {
  KDA_EV_BEGIN = 0,    /* before the chunk table */
  KDA_EV_TABLE = 1,    /* chunk table built */
  KDA_EV_PREP = 2,     /* prep done (qg, kg_t, decay) */
  KDA_EV_WY = 3,       /* WY done (w, u, aqk) */
  KDA_EV_WALK = 4,     /* walk (or group pass one) done */
  KDA_EV_COMPOSE = 5,  /* group transfers composed */
  KDA_EV_PASS2 = 6,    /* group pass two done */
  KDA_NUM_EVENTS = 7
};

/*
 * Workspace bytes the call described by `a` needs (0 is possible), written
 * to *bytes.  Reads only sizes and the path/groups fields.
 */
kda_status kda_chunk_fwd_workspace_size(const kda_chunk_args *a, size_t *bytes);

/*
 * The chunked forward.  Writes out; writes final_state (dense mode) or the
 * state_cache rows of the listed sequences (paged mode: read when
 * has_initial_state[n] != 0, then overwritten with the final state).  A
 * sequence of length 0 passes its start state through unchanged.  In paged
 * mode a sequence with state_indices[n] < 0 gets zero output rows and no
 * state I/O.  Chunks are 64 tokens from each sequence start; the last chunk
 * of a sequence may be shorter.
 */
kda_status kda_chunk_fwd(const kda_chunk_args *a);

/*
 * kda_chunk_fwd_noalloc -- kda_chunk_fwd for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation, arguments and results, but
 * a->workspace and a->workspace_bytes are ignored.  The workspace is a static
 * device array of the library, 64 MiB per device (allocated when the library's
 * code object loads on a device and held until the process ends); a call
 * whose kda_chunk_fwd_workspace_size() exceeds it returns KDA_ERR_WORKSPACE
 * and queues nothing.  Every call on one device shares that array: calls
 * whose queued work overlaps on one device (two streams, or two threads)
 * race and corrupt each other's results; serialise them.  The library makes
 * no hipMalloc / hipFree or allocating library call on this path; the array
 * needs no clearing between calls (each call initialises what it reads).
 */
kda_status kda_chunk_fwd_noalloc(const kda_chunk_args *a);

/*
 * Layout of the staged path's intermediates inside the workspace, for tests
 * and tools.  Offsets are in bytes from the workspace base; "chunks" is the
 * bound n_chunks_max = total_tokens / 64 + num_seqs used for sizing.  G is the
 * inclusive in-chunk cumulative log-decay, b = sigmoid(beta).
 *   chunk_offsets  int32 [N + 1]: first chunk index of each sequence, then
 *                  int32 [N]: the sequences in decreasing chunk count (in
 *                  quarter-octave classes; the walks start the longest
 *                  chains first)
 *   zero           1 KiB of zeros (source of the rows past a short chunk),
 *                  then a work counter of the WY kernel (int32) and, at
 *                  byte 1040, the longest sequence's chunk count (int32)
 *   table          int32x4 [chunks]: (sequence, first token, length, 0) per
 *                  chunk, length 0 past the last chunk
 *   qg             [T_tot, Hv, 128]  qn * exp(G)                        (P)
 *   kg_t           [chunks, Hv, 128, 64]  (kn * exp(G_last - G))^T      (P)
 *   decay          fp32 [chunks, Hv, 128]: exp(G_last)
 *   w              [T_tot, Hv, 128]  T (b kn exp(G)), T = (I + A_kk)^-1  (P)
 *   u              [chunks, Hv, 128 (v), 64 (t)]  (T (b v))^T           (P)
 *   aqk            [T_tot, Hv, 64]   sum_c qn_t kn_i exp(G_t - G_i), i <= t
 *                                    inside the chunk, 0 above         (P)
 *   scan           fp32 [G, N, Hv, 3, 128, 128] when the walk runs as a
 *                  group scan (G = groups > 1), else empty: per chunk group,
 *                  the transfer (plane 0, [k][j]), the partial state from zero
 *                  and the group's start state (planes 1 and 2, [v][k]); the
 *                  last group's planes 0 and 1 are not written (unused)
 * groups and walk_waves report the launch plan that kda_chunk_fwd takes for
 * these arguments (the chosen values when the arguments leave them at 0).
 * (P): the last axis is stored in MFMA fragment order: inside each block of
 * 32 elements, position 8 g + j holds element 4 g + j for j < 4 and
 * 16 + 4 g + (j - 4) for j >= 4.  Token axes of a short chunk are zero past
 * its length.  Element type: bf16 for KDA_BF16 inputs, fp32 for KDA_F32 and
 * KDA_F16 inputs.
 */
typedef struct kda_ws_layout {
  size_t chunk_offsets, zero, table, qg, kg_t, decay, w, u, aqk, scan, total;
  int64_t max_chunks;
  int32_t groups, walk_waves;
} kda_ws_layout;
kda_status kda_chunk_ws_layout(const kda_chunk_args *a, kda_ws_layout *layout);

/*
 * kda_decode_args -- one token per request over a paged state cache, state
 * updated in place (gated_delta_rule_decode's in-place V-first fp32 case).
 */
typedef struct kda_decode_args {
  size_t struct_size;          /* = sizeof(kda_decode_args) */
  const void *q;               /* (device) [n, Hqk, 128] dtype */
  const void *k;               /* (device) [n, Hqk, 128] dtype */
  const void *v;               /* (device) [n, Hv, 128] dtype */
  const void *g;               /* (device) [n, Hv, 128] dtype, log-decay (or
                                  the raw gate with A_log / dt_bias) */
  const void *beta;            /* (device) [n, Hv] dtype, logits */
  int32_t dtype;               /* kda_dtype */
  int32_t n;                   /* requests >= 0 */
  int32_t hqk, hv;             /* hv % hqk == 0 */
  float scale;
  int32_t use_qk_l2norm;
  void *state_cache;           /* (device) [num_slots, Hv, 128, 128] of
                                  state_dtype */
  const int32_t *state_indices;  /* (device) [n], distinct where >= 0, each
                                    < num_slots; < 0 = skip (zero output row,
                                    no state I/O); NULL = identity (slot n) */
  int32_t num_slots;
  void *out;                   /* (device) [n, Hv, 128] dtype */
  void *stream;                /* hipStream_t or NULL */
  /* Gate parameters (optional; both or neither).  With them, g holds a raw
     gate and the log-decay of a step is
       lower_bound * sigmoid(exp(A_log[h]) * (g + dt_bias[h][c]))
     (the activation of KdaTcVerify, page
     "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify"; the same form as
     the chunked forward).
     lower_bound must lie in [-5, 0] (KDA_ERR_UNSUPPORTED otherwise), which
     keeps every step log-decay in the [-5, 0] range stated above. */
  const float *A_log;          /* (device) [Hv] fp32, or NULL */
  const void *dt_bias;         /* (device) [Hv, 128] of dt_bias_dtype, or NULL */
  int32_t dt_bias_dtype;       /* KDA_F32 or KDA_BF16 */
  float lower_bound;
  /* Multi-token (speculative) decode, optional: gated_delta_rule_decode's
     [B, T] state_indices and num_accepted_tokens (page "mate.kda").  With
     tokens = T in [2, 8] (0 or 1: one token) q, k, v, g carry T tokens per
     request ([n, T, H, 128], beta [n, T, Hv], out [n, T, Hv, 128]).  With
     state_index_cols > 0 (>= T) state_indices is [n, state_index_cols]:
     request n starts from row state_indices[n][a - 1], a =
     num_accepted_tokens[n] (column 0 when that array is NULL), runs its
     tokens in order and after token t writes its state to row
     state_indices[n][t] when 0 <= that index < num_slots.  A start row
     outside [0, num_slots) or a count outside [1, state_index_cols] skips the
     request (zero output rows, no state traffic).  T > 1 and
     num_accepted_tokens need the 2-D index array. */
  int32_t tokens;
  int32_t state_index_cols;            /* 0: state_indices is [n] (or NULL) */
  const int32_t *num_accepted_tokens;  /* (device) [n] or NULL */
  /* Storage of state_cache: KDA_F32 (0) or KDA_BF16.  A bf16 state is
     widened for each token's arithmetic and rounded back (to nearest even)
     after each token, as repeated single-token decode would store it
     (gated_delta_rule_decode's bf16 state, page "mate.kda"). */
  int32_t state_dtype;
  /* Input strides (optional), in elements between consecutive tokens of
     q, k, v, g and beta (token n*T + t with T tokens per request); 0 means
     dense (hqk*128 for q and k, hv*128 for v
     and g, hv for beta).  Heads stay 128 elements apart inside a token (1
     for beta).  This serves views into a wider fused projection output,
     whose beta and g slices keep the projection's row stride and whose q
     may be a band view (fused_kda_prologue, page
     "vllm.models.kimi_k3.amd.ops.kda_chunk").  A nonzero stride is at least
     the dense one and at most 2^24; for q, k, v and g it also keeps every
     token row 16-byte aligned (a multiple of 16 bytes). */
  int64_t q_stride, k_stride, v_stride, g_stride, beta_stride;
  /* Elements between consecutive slots of state_cache (0: dense,
     hv*128*128).  Pools whose slots are padded to a cache page pass the
     padded stride (KdaTcVerify's state layout, page
     "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify"): at least
     hv*128*128 and a multiple of 8 elements. */
  int64_t state_slot_stride;
} kda_decode_args;

kda_status kda_decode(const kda_decode_args *a);

/*
 * kda_verify_args -- the record-based speculative verify step (KdaTcVerify,
 * page "vllm.models.kimi_k3.nvidia.recoverssm.cutedsl.verify": its argument
 * list, the window closed form of its step 4 and its corr / kg records).
 *
 * Request b owns token rows [query_start[b], query_start[b+1]) of q, k, v,
 * g, beta and out, at most `window` of them (rows past the window are not
 * read and their out rows are left as they are).  From the state S0 in slot
 * state_indices[b] (read only) each (request, value head) runs its tokens
 * with, over the window, the inclusive cumulative log-decay cum_t, the
 * (optionally L2-normalised) query qn_t and key kn_t, and b_t = sigmoid(beta):
 *   probes   p_t = e^cum_t kn_t,  r_t = scale e^cum_t qn_t,  w_i = e^-cum_i kn_i
 *   u_t = b_t (v_t - S0^T p_t - sum_{i<t} (w_i . p_t) u_i)
 *   o_t = S0^T r_t + sum_{i<=t} (w_i . r_t) u_i
 * (S0^T p: the V-first rows of S0 dotted with p), which equals the token
 * recurrence.  It writes out and the records, and no state:
 *   corr[b][h][t][:]        = u_t (fp32, 128 value channels)
 *   kg[b][h][t][0 .. 127]   = the raw key k_t of the head's query-key head
 *   kg[b][h][t][128 .. 255] = the raw gate g_t,
 * both in the input dtype, for t below the request's token count; record
 * rows past it are left as they are.  A slot outside [0, num_slots) gives zero
 * out rows and writes no records.  The step log-decays must lie in [-5, 0]
 * (the gate parameters guarantee it), so that e^(+-cum) stays inside fp32 over
 * 8 tokens.
 *
 * Errors: KDA_ERR_ARG (NULL args or pointer, bad struct_size, misaligned
 * base), KDA_ERR_DTYPE, KDA_ERR_SHAPE (heads, window outside [1, 8], slots,
 * strides), KDA_ERR_UNSUPPORTED (sizes past 2^31, lower_bound outside
 * [-5, 0]); nothing is queued on error.  Asynchronous on `stream`.
 */
typedef struct kda_verify_args {
  size_t struct_size;          /* = sizeof(kda_verify_args) */
  const void *q;               /* (device) [T, Hqk, 128] dtype (token stride q_stride) */
  const void *k;               /* (device) [T, Hqk, 128] dtype */
  const void *v;               /* (device) [T, Hv, 128] dtype */
  const void *g;               /* (device) [T, Hv, 128] dtype: log-decay, or the raw
                                  gate with A_log / dt_bias */
  const void *beta;            /* (device) [T, Hv] dtype, logits */
  int32_t dtype;               /* kda_dtype: KDA_F32, KDA_BF16 or KDA_F16 */
  const int32_t *query_start;  /* (device) [n + 1], non-decreasing */
  int32_t n;                   /* requests >= 0 */
  int32_t hqk, hv;             /* hv % hqk == 0 */
  int32_t window;              /* tokens per request at most, 1..8 */
  float scale;
  int32_t use_qk_l2norm;
  const void *state_cache;     /* (device) [num_slots, Hv, 128(V), 128(K)] of state_dtype */
  int32_t state_dtype;         /* KDA_F32 or KDA_BF16 */
  int64_t state_slot_stride;   /* elements between slots, 0 = hv*128*128 */
  const int32_t *state_indices;  /* (device) [n] */
  int32_t num_slots;
  float *corr;                 /* (device) [n, Hv, window, 128] fp32 */
  void *kg;                    /* (device) [n, Hv, window, 256] dtype */
  void *out;                   /* (device) [T, Hv, 128] dtype */
  const float *A_log;          /* (device) [Hv] fp32, or NULL (gate parameters, */
  const void *dt_bias;         /*  as kda_decode's) [Hv, 128] or NULL */
  int32_t dt_bias_dtype;
  float lower_bound;
  int64_t q_stride, k_stride, v_stride, g_stride, beta_stride;  /* 0 = dense */
  void *stream;                /* hipStream_t or NULL */
} kda_verify_args;

kda_status kda_verify(const kda_verify_args *a);

/*
 * kda_commit_args -- the state after the accepted prefix of each verify
 * window, rebuilt from the slot's state and kda_verify's records alone.
 *
 * The recurrence's step is S_t = diag(e^g_t) S_{t-1} + kn_t u_t^T, and u_t is
 * exactly the recorded correction, so for a = num_accepted_tokens[b] the
 * state after the first a window tokens is that step applied for
 * t = 0 .. a-1, with kn_t (L2-normalised when use_qk_l2norm) and g_t (through
 * the gate parameters when given) recomputed from the raw key and gate in kg.
 * It is written back to slot state_indices[b] in place (a bf16 state is
 * rounded to nearest even once).  The pages name the records but do not show
 * this step; it is the reading that makes them sufficient.  a = 0, a count
 * outside [0, window] or a slot outside [0, num_slots) leaves the request's
 * state alone.  The caller keeps a at most the request's verified token count
 * (record rows past it hold whatever was there).  Slots of one call must be
 * distinct.  Errors as kda_verify's; asynchronous on `stream`.
 */
typedef struct kda_commit_args {
  size_t struct_size;          /* = sizeof(kda_commit_args) */
  void *state_cache;           /* (device) [num_slots, Hv, 128, 128] of state_dtype, in place */
  int32_t state_dtype;         /* KDA_F32 or KDA_BF16 */
  int64_t state_slot_stride;   /* 0 = hv*128*128 */
  int32_t num_slots;
  const int32_t *state_indices;        /* (device) [n] */
  const int32_t *num_accepted_tokens;  /* (device) [n] */
  const float *corr;           /* (device) [n, Hv, window, 128] fp32 (from kda_verify) */
  const void *kg;              /* (device) [n, Hv, window, 256] dtype (from kda_verify) */
  int32_t dtype;               /* kg's kda_dtype */
  int32_t n, hv, window;
  int32_t use_qk_l2norm;
  const float *A_log;          /* as kda_verify's */
  const void *dt_bias;
  int32_t dt_bias_dtype;
  float lower_bound;
  void *stream;
} kda_commit_args;

kda_status kda_commit(const kda_commit_args *a);

/* Static text for a status code. */
const char *kda_status_str(int32_t status);
/* Detail of the calling thread's last failed call ("" if none). */
const char *kda_last_error(void);
/* Library version string. */
const char *kda_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H_ */
