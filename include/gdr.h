/*
 * gdr.h - C ABI of the gated delta rule forward pass on AMD MI355X (gfx950).
 *
 * The method (per value head, state S in R^{d_v x d_k}, value-by-key):
 *     S~  = S * alpha_t            (scalar gate)   or  S Diag(alpha_t) (channel gate)
 *     e_t = beta_t (v_t - S~ k_t)
 *     S   = S~ + e_t k_t^T
 *     o_t = S (scale q_t)          read after the write
 * as boxed in "You Could Have Come Up With Kimi Delta Attention" (opening
 * display; sections 3 and 4) and listed as five steps on the "gated_delta"
 * Mojo module page. The linear rule replaces the delta write by the additive
 * write S = S~ + v_t k_t^T ("From Attention to Learned Memory", section 1).
 * Gates arrive as g = log(alpha) <= 0 (the KDA page, section 4, notes that
 * implementations store this form and exponentiate it).
 *
 * Three entry points compute the same result:
 *   gdr_chunk_fwd       chunkwise prefill over a ragged batch (the chunk
 *                       regrouping of section 6 of the KDA page and section 4
 *                       of "From Attention to Learned Memory");
 *   gdr_recurrent_step  one token per sequence (the tokenwise recurrence);
 *   gdr_recurrent_fwd   the tokenwise recurrence over a ragged batch, the
 *                       state in registers across each sequence (the
 *                       "gated_delta" Mojo page's kernel).
 * gdr_linear_chunk_bwd and gdr_gated_linear_chunk_bwd give the gradients of
 * the linear rule, plain or with a scalar gate, chunkwise;
 * gdr_recurrent_bwd gives the gradients of the gated delta and gated linear
 * rules, tokenwise; gdr_chunk_bwd those of the delta rule (gate NONE or
 * SCALAR), chunkwise;
 * gdr_verify_ring and gdr_state_fold split a speculative-decode window into a
 * verify that writes no state and a fold of the accepted tokens.
 *
 * Memory. Every pointer is device memory owned by the caller; the library
 * neither allocates, frees nor keeps any of them after the call returns.
 * Work is enqueued on `stream` and runs asynchronously: outputs and the state
 * pool are ready once the stream has reached that point.
 *
 * Layouts (elements, row-major; P = products, 1 unless Gated DeltaProduct):
 *   q           [T_total, HK, DK]   token t starts at t * q_stride_t; the
 *                                   HK*DK values of one token are contiguous
 *   k           [T_total*P, HK, DK] row t*P + j (substep j of token t) starts
 *                                   at (t*P + j) * k_stride_t
 *   v           [T_total*P, HV, DV] row t*P + j starts at (t*P + j) * v_stride_t
 *   g           [T_total, HV] (SCALAR) or [T_total, HV, DK] (CHANNEL), fp32,
 *               finite and <= 0; any such gate is handled, however strong the
 *               decay (the chunked forms only ever exponentiate non-positive
 *               log-decays, or positive ones bounded by 80 where the channel
 *               gate's 16-token blocks allow it, and sum the rest pair by pair)
 *   beta        [T_total*P, HV] fp32, in (0, 1]
 *   o           [T_total, HV, DV]   contiguous, written (never read)
 *   state_pool  [num_slots, HV, DK, DV]: S^T per slot and value head, updated
 *               in place for the slots named by slot_idx; other slots are
 *               never touched ("gated_delta" Mojo page, tensor shapes)
 *   slot_idx    [N] int32, distinct, in [0, num_slots)
 *   cu_seqlens  [N+1] int32, 0 = cu[0] <= cu[1] <= ... <= cu[N] = T_total;
 *               sequence n is tokens cu[n] .. cu[n+1]-1 (prefill only)
 * Value head h reads key head h / (HV / HK) (grouped heads, Mojo page).
 * q, k, v, g, o and state_pool must start on 16-byte boundaries and the
 * token strides of q, k and v must be multiples of 16 bytes (the kernels move
 * rows in 16-byte units).
 *
 * Errors. Everything checkable on the host is checked before any work is
 * enqueued; on error nothing is launched and no memory is touched. Contents
 * of device arrays (cu_seqlens monotone, slots in range and distinct, finite
 * inputs) are the caller's contract; GDR_FLAG_DEBUG_CHECKS verifies the index
 * arrays on the device first (this synchronises the stream).
 *
 * Thread safety: the library keeps no state besides a thread-local error
 * message. Concurrent calls are safe when they write disjoint pool slots and
 * outputs.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR_ABI_VERSION 7

typedef enum gdr_status {
  GDR_OK = 0,
  GDR_E_INVALID = 1,      /* malformed arguments (null pointer, bad size, aliasing) */
  GDR_E_UNSUPPORTED = 2,  /* well-formed but not built (head dim, chunk size, dtype) */
  GDR_E_WORKSPACE = 3,    /* workspace missing or below the call's minimum (see below) */
  GDR_E_HIP = 4,          /* the HIP runtime reported an error at launch */
  GDR_E_DEVICE_CHECK = 5  /* GDR_FLAG_DEBUG_CHECKS found a bad cu_seqlens or slot_idx */
} gdr_status;

typedef enum gdr_dtype { GDR_F32 = 0, GDR_BF16 = 1 } gdr_dtype;

/* DELTA: the gated delta rule. LINEAR: S = S~ + v k^T (no prediction, no
 * beta; with gate NONE this is plain linear attention, alpha = 1). */
typedef enum gdr_rule { GDR_RULE_DELTA = 0, GDR_RULE_LINEAR = 1 } gdr_rule;

/* NONE: alpha = 1 (g ignored). SCALAR: one g per token and value head.
 * CHANNEL: one g per token, value head and key channel (KDA). */
typedef enum gdr_gate { GDR_GATE_NONE = 0, GDR_GATE_SCALAR = 1, GDR_GATE_CHANNEL = 2 } gdr_gate;

enum {
  GDR_FLAG_ZERO_INIT = 1u,     /* start every sequence from S = 0 instead of its pool slot */
  GDR_FLAG_DEBUG_CHECKS = 2u,  /* verify cu_seqlens / slot_idx on the device first */
  GDR_FLAG_QK_L2NORM = 4u      /* gdr_recurrent_fwd only: use q / |q| and k / |k| per token and
                                  key head, |x| = sqrt(sum x^2 + 1e-6) */
};

typedef struct gdr_args {
  const void *q;                /* [T_total, HK, DK] in_dtype                              */
  const void *k;                /* [T_total, HK, DK] in_dtype                              */
  const void *v;                /* [T_total, HV, DV] in_dtype                              */
  int64_t q_stride_t;           /* elements between tokens of q (>= HK*DK)                 */
  int64_t k_stride_t;           /* elements between tokens of k (>= HK*DK)                 */
  int64_t v_stride_t;           /* elements between tokens of v (>= HV*DV)                 */
  gdr_dtype in_dtype;           /* type of q, k, v                                         */
  const float *g;               /* log(alpha) <= 0; layout by gate; NULL for GATE_NONE     */
  const float *beta;            /* [T_total, HV]; required for DELTA, ignored for LINEAR   */
  void *o;                      /* [T_total, HV, DV] out_dtype; must not overlap any input */
  gdr_dtype out_dtype;
  void *state_pool;             /* [num_slots, HV, DK, DV] state_dtype, read and written   */
  gdr_dtype state_dtype;
  int64_t num_slots;
  const int32_t *slot_idx;      /* [N]                                                     */
  const int32_t *cu_seqlens;    /* [N+1] prefill; ignored (may be NULL) by the step        */
  int32_t N;                    /* sequences                                               */
  int32_t HK, HV;               /* key heads, value heads (HV % HK == 0)                   */
  int32_t DK, DV;               /* head dims, each 64 or 128                               */
  int64_t T_total;              /* tokens in q/k/v/o (the step requires T_total == N)      */
  float scale;                  /* query scale; callers normally pass DK^-1/2              */
  int32_t chunk_size;           /* gdr_chunk_fwd: tokens per chunk, 16, 32 or 64           */
  gdr_rule rule;
  gdr_gate gate;
  uint32_t flags;               /* GDR_FLAG_*                                              */
  int32_t products;             /* Gated DeltaProduct: n_h transitions per token, 1..8;    */
                                /* 0 means 1. Token t decays once, then applies the delta  */
                                /* (or linear) write of each substep j = 0..P-1 in order   */
                                /* with key, value and beta row t*P + j, then q_t reads    */
                                /* the state ("Linear attention visualized", section       */
                                /* "Gated Delta Product (GDP)")                            */
} gdr_args;

/* GDR_ABI_VERSION of the loaded library. */
int gdr_abi_version(void);

/* Preferred bytes of device workspace for gdr_chunk_fwd with these arguments;
 * 0 when the call runs one fused kernel and needs none. Returns 0 for
 * arguments that fail validation.
 *
 * Only the channel gate with bf16 inputs (KDA's delta rule or GLA's linear
 * rule, one transition per token) at chunk_size 64 uses a workspace:
 * it runs as a parallel per-chunk kernel that writes one record per (chunk,
 * value head) (the decayed keys and queries, the inverse of the chunk's unit
 * lower triangular system and the products the state recurrence needs; the
 * chunk regrouping of section 6 of the KDA page) and a state kernel that
 * reads them in chunk order. The workspace holds an fp32 state carry of
 * N * HV * DK * DV values plus records for a slice of flat chunks; the call
 * runs as many slices as it needs, so any size from the carry plus one
 * chunk's records for every value head (HV * 123392 bytes at DK = 128,
 * HV * 73984 at DK = 64) up works. The preferred size holds up to about
 * 128 MB (KDA) or 192 MB (GLA) of records per slice, the fastest measured;
 * a larger workspace makes no larger slices. */
size_t gdr_chunk_fwd_workspace_bytes(const gdr_args *a);

/* Chunkwise prefill over the ragged batch described by cu_seqlens: writes o
 * for every token and the final state of each sequence into its pool slot.
 * Zero-length sequences write their (initial) state back unchanged. N == 0 is
 * a no-op. chunk_size is the chunk length C of the chunked algorithm ("From
 * Attention to Learned Memory", section 4, which takes 16, 32 or 64): the
 * results are the same recurrence whatever C, up to rounding. 64 runs the
 * tuned kernels; 16 and 32 run the general kernel with each chunk in a
 * 64-row tile whose rows past C are zero (as for a sequence's last, partial
 * chunk), at the cost per chunk of a 64-token one. Other values return
 * GDR_E_UNSUPPORTED. `workspace` (device memory, 256-byte aligned, contents need not be
 * initialised and are garbage afterwards) may be NULL when the call needs
 * none; a call that needs one and gets less than its minimum returns
 * GDR_E_WORKSPACE before enqueuing anything. Calls that share a workspace
 * must not overlap in time. */
gdr_status gdr_chunk_fwd(const gdr_args *a, void *workspace, size_t ws_bytes,
                         hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call, arguments and results as gdr_chunk_fwd, with the library's own
 * static device scratch of GDR_NOALLOC_SCRATCH_BYTES in place of a caller
 * workspace. Calls that need no workspace run exactly as gdr_chunk_fwd. A
 * call whose minimum workspace (see gdr_chunk_fwd_workspace_bytes) exceeds
 * the scratch returns GDR_E_WORKSPACE before enqueuing anything. Allocates
 * nothing: the scratch is a file-scope device array, one per device, held
 * until the process ends, and every call on a device shares it, so calls
 * that overlap in time on one device race (serialise them, e.g. on one
 * stream). Its contents are never read before a call writes them. */
#define GDR_NOALLOC_SCRATCH_BYTES (64u << 20)
gdr_status gdr_chunk_fwd_noalloc(const gdr_args *a, hipStream_t stream);

/* One recurrent step: token n of q/k/v/g/beta belongs to sequence n
 * (T_total == N); reads and writes pool slot slot_idx[n] in place. */
gdr_status gdr_recurrent_step(const gdr_args *a, hipStream_t stream);

/* Tokenwise recurrence over the ragged batch described by cu_seqlens (same
 * arguments, layouts and results as gdr_chunk_fwd; chunk_size is ignored):
 * each (sequence, value head) walks its tokens in order with the state held
 * on chip, the schedule of the "gated_delta" Mojo page, suited to short
 * sequences and to serving that feeds a few tokens per sequence at a time.
 * With GDR_FLAG_QK_L2NORM, q and k are L2-normalised per token and key head
 * inside the kernel (that page's steps 2, 4 and 5), so q, k may be raw (for
 * example views into a fused qkv buffer through the token strides). Needs no
 * workspace. */
gdr_status gdr_recurrent_fwd(const gdr_args *a, hipStream_t stream);

/* Bytes of device workspace gdr_linear_chunk_bwd or gdr_gated_linear_chunk_bwd
 * needs with these arguments (0 for arguments they do not cover, or when
 * there is no work): an fp32 scratch pool of N * HV * D * D values and N
 * slot indices; with fp32 inputs also reversed copies of q, k (T_total * HK
 * * D elements each), v and dout (T_total * HV * D each) and an fp32 output
 * copy of T_total * HV * D; with grouped key heads (HV > HK) q and k
 * repeated over each group (T_total * HV * D elements each); with a gate or
 * grouped key heads two fp32 buffers of T_total * HV * D (dq and dk per value
 * head); with a gate two fp32 arrays of T_total * HV. */
size_t gdr_linear_chunk_bwd_workspace_bytes(const gdr_args *a);

/* Gradients of causal linear attention ("From Attention to Learned Memory",
 * section "Backward: reverse the boundary scan, then differentiate each
 * chunk"): for o_t = scale * S_t q_t, S_t = S_0 + sum_{tau <= t} v_tau k_tau^T
 * and a loss with upstream gradient dout (= dL/do), writes
 *   dq [T_total, HK, DK], dk [T_total, HK, DK], dv [T_total, HV, DV]
 * (contiguous, out_dtype). `a` describes the forward call: q, k, v, their
 * strides and in_dtype, cu_seqlens, HK and HV (HV a multiple of HK: value
 * head h reads key head h / (HV / HK), and dq, dk sum over each group), the
 * initial state S_0 read from state_pool[slot_idx[n]] (never written) unless
 * GDR_FLAG_ZERO_INIT, scale, chunk_size 64; `a->o` is ignored. dout is
 * [T_total, HV, DV], contiguous, in in_dtype. Covered: the linear rule with
 * gate NONE (a scalar gate is gdr_gated_linear_chunk_bwd), one transition
 * per token (else GDR_E_UNSUPPORTED). The final state's gradient is taken as
 * zero and the initial state's is not formed. `workspace` (device memory,
 * 256-byte aligned, at least gdr_linear_chunk_bwd_workspace_bytes) is
 * scratch; calls sharing one must not overlap. Each gradient runs as one
 * chunkwise forward pass with the roles of q, k, v and dout exchanged (dk and
 * dv walk every sequence's tokens backwards). */
gdr_status gdr_linear_chunk_bwd(const gdr_args *a, const void *dout, void *dq, void *dk, void *dv,
                                void *workspace, size_t ws_bytes, hipStream_t stream);

/* The same gradients for the linear rule with a scalar gate (same page and
 * section; the state decays as S_t = alpha_t S_{t-1} + v_t k_t^T with
 * a->g = log alpha, fp32 [T_total, HV]), plus the log-decays' gradient
 *   dg [T_total, HV] fp32:  dg_t = sum over the tokens i >= t of t's
 *   sequence of (q_i . dq_i - k_i . dk_i), dq_i and dk_i taken per value head
 * (each pair's decay exponent is the sum of the log-decays between them, so
 * a log-decay's gradient collects every pair that spans it). Requires gate
 * SCALAR (else GDR_E_UNSUPPORTED); dg is device memory, 4-byte aligned, not
 * overlapping any input or gradient. Everything else as gdr_linear_chunk_bwd;
 * the passes that walk backwards take each token's decay from the token
 * after it. */
gdr_status gdr_gated_linear_chunk_bwd(const gdr_args *a, const void *dout, void *dq, void *dk, void *dv,
                                      float *dg, void *workspace, size_t ws_bytes, hipStream_t stream);

/* Bytes of device workspace gdr_recurrent_bwd needs with these arguments
 * (0 when N == 0 or the arguments are invalid): fp32 checkpoints of the state
 * every 8 tokens ((T_total / 8 + N + 1) * HV * DK * DV values) and per-token
 * partial sums (T_total * HV * (DV / 32) * (2 or 3) * DK values, plus two
 * T_total * HV * (DV / 32) arrays). */
size_t gdr_recurrent_bwd_workspace_bytes(const gdr_args *a);

/* Gradients of the tokenwise recurrence of gdr_recurrent_fwd (the forward of
 * "You Could Have Come Up With Kimi Delta Attention", recurrent form, with the
 * gated variants of "Linear attention visualized"; the pages give no backward
 * for the delta rule, so this is that recurrence differentiated in reverse
 * mode) for a loss with upstream gradient dout = dL/do. `a` describes the
 * forward call: q, k, v, their strides and in_dtype, g, beta, rule, gate,
 * scale, cu_seqlens and the initial state from state_pool[slot_idx[n]] (read,
 * never written) unless GDR_FLAG_ZERO_INIT; `a->o` is ignored. Any rule and
 * gate, grouped heads, DK = DV in {64, 128}; one transition per token and no
 * GDR_FLAG_QK_L2NORM (else GDR_E_UNSUPPORTED). Writes
 *   dq, dk   [T_total, HK, DK] out_dtype (summed over the value heads of a
 *            key head), contiguous, 16-byte aligned
 *   dv       [T_total, HV, DV] out_dtype, contiguous, 16-byte aligned
 *   dbeta    [T_total, HV] fp32 (delta rule; ignored for the linear rule)
 *   dg       shaped like g, fp32 (gated calls; ignored for GATE_NONE)
 *   dstate0  [N, HV, DK, DV] fp32 or NULL: dL/dS_0 per sequence, transposed
 *            like the pool (also under ZERO_INIT: the gradient at the zero
 *            state); zeros for an empty sequence
 * dout is [T_total, HV, DV], contiguous, in in_dtype, 16-byte aligned. No
 * gradient buffer may overlap another, an input or the pool. The final
 * state's gradient is taken as zero (the loss reads the outputs only).
 * `workspace` (device, 256-byte aligned, at least
 * gdr_recurrent_bwd_workspace_bytes) is scratch. */
gdr_status gdr_recurrent_bwd(const gdr_args *a, const void *dout, void *dq, void *dk, void *dv, float *dbeta,
                             float *dg, float *dstate0, void *workspace, size_t ws_bytes, hipStream_t stream);

/* Bytes of device workspace gdr_chunk_bwd needs with these arguments (0 when
 * N == 0 or the arguments are invalid or not covered): four fp32 arrays of
 * (ceil(T_total / 64) + N) * HV * DK * DV values (the state at every chunk
 * start, its gradient after every chunk, and each chunk's reverse map M and
 * Y) and two of T_total * HV * DK (dq and dk per value head). */
size_t gdr_chunk_bwd_workspace_bytes(const gdr_args *a);

/* The gradients of gdr_recurrent_bwd (same arguments, outputs, layouts and
 * readings) for the delta rule with gate NONE or SCALAR, computed chunkwise
 * in the manner of "From Attention to Learned Memory", section "Backward:
 * reverse the boundary scan, then differentiate each chunk", applied to the
 * delta rule's chunk equations ("You Could Have Come Up With Kimi Delta
 * Attention", section 6): a forward walk stores the state at every chunk
 * start; a reverse walk carries the state's gradient from the sequence end
 * back over the chunk boundaries (each chunk's map is the transpose of the
 * forward chunk map's linear part, plus a term from the chunk's output
 * gradients); then every chunk's gradients are formed independently. fp32
 * arithmetic throughout (matrix products on fp32 MFMA). Other rules and gates
 * return GDR_E_UNSUPPORTED. `workspace` (device, 256-byte aligned, at least
 * gdr_chunk_bwd_workspace_bytes) is scratch; calls sharing one must not
 * overlap. */
gdr_status gdr_chunk_bwd(const gdr_args *a, const void *dout, void *dq, void *dk, void *dv, float *dbeta,
                         float *dg, float *dstate0, void *workspace, size_t ws_bytes, hipStream_t stream);

/* Speculative decoding ("gated_delta" Mojo page, its verify-ring, record and
 * fold functions, which it names without detail; the reading taken here):
 *
 * gdr_verify_ring runs gdr_recurrent_fwd over each sequence's window of draft
 * tokens (same arguments, outputs o, QK_L2NORM allowed, one transition per
 * token) but leaves state_pool untouched, and records every token's state
 * update in `ring` [T_total, HV, stride] fp32: the error e = beta (v - S~ k)
 * (v for the linear rule, DV values), the key it is written along (DK values,
 * normalised under QK_L2NORM), then the token's log-gate (1 value for SCALAR,
 * DK for CHANNEL, none for NONE); `stride` = gdr_ring_record_stride(a) (the
 * gdr_ring_record_elements(a) values rounded up to a multiple of 4). ring is
 * device memory, 16-byte aligned, not overlapping o, the inputs or the pool.
 *
 * gdr_state_fold then applies, for each sequence n, the records of its first
 * accepted[n] window tokens (accepted: [N] int32 device array, clamped to
 * [0, window length]) in order to pool slot slot_idx[n]:
 * S <- S~ + e k^T, with S~ the decayed state. The result equals the state the
 * recurrence reaches after those tokens. `a` is the verify's arguments (only
 * N, HK, HV, DK, DV, gate, state_pool, state_dtype, num_slots, slot_idx,
 * cu_seqlens and T_total are read). */
int gdr_ring_record_elements(const gdr_args *a);
int gdr_ring_record_stride(const gdr_args *a);
gdr_status gdr_verify_ring(const gdr_args *a, float *ring, hipStream_t stream);
gdr_status gdr_state_fold(const gdr_args *a, const float *ring, const int32_t *accepted,
                          hipStream_t stream);

/* Static description of a status code. */
const char *gdr_status_string(gdr_status s);

/* Detail of the last failure on the calling thread ("" if none). */
const char *gdr_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* GDR_H */
