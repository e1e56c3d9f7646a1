/*
 * slim.h -- C ABI of the MI355X (gfx950) causal linear self-attention library
 * (libslim.so).
 *
 * The operation (page "Sub-Linear Memory: How to Make Performers SLiM",
 * Subsection 2.1, eq. (2)-(4)):  for every batch b and head h, with a
 * feature map g: R^d -> R_+^M,
 *     R_l = R_0 + sum_{i<=l} V_i g(K_i)^T      (d x M)
 *     S_l = S_0 + sum_{i<=l} g(K_i)            (M)
 *     Y_l = R_l g(Q_l) / (S_l . g(Q_l))         l = 1..L
 * i.e. the causal (diagonal included) g(Q_l).g(K_i)-weighted average of the
 * values.  (R_0, S_0) is an optional initial state (zero by default), which
 * lets one long sequence be streamed through several calls.
 *
 * Evaluation follows the page's sliced scheme (Subsection 3.2, eq. (14)-(18)):
 * the sequence is cut into num_chunks slices of length c = ceil(L/num_chunks)
 * (the last one may be shorter); the backward (Subsection 3.3, updates
 * (19)-(20)) walks the slices in reverse, recomputing each slice's forward,
 * recovering each slice's entry state from the final state by subtraction and
 * carrying the gradient of the state.  No L x d x M prefix tensor is stored:
 * the workspace holds per-slice states for a bounded window of slices, so it
 * does not grow with L once L exceeds window_chunks * c.  Where one window
 * holds every slice, the forward can hand its per-slice states to the
 * backward (slim_state_bytes), which then skips rebuilding them.
 *
 * Feature maps (Subsection 2.1 names both kinds):
 *   SLIM_FEAT_FAVOR: g(x)_m = exp(w_m . x - |x|^2/2) / sqrt(M), w_m = row m of
 *                    W [M][d] (FAVOR+ positive random features; W is an input,
 *                    drawn by the caller, Gaussian or orthogonal).
 *   SLIM_FEAT_ELU1 : g(x)_j = elu(x_j) + 1, M must equal d, W must be NULL.
 *
 * Conventions for every entry point:
 *   - Layout: Q, K, V, Y, dY, dQ, dK, dV are contiguous row-major
 *     [B][H][L][d]; W is [M][d]; states R are [B][H][d][M], S [B][H][M], in
 *     desc.state_dtype (fp32 or fp64); phi is [B][H][L][M] fp32.
 *   - dtype: SLIM_F32 or SLIM_BF16 is the element type of Q, K, V, W, Y, dY,
 *     dQ, dK, dV.  States, statistics and all accumulation are fp32.
 *   - All pointers are device pointers (HIP).  The caller owns every buffer;
 *     the library never allocates, frees or synchronises.  Work is enqueued on
 *     `stream` (a hipStream_t; NULL = the default stream) and runs
 *     asynchronously.  Buffers must stay valid until the work completes.
 *   - Alignment: every tensor pointer and the workspace must be 16-byte
 *     aligned (256-byte for the workspace).
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; a failing check returns a status and enqueues nothing.
 *     SLIM_ERR_HIP means a launch failed (hipGetLastError); work enqueued
 *     before the failure may have run.  No exception crosses the ABI.
 *   - Supported shapes: d in {16, 32, 64, 128}; M in {16, 32, 64, 128, 256}
 *     (FAVOR+) or M == d (elu+1); 1 <= num_chunks <= L; L < 2^31.  Other
 *     shapes return SLIM_ERR_UNSUPPORTED.
 *   - Results are deterministic: no atomics, fixed reduction order.
 *
 * Key-side offset (FAVOR+; Subsection 2.1 relies on positive features for a
 * well-defined, stable division).  exp(w_m.k - |k|^2/2) can exceed the fp32
 * range for a W row of large norm and a key near it; since
 * w_m.k - |k|^2/2 <= |w_m|^2/2 for every key, every call evaluates the key
 * features as g(K) exp(-koff) with the one number
 *     koff = max(0, max_m |w_m|^2/2 - 60)
 * (computed on the device from W in fp32), which bounds each of them by
 * exp(60)/sqrt(M).  A factor common to all key features cancels in Y and in
 * dQ, dK, dV; it stays only in the states, so every state argument (R_in,
 * S_in, R_out, S_out of the forward and the decode step) holds the state
 * times exp(-koff), and every state-gradient argument (dR_out, dS_out,
 * dR_in, dS_in) the gradient with respect to that scaled state.  koff depends
 * on W alone, so calls that pass states between them with the same W agree;
 * for W with every |w_m|^2 <= 120 (Gaussian or orthogonal draws at d <= 64)
 * koff = 0 and the states are the plain sums.  elu+1: koff = 0.
 */
#ifndef SLIM_H
#define SLIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum slim_status {
    SLIM_OK = 0,
    SLIM_ERR_NULL = 1,        /* a required pointer is NULL */
    SLIM_ERR_SHAPE = 2,       /* B, H, L, d, M or num_chunks out of range */
    SLIM_ERR_DTYPE = 3,       /* unknown dtype or feature-map kind */
    SLIM_ERR_UNSUPPORTED = 4, /* valid but not compiled: see supported shapes */
    SLIM_ERR_WORKSPACE = 5,   /* workspace smaller than slim_workspace_bytes() */
    SLIM_ERR_ALIGN = 6,       /* misaligned pointer */
    SLIM_ERR_HIP = 7          /* a HIP launch failed */
} slim_status;

typedef enum slim_dtype { SLIM_F32 = 0, SLIM_BF16 = 1, SLIM_F64 = 2 } slim_dtype;
typedef enum slim_feat { SLIM_FEAT_FAVOR = 0, SLIM_FEAT_ELU1 = 1 } slim_feat;
/* SLIM_PASS_BWD_DW: the backward when it also computes dW (FAVOR+ only; a
 * larger workspace). */
typedef enum slim_pass {
    SLIM_PASS_FEATMAP = 0,
    SLIM_PASS_FWD = 1,
    SLIM_PASS_BWD = 2,
    SLIM_PASS_DECODE = 3,
    SLIM_PASS_BWD_DW = 4
} slim_pass;

typedef struct slim_desc {
    int64_t B, H, L;       /* batch, heads, sequence length */
    int64_t d, M;          /* head dim, number of features */
    int64_t num_chunks;    /* N slices; slice length c = ceil(L / N) */
    int64_t window_chunks; /* slices whose states are held at once; 0 = auto: enough for
                              about 4096 workgroups per launch, or all of them when the
                              backward's per-slice buffers for the whole sequence fit in
                              1 GiB, and never more than those buffers fit in 1 GiB (the
                              dW pass's own per-slice rows within another 1 GiB) */
    int32_t dtype;         /* slim_dtype of Q, K, V, W, Y, dY, dQ, dK, dV: SLIM_F32 or SLIM_BF16 */
    int32_t feat;          /* slim_feat */
    int32_t state_dtype;   /* element type of the states and their gradients (R_in, S_in,
                              R_out, S_out, dR_out, dS_out, dR_in, dS_in): SLIM_F32, or
                              SLIM_F64 (states passed between calls then keep the
                              precision of the internal fp64 carries; the decode step
                              then updates the state in fp64) */
    int32_t group_slices;  /* consecutive slices one workgroup walks, carrying the state
                              from one to the next (the page's slice loop, that many
                              slices at a time): one state per group is stored, scanned
                              and read back.  0 = automatic (slim_group_slices); 1 = one
                              slice per workgroup.  Results differ between groupings
                              only in fp32 rounding order. */
} slim_desc;

/* Host-only check of a descriptor for a pass; touches no GPU.  SLIM_PASS_DECODE
 * requires L == 1 (one token per head) and allows B*H up to 2^24. */
slim_status slim_validate(const slim_desc *desc, int pass);

/* Workspace bytes the pass needs (0 for SLIM_PASS_FEATMAP and SLIM_PASS_DECODE); 0 if the
 * descriptor is invalid.  Host-only. */
size_t slim_workspace_bytes(const slim_desc *desc, int pass);

/* Slices whose states one window holds (the resolved window_chunks, a whole number of
 * groups) in the forward and the plain backward; the backward with dW may hold fewer
 * (see window_chunks).  A given window_chunks is rounded down to whole groups (at
 * least one). */
int64_t slim_window_chunks(const slim_desc *desc);

/* Slices per group (desc.group_slices, or the automatic choice: the largest power of
 * two with groups of at most 2048 rows whose launches have at least 512 workgroups and
 * fill whole rounds of 512 workgroups, and for bf16 with M = 64 also of 768, to within
 * 10%; else 1).  0 if the descriptor is invalid.  Host-only. */
int64_t slim_group_slices(const slim_desc *desc);

/* Bytes of the `states` buffer slim_attn_fwd can fill for the backward: the state
 * entering every group of slices, [B*H][n + 1][d + 1][M] fp32 (n = ceil(L / (G c)),
 * the groups there are, G = slim_group_slices(desc), c the slice length), entry j
 * of a head holding R (rows e < d, stored [e][m] = R[e][m]) and S (row d) before
 * group j, i.e. after the first j G slices, scaled by exp(-koff): entry 0 the
 * initial state, the last entry the final state.  Only when one window holds every
 * slice (slim_window_chunks(desc) equal to the number of slices); else 0, and states
 * cannot be kept.  Host-only; 0 for an invalid descriptor. */
size_t slim_state_bytes(const slim_desc *desc);

/* Workspace bytes of a pass (SLIM_PASS_FWD, SLIM_PASS_BWD, SLIM_PASS_BWD_DW) when
 * the call is given a states buffer: slim_workspace_bytes less the room for the
 * slices' states, where the pass holds every slice in one window; otherwise
 * slim_workspace_bytes itself.  Host-only; 0 for an invalid descriptor. */
size_t slim_workspace_bytes_states(const slim_desc *desc, int pass);

/* Rows per tile with which the chunk kernels walk a slice for this
 * descriptor's (dtype, feat, d, M): 32, or 16 where 32-row tiles would not fit
 * a compute unit's LDS.  0 if the descriptor is invalid.  Host-only. */
int64_t slim_tile_rows(const slim_desc *desc);

/* Feature map (Subsection 2.1): phi[r][m] = g(X_r)_m in fp32 for the
 * B*H*L rows of X ([B][H][L][d], desc dtype).  FAVOR+: if row_offset is
 * non-NULL, row r is scaled by exp(-row_offset[r]) with
 * row_offset[r] = max_m (w_m . X_r - |X_r|^2/2) (so every value is at most
 * 1/sqrt(M)); if NULL, the unscaled value.  row_offset must be NULL for elu+1.
 * num_chunks is ignored. */
slim_status slim_featmap(const slim_desc *desc, const void *X, const void *W, float *phi, float *row_offset,
                         void *stream);

/* Forward (eq. (2) evaluated slice by slice, Subsection 3.2).
 * In : Q, K, V, W (NULL for elu+1); R_in, S_in = initial state (both NULL =
 *      zero, or both given), scaled by exp(-koff) (see "Key-side offset").
 * Out: Y; R_out, S_out = final state R_L, S_L times exp(-koff) (required;
 *      R_out/S_out may not alias R_in/S_in);
 *      koff = the key-side offset of W, one fp32 value on the device (NULL =
 *      not wanted);
 *      row_stats = per-row statistics for the backward, [B][H][L][2] fp32, or
 *      NULL = not wanted: for row l, 1/den'_l and o_l, where o_l is the query
 *      offset in the base-2 exponent domain (FAVOR+: -log2(e) max_m w_m.Q_l;
 *      elu+1: 0) and den'_l = S'_l . g'(Q_l) with the scaled state S'_l =
 *      S_l exp(-koff) and the query features taken as
 *      g'(Q_l)_m = exp(w_m.Q_l) 2^o_l (FAVOR+; elu+1: g itself), i.e.
 *      den_l = den'_l exp(koff - o_l ln 2 - |Q_l|^2/2) / sqrt(M).  8 bytes per
 *      row, the analogue of the log-sum-exp kept by softmax attention;
 *      states = the state entering every slice, slim_state_bytes(desc) bytes
 *      in the layout given there, for the backward to read instead of
 *      rebuilding them; NULL = not wanted.  SLIM_ERR_SHAPE where
 *      slim_state_bytes(desc) is 0 (the slices span several windows).
 * ws : device workspace of at least slim_workspace_bytes(desc, SLIM_PASS_FWD), or
 *      slim_workspace_bytes_states(desc, SLIM_PASS_FWD) with states (the
 *      slices' states are then built in states itself). */
slim_status slim_attn_fwd(const slim_desc *desc, const void *Q, const void *K, const void *V, const void *W,
                          const void *R_in, const void *S_in, void *Y, void *R_out, void *S_out, float *koff,
                          float *row_stats, float *states, void *ws, size_t ws_bytes, void *stream);

/* Size of the device array slim_attn_fwd_noalloc works in, per GPU: 64 MiB. */
#define SLIM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* The forward above for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, results and errors as slim_attn_fwd, without states, ws and ws_bytes: the
 * workspace is a file-scope device array of SLIM_NOALLOC_SCRATCH_BYTES that each
 * GPU the library runs on holds until the process ends (its address is looked up
 * once per device, on the first call there).  The call allocates and frees
 * nothing.
 * Window: the automatic window (desc.window_chunks == 0), shrunk to the most
 * slices whose workspace fits the array; or desc.window_chunks itself, which must
 * fit.  Returns SLIM_ERR_WORKSPACE, before anything is enqueued, when it does not
 * fit, or when even one slice per window does not (about 16*B*H*(d+1)*M bytes: two
 * state slots and the fp64 carries per head, so B*H up to about 250 at d = 64,
 * M = 256).  Results equal slim_attn_fwd's with the same window exactly, and with
 * another window up to the rounding of the fp64 carries to fp32 slots.
 * Every call on one GPU uses that GPU's one array: calls that overlap on one GPU
 * (other streams, other host threads) race and must be ordered by the caller.
 * Nothing in the array needs clearing between calls: every byte a call reads it
 * has written first. */
slim_status slim_attn_fwd_noalloc(const slim_desc *desc, const void *Q, const void *K, const void *V,
                                  const void *W, const void *R_in, const void *S_in, void *Y, void *R_out,
                                  void *S_out, float *koff, float *row_stats, void *stream);

/* Backward of the loss <dY, Y> + <dR_out, R_out> + <dS_out, S_out> of the
 * forward above (Subsection 3.3: a reverse walk over the slices that recomputes
 * each slice's forward and carries the gradient of the state).  Every slice's
 * entry state is rebuilt from the initial state with fp64 carries: within a
 * window by a forward prefix from the window's start state, which for a later
 * window is the state after it minus its slices' contributions (update (19));
 * when the sequence spans several windows, one extra sweep over all slices
 * first rebuilds the final state.  The forward's fp32 final state is not used
 * for this, since recovering small entry states from it by subtraction would
 * carry its rounding into every one of them.
 * In : Q, K, V, W as in the forward; dY; R_in, S_in = the forward's initial
 *      state (both NULL = zero, or both given);
 *      Y, row_stats = the output and row statistics of a forward call on the
 *      same inputs (any slice count), or both NULL.  Given, the backward takes
 *      every row's denominator from them and dden_l = -(dY_l . Y_l) / den_l
 *      from Y, instead of recomputing each slice's forward for them;
 *      states = what a forward call with the same descriptor and inputs wrote
 *      to its states argument, or NULL.  Where this pass holds every slice in
 *      one window (always so for SLIM_PASS_BWD when slim_state_bytes(desc) is
 *      not 0) the backward reads each slice's entry state from it instead of
 *      rebuilding them (the chunk-state pass and its prefix sum are skipped);
 *      the values are the ones the rebuild gives, bit for bit, so the results
 *      are the same.  Elsewhere it is ignored;
 *      dR_out, dS_out = incoming gradient of the final state (both NULL = zero).
 * Out: dQ, dK, dV; dR_in, dS_in = gradient w.r.t. the initial state (both NULL
 *      = not wanted, or both given);
 *      dW = gradient w.r.t. the FAVOR+ projection, [M][d] fp32, summed over all
 *      batch rows and heads (they share W), overwritten; NULL = not wanted.
 *      g depends on W only through w_m, with d g(x)_m / d w_m = g(x)_m x, so
 *      dW[m] = sum over the query and key rows x of (dL/dg(x)_m) g(x)_m x.
 *      The key-side offset is held constant: exact whenever koff = 0, and for
 *      states handed between calls with the same W (its factor cancels
 *      between the call that scales a state and the call that reads it).
 *      FAVOR+ only (SLIM_ERR_UNSUPPORTED for elu+1).  Deterministic: the
 *      per-row products are summed in a fixed order.
 * ws : device workspace of at least slim_workspace_bytes(desc, SLIM_PASS_BWD),
 *      or slim_workspace_bytes(desc, SLIM_PASS_BWD_DW) when dW is given (it
 *      adds two [B*H][window rows][M] buffers of the io dtype and the partial
 *      sums of dW); with states, slim_workspace_bytes_states of the same pass. */
slim_status slim_attn_bwd(const slim_desc *desc, const void *Q, const void *K, const void *V, const void *W,
                          const void *dY, const void *Y, const float *row_stats, const float *states,
                          const void *R_in, const void *S_in, const void *dR_out, const void *dS_out, void *dQ,
                          void *dK, void *dV, void *dR_in, void *dS_in, float *dW, void *ws, size_t ws_bytes,
                          void *stream);

/* Recurrent decode step: the iterative prefix-sum evaluation of Subsection
 * 2.1 (eq. (3)-(4)) advanced by one position.  For every b, h and the one new
 * token (q, k, v):
 *     R' = R + v g(k)^T,   S' = S + g(k),   y = R' g(q) / (S' . g(q)).
 * This is what slim_attn_fwd computes for its first row, and a run of decode
 * steps gives the same outputs and state as one slim_attn_fwd over the same
 * tokens (up to fp32 rounding order).
 * desc: L must be 1 (num_chunks therefore 1); window_chunks is ignored;
 *       state_dtype SLIM_F32 or SLIM_F64 (the state's type; with fp64 the
 *       update, the row dot products and the division are done in fp64, the
 *       features in fp32).
 * In : q, k, v [B][H][d] (desc dtype); W as in the forward (NULL for elu+1);
 *      R_in [B][H][d][M], S_in [B][H][M] (state_dtype) = the state before the
 *      token, times exp(-koff) like every state argument (both NULL = zero,
 *      i.e. the first token, or both given).
 * Out: y [B][H][d]; R_out, S_out = the state after the token, scaled likewise
 *      (required).
 *      R_out may be the same pointer as R_in and S_out as S_in (update in
 *      place); no other overlap of inputs and outputs is allowed.
 * No workspace.  Two calls that update the same state must be ordered (same
 * stream or synchronised). */
slim_status slim_decode_step(const slim_desc *desc, const void *q, const void *k, const void *v, const void *W,
                             const void *R_in, const void *S_in, void *y, void *R_out, void *S_out, void *stream);

const char *slim_status_string(slim_status s);

/* Kernel timing, for measurement tools.  slim_prof_enable(1) clears the
 * totals and starts bracketing every kernel the library launches with a pair
 * of hipEvents on the launch stream (a small, constant overhead per launch);
 * slim_prof_enable(0) stops.  slim_prof_count() and slim_prof_entry() first
 * wait for the recorded events to complete (they synchronise with those
 * events), then report per kernel name ("state", "scan_prefix", "fwd",
 * "scan_window", "scan_sum", "stats", "rowstat" (stats from the forward's row
 * statistics), "bwdq", "gstate", "bwdq_gstate" (the dQ
 * kernel with the gradient state folded in, for shapes where it fits),
 * "scan_grad", "bwdkv", "featmap", "decode"; with dW: "bwdq_dw" or
 * "bwdq_gstate_dw", "bwdkv_dw", "dw" (the row contraction), "dw_sum" (the sum
 * of its partials)) the summed GPU time in
 * milliseconds and the number of launches.  The name pointer stays
 * valid until the next slim_prof_enable(1).  Guarded by a process-wide mutex;
 * the timings are global to the process, not per stream. */
slim_status slim_prof_enable(int enable);
int slim_prof_count(void);
slim_status slim_prof_entry(int i, const char **name, double *total_ms, int64_t *launches);

/* ABI version: (major << 16) | minor. */
int slim_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SLIM_H */
