/*
 * gla.h -- C ABI of the MI355X (gfx950) chunkwise forward of GTR's key-only
 * gated linear attention.
 *
 * What is computed (GTR project page, "How GTR Works" and "A Kernel That
 * Makes Recurrence Fast"; ai.info summary of GTR, "Methodology in Plain
 * English"): for every batch element b and head h, the tokens of a
 * grid_h x grid_w patch grid are visited in one of four scan orders; along
 * that order a state S in R^{dk x dv} starts at zero and evolves as
 *
 *     S_t = diag(exp(gk_t)) S_{t-1} + k_t^T v_t,      o_t = q_t S_t,
 *
 * i.e. only the key-side dimensions decay (value-side decay fixed at one);
 * the output is written back at each token's own grid position. gk is the
 * log of the per-key-dimension decay (gk <= 0 is the contract; gk > 0 makes
 * the state grow and may overflow). No query scaling is applied.
 *
 * How it is computed: the chunkwise form, which the project page's kernel
 * section presents as the recurrence itself on another execution order.
 * Tokens are cut into chunks of `chunk` tokens. The three-phase schedule
 * runs three kernels back to back on the caller's stream:
 *   1. chunk summaries   -- for every (chunk, head) in parallel: the chunk's
 *                           total decay a_n and its state contribution U_n;
 *   2. boundary scan     -- S_{n+1} = diag(a_n) S_n + U_n along the chunks;
 *   3. chunk outputs     -- for every (chunk, head) in parallel: the causal
 *                           intra-chunk decayed score tile times V, plus the
 *                           readout of S_n.
 *
 * Memory layout (all tensors caller-owned device memory, contiguous,
 * row-major, raster token order):
 *   q, k, gk : [B][T][H][dk]      v, o : [B][T][H][dv]      T = grid_h*grid_w
 * dtype GLA_F16: q, k, v, gk, o are IEEE half. GLA_F32: they are float; q, k
 * and v are rounded to half for the matrix-core products, gk stays float.
 * Accumulation is float in both cases. Supported: dk, dv in {32, 64},
 * chunk in {16, 32, 64}. Device pointers must be 16-byte aligned; the
 * workspace 256-byte aligned.
 *
 * Value range: any finite half inputs (|x| <= 65504) with gk <= 0. Every
 * factor the kernels feed to a half-precision product has magnitude at most
 * that of the q, k or v element it scales; where the exact diagonal of a
 * chunk's score tile would need a larger factor, the kernels switch to float
 * operands or to a direct float sum (chosen per 16-token block from the
 * block's decay range and the magnitudes of its q and k rows). The state
 * summaries, boundary states and score blocks are held in half with a
 * power-of-two scale per row or block, so they have float's range. For
 * GLA_F32 inputs, |q|, |k| and |v| must not exceed 65504 (they are rounded
 * to half). An output whose exact value lies beyond the half range is +-Inf
 * in GLA_F16.
 *
 * Directions: `dir` is a HOST array of B codes (GLA_L2R..GLA_B2T), one per
 * batch element; pass B copies for a single direction. Left->right is the
 * raster order; top->bottom walks the columns left to right, each column top
 * to bottom; right->left and bottom->top are the full reversals of those.
 *
 * Schedules: besides the three kernels above, the forward can run as ONE
 * kernel (single pass): every (chunk, head) workgroup computes its summary,
 * publishes it, computes its intra-chunk part, then takes its entering state
 * from the summaries its predecessors publish (grouped in about sqrt(N)
 * segments, whose last chunks publish segment aggregates), and adds the
 * readout. Workgroups run in chunk-major order (chunk n of every chain,
 * then chunk n + 1) and only wait on earlier ones, with bounded waits. On
 * small grids with dv = 64 (at most 224 chunk-heads, no output gate) each
 * chunk-head runs as two workgroups of 32 value columns (the columns of the
 * state are independent recurrences). gla_fwd_schedule and
 * gla_auto_schedule say which schedule a call takes.
 *
 * Workspace: caller-owned device memory of gla_fwd_workspace_bytes bytes,
 * 256-byte aligned, of ANY contents. Its first 64 KiB are the single pass's
 * control words. The single pass runs only on a workspace that
 * gla_workspace_init has prepared: the library records the prepared start
 * addresses, and every single-pass call leaves the words zero again (also
 * across problem sizes). A workspace that was not prepared runs the three
 * phases, which need no control words, so a plain allocation is always
 * valid. If prepared memory is freed or written by anything other than this
 * library, call gla_workspace_release (or gla_workspace_init again) first.
 * Word 0 is a sticky error word: bit 0 set means a single-pass wait ran out
 * of its poll budget (the results of that call are invalid);
 * gla_workspace_status reads and clears it.
 *
 * Execution: asynchronous on `stream` (a hipStream_t passed as void*; NULL
 * is the default stream). No forward call allocates, synchronises or reads
 * device memory on the host, so every forward can be captured in a HIP
 * graph (gla_workspace_status alone synchronises). Calls may run
 * concurrently on different workspaces (never on one workspace). The library
 * keeps no pointer after a call returns, except the addresses of prepared
 * workspaces.
 *
 * Errors: arguments are checked on the host before any HIP call; a failing
 * check returns a negative status and touches nothing. A failed launch
 * returns GLA_E_HIP. Device faults surface at the caller's next
 * synchronisation. Values are not checked: NaN and Inf propagate.
 * Empty problems (B, H, grid_h or grid_w equal to 0) return GLA_OK and launch
 * nothing; pointers are then not examined.
 */
#ifndef GLA_H_
#define GLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { GLA_L2R = 0, GLA_R2L = 1, GLA_T2B = 2, GLA_B2T = 3 };
enum { GLA_F16 = 0, GLA_F32 = 1 };
enum {
  GLA_SCHED_AUTO = 0,
  GLA_SCHED_SINGLE_PASS = 1,  /* one workgroup per chunk, segmented look-back */
  GLA_SCHED_THREE_PHASE = 2,  /* summaries, boundary scan, outputs */
  GLA_SCHED_RUNS = 3          /* one workgroup per run of 4 (fp16) or 3 (fp32) chunks,
                                 decoupled look-back between runs */
};
enum {
  GLA_OK = 0,
  GLA_E_ARG = -1,          /* null/misaligned pointer, negative size, bad code */
  GLA_E_UNSUPPORTED = -2,  /* dk, dv or chunk outside the supported set */
  GLA_E_WORKSPACE = -3,    /* workspace smaller than gla_fwd_workspace_bytes */
  GLA_E_HIP = -4,          /* a HIP launch failed; see gla_last_error_detail */
  GLA_E_UNPREPARED = -5    /* single pass asked for on an unprepared workspace */
};

/* Library ABI version (incremented on any signature or layout change). */
int gla_abi_version(void);

/* Prepare a workspace for the single pass: zero its control words (its first
 * 64 KiB, including the sticky error word) with a kernel on `stream`
 * (graph-capturable) and record its start address as prepared.
 * workspace_bytes is the size of the buffer (at least 64 KiB). */
int gla_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Forget that a workspace was prepared (call before freeing it or using its
 * memory for anything else). Later forwards on it run the three phases
 * until it is prepared again. GLA_E_ARG for NULL. */
int gla_workspace_release(const void* workspace);

/* 1 if gla_workspace_init prepared this start address (and it was not
 * released since), else 0. */
int gla_workspace_is_prepared(const void* workspace);

/* Waits for the work queued on `stream`, then stores the workspace's sticky
 * error word in *error_bits (bit 0: a single-pass wait ran out, the results
 * of that call are invalid) and, if `clear` is nonzero, zeroes it.
 * Synchronises, so it cannot be captured in a graph. GLA_E_WORKSPACE if
 * workspace_bytes < 64 KiB; GLA_E_HIP if the copy fails. */
int gla_workspace_status(void* workspace, size_t workspace_bytes,
                         uint32_t* error_bits, int clear, void* stream);

/* Bytes of workspace gla_fwd needs for this problem (0 for an empty one, or
 * if the shape is unsupported or negative). The workspace may hold anything
 * on entry (see "Workspace" above for the prepared single-pass case). */
size_t gla_fwd_workspace_bytes(int B, int H, int grid_h, int grid_w, int dk,
                               int dv, int chunk);

/* Byte offsets, within the workspace, of the intermediate arrays, so that
 * callers (tests) can inspect them after the phase calls below:
 *   U : half  [B][H][N][dk][dv]   chunk summaries, row d stored divided by
 *                                 its scale sigU_n[d] = row_scale(m_n[d])
 *   a : float [B][H][N][dk][2]    pairs (a_n[d], m_n[d]): the per-chunk
 *                                 total decay exp(sum of gk) and the largest
 *                                 |U_n[d][e]| over e (before scaling)
 *   S : half  [B][H][N][dk][dv]   state entering each chunk, row d stored
 *                                 divided by its scale sigS_n[d]
 *   scales : float [B][H][N][dk]  sigS_n[d], at off_scales
 * row_scale(m) is 1 for m < 2^14 and otherwise the power of two 2^e that
 * brings m / 2^e into [2^13, 2^14); the stored row times its scale is the
 * value. These are the three phases' arrays, as gla_chunk_summaries and
 * gla_state_scan leave them; the single-pass and runs schedules reuse the
 * same regions for their own publications (summaries with the pairs
 * (a_n[d], sigU_n[d]), segment or run aggregates and inclusive states), which
 * are not meant to be read. N = ceil(T / chunk).
 * Returns GLA_OK or GLA_E_ARG/GLA_E_UNSUPPORTED. */
int gla_workspace_layout(int B, int H, int grid_h, int grid_w, int dk, int dv,
                         int chunk, size_t* off_U, size_t* off_a,
                         size_t* off_S, size_t* off_scales,
                         size_t* total_bytes);

/* The whole forward: o = GLA(q, k, v, gk) along dir[b] for each batch
 * element b (GTR project page, "A Kernel That Makes Recurrence Fast"), on
 * the schedule gla_auto_schedule names (the three phases on an unprepared
 * workspace). o must not be the same buffer as any input. */
int gla_fwd(const void* q, const void* k, const void* v, const void* gk,
            void* o, int B, int H, int grid_h, int grid_w, int dk, int dv,
            const int32_t* dir, int chunk, int dtype, void* workspace,
            size_t workspace_bytes, void* stream);

/* The forward with a carried state (ai.info summary of GTR, "Future
 * Directions": carrying the recurrent state across frames; the deployed
 * operator fixes it at zero, "Methodology in Plain English"). Same as
 * gla_fwd, except that the state before the first scan token is s0 instead
 * of zero, and the state after the last scan token, S_T, is written to
 * s_final:
 *   s0      : const float [B][H][dk][dv], or NULL for a zero state;
 *   s_final : float [B][H][dk][dv], or NULL to skip the hand-back.
 * Both are in the scan's own frame (no spatial order); 16-byte aligned
 * device memory owned by the caller. s_final may be the same buffer as s0
 * (the state is then updated in place; such a call runs the three phases)
 * but must not otherwise overlap s0 (GLA_E_ARG), the workspace or any
 * tensor of the call. With both NULL this is gla_fwd. */
int gla_fwd_state(const void* q, const void* k, const void* v, const void* gk,
                  void* o, int B, int H, int grid_h, int grid_w, int dk, int dv,
                  const int32_t* dir, int chunk, int dtype, const float* s0,
                  float* s_final, void* workspace, size_t workspace_bytes,
                  void* stream);

/* The forward with the GLA block's output gate fused into the store (ai.info
 * summary of GTR, "Methodology in Plain English": a data-dependent output
 * gate applied to the RMS-normalised output). Per (batch, token, head) row:
 *   y = o / sqrt(mean_e(o_e^2) + eps) * norm_weight * silu(gate),
 *   silu(z) = z / (1 + exp(-z)),
 * with o the forward of gla_fwd_state (same s0 / s_final semantics), which is
 * not written itself. gate: [B][T][H][dv] in the input dtype (16-byte
 * aligned, not the same buffer as y); norm_weight: float [dv] (16-byte
 * aligned), shared by the heads; eps >= 0. Same schedules as gla_fwd. */
int gla_fwd_gated(const void* q, const void* k, const void* v, const void* gk,
                  const void* gate, const float* norm_weight, float eps, void* y,
                  int B, int H, int grid_h, int grid_w, int dk, int dv,
                  const int32_t* dir, int chunk, int dtype, const float* s0,
                  float* s_final, void* workspace, size_t workspace_bytes,
                  void* stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): gla_fwd without a
 * workspace argument. The workspace is a static device array of 64 MiB
 * inside the library, one per GPU, held until the process ends; the call
 * allocates nothing (no hipMalloc, no library allocation). Problems whose
 * gla_fwd_workspace_bytes exceed 64 MiB return GLA_E_WORKSPACE (with the
 * sizes in gla_last_error_detail). The first call on a GPU also enqueues one
 * small kernel on `stream` that zeroes the array's control words. Every call
 * on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (concurrent streams or threads) race and give wrong results; serialise
 * them. Otherwise the same as gla_fwd (GTR project page, "A Kernel That
 * Makes Recurrence Fast"). */
int gla_fwd_noalloc(const void* q, const void* k, const void* v, const void* gk,
                    void* o, int B, int H, int grid_h, int grid_w, int dk,
                    int dv, const int32_t* dir, int chunk, int dtype,
                    void* stream);

/* gla_fwd_state with an explicit schedule: GLA_SCHED_AUTO (what gla_fwd and
 * gla_fwd_state do), GLA_SCHED_SINGLE_PASS, GLA_SCHED_THREE_PHASE or
 * GLA_SCHED_RUNS. The single pass returns GLA_E_UNPREPARED on a workspace
 * gla_workspace_init has not prepared, and GLA_E_UNSUPPORTED if the problem
 * does not fit its control words (more than 4096 chunks per chain, or more
 * chunk-heads per launch than the 64 KiB hold) or if s_final is s0. The runs
 * schedule (one workgroup per run of consecutive 64-token chunks of a chain,
 * the run's chunks exchanging their states through LDS, a decoupled
 * look-back between runs) takes the same workspace preparation, supports
 * chunk 64 only, and returns GLA_E_UNSUPPORTED for other chunk sizes, for
 * s_final equal to s0, with an output gate, or when its per-run words do not
 * fit the 64 KiB. Results agree up to rounding. */
int gla_fwd_schedule(const void* q, const void* k, const void* v,
                     const void* gk, void* o, int B, int H, int grid_h,
                     int grid_w, int dk, int dv, const int32_t* dir, int chunk,
                     int dtype, const float* s0, float* s_final, int schedule,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The schedule gla_fwd and gla_fwd_state take for this shape on a prepared
 * workspace (GLA_SCHED_SINGLE_PASS or GLA_SCHED_THREE_PHASE; the dtype does
 * not matter), or GLA_E_ARG / GLA_E_UNSUPPORTED for a bad shape. */
int gla_auto_schedule(int B, int H, int grid_h, int grid_w, int dk, int dv,
                      int chunk);

/* Phase 1 alone: chunk summaries into the workspace's U and a (for every
 * (chunk, head) in parallel; ai.info summary of GTR, "Methodology in Plain
 * English"). U_n = sum_j diag(exp(B_n - b_j)) k_j^T v_j with b_j the
 * in-chunk inclusive cumulative log-decay and B_n its last value;
 * a_n = exp(B_n). */
int gla_chunk_summaries(const void* k, const void* v, const void* gk, int B,
                        int H, int grid_h, int grid_w, int dk, int dv,
                        const int32_t* dir, int chunk, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Phase 2 alone: boundary-state scan over the chunk axis, S_0 = s0 (zero if
 * s0 is NULL), S_{n+1} = diag(a_n) S_n + U_n, from the workspace's U and a
 * into its S (project page, "A Kernel That Makes Recurrence Fast": only the
 * boundary states are carried sequentially). If s_final is not NULL, the
 * state after the last chunk is written there. s0 and s_final as in
 * gla_fwd_state. */
int gla_state_scan(int B, int H, int grid_h, int grid_w, int dk, int dv,
                   int chunk, const float* s0, float* s_final, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Phase 3 alone: every chunk's outputs from its tokens and the workspace's
 * S: o_i = sum_{j<=i} A_ij v_j + (q_i * exp(b_i)) S_n with
 * A_ij = sum_d q_i[d] k_j[d] exp(b_i[d] - b_j[d]) (project page, "A Kernel
 * That Makes Recurrence Fast": one output kernel takes both the in-chunk
 * scores times values and the contribution of the entering state). */
int gla_chunk_outputs(const void* q, const void* k, const void* v,
                      const void* gk, void* o, int B, int H, int grid_h,
                      int grid_w, int dk, int dv, const int32_t* dir,
                      int chunk, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Writes perm[t] = raster index of the token at scan position t, for
 * t = 0 .. grid_h*grid_w-1, with the same device index arithmetic the loads
 * and stores use (project page, "How GTR Works": four scan orders).
 * perm_dev is device memory of grid_h*grid_w int32. */
int gla_scan_perm(int32_t* perm_dev, int grid_h, int grid_w, int dir,
                  void* stream);

/* Spatial SwiGLU core: the channel mixer of a GTR block (ai.info summary of
 * GTR, "Methodology in Plain English"; project page, "How GTR Works"), a
 * SwiGLU whose non-gated path is filtered per channel by a 3x3 kernel over
 * the patch grid. With the input projections already applied by the caller,
 * a (gate branch) and u (value branch), this computes for every token (y, x)
 * of the grid and channel c
 *   h[y][x][c] = silu(a[y][x][c]) * (bias[c] +
 *                 sum_{i,j=0..2} weight[c][i][j] * u[y+i-1][x+j-1][c])
 * with u taken as zero outside the grid and silu(z) = z / (1 + exp(-z)).
 *   a, u, h : [B][T][F] device memory, raster token order (token = y*grid_w+x),
 *             IEEE half (GLA_F16) or float (GLA_F32); 16-byte aligned;
 *             h must not be the same buffer as a or u.
 *   weight  : float [F][3][3] device memory; bias: float [F] or NULL.
 * F must be a multiple of 8 (GLA_E_UNSUPPORTED otherwise). Accumulation is
 * float. Asynchronous on `stream`; allocates nothing. */
int gla_spatial_swiglu(const void* a, const void* u, const float* weight,
                       const float* bias, void* h, int B, int grid_h,
                       int grid_w, int F, int dtype, void* stream);

/* Static text for a status code; never NULL. */
const char* gla_status_string(int status);

/* Detail of the last GLA_E_HIP or GLA_E_UNPREPARED on the calling thread
 * ("" if none). */
const char* gla_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* GLA_H_ */
