/*
 * mom.h -- C ABI of the MI355X Mixture-of-Memories (MoM) layer library (forward, decode,
 * and the gradients for training)
 * (libmom.so, HIP kernels for gfx950).
 *
 * The layer (arXiv 2502.13685, "MoM: Linear Sequence Modeling with
 * Mixture-of-Memories") is split into the parts the pages describe:
 *   mom_route        linear router: matmul, softmax, top-k, renormalisation
 *                    (podcast.do-not-panic.com page, "Router mechanics, step by
 *                    step"; research.elamur.ai summary, "Summary").
 *   mom_dispatch     tokens reordered into contiguous per-memory segments
 *                    (podcast.do-not-panic.com page, "Solving scatter-gather
 *                    without new kernels").
 *   mom_project      shared query projection, per-memory key/value projections
 *                    (research.elamur.ai summary: each memory has its own
 *                    key/value projections), keys L2-normalised per head.
 *   gdn_chunk_fwd    the single-memory Gated DeltaNet operator run over each
 *                    segment (jxzklqfsx.com write-up, hardware-efficient
 *                    implementation section: each memory reuses the
 *                    single-memory operator; the gist.science page, "Core
 *                    mechanism", restates the forget/delta update).
 *   gla_chunk_fwd    the same operator for memories that use gated linear
 *                    attention, the plain linear update that the other rules
 *                    modify (jxzklqfsx.com write-up, "Linear Recurrent Memory";
 *                    research.elamur.ai summary: MoM works with different
 *                    update rules).
 *   gdn_chunk_bwd    the gradients of gdn_chunk_fwd (and gla_chunk_bwd of
 *                    gla_chunk_fwd), for training.
 *   gdn_chunk_fwd_train, gdn_chunk_bwd_saved
 *                    the same forward and gradients split for a training
 *                    step: the forward keeps its chunk factors and states for
 *                    the backward, which then does not recompute them.
 *   mom_route_count, mom_dispatch_counted, mom_dispatch_counted_part
 *                    route and histogram in one launch (prefill and decode).
 *   gdn_decode_step_combined
 *                    the decode step with the combine folded in.
 *   gdn_decode_step  one recurrent step per sequence (constant-cost inference,
 *                    jxzklqfsx.com write-up, introduction and inference section).
 *   mom_combine      router-weighted sum of the per-memory reads plus the
 *                    always-on shared memory (jxzklqfsx.com write-up,
 *                    Mixture-of-Memories section and hardware-efficient
 *                    implementation section).
 *   mom_combine_bwd, mom_route_bwd, mom_dispatch_bwd
 *                    the gradients of the combine, of the router weights
 *                    (top-k held fixed) and of the dispatch gathers, for
 *                    training.
 *
 * Recurrence of one memory, per head, on a state S [dk][dv] (float32):
 *   S <- a S;  S <- S + c k (v - S^T k)^T;  o = S^T q      (a = alpha, c = beta)
 * A memory that a token is not routed to is not touched at that token.
 *
 * Conventions for every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates or frees device memory and never synchronises; each call
 *     validates its arguments on the host, enqueues its kernels on `stream`
 *     (a hipStream_t; NULL = the null stream) and returns.
 *   - Arguments are checked before any launch.  A failed check returns a
 *     negative mom_status and enqueues nothing.  A launch error returns
 *     MOM_ERR_LAUNCH.  Kernel faults surface on the stream, as with any HIP call.
 *   - Every pointer must be 16-byte aligned.  Inputs must be finite.
 *   - Forget gates alpha lie in [0, 1]; alpha = 0 clears the state at that row
 *     (the chunked entry points hold log alpha at or above -30, a decay of
 *     ~9e-14, so the result stays finite and equals the clearing to float32
 *     resolution).  The gradient entry points need alpha > 0.
 *   - Identical inputs give bit-identical outputs (no floating-point atomics).
 *   - Layouts are row-major with the shapes given below.
 *
 * Sizes derived from mom_dims: NT = B*T tokens (token id = b*T + t),
 * NR = NT*topk routed rows, N = NR + NT packed rows, n_seg = (M+1)*B segments,
 * n_state = B*(M+1) state slots, slot of (b, m) = b*(M+1) + m.
 *
 * Packed row order: segment s = m*B + b holds the tokens of sequence b routed
 * to memory m in increasing position; segments follow each other in s order.
 * Memory m = M is the shared memory: its segments hold every token, so rows
 * NR + (b*T + t) belong to it, in token order.
 *
 * Storage types: when dims->dtype == MOM_DTYPE_F32, x and the weights are
 * float32 and q/k/v are float32.  When dims->dtype == MOM_DTYPE_BF16, x and the
 * weights are bfloat16 and q/k/v are IEEE binary16 (half): keys have unit norm
 * and the queries/values of the layer stay far inside the half range, and half
 * carries 8x the precision of bfloat16 into the recurrence's matrix-core
 * products.  Gates, router weights, outputs and states are always float32.
 *
 * Supported shapes: dk in {64,128}; dv in {64,128,256}, and for every entry
 * point but gdn_decode_step also any multiple of 128 up to 1024; chunk == 64,
 * or 16, 32 or 64 with float32 storage (MOM_DTYPE_F32);
 * D % 64 == 0, 64 <= D <= 8192; 1 <= topk <= M <= 64, topk <= 8; B,T >= 1;
 * N < 2^31.
 */
#ifndef MOM_H_
#define MOM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mom_status {
  MOM_OK = 0,
  MOM_ERR_NULL = -1,        /* a required pointer is NULL */
  MOM_ERR_DIMS = -2,        /* a size is out of range or inconsistent */
  MOM_ERR_UNSUPPORTED = -3, /* a shape or dtype outside the supported set */
  MOM_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
  MOM_ERR_WORKSPACE = -5,   /* workspace missing or smaller than required */
  MOM_ERR_LAUNCH = -6,      /* the HIP runtime refused a kernel launch */
  MOM_ERR_TOO_LARGE = -7    /* sizes exceed the fixed scratch of an allocation-free entry point */
} mom_status;

enum { MOM_DTYPE_F32 = 0, MOM_DTYPE_BF16 = 1 };

typedef struct mom_dims {
  int32_t B;      /* sequences */
  int32_t T;      /* tokens per sequence */
  int32_t D;      /* model width */
  int32_t H;      /* heads */
  int32_t dk;     /* key dimension per head */
  int32_t dv;     /* value dimension per head */
  int32_t M;      /* routed memories (the shared memory is index M) */
  int32_t topk;   /* memories selected per token */
  int32_t chunk;  /* chunk length of the chunkwise recurrence (64; float32: 16, 32 or 64) */
  int32_t dtype;  /* MOM_DTYPE_F32 or MOM_DTYPE_BF16 */
} mom_dims;

/* Router.  For each token: logit_m = x . w_r[m] + bias[m] (accumulated in
 * float64; products of the stored inputs are exact), top-k memories by
 * decreasing logit with ties to the lower index, weights = softmax over all M
 * renormalised over the selected k (= softmax of the selected logits).
 *   x     [NT][D]   (dtype)          w_r  [M][D] (dtype)
 *   bias  [M] float32 or NULL (= 0)
 *   idx   [NT][topk] int32 out       w    [NT][topk] float32 out            */
mom_status mom_route(const mom_dims* dims, const void* x, const void* w_r, const float* bias,
                     int32_t* idx, float* w, void* stream);

/* Dispatch: stable counting sort of the (token, memory) pairs by (memory,
 * sequence), tokens in increasing position, plus the gates in packed order.
 *   idx      [NT][topk] int32 in (every entry in [0, M), distinct per token)
 *   x        [NT][D] (dtype) in, only read when x_packed != NULL
 *   alpha    [NT][H][M+1] float32 in,  beta same
 *   seg_off  [n_seg+1] int32 out: segment s = m*B+b covers [seg_off[s], seg_off[s+1])
 *   perm     [N] int32 out: token of each packed row (rows >= NR: identity)
 *   inv      [NT][topk] int32 out: packed row of (token, j)
 *   x_packed [NR][D] (dtype) out or NULL: x gathered in packed order
 *   alpha_p  [N][H] float32 out: alpha[perm[r]][h][memory of r]; beta_p same
 *   ws       workspace of at least mom_workspace_bytes(dims, MOM_WS_DISPATCH)  */
mom_status mom_dispatch(const mom_dims* dims, const int32_t* idx, const void* x, const float* alpha,
                        const float* beta, int32_t* seg_off, int32_t* perm, int32_t* inv,
                        void* x_packed, float* alpha_p, float* beta_p, void* ws, size_t ws_bytes,
                        void* stream);

/* mom_dispatch without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The same outputs as mom_dispatch (bit for bit);
 * every other argument, layout and error as there.  The dispatch's counts
 * (int32 [M][B][ceil(T / 64)], M*B*ceil(T / 64) <= 32768) and their scan live
 * in a fixed 256 KiB array of the library's own in each GPU's memory, held from the
 * first call on that GPU until the process ends; larger sizes return
 * MOM_ERR_TOO_LARGE before any launch.  The call allocates nothing.  The
 * array's device address is looked up on the first call on each GPU, so
 * stream (NULL = the null stream) must belong to the current device (else
 * MOM_ERR_DIMS).  Every call on one GPU uses the same array: calls that can
 * overlap on that GPU (e.g. on two streams without ordering between them)
 * race and must be serialised by the caller. */
mom_status mom_dispatch_noalloc(const mom_dims* dims, const int32_t* idx, const void* x, const float* alpha,
                                const float* beta, int32_t* seg_off, int32_t* perm, int32_t* inv,
                                void* x_packed, float* alpha_p, float* beta_p, void* stream);

/* Route and histogram in one pass (podcast.do-not-panic.com page, "Solving
 * scatter-gather without new kernels": the counting sort's histogram comes
 * from the router's own pass): the outputs of mom_route, and the dispatch's
 * counts of every 64 positions of every sequence per memory (int32
 * [M][B][ceil(T / 64)], every entry written, nothing to clear) in ws (at
 * least mom_workspace_bytes(dims, MOM_WS_DISPATCH) bytes), which
 * mom_dispatch_counted and mom_dispatch_counted_part then read instead of
 * counting again.  One launch for bfloat16 rows with D = 1024 and M <= 16 or
 * D = 2048 and M <= 4, and for T == 1 (a decode step); other shapes run
 * mom_route's kernel and then the dispatch's counting kernel.  idx and w are those of mom_route (the
 * selections and weights of the same exact logits). */
mom_status mom_route_count(const mom_dims* dims, const void* x, const void* w_r, const float* bias,
                           int32_t* idx, float* w, void* ws, size_t ws_bytes, void* stream);

/* mom_dispatch when ws holds the counts mom_route_count wrote for the same idx
 * and dims: the same outputs, without the counting launch.  The counts are
 * left as they are, so the call can be repeated on them. */
mom_status mom_dispatch_counted(const mom_dims* dims, const int32_t* idx, const void* x, const float* alpha,
                                const float* beta, int32_t* seg_off, int32_t* perm, int32_t* inv,
                                void* x_packed, float* alpha_p, float* beta_p, void* ws, size_t ws_bytes,
                                void* stream);

/* mom_dispatch_part (parts as there) reading the counts of mom_route_count
 * from ws like mom_dispatch_counted; part 1 reads neither. */
mom_status mom_dispatch_counted_part(const mom_dims* dims, const int32_t* idx, const void* x, const float* alpha,
                                     const float* beta, int32_t* seg_off, int32_t* perm, int32_t* inv,
                                     void* x_packed, float* alpha_p, float* beta_p, void* ws, size_t ws_bytes,
                                     int32_t part, void* stream);

/* Projections.  q[t] = w_q x[t] for every token; for packed row r of memory m
 * (from seg_off): k[r] = w_k[m] x[perm[r]] normalised to unit L2 norm per head
 * (no epsilon), v[r] = w_v[m] x[perm[r]].  Accumulation in float32.
 *   x [NT][D], w_q [H*dk][D], w_k [M+1][H*dk][D], w_v [M+1][H*dv][D] (dtype)
 *   seg_off, perm: as written by mom_dispatch
 *   q [NT][H][dk], k [N][H][dk], v [N][H][dv] out (float32 or half, see above) */
mom_status mom_project(const mom_dims* dims, const void* x, const int32_t* perm,
                       const int32_t* seg_off, const void* w_q, const void* w_k, const void* w_v,
                       void* q, void* k, void* v, void* stream);

/* The same two steps in parts, so that the shared memory's path, which
 * needs no routing, can run on another stream beside the routed one:
 *   part 0 = everything (mom_dispatch / mom_project);
 *   part 1 = the shared memory: mom_dispatch_part writes its rows (row NR + t
 *            holds token t: perm, alpha_p, beta_p) and seg_off[M*B .. (M+1)*B]
 *            and reads neither idx nor inv nor ws (may be NULL);
 *            mom_project_part writes q (all tokens) and k, v of rows
 *            NR .. N and reads neither perm nor seg_off (may be NULL);
 *   part 2 = the routed memories: mom_dispatch_part writes their rows, inv and
 *            seg_off[0 .. M*B]; mom_project_part writes k, v of rows 0 .. NR
 *            (reads perm and seg_off as written by part 2).
 * Parts 1 and 2 write disjoint rows and only the common entry seg_off[M*B] =
 * NR twice (the same value).  Other arguments, layouts and errors as
 * mom_dispatch / mom_project; part outside 0..2 returns MOM_ERR_DIMS. */
mom_status mom_dispatch_part(const mom_dims* dims, const int32_t* idx, const void* x, const float* alpha,
                             const float* beta, int32_t* seg_off, int32_t* perm, int32_t* inv,
                             void* x_packed, float* alpha_p, float* beta_p, void* ws, size_t ws_bytes,
                             int32_t part, void* stream);
mom_status mom_project_part(const mom_dims* dims, const void* x, const int32_t* perm,
                            const int32_t* seg_off, const void* w_q, const void* w_k, const void* w_v,
                            void* q, void* k, void* v, int32_t part, void* stream);

/* Chunkwise Gated DeltaNet over packed segments.  Segment s (rows
 * [seg_off[s], seg_off[s+1]) of the row arrays) runs the recurrence above in
 * row order from state slot seg_state[s] (NULL: slot s); different segments
 * must use different slots.  Chunks of dims->chunk rows are processed in the
 * WY/UT form, which equals the token recurrence up to rounding.  With half
 * storage, when the call has so few segments and heads that the walk would
 * run at most 8 blocks and its segments are long, each segment is cut into
 * groups of chunks whose affine state maps are walked in parallel and then
 * chained (the long-segment scan): the same result up to rounding.
 *   q         [n_tok][H][dk] read at row row_token[r] (NULL: row r itself)
 *   k [N][H][dk], v [N][H][dv] (float32 or half per dims->dtype)
 *   alpha_p, beta_p [N][H] float32
 *   state_in  [n_state][H][dk][dv] float32 or NULL (zeros); may equal state_out
 *   state_out [n_state][H][dk][dv] float32; slots of segments run are written
 *             (an empty segment copies its state unchanged)
 *   o         [N][H][dv] float32: the read after each row's write
 * Preconditions: seg_off non-decreasing with seg_off[n_seg] <= n_rows,
 * row_token entries in [0, n_tok).  ws holds at least
 * gdn_chunk_workspace_bytes(dims, n_seg, n_rows) bytes (may be NULL when that
 * is 0); its contents on entry do not matter.                                */
mom_status gdn_chunk_fwd(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                         int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                         const int32_t* row_token, const void* q, const void* k, const void* v,
                         const float* alpha_p, const float* beta_p, const float* state_in,
                         float* state_out, float* o, void* ws, size_t ws_bytes, void* stream);

/* gla_chunk_fwd: as gdn_chunk_fwd (same arguments, layouts, workspace,
 * ownership and errors) for memories whose update is gated linear attention:
 *   S <- a S;  S <- S + c k v^T;  o = S^T q      (a = alpha, c = beta)
 * (a = c = 1: plain causal linear attention).  The pages' formula for this
 * basic linear update was lost in extraction; this reading keeps the Gated
 * DeltaNet gate inputs and drops the delta correction. */
mom_status gla_chunk_fwd(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                         int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                         const int32_t* row_token, const void* q, const void* k, const void* v,
                         const float* alpha_p, const float* beta_p, const float* state_in,
                         float* state_out, float* o, void* ws, size_t ws_bytes, void* stream);

/* Gradients of gdn_chunk_fwd (reverse mode), for training: given
 * d_o = dL/do and dstate_out = dL/d(final states), the gradients of L with
 * respect to the forward's inputs.  The pages give no backward formulas (the
 * jxzklqfsx.com write-up, introduction, states that the layer trains in linear
 * time); these are the chain rule applied to the recurrence above, evaluated
 * in the same chunk form (half operands on the matrix cores, float32
 * accumulation and states) for half storage (dims->dtype == MOM_DTYPE_BF16),
 * where every alpha of the rows run must be > 0 (d_alpha = d(log alpha) /
 * alpha); with float32 storage as a row-by-row reverse sweep in float32 that
 * recomputes the states from ones kept every 64 and every 8 rows (any alpha
 * in [0, 1]).
 *   inputs:   as gdn_chunk_fwd (dims, segments, slots, row_token, q, k, v,
 *             alpha_p, beta_p, state_in or NULL = zeros)
 *   d_o        [N][H][dv] float32
 *   dstate_out [n_state][H][dk][dv] float32 or NULL (zeros)
 *   dq         [N][H][dk] float32 out: per packed row, the gradient of the
 *              query as that row uses it (rows that read the same token are
 *              not summed; the caller adds them)
 *   dk [N][H][dk], dv [N][H][dv], d_alpha, d_beta [N][H] float32 out
 *   dstate_in  [n_state][H][dk][dv] float32 out: dL/d(entering state); the
 *              slots of the segments given are written (an empty segment
 *              copies its dstate_out), others are left as they are
 * Rows outside every segment are not written.  Different segments must use
 * different slots.  ws holds at least gdn_chunk_bwd_workspace_bytes(dims,
 * n_seg, n_rows) bytes; its contents on entry do not matter.  Other errors as
 * gdn_chunk_fwd. */
mom_status gdn_chunk_bwd(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                         int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                         const int32_t* row_token, const void* q, const void* k, const void* v,
                         const float* alpha_p, const float* beta_p, const float* state_in,
                         const float* d_o, const float* dstate_out, float* dq, float* dk, float* dv,
                         float* d_alpha, float* d_beta, float* dstate_in, void* ws, size_t ws_bytes,
                         void* stream);

/* gla_chunk_bwd: the gradients of gla_chunk_fwd, with the arguments, layouts,
 * workspace and errors of gdn_chunk_bwd. */
mom_status gla_chunk_bwd(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                         int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                         const int32_t* row_token, const void* q, const void* k, const void* v,
                         const float* alpha_p, const float* beta_p, const float* state_in,
                         const float* d_o, const float* dstate_out, float* dq, float* dk, float* dv,
                         float* d_alpha, float* d_beta, float* dstate_in, void* ws, size_t ws_bytes,
                         void* stream);

/* The forward pass of a training step: the outputs of gdn_chunk_fwd (same
 * arguments, layouts and errors), and ws, which must hold
 * gdn_chunk_bwd_workspace_bytes(dims, n_seg, n_rows) bytes, keeps what
 * gdn_chunk_bwd_saved reads: with half storage each chunk's solved triangular
 * factor, its inverse, the masked query-key products, the decay prefix sums
 * and the state entering the chunk (with float32 storage nothing: its
 * backward recomputes the states).  o and state_out equal gdn_chunk_fwd's bit
 * for bit when gdn_chunk_fwd walks every segment whole (with the
 * long-segment scan they agree to rounding). */
mom_status gdn_chunk_fwd_train(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                               int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                               const int32_t* row_token, const void* q, const void* k, const void* v,
                               const float* alpha_p, const float* beta_p, const float* state_in,
                               float* state_out, float* o, void* ws, size_t ws_bytes, void* stream);

/* gla_chunk_fwd_train: gla_chunk_fwd's outputs, with ws kept as in
 * gdn_chunk_fwd_train. */
mom_status gla_chunk_fwd_train(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                               int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                               const int32_t* row_token, const void* q, const void* k, const void* v,
                               const float* alpha_p, const float* beta_p, const float* state_in,
                               float* state_out, float* o, void* ws, size_t ws_bytes, void* stream);

/* gdn_chunk_bwd_saved: gdn_chunk_bwd when ws still holds what
 * gdn_chunk_fwd_train wrote for the same dims, segments, slots, rows, inputs
 * and state_in (the caller keeps them unchanged in between); it skips the
 * factor and state recomputation and its results equal gdn_chunk_bwd's bit
 * for bit.  Arguments, layouts and errors as gdn_chunk_bwd; ws is read and
 * then overwritten, so one training forward serves one backward. */
mom_status gdn_chunk_bwd_saved(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                               int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                               const int32_t* row_token, const void* q, const void* k, const void* v,
                               const float* alpha_p, const float* beta_p, const float* state_in,
                               const float* d_o, const float* dstate_out, float* dq, float* dk,
                               float* dv, float* d_alpha, float* d_beta, float* dstate_in, void* ws,
                               size_t ws_bytes, void* stream);

/* gla_chunk_bwd_saved: gdn_chunk_bwd_saved for gla_chunk_fwd_train's
 * workspace. */
mom_status gla_chunk_bwd_saved(const mom_dims* dims, int32_t n_seg, int32_t n_rows, int32_t n_tok,
                               int32_t n_state, const int32_t* seg_off, const int32_t* seg_state,
                               const int32_t* row_token, const void* q, const void* k, const void* v,
                               const float* alpha_p, const float* beta_p, const float* state_in,
                               const float* d_o, const float* dstate_out, float* dq, float* dk,
                               float* dv, float* d_alpha, float* d_beta, float* dstate_in, void* ws,
                               size_t ws_bytes, void* stream);

/* One recurrent step for n_seq sequences with one new token each (T = 1 view:
 * rows as written by mom_dispatch/mom_project for dims with B = n_seq, T = 1).
 * For sequence b and slot j < topk the memory is idx[b][j] and the packed row
 * inv[b][j]; slot topk is the shared memory M at row NR + b.  The state of
 * (b, memory) is updated in place; memories not selected are not touched.
 *   idx, inv  [n_seq][topk] int32
 *   q [n_seq][H][dk], k [N][H][dk], v [N][H][dv] (float32 or half)
 *   alpha, beta [n_seq][H][M+1] float32
 *   states [n_seq][M+1][H][dk][dv] float32, updated in place
 *   o [N][H][dv] float32 out (packed rows, as gdn_chunk_fwd)                   */
mom_status gdn_decode_step(const mom_dims* dims, int32_t n_seq, const int32_t* idx,
                           const int32_t* inv, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, float* states, float* o,
                           void* stream);

/* gla_decode_step: as gdn_decode_step (same arguments, layouts and errors) for
 * gated linear attention memories: S <- a S + c k v^T, o = S^T q. */
mom_status gla_decode_step(const mom_dims* dims, int32_t n_seq, const int32_t* idx,
                           const int32_t* inv, const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta, float* states, float* o,
                           void* stream);

/* gdn_decode_step_combined / gla_decode_step_combined: the decode step with
 * mom_combine folded in (jxzklqfsx.com write-up, Mixture-of-Memories section:
 * the layer's output is the weighted mixture of the memories' reads plus the
 * shared memory's).  One block per (sequence, head) updates the shared
 * memory's state and then the routed ones in order, and adds their reads as
 * mom_combine does (shared first, then w[s][j] times slot j's read, j
 * ascending, one fused multiply-add each), so out equals gdn_decode_step
 * followed by mom_combine bit for bit; no per-slot outputs are written.
 *   w   [n_seq][topk] float32 (from mom_route)
 *   out [n_seq][H][dv] float32 out
 * Other arguments, layouts and errors as gdn_decode_step (o replaced by out). */
mom_status gdn_decode_step_combined(const mom_dims* dims, int32_t n_seq, const int32_t* idx,
                                    const int32_t* inv, const float* w, const void* q, const void* k,
                                    const void* v, const float* alpha, const float* beta, float* states,
                                    float* out, void* stream);
mom_status gla_decode_step_combined(const mom_dims* dims, int32_t n_seq, const int32_t* idx,
                                    const int32_t* inv, const float* w, const void* q, const void* k,
                                    const void* v, const float* alpha, const float* beta, float* states,
                                    float* out, void* stream);

/* Combine: out[t] = o_shared[t] + sum_j w[t][j] * o_routed[row(t, j)], shared
 * first then j ascending, float32, row(t, j) = inv[t][j] (NULL: t*topk + j).
 *   o_routed [*][H][dv], o_shared [n_tok][H][dv], out [n_tok][H][dv] float32  */
mom_status mom_combine(const mom_dims* dims, int32_t n_tok, const int32_t* inv, const float* w,
                       const float* o_routed, const float* o_shared, float* out, void* stream);

/* Gradients of the combine (for training; the chain rule of the sum above):
 *   d_o_routed[row(t, j)] = w[t][j] dout[t],  d_o_shared[t] = dout[t],
 *   dw[t][j] = <dout[t], o_routed[row(t, j)]>  (sum over H * dv, one wave per
 *   token, fixed order).  Rows of d_o_routed no token reads are not written.
 *   dout [n_tok][H][dv], d_o_shared [n_tok][H][dv], d_o_routed [*][H][dv],
 *   dw [n_tok][topk] float32 out; other arguments as mom_combine.        */
mom_status mom_combine_bwd(const mom_dims* dims, int32_t n_tok, const int32_t* inv, const float* w,
                           const float* o_routed, const float* dout, float* d_o_routed, float* d_o_shared,
                           float* dw, void* stream);

/* Gradients of the router weights (for training), with the top-k choice held
 * fixed: no gradient flows through the selection, only through the
 * renormalised softmax weights of the selected memories.
 *   dl[t][idx_j] = w_j (dw_j - sum_j' w_j' dw_j'),  dl = 0 for the others
 *   dx[t] = sum_m dl[t][m] w_r[m]        ([NT][D] float32 out)
 *   dw_r[m] = sum_t dl[t][m] x[t]        ([M][D] float32 out)
 *   dbias[m] = sum_t dl[t][m]            ([M] float32 out, or NULL)
 * x, w_r as mom_route; idx, w as written by mom_route; dw [NT][topk] float32
 * (e.g. from mom_combine_bwd).  Sums over tokens run in a fixed order (tiles
 * of 256 tokens, then the tiles in order).  ws holds at least
 * mom_workspace_bytes(dims, MOM_WS_ROUTE_BWD) bytes. */
mom_status mom_route_bwd(const mom_dims* dims, const void* x, const void* w_r, const int32_t* idx,
                         const float* w, const float* dw, float* dx, float* dw_r, float* dbias, void* ws,
                         size_t ws_bytes, void* stream);

/* The dispatch gathers in reverse (for training): gate gradients per packed
 * row go back to [token][head][memory] (d_alpha[t][h][idx[t][j]] =
 * d_alpha_p[inv[t][j]][h], d_alpha[t][h][M] = d_alpha_p[NR + t][h], every
 * other memory 0; the same for beta), and the query gradients of a token's
 * rows are summed: dq[t] = dq_rows[NR + t] + sum_j dq_rows[inv[t][j]] (shared
 * row first, then j).
 *   idx, inv [NT][topk] int32 (mom_route, mom_dispatch)
 *   d_alpha_p, d_beta_p [N][H], dq_rows [N][H][dk] float32 (gdn_chunk_bwd)
 *   d_alpha, d_beta [NT][H][M+1], dq [NT][H][dk] float32 out               */
mom_status mom_dispatch_bwd(const mom_dims* dims, const int32_t* idx, const int32_t* inv,
                            const float* d_alpha_p, const float* d_beta_p, const float* dq_rows,
                            float* d_alpha, float* d_beta, float* dq, void* stream);

enum { MOM_WS_DISPATCH = 0, MOM_WS_CHUNK = 1, MOM_WS_ROUTE_BWD = 2 };
/* Workspace bytes an entry point needs for the layer's own sizes (0 = none):
 * MOM_WS_DISPATCH for mom_dispatch, MOM_WS_CHUNK for gdn_chunk_fwd over the
 * layer's n_seg = (M+1)*B segments and N rows, MOM_WS_ROUTE_BWD for
 * mom_route_bwd.  0 for invalid dims. */
size_t mom_workspace_bytes(const mom_dims* dims, int32_t which);

/* Workspace bytes gdn_chunk_fwd needs for n_seg segments over n_rows packed
 * rows (0 = none: the float32 path keeps everything on chip).  The bfloat16
 * path stores, per (chunk, head), the chunk's solved triangular factor and its
 * masked, decayed query-key products (half) and the log-decay prefix sums
 * (float32).  0 for invalid arguments. */
size_t gdn_chunk_workspace_bytes(const mom_dims* dims, int32_t n_seg, int32_t n_rows);

/* Workspace bytes gdn_chunk_bwd / gla_chunk_bwd need for n_seg segments over
 * n_rows packed rows: the forward's per-chunk factors, X = (I + A)^{-1}, and
 * the states entering and the state gradients leaving every chunk (all
 * half but the float32 decay sums).  0 for invalid arguments or float32 storage. */
size_t gdn_chunk_bwd_workspace_bytes(const mom_dims* dims, int32_t n_seg, int32_t n_rows);

/* Static text for a status code. */
const char* mom_status_string(int32_t status);

#ifdef __cplusplus
}
#endif
#endif /* MOM_H_ */
