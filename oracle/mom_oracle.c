/*
 * Reference checker for the Mixture-of-Memories (MoM) layer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, token-by-token fp64
 * implementation of what the layer computes.  It shares no code, header, table
 * or helper with the GPU library and must never be called by the product path:
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark use
 * it.  Every floating-point step runs in double precision, in the order the
 * definition states, with no blocking, fusion or reordering.
 *
 * Sources (web pages on "MoM: Linear Sequence Modeling with Mixture-of-Memories",
 * arXiv 2502.13685):
 *   [p1] jxzklqfsx.com write-up, sections "Mixture-of-Memories" and the
 *        hardware-efficient implementation section;
 *   [p2] research.elamur.ai summary, "Summary" paragraph;
 *   [p4] podcast.do-not-panic.com visual page, "Router mechanics, step by step"
 *        and "Solving scatter-gather without new kernels";
 *   [p5] gist.science page on Sparse Delta Memory, "Core mechanism", which
 *        restates the Gated DeltaNet forget / delta update.
 *
 * Readings taken where the pages are silent (formulas on [p1] were lost in
 * extraction): keys are L2-normalised per head with no epsilon; queries are
 * used as projected (no normalisation, no 1/sqrt(dk) scale); the output is read
 * after the write; the shared memory is added with weight 1; a memory that a
 * token is not routed to is left untouched (no decay, no write); routing ties go
 * to the lower memory index; there is no output projection after the mixture.
 *
 * Layouts (row-major, all double unless noted):
 *   x [NT][D], wr [M][D], bias [M] (or NULL), wq [H*dk][D],
 *   wk [M+1][H*dk][D], wv [M+1][H*dv][D], alpha/beta [NT][H][M+1],
 *   state [B][M+1][H][dk][dv].   Token t_g = b*T + t.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Router ([p4] "Router mechanics": one matmul, one softmax, one top-k, one
 * renormalisation; [p2] "a linear router sends each token to its top-k
 * memories").  For every token:
 *   logit_m = sum_d x[d] * wr[m][d] + bias[m]
 *   p       = softmax over all M logits
 *   top-k   = the k memories with the largest p, ties to the lower index.
 *             softmax is strictly increasing in the logit, so the order is
 *             decided on the logits themselves (fp64 exp could merge two
 *             nearby probabilities, the logits cannot).
 *   w_j     = p[idx_j] / sum_{j'} p[idx_j']      (renormalisation)
 * idx_j is listed by decreasing logit.                                       */
void oracle_route(int64_t n_tok, int D, int M, int K, const double* x, const double* wr,
                  const double* bias, int32_t* idx, double* w, double* logits_out) {
  double* logit = (double*)malloc(sizeof(double) * (size_t)M);
  double* p = (double*)malloc(sizeof(double) * (size_t)M);
  char* taken = (char*)malloc((size_t)M);
  for (int64_t t = 0; t < n_tok; ++t) {
    const double* xt = x + t * D;
    for (int m = 0; m < M; ++m) {
      double s = 0.0;
      for (int d = 0; d < D; ++d) s += xt[d] * wr[(int64_t)m * D + d];
      logit[m] = s + (bias ? bias[m] : 0.0);
      if (logits_out) logits_out[t * M + m] = logit[m];
    }
    /* softmax over all memories */
    double mx = logit[0];
    for (int m = 1; m < M; ++m)
      if (logit[m] > mx) mx = logit[m];
    double z = 0.0;
    for (int m = 0; m < M; ++m) {
      p[m] = exp(logit[m] - mx);
      z += p[m];
    }
    for (int m = 0; m < M; ++m) p[m] /= z;
    /* top-k: repeatedly take the largest remaining logit; a strict '>' keeps
       the lowest index among equal logits */
    memset(taken, 0, (size_t)M);
    for (int j = 0; j < K; ++j) {
      int best = -1;
      for (int m = 0; m < M; ++m) {
        if (taken[m]) continue;
        if (best < 0 || logit[m] > logit[best]) best = m;
      }
      taken[best] = 1;
      idx[t * K + j] = best;
    }
    /* renormalise the selected probabilities */
    double zs = 0.0;
    for (int j = 0; j < K; ++j) zs += p[idx[t * K + j]];
    for (int j = 0; j < K; ++j) w[t * K + j] = p[idx[t * K + j]] / zs;
  }
  free(logit);
  free(p);
  free(taken);
}

/* ------------------------------------------------------------------------- */
/* Dispatch as sequence reordering ([p4] "Solving scatter-gather without new
 * kernels": routed tokens are reordered into contiguous per-memory segments).
 * Rows are laid out memory by memory, batch by batch, tokens in increasing
 * position; the shared memory (index M) follows as one more group holding every
 * token in (b, t) order.  Segment s = m*B + b covers rows
 * [seg_off[s], seg_off[s+1]).  perm[row] = token; inv[token][j] = row of the
 * token's j-th routed memory.                                               */
void oracle_dispatch(int B, int T, int M, int K, const int32_t* idx, int32_t* seg_off,
                     int32_t* perm, int32_t* inv) {
  int32_t row = 0;
  for (int m = 0; m <= M; ++m) {
    for (int b = 0; b < B; ++b) {
      seg_off[m * B + b] = row;
      for (int t = 0; t < T; ++t) {
        int32_t tok = b * T + t;
        if (m == M) {
          perm[row++] = tok;
          continue;
        }
        for (int j = 0; j < K; ++j) {
          if (idx[(int64_t)tok * K + j] == m) {
            perm[row] = tok;
            inv[(int64_t)tok * K + j] = row;
            ++row;
          }
        }
      }
    }
  }
  seg_off[(M + 1) * B] = row;
}

/* ------------------------------------------------------------------------- */
/* Projections ([p2]: each memory has its own key/value projections; the query
 * projection is shared).  For one token x and one head h:
 *   q = Wq[h] x,  khat = Wk[m][h] x,  k = khat / ||khat||_2,  v = Wv[m][h] x. */
static void proj_rows(int D, int n_out, const double* W, const double* x, double* y) {
  for (int c = 0; c < n_out; ++c) {
    double s = 0.0;
    const double* wc = W + (int64_t)c * D;
    for (int d = 0; d < D; ++d) s += wc[d] * x[d];
    y[c] = s;
  }
}

static void l2_normalise(int n, double* k) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += k[i] * k[i];
  double r = sqrt(s);
  for (int i = 0; i < n; ++i) k[i] /= r;
}

/* q for one token, all heads: q[H*dk] */
void oracle_project_q(int D, int H, int dk, const double* x_tok, const double* wq, double* q) {
  proj_rows(D, H * dk, wq, x_tok, q);
}

/* k (normalised per head) and v of one token for one memory m: k[H*dk], v[H*dv] */
void oracle_project_kv(int D, int H, int dk, int dv, int m, const double* x_tok, const double* wk,
                       const double* wv, double* k, double* v) {
  proj_rows(D, H * dk, wk + (int64_t)m * H * dk * D, x_tok, k);
  for (int h = 0; h < H; ++h) l2_normalise(dk, k + h * dk);
  proj_rows(D, H * dv, wv + (int64_t)m * H * dv * D, x_tok, v);
}

/* ------------------------------------------------------------------------- */
/* One Gated DeltaNet step on a d_k x d_v matrix memory ([p5] "Core mechanism",
 * gated delta update, read densely; [p1] each memory uses the Gated DeltaNet
 * gate and update rule):
 *   forget:  S~ = a * S
 *   delta:   S  = S~ + c * k (v - S~^T k)^T
 *   read:    o  = S^T q          (after the write)
 * S is [dk][dv]: rows are key dimensions, columns value dimensions.           */
void oracle_gdn_step(int dk, int dv, double a, double c, const double* q, const double* k,
                     const double* v, double* S, double* o) {
  for (int i = 0; i < dk * dv; ++i) S[i] *= a;
  for (int j = 0; j < dv; ++j) {
    double pred = 0.0;
    for (int i = 0; i < dk; ++i) pred += S[i * dv + j] * k[i];
    double e = c * (v[j] - pred);
    for (int i = 0; i < dk; ++i) S[i * dv + j] += k[i] * e;
  }
  for (int j = 0; j < dv; ++j) {
    double s = 0.0;
    for (int i = 0; i < dk; ++i) s += S[i * dv + j] * q[i];
    o[j] = s;
  }
}

/* One step of gated linear attention, the plain linear recurrence that the
 * other update rules modify ([p1] "Linear Recurrent Memory": the basic
 * linear-attention RNN update, with gates and update rules as variations of
 * it; [p2] "Summary": MoM works with different update rules).  The formula
 * on [p1] was lost in extraction; the reading taken here keeps the Gated
 * DeltaNet gate inputs and drops the delta correction:
 *   forget:  S~ = a * S
 *   write:   S  = S~ + c * k v^T
 *   read:    o  = S^T q          (after the write)
 * a = c = 1 is plain causal linear attention.                                */
void oracle_gla_step(int dk, int dv, double a, double c, const double* q, const double* k,
                     const double* v, double* S, double* o) {
  for (int i = 0; i < dk * dv; ++i) S[i] *= a;
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[i * dv + j] += c * k[i] * v[j];
  for (int j = 0; j < dv; ++j) {
    double s = 0.0;
    for (int i = 0; i < dk; ++i) s += S[i * dv + j] * q[i];
    o[j] = s;
  }
}

/* Update rules of a memory: 0 = Gated DeltaNet, 1 = gated linear attention. */
typedef void (*oracle_step_fn)(int, int, double, double, const double*, const double*, const double*,
                               double*, double*);
static oracle_step_fn step_of(int rule) { return rule == 1 ? oracle_gla_step : oracle_gdn_step; }

/* The recurrence over one memory's own token sequence (length L): rows are the
 * tokens routed to that memory, in order.  q/k [L][dk], v/o [L][dv], a/c [L]. */
void oracle_gla_chain(int64_t L, int dk, int dv, const double* q, const double* k, const double* v,
                      const double* a, const double* c, double* S, double* o) {
  for (int64_t i = 0; i < L; ++i)
    oracle_gla_step(dk, dv, a[i], c[i], q + i * dk, k + i * dk, v + i * dv, S, o + i * dv);
}

void oracle_gdn_chain(int64_t L, int dk, int dv, const double* q, const double* k, const double* v,
                      const double* a, const double* c, double* S, double* o) {
  for (int64_t i = 0; i < L; ++i)
    oracle_gdn_step(dk, dv, a[i], c[i], q + i * dk, k + i * dk, v + i * dv, S, o + i * dv);
}

/* ------------------------------------------------------------------------- */
/* The whole layer, token by token.
 *
 * dims = {B, T, D, H, dk, dv, M, K}.  For each sequence b and head h, the
 * M+1 memories are kept side by side and the tokens are visited in order.  At
 * token t the memories in idx[t] plus the shared memory M take one step each
 * (with their own k, v and gates); every other memory is left as it is.  The
 * token's output mixes the per-memory reads with the router weights, the shared
 * memory entering with weight 1 ([p1] hardware-efficient implementation: each
 * memory reuses the single-memory operator and the outputs are summed with the
 * weights, equivalent to reading from the weighted mixture of memories; [p1]
 * shared memory: every token passes through it).
 *
 * Outputs (any may be NULL):
 *   idx [NT][K], w [NT][K]        router result
 *   o_routed [NT][K][H][dv]       per-memory read for the token's j-th memory
 *   o_shared [NT][H][dv]          shared-memory read
 *   out [NT][H][dv]               o_shared + sum_j w_j o_routed[j]
 *   out_mixed [NT][H][dv]         read from the mixed memory
 *                                 (S_shared + sum_j w_j S_idx_j)^T q
 *   state [B][M+1][H][dk][dv]     in: initial state (NULL input = zeros via
 *                                 state0 == NULL), out: final state
 *   q_out [NT][H][dk], k_out/v_out [NT][K+1][H][dk|dv]  projected vectors
 *                                 (slot K = shared memory)
 * Work is split over (b, h) pairs, which are independent.                    */
void oracle_layer_rule(int rule, const int32_t* dims, const double* x, const double* wr, const double* bias,
                       const double* wq, const double* wk, const double* wv, const double* alpha,
                       const double* beta, const double* state0, int32_t* idx, double* w,
                       double* o_routed, double* o_shared, double* out, double* out_mixed,
                       double* state, double* q_out, double* k_out, double* v_out) {
  const oracle_step_fn step = step_of(rule);
  const int B = dims[0], T = dims[1], D = dims[2], H = dims[3], dk = dims[4], dv = dims[5];
  const int M = dims[6], K = dims[7];
  const int64_t NT = (int64_t)B * T;
  const int64_t ssz = (int64_t)dk * dv;

  int32_t* idx_l = idx ? idx : (int32_t*)malloc(sizeof(int32_t) * NT * K);
  double* w_l = w ? w : (double*)malloc(sizeof(double) * NT * K);
  oracle_route(NT, D, M, K, x, wr, bias, idx_l, w_l, NULL);

  /* projections for every token: q, and k/v for its K routed memories + shared */
  double* q_all = (double*)malloc(sizeof(double) * NT * H * dk);
  double* k_all = (double*)malloc(sizeof(double) * NT * (K + 1) * H * dk);
  double* v_all = (double*)malloc(sizeof(double) * NT * (K + 1) * H * dv);
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < NT; ++t) {
    const double* xt = x + t * D;
    oracle_project_q(D, H, dk, xt, wq, q_all + t * H * dk);
    for (int j = 0; j <= K; ++j) {
      int m = (j < K) ? idx_l[t * K + j] : M;
      oracle_project_kv(D, H, dk, dv, m, xt, wk, wv, k_all + (t * (K + 1) + j) * H * dk,
                        v_all + (t * (K + 1) + j) * H * dv);
    }
  }
  if (q_out) memcpy(q_out, q_all, sizeof(double) * NT * H * dk);
  if (k_out) memcpy(k_out, k_all, sizeof(double) * NT * (K + 1) * H * dk);
  if (v_out) memcpy(v_out, v_all, sizeof(double) * NT * (K + 1) * H * dv);

  /* recurrence: one task per (b, h) */
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < B * H; ++bh) {
    const int b = bh / H, h = bh % H;
    double* S = (double*)malloc(sizeof(double) * (M + 1) * ssz);
    double* o = (double*)malloc(sizeof(double) * (K + 1) * dv);
    double* mix = out_mixed ? (double*)malloc(sizeof(double) * ssz) : NULL;
    for (int m = 0; m <= M; ++m) {
      double* Sm = S + m * ssz;
      if (state0) {
        memcpy(Sm, state0 + (((int64_t)b * (M + 1) + m) * H + h) * ssz, sizeof(double) * ssz);
      } else {
        memset(Sm, 0, sizeof(double) * ssz);
      }
    }
    for (int t = 0; t < T; ++t) {
      const int64_t tok = (int64_t)b * T + t;
      const double* qt = q_all + (tok * H + h) * dk;
      for (int j = 0; j <= K; ++j) {
        const int m = (j < K) ? idx_l[tok * K + j] : M;
        const double* kt = k_all + ((tok * (K + 1) + j) * H + h) * dk;
        const double* vt = v_all + ((tok * (K + 1) + j) * H + h) * dv;
        const double a = alpha[(tok * H + h) * (M + 1) + m];
        const double c = beta[(tok * H + h) * (M + 1) + m];
        step(dk, dv, a, c, qt, kt, vt, S + m * ssz, o + j * dv);
      }
      for (int e = 0; e < dv; ++e) {
        double s = o[K * dv + e];
        for (int j = 0; j < K; ++j) s += w_l[tok * K + j] * o[j * dv + e];
        if (out) out[(tok * H + h) * dv + e] = s;
        if (o_shared) o_shared[(tok * H + h) * dv + e] = o[K * dv + e];
        for (int j = 0; j < K; ++j)
          if (o_routed) o_routed[((tok * K + j) * H + h) * dv + e] = o[j * dv + e];
      }
      if (mix) {
        /* read from the weighted mixture of the memories after this token */
        for (int i = 0; i < ssz; ++i) {
          double s = S[M * ssz + i];
          for (int j = 0; j < K; ++j) s += w_l[tok * K + j] * S[idx_l[tok * K + j] * ssz + i];
          mix[i] = s;
        }
        for (int e = 0; e < dv; ++e) {
          double s = 0.0;
          for (int i = 0; i < dk; ++i) s += mix[i * dv + e] * qt[i];
          out_mixed[(tok * H + h) * dv + e] = s;
        }
      }
    }
    if (state) {
      for (int m = 0; m <= M; ++m)
        memcpy(state + (((int64_t)b * (M + 1) + m) * H + h) * ssz, S + m * ssz,
               sizeof(double) * ssz);
    }
    free(S);
    free(o);
    free(mix);
  }
  free(q_all);
  free(k_all);
  free(v_all);
  if (!idx) free(idx_l);
  if (!w) free(w_l);
}

/* The layer with Gated DeltaNet memories. */
void oracle_layer(const int32_t* dims, const double* x, const double* wr, const double* bias,
                  const double* wq, const double* wk, const double* wv, const double* alpha,
                  const double* beta, const double* state0, int32_t* idx, double* w,
                  double* o_routed, double* o_shared, double* out, double* out_mixed,
                  double* state, double* q_out, double* k_out, double* v_out) {
  oracle_layer_rule(0, dims, x, wr, bias, wq, wk, wv, alpha, beta, state0, idx, w, o_routed, o_shared, out,
                    out_mixed, state, q_out, k_out, v_out);
}

/* The sum out[t][h][:] = o_shared[t][h][:] + sum_j w[t][j] * o_routed[row(t,j)][h][:],
 * shared memory first, then j ascending.  o_routed rows are addressed through
 * inv (NULL = row t*K + j).  Used to check the combine step on its own.        */
void oracle_combine(int64_t n_tok, int K, int H, int dv, const int32_t* inv, const double* w,
                    const double* o_routed, const double* o_shared, double* out) {
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int e = 0; e < H * dv; ++e) {
      double s = o_shared[t * H * dv + e];
      for (int j = 0; j < K; ++j) {
        int64_t r = inv ? inv[t * K + j] : t * K + j;
        s += w[t * K + j] * o_routed[r * H * dv + e];
      }
      out[t * H * dv + e] = s;
    }
  }
}

/* Recurrences over many packed segments at once (the per-memory operator alone):
 * segment s covers rows [seg_off[s], seg_off[s+1]) and starts from state slot
 * seg_state[s] of state [n_state][H][dk][dv] (updated in place).  q is read at
 * row_token[row] (q [n_tok][H][dk]); k/v/a/c/o are indexed by row
 * (k [N][H][dk], v/o [N][H][dv], a/c [N][H]).  Only the segments listed in
 * `which` (n_which of them) are run; NULL = all.  Parallel over (segment, head). */
void oracle_segments_rule(int rule, int n_seg, const int32_t* seg_off, const int32_t* seg_state,
                          const int32_t* row_token, int H, int dk, int dv, const double* q,
                          const double* k, const double* v, const double* a, const double* c,
                          double* state, double* o, int n_which, const int32_t* which) {
  const oracle_step_fn step = step_of(rule);
  const int n_jobs = (which ? n_which : n_seg) * H;
  const int64_t ssz = (int64_t)dk * dv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int job = 0; job < n_jobs; ++job) {
    const int s = which ? which[job / H] : job / H;
    const int h = job % H;
    double* S = state + ((int64_t)seg_state[s] * H + h) * ssz;
    for (int64_t r = seg_off[s]; r < seg_off[s + 1]; ++r) {
      const int64_t tk = row_token ? row_token[r] : r;
      step(dk, dv, a[r * H + h], c[r * H + h], q + (tk * H + h) * dk, k + (r * H + h) * dk,
           v + (r * H + h) * dv, S, o + (r * H + h) * dv);
    }
  }
}

void oracle_segments(int n_seg, const int32_t* seg_off, const int32_t* seg_state,
                     const int32_t* row_token, int H, int dk, int dv, const double* q,
                     const double* k, const double* v, const double* a, const double* c,
                     double* state, double* o, int n_which, const int32_t* which) {
  oracle_segments_rule(0, n_seg, seg_off, seg_state, row_token, H, dk, dv, q, k, v, a, c, state, o, n_which,
                       which);
}

/* Projections of one head for a list of tokens: for i < n with token
 * tok = rows_tok[i]:  q[i] = Wq_h x_tok (if wq_h), k[i] = normalise(Wk_h x_tok),
 * v[i] = Wv_h x_tok.  wq_h/wk_h are [dk][D], wv_h is [dv][D].                 */
void oracle_project_head(int64_t n, const int32_t* rows_tok, int D, int dk, int dv,
                         const double* x, const double* wq_h, const double* wk_h,
                         const double* wv_h, double* q, double* k, double* v) {
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < n; ++i) {
    const double* xt = x + (int64_t)rows_tok[i] * D;
    if (wq_h) proj_rows(D, dk, wq_h, xt, q + i * dk);
    if (wk_h) {
      proj_rows(D, dk, wk_h, xt, k + i * dk);
      l2_normalise(dk, k + i * dk);
    }
    if (wv_h) proj_rows(D, dv, wv_h, xt, v + i * dv);
  }
}

/* ------------------------------------------------------------------------- */
/* Gradients of the recurrence: reverse-mode differentiation of the steps
 * above, what training needs ([p1] introduction: linear-complexity training;
 * [p2] "Summary": the layer is trained end to end).  The pages give no
 * backward formulas; these are the chain rule applied to each step as written.
 *
 * Gated DeltaNet step, forward from S_prev:
 *   S~ = a S_prev,  p = S~^T k,  e = c (v - p),  S = S~ + k e^T,  o = S^T q.
 * Reverse, given g = dL/dS (from later steps) and d_o = dL/do:
 *   g   += q d_o^T                  dq  = S d_o
 *   de   = g^T k                    dk  = g e
 *   dc   = de . (v - p)             dv  = c de          dp = -c de
 *   g~   = g + k dp^T               dk += S~ dp
 *   da   = <g~, S_prev>             dL/dS_prev = a g~
 * On entry dS holds g, on exit dL/dS_prev.  S_prev and S are the states
 * before and after the step.  dq, dk, dv are written, not accumulated.      */
void oracle_gdn_step_bwd(int dk, int dv, double a, double c, const double* q, const double* k,
                         const double* v, const double* S_prev, const double* S, const double* d_o,
                         double* dS, double* dq, double* dk_out, double* dv_out, double* da,
                         double* dc) {
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) dS[i * dv + j] += q[i] * d_o[j];
  for (int i = 0; i < dk; ++i) {
    double s = 0.0;
    for (int j = 0; j < dv; ++j) s += S[i * dv + j] * d_o[j];
    dq[i] = s;
  }
  double dcs = 0.0;
  for (int i = 0; i < dk; ++i) dk_out[i] = 0.0;
  for (int j = 0; j < dv; ++j) {
    double p = 0.0, de = 0.0;
    for (int i = 0; i < dk; ++i) {
      p += a * S_prev[i * dv + j] * k[i];
      de += dS[i * dv + j] * k[i];
    }
    const double r = v[j] - p;
    const double e = c * r;
    for (int i = 0; i < dk; ++i) dk_out[i] += dS[i * dv + j] * e;
    dcs += de * r;
    dv_out[j] = c * de;
    const double dp = -c * de;
    for (int i = 0; i < dk; ++i) {
      dk_out[i] += a * S_prev[i * dv + j] * dp;
      dS[i * dv + j] += k[i] * dp;
    }
  }
  double das = 0.0;
  for (int i = 0; i < dk * dv; ++i) {
    das += dS[i] * S_prev[i];
    dS[i] *= a;
  }
  *da = das;
  *dc = dcs;
}

/* Gated linear attention step, forward S = a S_prev + c k v^T, o = S^T q.
 * Reverse: g += q d_o^T; dq = S d_o; dk = c g v; dv = c g^T k;
 * dc = k^T g v; da = <g, S_prev>; dL/dS_prev = a g.                          */
void oracle_gla_step_bwd(int dk, int dv, double a, double c, const double* q, const double* k,
                         const double* v, const double* S_prev, const double* S, const double* d_o,
                         double* dS, double* dq, double* dk_out, double* dv_out, double* da,
                         double* dc) {
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) dS[i * dv + j] += q[i] * d_o[j];
  for (int i = 0; i < dk; ++i) {
    double s = 0.0, t = 0.0;
    for (int j = 0; j < dv; ++j) {
      s += S[i * dv + j] * d_o[j];
      t += dS[i * dv + j] * v[j];
    }
    dq[i] = s;
    dk_out[i] = c * t;
  }
  double dcs = 0.0;
  for (int j = 0; j < dv; ++j) {
    double s = 0.0;
    for (int i = 0; i < dk; ++i) s += dS[i * dv + j] * k[i];
    dv_out[j] = c * s;
    dcs += s * v[j];
  }
  double das = 0.0;
  for (int i = 0; i < dk * dv; ++i) {
    das += dS[i] * S_prev[i];
    dS[i] *= a;
  }
  *da = das;
  *dc = dcs;
}

typedef void (*oracle_step_bwd_fn)(int, int, double, double, const double*, const double*, const double*,
                                   const double*, const double*, const double*, double*, double*, double*,
                                   double*, double*, double*);

/* Steps between stored states in the reverse sweep.  The states inside a span
 * are recomputed from the span's first state by the same forward steps, so
 * they are bit-identical to a sweep that stores every state.                */
#define ORACLE_BWD_SPAN 64

/* Gradients of the recurrences over packed segments (the layout of
 * oracle_segments_rule).  Inputs: the forward's inputs, state0
 * [n_state][H][dk][dv] (the entering states; NULL = zeros), d_o [N][H][dv]
 * (dL/do) and dstate [n_state][H][dk][dv] (dL/d(final state); NULL = zeros).
 * Outputs: dq [N][H][dk] per row (the gradient of the query as used at that
 * row; rows that share a token are not summed), dk [N][H][dk], dv [N][H][dv],
 * da, dc [N][H], dstate0 [n_state][H][dk][dv] = dL/d(entering state).  A state
 * slot may be used by at most one segment; slots that no segment uses pass
 * dstate through.  Parallel over (segment, head).                            */
void oracle_segments_bwd_rule(int rule, int n_seg, const int32_t* seg_off, const int32_t* seg_state,
                              int n_state, const int32_t* row_token, int H, int dk, int dv,
                              const double* q, const double* k, const double* v, const double* a,
                              const double* c, const double* state0, const double* d_o,
                              const double* dstate, double* dq, double* dk_out, double* dv_out,
                              double* da, double* dc, double* dstate0) {
  const oracle_step_fn step = step_of(rule);
  const oracle_step_bwd_fn step_bwd = rule == 1 ? oracle_gla_step_bwd : oracle_gdn_step_bwd;
  const int64_t ssz = (int64_t)dk * dv;
  const int64_t n_all = (int64_t)n_state * H * ssz;
  for (int64_t i = 0; i < n_all; ++i) dstate0[i] = dstate ? dstate[i] : 0.0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int job = 0; job < n_seg * H; ++job) {
    const int s = job / H, h = job % H;
    const int64_t r0 = seg_off[s], L = seg_off[s + 1] - seg_off[s];
    const int64_t slot = ((int64_t)seg_state[s] * H + h) * ssz;
    const int64_t n_span = (L + ORACLE_BWD_SPAN - 1) / ORACLE_BWD_SPAN;
    double* ck = (double*)malloc(sizeof(double) * (size_t)((n_span + 1) * ssz));
    double* st = (double*)malloc(sizeof(double) * (size_t)((ORACLE_BWD_SPAN + 1) * ssz));
    double* o = (double*)malloc(sizeof(double) * (size_t)dv);
    double* g = dstate0 + slot;
    /* forward sweep: the state at the start of every span */
    for (int64_t i = 0; i < ssz; ++i) ck[i] = state0 ? state0[slot + i] : 0.0;
    for (int64_t sp = 0; sp < n_span; ++sp) {
      double* S = ck + (sp + 1) * ssz;
      memcpy(S, ck + sp * ssz, sizeof(double) * (size_t)ssz);
      const int64_t e = (sp + 1) * ORACLE_BWD_SPAN < L ? (sp + 1) * ORACLE_BWD_SPAN : L;
      for (int64_t i = sp * ORACLE_BWD_SPAN; i < e; ++i) {
        const int64_t r = r0 + i, tk = row_token ? row_token[r] : r;
        step(dk, dv, a[r * H + h], c[r * H + h], q + (tk * H + h) * dk, k + (r * H + h) * dk,
             v + (r * H + h) * dv, S, o);
      }
    }
    /* reverse sweep, span by span from the last */
    for (int64_t sp = n_span - 1; sp >= 0; --sp) {
      const int64_t b = sp * ORACLE_BWD_SPAN;
      const int64_t e = b + ORACLE_BWD_SPAN < L ? b + ORACLE_BWD_SPAN : L;
      memcpy(st, ck + sp * ssz, sizeof(double) * (size_t)ssz);
      for (int64_t i = b; i < e; ++i) {
        const int64_t r = r0 + i, tk = row_token ? row_token[r] : r;
        double* S = st + (i - b + 1) * ssz;
        memcpy(S, S - ssz, sizeof(double) * (size_t)ssz);
        step(dk, dv, a[r * H + h], c[r * H + h], q + (tk * H + h) * dk, k + (r * H + h) * dk,
             v + (r * H + h) * dv, S, o);
      }
      for (int64_t i = e - 1; i >= b; --i) {
        const int64_t r = r0 + i, tk = row_token ? row_token[r] : r;
        step_bwd(dk, dv, a[r * H + h], c[r * H + h], q + (tk * H + h) * dk, k + (r * H + h) * dk,
                 v + (r * H + h) * dv, st + (i - b) * ssz, st + (i - b + 1) * ssz, d_o + (r * H + h) * dv, g,
                 dq + (r * H + h) * dk, dk_out + (r * H + h) * dk, dv_out + (r * H + h) * dv, da + r * H + h,
                 dc + r * H + h);
      }
    }
    free(ck);
    free(st);
    free(o);
  }
}

/* ------------------------------------------------------------------------- */
/* Gradients of the combine, the router and the dispatch gathers (the chain
 * rule applied to their definitions above).
 *
 * Combine, out[t] = o_shared[t] + sum_j w[t][j] o_routed[row(t, j)]:
 *   d_routed[row(t, j)] = w[t][j] dout[t],   d_shared[t] = dout[t],
 *   dw[t][j] = <dout[t], o_routed[row(t, j)]>     (sums over H * dv)
 * row(t, j) = inv[t][j] (NULL: t*K + j).  d_routed rows no token reads are not
 * written.                                                                    */
void oracle_combine_bwd(int64_t n_tok, int K, int H, int dv, const int32_t* inv, const double* w,
                        const double* o_routed, const double* dout, double* d_routed, double* d_shared,
                        double* dw) {
  const int64_t E = (int64_t)H * dv;
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int64_t e = 0; e < E; ++e) d_shared[t * E + e] = dout[t * E + e];
    for (int j = 0; j < K; ++j) {
      const int64_t r = inv ? inv[t * K + j] : t * K + j;
      double s = 0.0;
      for (int64_t e = 0; e < E; ++e) {
        d_routed[r * E + e] = w[t * K + j] * dout[t * E + e];
        s += dout[t * E + e] * o_routed[r * E + e];
      }
      dw[t * K + j] = s;
    }
  }
}

/* Router, with the top-k choice held fixed (straight-through: no gradient
 * flows through the selection, only through the weights).  With
 * w_j = exp(l_{idx_j}) / sum_j' exp(l_{idx_j'}) (the renormalised softmax):
 *   dl[idx_j] = w_j (dw_j - sum_j' w_j' dw_j'),   dl[m] = 0 for m not selected
 *   dx[t] = sum_m dl[t][m] wr[m],  dwr[m] = sum_t dl[t][m] x[t],
 *   dbias[m] = sum_t dl[t][m]
 * x [n_tok][D], wr [M][D], idx/w/dw [n_tok][K]; dx [n_tok][D], dwr [M][D],
 * dbias [M] out.                                                              */
void oracle_route_bwd(int64_t n_tok, int D, int M, int K, const double* x, const double* wr,
                      const int32_t* idx, const double* w, const double* dw, double* dx, double* dwr,
                      double* dbias) {
  double* dl = (double*)malloc(sizeof(double) * (size_t)M);
  for (int64_t i = 0; i < (int64_t)M * D; ++i) dwr[i] = 0.0;
  for (int m = 0; m < M; ++m) dbias[m] = 0.0;
  for (int64_t t = 0; t < n_tok; ++t) {
    double sw = 0.0;
    for (int j = 0; j < K; ++j) sw += w[t * K + j] * dw[t * K + j];
    for (int m = 0; m < M; ++m) dl[m] = 0.0;
    for (int j = 0; j < K; ++j) dl[idx[t * K + j]] = w[t * K + j] * (dw[t * K + j] - sw);
    for (int d = 0; d < D; ++d) {
      double s = 0.0;
      for (int m = 0; m < M; ++m) s += dl[m] * wr[(int64_t)m * D + d];
      dx[t * D + d] = s;
    }
    for (int m = 0; m < M; ++m) {
      for (int d = 0; d < D; ++d) dwr[(int64_t)m * D + d] += dl[m] * x[t * D + d];
      dbias[m] += dl[m];
    }
  }
  free(dl);
}

/* The dispatch gathers in reverse.  Forward: packed row inv[t][j] takes the
 * gates alpha/beta[t][h][idx[t][j]] and reads q[t]; shared row NR + t takes
 * alpha/beta[t][h][M] and reads q[t].  Reverse:
 *   d_alpha[t][h][idx_j] = d_alpha_p[inv[t][j]][h], d_alpha[t][h][M] =
 *   d_alpha_p[NR + t][h], other memories 0 (the same for beta);
 *   dq[t] = dq_rows[NR + t] + sum_j dq_rows[inv[t][j]]   (shared first, then j)
 * d_alpha_p/d_beta_p [N][H], dq_rows [N][H][dk]; d_alpha/d_beta [n_tok][H][M+1],
 * dq [n_tok][H][dk] out.                                                      */
void oracle_dispatch_bwd(int64_t n_tok, int H, int dk, int M, int K, const int32_t* idx, const int32_t* inv,
                         const double* d_alpha_p, const double* d_beta_p, const double* dq_rows, double* d_alpha,
                         double* d_beta, double* dq) {
  const int64_t NR = n_tok * K;
  for (int64_t t = 0; t < n_tok; ++t) {
    for (int h = 0; h < H; ++h) {
      double* da = d_alpha + (t * H + h) * (M + 1);
      double* db = d_beta + (t * H + h) * (M + 1);
      for (int m = 0; m <= M; ++m) da[m] = db[m] = 0.0;
      da[M] = d_alpha_p[(NR + t) * H + h];
      db[M] = d_beta_p[(NR + t) * H + h];
      for (int j = 0; j < K; ++j) {
        const int64_t r = inv[t * K + j];
        da[idx[t * K + j]] = d_alpha_p[r * H + h];
        db[idx[t * K + j]] = d_beta_p[r * H + h];
      }
      for (int i = 0; i < dk; ++i) {
        double s = dq_rows[((NR + t) * H + h) * dk + i];
        for (int j = 0; j < K; ++j) s += dq_rows[((int64_t)inv[t * K + j] * H + h) * dk + i];
        dq[(t * H + h) * dk + i] = s;
      }
    }
  }
}
