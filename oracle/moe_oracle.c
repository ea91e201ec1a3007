/*
 * moe_oracle.c -- TEST INFRASTRUCTURE, not part of the product path.
 *
 * A plain, slow, obviously-correct CPU reference of one mixture-of-experts
 * layer's forward pass, computed in double precision.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header or table with the GPU library.
 *
 * What is computed, and where each step comes from:
 *
 *   route     Hugging Face Transformers docs, "Expert parallelism", section
 *             "Adding an implementation": the expert path receives, per token,
 *             the ids of its selected experts (top_k_index) and their routing
 *             weights (top_k_weights).  The pages do not state the selection
 *             rule; the reading used here is softmax top-k: pick the k largest
 *             logits (equal logits: the lower expert index wins), and weight
 *             each pick by its softmax probability renormalised over the picks.
 *
 *   dispatch  same page, section "Token dispatch": every (token, expert) pair
 *             is sent to the owner of that expert, which runs its experts on
 *             the rows it received.  On one device this is a stable counting
 *             sort of the pairs by expert: expert e owns rows
 *             [offsets[e], offsets[e+1]), in increasing pair order.
 *
 *   experts   "Tensor parallelism for inference", section "Packed strategies":
 *             gate and up projections are packed into one [E, hidden, 2*I]
 *             weight, applied as hidden @ W, and split in two along the last
 *             dimension with the gate half first.  The down projection
 *             (down_proj in the expert plan of "Expert parallelism", section
 *             "Overriding plans") is read with the same orientation,
 *             [E, I, hidden].  Activation: SwiGLU, silu(g) * u, with
 *             silu(z) = z / (1 + exp(-z)).  No biases.
 *
 *   combine   "Expert parallelism", sections "Token dispatch" and "Adding an
 *             implementation": each token's output is the sum of its experts'
 *             outputs scaled by the routing weights.
 *
 * Everything is accumulated in double, in the order the definitions state
 * (inner products in ascending index, the k slots of a token in ascending
 * slot order).  Threads split work by token only, so results do not depend
 * on the thread count.
 *
 * Element types of the x and weight arrays: ORACLE_F32 (IEEE float) or
 * ORACLE_BF16 (bfloat16 bit patterns, the upper 16 bits of a float).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

/* ---- element access ---------------------------------------------------- */

static double elem_to_double(const void* base, int dtype, int64_t i) {
  if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* Copy n consecutive elements starting at index i0 into a double row. */
static void row_to_double(const void* base, int dtype, int64_t i0, int64_t n, double* out) {
  for (int64_t j = 0; j < n; ++j) out[j] = elem_to_double(base, dtype, i0 + j);
}

/* ---- route -------------------------------------------------------------- */

/* Expert a (logit la) is preferred over expert b (logit lb) when its logit is
 * larger, or the logits compare equal and a has the lower index.  IEEE
 * comparison: -0.0 and +0.0 are equal. */
static int preferred(float la, int32_t a, float lb, int32_t b) {
  return la > lb || (la == lb && a < b);
}

/* logits [T, E] float32 -> idx [T, k] (slot 0 = most preferred), w [T, k]. */
int oracle_route(const float* logits, int64_t T, int32_t E, int32_t k, int32_t* idx, double* w) {
  if (T < 0 || E < 1 || k < 1 || k > E) return -1;
  unsigned char* taken = (unsigned char*)malloc((size_t)E);
  double* prob = (double*)malloc(sizeof(double) * (size_t)E);
  if (!taken || !prob) {
    free(taken);
    free(prob);
    return -2;
  }
  for (int64_t t = 0; t < T; ++t) {
    const float* l = logits + t * E;
    memset(taken, 0, (size_t)E);
    /* k rounds, each picking the most preferred expert not yet picked. */
    for (int32_t j = 0; j < k; ++j) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || preferred(l[e], e, l[best], best)) best = e;
      }
      taken[best] = 1;
      idx[t * k + j] = best;
    }
    /* Softmax over all E logits (shifted by the largest for range), then
     * renormalised over the k picks. */
    double m = (double)l[idx[t * k]];
    double z = 0.0;
    for (int32_t e = 0; e < E; ++e) {
      prob[e] = exp((double)l[e] - m);
      z += prob[e];
    }
    for (int32_t e = 0; e < E; ++e) prob[e] /= z;
    double s = 0.0;
    for (int32_t j = 0; j < k; ++j) s += prob[idx[t * k + j]];
    for (int32_t j = 0; j < k; ++j) w[t * k + j] = prob[idx[t * k + j]] / s;
  }
  free(taken);
  free(prob);
  return 0;
}

/* ---- dispatch ------------------------------------------------------------ */

/* pair_expert [P] holds the expert of pair p = t*k + j, or -1 when the pair is
 * not handled here.  Any other value outside [0, E) is an error.
 * Outputs: offsets [E+1], pair_row [P] (-1 for unhandled pairs),
 * row_token [offsets[E]] (token of each expert-ordered row). */
int oracle_dispatch(const int32_t* pair_expert, int64_t P, int32_t k, int32_t E,
                    int32_t* offsets, int32_t* pair_row, int32_t* row_token) {
  if (P < 0 || k < 1 || E < 1) return -1;
  for (int64_t p = 0; p < P; ++p)
    if (pair_expert[p] < -1 || pair_expert[p] >= E) return -3;
  int64_t* count = (int64_t*)calloc((size_t)E, sizeof(int64_t));
  int64_t* cursor = (int64_t*)malloc(sizeof(int64_t) * (size_t)E);
  if (!count || !cursor) {
    free(count);
    free(cursor);
    return -2;
  }
  for (int64_t p = 0; p < P; ++p)
    if (pair_expert[p] >= 0) count[pair_expert[p]] += 1;
  offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) offsets[e + 1] = (int32_t)(offsets[e] + count[e]);
  for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t p = 0; p < P; ++p) {
    int32_t e = pair_expert[p];
    if (e < 0) {
      pair_row[p] = -1;
      continue;
    }
    int64_t r = cursor[e]++;
    pair_row[p] = (int32_t)r;
    row_token[r] = (int32_t)(p / k);
  }
  free(count);
  free(cursor);
  return 0;
}

/* ---- one expert's feed-forward on one row ------------------------------ */

typedef struct {
  double* xrow; /* [d]   */
  double* wrow; /* [2I]  */
  double* g;    /* [I]   */
  double* u;    /* [I]   */
  double* y;    /* [d]   */
} ffn_scratch;

static int scratch_alloc(ffn_scratch* s, int32_t d, int32_t I) {
  int64_t wl = (2 * (int64_t)I > d) ? 2 * (int64_t)I : d;
  s->xrow = (double*)malloc(sizeof(double) * (size_t)d);
  s->wrow = (double*)malloc(sizeof(double) * (size_t)wl);
  s->g = (double*)malloc(sizeof(double) * (size_t)I);
  s->u = (double*)malloc(sizeof(double) * (size_t)I);
  s->y = (double*)malloc(sizeof(double) * (size_t)d);
  return (s->xrow && s->wrow && s->g && s->u && s->y) ? 0 : -2;
}

static void scratch_free(ffn_scratch* s) {
  free(s->xrow);
  free(s->wrow);
  free(s->g);
  free(s->u);
  free(s->y);
}

/* s->y = FFN_e(x[t]), the SwiGLU feed-forward of expert e on token t:
 *   g_i = sum_c x[t,c] * Wgu[e,c,i]        (gate: columns [0, I))
 *   u_i = sum_c x[t,c] * Wgu[e,c,I+i]      (up:   columns [I, 2I))
 *   h_i = silu(g_i) * u_i
 *   y_o = sum_i h_i * Wd[e,i,o]                                           */
static void expert_ffn_row(const void* x, int dtype, int64_t t, int32_t e, int32_t d, int32_t I,
                           const void* w_gate_up, const void* w_down, ffn_scratch* s) {
  const int64_t two_i = 2 * (int64_t)I;
  row_to_double(x, dtype, t * (int64_t)d, d, s->xrow);
  for (int32_t i = 0; i < I; ++i) {
    s->g[i] = 0.0;
    s->u[i] = 0.0;
  }
  for (int32_t c = 0; c < d; ++c) {
    row_to_double(w_gate_up, dtype, ((int64_t)e * d + c) * two_i, two_i, s->wrow);
    const double xc = s->xrow[c];
    for (int32_t i = 0; i < I; ++i) {
      s->g[i] += xc * s->wrow[i];
      s->u[i] += xc * s->wrow[I + i];
    }
  }
  for (int32_t i = 0; i < I; ++i) {
    const double gi = s->g[i];
    s->g[i] = gi / (1.0 + exp(-gi)) * s->u[i]; /* h_i, stored over g */
  }
  for (int32_t o = 0; o < d; ++o) s->y[o] = 0.0;
  for (int32_t i = 0; i < I; ++i) {
    row_to_double(w_down, dtype, ((int64_t)e * I + i) * d, d, s->wrow);
    const double hi = s->g[i];
    for (int32_t o = 0; o < d; ++o) s->y[o] += hi * s->wrow[o];
  }
}

/* ---- tokens: experts + combine ----------------------------------------- */

typedef struct {
  const void* x;
  int dtype;
  int32_t d, I, E, k;
  const int32_t* idx;
  const double* w;
  const void* w_gate_up;
  const void* w_down;
  const int64_t* tokens;
  int64_t n_tok;
  double* out;    /* [n_tok, d]            */
  double* y_pair; /* [n_tok, k, d] or NULL */
  int64_t lo, hi; /* this worker's slice of the token list */
  int status;
} tokens_job;

static void* tokens_worker(void* arg) {
  tokens_job* jb = (tokens_job*)arg;
  ffn_scratch s;
  if (scratch_alloc(&s, jb->d, jb->I) != 0) {
    scratch_free(&s);
    jb->status = -2;
    return NULL;
  }
  const int32_t d = jb->d, k = jb->k;
  for (int64_t n = jb->lo; n < jb->hi; ++n) {
    const int64_t t = jb->tokens[n];
    double* acc = jb->out + n * d;
    for (int32_t o = 0; o < d; ++o) acc[o] = 0.0;
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = jb->idx[t * k + j];
      double* yp = jb->y_pair ? jb->y_pair + (n * k + j) * d : NULL;
      if (e < 0) { /* pair not handled here: contributes nothing */
        if (yp)
          for (int32_t o = 0; o < d; ++o) yp[o] = 0.0;
        continue;
      }
      expert_ffn_row(jb->x, jb->dtype, t, e, d, jb->I, jb->w_gate_up, jb->w_down, &s);
      const double wj = jb->w[t * k + j];
      for (int32_t o = 0; o < d; ++o) acc[o] += wj * s.y[o];
      if (yp)
        for (int32_t o = 0; o < d; ++o) yp[o] = s.y[o];
    }
  }
  scratch_free(&s);
  jb->status = 0;
  return NULL;
}

/* For each listed token t = tokens[n]:
 *   out[n]          = sum_{j<k, idx[t,j] >= 0} w[t,j] * FFN_{idx[t,j]}(x[t])
 *   y_pair[n, j]    = FFN_{idx[t,j]}(x[t])   (zero row when idx[t,j] = -1)
 * x [T, d]; idx, w [T, k]; w_gate_up [E, d, 2I]; w_down [E, I, d]. */
int oracle_moe_tokens(const void* x, int dtype, int64_t T, int32_t d, int32_t E, int32_t k, int32_t I,
                      const int32_t* idx, const double* w, const void* w_gate_up, const void* w_down,
                      const int64_t* tokens, int64_t n_tok, int nthreads, double* out, double* y_pair) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || I < 1 || n_tok < 0) return -1;
  if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
  for (int64_t n = 0; n < n_tok; ++n) {
    if (tokens[n] < 0 || tokens[n] >= T) return -1;
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = idx[tokens[n] * k + j];
      if (e < -1 || e >= E) return -3;
    }
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (n_tok < nthreads) nthreads = n_tok > 0 ? (int)n_tok : 1;
  tokens_job* jobs = (tokens_job*)calloc((size_t)nthreads, sizeof(tokens_job));
  pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !th) {
    free(jobs);
    free(th);
    return -2;
  }
  for (int i = 0; i < nthreads; ++i) {
    tokens_job* jb = &jobs[i];
    jb->x = x;
    jb->dtype = dtype;
    jb->d = d;
    jb->I = I;
    jb->E = E;
    jb->k = k;
    jb->idx = idx;
    jb->w = w;
    jb->w_gate_up = w_gate_up;
    jb->w_down = w_down;
    jb->tokens = tokens;
    jb->n_tok = n_tok;
    jb->out = out;
    jb->y_pair = y_pair;
    jb->lo = n_tok * i / nthreads;
    jb->hi = n_tok * (i + 1) / nthreads;
    jb->status = -4;
  }
  int started = 0;
  for (int i = 1; i < nthreads; ++i) {
    if (pthread_create(&th[i], NULL, tokens_worker, &jobs[i]) != 0) break;
    started = i;
  }
  tokens_worker(&jobs[0]);
  for (int i = 1; i <= started; ++i) pthread_join(th[i], NULL);
  /* Slices whose thread could not be started run here, in order. */
  for (int i = started + 1; i < nthreads; ++i) tokens_worker(&jobs[i]);
  int status = 0;
  for (int i = 0; i < nthreads; ++i)
    if (jobs[i].status != 0) status = jobs[i].status;
  free(jobs);
  free(th);
  return status;
}
