/*
 * Oracle for the tree-structured gated delta rule. TEST INFRASTRUCTURE ONLY:
 * the tests, the smoke check and the bench's CPU-baseline leg call it; the
 * product path never does. It shares no code, header or table with the HIP
 * library.
 *
 * What it computes (TreeWY, "Speculative Verification for Gated DeltaNet
 * Hybrids", section 1 "Hybrid models and GDN layers", Eq. 1, and section 3
 * "Key rewrite"):
 *
 *   every token t walks to the state of its parent (or the sequence's initial
 *   state when the parent is -1), then
 *     alpha_t = exp(log_gate_t)
 *     u       = P k_t                       (P = parent state, d_v x d_k)
 *     vt_t    = beta_t (v_t - alpha_t u)    (the pseudo-value)
 *     S_t     = alpha_t P + vt_t k_t^T      (= alpha_t P (I - beta_t k_t k_t^T) + beta_t v_t k_t^T)
 *     o_t     = S_t q_t                     (post-update state)
 *
 * Flide ("Accelerating Decision Inference with Exact State Forking", section
 * 3.2.3) states that every branch computes what it would compute alone; in
 * this oracle that holds by construction, because a token only ever reads its
 * parent's state.
 *
 * Commit (TreeWY section 3 "Reconstruct on commit", Eq. 3) is checked here by
 * replay: the accepted path is walked from the initial state with the same
 * per-token update.
 *
 * The scalar type is chosen at compile time: ORACLE_F32 builds the fp32
 * oracle, otherwise fp64. Sums run in ascending index order. Build with
 * -O2 -ffp-contract=off and without fast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef ORACLE_F32
typedef float real;
#define REAL_EXP expf
#else
typedef double real;
#define REAL_EXP exp
#endif

enum {
  ORACLE_OK = 0,
  ORACLE_ERR_ARGS = -1,
  ORACLE_ERR_PARENT = -2,   /* parent >= t, < -1, or outside the token's sequence */
  ORACLE_ERR_SEQ = -3,      /* seq_start not a valid CSR over [0, T] */
  ORACLE_ERR_PATH = -4,     /* a commit path is not a root-to-node parent chain */
  ORACLE_ERR_NOMEM = -5,
};

int oracle_real_size(void) { return (int)sizeof(real); }

/* ------------------------------------------------------------------ helpers */

static int check_structure(int64_t T, int n_seq, const int32_t* seq_start, const int32_t* parent) {
  if (n_seq < 0 || T < 0) return ORACLE_ERR_ARGS;
  if (seq_start[0] != 0 || seq_start[n_seq] != T) return ORACLE_ERR_SEQ;
  for (int s = 0; s < n_seq; ++s) {
    if (seq_start[s + 1] < seq_start[s]) return ORACLE_ERR_SEQ;
    for (int64_t t = seq_start[s]; t < seq_start[s + 1]; ++t) {
      int32_t p = parent[t];
      if (p == -1) continue;
      if (p < seq_start[s] || p >= t) return ORACLE_ERR_PARENT;
    }
  }
  return ORACLE_OK;
}

/* One token of the recurrence. P and S are d_v x d_k row-major; S != P. */
static void step(int Dk, int Dv, const real* P, const real* k, const real* v, real g, real b, real* S,
                 real* vt_out) {
  real alpha = REAL_EXP(g);
  for (int i = 0; i < Dv; ++i) {
    real u = 0;
    for (int j = 0; j < Dk; ++j) u += P[(size_t)i * Dk + j] * k[j];
    real vt = b * (v[i] - alpha * u);
    if (vt_out) vt_out[i] = vt;
    for (int j = 0; j < Dk; ++j) S[(size_t)i * Dk + j] = alpha * P[(size_t)i * Dk + j] + vt * k[j];
  }
}

static void readout(int Dk, int Dv, const real* S, const real* q, real* o) {
  for (int i = 0; i < Dv; ++i) {
    real acc = 0;
    for (int j = 0; j < Dk; ++j) acc += S[(size_t)i * Dk + j] * q[j];
    o[i] = acc;
  }
}

/* ----------------------------------------------------------- thread pool */

typedef struct {
  int n_items;
  int next;
  pthread_mutex_t mu;
  int (*fn)(void* ctx, int item);
  void* ctx;
  int status;
} pool_t;

static void* pool_worker(void* arg) {
  pool_t* pl = (pool_t*)arg;
  for (;;) {
    pthread_mutex_lock(&pl->mu);
    int item = pl->next++;
    pthread_mutex_unlock(&pl->mu);
    if (item >= pl->n_items) break;
    int rc = pl->fn(pl->ctx, item);
    if (rc != ORACLE_OK) {
      pthread_mutex_lock(&pl->mu);
      if (pl->status == ORACLE_OK) pl->status = rc;
      pthread_mutex_unlock(&pl->mu);
    }
  }
  return NULL;
}

static int run_pool(int n_items, int n_threads, int (*fn)(void*, int), void* ctx) {
  pool_t pl;
  pl.n_items = n_items;
  pl.next = 0;
  pl.fn = fn;
  pl.ctx = ctx;
  pl.status = ORACLE_OK;
  pthread_mutex_init(&pl.mu, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > n_items) n_threads = n_items > 0 ? n_items : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)n_threads);
  if (!th) return ORACLE_ERR_NOMEM;
  int started = 0;
  for (int i = 0; i < n_threads; ++i)
    if (pthread_create(&th[i], NULL, pool_worker, &pl) == 0) ++started;
  if (started == 0) pool_worker(&pl);
  for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&pl.mu);
  return pl.status;
}

/* ---------------------------------------------------------------- forward */

typedef struct {
  int64_t T;
  int H, Dk, Dv, n_seq;
  const int32_t* seq_start;
  const int32_t* parent;
  const real *q, *k, *v, *g, *b, *init;
  real *out, *pv, *state_out;
  const int32_t* srow_head; /* [T] first state row for token t, -1 if none */
  const int32_t* srow_next; /* [n_state] next row for the same token, -1 ends */
} fwd_ctx;

static int fwd_item(void* vctx, int item) {
  fwd_ctx* c = (fwd_ctx*)vctx;
  int s = item / c->H, h = item % c->H;
  int64_t beg = c->seq_start[s], end = c->seq_start[s + 1], n = end - beg;
  size_t ssz = (size_t)c->Dv * c->Dk;
  if (n == 0) return ORACLE_OK;
  int32_t* pending = (int32_t*)calloc((size_t)n, sizeof(int32_t)); /* children not yet processed */
  real** live = (real**)calloc((size_t)n, sizeof(real*));
  real* zero = (real*)calloc(ssz, sizeof(real));
  if (!pending || !live || !zero) { free(pending); free(live); free(zero); return ORACLE_ERR_NOMEM; }
  for (int64_t t = beg; t < end; ++t)
    if (c->parent[t] >= 0) pending[c->parent[t] - beg]++;
  const real* init = c->init ? c->init + ((size_t)s * c->H + h) * ssz : zero;
  int rc = ORACLE_OK;
  for (int64_t t = beg; t < end; ++t) {
    int32_t p = c->parent[t];
    const real* P = (p < 0) ? init : live[p - beg];
    real* S = (real*)malloc(ssz * sizeof(real));
    if (!S) { rc = ORACLE_ERR_NOMEM; break; }
    size_t th = (size_t)t * c->H + h;
    step(c->Dk, c->Dv, P, c->k + th * c->Dk, c->v + th * c->Dv, c->g[th], c->b[th], S,
         c->pv ? c->pv + th * c->Dv : NULL);
    readout(c->Dk, c->Dv, S, c->q + th * c->Dk, c->out + th * c->Dv);
    for (int32_t r = c->srow_head[t]; r >= 0; r = c->srow_next[r])
      memcpy(c->state_out + ((size_t)r * c->H + h) * ssz, S, ssz * sizeof(real));
    if (p >= 0 && --pending[p - beg] == 0) { free(live[p - beg]); live[p - beg] = NULL; }
    if (pending[t - beg] > 0) live[t - beg] = S; else free(S);
  }
  for (int64_t i = 0; i < n; ++i) free(live[i]);
  free(pending); free(live); free(zero);
  return rc;
}

/*
 * q, k: [T, H, Dk]; v: [T, H, Dv]; log_gate, beta: [T, H]; init_state:
 * [n_seq, H, Dv, Dk] or NULL (zeros). out: [T, H, Dv]; pseudo_v: [T, H, Dv] or
 * NULL; state_out: [n_state, H, Dv, Dk] filled for the tokens in state_rows.
 */
int oracle_forward(int64_t T, int H, int Dk, int Dv, int n_seq, const int32_t* seq_start,
                   const int32_t* parent, const real* q, const real* k, const real* v,
                   const real* log_gate, const real* beta, const real* init_state, real* out,
                   real* pseudo_v, int32_t n_state, const int32_t* state_rows, real* state_out,
                   int n_threads) {
  if (H < 1 || Dk < 1 || Dv < 1 || !seq_start || !parent || !q || !k || !v || !log_gate || !beta || !out)
    return ORACLE_ERR_ARGS;
  if (n_state > 0 && (!state_rows || !state_out)) return ORACLE_ERR_ARGS;
  int rc = check_structure(T, n_seq, seq_start, parent);
  if (rc != ORACLE_OK) return rc;
  int32_t* head = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
  int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_state > 0 ? n_state : 1));
  if (!head || !next) { free(head); free(next); return ORACLE_ERR_NOMEM; }
  for (int64_t t = 0; t < T; ++t) head[t] = -1;
  for (int32_t r = n_state - 1; r >= 0; --r) {
    if (state_rows[r] < 0 || state_rows[r] >= T) { free(head); free(next); return ORACLE_ERR_ARGS; }
    next[r] = head[state_rows[r]];
    head[state_rows[r]] = r;
  }
  fwd_ctx c = {T, H, Dk, Dv, n_seq, seq_start, parent, q, k, v, log_gate, beta, init_state, out,
               pseudo_v, state_out, head, next};
  rc = run_pool(n_seq * H, n_threads, fwd_item, &c);
  free(head); free(next);
  return rc;
}

/* ----------------------------------------------------------------- commit */

typedef struct {
  int H, Dk, Dv;
  const int32_t *seq_start, *parent, *path_ptr, *path_nodes, *path_seq;
  const real *k, *v, *g, *b, *init;
  real* out_state;
} commit_ctx;

static int commit_item(void* vctx, int item) {
  commit_ctx* c = (commit_ctx*)vctx;
  int pth = item / c->H, h = item % c->H;
  size_t ssz = (size_t)c->Dv * c->Dk;
  int s = c->path_seq[pth];
  real* S = (real*)malloc(ssz * sizeof(real));
  real* N = (real*)malloc(ssz * sizeof(real));
  if (!S || !N) { free(S); free(N); return ORACLE_ERR_NOMEM; }
  if (c->init) memcpy(S, c->init + ((size_t)s * c->H + h) * ssz, ssz * sizeof(real));
  else memset(S, 0, ssz * sizeof(real));
  for (int32_t i = c->path_ptr[pth]; i < c->path_ptr[pth + 1]; ++i) {
    int32_t t = c->path_nodes[i];
    size_t th = (size_t)t * c->H + h;
    step(c->Dk, c->Dv, S, c->k + th * c->Dk, c->v + th * c->Dv, c->g[th], c->b[th], N, NULL);
    real* tmp = S; S = N; N = tmp;
  }
  memcpy(c->out_state + ((size_t)pth * c->H + h) * ssz, S, ssz * sizeof(real));
  free(S); free(N);
  return ORACLE_OK;
}

/*
 * Replays every accepted path from its sequence's initial state. A path lists
 * global token indices root -> accepted node; an empty path yields the initial
 * state. out_state: [n_path, H, Dv, Dk].
 */
int oracle_commit(int64_t T, int H, int Dk, int Dv, int n_seq, const int32_t* seq_start,
                  const int32_t* parent, const real* k, const real* v, const real* log_gate,
                  const real* beta, const real* init_state, int32_t n_path, const int32_t* path_ptr,
                  const int32_t* path_nodes, const int32_t* path_seq, real* out_state, int n_threads) {
  if (H < 1 || Dk < 1 || Dv < 1 || n_path < 0 || !seq_start || !parent || !k || !v || !log_gate || !beta ||
      (n_path > 0 && (!path_ptr || !path_nodes || !path_seq || !out_state)))
    return ORACLE_ERR_ARGS;
  int rc = check_structure(T, n_seq, seq_start, parent);
  if (rc != ORACLE_OK) return rc;
  for (int32_t p = 0; p < n_path; ++p) {
    int s = path_seq[p];
    if (s < 0 || s >= n_seq || path_ptr[p + 1] < path_ptr[p]) return ORACLE_ERR_PATH;
    int32_t prev = -1;
    for (int32_t i = path_ptr[p]; i < path_ptr[p + 1]; ++i) {
      int32_t t = path_nodes[i];
      if (t < seq_start[s] || t >= seq_start[s + 1] || parent[t] != prev) return ORACLE_ERR_PATH;
      prev = t;
    }
  }
  commit_ctx c = {H, Dk, Dv, seq_start, parent, path_ptr, path_nodes, path_seq, k, v, log_gate, beta,
                  init_state, out_state};
  return run_pool(n_path * H, n_threads, commit_item, &c);
}
