/*
 * rlk_oracle.c -- plain, slow, obviously-correct CPU oracle for selected-token
 * log-probability over a tile-decomposed vocabulary.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or constant with the GPU
 * library; the two agree only because both follow the same pages.
 *
 * Sources (web pages; cited by title and section):
 *   [PR289]  PR #289 "[WS2][PR4][Logp] feat: add distributed TP/CP logprob drift
 *            report" -- the stacked PR1 commit messages (contract: ShardingSpec,
 *            MaskSpec, ReductionSpec, (-inf, 0) as the identity partial, padded
 *            columns masked to -inf), the review excerpt of the op's apply()
 *            (target-range and non-finite-LSE checks), and the description's
 *            "Independent FP32 oracle" and "Comparison contract" sections.
 *   [I323]   Issue #323 "[WS2][Logprob] H100 validation and reproduction guide
 *            for Issue #241 PR1-PR5" -- "Test Order / 2. Six-Case TP/CP Matrix"
 *            (64 vocabulary tiles, real = padded vocabulary 151936).
 *
 * What is computed (the plain definitions; no tiles anywhere except in the
 * partials function, which exists only to pin the per-tile statistic):
 *
 *   LSE_r  = m + log( sum_{j < V_real} exp(x_rj - m) ),  m = max_{j < V_real} x_rj
 *   a_r    = mask_r != 0  and  tgt_r != ignore_index        (effective-active)
 *   logp_r = a_r ? x_r,tgt_r - LSE_r : +0.0
 *   d_rj   = a_r ? g_r * ([j == tgt_r] - exp(x_rj - LSE_r)) : 0   (j < V_real)
 *   d_rj   = 0                                                    (V_real <= j < V_pad)
 *
 * The tile decomposition of the pages is an exact regrouping of the LSE sum, so
 * the oracle takes the whole real vocabulary at once, as the pages' own oracle
 * does ([PR289] "Independent FP32 oracle": it works from the whole real
 * vocabulary in one pass and never goes through the sharded merge).  Arithmetic is
 * fp64; the sum runs sequentially in ascending column order.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - Non-finite inputs.  m is a NaN-propagating maximum.  m = -inf gives
 *     LSE = -inf without evaluating exp(-inf - -inf).  A NaN or +inf among the
 *     real columns makes the max-shifted sum NaN, so LSE = NaN.
 *   - Inactive rows (a_r false) still get an LSE; logp is +0.0 and the gradient
 *     row is all zeros ([PR289] "Comparison contract": LSE drift covers every
 *     logical row, logp drift only active rows).
 *   - An effective-active target outside [0, V_real) is an error ([PR289]
 *     apply(): active targets are validated against the real vocabulary size);
 *     the oracle writes NaN for that row's logp and reports the first such row.
 *   - A non-finite LSE on an effective-active row is an error ([PR289] apply():
 *     such a row is refused).
 *
 * Side outputs and extra gradients (entropy_row, bwd_ex_row below):
 *
 *   H_r    = -sum_{j < V_real} p_rj log p_rj,   p_rj = exp(x_rj - LSE_r),
 *            with 0 log 0 = 0 (a column at -inf contributes nothing)
 *   d_rj   = a_r g_r ([j == tgt_r] - p_rj) + gl_r p_rj - gh_r p_rj (log p_rj + H_r)
 *
 * The pages return the LSE as a direct diagnostic next to the selected logp
 * ([PR289] walkthrough: forward_with_lse), and the RL runs log the mean
 * entropy ([H100V] "H100 canonical TP/CP validation": log metrics such as mean
 * loss/entropy).  Readings: the LSE and entropy terms apply to every row (both
 * are defined on every row, as the LSE output is); the logp term only to
 * effective-active rows; a row whose real logits are all -inf has no
 * distribution, so its H is NaN, and so is any LSE or entropy gradient that
 * reaches it.  The entropy gradient is the derivative of the definition:
 * dH/dx_j = -p_j (log p_j + H).
 *
 * Parity pins: every function below is pinned by tests that do not use this
 * file's arithmetic (pure-Python brute force, closed forms, finite differences,
 * float64 library routines); see tests/test_oracle_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define ORC_OK 0
#define ORC_ERR_ARG 1
#define ORC_ERR_TARGET_RANGE 2
#define ORC_ERR_NONFINITE_LSE 3
#define ORC_ERR_NOMEM 4

/* ------------------------------------------------------------------------ */
/* bf16 decode: a bf16 value is the top 16 bits of an IEEE binary32, so the  */
/* decode is exact.                                                          */
/* ------------------------------------------------------------------------ */
double rlk_oracle_bf16_to_f64(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

static void decode_row(const uint16_t* src, int64_t n, double* dst) {
  for (int64_t j = 0; j < n; ++j) dst[j] = rlk_oracle_bf16_to_f64(src[j]);
}

/* ------------------------------------------------------------------------ */
/* Geometry.  [PR289] PR1 commit messages: the vocabulary is cut evenly, with */
/* the last bound pinned to the end for non-divisible sizes, and shards must */
/* be tile-aligned for cross-degree bitwise identity.  Reading: tile t spans */
/* [floor(t*V_pad/T), floor((t+1)*V_pad/T)); shard s holds tiles             */
/* [floor(s*T/S), floor((s+1)*T/S)).                                          */
/* ------------------------------------------------------------------------ */
int rlk_oracle_tile_bounds(int64_t padded_vocab, int32_t num_tiles, int64_t* bounds) {
  if (padded_vocab < 1 || num_tiles < 1 || (int64_t)num_tiles > padded_vocab || !bounds)
    return ORC_ERR_ARG;
  for (int32_t t = 0; t <= num_tiles; ++t) {
    /* exact integer floor; padded_vocab * t fits in int64 for any sane size */
    bounds[t] = (padded_vocab * (int64_t)t) / (int64_t)num_tiles;
  }
  return ORC_OK;
}

int rlk_oracle_shard_tiles(int32_t num_tiles, int32_t num_shards, int32_t* first_tile) {
  if (num_tiles < 1 || num_shards < 1 || num_shards > num_tiles || !first_tile)
    return ORC_ERR_ARG;
  for (int32_t s = 0; s <= num_shards; ++s)
    first_tile[s] = (int32_t)(((int64_t)s * num_tiles) / num_shards);
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Core row functions (fp64).                                                */
/* ------------------------------------------------------------------------ */

/* NaN-propagating maximum of a span; -inf for an empty span. */
static double span_max(const double* x, int64_t n) {
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    if (isnan(x[j])) return NAN;
    if (x[j] > m) m = x[j];
  }
  return m;
}

/* log of the sum of exp over a span, by the max-shifted definition. */
static double row_lse(const double* x, int64_t n) {
  double m = span_max(x, n);
  if (isnan(m)) return NAN;
  if (m == -INFINITY) return -INFINITY; /* empty or all -inf: no exp(-inf - -inf) */
  double sum = 0.0;
  for (int64_t j = 0; j < n; ++j) sum += exp(x[j] - m); /* ascending j */
  return m + log(sum);
}

static int row_active(const uint8_t* mask, const int32_t* tgt, int64_t r, int32_t ignore_index) {
  int m = mask ? (mask[r] != 0) : 1;
  return m && tgt[r] != ignore_index;
}

/* ------------------------------------------------------------------------ */
/* Threading: rows are split into contiguous blocks, one per thread.  The    */
/* per-row arithmetic does not depend on the split.                          */
/* ------------------------------------------------------------------------ */
typedef struct job job;
typedef void (*row_fn)(const job*, int64_t r, double* scratch);

struct job {
  /* inputs: exactly one of xd / xb is set */
  const double* xd;
  const uint16_t* xb;
  int64_t n_rows, real_vocab, padded_vocab, ld, ldd;
  const int32_t* tgt;
  const uint8_t* mask;
  int32_t ignore_index;
  const double* lse_in;
  const double* g;
  const double* ent_in; /* H per row (extended backward) */
  const double* gl;     /* d loss / d LSE per row, or NULL */
  const double* gh;     /* d loss / d H per row, or NULL */
  int32_t num_tiles;
  const int64_t* bounds;
  /* outputs */
  double* logp;
  double* lse;
  double* d;
  double* pmax;
  double* psum;
  double* pent; /* per-tile sum of exp(x - m) (x - m), or NULL */
  double* ent;  /* H per row out */
  row_fn fn;
  /* per-thread */
  int64_t r0, r1;
  int status;       /* worst error code seen by this thread */
  int64_t bad_row;  /* first row with that error */
};

/* Fetch row r as doubles (decoding bf16 into scratch when needed). */
static const double* get_row(const job* jb, int64_t r, double* scratch, int64_t n) {
  if (jb->xd) return jb->xd + r * jb->ld;
  decode_row(jb->xb + r * jb->ld, n, scratch);
  return scratch;
}

static void note_error(job* jb, int code, int64_t r) {
  /* target-range errors take precedence over non-finite LSE */
  if (jb->status == ORC_OK || (code == ORC_ERR_TARGET_RANGE && jb->status != code)) {
    jb->status = code;
    jb->bad_row = r;
  }
}

static void fwd_row(const job* cjb, int64_t r, double* scratch) {
  job* jb = (job*)cjb;
  const double* x = get_row(jb, r, scratch, jb->real_vocab);
  double lse = row_lse(x, jb->real_vocab);
  jb->lse[r] = lse;
  if (!row_active(jb->mask, jb->tgt, r, jb->ignore_index)) {
    jb->logp[r] = 0.0;
    return;
  }
  int32_t t = jb->tgt[r];
  if (t < 0 || (int64_t)t >= jb->real_vocab) {
    jb->logp[r] = NAN;
    note_error(jb, ORC_ERR_TARGET_RANGE, r);
    return;
  }
  jb->logp[r] = x[t] - lse;
  if (!isfinite(lse)) note_error(jb, ORC_ERR_NONFINITE_LSE, r);
}

static void bwd_row(const job* cjb, int64_t r, double* scratch) {
  job* jb = (job*)cjb;
  double* d = jb->d + r * jb->ldd;
  for (int64_t j = 0; j < jb->padded_vocab; ++j) d[j] = 0.0;
  if (!row_active(jb->mask, jb->tgt, r, jb->ignore_index)) return;
  int32_t t = jb->tgt[r];
  if (t < 0 || (int64_t)t >= jb->real_vocab) {
    for (int64_t j = 0; j < jb->real_vocab; ++j) d[j] = NAN;
    note_error(jb, ORC_ERR_TARGET_RANGE, r);
    return;
  }
  const double* x = get_row(jb, r, scratch, jb->real_vocab);
  double lse = jb->lse_in[r], g = jb->g[r];
  for (int64_t j = 0; j < jb->real_vocab; ++j) {
    double onehot = (j == (int64_t)t) ? 1.0 : 0.0;
    d[j] = g * (onehot - exp(x[j] - lse));
  }
}

/* Entropy of row r by the definition: LSE first (row_lse), then
 * -sum p_j log p_j over the real columns in ascending order, skipping p_j = 0
 * terms whose x_j is -inf (0 log 0 = 0). */
static void entropy_row(const job* cjb, int64_t r, double* scratch) {
  const job* jb = cjb;
  const double* x = get_row(jb, r, scratch, jb->real_vocab);
  double lse = row_lse(x, jb->real_vocab);
  if (!isfinite(lse)) {
    jb->ent[r] = NAN; /* no distribution (all -inf), or NaN / +inf inputs */
    return;
  }
  double h = 0.0;
  for (int64_t j = 0; j < jb->real_vocab; ++j) {
    if (x[j] == -INFINITY) continue;
    double lp = x[j] - lse;
    h -= exp(lp) * lp;
  }
  jb->ent[r] = h;
}

/* The extended backward of row r: the logp term on effective-active rows,
 * the LSE and entropy terms on every row where their upstream gradient is
 * given and nonzero. */
static void bwd_ex_row(const job* cjb, int64_t r, double* scratch) {
  job* jb = (job*)cjb;
  double* d = jb->d + r * jb->ldd;
  for (int64_t j = 0; j < jb->padded_vocab; ++j) d[j] = 0.0;
  const int act = row_active(jb->mask, jb->tgt, r, jb->ignore_index);
  const double g = (act && jb->g) ? jb->g[r] : 0.0;
  const double gl = jb->gl ? jb->gl[r] : 0.0;
  const double gh = jb->gh ? jb->gh[r] : 0.0;
  int32_t t = act ? jb->tgt[r] : -1;
  if (act && (t < 0 || (int64_t)t >= jb->real_vocab)) {
    for (int64_t j = 0; j < jb->real_vocab; ++j) d[j] = NAN;
    note_error(jb, ORC_ERR_TARGET_RANGE, r);
    return;
  }
  if (!act && gl == 0.0 && gh == 0.0) return;
  const double* x = get_row(jb, r, scratch, jb->real_vocab);
  const double lse = jb->lse_in[r];
  const double h = gh != 0.0 ? jb->ent_in[r] : 0.0;
  for (int64_t j = 0; j < jb->real_vocab; ++j) {
    const double oh = (j == (int64_t)t) ? 1.0 : 0.0;
    const double p = exp(x[j] - lse);
    double v = g * (oh - p) + gl * p;
    if (gh != 0.0 && !(x[j] == -INFINITY && isfinite(lse))) v -= gh * p * ((x[j] - lse) + h);
    d[j] = v;
  }
}

static void partials_row(const job* cjb, int64_t r, double* scratch) {
  const job* jb = cjb;
  const double* x = get_row(jb, r, scratch, jb->real_vocab);
  for (int32_t t = 0; t < jb->num_tiles; ++t) {
    int64_t lo = jb->bounds[t], hi = jb->bounds[t + 1];
    if (hi > jb->real_vocab) hi = jb->real_vocab; /* padded columns never count */
    double m = -INFINITY, s = 0.0, a = 0.0;
    if (hi > lo) {
      m = span_max(x + lo, hi - lo);
      if (isnan(m)) {
        s = NAN;
        a = NAN;
      } else if (m != -INFINITY) {
        for (int64_t j = lo; j < hi; ++j) {
          if (x[j] == -INFINITY) continue; /* exp(-inf) = 0 and 0 (-inf) counts as 0 */
          s += exp(x[j] - m);
          a += exp(x[j] - m) * (x[j] - m);
        }
      }
      /* m == -inf: no finite real logit, so (m, s, a) = (-inf, 0, 0) */
    }
    jb->pmax[r * jb->num_tiles + t] = m;
    jb->psum[r * jb->num_tiles + t] = s;
    if (jb->pent) jb->pent[r * jb->num_tiles + t] = a;
  }
}

static void* run_block(void* arg) {
  job* jb = (job*)arg;
  double* scratch = NULL;
  if (jb->xb) {
    /* one decoded row; only [0, V_real) is ever decoded, the tail stays NaN */
    int64_t len = jb->ld > 0 ? jb->ld : 1;
    scratch = (double*)malloc(sizeof(double) * (size_t)len);
    if (!scratch) {
      jb->status = ORC_ERR_NOMEM;
      return NULL;
    }
    for (int64_t j = 0; j < len; ++j) scratch[j] = NAN;
  }
  for (int64_t r = jb->r0; r < jb->r1; ++r) jb->fn(jb, r, scratch);
  free(scratch);
  return NULL;
}

static int run_rows(job* proto, int nthreads, int64_t* bad_row) {
  if (nthreads <= 0) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = n > 0 ? (int)n : 1;
  }
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > proto->n_rows) nthreads = proto->n_rows > 0 ? (int)proto->n_rows : 1;
  job jobs[256];
  pthread_t th[256];
  int started[256];
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = *proto;
    jobs[i].r0 = proto->n_rows * i / nthreads;
    jobs[i].r1 = proto->n_rows * (i + 1) / nthreads;
    jobs[i].status = ORC_OK;
    jobs[i].bad_row = -1;
    started[i] = (nthreads > 1) && pthread_create(&th[i], NULL, run_block, &jobs[i]) == 0;
    if (!started[i]) run_block(&jobs[i]);
  }
  int status = ORC_OK;
  int64_t first_bad = -1;
  for (int i = 0; i < nthreads; ++i) {
    if (started[i]) pthread_join(th[i], NULL);
  }
  /* report the lowest-index row carrying the highest-precedence error */
  for (int pass = 0; pass < 3 && status == ORC_OK; ++pass) {
    int want = pass == 0 ? ORC_ERR_NOMEM : pass == 1 ? ORC_ERR_TARGET_RANGE : ORC_ERR_NONFINITE_LSE;
    for (int i = 0; i < nthreads; ++i) {
      if (jobs[i].status == want) {
        status = want;
        first_bad = jobs[i].bad_row;
        break;
      }
    }
  }
  if (bad_row) *bad_row = first_bad;
  return status;
}

/* ------------------------------------------------------------------------ */
/* Public entry points.  Logits are either fp64 ([N, ld] doubles) or bf16    */
/* bit patterns ([N, ld] uint16).  Only columns [0, V_real) are ever read.   */
/* `mask` may be NULL (every row active).  nthreads <= 0 uses every online   */
/* core.  Return value: 0, or the error code; *bad_row gets the first row    */
/* with that error (or -1).                                                  */
/* ------------------------------------------------------------------------ */
static int check_common(int64_t n_rows, int64_t real_vocab, int64_t ld, const void* x,
                        const int32_t* tgt) {
  if (n_rows < 0 || real_vocab < 1 || ld < real_vocab) return ORC_ERR_ARG;
  if (n_rows > 0 && (!x || !tgt)) return ORC_ERR_ARG;
  return ORC_OK;
}

static int fwd_impl(const double* xd, const uint16_t* xb, int64_t n_rows, int64_t real_vocab,
                    int64_t ld, const int32_t* tgt, const uint8_t* mask, int32_t ignore_index,
                    double* logp, double* lse, int64_t* bad_row, int nthreads) {
  if (bad_row) *bad_row = -1;
  int rc = check_common(n_rows, real_vocab, ld, xd ? (const void*)xd : (const void*)xb, tgt);
  if (rc) return rc;
  if (n_rows == 0) return ORC_OK;
  if (!logp || !lse) return ORC_ERR_ARG;
  job jb;
  memset(&jb, 0, sizeof jb);
  jb.xd = xd;
  jb.xb = xb;
  jb.n_rows = n_rows;
  jb.real_vocab = real_vocab;
  jb.ld = ld;
  jb.tgt = tgt;
  jb.mask = mask;
  jb.ignore_index = ignore_index;
  jb.logp = logp;
  jb.lse = lse;
  jb.fn = fwd_row;
  return run_rows(&jb, nthreads, bad_row);
}

int rlk_oracle_fwd_f64(const double* x, int64_t n_rows, int64_t real_vocab, int64_t ld,
                       const int32_t* tgt, const uint8_t* mask, int32_t ignore_index,
                       double* logp, double* lse, int64_t* bad_row, int nthreads) {
  return fwd_impl(x, NULL, n_rows, real_vocab, ld, tgt, mask, ignore_index, logp, lse, bad_row,
                  nthreads);
}

int rlk_oracle_fwd_bf16(const uint16_t* x, int64_t n_rows, int64_t real_vocab, int64_t ld,
                        const int32_t* tgt, const uint8_t* mask, int32_t ignore_index,
                        double* logp, double* lse, int64_t* bad_row, int nthreads) {
  return fwd_impl(NULL, x, n_rows, real_vocab, ld, tgt, mask, ignore_index, logp, lse, bad_row,
                  nthreads);
}

static int bwd_impl(const double* xd, const uint16_t* xb, int64_t n_rows, int64_t real_vocab,
                    int64_t padded_vocab, int64_t ld, const int32_t* tgt, const uint8_t* mask,
                    int32_t ignore_index, const double* lse, const double* g, double* d,
                    int64_t ldd, int64_t* bad_row, int nthreads) {
  if (bad_row) *bad_row = -1;
  int rc = check_common(n_rows, real_vocab, ld, xd ? (const void*)xd : (const void*)xb, tgt);
  if (rc) return rc;
  if (padded_vocab < real_vocab || ldd < padded_vocab) return ORC_ERR_ARG;
  if (n_rows == 0) return ORC_OK;
  if (!lse || !g || !d) return ORC_ERR_ARG;
  job jb;
  memset(&jb, 0, sizeof jb);
  jb.xd = xd;
  jb.xb = xb;
  jb.n_rows = n_rows;
  jb.real_vocab = real_vocab;
  jb.padded_vocab = padded_vocab;
  jb.ld = ld;
  jb.ldd = ldd;
  jb.tgt = tgt;
  jb.mask = mask;
  jb.ignore_index = ignore_index;
  jb.lse_in = lse;
  jb.g = g;
  jb.d = d;
  jb.fn = bwd_row;
  return run_rows(&jb, nthreads, bad_row);
}

int rlk_oracle_bwd_f64(const double* x, int64_t n_rows, int64_t real_vocab, int64_t padded_vocab,
                       int64_t ld, const int32_t* tgt, const uint8_t* mask, int32_t ignore_index,
                       const double* lse, const double* g, double* d, int64_t ldd,
                       int64_t* bad_row, int nthreads) {
  return bwd_impl(x, NULL, n_rows, real_vocab, padded_vocab, ld, tgt, mask, ignore_index, lse, g,
                  d, ldd, bad_row, nthreads);
}

int rlk_oracle_bwd_bf16(const uint16_t* x, int64_t n_rows, int64_t real_vocab,
                        int64_t padded_vocab, int64_t ld, const int32_t* tgt,
                        const uint8_t* mask, int32_t ignore_index, const double* lse,
                        const double* g, double* d, int64_t ldd, int64_t* bad_row,
                        int nthreads) {
  return bwd_impl(NULL, x, n_rows, real_vocab, padded_vocab, ld, tgt, mask, ignore_index, lse, g,
                  d, ldd, bad_row, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Fused LM-head variant: the logits are z = h . W^T over the real vocabulary */
/* rows of W, computed in fp64 from the bf16 inputs; the selected-token logp  */
/* then follows from z exactly as for materialised logits (rlk_oracle_fwd_f64 */
/* on z).  The pages name an optional fused kernel without describing it      */
/* ([I323] "Validation Boundary": the optional PR6 fused kernel); the reading */
/* here is the plain one: the same log-softmax, over logits that are a GEMM.  */
/*   h  bf16 [n_rows, ld_h], K = hidden_dim <= ld_h                           */
/*   W  bf16 [>= real_vocab rows, ld_w], K <= ld_w; rows >= real_vocab unread */
/*   z  fp64 [n_rows, real_vocab] out                                         */
/* ------------------------------------------------------------------------ */
typedef struct {
  const double* hd;  /* decoded hidden rows, [n_rows][k] */
  const uint16_t* w;
  int64_t n_rows, k, ld_w, real_vocab;
  double* z;
  int64_t j0, j1; /* this thread's vocabulary rows */
  int status;
} mm_job;

/* Threads split the vocabulary rows; each W row is decoded once and dotted
 * with every hidden row, summing over k in ascending order. */
static void* mm_block(void* arg) {
  mm_job* jb = (mm_job*)arg;
  double* wr = (double*)malloc(sizeof(double) * (size_t)(jb->k > 0 ? jb->k : 1));
  if (!wr) {
    jb->status = ORC_ERR_NOMEM;
    return NULL;
  }
  for (int64_t j = jb->j0; j < jb->j1; ++j) {
    decode_row(jb->w + j * jb->ld_w, jb->k, wr);
    for (int64_t r = 0; r < jb->n_rows; ++r) {
      const double* hr = jb->hd + r * jb->k;
      double acc = 0.0;
      for (int64_t q = 0; q < jb->k; ++q) acc += hr[q] * wr[q]; /* ascending k */
      jb->z[r * jb->real_vocab + j] = acc;
    }
  }
  free(wr);
  return NULL;
}

int rlk_oracle_lmhead_logits(const uint16_t* h, const uint16_t* w, int64_t n_rows,
                             int64_t hidden_dim, int64_t real_vocab, int64_t ld_h, int64_t ld_w,
                             double* z, int nthreads) {
  if (n_rows < 0 || hidden_dim < 1 || real_vocab < 1 || ld_h < hidden_dim || ld_w < hidden_dim)
    return ORC_ERR_ARG;
  if (n_rows == 0) return ORC_OK;
  if (!h || !w || !z) return ORC_ERR_ARG;
  double* hd = (double*)malloc(sizeof(double) * (size_t)n_rows * (size_t)hidden_dim);
  if (!hd) return ORC_ERR_NOMEM;
  for (int64_t r = 0; r < n_rows; ++r) decode_row(h + r * ld_h, hidden_dim, hd + r * hidden_dim);
  if (nthreads <= 0) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = n > 0 ? (int)n : 1;
  }
  if (nthreads > 256) nthreads = 256;
  if ((int64_t)nthreads > real_vocab) nthreads = (int)real_vocab;
  mm_job jobs[256];
  pthread_t th[256];
  int started[256];
  for (int i = 0; i < nthreads; ++i) {
    jobs[i].hd = hd;
    jobs[i].w = w;
    jobs[i].n_rows = n_rows;
    jobs[i].k = hidden_dim;
    jobs[i].ld_w = ld_w;
    jobs[i].real_vocab = real_vocab;
    jobs[i].z = z;
    jobs[i].j0 = real_vocab * i / nthreads;
    jobs[i].j1 = real_vocab * (i + 1) / nthreads;
    jobs[i].status = ORC_OK;
    started[i] = (nthreads > 1) && pthread_create(&th[i], NULL, mm_block, &jobs[i]) == 0;
    if (!started[i]) mm_block(&jobs[i]);
  }
  int status = ORC_OK;
  for (int i = 0; i < nthreads; ++i) {
    if (started[i]) pthread_join(th[i], NULL);
    if (jobs[i].status != ORC_OK) status = jobs[i].status;
  }
  free(hd);
  return status;
}

/* Per-tile (max, sumexp) partials, [N][T] row-major, by the plain definition
 * over each tile's real columns ([PR289] PR1 commit messages: padded columns
 * are masked before the local partials; a padding-only or all -inf tile gives
 * the (-inf, 0) identity).  Used only to pin the GPU's stage-1 statistic. */
static int partials_impl(const double* xd, const uint16_t* xb, int64_t n_rows,
                         int64_t real_vocab, int64_t padded_vocab, int64_t ld, int32_t num_tiles,
                         double* pmax, double* psum, double* pent, int nthreads) {
  if (n_rows < 0 || real_vocab < 1 || padded_vocab < real_vocab || ld < padded_vocab)
    return ORC_ERR_ARG;
  if (num_tiles < 1 || (int64_t)num_tiles > padded_vocab) return ORC_ERR_ARG;
  if (n_rows == 0) return ORC_OK;
  if ((!xd && !xb) || !pmax || !psum) return ORC_ERR_ARG;
  int64_t* bounds = (int64_t*)malloc(sizeof(int64_t) * (size_t)(num_tiles + 1));
  if (!bounds) return ORC_ERR_NOMEM;
  rlk_oracle_tile_bounds(padded_vocab, num_tiles, bounds);
  job jb;
  memset(&jb, 0, sizeof jb);
  jb.xd = xd;
  jb.xb = xb;
  jb.n_rows = n_rows;
  jb.real_vocab = real_vocab;
  jb.padded_vocab = padded_vocab;
  jb.ld = ld;
  jb.num_tiles = num_tiles;
  jb.bounds = bounds;
  jb.pmax = pmax;
  jb.psum = psum;
  jb.pent = pent;
  jb.fn = partials_row;
  int rc = run_rows(&jb, nthreads, NULL);
  free(bounds);
  return rc;
}

/* pent (may be NULL): per tile, sum of exp(x - m) (x - m) over the tile's
 * real finite columns -- the entropy's per-tile statistic. */
int rlk_oracle_tile_partials_f64(const double* x, int64_t n_rows, int64_t real_vocab,
                                 int64_t padded_vocab, int64_t ld, int32_t num_tiles,
                                 double* pmax, double* psum, double* pent, int nthreads) {
  return partials_impl(x, NULL, n_rows, real_vocab, padded_vocab, ld, num_tiles, pmax, psum,
                       pent, nthreads);
}

int rlk_oracle_tile_partials_bf16(const uint16_t* x, int64_t n_rows, int64_t real_vocab,
                                  int64_t padded_vocab, int64_t ld, int32_t num_tiles,
                                  double* pmax, double* psum, double* pent, int nthreads) {
  return partials_impl(NULL, x, n_rows, real_vocab, padded_vocab, ld, num_tiles, pmax, psum,
                       pent, nthreads);
}

/* Entropy H_r of every row (fp64), by the definition in the header. */
static int entropy_impl(const double* xd, const uint16_t* xb, int64_t n_rows,
                        int64_t real_vocab, int64_t ld, double* ent, int nthreads) {
  if (n_rows < 0 || real_vocab < 1 || ld < real_vocab) return ORC_ERR_ARG;
  if (n_rows == 0) return ORC_OK;
  if ((!xd && !xb) || !ent) return ORC_ERR_ARG;
  job jb;
  memset(&jb, 0, sizeof jb);
  jb.xd = xd;
  jb.xb = xb;
  jb.n_rows = n_rows;
  jb.real_vocab = real_vocab;
  jb.ld = ld;
  jb.ent = ent;
  jb.fn = entropy_row;
  return run_rows(&jb, nthreads, NULL);
}

int rlk_oracle_entropy_f64(const double* x, int64_t n_rows, int64_t real_vocab, int64_t ld,
                           double* ent, int nthreads) {
  return entropy_impl(x, NULL, n_rows, real_vocab, ld, ent, nthreads);
}

int rlk_oracle_entropy_bf16(const uint16_t* x, int64_t n_rows, int64_t real_vocab, int64_t ld,
                            double* ent, int nthreads) {
  return entropy_impl(NULL, x, n_rows, real_vocab, ld, ent, nthreads);
}

/* The extended backward: d = a g (onehot - p) + gl p - gh p (log p + H) on the
 * real columns, 0 on the padded ones.  g, gl, gh may each be NULL (zero); ent
 * is read only where gh is given.  Errors as for the plain backward. */
static int bwd_ex_impl(const double* xd, const uint16_t* xb, int64_t n_rows, int64_t real_vocab,
                       int64_t padded_vocab, int64_t ld, const int32_t* tgt, const uint8_t* mask,
                       int32_t ignore_index, const double* lse, const double* ent,
                       const double* g, const double* gl, const double* gh, double* d,
                       int64_t ldd, int64_t* bad_row, int nthreads) {
  if (bad_row) *bad_row = -1;
  int rc = check_common(n_rows, real_vocab, ld, xd ? (const void*)xd : (const void*)xb, tgt);
  if (rc) return rc;
  if (padded_vocab < real_vocab || ldd < padded_vocab) return ORC_ERR_ARG;
  if (n_rows == 0) return ORC_OK;
  if (!lse || !d || (gh && !ent)) return ORC_ERR_ARG;
  job jb;
  memset(&jb, 0, sizeof jb);
  jb.xd = xd;
  jb.xb = xb;
  jb.n_rows = n_rows;
  jb.real_vocab = real_vocab;
  jb.padded_vocab = padded_vocab;
  jb.ld = ld;
  jb.ldd = ldd;
  jb.tgt = tgt;
  jb.mask = mask;
  jb.ignore_index = ignore_index;
  jb.lse_in = lse;
  jb.ent_in = ent;
  jb.g = g;
  jb.gl = gl;
  jb.gh = gh;
  jb.d = d;
  jb.fn = bwd_ex_row;
  return run_rows(&jb, nthreads, bad_row);
}

int rlk_oracle_bwd_ex_f64(const double* x, int64_t n_rows, int64_t real_vocab,
                          int64_t padded_vocab, int64_t ld, const int32_t* tgt,
                          const uint8_t* mask, int32_t ignore_index, const double* lse,
                          const double* ent, const double* g, const double* gl,
                          const double* gh, double* d, int64_t ldd, int64_t* bad_row,
                          int nthreads) {
  return bwd_ex_impl(x, NULL, n_rows, real_vocab, padded_vocab, ld, tgt, mask, ignore_index, lse,
                     ent, g, gl, gh, d, ldd, bad_row, nthreads);
}

int rlk_oracle_bwd_ex_bf16(const uint16_t* x, int64_t n_rows, int64_t real_vocab,
                           int64_t padded_vocab, int64_t ld, const int32_t* tgt,
                           const uint8_t* mask, int32_t ignore_index, const double* lse,
                           const double* ent, const double* g, const double* gl,
                           const double* gh, double* d, int64_t ldd, int64_t* bad_row,
                           int nthreads) {
  return bwd_ex_impl(NULL, x, n_rows, real_vocab, padded_vocab, ld, tgt, mask, ignore_index, lse,
                     ent, g, gl, gh, d, ldd, bad_row, nthreads);
}
