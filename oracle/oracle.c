/*
 * CPU oracle for HiP mask estimation and block-sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file's library: only the test suite, the smoke check and the
 * bench's CPU-baseline leg do.  It shares no code with the GPU library.
 *
 * Plain, slow and literal on purpose: scalar loops, every value widened to
 * double (fp32, bf16 and fp8-e5m2 inputs convert to double exactly), no
 * blocking, no fusion, no reordering beyond what the method states.
 *
 * Sources (the web pages this follows):
 *  - "A Training-free Sub-quadratic Cost Transformer Model Serving Framework
 *    With Hierarchically Pruned Attention", Author Rebuttal to the Reviewer
 *    RsGC, Q2: the four-step iteration (split T into k chunks; halve every
 *    chunk; score each chunk by the dot product of the query with the key at
 *    the chunk's centre; keep the global top-k and repeat until a chunk is no
 *    larger than b_k).  Same page, reviewer NLBm, Q1: queries and keys are
 *    grouped in blocks b_q and b_k.
 *  - Same page, reviewer NLBm, W2: the sparse attention kernel takes, per
 *    row, the indices of the non-zero blocks and their count (nnz).
 *  - Summary page "A Training-Free Sub-quadratic Cost Transformer Model
 *    Serving Framework with Hierarchically Pruned Attention", Approach:
 *    chunks are represented by their centre tokens; top-k is approximate.
 *  - SGLang pull request "Support Efficient Sparse HiP Attention (InfiniteHiP)
 *    ...", the launch command for the Qwen2.5-VL model: HiP runs with the KV
 *    cache stored as fp8 e5m2; its layer configuration pairs HiP with a
 *    sliding window and a "streaming" (attention-sink) dense part.
 *  - Rebuttal page, reviewer T2wK, Q1: HiP retrieves long-range keys and a
 *    sliding window the local ones, and the two combine well.
 *
 * Readings taken where the pages are silent (each is pinned by a test):
 *  R1 chunk boundaries live on key-block boundaries; the search stops when
 *     every chunk is one block.  K_b = k / block_k chunks are kept.
 *  R2 initial chunks [floor(i*N/K_b), floor((i+1)*N/K_b)), i < K_b.
 *  R3 a chunk [a,e) of >= 2 blocks splits at m = a + floor((e-a)/2);
 *     1-block chunks pass through unsplit and are scored again.
 *  R4 centre token of [a,e): floor((a*b_k + min(e*b_k, T_p)) / 2), the upper
 *     middle of its tokens.
 *  R5 chunk score: max over the query heads of the KV group and the rows of
 *     the query block of q . k_centre (raw dot product, no 1/sqrt(d)); with a
 *     causal mask, a row at position p votes only for centres t <= p; no
 *     voter gives -inf.
 *  R6 ranking: score descending, then chunk start ascending.
 *  R7 if the query block sees no more than K_b blocks, all are selected.
 *  R8 attention: exact softmax of q . k / sqrt(d) over the tokens of the
 *     first nnz listed blocks that the row may see (token < T_p, and token
 *     <= its position when causal); an empty set gives a zero row; listed
 *     ids outside [0, N_p) are ignored.
 *  R9 an fp8 KV cache stores each K and V element as one OCP E5M2 code with
 *     no scale factor (the launch command names the format and nothing
 *     else); the method then runs unchanged on the decoded values, with the
 *     query in its own element type.
 *  R10 dense part: `sink` and `window` (tokens, multiples of b_k) make the
 *     first S_b = sink/b_k blocks and the last W_b = window/b_k of the N_p
 *     blocks a query block sees (fewer when N_p is small: sink first) part
 *     of every row's key set.  The search runs over the blocks between them
 *     only, so the index list holds searched blocks; attention takes the
 *     union of the dense blocks and the listed ones (a listed id inside a
 *     dense range adds nothing).
 *  R11 multi-stage search (a stage list, as InfiniteHiP configures it): see
 *     or_mask_stages_one.
 *
 * or_mask_reach (near-tie-tolerant search) follows the same steps but lets
 * every score move by half a relative tolerance, branching at each cut the
 * tolerance makes ambiguous; it lists every final result the search can then
 * reach.  A GPU that ranks fp32 scores may legitimately take any of them.
 *
 * Layouts (contiguous, head-major): q [B,Hq,Tq,d]; K, V [B,Hkv,T_cap,d] with
 * rows 0..T-1 valid; indices [B,Hkv,NQB,K_b] (ascending, -1 past nnz);
 * nnz [B,Hkv,NQB]; query head h belongs to KV head h / (Hq/Hkv).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1
#define OR_E5M2 2

typedef struct {
  int64_t B, Hq, Hkv, Tq, T, T_cap, d;
  int64_t k, block_k, block_q;
  int32_t causal;
  int32_t dtype;    /* element type of q */
  int32_t kv_dtype; /* element type of K and V */
  int64_t sink, window; /* R10, in tokens (0 = none) */
} or_shape;

/* Optional search trace of one problem; arrays hold max_rounds * cap. */
typedef struct {
  int32_t max_rounds, cap; /* cap >= 2*K_b */
  int32_t rounds;          /* out */
  int32_t *n_cand;         /* [max_rounds] */
  int64_t *cand_start, *cand_end, *cand_centre; /* [max_rounds*cap] */
  double *cand_score;
  int32_t *cand_kept;
  double *rel_margin;      /* [max_rounds] */
} or_trace;

/* One OCP 8-bit float in the E5M2 layout: sign bit, 5 exponent bits with
 * bias 15, 2 mantissa bits.  Exponent 0 is zero or subnormal (m/4 * 2^-14);
 * exponent 31 is infinity (m = 0) or NaN; otherwise (1 + m/4) * 2^(e-15). */
double or_e5m2_value(uint8_t code) {
  const int sign = code >> 7, e = (code >> 2) & 31, m = code & 3;
  double mag;
  if (e == 31) mag = m == 0 ? INFINITY : NAN;
  else if (e == 0) mag = ldexp(m / 4.0, -14);
  else mag = ldexp(1.0 + m / 4.0, e - 15);
  return sign ? -mag : mag;
}

static double elem(const void *base, int32_t dtype, int64_t i) {
  if (dtype == OR_F32) return (double)((const float *)base)[i];
  if (dtype == OR_E5M2) return or_e5m2_value(((const uint8_t *)base)[i]);
  uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int64_t nqb_of(const or_shape *s) { return (s->Tq + s->block_q - 1) / s->block_q; }

/* Query rows [*r0, *r1) of query block qb and the number of visible keys. */
static int64_t rows_and_tp(const or_shape *s, int64_t qb, int64_t *r0, int64_t *r1) {
  *r0 = qb * s->block_q;
  *r1 = *r0 + s->block_q < s->Tq ? *r0 + s->block_q : s->Tq;
  if (!s->causal) return s->T;
  return s->T - s->Tq + (*r1 - 1) + 1; /* position of the last row, plus one */
}

static int64_t position(const or_shape *s, int64_t i) { return s->T - s->Tq + i; }

/* R10: the dense blocks of a query block that sees Np blocks are [0, *sb)
 * and [Np - *wb, Np). */
static void dense_blocks(const or_shape *s, int64_t Np, int64_t *sb, int64_t *wb) {
  int64_t a = s->sink / s->block_k, w = s->window / s->block_k;
  if (a > Np) a = Np;
  if (w > Np - a) w = Np - a;
  *sb = a;
  *wb = w;
}

static double dot_qk(const or_shape *s, const void *q, const void *K, int64_t b, int64_t h,
                     int64_t i, int64_t g, int64_t t) {
  int64_t qo = ((b * s->Hq + h) * s->Tq + i) * s->d;
  int64_t ko = ((b * s->Hkv + g) * s->T_cap + t) * s->d;
  double acc = 0.0;
  for (int64_t x = 0; x < s->d; x++) acc += elem(q, s->dtype, qo + x) * elem(K, s->kv_dtype, ko + x);
  return acc;
}

typedef struct {
  int64_t a, e, t;
  double score;
} cand_t;

/* R2: the K_b initial chunks of the M searched blocks from block `first`. */
static void initial_chunks(int64_t first, int64_t M, int64_t Kb, int64_t *ca, int64_t *ce) {
  for (int64_t i = 0; i < Kb; i++) {
    ca[i] = first + i * M / Kb;
    ce[i] = first + (i + 1) * M / Kb;
  }
}

/* R3: the candidates of a round, the halves of every kept chunk of more than
 * tb blocks and every other chunk unchanged (tb = 1 in the one-stage search;
 * R11: a stage's chunk size in the multi-stage search); returns their number. */
static int64_t halve_all(const int64_t *ca, const int64_t *ce, int64_t Kb, int64_t tb, int64_t *a,
                         int64_t *e) {
  int64_t n = 0;
  for (int64_t i = 0; i < Kb; i++) {
    if (ce[i] - ca[i] > tb) {
      int64_t m = ca[i] + (ce[i] - ca[i]) / 2;
      a[n] = ca[i]; e[n] = m; n++;
      a[n] = m; e[n] = ce[i]; n++;
    } else {
      a[n] = ca[i]; e[n] = ce[i]; n++;
    }
  }
  return n;
}

/* R4, R5: the score of candidate chunk [a, e) (in blocks) for the query
 * rows [r0, r1) of KV head g: the largest q . K[t] over the group's query
 * heads and the rows allowed to vote, t the chunk's centre token (*t_out). */
static double chunk_score(const or_shape *s, const void *q, const void *K, int64_t b, int64_t g,
                          int64_t r0, int64_t r1, int64_t Tp, int64_t a, int64_t e,
                          int64_t *t_out) {
  const int64_t G = s->Hq / s->Hkv;
  int64_t lo = a * s->block_k;
  int64_t hi = e * s->block_k < Tp ? e * s->block_k : Tp;
  int64_t t = (lo + hi) / 2;
  double best = -INFINITY;
  for (int64_t h = g * G; h < (g + 1) * G; h++)
    for (int64_t i = r0; i < r1; i++) {
      if (s->causal && position(s, i) < t) continue;
      double v = dot_qk(s, q, K, b, h, i, g, t);
      if (v > best) best = v;
    }
  *t_out = t;
  return best;
}

/* Relative score gap at a top-k cut between the last kept score hiS and the
 * first dropped score loS (0 when both are 0). */
static double cut_margin(double hiS, double loS) {
  double den = fabs(hiS) > fabs(loS) ? fabs(hiS) : fabs(loS);
  return den == 0.0 ? 0.0 : (hiS - loS) / den;
}

/* R6: true when x ranks before y. */
static int ranks_before(const cand_t *x, const cand_t *y) {
  if (x->score != y->score) return x->score > y->score;
  return x->a < y->a;
}

static int cmp_i32(const void *x, const void *y) {
  int32_t u = *(const int32_t *)x, v = *(const int32_t *)y;
  return (u > v) - (u < v);
}

int or_mask_one(const or_shape *s, const void *q, const void *K, int64_t b, int64_t g, int64_t qb,
                int32_t *idx, int32_t *nnz, double *margin, or_trace *tr) {
  const int64_t Kb = s->k / s->block_k;
  int64_t r0, r1;
  const int64_t Tp = rows_and_tp(s, qb, &r0, &r1);
  const int64_t Np = (Tp + s->block_k - 1) / s->block_k;
  if (tr) tr->rounds = 0;
  for (int64_t j = 0; j < Kb; j++) idx[j] = -1;
  /* R10: the search covers the blocks [lo, lo + M) between the dense parts */
  int64_t sb, wb;
  dense_blocks(s, Np, &sb, &wb);
  const int64_t lo = sb, M = Np - sb - wb;

  if (M <= Kb) { /* R7: the block sees few enough keys to attend to all */
    for (int64_t j = 0; j < M; j++) idx[j] = (int32_t)(lo + j);
    *nnz = (int32_t)M;
    *margin = INFINITY;
    return 0;
  }

  /* Step 1: uniform split into K_b chunks (R2). */
  int64_t *ca = malloc(sizeof(int64_t) * Kb), *ce = malloc(sizeof(int64_t) * Kb);
  int64_t *ha = malloc(sizeof(int64_t) * 2 * Kb), *he = malloc(sizeof(int64_t) * 2 * Kb);
  cand_t *cand = malloc(sizeof(cand_t) * 2 * Kb);
  if (!ca || !ce || !ha || !he || !cand) {
    free(ca); free(ce); free(ha); free(he); free(cand);
    return -1;
  }
  initial_chunks(lo, M, Kb, ca, ce);
  double min_rel = INFINITY;
  int32_t round = 0;

  for (;;) {
    int wide = 0;
    for (int64_t i = 0; i < Kb; i++) wide |= (ce[i] - ca[i] >= 2);
    if (!wide) break; /* Step 4 exit: every chunk is a single block */

    /* Step 2: halve every chunk (R3). */
    const int64_t n = halve_all(ca, ce, Kb, 1, ha, he);
    for (int64_t c = 0; c < n; c++) { cand[c].a = ha[c]; cand[c].e = he[c]; }

    /* Step 3: score each candidate by its centre key (R4, R5). */
    for (int64_t c = 0; c < n; c++)
      cand[c].score = chunk_score(s, q, K, b, g, r0, r1, Tp, cand[c].a, cand[c].e, &cand[c].t);

    /* Step 4: global top-K_b by (score desc, start asc): a stable insertion sort. */
    for (int64_t c = 1; c < n; c++) {
      cand_t x = cand[c];
      int64_t j = c - 1;
      while (j >= 0 && ranks_before(&x, &cand[j])) { cand[j + 1] = cand[j]; j--; }
      cand[j + 1] = x;
    }
    double rel = INFINITY;
    if (n > Kb && cand[Kb].score != -INFINITY) rel = cut_margin(cand[Kb - 1].score, cand[Kb].score);
    if (rel < min_rel) min_rel = rel;

    if (tr && round < tr->max_rounds) {
      tr->n_cand[round] = (int32_t)n;
      tr->rel_margin[round] = rel;
      for (int64_t c = 0; c < n && c < tr->cap; c++) {
        int64_t o = (int64_t)round * tr->cap + c;
        tr->cand_start[o] = cand[c].a;
        tr->cand_end[o] = cand[c].e;
        tr->cand_centre[o] = cand[c].t;
        tr->cand_score[o] = cand[c].score;
        tr->cand_kept[o] = c < Kb;
      }
    }
    for (int64_t i = 0; i < Kb; i++) { ca[i] = cand[i].a; ce[i] = cand[i].e; }
    round++;
  }
  if (tr) tr->rounds = round;

  for (int64_t i = 0; i < Kb; i++) idx[i] = (int32_t)ca[i];
  qsort(idx, (size_t)Kb, sizeof(int32_t), cmp_i32);
  *nnz = (int32_t)Kb;
  *margin = min_rel;
  free(ca); free(ce); free(ha); free(he); free(cand);
  return 0;
}

int or_mask_all(const or_shape *s, const void *q, const void *K, int32_t *indices, int32_t *nnz,
                double *margin, int32_t nthreads) {
  const int64_t Kb = s->k / s->block_k, nqb = nqb_of(s);
  const int64_t P = s->B * s->Hkv * nqb;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : err)
  for (int64_t p = 0; p < P; p++) {
    int64_t b = p / (s->Hkv * nqb), g = (p / nqb) % s->Hkv, qb = p % nqb;
    err |= or_mask_one(s, q, K, b, g, qb, indices + p * Kb, nnz + p, margin + p, NULL);
  }
  return err ? -1 : 0;
}

/* ------------------------------------------------------------------------
 * Near-tie-tolerant search (checks results where the cut is ambiguous).
 *
 * The search is a discrete decision on floating-point scores: when two
 * candidates at a top-k cut score within rounding of each other, a GPU that
 * accumulates in fp32 may keep the other one and, from there, follow another
 * subtree (rebuttal page, reviewer RsGC, Q2: the kept set of each round
 * decides the next round's candidates).  This enumerates every final list
 * the search can reach when each candidate's score may move by up to
 * delta = (tol / 2) * |score|: at every round, a kept set S of K_b
 * candidates is allowed when
 *     min over S of (score + delta) >= max over the rest of (score - delta).
 * At a round whose relative cut gap (the margin of or_mask_one) is at least
 * tol, only the exact top-K_b satisfies this (up to exact equality of the
 * two bounds), so a problem without near-ties reaches exactly the list
 * or_mask_one returns.
 *
 * With `target` (K_b ascending block ids), only paths that can still end at
 * the target are followed: a candidate holding a target block must be kept.
 * Returns the number of distinct final lists reached (1 or 0 with a target),
 * storing up to max_leaves of them (K_b ids each, ascending) in `leaves`
 * (may be NULL); -1 if more than max_nodes kept sets were visited, -2 on an
 * allocation failure.
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t chunk; /* blocks: stage 0 cuts chunks of this size; a later stage halves kept chunks
                    until none is larger */
  int64_t keep;  /* chunks kept per round (0 for stage 0: every chunk) */
} or_stage;

typedef struct {
  const or_shape *s;
  const void *q, *K;
  int64_t b, g, r0, r1, Tp, Kb;
  const or_stage *st; /* stages 1.. of the search (st[0] unused) */
  int32_t nst;
  double tol;
  const int32_t *target;
  int32_t *leaves;
  int64_t max_leaves, n_leaves, n_found;
  int64_t nodes, max_nodes;
  int32_t *leaf_buf; /* K_b scratch */
  int status;
} reach_ctx;

static int contains_target(const reach_ctx *c, int64_t a, int64_t e) {
  for (int64_t j = 0; j < c->Kb; j++)
    if (c->target[j] >= a && c->target[j] < e) return 1;
  return 0;
}

static void reach_leaf(reach_ctx *c, const int64_t *ca, int64_t nk) {
  for (int64_t i = 0; i < nk; i++) c->leaf_buf[i] = (int32_t)ca[i];
  qsort(c->leaf_buf, (size_t)nk, sizeof(int32_t), cmp_i32);
  for (int64_t i = nk; i < c->Kb; i++) c->leaf_buf[i] = -1;
  if (c->target) {
    if (c->n_found == 0 && memcmp(c->leaf_buf, c->target, sizeof(int32_t) * c->Kb) == 0) {
      c->n_found = 1;
      if (c->leaves && c->max_leaves > 0) memcpy(c->leaves, c->leaf_buf, sizeof(int32_t) * c->Kb);
    }
    return;
  }
  /* distinct lists only: a list is compared with the stored ones, so past
   * max_leaves stored lists the count becomes an upper bound */
  const int64_t stored = c->n_found < c->max_leaves ? c->n_found : c->max_leaves;
  for (int64_t l = 0; c->leaves && l < stored; l++)
    if (memcmp(c->leaves + l * c->Kb, c->leaf_buf, sizeof(int32_t) * c->Kb) == 0) return;
  if (c->leaves && c->n_found < c->max_leaves)
    memcpy(c->leaves + c->n_found * c->Kb, c->leaf_buf, sizeof(int32_t) * c->Kb);
  c->n_found++;
}

/* Visits every allowed kept set of the round of stage `stage` whose nk
 * chunks are (ca, ce); `fresh`: the stage's first round, which always runs. */
static void reach_round(reach_ctx *c, int32_t stage, int fresh, const int64_t *ca,
                        const int64_t *ce, int64_t nk) {
  if (c->status || (c->target && c->n_found)) return;
  const int64_t tb = c->st[stage].chunk, Kb = c->st[stage].keep;
  int wide = 0;
  for (int64_t i = 0; i < nk; i++) wide |= (ce[i] - ca[i] > tb);
  if (!wide && !fresh) { /* the stage is done: the next one, or the result */
    if (stage + 1 < c->nst) reach_round(c, stage + 1, 1, ca, ce, nk);
    else reach_leaf(c, ca, nk);
    return;
  }
  if (++c->nodes > c->max_nodes) { c->status = -1; return; }

  /* halve (R3) and score (R4, R5) every chunk */
  int64_t n = 0;
  const int64_t cap = 2 * nk;
  int64_t *a = malloc(sizeof(int64_t) * cap), *e = malloc(sizeof(int64_t) * cap);
  double *lo = malloc(sizeof(double) * cap), *hi = malloc(sizeof(double) * cap);
  double *th = malloc(sizeof(double) * 2 * cap);
  char *req = malloc((size_t)cap), *in = malloc((size_t)cap);
  int64_t *pool = malloc(sizeof(int64_t) * cap), *pick = malloc(sizeof(int64_t) * cap);
  int64_t *na = malloc(sizeof(int64_t) * cap), *ne = malloc(sizeof(int64_t) * cap);
  /* kept sets already visited this round (as candidate membership strings) */
  int64_t seen_cap = 16, n_seen = 0;
  char *seen = malloc((size_t)(seen_cap * cap));
  int64_t keep = 0;
  if (!a || !e || !lo || !hi || !th || !req || !in || !pool || !pick || !na || !ne || !seen) {
    c->status = -2;
    goto done;
  }
  n = halve_all(ca, ce, nk, tb, a, e);
  keep = n < Kb ? n : Kb;
  int64_t n_req = 0;
  for (int64_t j = 0; j < n; j++) {
    int64_t t;
    double sc = chunk_score(c->s, c->q, c->K, c->b, c->g, c->r0, c->r1, c->Tp, a[j], e[j], &t);
    double dl = isfinite(sc) ? 0.5 * c->tol * fabs(sc) : 0.0;
    lo[j] = sc - dl;
    hi[j] = sc + dl;
    th[2 * j] = lo[j];
    th[2 * j + 1] = hi[j];
    req[j] = c->target ? (char)contains_target(c, a[j], e[j]) : 0;
    n_req += req[j];
  }
  if (n_req > keep) goto done; /* the target's blocks cannot all survive */

  /* A kept set S is allowed iff some threshold th has every member with
   * hi >= th and every other candidate with lo <= th; it suffices to try
   * the bounds themselves as th.  For each: candidates with lo > th must be
   * kept, those with hi < th dropped, the others are free. */
  for (int64_t k = 0; k < 2 * n && !c->status; k++) {
    const double t0 = th[k];
    int64_t base = 0, np = 0, bad = 0;
    for (int64_t j = 0; j < n; j++) {
      const int must_in = lo[j] > t0, must_out = hi[j] < t0;
      if (must_in || req[j]) {
        if (must_out) bad = 1;
        in[j] = 1;
        base++;
      } else {
        in[j] = 0;
        if (!must_out) pool[np++] = j;
      }
    }
    const int64_t need = keep - base;
    if (bad || need < 0 || need > np) continue;
    /* every choice of `need` free candidates, in lexicographic order */
    for (int64_t i = 0; i < need; i++) pick[i] = i;
    for (;;) {
      for (int64_t i = 0; i < need; i++) in[pool[pick[i]]] = 1;
      int dup = 0;
      for (int64_t v = 0; v < n_seen && !dup; v++) dup = memcmp(seen + v * cap, in, (size_t)n) == 0;
      if (!dup) {
        if (n_seen == seen_cap) {
          char *grown = realloc(seen, (size_t)(2 * seen_cap * cap));
          if (!grown) { c->status = -2; break; }
          seen = grown;
          seen_cap *= 2;
        }
        memcpy(seen + n_seen * cap, in, (size_t)n);
        n_seen++;
        int64_t m = 0;
        for (int64_t j = 0; j < n; j++)
          if (in[j]) { na[m] = a[j]; ne[m] = e[j]; m++; }
        reach_round(c, stage, 0, na, ne, m);
        if (c->status || (c->target && c->n_found)) break;
      }
      for (int64_t i = 0; i < need; i++) in[pool[pick[i]]] = 0;
      int64_t i = need - 1;
      while (i >= 0 && pick[i] == np - need + i) i--;
      if (i < 0) break;
      pick[i]++;
      for (int64_t j = i + 1; j < need; j++) pick[j] = pick[j - 1] + 1;
    }
  }
done:
  free(a); free(e); free(lo); free(hi); free(th); free(req); free(in); free(pool); free(pick);
  free(na); free(ne); free(seen);
}

int64_t or_mask_reach(const or_shape *s, const void *q, const void *K, int64_t b, int64_t g,
                      int64_t qb, double tol, const int32_t *target, int32_t *leaves,
                      int64_t max_leaves, int64_t max_nodes) {
  const int64_t Kb = s->k / s->block_k;
  int64_t r0, r1;
  const int64_t Tp = rows_and_tp(s, qb, &r0, &r1);
  const int64_t Np = (Tp + s->block_k - 1) / s->block_k;
  int64_t sb, wb;
  dense_blocks(s, Np, &sb, &wb);
  const int64_t first = sb, M = Np - sb - wb;
  const or_stage one[2] = {{0, 0}, {1, Kb}}; /* one stage: halve to single blocks, keep K_b */
  reach_ctx c = {s, q, K, b, g, r0, r1, Tp, Kb, one, 2, tol, target, leaves, max_leaves, 0, 0,
                 0, max_nodes, NULL, 0};
  if (Kb >= M) { /* R7: one possible result */
    int ok = 1;
    for (int64_t j = 0; j < Kb && target; j++) ok &= target[j] == (j < M ? first + j : -1);
    if (leaves && max_leaves > 0 && ok)
      for (int64_t j = 0; j < Kb; j++) leaves[j] = (int32_t)(j < M ? first + j : -1);
    return ok;
  }
  int64_t *ca = malloc(sizeof(int64_t) * Kb), *ce = malloc(sizeof(int64_t) * Kb);
  c.leaf_buf = malloc(sizeof(int32_t) * Kb);
  if (!ca || !ce || !c.leaf_buf) { free(ca); free(ce); free(c.leaf_buf); return -2; }
  initial_chunks(first, M, Kb, ca, ce);
  reach_round(&c, 1, 1, ca, ce, Kb);
  free(ca); free(ce); free(c.leaf_buf);
  return c.status ? c.status : c.n_found;
}

/* ------------------------------------------------------------------------
 * R11 multi-stage search (InfiniteHiP's stage list).
 *
 * The SGLang pull request's layer configuration lists stages, each with a
 * chunk size and a number of keys kept (stage_chunk_size 128 -> 32 -> 8,
 * stage_k null -> 32768 -> 8192), and the InfiniteHiP pages describe the
 * pruning as modular and hierarchical; the rebuttal page (reviewer KprR, W3;
 * reviewer T2wK, Q1) says users now choose per iteration how many chunks are
 * kept and how each chunk is broken down.  Reading, with sizes in key blocks:
 *  - stage 0 (its k is null) cuts the searched blocks into consecutive
 *    chunks of st[0].chunk blocks (the last one takes what is left) and
 *    keeps every one;
 *  - a later stage s runs the one-stage iteration on the chunks the previous
 *    stage kept: every chunk larger than st[s].chunk blocks is halved as in
 *    R3 (others pass through and are scored again), the candidates are
 *    scored as in R4/R5 and the st[s].keep best (R6) are kept; rounds repeat
 *    while a kept chunk is larger than st[s].chunk.  A stage runs at least
 *    one round, so it always applies its own kept count (chunks that already
 *    fit are only scored again and ranked);
 *  - the last stage's chunk size is one block, so its kept chunks are the
 *    result: ascending, nnz = their count (at most st[last].keep);
 *  - if the searched blocks number at most st[last].keep, all are selected
 *    (R7).
 * The stage's query block size and stride (which query rows of a chunked-
 * prefill block vote) are not part of this reading: it serves per-row
 * problems.  With st[0].chunk = M / K_b (M a multiple of K_b) and one later
 * stage {1, K_b}, this is the one-stage search (or_mask_one) exactly.
 * Returns -3 for an invalid stage list: nst >= 2, st[0].keep == 0,
 * st[s].keep >= 1 and st[s].chunk < st[s-1].chunk for s >= 1, the last
 * chunk 1, and k == st[last].keep * block_k.
 * ------------------------------------------------------------------------ */
/* R11 stage 0: consecutive chunks of c0 blocks over the M searched blocks
 * from block `first`, the last one taking what is left; returns their number. */
static int64_t stage0_chunks(int64_t first, int64_t M, int64_t c0, int64_t *ca, int64_t *ce) {
  const int64_t n = (M + c0 - 1) / c0;
  for (int64_t j = 0; j < n; j++) {
    ca[j] = first + j * c0;
    ce[j] = first + (j + 1) * c0 < first + M ? first + (j + 1) * c0 : first + M;
  }
  return n;
}

static int stages_valid(const or_shape *s, const or_stage *st, int32_t nst) {
  if (nst < 2 || st[0].keep != 0 || st[0].chunk < 1 || st[nst - 1].chunk != 1) return 0;
  for (int32_t j = 1; j < nst; j++)
    if (st[j].keep < 1 || st[j].chunk >= st[j - 1].chunk) return 0;
  return s->k == st[nst - 1].keep * s->block_k;
}

int or_mask_stages_one(const or_shape *s, const or_stage *st, int32_t nst, const void *q,
                       const void *K, int64_t b, int64_t g, int64_t qb, int32_t *idx,
                       int32_t *nnz, double *margin, or_trace *tr) {
  if (!stages_valid(s, st, nst)) return -3;
  const int64_t Kb = st[nst - 1].keep;
  int64_t r0, r1;
  const int64_t Tp = rows_and_tp(s, qb, &r0, &r1);
  const int64_t Np = (Tp + s->block_k - 1) / s->block_k;
  int64_t sb, wb;
  dense_blocks(s, Np, &sb, &wb);
  const int64_t first = sb, M = Np - sb - wb;
  for (int64_t j = 0; j < Kb; j++) idx[j] = -1;
  *margin = INFINITY;
  if (tr) tr->rounds = 0;
  if (Kb >= M) { /* R7 */
    for (int64_t j = 0; j < M; j++) idx[j] = (int32_t)(first + j);
    *nnz = (int32_t)M;
    return 0;
  }
  /* stage 0: consecutive chunks of st[0].chunk blocks */
  const int64_t c0 = st[0].chunk, n0 = (M + c0 - 1) / c0;
  int64_t cap = 2 * n0;
  for (int32_t j = 1; j < nst; j++) cap = cap > 2 * st[j].keep ? cap : 2 * st[j].keep;
  int64_t *ca = malloc(sizeof(int64_t) * cap), *ce = malloc(sizeof(int64_t) * cap);
  int64_t *ha = malloc(sizeof(int64_t) * cap), *he = malloc(sizeof(int64_t) * cap);
  cand_t *cand = malloc(sizeof(cand_t) * cap);
  if (!ca || !ce || !ha || !he || !cand) {
    free(ca); free(ce); free(ha); free(he); free(cand);
    return -1;
  }
  int64_t nk = stage0_chunks(first, M, c0, ca, ce);
  double min_rel = INFINITY;
  for (int32_t stage = 1; stage < nst; stage++) {
    const int64_t tb = st[stage].chunk, keep = st[stage].keep;
    for (int fresh = 1;; fresh = 0) {
      int wide = 0;
      for (int64_t i = 0; i < nk; i++)
        if (ce[i] - ca[i] > tb) wide = 1;
      if (!wide && !fresh) break; /* the stage is done */
      const int64_t n = halve_all(ca, ce, nk, tb, ha, he);
      for (int64_t c = 0; c < n; c++) {
        cand[c].a = ha[c];
        cand[c].e = he[c];
        cand[c].score = chunk_score(s, q, K, b, g, r0, r1, Tp, ha[c], he[c], &cand[c].t);
      }
      /* global top-keep by (score desc, start asc): a stable insertion sort */
      for (int64_t c = 1; c < n; c++) {
        cand_t x = cand[c];
        int64_t j = c - 1;
        while (j >= 0 && ranks_before(&x, &cand[j])) { cand[j + 1] = cand[j]; j--; }
        cand[j + 1] = x;
      }
      const int64_t kept = n < keep ? n : keep;
      double rel = INFINITY;
      if (n > keep && cand[keep].score != -INFINITY) rel = cut_margin(cand[keep - 1].score, cand[keep].score);
      if (rel < min_rel) min_rel = rel;
      if (tr && tr->rounds < tr->max_rounds) {
        const int32_t r = tr->rounds++;
        tr->n_cand[r] = (int32_t)n;
        tr->rel_margin[r] = rel;
        for (int64_t c = 0; c < n && c < tr->cap; c++) {
          const int64_t o = (int64_t)r * tr->cap + c;
          tr->cand_start[o] = cand[c].a;
          tr->cand_end[o] = cand[c].e;
          tr->cand_centre[o] = cand[c].t;
          tr->cand_score[o] = cand[c].score;
          tr->cand_kept[o] = c < kept;
        }
      }
      for (int64_t i = 0; i < kept; i++) { ca[i] = cand[i].a; ce[i] = cand[i].e; }
      nk = kept;
    }
  }
  int rc = 0;
  if (nk > Kb) { /* cannot happen: the last stage keeps at most K_b chunks */
    rc = -1;
  } else {
    for (int64_t i = 0; i < nk; i++) idx[i] = (int32_t)ca[i];
    qsort(idx, (size_t)nk, sizeof(int32_t), cmp_i32);
    *nnz = (int32_t)nk;
    *margin = min_rel;
  }
  free(ca); free(ce); free(ha); free(he); free(cand);
  return rc;
}

int or_mask_stages_all(const or_shape *s, const or_stage *st, int32_t nst, const void *q,
                       const void *K, int32_t *indices, int32_t *nnz, double *margin,
                       int32_t nthreads) {
  if (!stages_valid(s, st, nst)) return -3;
  const int64_t Kb = st[nst - 1].keep, nqb = nqb_of(s);
  const int64_t P = s->B * s->Hkv * nqb;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads) reduction(| : err)
  for (int64_t p = 0; p < P; p++) {
    int64_t b = p / (s->Hkv * nqb), g = (p / nqb) % s->Hkv, qb = p % nqb;
    err |= or_mask_stages_one(s, st, nst, q, K, b, g, qb, indices + p * Kb, nnz + p, margin + p,
                              NULL);
  }
  return err ? -1 : 0;
}

/* The near-tie-tolerant search over a stage list (see or_mask_reach). */
int64_t or_mask_stages_reach(const or_shape *s, const or_stage *st, int32_t nst, const void *q,
                             const void *K, int64_t b, int64_t g, int64_t qb, double tol,
                             const int32_t *target, int32_t *leaves, int64_t max_leaves,
                             int64_t max_nodes) {
  if (!stages_valid(s, st, nst)) return -3;
  const int64_t Kb = st[nst - 1].keep;
  int64_t r0, r1;
  const int64_t Tp = rows_and_tp(s, qb, &r0, &r1);
  const int64_t Np = (Tp + s->block_k - 1) / s->block_k;
  int64_t sb, wb;
  dense_blocks(s, Np, &sb, &wb);
  const int64_t first = sb, M = Np - sb - wb;
  reach_ctx c = {s, q, K, b, g, r0, r1, Tp, Kb, st, nst, tol, target, leaves, max_leaves, 0, 0,
                 0, max_nodes, NULL, 0};
  if (Kb >= M) { /* R7: one possible result */
    int ok = 1;
    for (int64_t j = 0; j < Kb && target; j++) ok &= target[j] == (j < M ? first + j : -1);
    if (leaves && max_leaves > 0 && ok)
      for (int64_t j = 0; j < Kb; j++) leaves[j] = (int32_t)(j < M ? first + j : -1);
    return ok;
  }
  const int64_t c0 = st[0].chunk, n0 = (M + c0 - 1) / c0;
  int64_t *ca = malloc(sizeof(int64_t) * n0), *ce = malloc(sizeof(int64_t) * n0);
  c.leaf_buf = malloc(sizeof(int32_t) * Kb);
  if (!ca || !ce || !c.leaf_buf) { free(ca); free(ce); free(c.leaf_buf); return -2; }
  reach_round(&c, 1, 1, ca, ce, stage0_chunks(first, M, c0, ca, ce));
  free(ca); free(ce); free(c.leaf_buf);
  return c.status ? c.status : c.n_found;
}

/* R8: one output row in fp64. */
int or_attn_row(const or_shape *s, const void *q, const void *K, const void *V,
                const int32_t *indices, const int32_t *nnz, int64_t b, int64_t h, int64_t i,
                double *out) {
  const int64_t G = s->Hq / s->Hkv, Kb = s->k / s->block_k, nqb = nqb_of(s);
  const int64_t g = h / G, qb = i / s->block_q;
  int64_t r0, r1;
  const int64_t Tp = rows_and_tp(s, qb, &r0, &r1);
  const int64_t Np = (Tp + s->block_k - 1) / s->block_k;
  const int64_t limit = s->causal ? position(s, i) : s->T - 1; /* last visible token */
  const int64_t p = (b * s->Hkv + g) * nqb + qb;
  const int32_t *list = indices + p * Kb;
  int64_t cnt = nnz[p];
  if (cnt < 0) cnt = 0;
  if (cnt > Kb) cnt = Kb;
  const double scale = 1.0 / sqrt((double)s->d);
  /* R10: the row's blocks are the dense ones, then the listed ones outside
   * the dense ranges; entry n of this sequence is block blk_at(n) or -1 */
  int64_t sb, wb;
  dense_blocks(s, Np, &sb, &wb);
  const int64_t nd = sb + wb;
#define BLK_AT(n)                                                                   \
  ((n) < sb ? (n)                                                                   \
   : (n) < nd ? Np - wb + ((n) - sb)                                                \
   : (list[(n) - nd] < 0 || list[(n) - nd] >= Np || list[(n) - nd] < sb ||          \
      list[(n) - nd] >= Np - wb) ? -1 : list[(n) - nd])

  for (int64_t x = 0; x < s->d; x++) out[x] = 0.0;
  /* pass 1: the largest logit, for a stable softmax */
  double mx = -INFINITY;
  int64_t seen = 0;
  for (int64_t n = 0; n < nd + cnt; n++) {
    int64_t blk = BLK_AT(n);
    if (blk < 0) continue;
    for (int64_t t = blk * s->block_k; t < (blk + 1) * s->block_k && t < Tp; t++) {
      if (t > limit) continue;
      double l = dot_qk(s, q, K, b, h, i, g, t) * scale;
      if (l > mx) mx = l;
      seen++;
    }
  }
  if (seen == 0) return 0;
  /* pass 2: weights and the weighted sum of values */
  double den = 0.0;
  for (int64_t n = 0; n < nd + cnt; n++) {
    int64_t blk = BLK_AT(n);
    if (blk < 0) continue;
    for (int64_t t = blk * s->block_k; t < (blk + 1) * s->block_k && t < Tp; t++) {
      if (t > limit) continue;
      double w = exp(dot_qk(s, q, K, b, h, i, g, t) * scale - mx);
      den += w;
      int64_t vo = ((b * s->Hkv + g) * s->T_cap + t) * s->d;
      for (int64_t x = 0; x < s->d; x++) out[x] += w * elem(V, s->kv_dtype, vo + x);
    }
  }
#undef BLK_AT
  for (int64_t x = 0; x < s->d; x++) out[x] /= den;
  return 0;
}

int or_attn_all(const or_shape *s, const void *q, const void *K, const void *V,
                const int32_t *indices, const int32_t *nnz, double *out, int32_t nthreads) {
  const int64_t R = s->B * s->Hq * s->Tq;
#pragma omp parallel for schedule(dynamic, 4) num_threads(nthreads)
  for (int64_t r = 0; r < R; r++) {
    int64_t b = r / (s->Hq * s->Tq), h = (r / s->Tq) % s->Hq, i = r % s->Tq;
    or_attn_row(s, q, K, V, indices, nnz, b, h, i, out + r * s->d);
  }
  return 0;
}
