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

/* R3: the candidates of a round, the halves of every kept chunk of >= 2
 * blocks and every one-block chunk unchanged; returns their number. */
static int64_t halve_all(const int64_t *ca, const int64_t *ce, int64_t Kb, int64_t *a, int64_t *e) {
  int64_t n = 0;
  for (int64_t i = 0; i < Kb; i++) {
    if (ce[i] - ca[i] >= 2) {
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
    const int64_t n = halve_all(ca, ce, Kb, ha, he);
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
    if (n > Kb && cand[Kb].score != -INFINITY) {
      double hiS = cand[Kb - 1].score, loS = cand[Kb].score;
      double den = fabs(hiS) > fabs(loS) ? fabs(hiS) : fabs(loS);
      rel = den == 0.0 ? 0.0 : (hiS - loS) / den;
    }
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
  const or_shape *s;
  const void *q, *K;
  int64_t b, g, r0, r1, Tp, Kb;
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

static void reach_leaf(reach_ctx *c, const int64_t *ca) {
  for (int64_t i = 0; i < c->Kb; i++) c->leaf_buf[i] = (int32_t)ca[i];
  qsort(c->leaf_buf, (size_t)c->Kb, sizeof(int32_t), cmp_i32);
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

/* Visits every allowed kept set of the round whose chunks are (ca, ce). */
static void reach_round(reach_ctx *c, const int64_t *ca, const int64_t *ce) {
  const int64_t Kb = c->Kb;
  if (c->status || (c->target && c->n_found)) return;
  int wide = 0;
  for (int64_t i = 0; i < Kb; i++) wide |= (ce[i] - ca[i] >= 2);
  if (!wide) { reach_leaf(c, ca); return; }
  if (++c->nodes > c->max_nodes) { c->status = -1; return; }

  /* halve (R3) and score (R4, R5) every chunk */
  int64_t n = 0;
  int64_t *a = malloc(sizeof(int64_t) * 2 * Kb), *e = malloc(sizeof(int64_t) * 2 * Kb);
  double *lo = malloc(sizeof(double) * 2 * Kb), *hi = malloc(sizeof(double) * 2 * Kb);
  double *th = malloc(sizeof(double) * 4 * Kb);
  char *req = malloc((size_t)(2 * Kb)), *in = malloc((size_t)(2 * Kb));
  int64_t *pool = malloc(sizeof(int64_t) * 2 * Kb), *pick = malloc(sizeof(int64_t) * 2 * Kb);
  int64_t *na = malloc(sizeof(int64_t) * Kb), *ne = malloc(sizeof(int64_t) * Kb);
  /* kept sets already visited this round (as candidate membership strings) */
  int64_t seen_cap = 16, n_seen = 0;
  char *seen = malloc((size_t)(seen_cap * 2 * Kb));
  if (!a || !e || !lo || !hi || !th || !req || !in || !pool || !pick || !na || !ne || !seen) {
    c->status = -2;
    goto done;
  }
  n = halve_all(ca, ce, Kb, a, e);
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
  if (n_req > Kb) goto done; /* the target's blocks cannot all survive */

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
    const int64_t need = Kb - base;
    if (bad || need < 0 || need > np) continue;
    /* every choice of `need` free candidates, in lexicographic order */
    for (int64_t i = 0; i < need; i++) pick[i] = i;
    for (;;) {
      for (int64_t i = 0; i < need; i++) in[pool[pick[i]]] = 1;
      int dup = 0;
      for (int64_t v = 0; v < n_seen && !dup; v++) dup = memcmp(seen + v * 2 * Kb, in, (size_t)n) == 0;
      if (!dup) {
        if (n_seen == seen_cap) {
          char *grown = realloc(seen, (size_t)(2 * seen_cap * 2 * Kb));
          if (!grown) { c->status = -2; break; }
          seen = grown;
          seen_cap *= 2;
        }
        memcpy(seen + n_seen * 2 * Kb, in, (size_t)n);
        n_seen++;
        int64_t m = 0;
        for (int64_t j = 0; j < n; j++)
          if (in[j]) { na[m] = a[j]; ne[m] = e[j]; m++; }
        reach_round(c, na, ne);
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
  reach_ctx c = {s, q, K, b, g, r0, r1, Tp, Kb, tol, target, leaves, max_leaves, 0, 0,
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
  reach_round(&c, ca, ce);
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
