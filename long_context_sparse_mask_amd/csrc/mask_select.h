// Selection step of the hierarchical top-k search, shared by the per-row
// (decode) and per-query-block (prefill) mask kernels.
//
// Rebuttal page "A Training-free Sub-quadratic Cost Transformer Model Serving
// Framework With Hierarchically Pruned Attention", reviewer RsGC, Q2, step 4:
// keep the k most important chunks of all 2k candidates, then split them
// again.  Candidates live in LDS as (start, end) block ranges, double
// buffered; an empty slot has start -1 and key 0.  A candidate's key packs
// its score (IEEE order mapped onto unsigned order) above the complement of
// its start, so a larger key ranks first and equal scores prefer the lower
// start.
#pragma once

#include "hipsa_internal.h"

namespace hipsa {

constexpr int kSpan = 16;  // keys compared per batch of LDS reads

// Ranks the n candidates of buffer (ca, ce) by key and writes the halves of
// the K_b best into buffer (na, ne) at slots 2*rank and 2*rank+1 (a one-block
// chunk is copied to 2*rank with an empty slot after it).  Sets *more when a
// kept chunk still spans several blocks.  `key` must hold n valid entries
// followed by kSpan zeros; `rk` must hold n zeros on entry (the caller clears
// it before the barrier that ends scoring).  A candidate's rank is the number
// of keys above its own: all 256 threads share the comparisons, thread t
// counting for candidate t % n over the kSpan keys of batch t / n, and the
// counts meet in `rk`.  Called by all 256 threads; contains one barrier.
__device__ inline void select_top(const int32_t *ca, const int32_t *ce, const uint64_t *key,
                                  int32_t *rk, int n, int Kb, int32_t *na, int32_t *ne,
                                  int32_t *more) {
  const int parts = (n + kSpan - 1) / kSpan;
  if (256 % n == 0) {
    // every batch of thread t is for the same candidate t % n: the batches'
    // reads are issued together and the counts meet in one atomic
    const int c = threadIdx.x % n, stride = 256 / n;
    const uint64_t kc = key[c];
    int r = 0;
#pragma unroll 4
    for (int p = threadIdx.x / n; p < parts; p += stride) {
      uint64_t kk[kSpan];
#pragma unroll
      for (int u = 0; u < kSpan; u++) kk[u] = key[p * kSpan + u];
#pragma unroll
      for (int u = 0; u < kSpan; u++) r += kk[u] > kc;
    }
    if (r && kc) atomicAdd(&rk[c], r);
  } else {
    for (int t = threadIdx.x; t < n * parts; t += 256) {
      const int c = t % n, j0 = (t / n) * kSpan;
      const uint64_t kc = key[c];
      uint64_t kk[kSpan];
#pragma unroll
      for (int u = 0; u < kSpan; u++) kk[u] = key[j0 + u];
      int r = 0;
#pragma unroll
      for (int u = 0; u < kSpan; u++) r += kk[u] > kc;
      if (r && kc) atomicAdd(&rk[c], r);
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < n; c += 256) {
    const int r = rk[c];
    if (key[c] == 0 || r >= Kb) continue;
    const int32_t lo = ca[c], hi = ce[c];
    const bool split = hi - lo >= 2;
    const int32_t m = lo + (hi - lo) / 2;
    na[2 * r] = lo;
    ne[2 * r] = split ? m : hi;
    na[2 * r + 1] = split ? m : -1;
    ne[2 * r + 1] = split ? hi : -1;
    if (split) *more = 1;
  }
}

// The K_b kept one-block chunks sit at the even slots of `fin`; writes their
// block ids to out[0..K_b) in ascending order: an id's place is the number of
// smaller ids.  When 256 is a multiple of K_b and 16 <= K_b <= 128, 256 / K_b
// threads share an id's comparisons and the counts meet in `pos` (K_b zeros
// on entry, visible to every thread: cleared before a barrier), one barrier;
// otherwise thread c counts for id c alone.  Called by all 256 threads.
__device__ inline void write_ascending(const int32_t *fin, int Kb, int32_t *pos, int32_t *out) {
  if (256 % Kb == 0 && Kb >= 16 && Kb <= 128) {
    const int parts = 256 / Kb, span = Kb / parts;  // a power of two, >= 1
    const int c = threadIdx.x % Kb, j0 = (threadIdx.x / Kb) * span;
    const int32_t v = fin[2 * c];
    int r = 0;
    for (int u0 = 0; u0 < span; u0 += 4) {
      int32_t kk[4];
#pragma unroll
      for (int u = 0; u < 4; u++) kk[u] = fin[2 * (j0 + min(u0 + u, span - 1))];
#pragma unroll
      for (int u = 0; u < 4; u++) r += (u0 + u < span) & (kk[u] < v);
    }
    if (r) atomicAdd(&pos[c], r);
    __syncthreads();
    if (threadIdx.x < Kb) out[pos[c]] = v;
    return;
  }
  for (int c = threadIdx.x; c < Kb; c += 256) {
    const int32_t v = fin[2 * c];
    int r = 0;
#pragma unroll 4
    for (int j0 = 0; j0 < Kb; j0 += kSpan) {  // batches' reads issued together
      int32_t kk[kSpan];
#pragma unroll
      for (int u = 0; u < kSpan; u++) kk[u] = fin[2 * min(j0 + u, Kb - 1)];
#pragma unroll
      for (int u = 0; u < kSpan; u++) r += (j0 + u < Kb) & (kk[u] < v);
    }
    out[r] = v;
  }
}

// Candidate slot cs (of 2 K_b) of the first round: half cs % 2 of initial
// chunk cs / 2 of the uniform partition of the M searched blocks from block
// `first`, first + [floor(c*M/K_b), floor((c+1)*M/K_b)) (exact in double); a
// one-block chunk fills slot 2c and leaves slot 2c+1 empty (start -1).
__device__ inline void initial_slot(int32_t first, int32_t M, int Kb, int cs, int32_t *a, int32_t *e) {
  const int c = cs >> 1;
  const int32_t lo = first + (int32_t)((double)c * M / Kb);
  const int32_t hi = first + (int32_t)((double)(c + 1) * M / Kb);
  const bool split = hi - lo >= 2;
  const int32_t m = lo + (hi - lo) / 2;
  *a = (cs & 1) ? (split ? m : -1) : lo;
  *e = (cs & 1) ? (split ? hi : -1) : (split ? m : hi);
}

// All 2 K_b first-round slots into (ca, ce).
__device__ inline void initial_candidates(int32_t first, int32_t M, int Kb, int32_t *ca, int32_t *ce) {
  for (int cs = threadIdx.x; cs < 2 * Kb; cs += 256) initial_slot(first, M, Kb, cs, &ca[cs], &ce[cs]);
}

}  // namespace hipsa
