// Hierarchical top-k search of one per-row problem, shared by the decode mask
// kernel and the one-launch decode step.
//
// Method: rebuttal page "A Training-free Sub-quadratic Cost Transformer Model
// Serving Framework With Hierarchically Pruned Attention", reviewer RsGC, Q2
// (split into k chunks, halve, score by the centre key, keep the global top-k,
// repeat to block size).
#pragma once

#include <type_traits>

#include "decode_score.h"
#include "hipsa_internal.h"
#include "mask_select.h"

namespace hipsa {

// Runs the search of one problem (b, KV head g, query row i) whose row sees
// Tp keys, over the M > K_b blocks from block `first`: each round scores the
// 2 K_b current candidates (score_slots: centre rows gathered row by row
// through LDS tiles, matrix cores for a bf16 query), then ranks them and
// halves the K_b best (select_top); two barriers per round.  Writes the K_b
// kept block ids in ascending order to out[0..K_b) (global memory or LDS).
// Called by all 256 threads; ends after the write (the caller synchronises
// before reading `out` from LDS).  UNROLL: tiles in flight per wave.
// Matrix-core tiles of 16 candidates per wave and round (UNROLL) for K_b
// (2 K_b candidates over 4 waves), used by the mask kernel and the step alike.
inline int search_tiles_per_wave(int Kb) { return ((2 * Kb + 15) / 16 + 3) / 4; }

//
// SPREAD (one-launch step): the problem's S split workgroups run the same
// search at the same time on one XCD, so after each round's scoring split
// `split` also loads its 1/S share of the centre rows of all halves of the
// current candidates: a superset of the next round's candidates, whose rows
// the next round then finds in the XCD's L2.  The prefetched values are only
// folded into a sink (they complete before the next round's gathers, which
// are issued after them).
template <typename E, typename KE, int D, int GMAX, int UNROLL, bool PAGED, bool SPREAD = false>
__device__ __forceinline__ void search_row(const void *q, const void *K, const Shape &s, const Pages &pg,
                                             uint32_t b, uint32_t g, uint32_t i, int32_t Tp, int32_t first,
                                             int32_t M, int32_t *out, int split = 0, int S = 1) {
  const int tid = threadIdx.x;
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const int32_t Kb = s.Kb;
  __shared__ int32_t cand_a[2][2 * kMaxKb], cand_e[2][2 * kMaxKb];
  __shared__ uint64_t key[2 * kMaxKb + kSpan];
  __shared__ int32_t rk[2 * kMaxKb];
  __shared__ int32_t flag[2];
  __shared__ int32_t pos[kMaxKb];  // places of the kept ids (write_ascending)
  constexpr bool kMfma = std::is_same<E, uint16_t>::value;
  __shared__ __align__(16) uint8_t stage[stage_bytes<E, KE, D>()];
  extern __shared__ int32_t ptab[];  // paged: the sequence's page numbers

  const E *qbase = reinterpret_cast<const E *>(q) + ((int64_t)(b * s.Hq + g * s.G) * Tq + i) * D;
  const KE *Kbase = reinterpret_cast<const KE *>(K);
  const int64_t kvoff = PAGED ? 0 : (int64_t)(b * Hkv + g) * s.T_cap * D;
  const int ps = pg.ps_shift;
  // element offset of the K row of position t
  auto row_of = [&](int32_t t) -> int64_t {
    if constexpr (PAGED) return paged_row(ptab[t >> ps], g, Hkv, t, ps) * D;
    else return kvoff + (int64_t)t * D;
  };

  QueryOps<E, D, GMAX> qo;
  qo.load(qbase, (int64_t)Tq * D, s.G);

  const int n = 2 * Kb;
  // Round 0's candidates are the halves of the initial chunks, known without
  // LDS: with a contiguous cache and one tile per wave (K_b <= 32) the wave
  // gathers its tile's centre rows now, beside the query loads, ahead of the
  // set-up barrier (128k x 4 step 24.42 -> 23.99 us, three interleaved pairs;
  // with two tiles per wave, K_b = 64 at 1M tokens, 32.79 -> 33.04 us).
  constexpr bool kEarly = kMfma && !PAGED && UNROLL == 1;
  using TG = TileGather<std::conditional_t<kEarly, KE, uint16_t>, D>;
  uint4 first0[kEarly ? UNROLL : 1][kEarly ? TG::kLoads : 1];
  if constexpr (kEarly) {
    auto centre0 = [&](int c) -> int32_t {
      int32_t a, e;
      initial_slot(first, M, Kb, c < n ? c : 0, &a, &e);
      const int32_t lo = a << s.bk_shift, hi = min(e << s.bk_shift, Tp);
      return c < n && a >= 0 ? (lo + hi) >> 1 : 0;
    };
    gather_batch<KE, D, UNROLL, false>(Kbase, row_of, centre0, tid >> 6, (n + 15) / 16, first0);
  }
  // paged: page numbers to LDS, issued after the query loads so that both
  // are in flight together (read after the first barrier)
  if constexpr (PAGED) stage_pages(pg, b, Tp, ptab);
  initial_candidates(first, M, Kb, cand_a[0], cand_e[0]);
  if (tid < kSpan) key[n + tid] = 0;  // padding read by the rank batches
  if (tid == 0) flag[0] = 1;          // M > K_b: the first round always runs
  for (int c = tid; c < Kb; c += 256) pos[c] = 0;
  __syncthreads();

  uint4 pf = make_uint4(0u, 0u, 0u, 0u);  // SPREAD: the last prefetched slice
  uint32_t sink = 0;
  int cur = 0;
  for (int round = 0;; round++, cur ^= 1) {
    if (!flag[round & 1]) break;  // uniform: read after a barrier
    if (tid == 0) flag[(round + 1) & 1] = 0;  // its last readers are two barriers back
    const int32_t *ca = cand_a[cur], *ce = cand_e[cur];
    for (int c = tid; c < n; c += 256) rk[c] = 0;  // rank counts of this round

    // ---- 1. scoring
    if constexpr (kEarly) {
      if (round == 0)
        score_slots<E, KE, D, GMAX, UNROLL>(qo, Kbase, row_of, ca, ce, n, Tp, s, key, stage, &first0);
      else
        score_slots<E, KE, D, GMAX, UNROLL>(qo, Kbase, row_of, ca, ce, n, Tp, s, key, stage);
    } else {
      score_slots<E, KE, D, GMAX, UNROLL>(qo, Kbase, row_of, ca, ce, n, Tp, s, key, kMfma ? stage : nullptr);
    }
    if (SPREAD && S > 1) {  // uniform
      sink ^= pf.x ^ pf.w;  // issued before this round's gathers: complete
      // this split's share of the 2n halves (half j of slot j / 2), one
      // 16-byte piece per lane, rows of LPR lanes; branch-free (row 0 when
      // there is nothing to load)
      constexpr int LPR = D * (int)sizeof(KE) / 16;
      const int per = (2 * n + S - 1) / S, r = tid / LPR, ch = split * per + r;
      const int c = (ch >> 1) < n ? (ch >> 1) : 0;
      const int32_t lo_b = ca[c], hi_b = ce[c];
      const bool halves = hi_b - lo_b >= 2;
      const int32_t m = lo_b + (hi_b - lo_b) / 2;
      const int32_t a2 = (ch & 1) ? (halves ? m : -1) : lo_b, e2 = (ch & 1) || halves ? (ch & 1 ? hi_b : m) : hi_b;
      const bool live = r < per && ch < 2 * n && lo_b >= 0 && a2 >= 0;
      const int32_t lo = a2 << s.bk_shift, hi = min(e2 << s.bk_shift, Tp);
      const int32_t t = live ? (lo + hi) >> 1 : 0;
      pf = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(Kbase + row_of(t)) + 16 * (tid % LPR));
    }
    __syncthreads();

    // ---- 2. selection: the K_b best write their halves into the other buffer
    select_top(ca, ce, key, rk, n, Kb, cand_a[cur ^ 1], cand_e[cur ^ 1], &flag[(round + 1) & 1]);
    __syncthreads();
  }


  // the kept one-block chunks sit at the even slots of the current buffer
  write_ascending(cand_a[cur], Kb, pos, out);
  if constexpr (SPREAD)
    if (Tp < 0 && sink == 0x9e3779b9u) out[0] = (int32_t)sink;  // never: keeps the prefetches
}

}  // namespace hipsa
