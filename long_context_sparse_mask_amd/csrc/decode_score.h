// Scoring of candidate chunks of a per-row problem by their centre keys: the
// query operands (loaded once) and one round's scores, shared by the
// one-stage and multi-stage decode mask kernels.
//
// Method: rebuttal page "A Training-free Sub-quadratic Cost Transformer Model
// Serving Framework With Hierarchically Pruned Attention", reviewer RsGC, Q2,
// step 3 (a chunk's importance is the dot product of the query with the key
// at its centre).  For a bf16 query each wave scores 16 candidates per
// v_mfma_f32_16x16x32_bf16 tile against the query heads of the group
// (zero-padded to 16 rows) and takes the max over the valid head rows of the
// accumulator; fp32 queries use 16-byte VALU dot products with DPP sums.
// fp8 (E5M2) keys are loaded as 8-byte slices and widened exactly to bf16
// operands.  Every load of a batch is issued before any is used (an empty slot
// reads row 0 and discards it), so a round pays one memory latency per batch.
#pragma once

#include <cstddef>
#include <type_traits>

#include "hipsa_internal.h"

namespace hipsa {

// LDS tiles per wave of the row-by-row gathers (score_slots' `stage`: 4 waves
// x kStageTiles x TileGather<KE, D>::kBytes).
constexpr int kStageTiles = 2;
template <typename E, typename KE, int D>
constexpr int stage_bytes() {
  if constexpr (std::is_same<E, uint16_t>::value) return 4 * kStageTiles * TileGather<KE, D>::kBytes;
  else return 16;  // the VALU path stages nothing
}

// Query operands of a problem's group of query heads.  MFMA: lane l holds
// head l%16 (zero when past the group), dims 32*ks + 8*(l/16) .. +7.  VALU:
// every head, dims cs*VEC .. +VEC-1 for the lane's column slice cs.
template <typename E, int D, int GMAX>
struct QueryOps {
  static constexpr bool kMfma = std::is_same<E, uint16_t>::value;
  static constexpr int VEC = Vec<E>::N;
  static constexpr int TPR = D / VEC;  // VALU path: lanes per key row
  static constexpr int KS = D / 32;    // MFMA path: k-steps of 32 over the head dim
  uint4 qa[kMfma ? KS : 1];
  float qv[kMfma ? 1 : GMAX][VEC];

  // qbase: head 0 of the group at the problem's query row; hstride: elements
  // between consecutive heads' rows.
  __device__ __forceinline__ void load(const E *qbase, int64_t hstride, int G) {
    const int tid = threadIdx.x, lane = tid & 63;
    if constexpr (kMfma) {
      const int h = lane & 15;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const uint4 r = Vec<E>::raw(qbase + (int64_t)min(h, G - 1) * hstride + 32 * ks + 8 * (lane >> 4));
        qa[ks] = h < G ? r : make_uint4(0, 0, 0, 0);
      }
    } else {
      const int cs = tid % TPR;
      uint4 r[GMAX];
#pragma unroll
      for (int h = 0; h < GMAX; h++) r[h] = Vec<E>::raw(qbase + (int64_t)min(h, G - 1) * hstride + cs * VEC);
#pragma unroll
      for (int h = 0; h < GMAX; h++) Vec<E>::widen(r[h], h < G, qv[h]);
    }
  }
};

// Row-by-row gathers of one batch of a wave's candidate tiles (the tiles
// t0, t0 + 4, ..., UNROLL of them): lane loads TileGather's 16-byte pieces of
// the centre rows of slots 16 (t0 + 4u) + TG::row(j), centre(c) giving the
// centre token of slot c (0 for an empty slot or c >= n: row 0 is read and
// discarded).  TRIM: tiles from ntile on are skipped.
template <typename KE, int D, int UNROLL, bool TRIM, typename RowOf, typename CentreOf>
__device__ __forceinline__ void gather_batch(const KE *Kbase, RowOf row_of, CentreOf centre, int t0, int ntile,
                                             uint4 (&v)[UNROLL][TileGather<KE, D>::kLoads]) {
  using TG = TileGather<KE, D>;
#pragma unroll
  for (int u = 0; u < UNROLL; u++) {
    if (TRIM && t0 + 4 * u >= ntile) break;  // uniform
#pragma unroll
    for (int j = 0; j < TG::kLoads; j++) v[u][j] = TG::load(Kbase + row_of(centre(16 * (t0 + 4 * u) + TG::row(j))));
  }
}

// Scores one gathered batch (gather_batch): its tiles go through the wave's
// LDS tiles (`mine`) into matrix-core operands, and key[c] = rank_key(max over
// the group's heads, start) for the batch's slots c < n (0 for an empty slot).
template <typename E, typename KE, int D, int GMAX, int UNROLL, bool TRIM>
__device__ __forceinline__ void score_batch(const QueryOps<E, D, GMAX> &qo,
                                            const uint4 (&v)[UNROLL][TileGather<KE, D>::kLoads], int t0,
                                            int ntile, const int32_t *ca, int n, const Shape &s, uint64_t *key,
                                            uint8_t *mine) {
  using TG = TileGather<KE, D>;
  constexpr int KS = QueryOps<E, D, GMAX>::KS;
  const int lane = threadIdx.x & 63;
  const uint4 *qa = qo.qa;
#pragma unroll
  for (int u0 = 0; u0 < UNROLL; u0 += kStageTiles) {
#pragma unroll
    for (int du = 0; du < kStageTiles; du++)
      if (u0 + du < UNROLL && (!TRIM || t0 + 4 * (u0 + du) < ntile)) TG::put(v[u0 + du], mine + du * TG::kBytes);
    wave_lds_sync();
#pragma unroll
    for (int du = 0; du < kStageTiles; du++) {
      const int u = u0 + du;
      if (u >= UNROLL || (TRIM && t0 + 4 * u >= ntile)) break;
      typename TG::raw_t kr[KS];
      TG::get(mine + du * TG::kBytes, kr);
      const int c = 16 * (t0 + 4 * u) + (lane & 15);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[ks]), as_bf16x8(Kv8<KE>::bf16(kr[ks])), acc,
                                                      0, 0, 0);
      float best = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (4 * (lane >> 4) + r < s.G) best = fmaxf(best, acc[r]);
      if (GMAX > 4) best = fmaxf(best, __shfl_xor(best, 16, 64));
      if (GMAX > 8) best = fmaxf(best, __shfl_xor(best, 32, 64));
      if (lane < 16 && c < n) key[c] = ca[c] >= 0 ? rank_key(best, ca[c]) : 0ull;
    }
    wave_lds_sync();  // the next tiles overwrite these
  }
}

// Scores candidate slots [0, n) with chunks (ca[c], ce[c]) in blocks (start
// -1: an empty slot) and writes key[c] = rank_key(score, start), or 0 for an
// empty slot.  Tp: the row's visible length; row_of(t): element offset of the
// K row of position t.  UNROLL: tiles (MFMA) or rows (VALU) per lane whose
// loads are issued together; TRIM: the MFMA path skips a batch's tiles past
// n (for callers whose n varies below what UNROLL was sized for).  With
// `first` non-null (MFMA, `stage` non-null) the wave's first batch was
// gathered already (gather_batch with t0 = the wave) into *first.  Called by
// all 256 threads; LDS reads of ca/ce, no barrier.
template <typename E, typename KE, int D, int GMAX, int UNROLL, bool TRIM = false, typename RowOf,
          typename FirstT = std::nullptr_t>
__device__ __forceinline__ void score_slots(const QueryOps<E, D, GMAX> &qo, const KE *Kbase, RowOf row_of,
                                            const int32_t *ca, const int32_t *ce, int n, int32_t Tp,
                                            const Shape &s, uint64_t *key, uint8_t *stage = nullptr,
                                            FirstT first = nullptr) {
  constexpr bool kMfma = QueryOps<E, D, GMAX>::kMfma;
  constexpr int VEC = QueryOps<E, D, GMAX>::VEC;
  constexpr int TPR = QueryOps<E, D, GMAX>::TPR;
  constexpr int RPP = 256 / TPR;  // VALU path: rows per pass
  constexpr int KS = QueryOps<E, D, GMAX>::KS;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint4 *qa = qo.qa;
  const auto &qv = qo.qv;
  if constexpr (kMfma) {
    const int ntile = (n + 15) / 16;
    if (stage) {  // uniform: rows gathered row by row, through the wave's LDS tiles
      using TG = TileGather<KE, D>;
      uint8_t *mine = stage + wave * kStageTiles * TG::kBytes;
      // centre token of slot c (0 for an empty slot: row 0 is read and discarded)
      auto centre = [&](int c) -> int32_t {
        const int cc = c < n ? c : 0;
        const int32_t lo_b = ca[cc], hi_b = ce[cc];
        const int32_t lo = lo_b << s.bk_shift, hi = min(hi_b << s.bk_shift, Tp);
        return c < n && lo_b >= 0 ? (lo + hi) >> 1 : 0;
      };
      int t0 = wave;
      if constexpr (!std::is_same<FirstT, std::nullptr_t>::value) {
        score_batch<E, KE, D, GMAX, UNROLL, TRIM>(qo, *first, t0, ntile, ca, n, s, key, mine);
        t0 += 4 * UNROLL;
      }
      for (; t0 < ntile; t0 += 4 * UNROLL) {
        uint4 v[UNROLL][TG::kLoads];
        gather_batch<KE, D, UNROLL, TRIM>(Kbase, row_of, centre, t0, ntile, v);
        score_batch<E, KE, D, GMAX, UNROLL, TRIM>(qo, v, t0, ntile, ca, n, s, key, mine);
      }
      return;
    }
    for (int t0 = wave; t0 < ntile; t0 += 4 * UNROLL) {
      typename Kv8<KE>::raw_t kr[UNROLL][KS];
      bool live[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; u++) {
        if (TRIM && t0 + 4 * u >= ntile) break;  // uniform: the wave's tiles are done
        const int c = 16 * (t0 + 4 * u) + (lane & 15);
        const int cc = c < n ? c : 0;
        const int32_t lo_b = ca[cc], hi_b = ce[cc];
        live[u] = c < n && lo_b >= 0;
        const int32_t lo = lo_b << s.bk_shift, hi = min(hi_b << s.bk_shift, Tp);
        const int32_t t = live[u] ? (lo + hi) >> 1 : 0;  // centre token (upper middle)
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
          kr[u][ks] = Kv8<KE>::raw(Kbase + row_of(t) + 32 * ks + 8 * (lane >> 4));
      }
#pragma unroll
      for (int u = 0; u < UNROLL; u++) {
        if (TRIM && t0 + 4 * u >= ntile) break;
        const int c = 16 * (t0 + 4 * u) + (lane & 15);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[ks]),
                                                        as_bf16x8(Kv8<KE>::bf16(kr[u][ks])), acc, 0, 0, 0);
        // acc[r] = score of head 4*(lane/16)+r for candidate lane%16
        float best = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; r++)
          if (4 * (lane >> 4) + r < s.G) best = fmaxf(best, acc[r]);
        if (GMAX > 4) best = fmaxf(best, __shfl_xor(best, 16, 64));
        if (GMAX > 8) best = fmaxf(best, __shfl_xor(best, 32, 64));
        if (lane < 16 && c < n) key[c] = live[u] ? rank_key(best, ca[c]) : 0ull;
      }
    }
  } else {
    const int rg = tid / TPR, cs = tid % TPR;
    for (int base = 0; base < n; base += RPP * UNROLL) {
      uint4 raw[UNROLL];
      bool live[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; u++) {
        const int c = base + u * RPP + rg;
        const int cc = c < n ? c : 0;
        const int32_t lo_b = ca[cc], hi_b = ce[cc];
        live[u] = c < n && lo_b >= 0;
        const int32_t lo = lo_b << s.bk_shift, hi = min(hi_b << s.bk_shift, Tp);
        const int32_t t = live[u] ? (lo + hi) >> 1 : 0;  // centre token (upper middle)
        raw[u] = Vec<E>::raw(Kbase + row_of(t) + cs * VEC);
      }
#pragma unroll
      for (int u = 0; u < UNROLL; u++) {
        const int c = base + u * RPP + rg;
        float kv[VEC];
        Vec<E>::widen(raw[u], live[u], kv);
        float best = -INFINITY;
#pragma unroll
        for (int h = 0; h < GMAX; h++) {
          float p = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; e++) p = fmaf(qv[h][e], kv[e], p);
          p = group_sum<TPR>(p);
          if (h < s.G) best = fmaxf(best, p);
        }
        if (cs == 0 && c < n) key[c] = live[u] ? rank_key(best, ca[c]) : 0ull;
      }
    }
  }
}

}  // namespace hipsa
