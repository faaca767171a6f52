// Pipelined hierarchical top-k search of one per-row problem (bf16 query and
// keys), shared by the decode mask kernel and the one-launch decode step.
//
// Method: rebuttal page "A Training-free Sub-quadratic Cost Transformer Model
// Serving Framework With Hierarchically Pruned Attention", reviewer RsGC, Q2
// (split into k chunks, halve, score by the centre key, keep the global top-k,
// repeat to block size).
#pragma once

#include "hipsa_internal.h"
#include "mask_select.h"

namespace hipsa {

// Pipelined variant for bf16 queries and keys, contiguous layout, K_b <= 32.  The children of every current
// candidate are a superset of the next round's candidates, so in round r
// waves 1-3 load and score all 4*K_b children of C_r on the matrix cores
// while wave 0 ranks C_r with the keys the other waves produced in round r-1.
// The dependent memory latency then overlaps the selection instead of
// following it, and a round needs one barrier.  Keys of the next round's
// candidates are looked up through `srcs` (the child slot that holds each
// candidate's key).  The speculation doubles the rows gathered per round,
// which pays while a round's gather costs mostly latency (up to 128 rows);
// at K_b = 64 (256 rows per round, and a 128-candidate ranking on one wave)
// the plain kernel is faster.  The limit, kPipeMaxKb, is in hipsa_internal.h.

// Scores slots [0, nslot): the current candidates (ca, ce), or with
// `children` child (cs & 1) of current candidate cs / 2, or with INIT the
// first round's slots computed in registers from (first, M, K_b) (no LDS, so
// no barrier has to precede it).  Wave wi of nw takes tiles wi, wi + nw, ...
template <typename KE, int D, int GMAX, int TPW, bool INIT = false, typename RowOf>
__device__ inline void score_children(const KE *Kbase, RowOf row_of, const uint4 *qa, int32_t Tp, int bk_shift,
                                      int G, const int32_t *ca, const int32_t *ce, int nslot,
                                      bool children, int wi, int nw, uint64_t *dst, int32_t first = 0,
                                      int32_t M = 0, int Kb = 1) {
  constexpr int KS = D / 32;
  const int lane = threadIdx.x & 63;
  const int ntile = (nslot + 15) / 16;
  for (int t0 = wi; t0 < ntile; t0 += nw * TPW) {
    typename Kv8<KE>::raw_t kr[TPW][KS];
    bool live[TPW];
    int32_t start[TPW];
#pragma unroll
    for (int u = 0; u < TPW; u++) {
      const int cs = 16 * (t0 + nw * u) + (lane & 15);
      // slot cs: a current candidate, or child (cs & 1) of current candidate cs >> 1
      const int c = children ? (cs >> 1) : cs;
      const int cc = c < (children ? nslot / 2 : nslot) ? c : 0;
      int32_t plo, phi;
      if constexpr (INIT) initial_slot(first, M, Kb, cc, &plo, &phi);
      else plo = ca[cc], phi = ce[cc];
      int32_t lo = plo, hi = phi;
      bool ok = cs < nslot && plo >= 0;
      if (children) {
        const bool split = phi - plo >= 2;
        const int32_t m = plo + (phi - plo) / 2;
        const int j = cs & 1;
        lo = (split && j) ? m : plo;
        hi = (split && !j) ? m : phi;
        ok = ok && (split || j == 0);
      }
      live[u] = ok;
      start[u] = lo;
      const int32_t tlo = lo << bk_shift, thi = min(hi << bk_shift, Tp);
      const int32_t t = ok ? (tlo + thi) >> 1 : 0;  // centre token (upper middle)
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        kr[u][ks] = Kv8<KE>::raw(Kbase + row_of(t) + 32 * ks + 8 * (lane >> 4));
    }
#pragma unroll
    for (int u = 0; u < TPW; u++) {
      const int cs = 16 * (t0 + nw * u) + (lane & 15);
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[ks]), as_bf16x8(Kv8<KE>::bf16(kr[u][ks])), acc, 0, 0, 0);
      float best = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; r++)
        if (4 * (lane >> 4) + r < G) best = fmaxf(best, acc[r]);
      if (GMAX > 4) best = fmaxf(best, __shfl_xor(best, 16, 64));
      if (GMAX > 8) best = fmaxf(best, __shfl_xor(best, 32, 64));
      if (lane < 16 && cs < nslot) dst[cs] = live[u] ? rank_key(best, start[u]) : 0ull;
    }
  }
}

// Runs the pipelined search of one problem (b, KV head g, query row i) whose
// row sees Tp keys, over the M > K_b blocks from block `first`, and writes
// the K_b kept block ids in ascending order to out[0..K_b) (global memory or
// LDS).  Called by all 256 threads of the workgroup; ends after the write
// (the caller synchronises before reading `out` from LDS).
template <typename KE, int D, int GMAX, int TPW, bool PAGED>
__device__ __forceinline__ void search_pipe(const void *q, const void *K, const Shape &s, const Pages &pg,
                                            uint32_t b, uint32_t g, uint32_t i, int32_t Tp, int32_t first,
                                            int32_t M, int32_t *out) {
  constexpr int KS = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const int32_t Kb = s.Kb;
  __shared__ int32_t cand_a[2][2 * kPipeMaxKb], cand_e[2][2 * kPipeMaxKb];
  __shared__ int32_t srcs[2][2 * kPipeMaxKb];
  __shared__ uint64_t spec[2][4 * kPipeMaxKb];
  __shared__ uint64_t key[2 * kPipeMaxKb + kSpan];
  __shared__ int32_t flag[2];
  extern __shared__ int32_t ptab[];  // paged: the sequence's page numbers

  const uint16_t *qbase = reinterpret_cast<const uint16_t *>(q) + ((int64_t)(b * s.Hq + g * s.G) * Tq + i) * D;
  const KE *Kbase = reinterpret_cast<const KE *>(K);
  const int64_t kvoff = PAGED ? 0 : (int64_t)(b * Hkv + g) * s.T_cap * D;
  const int ps = pg.ps_shift;
  auto row_of = [&](int32_t t) -> int64_t {
    if constexpr (PAGED) return paged_row(ptab[t >> ps], g, Hkv, t, ps) * D;
    else return kvoff + (int64_t)t * D;
  };
  uint4 qa[KS];
  {
    const int h = lane & 15;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const uint4 r = *reinterpret_cast<const uint4 *>(qbase + (int64_t)min(h, s.G - 1) * Tq * D + 32 * ks + 8 * (lane >> 4));
      qa[ks] = h < s.G ? r : make_uint4(0, 0, 0, 0);
    }
  }

  const int n = 2 * Kb;
  // paged: page numbers to LDS, issued after the query loads so that both
  // are in flight together (read after the first barrier)
  if constexpr (PAGED) stage_pages(pg, b, Tp, ptab);
  initial_candidates(first, M, Kb, cand_a[0], cand_e[0]);
  for (int c = tid; c < n; c += 256) srcs[0][c] = c;
  if (tid < kSpan) key[n + tid] = 0;
  if (tid == 0) flag[0] = 1;  // M > K_b: the first round always runs
  if constexpr (PAGED) __syncthreads();  // the page numbers
  // keys of the first candidates (all waves), kept where round 0 looks them
  // up; the slots come from registers, so these gathers issue beside the
  // query loads instead of after a barrier
  score_children<KE, D, GMAX, TPW, true>(Kbase, row_of, qa, Tp, s.bk_shift, s.G, nullptr, nullptr, n, false,
                                     wave, 4, spec[1], first, M, Kb);
  __syncthreads();

  int cur = 0;
  for (int round = 0;; round++, cur ^= 1) {
    if (!flag[round & 1]) break;  // uniform: read after a barrier
    if (wave == 0) {
      // gather this round's keys, rank them, emit the kept chunks' halves
      if (lane == 0) flag[(round + 1) & 1] = 0;
      const uint64_t *prev = spec[cur ^ 1];
      for (int c = lane; c < n; c += 64) key[c] = prev[srcs[cur][c]];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int32_t *ca = cand_a[cur], *ce = cand_e[cur];
      int32_t *na = cand_a[cur ^ 1], *ne = cand_e[cur ^ 1], *nsrc = srcs[cur ^ 1];
      for (int c = lane; c < n; c += 64) {
        const uint64_t kc = key[c];
        int r = 0;
        for (int j0 = 0; j0 < n; j0 += kSpan) {
          uint64_t kk[kSpan];
#pragma unroll
          for (int u = 0; u < kSpan; u++) kk[u] = key[j0 + u];
#pragma unroll
          for (int u = 0; u < kSpan; u++) r += kk[u] > kc;
        }
        if (kc != 0 && r < Kb) {
          const int32_t lo = ca[c], hi = ce[c];
          const bool split = hi - lo >= 2;
          const int32_t m = lo + (hi - lo) / 2;
          na[2 * r] = lo;
          ne[2 * r] = split ? m : hi;
          na[2 * r + 1] = split ? m : -1;
          ne[2 * r + 1] = split ? hi : -1;
          nsrc[2 * r] = 2 * c;          // child slots of candidate c in this round's table
          nsrc[2 * r + 1] = 2 * c + 1;
          if (split) flag[(round + 1) & 1] = 1;
        }
      }
    } else {
      // speculative: score every child of every current candidate
      score_children<KE, D, GMAX, TPW>(Kbase, row_of, qa, Tp, s.bk_shift, s.G, cand_a[cur], cand_e[cur], 2 * n,
                                   true, wave - 1, 3, spec[cur]);
    }
    __syncthreads();
  }

  // the kept one-block chunks sit at the even slots of the current buffer
  write_ascending(cand_a[cur], Kb, out);
}

}  // namespace hipsa
