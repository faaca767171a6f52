// Hierarchical top-k key-block selection for per-row problems (block_q == 1):
// decode, or any query row scored on its own.
//
// Method: rebuttal page "A Training-free Sub-quadratic Cost Transformer Model
// Serving Framework With Hierarchically Pruned Attention", reviewer RsGC, Q2
// (split into k chunks, halve, score by the centre key, keep the global top-k,
// repeat to block size); chunks stand for their centre tokens (summary page,
// Approach).
//
// One workgroup (256 threads, 4 wave64s) owns one problem (b, kv head g,
// query row i).  The candidate list (2*K_b slots; a one-block chunk fills one
// slot of its pair and leaves the other empty) is double-buffered in LDS, so
// a round is two phases separated by barriers:
//   1. scoring.  Centre rows of K are read straight into matrix-core
//      operands: for bf16 each wave scores 16 candidates per
//      v_mfma_f32_16x16x32_bf16 tile against the query heads of the group
//      (zero-padded to 16 rows), then takes the max over the valid head rows
//      of the accumulator; fp32 inputs use 16-byte VALU dot products with DPP
//      reductions instead.  Every load of a round is issued before any is used
//      (an empty slot reads row 0 and discards it), so a round pays one memory
//      latency;
//   2. selection.  A candidate's rank is the number of keys above its own
//      (key = score, then lower start, packed in one 64-bit integer); a
//      kept candidate writes its two halves (or itself and an empty slot)
//      straight into the other buffer, and a kept chunk wider than one block
//      sets the flag that runs the next round.
// Rounds are serially dependent (the next centres depend on this round's
// top-k), so the kernel is bound by one dependent memory round trip plus the
// round's LDS work per round, not by bandwidth.
#include <type_traits>

#include "hipsa_internal.h"
#include "mask_select.h"

namespace hipsa {
namespace {

template <typename E, int D, int GMAX, int UNROLL>
__global__ __launch_bounds__(256) void mask_decode_kernel(MaskArgs a) {
  constexpr bool kMfma = std::is_same<E, uint16_t>::value;
  constexpr int VEC = Vec<E>::N;
  constexpr int TPR = D / VEC;   // VALU path: lanes per key row
  constexpr int RPP = 256 / TPR; // VALU path: rows per pass
  constexpr int KS = D / 32;     // MFMA path: k-steps of 32 over the head dim
  const Shape &s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const uint32_t prob = blockIdx.x;
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int32_t Tp = s.causal ? (int32_t)(s.T - s.Tq + i + 1) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t Kb = s.Kb;
  int32_t *out = a.indices + (int64_t)prob * Kb;

  if (Np <= Kb) {  // the row sees few enough blocks to keep them all
    for (int j = tid; j < Kb; j += 256) out[j] = j < Np ? j : -1;
    if (tid == 0) a.nnz[prob] = Np;
    return;
  }

  __shared__ int32_t cand_a[2][2 * kMaxKb], cand_e[2][2 * kMaxKb];
  __shared__ uint64_t key[2 * kMaxKb + kSpan];
  __shared__ int32_t rk[2 * kMaxKb];
  __shared__ int32_t flag[2];

  const E *qbase = reinterpret_cast<const E *>(a.q) + ((int64_t)(b * s.Hq + g * s.G) * Tq + i) * D;
  const E *Kbase = reinterpret_cast<const E *>(a.K) + (int64_t)(b * Hkv + g) * s.T_cap * D;

  // Query operands, loaded once.  MFMA: lane l holds head l%16 (zero when
  // past the group), dims 32*ks + 8*(l/16) .. +7.  VALU: every head, dims
  // cs*VEC .. +VEC-1.
  uint4 qa[kMfma ? KS : 1];
  float qv[kMfma ? 1 : GMAX][VEC];
  if constexpr (kMfma) {
    const int h = lane & 15;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const uint4 r = Vec<E>::raw(qbase + (int64_t)min(h, s.G - 1) * Tq * D + 32 * ks + 8 * (lane >> 4));
      qa[ks] = h < s.G ? r : make_uint4(0, 0, 0, 0);
    }
  } else {
    const int cs = tid % TPR;
    uint4 r[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; h++)
      r[h] = Vec<E>::raw(qbase + (int64_t)min(h, s.G - 1) * Tq * D + cs * VEC);
#pragma unroll
    for (int h = 0; h < GMAX; h++) Vec<E>::widen(r[h], h < s.G, qv[h]);
  }

  const int n = 2 * Kb;
  initial_candidates(Np, Kb, cand_a[0], cand_e[0]);
  if (tid < kSpan) key[n + tid] = 0;  // padding read by the rank batches
  if (tid == 0) flag[0] = 1;          // N_p > K_b: the first round always runs
  __syncthreads();

  int cur = 0;
  for (int round = 0;; round++, cur ^= 1) {
    if (!flag[round & 1]) break;  // uniform: read after a barrier
    if (tid == 0) flag[(round + 1) & 1] = 0;  // its last readers are two barriers back
    const int32_t *ca = cand_a[cur], *ce = cand_e[cur];

    // ---- 1. scoring
    if constexpr (kMfma) {
      const int ntile = (n + 15) / 16;
      for (int t0 = wave; t0 < ntile; t0 += 4 * UNROLL) {
        uint4 kr[UNROLL][KS];
        bool live[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; u++) {
          const int c = 16 * (t0 + 4 * u) + (lane & 15);
          const int cc = c < n ? c : 0;
          const int32_t lo_b = ca[cc], hi_b = ce[cc];
          live[u] = c < n && lo_b >= 0;
          const int32_t lo = lo_b << s.bk_shift, hi = min(hi_b << s.bk_shift, Tp);
          const int32_t t = live[u] ? (lo + hi) >> 1 : 0;  // centre token (upper middle)
#pragma unroll
          for (int ks = 0; ks < KS; ks++)
            kr[u][ks] = Vec<E>::raw(Kbase + (int64_t)t * D + 32 * ks + 8 * (lane >> 4));
        }
#pragma unroll
        for (int u = 0; u < UNROLL; u++) {
          const int c = 16 * (t0 + 4 * u) + (lane & 15);
          f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ks++)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[ks]), as_bf16x8(kr[u][ks]),
                                                          acc, 0, 0, 0);
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
          raw[u] = Vec<E>::raw(Kbase + (int64_t)t * D + cs * VEC);
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
    __syncthreads();

    // ---- 2. selection: the K_b best write their halves into the other buffer
    select_top(ca, ce, key, rk, n, Kb, cand_a[cur ^ 1], cand_e[cur ^ 1], &flag[(round + 1) & 1]);
    __syncthreads();
  }

  // the kept one-block chunks sit at the even slots of the current buffer
  write_ascending(cand_a[cur], Kb, out);
  if (tid == 0) a.nnz[prob] = Kb;
}

template <typename E, int D, int GMAX>
void launch_g(const MaskArgs &a, hipStream_t st) {
  constexpr bool kMfma = std::is_same<E, uint16_t>::value;
  constexpr int RPP = 256 / (D / Vec<E>::N);
  const int n = 2 * a.s.Kb;
  // loads in flight per lane per round: candidate tiles per wave (MFMA) or
  // candidate rows per lane (VALU)
  const int per = kMfma ? ((n + 15) / 16 + 3) / 4 : (n + RPP - 1) / RPP;
  const dim3 grid((unsigned)a.s.problems), block(256);
  if (per <= 1) hipLaunchKernelGGL((mask_decode_kernel<E, D, GMAX, 1>), grid, block, 0, st, a);
  else if (per <= 2) hipLaunchKernelGGL((mask_decode_kernel<E, D, GMAX, 2>), grid, block, 0, st, a);
  else if (per <= 4) hipLaunchKernelGGL((mask_decode_kernel<E, D, GMAX, 4>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((mask_decode_kernel<E, D, GMAX, 8>), grid, block, 0, st, a);
}

template <typename E, int D>
hipError_t launch_d(const MaskArgs &a, hipStream_t st) {
  const int G = a.s.G;
  if (G <= 1) launch_g<E, D, 1>(a, st);
  else if (G <= 2) launch_g<E, D, 2>(a, st);
  else if (G <= 4) launch_g<E, D, 4>(a, st);
  else if (G <= 8) launch_g<E, D, 8>(a, st);
  else launch_g<E, D, 16>(a, st);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mask_decode(const MaskArgs &a, hipStream_t st) {
  if (a.s.dtype == HIPSA_BF16)
    return a.s.d == 64 ? launch_d<uint16_t, 64>(a, st) : launch_d<uint16_t, 128>(a, st);
  return a.s.d == 64 ? launch_d<float, 64>(a, st) : launch_d<float, 128>(a, st);
}

}  // namespace hipsa
