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
// query row i) and runs every round.  Per round:
//   1. each kept chunk of >= 2 blocks is split into two candidate slots,
//      a one-block chunk fills one slot and leaves the other empty;
//   2. candidate centre rows of K are read with coalesced 16-byte loads, a
//      group of d/VEC consecutive lanes per row, all rows of the round in
//      flight at once; lanes hold their slice of every query head of the
//      group and reduce the G dot products with cross-lane adds, then take
//      the max over heads;
//   3. each candidate's rank is the number of keys above its own (key = score
//      then lower start, both packed in one 64-bit integer), and the K_b best
//      are written to the chunk list in rank order.
// The round count is fixed by the data; rounds are serially dependent (the
// next centres depend on this round's top-k), so this kernel is bound by the
// latency of one dependent HBM gather per round, not by bandwidth.
#include "hipsa_internal.h"

namespace hipsa {
namespace {

template <typename E, int D, int GMAX>
__global__ __launch_bounds__(256) void mask_decode_kernel(MaskArgs a) {
  constexpr int VEC = Vec<E>::N;
  constexpr int TPR = D / VEC;   // lanes per key row
  constexpr int RPP = 256 / TPR; // rows per pass over the workgroup
  constexpr int UNROLL = 8;      // rows in flight per lane
  const Shape &s = a.s;
  const int tid = threadIdx.x;
  const int rg = tid / TPR, cs = tid % TPR;

  const int64_t prob = blockIdx.x;
  const int64_t i = prob % s.Tq;
  const int64_t g = (prob / s.Tq) % s.Hkv;
  const int64_t b = prob / (s.Tq * s.Hkv);
  const int64_t Tp = s.causal ? s.T - s.Tq + i + 1 : s.T;
  const int32_t Np = (int32_t)((Tp + s.bk - 1) / s.bk);
  const int32_t Kb = s.Kb;
  int32_t *out = a.indices + prob * Kb;

  if (Np <= Kb) {  // the row sees few enough blocks to keep them all
    for (int j = tid; j < Kb; j += 256) out[j] = j < Np ? j : -1;
    if (tid == 0) a.nnz[prob] = Np;
    return;
  }

  __shared__ int32_t ca[kMaxKb], ce[kMaxKb];
  __shared__ int32_t cand_a[2 * kMaxKb], cand_e[2 * kMaxKb];
  __shared__ uint64_t key[2 * kMaxKb];

  // This lane's slice of every query head in the group.
  float qv[GMAX][VEC];
  const E *qbase = reinterpret_cast<const E *>(a.q) + ((b * s.Hq + g * s.G) * s.Tq + i) * D;
#pragma unroll
  for (int h = 0; h < GMAX; h++) {
    if (h < s.G) {
      Vec<E>::load(qbase + (int64_t)h * s.Tq * D + cs * VEC, qv[h]);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; e++) qv[h][e] = 0.f;
    }
  }
  const E *Kbase = reinterpret_cast<const E *>(a.K) + (b * s.Hkv + g) * s.T_cap * D;

  for (int c = tid; c < Kb; c += 256) {  // initial uniform partition
    ca[c] = (int32_t)((int64_t)c * Np / Kb);
    ce[c] = (int32_t)((int64_t)(c + 1) * Np / Kb);
  }
  __syncthreads();

  const int n = 2 * Kb;
  for (;;) {
    int wide = 0;
    for (int c = tid; c < Kb; c += 256) wide |= (ce[c] - ca[c] >= 2);
    if (!__syncthreads_or(wide)) break;

    for (int c = tid; c < Kb; c += 256) {  // halve every chunk
      const int32_t lo = ca[c], hi = ce[c];
      if (hi - lo >= 2) {
        const int32_t m = lo + (hi - lo) / 2;
        cand_a[2 * c] = lo; cand_e[2 * c] = m;
        cand_a[2 * c + 1] = m; cand_e[2 * c + 1] = hi;
      } else {
        cand_a[2 * c] = lo; cand_e[2 * c] = hi;
        cand_a[2 * c + 1] = -1; cand_e[2 * c + 1] = -1;
      }
    }
    __syncthreads();

    for (int base = 0; base < n; base += RPP * UNROLL) {  // score by centre keys
      float kv[UNROLL][VEC];
      bool live[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; u++) {
        const int c = base + u * RPP + rg;
        live[u] = c < n && cand_a[c] >= 0;
        if (live[u]) {
          const int64_t lo = (int64_t)cand_a[c] * s.bk;
          const int64_t hi = min((int64_t)cand_e[c] * s.bk, Tp);
          const int64_t t = (lo + hi) / 2;  // centre token (upper middle)
          Vec<E>::load(Kbase + t * D + cs * VEC, kv[u]);
        } else {
#pragma unroll
          for (int e = 0; e < VEC; e++) kv[u][e] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; u++) {
        const int c = base + u * RPP + rg;
        float best = -INFINITY;
#pragma unroll
        for (int h = 0; h < GMAX; h++) {
          float p = 0.f;
#pragma unroll
          for (int e = 0; e < VEC; e++) p = fmaf(qv[h][e], kv[u][e], p);
          p = group_sum<TPR>(p);
          if (h < s.G) best = fmaxf(best, p);
        }
        if (cs == 0 && c < n) key[c] = live[u] ? rank_key(best, cand_a[c]) : 0ull;
      }
    }
    __syncthreads();

    for (int c = tid; c < n; c += 256) {  // global top-K_b by rank counting
      const uint64_t kc = key[c];
      if (kc == 0) continue;
      int r = 0;
      for (int j = 0; j < n; j++) r += key[j] > kc;
      if (r < Kb) { ca[r] = cand_a[c]; ce[r] = cand_e[c]; }
    }
    __syncthreads();
  }

  for (int c = tid; c < Kb; c += 256) {  // ascending block ids
    const int32_t v = ca[c];
    int r = 0;
    for (int j = 0; j < Kb; j++) r += ca[j] < v;
    out[r] = v;
  }
  if (tid == 0) a.nnz[prob] = Kb;
}

template <typename E, int D>
hipError_t launch_d(const MaskArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)a.s.problems), block(256);
  const int G = a.s.G;
  if (G <= 1) hipLaunchKernelGGL((mask_decode_kernel<E, D, 1>), grid, block, 0, st, a);
  else if (G <= 2) hipLaunchKernelGGL((mask_decode_kernel<E, D, 2>), grid, block, 0, st, a);
  else if (G <= 4) hipLaunchKernelGGL((mask_decode_kernel<E, D, 4>), grid, block, 0, st, a);
  else if (G <= 8) hipLaunchKernelGGL((mask_decode_kernel<E, D, 8>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((mask_decode_kernel<E, D, 16>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mask_decode(const MaskArgs &a, hipStream_t st) {
  if (a.s.dtype == HIPSA_BF16)
    return a.s.d == 64 ? launch_d<uint16_t, 64>(a, st) : launch_d<uint16_t, 128>(a, st);
  return a.s.d == 64 ? launch_d<float, 64>(a, st) : launch_d<float, 128>(a, st);
}

}  // namespace hipsa
