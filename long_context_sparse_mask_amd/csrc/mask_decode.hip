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
//      operands: for a bf16 query each wave scores 16 candidates per
//      v_mfma_f32_16x16x32_bf16 tile against the query heads of the group
//      (zero-padded to 16 rows), then takes the max over the valid head rows
//      of the accumulator; fp32 inputs use 16-byte VALU dot products with DPP
//      reductions instead.  fp8 (E5M2) keys are loaded as 8-byte slices and
//      widened exactly to bf16 operands in registers.  Every load of a round
//      is issued before any is used (an empty slot reads row 0 and discards
//      it), so a round pays one memory latency;
//   2. selection.  A candidate's rank is the number of keys above its own
//      (key = score, then lower start, packed in one 64-bit integer), the
//      comparisons shared by all 256 threads; a kept candidate writes its
//      two halves (or itself and an empty slot) straight into the other
//      buffer, and a kept chunk wider than one block sets the flag that runs
//      the next round.
// Rounds are serially dependent (the next centres depend on this round's
// top-k), so the kernel is bound by one dependent memory round trip plus the
// round's LDS work per round, not by bandwidth.  With a paged KV cache the
// problem's page numbers are staged in LDS before the first round, so a
// centre row costs no extra memory trip.
#include <type_traits>

#include "decode_score.h"
#include "decode_search.h"
#include "hipsa_internal.h"
#include "mask_select.h"

namespace hipsa {
namespace {

template <typename E, typename KE, int D, int GMAX, int UNROLL, bool PAGED>
__global__ __launch_bounds__(256) void mask_decode_kernel(MaskArgs a) {
  const Shape &s = a.s;
  const int tid = threadIdx.x;

  const uint32_t prob = xcd_swizzle(blockIdx.x, gridDim.x);
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int32_t Tp = s.causal ? (int32_t)(s.T - s.Tq + i + 1) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t Kb = s.Kb;
  int32_t *out = a.indices + (int64_t)prob * Kb;

  // the search covers the M blocks from `first` between the dense sink and
  // window blocks (none of either by default)
  const Dense dn(s, Np);
  const int32_t first = dn.Sb, M = Np - dn.Sb - dn.Wb;
  if (M <= Kb) {  // the row sees few enough blocks to keep them all
    for (int j = tid; j < Kb; j += 256) out[j] = j < M ? first + j : -1;
    if (tid == 0) a.nnz[prob] = M;
    return;
  }

  __shared__ int32_t cand_a[2][2 * kMaxKb], cand_e[2][2 * kMaxKb];
  __shared__ uint64_t key[2 * kMaxKb + kSpan];
  __shared__ int32_t rk[2 * kMaxKb];
  __shared__ int32_t flag[2];
  constexpr bool kMfma = std::is_same<E, uint16_t>::value;
  __shared__ __align__(16) uint8_t stage[stage_bytes<E, KE, D>()];
  extern __shared__ int32_t ptab[];  // paged: the sequence's page numbers

  const E *qbase = reinterpret_cast<const E *>(a.q) + ((int64_t)(b * s.Hq + g * s.G) * Tq + i) * D;
  const KE *Kbase = reinterpret_cast<const KE *>(a.K);
  const int64_t kvoff = PAGED ? 0 : (int64_t)(b * Hkv + g) * s.T_cap * D;
  const int ps = a.pg.ps_shift;
  // element offset of the K row of position t
  auto row_of = [&](int32_t t) -> int64_t {
    if constexpr (PAGED) return paged_row(ptab[t >> ps], g, Hkv, t, ps) * D;
    else return kvoff + (int64_t)t * D;
  };

  QueryOps<E, D, GMAX> qo;
  qo.load(qbase, (int64_t)Tq * D, s.G);

  const int n = 2 * Kb;
  // paged: page numbers to LDS, issued after the query loads so that both
  // are in flight together (read after the first barrier)
  if constexpr (PAGED) stage_pages(a.pg, b, Tp, ptab);
  initial_candidates(first, M, Kb, cand_a[0], cand_e[0]);
  if (tid < kSpan) key[n + tid] = 0;  // padding read by the rank batches
  if (tid == 0) flag[0] = 1;          // M > K_b: the first round always runs
  __syncthreads();

  int cur = 0;
  for (int round = 0;; round++, cur ^= 1) {
    if (!flag[round & 1]) break;  // uniform: read after a barrier
    if (tid == 0) flag[(round + 1) & 1] = 0;  // its last readers are two barriers back
    const int32_t *ca = cand_a[cur], *ce = cand_e[cur];
    for (int c = tid; c < n; c += 256) rk[c] = 0;  // rank counts of this round

    // ---- 1. scoring
    score_slots<E, KE, D, GMAX, UNROLL>(qo, Kbase, row_of, ca, ce, n, Tp, s, key, kMfma ? stage : nullptr);
    __syncthreads();

    // ---- 2. selection: the K_b best write their halves into the other buffer
    select_top(ca, ce, key, rk, n, Kb, cand_a[cur ^ 1], cand_e[cur ^ 1], &flag[(round + 1) & 1]);
    __syncthreads();
  }

  // the kept one-block chunks sit at the even slots of the current buffer
  write_ascending(cand_a[cur], Kb, out);
  if (tid == 0) a.nnz[prob] = Kb;
}

// Pipelined kernel (decode_search.h) for bf16 queries and keys, contiguous layout, K_b <= 32.
template <typename KE, int D, int GMAX, int TPW, bool PAGED>
__global__ __launch_bounds__(256) void mask_decode_pipe(MaskArgs a) {
  const Shape &s = a.s;
  const int tid = threadIdx.x;

  const uint32_t prob = xcd_swizzle(blockIdx.x, gridDim.x);
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int32_t Tp = s.causal ? (int32_t)(s.T - s.Tq + i + 1) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t Kb = s.Kb;
  int32_t *out = a.indices + (int64_t)prob * Kb;

  const Dense dn(s, Np);  // the search covers the M blocks from `first` between the dense parts
  const int32_t first = dn.Sb, M = Np - dn.Sb - dn.Wb;
  if (M <= Kb) {
    for (int j = tid; j < Kb; j += 256) out[j] = j < M ? first + j : -1;
    if (tid == 0) a.nnz[prob] = M;
    return;
  }

  search_pipe<KE, D, GMAX, TPW, PAGED>(a.q, a.K, s, a.pg, b, g, i, Tp, first, M, out);
  if (tid == 0) a.nnz[prob] = Kb;
}

// dynamic LDS: the page numbers of a whole sequence when paged
size_t page_lds(const MaskArgs &a) { return a.pg.table ? (size_t)a.pg.seq_pages * sizeof(int32_t) : 0; }

template <typename KE, int D, int GMAX, bool PAGED>
void launch_pipe(const MaskArgs &a, hipStream_t st) {
  const int tiles = (4 * a.s.Kb + 15) / 16;  // child tiles per round, over 3 waves
  const int per = (tiles + 2) / 3;
  const dim3 grid((unsigned)a.s.problems), block(256);
  const size_t lds = page_lds(a);
  static_assert(((4 * kPipeMaxKb + 15) / 16 + 2) / 3 <= 4, "child tiles per wave exceed the largest TPW");
  if (per <= 1) hipLaunchKernelGGL((mask_decode_pipe<KE, D, GMAX, 1, PAGED>), grid, block, lds, st, a);
  else if (per <= 2) hipLaunchKernelGGL((mask_decode_pipe<KE, D, GMAX, 2, PAGED>), grid, block, lds, st, a);
  else hipLaunchKernelGGL((mask_decode_pipe<KE, D, GMAX, 4, PAGED>), grid, block, lds, st, a);
}

template <typename E, typename KE, int D, int GMAX, bool PAGED>
void launch_g(const MaskArgs &a, hipStream_t st) {
  constexpr bool kMfma = std::is_same<E, uint16_t>::value;
  constexpr int RPP = 256 / (D / Vec<E>::N);
  const int n = 2 * a.s.Kb;
  // loads in flight per lane per round: candidate tiles per wave (MFMA) or
  // candidate rows per lane (VALU)
  const int per = kMfma ? ((n + 15) / 16 + 3) / 4 : (n + RPP - 1) / RPP;
  const dim3 grid((unsigned)a.s.problems), block(256);
  const size_t lds = page_lds(a);
  if (per <= 1) hipLaunchKernelGGL((mask_decode_kernel<E, KE, D, GMAX, 1, PAGED>), grid, block, lds, st, a);
  else if (per <= 2) hipLaunchKernelGGL((mask_decode_kernel<E, KE, D, GMAX, 2, PAGED>), grid, block, lds, st, a);
  else if (per <= 4) hipLaunchKernelGGL((mask_decode_kernel<E, KE, D, GMAX, 4, PAGED>), grid, block, lds, st, a);
  else hipLaunchKernelGGL((mask_decode_kernel<E, KE, D, GMAX, 8, PAGED>), grid, block, lds, st, a);
}

// E: query element type; KE: key element type (E itself, or E5M2 codes
// under a bf16 query).
template <typename E, typename KE, int D, bool PAGED>
hipError_t launch_d(const MaskArgs &a, hipStream_t st) {
  const int G = a.s.G;
  // The pipelined kernel for bf16 keys in the contiguous layout only: with
  // fp8 keys (half the bytes per row) or a paged cache the plain kernel
  // measured faster per step at K_b = 32.
  if constexpr (std::is_same<E, uint16_t>::value && std::is_same<KE, uint16_t>::value && !PAGED) {
    if (a.s.Kb <= kPipeMaxKb) {
      if (G <= 1) launch_pipe<KE, D, 1, PAGED>(a, st);
      else if (G <= 2) launch_pipe<KE, D, 2, PAGED>(a, st);
      else if (G <= 4) launch_pipe<KE, D, 4, PAGED>(a, st);
      else if (G <= 8) launch_pipe<KE, D, 8, PAGED>(a, st);
      else launch_pipe<KE, D, 16, PAGED>(a, st);
      return hipGetLastError();
    }
  }
  if (G <= 1) launch_g<E, KE, D, 1, PAGED>(a, st);
  else if (G <= 2) launch_g<E, KE, D, 2, PAGED>(a, st);
  else if (G <= 4) launch_g<E, KE, D, 4, PAGED>(a, st);
  else if (G <= 8) launch_g<E, KE, D, 8, PAGED>(a, st);
  else launch_g<E, KE, D, 16, PAGED>(a, st);
  return hipGetLastError();
}

template <bool PAGED>
hipError_t launch_layout(const MaskArgs &a, hipStream_t st) {
  const bool d64 = a.s.d == 64;
  if (a.s.dtype == HIPSA_BF16)
    return d64 ? launch_d<uint16_t, uint16_t, 64, PAGED>(a, st) : launch_d<uint16_t, uint16_t, 128, PAGED>(a, st);
  if (a.s.dtype == HIPSA_BF16_E5M2)
    return d64 ? launch_d<uint16_t, uint8_t, 64, PAGED>(a, st) : launch_d<uint16_t, uint8_t, 128, PAGED>(a, st);
  return d64 ? launch_d<float, float, 64, PAGED>(a, st) : launch_d<float, float, 128, PAGED>(a, st);
}

}  // namespace

hipError_t launch_mask_decode(const MaskArgs &a, hipStream_t st) {
  return a.pg.table ? launch_layout<true>(a, st) : launch_layout<false>(a, st);
}

}  // namespace hipsa
