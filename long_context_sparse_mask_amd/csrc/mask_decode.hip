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
//   1. scoring.  Centre rows of K are gathered row by row (the lanes of a
//      quarter-wave read one row together) into per-wave LDS tiles and read
//      back as matrix-core operands: for a bf16 query each wave scores 16
//      candidates per
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

// With a bf16 query, `S` workgroups per problem (its splits, on one XCD by
// xcd_swizzle) run the same search, each prefetching its share of every
// round's next candidates into the XCD's L2 (search_row's SPREAD); split 0
// writes the list.  The grid holds problems * S workgroups.
template <typename E, typename KE, int D, int GMAX, int UNROLL, bool PAGED>
__global__ __launch_bounds__(256) void mask_decode_kernel(MaskArgs a, int S) {
  const Shape &s = a.s;
  const int tid = threadIdx.x;

  const uint32_t wgi = xcd_swizzle(blockIdx.x, gridDim.x);
  const uint32_t prob = wgi / (uint32_t)S, split = wgi % (uint32_t)S;
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
    if (split != 0) return;
    for (int j = tid; j < Kb; j += 256) out[j] = j < M ? first + j : -1;
    if (tid == 0) a.nnz[prob] = M;
    return;
  }

  if constexpr (std::is_same<E, uint16_t>::value) {
    __shared__ int32_t discard[kMaxKb];  // the list of splits other than 0
    search_row<E, KE, D, GMAX, UNROLL, PAGED, true>(a.q, a.K, s, a.pg, b, g, i, Tp, first, M,
                                                    split == 0 ? out : discard, (int)split, S);
  } else {
    search_row<E, KE, D, GMAX, UNROLL, PAGED>(a.q, a.K, s, a.pg, b, g, i, Tp, first, M, out);
  }
  if (tid == 0 && split == 0) a.nnz[prob] = Kb;
}

// dynamic LDS: the page numbers of a whole sequence when paged
size_t page_lds(const MaskArgs &a) { return a.pg.table ? (size_t)a.pg.seq_pages * sizeof(int32_t) : 0; }

template <typename E, typename KE, int D, int GMAX, bool PAGED>
void launch_g(const MaskArgs &a, hipStream_t st) {
  constexpr bool kMfma = std::is_same<E, uint16_t>::value;
  constexpr int RPP = 256 / (D / Vec<E>::N);
  const int n = 2 * a.s.Kb;
  // loads in flight per lane per round: candidate tiles per wave (MFMA) or
  // candidate rows per lane (VALU)
  const int per = kMfma ? search_tiles_per_wave(a.s.Kb) : (n + RPP - 1) / RPP;
  // splits per problem: up to 8 while the grid stays within one workgroup per
  // CU, for a bf16 query and at least 16 problems (with 8 problems, 32k and
  // 1M tokens, 8 splits measured slower: masks 7.84 -> 8.46 and 21.7 -> 22.4 us)
  int S = 1;
  if (kMfma && a.s.problems >= 16)
    while (S < 8 && a.s.problems * (2 * S) <= 256) S *= 2;
  const dim3 grid((unsigned)(a.s.problems * S)), block(256);
  const size_t lds = page_lds(a);
  if (per <= 1) hipLaunchKernelGGL((mask_decode_kernel<E, KE, D, GMAX, 1, PAGED>), grid, block, lds, st, a, S);
  else if (per <= 2) hipLaunchKernelGGL((mask_decode_kernel<E, KE, D, GMAX, 2, PAGED>), grid, block, lds, st, a, S);
  else if (per <= 4) hipLaunchKernelGGL((mask_decode_kernel<E, KE, D, GMAX, 4, PAGED>), grid, block, lds, st, a, S);
  else hipLaunchKernelGGL((mask_decode_kernel<E, KE, D, GMAX, 8, PAGED>), grid, block, lds, st, a, S);
}

// E: query element type; KE: key element type (E itself, or E5M2 codes
// under a bf16 query).
template <typename E, typename KE, int D, bool PAGED>
hipError_t launch_d(const MaskArgs &a, hipStream_t st) {
  const int G = a.s.G;
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
