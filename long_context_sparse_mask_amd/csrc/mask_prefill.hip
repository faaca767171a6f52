// Hierarchical top-k key-block selection for query blocks of 64 rows
// (chunked prefill, bf16).
//
// Method: rebuttal page "A Training-free Sub-quadratic Cost Transformer Model
// Serving Framework With Hierarchically Pruned Attention", reviewer RsGC, Q2
// (split into k chunks, halve, score each half by its centre key, keep the
// global top-k, repeat to block size), with query blocks of b_q rows
// (reviewer NLBm, Q1).  A chunk's score is the max of q . k_centre over the
// query heads of the KV group and the rows of the block; a causal row votes
// only for centres at or before its own position.
//
// One workgroup (4 wave64s) per (b, kv head, query block).  Scoring a round
// is a dense [rows x d] . [d x candidates] product per query head, so it runs
// on v_mfma_f32_32x32x16_bf16: A = 32 query rows, B = 32 candidate centre
// rows read straight from K, one 32x32 fp32 tile per (row tile, candidate
// tile).  Each lane masks the rows that cannot vote for its candidate column
// and takes the column max in registers; one cross-half exchange finishes the
// 64-row max, and the per-head results meet in LDS through a 64-bit atomic
// max on the candidate's ranking key (score above complemented start).
// Selection and the final ascending write are the same as for decode.
#include "hipsa_internal.h"
#include "mask_select.h"

namespace hipsa {
namespace {

template <int D>
__global__ __launch_bounds__(256) void mask_prefill_kernel(MaskArgs a) {
  constexpr int KS = D / 16;  // k-steps of 16 over the head dim
  constexpr int BQ = 64;
  const Shape &s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const uint32_t prob = xcd_swizzle(blockIdx.x, gridDim.x);  // query blocks of one KV head share an L2
  const uint32_t nqb = (uint32_t)s.nqb, Hkv = (uint32_t)s.Hkv, Tq = (uint32_t)s.Tq;
  const uint32_t qb = prob % nqb, g = (prob / nqb) % Hkv, b = prob / (nqb * Hkv);
  const int32_t r0 = (int32_t)qb * BQ;
  const int32_t r1 = min(r0 + BQ, (int32_t)Tq);
  const int32_t pos0 = (int32_t)(s.T - s.Tq) + r0;  // position of the block's first row
  const int32_t Tp = s.causal ? pos0 + (r1 - r0) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t Kb = s.Kb;
  int32_t *out = a.indices + (int64_t)prob * Kb;

  if (Np <= Kb) {
    for (int j = tid; j < Kb; j += 256) out[j] = j < Np ? j : -1;
    if (tid == 0) a.nnz[prob] = Np;
    return;
  }

  __shared__ int32_t cand_a[2][2 * kMaxKb], cand_e[2][2 * kMaxKb];
  __shared__ uint64_t key[2][2 * kMaxKb + kSpan];
  __shared__ int32_t rk[2 * kMaxKb];
  __shared__ int32_t flag[2];

  const uint16_t *Qb = reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)(b * s.Hq + g * s.G) * Tq + r0) * D;
  const uint16_t *Kbase = reinterpret_cast<const uint16_t *>(a.K) + (int64_t)(b * Hkv + g) * s.T_cap * D;
  const int n = 2 * Kb, nct = (n + 31) / 32;
  const int half = lane >> 5, col = lane & 31;

  initial_candidates(Np, Kb, cand_a[0], cand_e[0]);
  for (int c = tid; c < n + kSpan; c += 256) key[0][c] = key[1][c] = 0;
  if (tid == 0) flag[0] = 1;
  __syncthreads();

  int cur = 0;
  for (int round = 0;; round++, cur ^= 1) {
    if (!flag[round & 1]) break;
    if (tid == 0) flag[(round + 1) & 1] = 0;
    const int32_t *ca = cand_a[cur], *ce = cand_e[cur];
    uint64_t *kcur = key[cur];
    for (int c = tid; c < n + kSpan; c += 256) key[cur ^ 1][c] = 0;  // read last round; free now

    // ---- 1. scoring: waves take the group's heads in turn
    for (int h = wave; h < s.G; h += 4) {
      // A operand: rows rt*32 + col of this head, dims 16*ks + 8*half .. +7
      uint4 qa[2][KS];
#pragma unroll
      for (int rt = 0; rt < 2; rt++) {
        const int row = min(rt * 32 + col, r1 - r0 - 1);  // clamp ragged rows (masked below)
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
          qa[rt][ks] = *reinterpret_cast<const uint4 *>(Qb + ((int64_t)h * Tq + row) * D + 16 * ks + 8 * half);
      }
      for (int ct = 0; ct < nct; ct++) {
        const int c = 32 * ct + col;
        const int cc = c < n ? c : 0;
        const int32_t lo_b = ca[cc], hi_b = ce[cc];
        const bool live = c < n && lo_b >= 0;
        const int32_t lo = lo_b << s.bk_shift, hi = min(hi_b << s.bk_shift, Tp);
        const int32_t t = live ? (lo + hi) >> 1 : 0;  // centre token (upper middle)
        uint4 kb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
          kb[ks] = *reinterpret_cast<const uint4 *>(Kbase + (int64_t)t * D + 16 * ks + 8 * half);
        float best = -INFINITY;
#pragma unroll
        for (int rt = 0; rt < 2; rt++) {
          f32x16_t acc = {};
#pragma unroll
          for (int ks = 0; ks < KS; ks++)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[rt][ks]), as_bf16x8(kb[ks]),
                                                          acc, 0, 0, 0);
          // acc[r]: row rt*32 + 8*(r/4) + 4*half + r%4, candidate column col
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int ri = rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool votes = r0 + ri < r1 && (!s.causal || pos0 + ri >= t);
            if (votes) best = fmaxf(best, acc[r]);
          }
        }
        best = fmaxf(best, __shfl_xor(best, 32, 64));
        if (half == 0 && live) atomicMax((unsigned long long *)&kcur[c], (unsigned long long)rank_key(best, lo_b));
      }
    }
    __syncthreads();

    // ---- 2. selection
    select_top(ca, ce, kcur, rk, n, Kb, cand_a[cur ^ 1], cand_e[cur ^ 1], &flag[(round + 1) & 1]);
    __syncthreads();
  }

  write_ascending(cand_a[cur], Kb, out);
  if (tid == 0) a.nnz[prob] = Kb;
}

}  // namespace

hipError_t launch_mask_prefill(const MaskArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)a.s.problems), block(256);
  if (a.s.d == 64) hipLaunchKernelGGL(mask_prefill_kernel<64>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(mask_prefill_kernel<128>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace hipsa
