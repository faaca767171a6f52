// Hierarchical top-k key-block selection for query blocks of 64 rows
// (chunked prefill: bf16 queries, bf16 or fp8 E5M2 keys).
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
// Selection and the final ascending write are the same as for decode.  fp8
// centre rows are loaded as 8-byte slices and widened exactly to bf16 on
// their way into LDS.  With a paged KV cache the sequence's page numbers are
// staged in LDS before the first round.
#include "hipsa_internal.h"
#include "mask_select.h"

namespace hipsa {
namespace {

// ONEHEAD: the group has at most 4 query heads, so each wave owns one head
// for the whole search and keeps its query operands in registers.
template <typename KE, int D, bool ONEHEAD, bool PAGED>
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

  const Dense dn(s, Np);  // the search covers the M blocks from `first` between the dense parts
  const int32_t first = dn.Sb, M = Np - dn.Sb - dn.Wb;
  if (M <= Kb) {
    for (int j = tid; j < Kb; j += 256) out[j] = j < M ? first + j : -1;
    if (tid == 0) a.nnz[prob] = M;
    return;
  }

  __shared__ int32_t cand_a[2][2 * kMaxKb], cand_e[2][2 * kMaxKb];
  __shared__ uint64_t key[2][2 * kMaxKb + kSpan];
  __shared__ int32_t rk[2 * kMaxKb];
  __shared__ int32_t pos[kMaxKb];  // places of the kept ids (write_ascending)
  __shared__ int32_t flag[2];

  const uint16_t *Qb = reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)(b * s.Hq + g * s.G) * Tq + r0) * D;
  extern __shared__ int32_t ptab[];  // paged: the sequence's page numbers
  const KE *Kbase = reinterpret_cast<const KE *>(a.K);
  const int64_t kvoff = PAGED ? 0 : (int64_t)(b * Hkv + g) * s.T_cap * D;
  const int ps = a.pg.ps_shift;
  auto row_of = [&](int32_t t) -> int64_t {
    if constexpr (PAGED) return paged_row(ptab[t >> ps], g, Hkv, t, ps) * D;
    else return kvoff + (int64_t)t * D;
  };
  const int n = 2 * Kb, nct = (n + 31) / 32;
  // staging of 64 candidates' centre rows: SLR lanes per row, SRP rows per
  // pass, SP passes; rows padded to CRS elements (a column read of the 32
  // rows of a tile then falls in distinct banks per 16 lanes)
  constexpr int SLR = D / 8, SRP = 256 / SLR, SP = 64 / SRP, CRS = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t cst[64 * CRS];
  typename Kv8<KE>::raw_t srow[SP];
  const int half = lane >> 5, col = lane & 31;

  // A operand: rows rt*32 + col of head h, dims 16*ks + 8*half .. +7
  uint4 qa[2][KS];
#define HIPSA_LOAD_QUERIES(H)                                                                    \
  do {                                                                                           \
    _Pragma("unroll") for (int rt = 0; rt < 2; rt++) {                                           \
      const int row_ = min(rt * 32 + col, r1 - r0 - 1); /* ragged rows are masked below */       \
      _Pragma("unroll") for (int ks = 0; ks < KS; ks++)                                          \
        qa[rt][ks] = *reinterpret_cast<const uint4 *>(Qb + ((int64_t)(H) * Tq + row_) * D + 16 * ks + 8 * half); \
    }                                                                                            \
  } while (0)
  auto load_queries = [&](int h) { HIPSA_LOAD_QUERIES(h); };
  if (ONEHEAD) HIPSA_LOAD_QUERIES(min(wave, s.G - 1));

  // paged: page numbers to LDS, issued after the query loads so that both
  // are in flight together (read after the first barrier)
  if constexpr (PAGED) stage_pages(a.pg, b, Tp, ptab);
  initial_candidates(first, M, Kb, cand_a[0], cand_e[0]);
  for (int c = tid; c < n + kSpan; c += 256) key[0][c] = key[1][c] = 0;
  for (int c = tid; c < Kb; c += 256) pos[c] = 0;
  if (tid == 0) flag[0] = 1;
  __syncthreads();

  int cur = 0;
  for (int round = 0;; round++, cur ^= 1) {
    if (!flag[round & 1]) break;
    if (tid == 0) flag[(round + 1) & 1] = 0;
    const int32_t *ca = cand_a[cur], *ce = cand_e[cur];
    uint64_t *kcur = key[cur];
    for (int c = tid; c < n + kSpan; c += 256) key[cur ^ 1][c] = 0;  // read last round; free now
    for (int c = tid; c < n; c += 256) rk[c] = 0;                     // rank counts of this round

    // ---- 1. scoring, 64 candidates at a time: the workgroup loads their
    // centre rows once (whole rows, D/8 lanes each) into LDS, then every wave
    // scores them for its heads with B operands read from LDS
    for (int ct0 = 0; ct0 < nct; ct0 += 2) {
      if (ct0 > 0) __syncthreads();  // previous candidates' rows fully read
#pragma unroll
      for (int u = 0; u < SP; u++) {
        const int rrow = u * SRP + tid / SLR;  // candidate 32*ct0 + rrow
        const int c = 32 * ct0 + rrow;
        const int cc = c < n ? c : 0;
        const int32_t lo_b = ca[cc], hi_b = ce[cc];
        const bool live = c < n && lo_b >= 0;
        const int32_t lo = lo_b << s.bk_shift, hi = min(hi_b << s.bk_shift, Tp);
        const int32_t t = live ? (lo + hi) >> 1 : 0;  // centre token (upper middle)
        srow[u] = Kv8<KE>::raw(Kbase + row_of(t) + 8 * (tid % SLR));
      }
#pragma unroll
      for (int u = 0; u < SP; u++)
        *reinterpret_cast<uint4 *>(&cst[(u * SRP + tid / SLR) * CRS + 8 * (tid % SLR)]) = Kv8<KE>::bf16(srow[u]);
      __syncthreads();
      for (int h = wave; h < s.G; h += 4) {
        if (!ONEHEAD) load_queries(h);
#pragma unroll
        for (int u = 0; u < 2; u++) {
          if (ct0 + u >= nct) break;  // uniform
          const int c = 32 * (ct0 + u) + col;
          const int cc = c < n ? c : 0;
          const int32_t lo_b = ca[cc], hi_b = ce[cc];
          const bool live = c < n && lo_b >= 0;
          const int32_t lo = lo_b << s.bk_shift, hi = min(hi_b << s.bk_shift, Tp);
          const int32_t t = live ? (lo + hi) >> 1 : 0;
          // the tile's B operands are read from LDS together (one latency), and
          // the two row tiles are independent accumulation chains, interleaved
          uint4 kb[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ks++)
            kb[ks] = *reinterpret_cast<const uint4 *>(&cst[(32 * u + col) * CRS + 16 * ks + 8 * half]);
          f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
          for (int ks = 0; ks < KS; ks++)
#pragma unroll
            for (int rt = 0; rt < 2; rt++)
              acc[rt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa[rt][ks]), as_bf16x8(kb[ks]), acc[rt], 0, 0, 0);
          // acc[rt][r]: row rt*32 + 8*(r/4) + 4*half + r%4, candidate column col.
          // When every lane's centre is at or before the block's first row and
          // the block is full, every row votes (the common case: only chunks
          // near the diagonal need the per-row test).
          float best = -INFINITY;
          const bool all_vote = r1 - r0 == BQ && (!s.causal || t <= pos0);
          if (__builtin_amdgcn_ballot_w64(!all_vote) == 0) {  // uniform
            float mx[4];
#pragma unroll
            for (int j = 0; j < 4; j++)
              mx[j] = fmaxf(fmaxf(acc[j >> 1][8 * (j & 1)], acc[j >> 1][8 * (j & 1) + 1]),
                            fmaxf(acc[j >> 1][8 * (j & 1) + 2], acc[j >> 1][8 * (j & 1) + 3]));
#pragma unroll
            for (int r = 4; r < 8; r++)
#pragma unroll
              for (int j = 0; j < 4; j++) mx[j] = fmaxf(mx[j], acc[j >> 1][8 * (j & 1) + r]);
            best = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
          } else {
#pragma unroll
            for (int rt = 0; rt < 2; rt++) {
#pragma unroll
              for (int r = 0; r < 16; r++) {
                const int ri = rt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                const bool votes = r0 + ri < r1 && (!s.causal || pos0 + ri >= t);
                best = votes ? fmaxf(best, acc[rt][r]) : best;
              }
            }
          }
          best = xor32_max(best);
          if (half == 0 && live) atomicMax((unsigned long long *)&kcur[c], (unsigned long long)rank_key(best, lo_b));
        }
      }
    }
    __syncthreads();

    // ---- 2. selection
    select_top(ca, ce, kcur, rk, n, Kb, cand_a[cur ^ 1], cand_e[cur ^ 1], &flag[(round + 1) & 1]);
    __syncthreads();
  }

#undef HIPSA_LOAD_QUERIES
  write_ascending(cand_a[cur], Kb, pos, out);
  if (tid == 0) a.nnz[prob] = Kb;
}

template <typename KE, bool PAGED>
void launch_k(const MaskArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)a.s.problems), block(256);
  const size_t lds = PAGED ? (size_t)a.pg.seq_pages * sizeof(int32_t) : 0;
  const bool one = a.s.G <= 4;
  if (a.s.d == 64) {
    if (one) hipLaunchKernelGGL((mask_prefill_kernel<KE, 64, true, PAGED>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((mask_prefill_kernel<KE, 64, false, PAGED>), grid, block, lds, st, a);
  } else {
    if (one) hipLaunchKernelGGL((mask_prefill_kernel<KE, 128, true, PAGED>), grid, block, lds, st, a);
    else hipLaunchKernelGGL((mask_prefill_kernel<KE, 128, false, PAGED>), grid, block, lds, st, a);
  }
}

template <bool PAGED>
void launch_layout(const MaskArgs &a, hipStream_t st) {
  if (a.s.dtype == HIPSA_BF16_E5M2) launch_k<uint8_t, PAGED>(a, st);
  else launch_k<uint16_t, PAGED>(a, st);
}

}  // namespace

hipError_t launch_mask_prefill(const MaskArgs &a, hipStream_t st) {
  if (a.pg.table) launch_layout<true>(a, st);
  else launch_layout<false>(a, st);
  return hipGetLastError();
}

}  // namespace hipsa
