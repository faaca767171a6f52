// One decode step in one launch: the hierarchical top-k search of a problem
// and its block-sparse attention, followed by the merge of the split partials.
//
// The pages report decode latency as masking plus sparse attention (rebuttal
// page "A Training-free Sub-quadratic Cost Transformer Model Serving Framework
// With Hierarchically Pruned Attention", reviewer KprR, W2), and the mask is
// consumed by the attention right away unless it is reused across steps
// (summary page, Limitations: the mask refresh interval).  Run as two
// launches, the attention kernel waits for the mask kernel to end and then
// reads the lists back from memory.  Here every split workgroup of a problem
// runs the problem's search itself (search_row), holds the kept blocks in
// LDS and attends its share of them (attend_split); no workgroup waits for
// another.  The search is latency-bound (serially dependent rounds of row
// gathers) and cheap, so running it once per split costs little time: the
// splits of a problem run on one XCD (xcd_swizzle), where they read the
// same centre rows through its L2, and after each round each split loads
// its share of the rows the next round may need, so that round finds them
// all in the L2 (search_row's SPREAD).  Split 0 also writes the lists, so a
// later step can reuse the mask through hip_sparse_attn.
//
// The last split workgroup of a problem to finish merges the splits'
// partials (no second launch).  Results are bit for bit those of
// hip_mask_estimate followed by hip_sparse_attn: the same search, the same
// split assignment of the same ascending list, the same merge arithmetic
// (merge_partials).
#include <cstdint>
#include <type_traits>

#include "decode_search.h"
#include "decode_split.h"
#include "hipsa_internal.h"
#include "mask_select.h"

namespace hipsa {
namespace {

// bf16 query, bf16 or fp8 (E5M2) K/V, K_b <= kStepMaxKb; UNROLL as the mask
// kernel takes it (search_tiles_per_wave).  PAGED: the search stages the
// sequence's page numbers in dynamic LDS, as the mask kernel does.
//
// The search's operands lead the argument list as scalars (q, K, the grid
// size and the shape fields it reads, 12 dwords; `packed` holds bk_shift in
// bits 0-3, causal in bit 4, G in bits 5-9, K_b in bits 10-17, `dense` the
// sink and window blocks in its halves): the dispatcher preloads them into
// scalar registers, so the query and round-0 loads issue without waiting for
// a kernel-argument read; the rest of `a` is read from memory when the
// attention needs it.
template <typename KE, int D, int GMAX, int UNROLL, int TOK, bool WIDE, bool PAGED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void decode_step_kernel(
    const void *q, const void *K, uint32_t nwg, int32_t splits, int32_t Tq_, int32_t Hkv_, int32_t T_,
    int32_t T_cap, uint32_t packed, uint32_t dense, StepArgs a) {
  Shape s = a.at.s;  // the fields the search reads, from the preloaded arguments
  s.Tq = Tq_; s.Hkv = Hkv_; s.T = T_; s.T_cap = T_cap;
  s.bk_shift = (int32_t)(packed & 15); s.bk = 1 << s.bk_shift; s.causal = (int32_t)((packed >> 4) & 1);
  s.G = (int32_t)((packed >> 5) & 31); s.Kb = (int32_t)((packed >> 10) & 255); s.Hq = (int64_t)s.G * Hkv_;
  s.sink_b = (int32_t)(dense & 0xffff); s.window_b = (int32_t)(dense >> 16);
  const int tid = threadIdx.x;
  const uint32_t S = (uint32_t)splits;
  const uint32_t wgi = xcd_swizzle(blockIdx.x, nwg);
  const uint32_t split = wgi % S, prob = wgi / S;
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int32_t Tp = s.causal ? (int32_t)(s.T - s.Tq + i + 1) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t Kb = s.Kb;
  const Dense dn(s, Np);  // the search covers the M blocks from `first` between the dense parts
  const int32_t first = dn.Sb, M = Np - dn.Sb - dn.Wb;

  __shared__ int32_t list[kStepMaxKb];
  __shared__ int32_t cnt;
  if (M <= Kb) {  // the row sees few enough blocks to keep them all
    for (int j = tid; j < Kb; j += 256) list[j] = j < M ? first + j : -1;
    if (tid == 0) cnt = M;
  } else {
    search_row<uint16_t, KE, D, GMAX, UNROLL, PAGED, true>(q, K, s, a.at.pg, b, g, i, Tp, first, M, list,
                                                          (int)split, (int)S);
    if (tid == 0) cnt = Kb;
  }
  __syncthreads();
  if (split == 0) {  // the mask, for later steps that reuse it
    int32_t *out = a.indices + (int64_t)prob * Kb;
    for (int j = tid; j < Kb; j += 256) out[j] = list[j];
    if (tid == 0) a.nnz[prob] = cnt;
  }
  attend_split<KE, D, GMAX, TOK, PAGED, WIDE, true>(a.at, prob, split, list, &cnt);
  if (S == 1) return;  // the only split wrote the output

  // Arrival: the last split workgroup of the problem to finish merges the S
  // partials.  The partials, the arrival counter and the merger's reads of
  // the partials are all agent-scope atomic accesses: gfx950 performs such
  // stores and loads at the device's coherence point (the stores write
  // through, the loads bypass non-coherent caches), so once every thread's
  // partial stores have completed (the explicit wait: a workgroup barrier
  // does not wait for stores) and the counter has been incremented, the
  // workgroup that sees S - 1 earlier arrivals reads every partial as
  // written.  No cache write-back or invalidation is needed.  (Agent-scope
  // release/acquire fences around the counter, which write back and
  // invalidate the L2, measured 3.8 us slower per 128k x 4 step.)
  __shared__ uint32_t before;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    before = __hip_atomic_fetch_add(a.arrived + prob, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (before != S - 1) return;
  if (tid == 0) __hip_atomic_store(a.arrived + prob, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint32_t G = (uint32_t)s.G;
  const int64_t sstride = (int64_t)G * (D + 2);
  auto load = [](const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // thread tid merges NX dimensions of head tid / TPH, so the m and l of a
  // head's partials are loaded once beside its o values: one memory round trip
  constexpr int NX = D * GMAX / 256 > 1 ? D * GMAX / 256 : 1;
  constexpr int TPH = D / NX;  // threads per head
  const uint32_t h = tid / TPH;
  if (h >= G) return;
  int xs[NX];
#pragma unroll
  for (int j = 0; j < NX; j++) xs[j] = tid % TPH + j * TPH;
  const float *ph = a.at.ws + ((int64_t)prob * S * G + h) * (D + 2);
  float v[NX];
  if (S <= 16) merge_partials_nx<16, NX>(ph, (int)S, sstride, xs, load, v);
  else merge_partials_nx<32, NX>(ph, (int)S, sstride, xs, load, v);
  uint16_t *out = reinterpret_cast<uint16_t *>(a.at.out) + ((int64_t)(b * s.Hq + g * G + h) * Tq + i) * D;
#pragma unroll
  for (int j = 0; j < NX; j++) store_elem(out + xs[j], v[j]);
}

constexpr size_t kLdsPerWorkgroup = 160 * 1024;

// Static LDS bytes of a kernel (SIZE_MAX when the query fails; the error is
// cleared, so that it is not reported by a later call).
size_t static_lds(const void *kernel) {
  hipFuncAttributes at;
  if (hipFuncGetAttributes(&at, kernel) == hipSuccess) return at.sharedSizeBytes;
  (void)hipGetLastError();
  return SIZE_MAX;
}

// Launches one instantiation; with a paged cache only if its static LDS and
// the sequence's page numbers fit a workgroup (false: nothing launched).
template <typename KE, int D, int GMAX, int UNROLL, int TOK, bool WIDE, bool PAGED>
bool launch_one(const StepArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)(a.at.s.problems * a.at.splits)), block(256);
  auto kernel = decode_step_kernel<KE, D, GMAX, UNROLL, TOK, WIDE, PAGED>;
  size_t lds = 0;
  if constexpr (PAGED) {
    static const size_t fixed = static_lds(reinterpret_cast<const void *>(kernel));
    lds = (size_t)a.at.pg.seq_pages * sizeof(int32_t);
    if (fixed == SIZE_MAX || fixed + lds > kLdsPerWorkgroup) return false;
  }
  const Shape &s = a.at.s;
  // packed fields: bk_shift <= 6, G <= 16, K_b <= kStepMaxKb, sink and window blocks <= kMaxDenseBlocks
  static_assert(kStepMaxKb <= 255 && kMaxGroup <= 31 && kMaxDenseBlocks <= 0xffff, "packed step arguments");
  const uint32_t packed = (uint32_t)s.bk_shift | (uint32_t)(s.causal != 0) << 4 | (uint32_t)s.G << 5 |
                          (uint32_t)s.Kb << 10;
  const uint32_t dense = (uint32_t)s.sink_b | (uint32_t)s.window_b << 16;
  hipLaunchKernelGGL(kernel, grid, block, lds, st, a.at.q, a.at.K, grid.x, a.at.splits, (int32_t)s.Tq,
                     (int32_t)s.Hkv, (int32_t)s.T, (int32_t)s.T_cap, packed, dense, a);
  return true;
}

template <typename KE, int D, int GMAX, int UNROLL, bool PAGED>
bool launch_tok(const StepArgs &a, hipStream_t st) {
  const bool wide = (int64_t)a.at.s.problems * a.at.splits >= kWideGrid;
  const int tok = attn_decode_tokens(a.at.s);
  constexpr int G8 = GMAX <= 8 ? GMAX : 8;
  if (GMAX <= 8 && tok == 256) return launch_one<KE, D, G8, UNROLL, 256, true, PAGED>(a, st);
  if (GMAX <= 8 && tok == 128)
    return wide ? launch_one<KE, D, G8, UNROLL, 128, true, PAGED>(a, st)
                : launch_one<KE, D, G8, UNROLL, 128, false, PAGED>(a, st);
  return wide ? launch_one<KE, D, GMAX, UNROLL, 64, true, PAGED>(a, st)
              : launch_one<KE, D, GMAX, UNROLL, 64, false, PAGED>(a, st);
}

template <typename KE, int D, int GMAX, bool PAGED>
bool launch_g(const StepArgs &a, hipStream_t st) {
  static_assert(((2 * kStepMaxKb + 15) / 16 + 3) / 4 <= 2, "UNROLL 1 or 2 covers K_b <= kStepMaxKb");
  if (search_tiles_per_wave(a.at.s.Kb) <= 1) return launch_tok<KE, D, GMAX, 1, PAGED>(a, st);
  return launch_tok<KE, D, GMAX, 2, PAGED>(a, st);
}

template <typename KE, int D, bool PAGED>
bool launch_d(const StepArgs &a, hipStream_t st) {
  const int G = a.at.s.G;
  if (G <= 1) return launch_g<KE, D, 1, PAGED>(a, st);
  if (G <= 2) return launch_g<KE, D, 2, PAGED>(a, st);
  if (G <= 4) return launch_g<KE, D, 4, PAGED>(a, st);
  if (G <= 8) return launch_g<KE, D, 8, PAGED>(a, st);
  return launch_g<KE, D, 16, PAGED>(a, st);
}

template <bool PAGED>
bool launch_layout(const StepArgs &a, hipStream_t st) {
  const Shape &s = a.at.s;
  if (s.dtype == HIPSA_BF16_E5M2)
    return s.d == 64 ? launch_d<uint8_t, 64, PAGED>(a, st) : launch_d<uint8_t, 128, PAGED>(a, st);
  return s.d == 64 ? launch_d<uint16_t, 64, PAGED>(a, st) : launch_d<uint16_t, 128, PAGED>(a, st);
}

}  // namespace

// The one-launch form runs a problem's search once per split workgroup.  It
// pays while the grid has at most one workgroup per CU and a problem few
// splits: measured against the two calls, it saves 1.1 us per 128k x 4 step
// (32 problems x 8 splits) and 1.6 us at 32k (8 problems x 16 splits), but
// cost 2.0 us at 32k over 32 splits (32 searches of the same rows and a
// 32-way merge in one workgroup) and 19.7 us with a 4096-token window
// (32 problems x 25 splits: about three searches per CU).
constexpr int64_t kMaxStepGrid = 256;
constexpr int32_t kMaxStepSplits = 16;

bool one_launch(const Shape &s, int32_t splits) {
  return s.dtype != HIPSA_F32 && s.Kb <= kStepMaxKb && splits <= kMaxStepSplits &&
         s.problems * splits <= kMaxStepGrid;
}

hipError_t launch_decode_step(const StepArgs &a, hipStream_t st) {
  const Shape &s = a.at.s;
  // The one-launch form serves a bf16 query with bf16 or fp8 keys, either
  // layout, and K_b <= kStepMaxKb (paged: if the page numbers fit in LDS
  // beside the kernel's own arrays); otherwise, or when its redundant
  // searches would cost more than the launch they save, the two calls'
  // kernels run in turn on the same lists.
  const bool fused = one_launch(s, a.at.splits) &&
                     (a.at.pg.table ? launch_layout<true>(a, st) : launch_layout<false>(a, st));
  if (!fused) {
    MaskArgs m{a.at.q, a.at.K, a.indices, a.nnz, s, a.at.pg};
    hipError_t e = launch_mask_decode(m, st);
    if (e != hipSuccess) return e;
    AttnArgs at = a.at;
    at.indices = a.indices;
    at.nnz = a.nnz;
    return launch_attn_decode(at, st);
  }
  return hipGetLastError();  // the last split workgroup of each problem merged the partials
}

size_t decode_step_workspace(const Shape &s) {
  if (s.problems == 0) return 0;
  const size_t partials = (attn_decode_workspace(s) + 255) / 256 * 256;
  return partials + (size_t)s.problems * sizeof(uint32_t);
}

}  // namespace hipsa
