// Multi-stage hierarchical top-k key-block selection for per-row problems
// (block_q == 1), configured by a stage list as InfiniteHiP is served.
//
// Method.  The SGLang pull request "Support Efficient Sparse HiP Attention
// (InfiniteHiP) ..." configures each layer with a list of stages, each with a
// chunk size and a number of keys kept (stage_chunk_size, stage_k, the first
// k null); the InfiniteHiP pages describe the pruning as modular and
// hierarchical, and the rebuttal page "A Training-free Sub-quadratic Cost
// Transformer Model Serving Framework With Hierarchically Pruned Attention"
// (reviewer KprR, W3; reviewer T2wK, Q1) says the number of chunks kept and
// how each chunk is broken down are chosen per iteration.  Reading, in key
// blocks:
//   - stage 0 cuts the searched blocks into consecutive chunks of chunk[0]
//     blocks (the last one takes what is left) and keeps every one;
//   - each later stage runs rounds of the one-stage iteration (same page,
//     reviewer RsGC, Q2): halve every kept chunk wider than the stage's chunk
//     size (narrower ones pass through and are scored again), score each
//     candidate by its centre key, keep the stage's number of best candidates
//     (score descending, then lower start); at least one round, and more while
//     a kept chunk is wider than the chunk size;
//   - the last stage's chunk size is one block: its kept chunks are the list
//     (ascending, nnz = their count).
//
// One workgroup (256 threads, 4 wave64s) owns one problem (b, kv head g,
// query row i).  LDS holds
//   A    the kept chunks (start, end), compact;
//   B    two slots per kept chunk: its halves, or the chunk and an empty slot;
//   key  one 64-bit ranking key per slot of B (score, then lower start; 0 for
//        an empty slot).
// A round builds B from A, scores B (score_slots: MFMA or VALU dot products of
// the query heads with the centre keys), finds the kept set and compacts it
// into A.  A first round can hold thousands of candidates (stage 0 chunks
// of a long context), so the kept set is found by a radix select on the keys
// (linear in the candidates) instead of the one-stage kernel's rank by count
// (quadratic): 8-bit digits from the top, one LDS histogram per digit, until
// the digit prefix of the keep-th largest key holds exactly the keys still
// needed.  Keys of live candidates are distinct (their starts are), so the
// kept set is exactly the candidates whose key is at least that threshold,
// whatever the slot order.
#include <algorithm>
#include <type_traits>

#include "decode_score.h"
#include "hipsa_internal.h"

namespace hipsa {
namespace {

// Rounds of one problem: each round of a stage halves its widest chunks or
// is the stage's first, so a problem runs at most nst + 31 * (nst - 1) rounds
// (chunks are at most 2^31 blocks wide); the bound only guards the loop.
constexpr int kMaxRounds = 512;
// Keys per thread in the selection: slot tid + 256 u holds key u of thread tid.
constexpr int kKpt = 2 * kMaxStageChunks / 256;

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROWS, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes of a wave: DPP shifts within rows of
// 16 lanes, then broadcasts of lanes 15 and 31 into the later rows.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v) {
  v += dpp_u32<0x111, 0xf>(v);  // row_shr:1
  v += dpp_u32<0x112, 0xf>(v);  // row_shr:2
  v += dpp_u32<0x114, 0xf>(v);  // row_shr:4
  v += dpp_u32<0x118, 0xf>(v);  // row_shr:8
  v += dpp_u32<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_u32<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

// Threshold of the `keep` largest non-zero keys of a round: the value thr
// such that exactly min(keep, live) keys are >= thr (1 when at most `keep`
// keys are live).  kr[u] is the key of slot tid + 256 u for u < nu (0 for an
// empty slot or past the round's slots); non-zero keys are distinct.  One
// pass per 8-bit digit from the top: an LDS histogram of the digit over the
// keys that share the digits found so far, then every wave finds the digit
// of the keep-th largest key from the histogram by itself, so a pass has one
// barrier.  The passes of a kernel use three histograms in turn (pass p
// uses hist + 256 (p % 3)); each pass clears the next one, whose last readers
// were two passes back.  hist + 256 (pass % 3) must be zero on entry.
// Called by all 256 threads.
__device__ uint64_t radix_threshold(const uint64_t (&kr)[kKpt], int nu, uint32_t keep,
                                    uint32_t *hist, int &pass) {
  const int lane = threadIdx.x & 63;
  uint64_t prefix = 0;
  uint32_t need = keep;
  for (int shift = 56; shift >= 0; shift -= 8) {
    uint32_t *h = hist + 256 * (pass % 3);
    hist[256 * ((pass + 1) % 3) + threadIdx.x] = 0;
    pass++;
    // keys that share the digits above `shift` with the prefix
    const uint64_t hm = shift == 56 ? 0ull : ~0ull << (shift + 8);
#pragma unroll
    for (int u = 0; u < kKpt; u++) {
      if (u < nu) {  // uniform
        const uint64_t k = kr[u];
        const bool in = k != 0 && ((k ^ prefix) & hm) == 0;
        const uint32_t d = (uint32_t)(k >> shift) & 255u;
        if (in) atomicAdd(&h[d], 1u);
      }
    }
    __syncthreads();
    // lane l holds digits 255-4l .. 252-4l, the highest first
    uint32_t cnt[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      cnt[j] = h[255 - 4 * lane - j];
      sum += cnt[j];
    }
    const uint32_t incl = wave_prefix_sum(sum);
    if (__builtin_amdgcn_readlane(incl, 63) <= need)
      return prefix ? prefix : 1ull;  // every key sharing the prefix is kept (at most `keep` live)
    uint32_t above = incl - sum;  // keys with a higher digit
    int hit = -1;
    uint32_t rest = 0, hc = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (above < need && need <= above + cnt[j]) {
        hit = 255 - 4 * lane - j;
        rest = need - above;
        hc = cnt[j];
      }
      above += cnt[j];
    }
    const int hl = __builtin_ctzll(__ballot(hit >= 0));  // the one lane holding the digit
    prefix |= (uint64_t)__builtin_amdgcn_readlane(hit, hl) << shift;
    need = __builtin_amdgcn_readlane(rest, hl);
    if (__builtin_amdgcn_readlane(hc, hl) == need) break;  // the digit's keys are exactly those needed
  }
  return prefix;
}

// Copies the slots (bs, be) whose key is >= thr (kr as in radix_threshold) to
// (as, ae), compact, and returns their count.  Each wave counts its kept
// slots, then writes them from its offset.  Sets *wide when a kept chunk is
// wider than tb blocks.  Called by all 256 threads; one barrier.
__device__ int compact_kept(const uint64_t (&kr)[kKpt], int nu, uint64_t thr, const int32_t *bs,
                            const int32_t *be, int32_t tb, int32_t *as, int32_t *ae,
                            int32_t *wcnt, int32_t *wide) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < kKpt; u++)
    if (u < nu) cnt += __popcll(__ballot(kr[u] >= thr));
  if (lane == 0) wcnt[wave] = cnt;
  __syncthreads();
  int off = 0;
  for (int v = 0; v < wave; v++) off += wcnt[v];
  const int total = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
  bool w = false;
#pragma unroll
  for (int u = 0; u < kKpt; u++) {
    if (u < nu) {
      const bool kept = kr[u] >= thr;
      const uint64_t m = __ballot(kept);
      if (kept) {
        const int c = threadIdx.x + 256 * u, pos = off + __popcll(m & ((1ull << lane) - 1));
        const int32_t lo = bs[c], hi = be[c];
        as[pos] = lo;
        ae[pos] = hi;
        w |= hi - lo > tb;
      }
      off += __popcll(m);
    }
  }
  if (__ballot(w) && lane == 0) *wide = 1;
  return total;
}

template <typename E, typename KE, int D, int GMAX, int UNROLL, bool PAGED>
__global__ __launch_bounds__(256) void mask_stages_kernel(StageArgs a) {
  const Shape &s = a.m.s;
  const int tid = threadIdx.x;

  const uint32_t S = (uint32_t)a.splits;
  const uint32_t wgi = xcd_swizzle(blockIdx.x, gridDim.x);
  const uint32_t prob = wgi / S, split = wgi % S;
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int32_t Tp = s.causal ? (int32_t)(s.T - s.Tq + i + 1) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t Kb = s.Kb;
  int32_t *out = a.m.indices + (int64_t)prob * Kb;

  // the search covers the M blocks from `first` between the dense parts
  const Dense dn(s, Np);
  const int32_t first = dn.Sb, M = Np - dn.Sb - dn.Wb;
  if (M <= Kb) {  // the row sees few enough blocks to keep them all
    if (split != 0) return;
    for (int j = tid; j < Kb; j += 256) out[j] = j < M ? first + j : -1;
    if (tid == 0) a.m.nnz[prob] = M;
    return;
  }

  extern __shared__ __align__(16) uint64_t lds[];
  const int cap = a.cap;
  uint64_t *key = lds;                                         // [2 cap]
  int32_t *bs = reinterpret_cast<int32_t *>(key + 2 * cap);    // [2 cap]
  int32_t *be = bs + 2 * cap;                                  // [2 cap]
  int32_t *as = be + 2 * cap, *ae = as + cap;                  // [cap] each
  int32_t *ptab = ae + cap;                                    // paged: the sequence's pages
  // row-gather tiles (when the launch has room for them)
  uint8_t *stg = a.stage_off >= 0 ? reinterpret_cast<uint8_t *>(lds) + a.stage_off : nullptr;
  __shared__ uint32_t hist[3 * 256];
  __shared__ int32_t wcnt[4];
  __shared__ int32_t flag[2];  // by round parity: a kept chunk is wider than the stage's size
  __shared__ int32_t pos[128];  // places of the final list's ids (K_b <= 128)

  const E *qbase = reinterpret_cast<const E *>(a.m.q) + ((int64_t)(b * s.Hq + g * s.G) * Tq + i) * D;
  const KE *Kbase = reinterpret_cast<const KE *>(a.m.K);
  const int64_t kvoff = PAGED ? 0 : (int64_t)(b * Hkv + g) * s.T_cap * D;
  const int ps = a.m.pg.ps_shift;
  // element offset of the K row of position t
  auto row_of = [&](int32_t t) -> int64_t {
    if constexpr (PAGED) return paged_row(ptab[t >> ps], g, Hkv, t, ps) * D;
    else return kvoff + (int64_t)t * D;
  };

  QueryOps<E, D, GMAX> qo;
  qo.load(qbase, (int64_t)Tq * D, s.G);
  if constexpr (PAGED) stage_pages(a.m.pg, b, Tp, ptab);

  // stage 0: consecutive chunks of chunk[0] blocks, the last one takes the rest
  const int32_t c0 = a.chunk[0], tb1 = a.chunk[1];
  int nk = (M + c0 - 1) / c0;
  // slot c of stage 1's first round: a half of stage-0 chunk c / 2, or the
  // chunk and an empty slot when it is no wider than stage 1's chunk size
  auto first_slot = [&](int c, int32_t *lo, int32_t *hi) {
    const int32_t a0 = first + (c >> 1) * c0, e0 = min(a0 + c0, first + M);
    const bool halve = e0 - a0 > tb1;
    const int32_t m = a0 + (e0 - a0) / 2;
    *lo = (c & 1) ? (halve ? m : -1) : a0;
    *hi = (c & 1) ? (halve ? e0 : -1) : (halve ? m : e0);
  };
  bool scored = false;  // the first round's keys are already in `key` (split search)
  if (S > 1) {
    // this workgroup's share of the first round: slots [c_lo, c_lo + cnt)
    const int n1 = 2 * nk;
    const int per = ((n1 + (int)S - 1) / (int)S + 15) / 16 * 16;
    const int c_lo = min((int)split * per, n1), cnt = min(c_lo + per, n1) - c_lo;
    for (int c = tid; c < cnt; c += 256) first_slot(c_lo + c, &bs[c], &be[c]);
    __syncthreads();
    score_slots<E, KE, D, GMAX, UNROLL, true>(qo, Kbase, row_of, bs, be, cnt, Tp, s, key, stg);
    __syncthreads();
    uint64_t *gk = a.keys + (int64_t)prob * a.n1max;
    for (int c = tid; c < cnt; c += 256)
      __hip_atomic_store(gk + c_lo + c, key[c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Arrival, as in the decode step's merge: the keys are agent-scope atomic
    // stores (written through to the device's coherence point); once every
    // thread's stores have completed (the explicit wait: a barrier does not
    // wait for stores) the counter is incremented, and the workgroup that
    // sees S - 1 earlier arrivals reads every key with agent-scope loads.
    __shared__ uint32_t before;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      before = __hip_atomic_fetch_add(a.arrived + prob, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (before != S - 1) return;
    if (tid == 0) __hip_atomic_store(a.arrived + prob, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int c = tid; c < n1; c += 256) {
      key[c] = __hip_atomic_load(gk + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      first_slot(c, &bs[c], &be[c]);
    }
    scored = true;
  }
  for (int j = tid; j < nk; j += 256) {
    as[j] = first + j * c0;
    ae[j] = min(first + (j + 1) * c0, first + M);
  }
  hist[tid] = hist[256 + tid] = hist[512 + tid] = 0;
  if (tid < 128) pos[tid] = 0;
  __syncthreads();

  int stage = 1, r = 0, pass = 0;
  bool fresh = true;  // the stage has run no round yet
  for (int guard = 0; guard < kMaxRounds; guard++, r++) {
    // the stage is done when no chunk kept by the last round is wider than
    // its chunk size (uniform: an LDS flag read after a barrier)
    if (!fresh && !flag[(r - 1) & 1]) {
      if (++stage == a.nst) break;
      fresh = true;
    }
    fresh = false;
    const int32_t tb = a.chunk[stage];
    if (tid == 0) flag[r & 1] = 0;  // set by this round; last read at the top of round r - 1
    const int n = 2 * nk, nu = (n + 255) / 256;
    if (!scored) {
      // candidates: the halves of the chunks wider than tb, the others as they are
      for (int j = tid; j < nk; j += 256) {
        const int32_t lo = as[j], hi = ae[j];
        const bool halve = hi - lo > tb;
        const int32_t m = lo + (hi - lo) / 2;
        bs[2 * j] = lo;
        be[2 * j] = halve ? m : hi;
        bs[2 * j + 1] = halve ? m : -1;
        be[2 * j + 1] = halve ? hi : -1;
      }
      __syncthreads();
      score_slots<E, KE, D, GMAX, UNROLL, true>(qo, Kbase, row_of, bs, be, n, Tp, s, key, stg);
      __syncthreads();
    }
    scored = false;
    uint64_t kr[kKpt];
#pragma unroll
    for (int u = 0; u < kKpt; u++) {
      const int c = tid + 256 * u;
      kr[u] = u < nu && c < n ? key[c] : 0ull;
    }
    const uint64_t thr = radix_threshold(kr, nu, (uint32_t)a.keep[stage], hist, pass);
    nk = compact_kept(kr, nu, thr, bs, be, tb, as, ae, wcnt, &flag[r & 1]);
    __syncthreads();
  }

  // the last stage's kept chunks are single blocks: the list, ascending (a
  // block's place is the number of smaller kept blocks).  When 256 is a
  // multiple of K_b and 16 <= K_b <= 128, 256 / K_b threads share a block's
  // comparisons and the counts meet in `pos`.
  if (256 % Kb == 0 && Kb >= 16 && Kb <= 128) {
    const int parts = 256 / Kb, span = Kb / parts;
    const int j = tid % Kb, u0 = (tid / Kb) * span;
    const int32_t v = j < nk ? as[j] : 0;
    int rk = 0;
    for (int t0 = 0; t0 < span; t0 += 4) {
      int32_t vv[4];
#pragma unroll
      for (int t = 0; t < 4; t++) vv[t] = as[max(min(u0 + min(t0 + t, span - 1), nk - 1), 0)];
#pragma unroll
      for (int t = 0; t < 4; t++) rk += (t0 + t < span) & (u0 + t0 + t < nk) & (vv[t] < v);
    }
    if (j < nk && rk) atomicAdd(&pos[j], rk);
    __syncthreads();
    if (tid < Kb) {
      if (tid < nk) out[pos[tid]] = v;
      else out[tid] = -1;
    }
    if (tid == 0) a.m.nnz[prob] = nk;
    return;
  }
  for (int j = tid; j < Kb; j += 256) {
    if (j < nk) {
      const int32_t v = as[j];
      int rk = 0;
      for (int u0 = 0; u0 < nk; u0 += 16) {
        int32_t vv[16];
#pragma unroll
        for (int t = 0; t < 16; t++) vv[t] = as[min(u0 + t, nk - 1)];
#pragma unroll
        for (int t = 0; t < 16; t++) rk += (u0 + t < nk) && vv[t] < v;
      }
      if (rk < Kb) out[rk] = v;  // always: the last stage keeps at most K_b
    } else {
      out[j] = -1;
    }
  }
  if (tid == 0) a.m.nnz[prob] = nk;
}

template <typename E, typename KE, int D, int GMAX, bool PAGED>
void launch_g(const StageArgs &a, size_t lds, hipStream_t st) {
  constexpr bool kMfma = std::is_same<E, uint16_t>::value;
  constexpr int RPP = 256 / (D / Vec<E>::N);
  const int n = 2 * a.cap;  // the most candidate slots of a round
  // loads in flight per lane: candidate tiles per wave (MFMA) or rows per lane (VALU)
  const int per = kMfma ? ((n + 15) / 16 + 3) / 4 : (n + RPP - 1) / RPP;
  const dim3 grid((unsigned)(a.m.s.problems * a.splits)), block(256);
  if (per <= 2) hipLaunchKernelGGL((mask_stages_kernel<E, KE, D, GMAX, 2, PAGED>), grid, block, lds, st, a);
  else hipLaunchKernelGGL((mask_stages_kernel<E, KE, D, GMAX, 8, PAGED>), grid, block, lds, st, a);
}

template <typename E, typename KE, int D, bool PAGED>
void launch_d(const StageArgs &a, size_t lds, hipStream_t st) {
  const int G = a.m.s.G;
  if (G <= 1) launch_g<E, KE, D, 1, PAGED>(a, lds, st);
  else if (G <= 2) launch_g<E, KE, D, 2, PAGED>(a, lds, st);
  else if (G <= 4) launch_g<E, KE, D, 4, PAGED>(a, lds, st);
  else if (G <= 8) launch_g<E, KE, D, 8, PAGED>(a, lds, st);
  else launch_g<E, KE, D, 16, PAGED>(a, lds, st);
}

template <bool PAGED>
void launch_layout(const StageArgs &a, size_t lds, hipStream_t st) {
  const bool d64 = a.m.s.d == 64;
  if (a.m.s.dtype == HIPSA_BF16) {
    if (d64) launch_d<uint16_t, uint16_t, 64, PAGED>(a, lds, st);
    else launch_d<uint16_t, uint16_t, 128, PAGED>(a, lds, st);
  } else if (a.m.s.dtype == HIPSA_BF16_E5M2) {
    if (d64) launch_d<uint16_t, uint8_t, 64, PAGED>(a, lds, st);
    else launch_d<uint16_t, uint8_t, 128, PAGED>(a, lds, st);
  } else {
    if (d64) launch_d<float, float, 64, PAGED>(a, lds, st);
    else launch_d<float, float, 128, PAGED>(a, lds, st);
  }
}

}  // namespace

// Dynamic LDS of one workgroup: key (8 bytes) and B (8 bytes) per slot, two
// slots per chunk, A 8 bytes per chunk, the page numbers when paged, then the
// row-gather tiles of the matrix-core path when they fit beside the rest.
constexpr size_t kLdsBudget = 160 * 1024 - 4096;  // per workgroup, less the static arrays

size_t lists_lds(const StageArgs &a) {
  const size_t chunks = (size_t)a.cap * (2 * 8 + 2 * 8 + 8);
  const size_t pages = a.m.pg.table ? (size_t)a.m.pg.seq_pages * sizeof(int32_t) : 0;
  return (chunks + pages + 15) / 16 * 16;
}

size_t tiles_lds(const StageArgs &a) {
  if (a.m.s.dtype == HIPSA_F32) return 0;
  const bool d64 = a.m.s.d == 64;
  if (a.m.s.dtype == HIPSA_BF16)
    return d64 ? stage_bytes<uint16_t, uint16_t, 64>() : stage_bytes<uint16_t, uint16_t, 128>();
  return d64 ? stage_bytes<uint16_t, uint8_t, 64>() : stage_bytes<uint16_t, uint8_t, 128>();
}

size_t mask_stages_lds(const StageArgs &a) {
  return lists_lds(a) + (a.stage_off >= 0 ? tiles_lds(a) : 0);
}

// The first round of stage 1 holds 2 * n0 candidates (n0 stage-0 chunks);
// one workgroup gathers them at about 40 GB/s (per-CU gather throughput), so
// a wide first round is spread over several workgroups per problem, each
// scoring at least kSplitSlots slots, with at most one workgroup per CU in
// all.  Rounds of up to kSplitFrom slots stay in one workgroup: the round
// trip of the keys through memory and the arrival cost about as much as the
// spread saves there.
constexpr int kSplitFrom = 1024;
constexpr int kSplitSlots = 128;

size_t mask_stages_plan(StageArgs *a) {
  const Shape &s = a->m.s;
  const int64_t blocks = (s.T + s.bk - 1) / s.bk;
  a->n1max = (int32_t)(2 * ((blocks + a->chunk[0] - 1) / a->chunk[0]));
  a->splits = 1;
  if (s.problems > 0 && a->n1max > kSplitFrom) {
    const int64_t by_cu = 256 / s.problems;
    const int64_t by_slots = (a->n1max + kSplitSlots - 1) / kSplitSlots;
    a->splits = (int32_t)std::max<int64_t>(1, std::min(by_cu, by_slots));
  }
  if (a->splits == 1) return 0;
  const size_t keys = ((size_t)s.problems * a->n1max * sizeof(uint64_t) + 255) / 256 * 256;
  return keys + (size_t)s.problems * sizeof(uint32_t);
}

hipError_t launch_mask_stages(const StageArgs &a0, hipStream_t st) {
  StageArgs a = a0;
  const size_t tiles = tiles_lds(a);
  a.stage_off = tiles > 0 && lists_lds(a) + tiles <= kLdsBudget ? (int32_t)lists_lds(a) : -1;
  const size_t lds = mask_stages_lds(a);
  if (a.m.pg.table) launch_layout<true>(a, lds, st);
  else launch_layout<false>(a, lds, st);
  return hipGetLastError();
}

}  // namespace hipsa
