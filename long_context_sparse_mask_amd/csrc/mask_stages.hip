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
#include "decode_score.h"
#include "hipsa_internal.h"

namespace hipsa {
namespace {

// Rounds of one problem: each round of a stage halves its widest chunks or
// is the stage's first, so a problem runs at most nst + 31 * (nst - 1) rounds
// (chunks are at most 2^31 blocks wide); the bound only guards the loop.
constexpr int kMaxRounds = 512;

struct Select {
  uint64_t prefix;  // digits of the threshold found so far (lower digits zero)
  uint32_t need;    // keys still to keep among those sharing the prefix
  uint32_t done;
};

__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int32_t wave_max(int32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}

// Threshold of the `keep` largest non-zero keys of key[0..n): the value thr
// such that exactly min(keep, live) keys are >= thr (1 when at most `keep`
// keys are live).  Non-zero keys must be distinct.  `hist` (256 counters)
// must be zero on entry and is zero on return.  Called by all 256 threads;
// two barriers per digit.
__device__ uint64_t radix_threshold(const uint64_t *key, int n, uint32_t keep, uint32_t *hist,
                                    Select *sel) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t prefix = 0;
  uint32_t need = keep;
  for (int shift = 56; shift >= 0; shift -= 8) {
    // keys that share the digits above `shift` with the prefix
    const uint64_t hm = shift == 56 ? 0ull : ~0ull << (shift + 8);
    for (int c = tid; c < n; c += 256) {
      const uint64_t k = key[c];
      const bool in = k != 0 && ((k ^ prefix) & hm) == 0;
      const uint32_t d = (uint32_t)(k >> shift) & 255u;
      const uint64_t act = __ballot(in);
      if (act == 0) continue;
      // Scores of one problem share their top digits, so most lanes of a wave
      // often add to one counter: those add once, through the first lane.
      const int leader = __builtin_ctzll(act);
      const uint32_t d0 = __builtin_amdgcn_readlane(d, leader);
      const uint64_t same = __ballot(in && d == d0);
      if (in && d != d0) atomicAdd(&hist[d], 1u);
      if (lane == leader) atomicAdd(&hist[d0], (uint32_t)__popcll(same));
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 255-4l .. 252-4l, the highest first
      uint32_t cnt[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        cnt[j] = hist[255 - 4 * lane - j];
        sum += cnt[j];
      }
      const uint32_t incl = wave_inclusive_sum(sum);
      const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
      if (total <= need) {
        // every key sharing the prefix is kept (only when at most `keep` keys
        // are live: later digits always hold more keys than are needed)
        if (lane == 0) *sel = Select{prefix ? prefix : 1ull, 0u, 1u};
      } else {
        uint32_t above = incl - sum;  // keys with a higher digit
#pragma unroll
        for (int j = 0; j < 4; j++) {
          if (above < need && need <= above + cnt[j]) {
            const uint32_t rest = need - above;
            *sel = Select{prefix | ((uint64_t)(255 - 4 * lane - j) << shift), rest, cnt[j] == rest};
          }
          above += cnt[j];
        }
      }
#pragma unroll
      for (int j = 0; j < 4; j++) hist[255 - 4 * lane - j] = 0;
    }
    __syncthreads();
    prefix = sel->prefix;
    need = sel->need;
    if (sel->done) break;
  }
  return prefix;
}

// Copies the slots (bs, be) of key >= thr to (as, ae), compact, in slot order;
// returns their count and sets *maxw to the widest kept chunk.  Each wave
// counts the kept slots of its 64-slot groups, then writes them from its
// offset.  Called by all 256 threads; one barrier.
__device__ int compact_kept(const uint64_t *key, const int32_t *bs, const int32_t *be, int n,
                            uint64_t thr, int32_t *as, int32_t *ae, int32_t *wcnt, int32_t *wmax,
                            int32_t *maxw) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int cnt = 0;
  int32_t w = 0;
  for (int c = wave * 64 + lane; c - lane < n; c += 256) {
    const bool kept = c < n && key[c] >= thr;
    cnt += __popcll(__ballot(kept));
    if (kept) w = max(w, be[c] - bs[c]);
  }
  w = wave_max(w);
  if (lane == 0) {
    wcnt[wave] = cnt;
    wmax[wave] = w;
  }
  __syncthreads();
  int off = 0;
  for (int v = 0; v < wave; v++) off += wcnt[v];
  *maxw = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const int total = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
  for (int c = wave * 64 + lane; c - lane < n; c += 256) {
    const bool kept = c < n && key[c] >= thr;
    const uint64_t m = __ballot(kept);
    if (kept) {
      const int pos = off + __popcll(m & ((1ull << lane) - 1));
      as[pos] = bs[c];
      ae[pos] = be[c];
    }
    off += __popcll(m);
  }
  return total;
}

template <typename E, typename KE, int D, int GMAX, int UNROLL, bool PAGED>
__global__ __launch_bounds__(256) void mask_stages_kernel(StageArgs a) {
  const Shape &s = a.m.s;
  const int tid = threadIdx.x;

  const uint32_t prob = xcd_swizzle(blockIdx.x, gridDim.x);
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
    for (int j = tid; j < Kb; j += 256) out[j] = j < M ? first + j : -1;
    if (tid == 0) a.m.nnz[prob] = M;
    return;
  }

  extern __shared__ uint64_t lds[];
  const int cap = a.cap;
  uint64_t *key = lds;                                         // [2 cap]
  int32_t *bs = reinterpret_cast<int32_t *>(key + 2 * cap);    // [2 cap]
  int32_t *be = bs + 2 * cap;                                  // [2 cap]
  int32_t *as = be + 2 * cap, *ae = as + cap;                  // [cap] each
  int32_t *ptab = ae + cap;                                    // paged: the sequence's pages
  __shared__ uint32_t hist[256];
  __shared__ Select sel;
  __shared__ int32_t wcnt[4], wmax[4];

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
  const int32_t c0 = a.chunk[0];
  int nk = (M + c0 - 1) / c0;
  for (int j = tid; j < nk; j += 256) {
    as[j] = first + j * c0;
    ae[j] = min(first + (j + 1) * c0, first + M);
  }
  hist[tid] = 0;
  int32_t maxw = min(c0, M);  // widest kept chunk
  __syncthreads();

  int stage = 1;
  bool fresh = true;  // the stage has run no round yet
  for (int round = 0; round < kMaxRounds; round++) {
    const int32_t tb = a.chunk[stage];
    if (!fresh && maxw <= tb) {  // the stage is done (uniform: LDS values after a barrier)
      if (++stage == a.nst) break;
      fresh = true;
      continue;
    }
    fresh = false;
    // candidates: the halves of the chunks wider than tb, the others as they are
    for (int j = tid; j < nk; j += 256) {
      const int32_t lo = as[j], hi = ae[j];
      const bool split = hi - lo > tb;
      const int32_t m = lo + (hi - lo) / 2;
      bs[2 * j] = lo;
      be[2 * j] = split ? m : hi;
      bs[2 * j + 1] = split ? m : -1;
      be[2 * j + 1] = split ? hi : -1;
    }
    const int n = 2 * nk;
    __syncthreads();
    score_slots<E, KE, D, GMAX, UNROLL>(qo, Kbase, row_of, bs, be, n, Tp, s, key);
    __syncthreads();
    const uint64_t thr = radix_threshold(key, n, (uint32_t)a.keep[stage], hist, &sel);
    nk = compact_kept(key, bs, be, n, thr, as, ae, wcnt, wmax, &maxw);
    __syncthreads();
  }

  // the last stage's kept chunks are single blocks: the list, ascending
  for (int j = tid; j < Kb; j += 256) {
    if (j < nk) {
      const int32_t v = as[j];
      int r = 0;
      for (int u = 0; u < nk; u++) r += as[u] < v;
      if (r < Kb) out[r] = v;  // always: the last stage keeps at most K_b
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
  const dim3 grid((unsigned)a.m.s.problems), block(256);
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

size_t mask_stages_lds(const StageArgs &a) {
  // key (8 bytes) and B (8 bytes) per slot, two slots per chunk; A 8 bytes per chunk
  const size_t chunks = (size_t)a.cap * (2 * 8 + 2 * 8 + 8);
  return chunks + (a.m.pg.table ? (size_t)a.m.pg.seq_pages * sizeof(int32_t) : 0);
}

hipError_t launch_mask_stages(const StageArgs &a, hipStream_t st) {
  const size_t lds = mask_stages_lds(a);
  if (a.m.pg.table) launch_layout<true>(a, lds, st);
  else launch_layout<false>(a, lds, st);
  return hipGetLastError();
}

}  // namespace hipsa
