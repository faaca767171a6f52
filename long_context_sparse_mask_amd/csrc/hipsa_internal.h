// Internal declarations shared by the HIP kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hipsa.h"

namespace hipsa {

constexpr int kMaxKb = 512;   // largest K_b = k / block_k the kernels accept
constexpr int kMaxGroup = 16; // largest Hq / Hkv
constexpr int kMaxDenseBlocks = 256;  // largest (sink + window) / block_k
// Scratch array of hip_sparse_attn_noalloc (per GPU, library-owned).
constexpr size_t kNoAllocScratchBytes = size_t(8) << 20;
// Its address on the device that runs `stream` (looked up once per device).
hipError_t noalloc_scratch(hipStream_t stream, void **ptr);

// Validated shape of one call, in the units the kernels use.
struct Shape {
  int64_t B, Hq, Hkv, Tq, T, T_cap, d;
  int32_t G, Kb, bk, bq, causal, dtype;
  int32_t bk_shift;  // log2(bk)
  int64_t nqb;     // query blocks per (b, kv head)
  int64_t problems; // B * Hkv * nqb
  int32_t sink_b, window_b;  // dense part, in blocks (0 = none)
};

// Paged K/V: K and V are [num_pages, Hkv, page_size, d] and key position t of
// sequence b lives in page table[b * max_pages + t / page_size].  table ==
// nullptr means the contiguous [B, Hkv, T_cap, d] layout.
struct Pages {
  const int32_t *table;
  int64_t max_pages;
  int32_t ps_shift;      // log2(page_size), >= log2(block_k)
  int32_t last_page;     // num_pages - 1: table entries are clamped to [0, last_page]
  int32_t seq_pages;     // ceil(T / page_size): the table entries a sequence uses
};
constexpr int kMaxSeqPagesOnChip = 16384;  // mask kernels stage a sequence's pages in LDS
// Largest K_b of the one-launch decode step (its kept blocks stay in LDS).
constexpr int kStepMaxKb = 64;

struct MaskArgs {
  const void *q, *K;
  int32_t *indices, *nnz;
  Shape s;
  Pages pg;
};

struct AttnArgs {
  const void *q, *K, *V;
  const int32_t *indices, *nnz;
  void *out;
  float *ws;
  Shape s;
  int32_t splits;  // decode: key splits per problem
  float scale;     // 1 / sqrt(d)
  Pages pg;
};

// One decode step: the search and the split attention of a problem in one
// launch, then the merge; indices/nnz receive the mask like hip_mask_estimate.
struct StepArgs {
  AttnArgs at;  // at.indices, at.nnz unused: the lists stay on chip
  int32_t *indices, *nnz;
  uint32_t *arrived;  // per problem: split workgroups done (zero between calls)
};

// Multi-stage search (per-row problems): stage 0 cuts chunks of chunk[0]
// blocks and keeps them all; stage j >= 1 halves the kept chunks wider than
// chunk[j] blocks and keeps the keep[j] best per round.
constexpr int kMaxStages = 8;
constexpr int kMaxStageChunks = 2048;  // largest stage-0 chunk count and per-round keep
struct StageArgs {
  MaskArgs m;           // m.s.Kb = keep[nst - 1]
  int32_t nst;
  int32_t chunk[kMaxStages];  // blocks, strictly decreasing, chunk[nst - 1] == 1
  int32_t keep[kMaxStages];   // keep[0] unused
  int32_t cap;          // LDS capacity in chunks: stage-0 count and every keep fit
  // Wide first rounds: `splits` workgroups per problem score the first round
  // of stage 1 (2 * stage-0 chunks slots), store the keys in `keys`
  // [problems, n1max], and the last to arrive (`arrived`, zero between calls)
  // runs the rest of the search.  splits == 1: one workgroup does it all.
  int32_t splits;
  int32_t n1max;
  uint64_t *keys;
  uint32_t *arrived;
  int32_t stage_off;  // byte offset in dynamic LDS of the row-gather tiles, -1: none
};
hipError_t launch_mask_stages(const StageArgs &a, hipStream_t st);
size_t mask_stages_lds(const StageArgs &a);  // dynamic LDS bytes of one workgroup
// Workgroups per problem for the first round (fills splits), and the
// workspace bytes that needs (keys, then one arrival counter per problem).
size_t mask_stages_plan(StageArgs *a);

// Decode / per-row problems (block_q == 1).
hipError_t launch_mask_decode(const MaskArgs &a, hipStream_t st);
hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t st);
hipError_t launch_attn_combine(const AttnArgs &a, hipStream_t st);  // merge of the split partials
hipError_t launch_decode_step(const StepArgs &a, hipStream_t st);
size_t attn_decode_workspace(const Shape &s);
size_t decode_step_workspace(const Shape &s);  // partials, then one arrival counter per problem
int32_t attn_decode_splits(const Shape &s);
int attn_decode_tokens(const Shape &s);  // tokens per split workgroup
constexpr int64_t kWideGrid = 1024;  // split workgroups from which V rows are read 16 bytes per lane

// Chunked prefill (block_q == 64, bf16).
hipError_t launch_mask_prefill(const MaskArgs &a, hipStream_t st);
hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t st);

// ------------------------------------------------------------------ device helpers

// Tokens in a row's key sequence: the dense entries and the list.
inline int64_t entry_tokens(const Shape &s) {
  return (int64_t)(s.Kb + s.sink_b + s.window_b) * s.bk;
}

// Dense part of a query block that sees Np key blocks: sink blocks [0, Sb)
// and window blocks [Np - Wb, Np), the sink first when they overlap.  The
// search covers the blocks between them.
struct Dense {
  int32_t Sb, Wb;
  __device__ Dense(const Shape &s, int32_t Np) {
    Sb = min(s.sink_b, Np);
    Wb = min(s.window_b, Np - Sb);
  }
};

// Block of entry n of a row's key sequence, or -1 if the entry holds none.
// The sequence is the dense part, at fixed entries (sink: 0 .. sink_b-1,
// window: sink_b .. sink_b+window_b-1, unused when the row sees fewer
// blocks), then the list: an id past nnz (cnt), outside [0, Np) or inside
// the dense part adds nothing.  Branch-free: the list entry is always read.
__device__ inline int32_t entry_block(int n, const int32_t *list, int cnt, const Shape &s,
                                      int32_t Np, const Dense &dn) {
  const int nd = s.sink_b + s.window_b;
  const int m = n - nd;
  const int32_t lb = list[min(max(m, 0), s.Kb - 1)];
  const int j = n - s.sink_b;
  const int32_t db = n < s.sink_b ? (n < dn.Sb ? n : -1) : (j < dn.Wb ? Np - dn.Wb + j : -1);
  const bool lok = m < cnt && lb >= dn.Sb && lb < Np - dn.Wb;
  return m < 0 ? db : (lok ? lb : -1);
}

// Paged K/V addressing.  page_at() reads one table entry (clamped into the
// pool, so a bad table cannot send a load out of bounds); paged_row() is the
// row, in units of d elements, of position t of KV head g in that page.
__device__ inline int32_t page_at(const Pages &pg, uint32_t b, int32_t logical_page) {
  const int32_t p = pg.table[(int64_t)b * pg.max_pages + logical_page];
  return min(max(p, 0), pg.last_page);
}
__device__ inline int64_t paged_row(int32_t page, uint32_t g, uint32_t Hkv, int32_t t, int ps_shift) {
  return (((int64_t)page * Hkv + g) << ps_shift) + (t & ((1 << ps_shift) - 1));
}
// The mask kernels stage the pages of positions 0 .. Tp-1 of sequence b in
// LDS once (every round then finds a centre row without another memory trip).
// Called by the 256 threads of a mask workgroup.  Each thread issues a batch
// of 16 loads (addresses clamped, no branches) before storing any, so a batch
// costs one memory latency, not 16.  The first batch (4096 pages) is
// straight-line code: at the head of a loop the compiler waits for every load
// in flight, the caller's too.
__device__ inline void stage_pages(const Pages &pg, uint32_t b, int32_t Tp, int32_t *ptab) {
  constexpr int U = 16;
  const int32_t n = ((Tp - 1) >> pg.ps_shift) + 1;
  const int32_t *row = pg.table + (int64_t)b * pg.max_pages;
  constexpr int32_t stride = 256;
  auto batch = [&](int32_t j0) {
    int32_t v[U];
#pragma unroll
    for (int u = 0; u < U; u++) v[u] = row[min(j0 + u * stride, n - 1)];
#pragma unroll
    for (int u = 0; u < U; u++)
      if (j0 + u * stride < n) ptab[j0 + u * stride] = min(max(v[u], 0), pg.last_page);
  };
  batch((int32_t)threadIdx.x);
  for (int32_t j0 = (int32_t)threadIdx.x + U * stride; j0 < n; j0 += U * stride) batch(j0);
}

// Workgroup -> logical work item, XCD-aware.  gfx950 dispatches the
// workgroups of a launch round-robin over its 8 XCDs (workgroup x runs on
// XCD x % 8), and each XCD has its own L2.  This bijection on [0, P) gives
// XCD j a contiguous range of logical items (ceil or floor of P/8), so items
// that are adjacent in logical order (the query blocks of one KV head, which
// select overlapping key blocks) share an L2.  The decode kernels use it on
// (problem, split) and (problem, head) items numbered problem-major, so a
// problem's mask, its split workgroups and its merge all run on the same XCD
// (for P a multiple of 8; otherwise on neighbouring ones), and the list and
// the partials are read on the XCD that wrote them.
// XCD j's range starts at j*q + min(j, r): the first r XCDs take q + 1 items.
// Written without a branch, so the scalar code around it stays one block.
__device__ inline uint32_t xcd_swizzle(uint32_t x, uint32_t P) {
  constexpr uint32_t kXcd = 8;
  const uint32_t q = P / kXcd, r = P % kXcd, xcd = x % kXcd, i = x / kXcd;
  return xcd * q + min(xcd, r) + i;
}


// 16-byte vector loads widened to fp32.  bf16 widens exactly by a 16-bit shift.
template <typename E> struct Vec;
// raw() issues the load; widen() converts (and zeroes the slice when `keep`
// is false), so a batch of loads can be issued without branches and all be
// in flight at once.
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ static inline uint4 raw(const float *p) { return *reinterpret_cast<const uint4 *>(p); }
  __device__ static inline void widen(uint4 x, bool keep, float (&v)[4]) {
    v[0] = keep ? __uint_as_float(x.x) : 0.f;
    v[1] = keep ? __uint_as_float(x.y) : 0.f;
    v[2] = keep ? __uint_as_float(x.z) : 0.f;
    v[3] = keep ? __uint_as_float(x.w) : 0.f;
  }
  __device__ static inline void load(const float *p, float (&v)[4]) { widen(raw(p), true, v); }
};
template <> struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ static inline uint4 raw(const uint16_t *p) {
    return *reinterpret_cast<const uint4 *>(p);
  }
  __device__ static inline void widen(uint4 x, bool keep, float (&v)[8]) {
    const uint32_t w[4] = {keep ? x.x : 0u, keep ? x.y : 0u, keep ? x.z : 0u, keep ? x.w : 0u};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static inline void load(const uint16_t *p, float (&v)[8]) { widen(raw(p), true, v); }
};

// ------------------------------------------------------------------ fp8 K/V (OCP E5M2)
// gfx950 converts OCP E5M2 codes ("bf8" in the ISA) in hardware, two per
// instruction, taken from the low or the high 16-bit half of a register:
// v_cvt_pk_f32_bf8 to two fp32, v_cvt_scalef32_pk_bf16_bf8 (scale 1) to two
// bf16.  Both are exact for every finite code: an E5M2 value has 2 mantissa
// bits and magnitude 2^-16 .. 57344, so it is also an fp32 and a bf16 value.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <bool HI> __device__ inline uint32_t e5m2x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
}
template <bool HI> __device__ inline f32x2_t e5m2x2_to_f32x2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_bf8(w, HI);
}

// Eight consecutive elements of a K or V row as one bf16 matrix-core operand
// (16 bytes).  raw() issues the load (16 bytes of bf16, or 8 bytes of E5M2
// codes); bf16() converts once the load has landed, so a batch of loads can
// all be in flight before the first conversion.
template <typename KE> struct Kv8;
template <> struct Kv8<uint16_t> {
  using raw_t = uint4;
  __device__ static inline raw_t raw(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
  __device__ static inline uint4 bf16(raw_t r) { return r; }
};
template <> struct Kv8<uint8_t> {
  using raw_t = uint2;
  __device__ static inline raw_t raw(const uint8_t *p) { return *reinterpret_cast<const uint2 *>(p); }
  __device__ static inline uint4 bf16(raw_t r) {
    return make_uint4(e5m2x2_to_bf16x2<false>(r.x), e5m2x2_to_bf16x2<true>(r.x),
                      e5m2x2_to_bf16x2<false>(r.y), e5m2x2_to_bf16x2<true>(r.y));
  }
};

// Gathers of 16 key rows in matrix-core operand layout, through LDS.  In the
// operand layout the 16 lanes of a quarter-wave read 16 different rows, and a
// CU then fetches each 128-byte line of a row in two halves: measured on
// MI355X, one workgroup gathers random 256-byte rows at about 17 GB/s that
// way and at about 30 GB/s when the lanes of a quarter-wave read one row
// together (16 bytes each).  So a tile is loaded row by row
// (kLanesPerRow lanes per row, kRowsPerLoad rows per load), written to a
// per-wave LDS tile whose rows are padded by 16 bytes (the transposed reads
// then hit distinct banks), and read back in operand layout: lane l gets row
// l % 16, elements 32 ks + 8 (l / 16) .. + 7 of k-step ks.
template <typename KE, int D>
struct TileGather {
  static constexpr int kRowBytes = D * (int)sizeof(KE);
  static constexpr int kLanesPerRow = kRowBytes / 16;
  static constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  static constexpr int kLoads = 16 / kRowsPerLoad;
  static constexpr int kStride = kRowBytes + 16;
  static constexpr int kBytes = 16 * kStride;  // LDS bytes of one tile
  static constexpr int KS = D / 32;
  using raw_t = typename Kv8<KE>::raw_t;

  // tile row that this lane loads in load j
  __device__ static int row(int j) { return j * kRowsPerLoad + (int)(threadIdx.x & 63) / kLanesPerRow; }
  // this lane's 16 bytes of the row that starts at `p`
  __device__ static uint4 load(const KE *p) {
    return *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(p) +
                                            16 * ((int)(threadIdx.x & 63) % kLanesPerRow));
  }
  __device__ static void put(const uint4 (&v)[kLoads], uint8_t *tile) {
#pragma unroll
    for (int j = 0; j < kLoads; j++)
      *reinterpret_cast<uint4 *>(tile + row(j) * kStride + 16 * ((int)(threadIdx.x & 63) % kLanesPerRow)) = v[j];
  }
  __device__ static void get(const uint8_t *tile, raw_t (&out)[KS]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
      out[ks] = *reinterpret_cast<const raw_t *>(tile + (lane & 15) * kStride +
                                                 (32 * ks + 8 * (lane >> 4)) * (int)sizeof(KE));
  }
};

// Orders a wave's LDS accesses before and after it (a wave reading back what
// it wrote itself).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// N consecutive elements of a V row (N*sizeof(KE) = 2, 4, 8 or 16 bytes)
// widened to fp32; a load that is not kept reads as zeros.
template <typename KE, int N> struct KvN;
template <> struct KvN<uint16_t, 2> {
  using raw_t = uint32_t;
  __device__ static inline raw_t raw(const uint16_t *p) { return *reinterpret_cast<const uint32_t *>(p); }
  __device__ static inline void widen(raw_t w, bool keep, float (&v)[2]) {
    w = keep ? w : 0u;
    v[0] = __uint_as_float(w << 16);
    v[1] = __uint_as_float(w & 0xffff0000u);
  }
};
template <> struct KvN<uint8_t, 2> {
  using raw_t = uint32_t;
  __device__ static inline raw_t raw(const uint8_t *p) { return *reinterpret_cast<const uint16_t *>(p); }
  __device__ static inline void widen(raw_t w, bool keep, float (&v)[2]) {
    const f32x2_t a = e5m2x2_to_f32x2<false>(keep ? w : 0u);
    v[0] = a.x;
    v[1] = a.y;
  }
};
template <> struct KvN<uint8_t, 4> {
  using raw_t = uint32_t;
  __device__ static inline raw_t raw(const uint8_t *p) { return *reinterpret_cast<const uint32_t *>(p); }
  __device__ static inline void widen(raw_t w, bool keep, float (&v)[4]) {
    w = keep ? w : 0u;
    const f32x2_t a = e5m2x2_to_f32x2<false>(w), b = e5m2x2_to_f32x2<true>(w);
    v[0] = a.x;
    v[1] = a.y;
    v[2] = b.x;
    v[3] = b.y;
  }
};
template <> struct KvN<uint16_t, 8> {
  using raw_t = uint4;
  __device__ static inline raw_t raw(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }
  __device__ static inline void widen(raw_t r, bool keep, float (&v)[8]) {
    const uint32_t w[4] = {keep ? r.x : 0u, keep ? r.y : 0u, keep ? r.z : 0u, keep ? r.w : 0u};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <> struct KvN<uint8_t, 8> {
  using raw_t = uint2;
  __device__ static inline raw_t raw(const uint8_t *p) { return *reinterpret_cast<const uint2 *>(p); }
  __device__ static inline void widen(raw_t r, bool keep, float (&v)[8]) {
    const uint32_t x = keep ? r.x : 0u, y = keep ? r.y : 0u;
    const f32x2_t a = e5m2x2_to_f32x2<false>(x), b = e5m2x2_to_f32x2<true>(x);
    const f32x2_t c = e5m2x2_to_f32x2<false>(y), d = e5m2x2_to_f32x2<true>(y);
    v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y;
    v[4] = c.x; v[5] = c.y; v[6] = d.x; v[7] = d.y;
  }
};

// MFMA operand / accumulator vectors (gfx950 bf16 matrix cores).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__device__ inline bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// fp32 -> bf16 bits, round to nearest even (inputs here are finite).
__device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline void store_elem(float *p, float v) { *p = v; }
__device__ inline void store_elem(uint16_t *p, float v) { *p = f32_to_bf16(v); }

// Ranking key of a candidate chunk: larger key = ranked earlier.  Score
// descending first (IEEE order mapped onto unsigned order, -0 folded into +0),
// then chunk start ascending.  0 is below every real key (empty slot).
__device__ inline uint64_t rank_key(float score, int32_t start) {
  float s = score + 0.0f;
  uint32_t u = __float_as_uint(s);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(0x7fffffff - start);
}

// Cross-lane reductions.  DPP moves (quad permutes, row mirrors and
// rotates) run as VALU operand modifiers; steps that cross a 16-lane row use
// gfx950's permlane swaps, which exchange rows (16 lanes) or halves (32
// lanes) of a wave on the VALU instead of routing through LDS.  Called with
// the same value as both operands, permlane16_swap returns the even rows
// duplicated in .x and the odd rows duplicated in .y (permlane32_swap: the
// low half and the high half), so combining .x with .y gives lane i and lane
// i^16 (i^32) the same result.
template <int CTRL> __device__ inline float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7-i within 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- 15-i within 16 lanes
constexpr int kDppRor8 = 0x128;       // lane i <- (i+8) mod 16 within 16 lanes

typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
__device__ inline u32x2_t swap16(float v) {
  const unsigned u = __float_as_uint(v);
  return __builtin_amdgcn_permlane16_swap(u, u, false, false);
}
__device__ inline u32x2_t swap32(float v) {
  const unsigned u = __float_as_uint(v);
  return __builtin_amdgcn_permlane32_swap(u, u, false, false);
}
__device__ inline float xor16_sum(float v) { const u32x2_t r = swap16(v); return __uint_as_float(r.x) + __uint_as_float(r.y); }
__device__ inline float xor32_sum(float v) { const u32x2_t r = swap32(v); return __uint_as_float(r.x) + __uint_as_float(r.y); }
__device__ inline float xor16_max(float v) { const u32x2_t r = swap16(v); return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y)); }
__device__ inline float xor32_max(float v) { const u32x2_t r = swap32(v); return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y)); }

// Sum over aligned groups of W lanes (W a power of two <= 64); every lane of a
// group ends with the group's sum.
template <int W> __device__ inline float group_sum(float v) {
  if (W >= 2) v += dpp_mov<kDppXor1>(v);
  if (W >= 4) v += dpp_mov<kDppXor2>(v);
  if (W >= 8) v += dpp_mov<kDppHalfMirror>(v);
  if (W >= 16) v += dpp_mov<kDppMirror>(v);
  if (W >= 32) v = xor16_sum(v);
  if (W >= 64) v = xor32_sum(v);
  return v;
}
// Sum (max) over the lanes of a wave that share lane % W (W = 8, 16, 32 or 64):
// the reduction across groups of W lanes.
template <int W> __device__ inline float across_sum(float v) {
  if (W <= 8) v += dpp_mov<kDppRor8>(v);
  if (W <= 16) v = xor16_sum(v);
  if (W <= 32) v = xor32_sum(v);
  return v;
}
template <int W> __device__ inline float across_max(float v) {
  if (W <= 8) v = fmaxf(v, dpp_mov<kDppRor8>(v));
  if (W <= 16) v = xor16_max(v);
  if (W <= 32) v = xor32_max(v);
  return v;
}

}  // namespace hipsa
