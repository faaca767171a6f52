// Block-sparse attention for per-row problems (block_q == 1): decode.
//
// Input contract: per (b, kv head, row) a list of key-block ids and its
// length nnz (rebuttal page "A Training-free Sub-quadratic Cost Transformer
// Model Serving Framework With Hierarchically Pruned Attention", reviewer
// NLBm, W2).  Exact softmax over the listed blocks' visible tokens.
//
// A row's key sequence is its dense part (sink and window blocks, if any)
// followed by the listed blocks; entry_block() maps an entry to its block.
//
// Decode attention reads each selected K/V byte once (~4 flops per byte), so
// it is bound by memory.  The K_b*block_k selected tokens of a problem are
// split over S workgroups of TOK tokens (TOK chosen so the launch has >= 512
// workgroups when it can); each of the 4 waves of a split workgroup owns
// TOK/4 token slots.  A wave maps its slots to key rows (an invalid slot
// reads row 0 and is masked, so every load is issued unconditionally),
// issues all of its query, K and V loads at once, and computes the softmax
// statistics (max, sum) and the unnormalised P.V of its slots on its own.
// The four waves are merged with log-sum-exp weights through LDS after one
// barrier, and the workgroup writes (max, sum, output) per head to the
// workspace.  A second kernel merges the S partials of each (problem, head)
// and writes the output; with a single split the split workgroup writes the
// normalised output itself and no merge is launched.  (Merging inside the
// split kernel through a device-scope fence and an arrival counter measured
// slower on gfx950: the fences serialise across workgroups.)  Workgroups map
// to (problem, split) and (problem, head) through xcd_swizzle(), so a
// problem's splits and merge run on the XCD that ran its mask.
//
// With a paged KV cache each lane also reads the page of its slot's token
// from the table (one more dependent load, cached: a block's tokens share a
// page) and addresses its K and V rows through it.
//
// After its loads land, a workgroup's remaining time is pure ALU work, which
// sits in the kernel's tail, so the kernels keep it small: logits on the
// matrix cores for bf16, no per-head tests inside unrolled loops (heads past
// the group are computed and dropped), and no cross-lane reduction of the
// outputs in the bf16 kernel.
#include <type_traits>

#include "decode_split.h"
#include "hipsa_internal.h"

namespace hipsa {
namespace {

// fp32 split workgroup (any dtype works; bf16 uses attn_decode_mfma).  A key
// row is read by TPR = D/VEC lanes (16 bytes each); logits are VALU dot
// products closed by DPP sums over the row's lanes, and P.V accumulates per
// lane and is summed across the wave's row groups with DPP/permlane steps.
// All GMAX heads are computed (the loads of heads past the group repeat the
// last head); only the stores are limited to the group.
template <typename E, int D, int GMAX, int TOK, bool PAGED>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnArgs a) {
  constexpr int VEC = Vec<E>::N;
  constexpr int TPR = D / VEC;            // lanes per key row (8, 16 or 32)
  constexpr int RPW = 64 / TPR;           // rows per wave-wide load
  constexpr int TPW = TOK / 4;            // token slots per wave
  constexpr int RPL = TPW / RPW;          // K rows (and V rows) per lane
  constexpr int HG = GMAX < 4 ? GMAX : 4; // heads per pass over the registers
  static_assert(RPL >= 1 && TPW % RPW == 0, "split too small for the row mapping");
  const Shape &s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rgl = lane / TPR, cs = lane % TPR;
  const uint32_t S = (uint32_t)a.splits;
  const uint32_t wgi = xcd_swizzle(blockIdx.x, gridDim.x);
  const uint32_t split = wgi % S, prob = wgi / S;
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int32_t Tp = s.causal ? (int32_t)(s.T - s.Tq + i + 1) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t *list = a.indices + (int64_t)prob * s.Kb;
  const int32_t cnt = min(max(a.nnz[prob], 0), s.Kb);
  const int base_blk = (int)split * (TOK >> s.bk_shift);
  const Dense dn(s, Np);

  __shared__ float wm[4][GMAX], wl[4][GMAX];
  __shared__ float wo[4][GMAX][D];

  const int64_t kvoff = PAGED ? 0 : (int64_t)(b * Hkv + g) * s.T_cap * D;
  const E *Kp = reinterpret_cast<const E *>(a.K);
  const E *Vp = reinterpret_cast<const E *>(a.V);
  const E *qbase = reinterpret_cast<const E *>(a.q) + ((int64_t)(b * s.Hq + g * s.G) * Tq + i) * D;

  // Token slot u of this lane: wave*TPW + u*RPW + rgl.  A slot past the list,
  // or whose block id is out of range or past the causal limit, reads row 0
  // and is masked, so every load is issued unconditionally.
  int32_t tk[RPL];
  uint4 kr[RPL], vr[RPL], qr[GMAX];
#pragma unroll
  for (int u = 0; u < RPL; u++) {
    const int j = wave * TPW + u * RPW + rgl;
    const int32_t blk = entry_block(base_blk + (j >> s.bk_shift), list, cnt, s, Np, dn);
    const bool ok = blk >= 0;
    const int32_t t = ((ok ? blk : 0) << s.bk_shift) + (j & (s.bk - 1));
    tk[u] = (ok && t < Tp) ? t : -1;
    const int32_t ts = tk[u] >= 0 ? tk[u] : 0;
    int64_t row;
    if constexpr (PAGED) row = paged_row(page_at(a.pg, b, ts >> a.pg.ps_shift), g, Hkv, ts, a.pg.ps_shift) * D;
    else row = kvoff + (int64_t)ts * D;
    row += cs * VEC;
    kr[u] = Vec<E>::raw(Kp + row);
    vr[u] = Vec<E>::raw(Vp + row);
  }
#pragma unroll
  for (int h = 0; h < GMAX; h++) qr[h] = Vec<E>::raw(qbase + (int64_t)min(h, s.G - 1) * Tq * D + cs * VEC);

#pragma unroll
  for (int h0 = 0; h0 < GMAX; h0 += HG) {
    float qv[HG][VEC];
#pragma unroll
    for (int hh = 0; hh < HG; hh++) Vec<E>::widen(qr[h0 + hh], true, qv[hh]);
    // logits of this wave's slots: TPR lanes per row, DPP sums within a row group
    float sc[RPL][HG];
#pragma unroll
    for (int u = 0; u < RPL; u++) {
      float kv[VEC];
      Vec<E>::widen(kr[u], true, kv);
#pragma unroll
      for (int hh = 0; hh < HG; hh++) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; e++) p = fmaf(qv[hh][e], kv[e], p);
        p = group_sum<TPR>(p);
        sc[u][hh] = tk[u] >= 0 ? p * a.scale : -INFINITY;
      }
    }
    // softmax statistics of the wave's slots and P.V, all in registers
    float acc[HG][VEC];
#pragma unroll
    for (int hh = 0; hh < HG; hh++) {
      float m = sc[0][hh];
#pragma unroll
      for (int u = 1; u < RPL; u++) m = fmaxf(m, sc[u][hh]);
      m = across_max<TPR>(m);
      float l = 0.f;
#pragma unroll
      for (int u = 0; u < RPL; u++) {
        sc[u][hh] = sc[u][hh] == -INFINITY ? 0.f : __expf(sc[u][hh] - m);
        l += sc[u][hh];
      }
      l = across_sum<TPR>(l);
      if (lane == 0) { wm[wave][h0 + hh] = m; wl[wave][h0 + hh] = l; }
#pragma unroll
      for (int e = 0; e < VEC; e++) acc[hh][e] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < RPL; u++) {
      float vv[VEC];
      Vec<E>::widen(vr[u], tk[u] >= 0, vv);
#pragma unroll
      for (int hh = 0; hh < HG; hh++)
#pragma unroll
        for (int e = 0; e < VEC; e++) acc[hh][e] = fmaf(sc[u][hh], vv[e], acc[hh][e]);
    }
#pragma unroll
    for (int hh = 0; hh < HG; hh++)
#pragma unroll
      for (int e = 0; e < VEC; e++) acc[hh][e] = across_sum<TPR>(acc[hh][e]);
    if (rgl == 0) {
#pragma unroll
      for (int hh = 0; hh < HG; hh++)
#pragma unroll
        for (int e = 0; e < VEC; e += 4)
          *reinterpret_cast<float4 *>(&wo[wave][h0 + hh][cs * VEC + e]) =
              make_float4(acc[hh][e], acc[hh][e + 1], acc[hh][e + 2], acc[hh][e + 3]);
    }
  }
  __syncthreads();

  // merge the four waves (log-sum-exp weights); partials to the workspace, or
  // with a single split the normalised output itself (no merge launch follows)
  float *mine = a.ws + ((int64_t)(prob * S + split) * s.G) * (D + 2);
  for (int o = tid; o < s.G * D; o += 256) {
    const int h = o / D, x = o % D;
    float M = wm[0][h];
#pragma unroll
    for (int w = 1; w < 4; w++) M = fmaxf(M, wm[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const float c = wm[w][h] == -INFINITY ? 0.f : __expf(wm[w][h] - M);
      L = fmaf(c, wl[w][h], L);
      O = fmaf(c, wo[w][h][x], O);
    }
    if (S == 1) {
      E *out = reinterpret_cast<E *>(a.out) + ((int64_t)(b * s.Hq + g * s.G + h) * Tq + i) * D;
      store_elem(out + x, L > 0.f ? O / L : 0.f);
    } else {
      float *dst = mine + (int64_t)h * (D + 2);
      dst[2 + x] = O;
      if (x == 0) { dst[0] = M; dst[1] = L; }
    }
  }
}

// Split workgroup on the matrix cores for a bf16 query (decode_split.h).
template <typename KE, int D, int GMAX, int TOK, bool PAGED, bool WIDE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 2))) void attn_decode_mfma(AttnArgs a) {
  const uint32_t S = (uint32_t)a.splits;
  const uint32_t wgi = xcd_swizzle(blockIdx.x, gridDim.x);
  const uint32_t split = wgi % S, prob = wgi / S;
  attend_split<KE, D, GMAX, TOK, PAGED, WIDE>(a, prob, split, a.indices + (int64_t)prob * a.s.Kb,
                                              a.nnz + prob);
}

// Merge the S partials of one (problem, query head): one workgroup of D lanes
// (merge_partials).  CH is 16 or 32, chosen so that up to 32 partials take
// one memory round trip.  The merge takes its arguments one by one, 36 bytes in all: the library is
// built with kernel-argument preloading (gfx950's dispatcher writes the first
// argument dwords into scalar registers before the first instruction), so
// they need no scalar-cache read.  Fields spread over the full argument block
// took two or three cache misses one after another.
template <typename E, int D, int CH>
__global__ __launch_bounds__(128) void attn_decode_combine(const float *ws, void *outp, int32_t S_,
                                                           int32_t G_, int32_t Tq_, int32_t Hkv_, int32_t Hq_) {
  const int S = S_;
  const uint32_t G = (uint32_t)G_;
  const uint32_t ph = xcd_swizzle(blockIdx.x, gridDim.x);
  const uint32_t prob = ph / G;
  const int h = (int)(ph % G);
  const uint32_t Tq = (uint32_t)Tq_, Hkv = (uint32_t)Hkv_;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int x = threadIdx.x;  // launched with D lanes
  const float *ph_ = ws + ((int64_t)prob * S * G + h) * (int64_t)(D + 2);
  const int64_t sstride = (int64_t)G * (D + 2);
  E *out = reinterpret_cast<E *>(outp) + ((int64_t)(b * (uint32_t)Hq_ + g * G + h) * Tq + i) * D;
  // S >= 2: launched only for several splits
  store_elem(out + x, merge_partials<CH>(ph_, S, sstride, x, [](const float *p) { return *p; }));
}

// Tokens per split workgroup.  A split that covers a row's whole key
// sequence is used whenever it can (one split: the split workgroup writes the
// output and no merge follows).
//  * bf16 query, groups of up to 8 query heads: 256, 128 or 64, the largest
//    that still gives at least kMinSplitGrid workgroups (one per CU), or half
//    that many when K_b <= kStepMaxKb (the shapes the one-launch decode
//    step serves).  That step runs the problem's search in every split
//    workgroup, so more than one workgroup per CU slows its search, and fewer
//    splits per problem mean fewer searches and a shorter merge: at 32k
//    (8 problems) 16 splits of 128 tokens measured 16.8 us per step against
//    18.4 us for the two calls over 32 splits of 64, and the attention call
//    alone 8.4 against 8.7 us.  The attention reads measured even between
//    128- and 256-token splits at 128k x 4.  256-token splits read V rows 16
//    bytes per lane, which keeps a wave under its 63 loads in flight.
//  * fp32: 128 or 64, the larger when it gives >= 512 workgroups; 64 at
//    d = 128 (a lane's K and V rows must fit in registers).
//  * groups of more than 8 query heads: 64 (the per-head probabilities and
//    outputs of a lane must fit).
template <typename E, int D>
constexpr int max_tokens() {
  return std::is_same<E, uint16_t>::value ? 256 : D == 128 ? 64 : 128;
}
constexpr int64_t kMinSplitGrid = 256;

template <typename E, int D>
int tokens_per_split(const Shape &s) {
  const int64_t total = entry_tokens(s);
  if (s.G > 8) return 64;
  if constexpr (std::is_same<E, uint16_t>::value) {
    const int64_t min_grid = s.Kb <= kStepMaxKb ? kMinSplitGrid / 2 : kMinSplitGrid;
    for (int tok = 256; tok >= 128; tok /= 2)
      if (total <= tok || s.problems * ((total + tok - 1) / tok) >= min_grid) return tok;
    return 64;
  }
  if (max_tokens<E, D>() >= 128 && (total <= 128 || s.problems * ((total + 127) / 128) >= 512))
    return 128;
  return 64;
}

int tokens_for(const Shape &s) {
  if (s.dtype != HIPSA_F32)  // bf16 query: the matrix-core kernel, for either K/V type
    return s.d == 64 ? tokens_per_split<uint16_t, 64>(s) : tokens_per_split<uint16_t, 128>(s);
  return s.d == 64 ? tokens_per_split<float, 64>(s) : tokens_per_split<float, 128>(s);
}

// E: query / output element type; KE: K/V element type (E itself, or E5M2
// codes under a bf16 query).  From kWideGrid split workgroups (about four
// per CU and more) the bf16 kernel reads V rows 16 bytes per lane; below,
// 2-4 bytes per lane.

template <typename KE, int D, int GMAX, bool PAGED, bool WIDE>
void launch_mfma(const AttnArgs &a, dim3 grid, hipStream_t st, int tok) {
  constexpr int G8 = GMAX <= 8 ? GMAX : 8;
  if (GMAX <= 8 && tok == 256) hipLaunchKernelGGL((attn_decode_mfma<KE, D, G8, 256, PAGED, true>), grid, dim3(256), 0, st, a);
  else if (GMAX <= 8 && tok == 128) hipLaunchKernelGGL((attn_decode_mfma<KE, D, G8, 128, PAGED, WIDE>), grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL((attn_decode_mfma<KE, D, GMAX, 64, PAGED, WIDE>), grid, dim3(256), 0, st, a);
}

template <typename E, typename KE, int D, int GMAX, bool PAGED>
void launch_t(const AttnArgs &a, hipStream_t st, int tok) {
  constexpr int kMaxTok = max_tokens<E, D>();
  const dim3 grid((unsigned)(a.s.problems * a.splits)), block(256);
  if constexpr (std::is_same<E, uint16_t>::value) {
    if ((int64_t)a.s.problems * a.splits >= kWideGrid) launch_mfma<KE, D, GMAX, PAGED, true>(a, grid, st, tok);
    else launch_mfma<KE, D, GMAX, PAGED, false>(a, grid, st, tok);
  } else {
    if (tok == 128) {
      if constexpr (kMaxTok >= 128) hipLaunchKernelGGL((attn_decode_kernel<E, D, GMAX, 128, PAGED>), grid, block, 0, st, a);
    } else {
      hipLaunchKernelGGL((attn_decode_kernel<E, D, GMAX, 64, PAGED>), grid, block, 0, st, a);
    }
  }
}

template <typename E, typename KE, int D, bool PAGED>
hipError_t launch_d(const AttnArgs &a, hipStream_t st) {
  const int G = a.s.G, tok = tokens_per_split<E, D>(a.s);
  if (G <= 1) launch_t<E, KE, D, 1, PAGED>(a, st, tok);
  else if (G <= 2) launch_t<E, KE, D, 2, PAGED>(a, st, tok);
  else if (G <= 4) launch_t<E, KE, D, 4, PAGED>(a, st, tok);
  else if (G <= 8) launch_t<E, KE, D, 8, PAGED>(a, st, tok);
  else launch_t<E, KE, D, 16, PAGED>(a, st, tok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attn_combine(a, st);
}

template <typename E, int D>
void launch_combine_t(const AttnArgs &a, hipStream_t st) {
  const dim3 cgrid((unsigned)(a.s.problems * a.s.G));
  const int32_t Tq = (int32_t)a.s.Tq, Hkv = (int32_t)a.s.Hkv, Hq = (int32_t)a.s.Hq;
  if (a.splits <= 16)
    hipLaunchKernelGGL((attn_decode_combine<E, D, 16>), cgrid, dim3(D), 0, st, a.ws, a.out, a.splits, a.s.G, Tq, Hkv, Hq);
  else
    hipLaunchKernelGGL((attn_decode_combine<E, D, 32>), cgrid, dim3(D), 0, st, a.ws, a.out, a.splits, a.s.G, Tq, Hkv, Hq);
}

}  // namespace

hipError_t launch_attn_combine(const AttnArgs &a, hipStream_t st) {
  if (a.splits == 1) return hipSuccess;  // one split wrote the output itself
  const bool bf16 = a.s.dtype != HIPSA_F32;
  if (a.s.d == 64) bf16 ? launch_combine_t<uint16_t, 64>(a, st) : launch_combine_t<float, 64>(a, st);
  else bf16 ? launch_combine_t<uint16_t, 128>(a, st) : launch_combine_t<float, 128>(a, st);
  return hipGetLastError();
}

int attn_decode_tokens(const Shape &s) { return tokens_for(s); }

int32_t attn_decode_splits(const Shape &s) {
  const int tok = tokens_for(s);
  return (int32_t)((entry_tokens(s) + tok - 1) / tok);
}

size_t attn_decode_workspace(const Shape &s) {
  return (size_t)s.problems * attn_decode_splits(s) * s.G * (s.d + 2) * sizeof(float);
}

namespace {
template <bool PAGED>
hipError_t launch_layout(const AttnArgs &a, hipStream_t st) {
  const bool d64 = a.s.d == 64;
  if (a.s.dtype == HIPSA_BF16)
    return d64 ? launch_d<uint16_t, uint16_t, 64, PAGED>(a, st) : launch_d<uint16_t, uint16_t, 128, PAGED>(a, st);
  if (a.s.dtype == HIPSA_BF16_E5M2)
    return d64 ? launch_d<uint16_t, uint8_t, 64, PAGED>(a, st) : launch_d<uint16_t, uint8_t, 128, PAGED>(a, st);
  return d64 ? launch_d<float, float, 64, PAGED>(a, st) : launch_d<float, float, 128, PAGED>(a, st);
}
}  // namespace

hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t st) {
  return a.pg.table ? launch_layout<true>(a, st) : launch_layout<false>(a, st);
}

}  // namespace hipsa
