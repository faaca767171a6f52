// Block-sparse attention for per-row problems (block_q == 1): decode.
//
// Input contract: per (b, kv head, row) a list of key-block ids and its
// length nnz (rebuttal page "A Training-free Sub-quadratic Cost Transformer
// Model Serving Framework With Hierarchically Pruned Attention", reviewer
// NLBm, W2).  Exact softmax over the listed blocks' visible tokens.
//
// Decode attention reads each selected K/V byte once (~4 flops per byte), so
// it is bound by memory: the kernels keep many independent loads in flight
// and add as few dependent round trips as possible.  The K_b*block_k selected
// tokens of a problem are split over S workgroups of TOK tokens (TOK chosen
// so the launch has >= 512 workgroups when it can).  A split workgroup:
//   1. maps its TOK token slots to key rows (an invalid slot reads row 0 and
//      is masked) and issues every query, K and V load of its slice at once.
//      bf16 logits run on v_mfma_f32_16x16x32_bf16 (the group's query heads,
//      zero-padded to 16 rows, against 16 key rows per tile read straight
//      into the B operand); fp32 logits use 16-byte VALU dot products with
//      DPP reductions;
//   2. one wave per head takes the max and exponentials; P.V accumulates in
//      fp32 on the VALU over coalesced V rows and is reduced across row
//      groups once, through LDS;
//   3. writes its (max, sum, unnormalised output) per head to the workspace.
// A second kernel merges the S partials of each (problem, head) with
// log-sum-exp weights and writes the output.  (Merging inside the split
// kernel through a device-scope fence and an arrival counter measured
// slower on gfx950: the fences serialise across workgroups.)
#include <type_traits>

#include "hipsa_internal.h"

namespace hipsa {
namespace {

template <typename E, int D, int GMAX, int TOK>
__global__ __launch_bounds__(256) void attn_decode_kernel(AttnArgs a) {
  constexpr bool kMfma = std::is_same<E, uint16_t>::value;
  constexpr int VEC = Vec<E>::N;
  constexpr int TPR = D / VEC;            // lanes per V row
  constexpr int RPP = 256 / TPR;          // V rows per pass
  constexpr int RPT = TOK / RPP;          // V rows per lane
  constexpr int HG = GMAX < 4 ? GMAX : 4; // heads reduced per LDS pass
  constexpr int KS = D / 32;              // MFMA k-steps
  constexpr int KTW = TOK / 64;           // MFMA key tiles of 16 per wave
  const Shape &s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = tid / TPR, cs = tid % TPR;
  const uint32_t S = (uint32_t)a.splits;
  const uint32_t split = blockIdx.x % S, prob = blockIdx.x / S;
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int32_t Tp = s.causal ? (int32_t)(s.T - s.Tq + i + 1) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t *list = a.indices + (int64_t)prob * s.Kb;
  const int32_t cnt = min(max(a.nnz[prob], 0), s.Kb);
  const int base_blk = (int)split * (TOK >> s.bk_shift);

  __shared__ float pr[GMAX][TOK];
  __shared__ float red[RPP][HG][D];
  __shared__ float stat_m[GMAX], stat_l[GMAX];

#define HIPSA_TOKEN(J, OUT)                                                     \
  do {                                                                          \
    const int n_ = base_blk + ((J) >> s.bk_shift);                              \
    const int32_t blk_ = list[min(n_, s.Kb - 1)];                               \
    const bool ok_ = n_ < cnt && blk_ >= 0 && blk_ < Np;                        \
    const int32_t t_ = ((ok_ ? blk_ : 0) << s.bk_shift) + ((J) & (s.bk - 1));   \
    OUT = (ok_ && t_ < Tp) ? t_ : -1;                                           \
  } while (0)

  const int64_t kvoff = (int64_t)(b * Hkv + g) * s.T_cap * D;
  const E *Kp = reinterpret_cast<const E *>(a.K) + kvoff;
  const E *Vp = reinterpret_cast<const E *>(a.V) + kvoff;
  const E *qbase = reinterpret_cast<const E *>(a.q) + ((int64_t)(b * s.Hq + g * s.G) * Tq + i) * D;

  // V rows of this lane (coalesced: TPR lanes per row), all in flight
  uint4 vr[RPT];
  int32_t vt[RPT];
#pragma unroll
  for (int u = 0; u < RPT; u++) {
    HIPSA_TOKEN(u * RPP + rg, vt[u]);
    vr[u] = Vec<E>::raw(Vp + (int64_t)(vt[u] >= 0 ? vt[u] : 0) * D + cs * VEC);
  }

  if constexpr (kMfma) {
    // query heads of the group as the A operand: lane l holds head l%16
    uint4 qa[KS];
    {
      const int h = lane & 15;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const uint4 r = Vec<E>::raw(qbase + (int64_t)min(h, s.G - 1) * Tq * D + 32 * ks + 8 * (lane >> 4));
        qa[ks] = h < s.G ? r : make_uint4(0, 0, 0, 0);
      }
    }
    // K rows as B operands: lane l holds key 16*kt + l%16, dims 32*ks + 8*(l/16)
    uint4 kr[KTW][KS];
    int32_t kt_tok[KTW];
#pragma unroll
    for (int u = 0; u < KTW; u++) {
      HIPSA_TOKEN(16 * (wave + 4 * u) + (lane & 15), kt_tok[u]);
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        kr[u][ks] = Vec<E>::raw(Kp + (int64_t)(kt_tok[u] >= 0 ? kt_tok[u] : 0) * D + 32 * ks + 8 * (lane >> 4));
    }
#pragma unroll
    for (int u = 0; u < KTW; u++) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ks++)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[ks]), as_bf16x8(kr[u][ks]), acc, 0, 0, 0);
      // acc[r]: head 4*(lane/16) + r, key 16*(wave + 4u) + lane%16
      const int j = 16 * (wave + 4 * u) + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int h = 4 * (lane >> 4) + r;
        if (h < s.G) pr[h][j] = kt_tok[u] >= 0 ? acc[r] * a.scale : -INFINITY;
      }
    }
  } else {
    // fp32: K rows with the same mapping as V, VALU dot products
    float qv[GMAX][VEC];
    {
      uint4 r[GMAX];
#pragma unroll
      for (int h = 0; h < GMAX; h++) r[h] = Vec<E>::raw(qbase + (int64_t)min(h, s.G - 1) * Tq * D + cs * VEC);
#pragma unroll
      for (int h = 0; h < GMAX; h++) Vec<E>::widen(r[h], h < s.G, qv[h]);
    }
    uint4 kraw[RPT];
#pragma unroll
    for (int u = 0; u < RPT; u++) kraw[u] = Vec<E>::raw(Kp + (int64_t)(vt[u] >= 0 ? vt[u] : 0) * D + cs * VEC);
#pragma unroll
    for (int u = 0; u < RPT; u++) {
      float kv[VEC];
      Vec<E>::widen(kraw[u], vt[u] >= 0, kv);
      const int j = u * RPP + rg;
#pragma unroll
      for (int h = 0; h < GMAX; h++) {
        float p = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; e++) p = fmaf(qv[h][e], kv[e], p);
        p = group_sum<TPR>(p);
        if (cs == 0 && h < s.G) pr[h][j] = vt[u] >= 0 ? p * a.scale : -INFINITY;
      }
    }
  }
#undef HIPSA_TOKEN
  __syncthreads();

  // per-head max and exponentials: one wave per head, TOK/64 slots per lane
  for (int h = wave; h < s.G; h += 4) {
    float x[TOK / 64];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < TOK / 64; u++) {
      x[u] = pr[h][lane + 64 * u];
      m = fmaxf(m, x[u]);
    }
    m = wave_max(m);
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < TOK / 64; u++) {
      const float e = x[u] == -INFINITY ? 0.f : __expf(x[u] - m);
      pr[h][lane + 64 * u] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) { stat_m[h] = m; stat_l[h] = l; }
  }
  __syncthreads();

  // P.V, HG heads per LDS reduction pass; partial results to the workspace
  float *mine = a.ws + ((int64_t)(prob * S + split) * s.G) * (D + 2);
  for (int h0 = 0; h0 < s.G; h0 += HG) {
    float acc[HG][VEC];
#pragma unroll
    for (int hh = 0; hh < HG; hh++)
#pragma unroll
      for (int e = 0; e < VEC; e++) acc[hh][e] = 0.f;
#pragma unroll
    for (int u = 0; u < RPT; u++) {
      float vv[VEC];
      Vec<E>::widen(vr[u], vt[u] >= 0, vv);
      const int j = u * RPP + rg;
#pragma unroll
      for (int hh = 0; hh < HG; hh++) {
        const float p = (h0 + hh < s.G) ? pr[h0 + hh][j] : 0.f;
#pragma unroll
        for (int e = 0; e < VEC; e++) acc[hh][e] = fmaf(p, vv[e], acc[hh][e]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < HG; hh++)
#pragma unroll
      for (int e = 0; e < VEC; e++) red[rg][hh][cs * VEC + e] = acc[hh][e];
    __syncthreads();
    for (int o = tid; o < HG * D; o += 256) {
      const int hh = o / D, x = o % D;
      if (h0 + hh >= s.G) continue;
      float sum = 0.f;
#pragma unroll 8
      for (int r = 0; r < RPP; r++) sum += red[r][hh][x];
      float *dst = mine + (int64_t)(h0 + hh) * (D + 2);
      dst[2 + x] = sum;
      if (x == 0) { dst[0] = stat_m[h0 + hh]; dst[1] = stat_l[h0 + hh]; }
    }
    __syncthreads();
  }
}

// Merge the S partials of one (problem, query head): one workgroup of D lanes,
// every load of a batch issued before any is used.
template <typename E, int D>
__global__ __launch_bounds__(128) void attn_decode_combine(AttnArgs a) {
  constexpr int CH = 16;  // partials in flight per lane
  const Shape &s = a.s;
  const int S = a.splits;
  const uint32_t ph = blockIdx.x;
  const uint32_t prob = ph / (uint32_t)s.G;
  const int h = (int)(ph % (uint32_t)s.G);
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int x = threadIdx.x;
  if (x >= D) return;
  const float *ph_ = a.ws + ((int64_t)prob * S * s.G + h) * (int64_t)(D + 2);
  const int64_t sstride = (int64_t)s.G * (D + 2);
  float M = -INFINITY, L = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < S; s0 += CH) {
    float mm[CH], ll[CH], oo[CH];
#pragma unroll
    for (int u = 0; u < CH; u++) {
      const int sp = min(s0 + u, S - 1);
      mm[u] = ph_[sp * sstride];
      ll[u] = ph_[sp * sstride + 1];
      oo[u] = ph_[sp * sstride + 2 + x];
    }
#pragma unroll
    for (int u = 0; u < CH; u++) {
      const float mu = s0 + u < S ? mm[u] : -INFINITY;
      const float Mn = fmaxf(M, mu);
      const float c0 = M == -INFINITY ? 0.f : __expf(M - Mn);
      const float c1 = mu == -INFINITY ? 0.f : __expf(mu - Mn);
      L = L * c0 + ll[u] * c1;
      acc = acc * c0 + oo[u] * c1;
      M = Mn;
    }
  }
  const float v = L > 0.f ? acc / L : 0.f;
  E *out = reinterpret_cast<E *>(a.out) + ((int64_t)(b * s.Hq + g * s.G + h) * Tq + i) * D;
  store_elem(out + x, v);
}

// tokens per split workgroup: the largest of 256, 128, 64 that still gives
// >= 512 workgroups (64 when none does); fp32 at d=128 stops at 128
template <typename E, int D>
int tokens_per_split(const Shape &s) {
  const int64_t total = (int64_t)s.Kb * s.bk;
  const int maxtok = (std::is_same<E, float>::value && D == 128) ? 128 : 256;
  for (int tok = maxtok; tok > 64; tok >>= 1)
    if (s.problems * ((total + tok - 1) / tok) >= 512) return tok;
  return 64;
}

int tokens_for(const Shape &s) {
  if (s.dtype == HIPSA_BF16)
    return s.d == 64 ? tokens_per_split<uint16_t, 64>(s) : tokens_per_split<uint16_t, 128>(s);
  return s.d == 64 ? tokens_per_split<float, 64>(s) : tokens_per_split<float, 128>(s);
}

template <typename E, int D, int GMAX>
void launch_t(const AttnArgs &a, hipStream_t st, int tok) {
  const dim3 grid((unsigned)(a.s.problems * a.splits)), block(256);
  if (tok == 256) {
    if constexpr (!(std::is_same<E, float>::value && D == 128))
      hipLaunchKernelGGL((attn_decode_kernel<E, D, GMAX, 256>), grid, block, 0, st, a);
  } else if (tok == 128) {
    hipLaunchKernelGGL((attn_decode_kernel<E, D, GMAX, 128>), grid, block, 0, st, a);
  } else {
    hipLaunchKernelGGL((attn_decode_kernel<E, D, GMAX, 64>), grid, block, 0, st, a);
  }
}

template <typename E, int D>
hipError_t launch_d(const AttnArgs &a, hipStream_t st) {
  const int G = a.s.G, tok = tokens_per_split<E, D>(a.s);
  if (G <= 1) launch_t<E, D, 1>(a, st, tok);
  else if (G <= 2) launch_t<E, D, 2>(a, st, tok);
  else if (G <= 4) launch_t<E, D, 4>(a, st, tok);
  else if (G <= 8) launch_t<E, D, 8>(a, st, tok);
  else launch_t<E, D, 16>(a, st, tok);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_decode_combine<E, D>), dim3((unsigned)(a.s.problems * G)), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace

int32_t attn_decode_splits(const Shape &s) {
  const int tok = tokens_for(s);
  return (int32_t)(((int64_t)s.Kb * s.bk + tok - 1) / tok);
}

size_t attn_decode_workspace(const Shape &s) {
  return (size_t)s.problems * attn_decode_splits(s) * s.G * (s.d + 2) * sizeof(float);
}

hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t st) {
  if (a.s.dtype == HIPSA_BF16)
    return a.s.d == 64 ? launch_d<uint16_t, 64>(a, st) : launch_d<uint16_t, 128>(a, st);
  return a.s.d == 64 ? launch_d<float, 64>(a, st) : launch_d<float, 128>(a, st);
}

}  // namespace hipsa
