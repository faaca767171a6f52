// Block-sparse attention for per-row problems (block_q == 1): decode.
//
// Input contract: per (b, kv head, row) a list of key-block ids and its
// length nnz (rebuttal page "A Training-free Sub-quadratic Cost Transformer
// Model Serving Framework With Hierarchically Pruned Attention", reviewer
// NLBm, W2).  Exact softmax over the listed blocks' visible tokens.
//
// Decode attention reads each selected K/V byte once and does ~4 flops per
// byte, so it is bound by HBM bandwidth.  The work of one problem (K_b blocks)
// is split over `splits` workgroups of 64 tokens each (64 / block_k blocks),
// so a step launches problems x splits workgroups, enough to keep every CU's
// memory pipeline full.  Each workgroup:
//   - maps its 64 token slots to key rows (an invalid slot gets -inf);
//   - loads its K and V rows with 16-byte coalesced loads, d/VEC lanes per
//     row, all rows issued before any arithmetic so the loads overlap;
//   - forms the G x 64 logits with cross-lane adds, takes the per-head max and
//     exponentials with wave reductions, accumulates P.V per lane and reduces
//     the row groups through LDS;
//   - writes (max, sum, unnormalised output) per head to the workspace.
// A second small kernel merges the splits of each (problem, head) with the
// usual log-sum-exp rescaling and writes the output in the element type.
#include "hipsa_internal.h"

namespace hipsa {
namespace {

constexpr int kTok = 64;  // token slots per split workgroup

template <typename E, int D, int GMAX>
__global__ __launch_bounds__(256) void attn_decode_split(AttnArgs a) {
  constexpr int VEC = Vec<E>::N;
  constexpr int TPR = D / VEC;            // lanes per row
  constexpr int RPP = 256 / TPR;          // rows per pass
  constexpr int RPT = kTok / RPP;         // rows per lane
  constexpr int HG = GMAX < 4 ? GMAX : 4; // heads reduced per LDS pass
  const Shape &s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = tid / TPR, cs = tid % TPR;
  const int S = a.splits;
  const uint32_t split = blockIdx.x % (uint32_t)S;
  const uint32_t prob = blockIdx.x / (uint32_t)S;
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int32_t Tp = s.causal ? (int32_t)(s.T - s.Tq + i + 1) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t *list = a.indices + (int64_t)prob * s.Kb;
  const int bps = kTok >> s.bk_shift;  // blocks per split

  __shared__ int32_t tok[kTok];
  __shared__ float pr[GMAX][kTok];
  __shared__ float red[RPP][HG][D];
  __shared__ float stat_m[GMAX], stat_l[GMAX];

  // Issue the independent loads together: this lane's query slices, the
  // count and the block id (one memory round trip instead of three).
  float qv[GMAX][VEC];
  {
    const E *qbase =
        reinterpret_cast<const E *>(a.q) + ((int64_t)(b * s.Hq + g * s.G) * Tq + i) * D;
    uint4 r[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; h++)
      r[h] = Vec<E>::raw(qbase + (int64_t)min(h, s.G - 1) * Tq * D + cs * VEC);
#pragma unroll
    for (int h = 0; h < GMAX; h++) Vec<E>::widen(r[h], h < s.G, qv[h]);
  }
  if (tid < kTok) {
    const int n = split * bps + (tid >> s.bk_shift);
    const int32_t cnt = a.nnz[prob];
    const int32_t blk = list[n < s.Kb ? n : 0];
    const bool okb = n < min(max(cnt, 0), s.Kb) && blk >= 0 && blk < Np;
    const int32_t tt = okb ? (blk << s.bk_shift) + (tid & (s.bk - 1)) : 0;
    tok[tid] = (okb && tt < Tp) ? tt : -1;
  }
  __syncthreads();

  const int64_t kvoff = (int64_t)(b * Hkv + g) * s.T_cap * D;
  const E *Kp = reinterpret_cast<const E *>(a.K) + kvoff;
  const E *Vp = reinterpret_cast<const E *>(a.V) + kvoff;
  float kv[RPT][VEC], vv[RPT][VEC];
  {
    uint4 rk[RPT], rv[RPT];
    bool ok[RPT];
#pragma unroll
    for (int u = 0; u < RPT; u++) {  // all K and V loads in flight together
      const int32_t t = tok[u * RPP + rg];
      ok[u] = t >= 0;
      const int64_t row = (int64_t)(ok[u] ? t : 0) * D + cs * VEC;
      rk[u] = Vec<E>::raw(Kp + row);
      rv[u] = Vec<E>::raw(Vp + row);
    }
#pragma unroll
    for (int u = 0; u < RPT; u++) {
      Vec<E>::widen(rk[u], ok[u], kv[u]);
      Vec<E>::widen(rv[u], ok[u], vv[u]);
    }
  }

  // logits
#pragma unroll
  for (int u = 0; u < RPT; u++) {
    const int j = u * RPP + rg;
    const bool ok = tok[j] >= 0;
#pragma unroll
    for (int h = 0; h < GMAX; h++) {
      float p = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; e++) p = fmaf(qv[h][e], kv[u][e], p);
      p = group_sum<TPR>(p);
      if (cs == 0 && h < s.G) pr[h][j] = ok ? p * a.scale : -INFINITY;
    }
  }
  __syncthreads();

  // per-head max and exponentials (one wave per head, lane = token slot)
  for (int h = wave; h < s.G; h += 4) {
    const float x = pr[h][lane];
    const float m = wave_max(x);
    const float e = (x == -INFINITY) ? 0.f : __expf(x - m);
    const float l = wave_sum(e);
    pr[h][lane] = e;
    if (lane == 0) { stat_m[h] = m; stat_l[h] = l; }
  }
  __syncthreads();

  // P.V, HG heads per LDS reduction pass
  float *ws = a.ws + ((int64_t)(prob * S + split) * s.G) * (D + 2);
  for (int h0 = 0; h0 < s.G; h0 += HG) {
    float acc[HG][VEC];
#pragma unroll
    for (int hh = 0; hh < HG; hh++)
#pragma unroll
      for (int e = 0; e < VEC; e++) acc[hh][e] = 0.f;
#pragma unroll
    for (int u = 0; u < RPT; u++) {
      const int j = u * RPP + rg;
#pragma unroll
      for (int hh = 0; hh < HG; hh++) {
        const float p = (h0 + hh < s.G) ? pr[h0 + hh][j] : 0.f;
#pragma unroll
        for (int e = 0; e < VEC; e++) acc[hh][e] = fmaf(p, vv[u][e], acc[hh][e]);
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
#pragma unroll 4
      for (int r = 0; r < RPP; r++) sum += red[r][hh][x];
      float *dst = ws + (int64_t)(h0 + hh) * (D + 2);
      dst[2 + x] = sum;
      if (x == 0) { dst[0] = stat_m[h0 + hh]; dst[1] = stat_l[h0 + hh]; }
    }
    __syncthreads();
  }
}

// Merge the splits of one (problem, query head): one workgroup of D lanes.
// All loads of a phase are issued before any is used, so the merge costs two
// memory round trips whatever the split count.
template <typename E, int D>
__global__ __launch_bounds__(128) void attn_decode_combine(AttnArgs a) {
  constexpr int CH = 16;  // loads in flight per lane
  const Shape &s = a.s;
  const int S = a.splits;
  const uint32_t ph = blockIdx.x;
  const uint32_t prob = ph / (uint32_t)s.G;
  const int h = (int)(ph % (uint32_t)s.G);
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int x = threadIdx.x;
  const float *ws = a.ws + ((int64_t)prob * S * s.G + h) * (int64_t)(D + 2);
  const int64_t stride = (int64_t)s.G * (D + 2);
  __shared__ float wgt[kMaxKb * 64 / kTok];  // per-split weight exp(m_s - M), then l_s * weight
  __shared__ float red[128];

  // phase 1: every split's running max and sum
  float M = -INFINITY;
  for (int sp = x; sp < S; sp += 128) M = fmaxf(M, ws[sp * stride]);
  red[x] = M;
  __syncthreads();
  for (int w = 64; w >= 1; w >>= 1) {
    if (x < w) red[x] = fmaxf(red[x], red[x + w]);
    __syncthreads();
  }
  M = red[0];
  __syncthreads();
  float L = 0.f;
  for (int sp = x; sp < S; sp += 128) {
    const float m = ws[sp * stride];
    const float w = (m == -INFINITY) ? 0.f : __expf(m - M);
    wgt[sp] = w;
    L = fmaf(w, ws[sp * stride + 1], L);
  }
  red[x] = L;
  __syncthreads();
  for (int w = 64; w >= 1; w >>= 1) {
    if (x < w) red[x] += red[x + w];
    __syncthreads();
  }
  L = red[0];
  if (x >= D) return;

  // phase 2: weighted sum of the unnormalised outputs, CH splits in flight
  float acc = 0.f;
  for (int sp0 = 0; sp0 < S; sp0 += CH) {
    float o[CH];
#pragma unroll
    for (int u = 0; u < CH; u++) o[u] = sp0 + u < S ? ws[(sp0 + u) * stride + 2 + x] : 0.f;
#pragma unroll
    for (int u = 0; u < CH; u++)
      if (sp0 + u < S) acc = fmaf(wgt[sp0 + u], o[u], acc);
  }
  const float v = L > 0.f ? acc / L : 0.f;
  E *out = reinterpret_cast<E *>(a.out) + ((int64_t)(b * s.Hq + g * s.G + h) * Tq + i) * D;
  store_elem(out + x, v);
}

template <typename E, int D>
hipError_t launch_d(const AttnArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)(a.s.problems * a.splits)), block(256);
  const int G = a.s.G;
  if (G <= 1) hipLaunchKernelGGL((attn_decode_split<E, D, 1>), grid, block, 0, st, a);
  else if (G <= 2) hipLaunchKernelGGL((attn_decode_split<E, D, 2>), grid, block, 0, st, a);
  else if (G <= 4) hipLaunchKernelGGL((attn_decode_split<E, D, 4>), grid, block, 0, st, a);
  else if (G <= 8) hipLaunchKernelGGL((attn_decode_split<E, D, 8>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attn_decode_split<E, D, 16>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_decode_combine<E, D>), dim3((unsigned)(a.s.problems * G)), dim3(128), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace

int32_t attn_decode_splits(const Shape &s) { return (s.Kb * s.bk + kTok - 1) / kTok; }

size_t attn_decode_workspace(const Shape &s) {
  return (size_t)s.problems * attn_decode_splits(s) * s.G * (s.d + 2) * sizeof(float);
}

hipError_t launch_attn_decode(const AttnArgs &a, hipStream_t st) {
  if (a.s.dtype == HIPSA_BF16)
    return a.s.d == 64 ? launch_d<uint16_t, 64>(a, st) : launch_d<uint16_t, 128>(a, st);
  return a.s.d == 64 ? launch_d<float, 64>(a, st) : launch_d<float, 128>(a, st);
}

}  // namespace hipsa
