// Block-sparse attention for query blocks of 64 rows (chunked prefill, bf16).
//
// Input contract: per (b, kv head, query block) a list of key-block ids and
// its length nnz (rebuttal page "A Training-free Sub-quadratic Cost
// Transformer Model Serving Framework With Hierarchically Pruned Attention",
// reviewer NLBm, W2).  Exact causal softmax over the listed blocks' tokens.
//
// Prefill attention is a dense contraction per selected key tile, so it runs
// on the matrix cores.  One workgroup of 4 wave64s serves one (b, kv head,
// query block) and four query heads of the group (one per wave), so every
// K/V tile fetched from HBM feeds four heads.  Per tile of 64 keys:
//   - all lanes stage K (row-major, padded rows) and V (transposed to d-major
//     so that an MFMA operand can take 8 consecutive keys of one d) in LDS;
//     the global loads of the next tile are issued before this tile's math;
//   - each wave forms S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (keys down
//     the rows, its 64 queries across the columns), so a query's scores sit
//     in one lane pair and the online-softmax max and sum need no more than
//     one cross-half exchange;
//   - P^T is rounded to bf16 in registers and used directly as the B operand
//     of O^T += V^T . P^T: the register order of S^T defines the key order of
//     the k-steps, and V^T is read from LDS in that same order.
#include "hipsa_internal.h"

namespace hipsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__global__ __launch_bounds__(256) void attn_prefill_kernel(AttnArgs a) {
  constexpr int KS = D / 16;   // k-steps of S^T over the head dim
  constexpr int DT = D / 32;   // 32-row tiles of O^T
  constexpr int BQ = 64, KT = 64;
  constexpr int KPAD = D + 8;  // K tile row stride (elements)
  constexpr int VPAD = KT + 8; // V^T row stride (elements)
  constexpr int TPR = D / 8;   // loader: lanes per K row
  constexpr int RPP = 256 / TPR;
  constexpr int KP = KT / RPP; // loader: K rows per lane
  constexpr int VP = D / 32;   // loader: V chunks per lane
  const Shape &s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;

  const uint32_t hchunks = (uint32_t)(s.G + 3) / 4;
  const uint32_t prob = blockIdx.x / hchunks, hc = blockIdx.x % hchunks;
  const uint32_t nqb = (uint32_t)s.nqb, Hkv = (uint32_t)s.Hkv, Tq = (uint32_t)s.Tq;
  const uint32_t qb = prob % nqb, g = (prob / nqb) % Hkv, b = prob / (nqb * Hkv);
  const int h = (int)hc * 4 + wave;
  const bool active = h < s.G;  // uniform per wave
  const int32_t r0 = (int32_t)qb * BQ;
  const int32_t r1 = min(r0 + BQ, (int32_t)Tq);
  const int32_t pos0 = (int32_t)(s.T - s.Tq) + r0;
  const int32_t Tp = s.causal ? pos0 + (r1 - r0) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t cnt = min(max(a.nnz[prob], 0), s.Kb);
  const int bpt = KT >> s.bk_shift;  // key blocks per tile
  const int ntiles = (cnt + bpt - 1) / bpt;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VPAD];
  __shared__ __attribute__((aligned(16))) int32_t tok[KT];
  __shared__ int32_t lst[kMaxKb];

  const int32_t *list = a.indices + (int64_t)prob * s.Kb;
  for (int j = tid; j < cnt; j += 256) lst[j] = list[j];

  const int64_t kvoff = (int64_t)(b * Hkv + g) * s.T_cap * D;
  const uint16_t *Kg = reinterpret_cast<const uint16_t *>(a.K) + kvoff;
  const uint16_t *Vg = reinterpret_cast<const uint16_t *>(a.V) + kvoff;
  const int hq = min(h, s.G - 1);
  const uint16_t *Qg = reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)(b * s.Hq + g * s.G + hq) * Tq + r0) * D;

  // B operand of S^T: Q[query qt*32 + col][16ks + 8*half .. +7]
  uint4 qf[2][KS];
#pragma unroll
  for (int qt = 0; qt < 2; qt++) {
    const int row = min(qt * 32 + col, r1 - r0 - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
      qf[qt][ks] = *reinterpret_cast<const uint4 *>(Qg + (int64_t)row * D + 16 * ks + 8 * half);
  }
  __syncthreads();  // lst ready

  auto token = [&](int tl, int j) -> int32_t {
    const int n = tl * bpt + (j >> s.bk_shift);
    if (n >= cnt) return -1;
    const int32_t blk = lst[n];
    if (blk < 0 || blk >= Np) return -1;
    const int32_t t = (blk << s.bk_shift) + (j & (s.bk - 1));
    return t < Tp ? t : -1;
  };

  uint4 kreg[KP], vreg[VP];
  int32_t vkey_tok = 0;
  auto gload = [&](int tl) {
#pragma unroll
    for (int u = 0; u < KP; u++) {
      const int32_t t = token(tl, u * RPP + tid / TPR);
      kreg[u] = *reinterpret_cast<const uint4 *>(Kg + (int64_t)(t >= 0 ? t : 0) * D + (tid % TPR) * 8);
    }
    vkey_tok = token(tl, tid & 63);
#pragma unroll
    for (int u = 0; u < VP; u++)
      vreg[u] = *reinterpret_cast<const uint4 *>(Vg + (int64_t)(vkey_tok >= 0 ? vkey_tok : 0) * D +
                                                 ((tid >> 6) + 4 * u) * 8);
  };
  auto lstore = [&]() {
#pragma unroll
    for (int u = 0; u < KP; u++)
      *reinterpret_cast<uint4 *>(&Ks[(u * RPP + tid / TPR) * KPAD + (tid % TPR) * 8]) = kreg[u];
    const int key = tid & 63;
#pragma unroll
    for (int u = 0; u < VP; u++) {
      const int d0 = ((tid >> 6) + 4 * u) * 8;
      const uint32_t w[4] = {vreg[u].x, vreg[u].y, vreg[u].z, vreg[u].w};
#pragma unroll
      for (int e = 0; e < 4; e++) {
        Vt[(d0 + 2 * e) * VPAD + key] = (uint16_t)(w[e] & 0xffffu);
        Vt[(d0 + 2 * e + 1) * VPAD + key] = (uint16_t)(w[e] >> 16);
      }
    }
    if (tid < KT) tok[tid] = vkey_tok;
  };

  f32x16_t o[DT][2];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) o[dt][0] = o[dt][1] = f32x16_t{};
  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  const float sl2 = a.scale * kLog2e;

  if (ntiles > 0) {
    gload(0);
    lstore();
  }
  __syncthreads();

  for (int tl = 0; tl < ntiles; tl++) {
    if (tl + 1 < ntiles) gload(tl + 1);
    if (active) {
      // S^T tiles: keys kt*32 + 8*(r/4) + 4*half + r%4, query qt*32 + col
      f32x16_t sacc[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; kt++) {
        uint4 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
          kf[ks] = *reinterpret_cast<const uint4 *>(&Ks[(kt * 32 + col) * KPAD + 16 * ks + 8 * half]);
#pragma unroll
        for (int qt = 0; qt < 2; qt++) {
          f32x16_t acc = {};
#pragma unroll
          for (int ks = 0; ks < KS; ks++)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf[ks]), as_bf16x8(qf[qt][ks]),
                                                          acc, 0, 0, 0);
          sacc[kt][qt] = acc;
        }
      }
      // this lane's key tokens: groups of 4 consecutive keys
      int4 tk[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; kt++)
#pragma unroll
        for (int gq = 0; gq < 4; gq++)
          tk[kt][gq] = *reinterpret_cast<const int4 *>(&tok[kt * 32 + 8 * gq + 4 * half]);

      bf16x8_t pf[2][4];
#pragma unroll
      for (int qt = 0; qt < 2; qt++) {
        const int qq = qt * 32 + col;
        const bool qvalid = r0 + qq < r1;
        const int32_t qpos = pos0 + qq;
        float x[2][16];
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int4 t4 = tk[kt][r >> 2];
            const int32_t t = (r & 3) == 0 ? t4.x : (r & 3) == 1 ? t4.y : (r & 3) == 2 ? t4.z : t4.w;
            const bool ok = qvalid && t >= 0 && (!s.causal || t <= qpos);
            x[kt][r] = ok ? sacc[kt][qt][r] * sl2 : -INFINITY;
            mx = fmaxf(mx, x[kt][r]);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(m[qt], mx);
        const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[qt] - mnew);
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; kt++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const float p = x[kt][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[kt][r] - mnew);
            ps += p;
            pf[qt][kt * 2 + (r >> 3)][r & 7] = (__bf16)p;
          }
        l[qt] = l[qt] * alpha + ps;
        m[qt] = mnew;
#pragma unroll
        for (int dt = 0; dt < DT; dt++) o[dt][qt] *= alpha;
      }
      // O^T += V^T . P^T over 4 k-steps of 16 keys
#pragma unroll
      for (int ks = 0; ks < 4; ks++) {
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
          const uint16_t *vrow = &Vt[(dt * 32 + col) * VPAD + 16 * ks + 4 * half];
          const uint2 lo = *reinterpret_cast<const uint2 *>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 8);
          const bf16x8_t vf = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
          for (int qt = 0; qt < 2; qt++)
            o[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qt][ks], o[dt][qt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
    if (tl + 1 < ntiles) lstore();
    __syncthreads();
  }

  if (!active) return;
  uint16_t *Og = reinterpret_cast<uint16_t *>(a.out) + ((int64_t)(b * s.Hq + g * s.G + h) * Tq + r0) * D;
#pragma unroll
  for (int qt = 0; qt < 2; qt++) {
    const float lt = l[qt] + __shfl_xor(l[qt], 32, 64);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int qq = qt * 32 + col;
    if (r0 + qq >= r1) continue;
#pragma unroll
    for (int dt = 0; dt < DT; dt++)
#pragma unroll
      for (int gq = 0; gq < 4; gq++) {
        const int d = dt * 32 + 8 * gq + 4 * half;
        uint2 w;
        w.x = (uint32_t)f32_to_bf16(o[dt][qt][4 * gq] * inv) |
              ((uint32_t)f32_to_bf16(o[dt][qt][4 * gq + 1] * inv) << 16);
        w.y = (uint32_t)f32_to_bf16(o[dt][qt][4 * gq + 2] * inv) |
              ((uint32_t)f32_to_bf16(o[dt][qt][4 * gq + 3] * inv) << 16);
        *reinterpret_cast<uint2 *>(Og + (int64_t)qq * D + d) = w;
      }
  }
}

}  // namespace

hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t st) {
  const unsigned hchunks = (unsigned)(a.s.G + 3) / 4;
  const dim3 grid((unsigned)(a.s.problems * hchunks)), block(256);
  if (a.s.d == 64) hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace hipsa
