// One split workgroup of block-sparse decode attention on the matrix cores
// (bf16 query; bf16 or fp8 E5M2 K/V), shared by the decode attention kernel
// and the one-launch decode step.
//
// Input contract: per (b, kv head, row) a list of key-block ids and its
// length nnz (rebuttal page "A Training-free Sub-quadratic Cost Transformer
// Model Serving Framework With Hierarchically Pruned Attention", reviewer
// NLBm, W2).  Exact softmax over the listed blocks' visible tokens.
#pragma once

#include "hipsa_internal.h"

namespace hipsa {

// Split `split` of problem `prob` over the row's key sequence (dense part,
// then `list`[0..*nnz), in global memory or LDS), bf16 query, bf16 or fp8
// (E5M2) K/V.  Per wave, TPW = TOK/4 token slots:
//   * the query heads of the group are the A operand of
//     v_mfma_f32_16x16x32_bf16 (lane l holds head l%16, zero past the
//     group) and the wave's K rows, 16 per tile, the B operand (lane l holds
//     slot 16u + l%16), so the logits of (head, slot) land in the
//     accumulators: lane l, register r -> head 4*(l/16) + r, slot 16u + l%16;
//   * softmax statistics are taken in that layout (DPP within 16-lane rows)
//     and the probabilities go to a per-wave LDS table;
//   * P.V runs with lanes owning output dimensions: a lane loads EPL
//     consecutive elements of a V row (4 bytes, or 2 for fp8 at d = 64), the
//     probabilities are LDS broadcasts, and each lane accumulates its
//     dimensions over every slot of the wave; when a row takes half a wave
//     the two halves take alternate rows and are summed once at the end.
//   * WIDE: a lane loads 8 consecutive elements (16 bytes of bf16, 8 of
//     fp8), so one wave-wide load covers RPV = 4 rows (d = 128) or 8 (d = 64)
//     and each row group of lanes takes every RPV-th slot; the probabilities
//     of a row group's slots are contiguous in the LDS table (vector reads),
//     and the row groups are summed once at the end.  Fewer, wider loads
//     pay when the grid is large (several workgroups per CU); on a grid of
//     about two workgroups per CU the narrow form measured faster.
// fp8 K rows are loaded as 8-byte slices and widened to bf16 operands in
// registers (exact: every E5M2 value is a bf16 value).
// Query loads are issued first: loads complete in order, so the first
// matrix op then waits for the query and its K rows, not for the V rows
// issued after them.
template <typename KE, int D, int GMAX, int TOK, bool PAGED, bool WIDE, bool COHERENT = false>
__device__ __forceinline__ void attend_split(const AttnArgs &a, uint32_t prob, uint32_t split,
                                             const int32_t *list, const int32_t *nnz) {
  constexpr int KS = D / 32;            // MFMA k-steps over the head dim
  constexpr int TPW = TOK / 4;          // token slots per wave
  constexpr int NT = TPW / 16;          // 16-slot tiles per wave
  constexpr int EPL = WIDE ? 8 : (sizeof(KE) == 1 && D == 128) ? 4 : 2;  // V elements per lane
  constexpr int LPV = D / EPL < 64 ? D / EPL : 64;  // lanes per V row
  constexpr int RPV = 64 / LPV;         // V rows per wave-wide load
  constexpr int NV = TPW / RPV;         // V loads per lane
  static_assert(NT >= 1 && TPW % RPV == 0 && NV >= 1 && (WIDE || RPV <= 2), "split too small");
  const Shape &s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t S = (uint32_t)a.splits;
  const uint32_t Tq = (uint32_t)s.Tq, Hkv = (uint32_t)s.Hkv;
  const uint32_t i = prob % Tq, g = (prob / Tq) % Hkv, b = prob / (Tq * Hkv);
  const int32_t Tp = s.causal ? (int32_t)(s.T - s.Tq + i + 1) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t cnt = min(max(*nnz, 0), s.Kb);
  const int base_blk = (int)split * (TOK >> s.bk_shift);
  const Dense dn(s, Np);

  __shared__ __align__(16) float pw[4][GMAX][TPW];
  __shared__ float wm[4][GMAX], wl[4][GMAX];
  __shared__ __align__(16) float wo[4][GMAX][D];

  const int64_t kvoff = PAGED ? 0 : (int64_t)(b * Hkv + g) * s.T_cap * D;
  const KE *Kp = reinterpret_cast<const KE *>(a.K);
  const KE *Vp = reinterpret_cast<const KE *>(a.V);
  const int ps = a.pg.ps_shift;
  // element offset of the K/V row of position t (>= 0) in page pg (paged)
  auto row_of = [&](int32_t t, int32_t pg) -> int64_t {
    if constexpr (PAGED) return paged_row(pg, g, Hkv, t, ps) * D;
    else return kvoff + (int64_t)t * D;
  };
  const uint16_t *qbase = reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)(b * s.Hq + g * s.G) * Tq + i) * D;

  // Token of slot lane % TPW of this wave (row of K/V), or -1 when the slot is
  // past the list, its block id is out of range or the token is past the
  // causal limit.  Such slots read row 0 and are masked, so every load is
  // unconditional.  Other lanes' slots come by shuffle (readlane when the
  // row is the same for the whole wave).
  int32_t tk_lane;
  {
    const int j = wave * TPW + lane % TPW;
    const int32_t blk = entry_block(base_blk + (j >> s.bk_shift), list, cnt, s, Np, dn);
    const bool ok = blk >= 0;
    const int32_t t = ((ok ? blk : 0) << s.bk_shift) + (j & (s.bk - 1));
    tk_lane = (ok && t < Tp) ? t : -1;
  }
  int32_t pg_lane = 0;  // paged: page of the slot's token (of position 0 for a masked slot)
  if constexpr (PAGED) pg_lane = page_at(a.pg, b, (tk_lane >= 0 ? tk_lane : 0) >> ps);

  uint4 qa[KS];
  {
    const int h = lane & 15;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      const uint4 r = *reinterpret_cast<const uint4 *>(qbase + (int64_t)min(h, s.G - 1) * Tq * D + 32 * ks + 8 * (lane >> 4));
      qa[ks] = h < s.G ? r : make_uint4(0, 0, 0, 0);
    }
  }
  int32_t kt[NT];
  typename Kv8<KE>::raw_t kr[NT][KS];
#pragma unroll
  for (int u = 0; u < NT; u++) {
    kt[u] = __shfl(tk_lane, 16 * u + (lane & 15), 64);
    const int32_t kpg = PAGED ? __shfl(pg_lane, 16 * u + (lane & 15), 64) : 0;
    const int64_t krow = row_of(kt[u] >= 0 ? kt[u] : 0, kpg);
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
      kr[u][ks] = Kv8<KE>::raw(Kp + krow + 32 * ks + 8 * (lane >> 4));
  }
  int32_t vt[NV];
  typename KvN<KE, EPL>::raw_t vr[NV];
#pragma unroll
  for (int v = 0; v < NV; v++) {
    // WIDE: row group lane / LPV takes slots RPV * v + lane / LPV
    vt[v] = RPV == 1 ? __builtin_amdgcn_readlane(tk_lane, v) : __shfl(tk_lane, RPV * v + lane / LPV, 64);
    int32_t vpg = 0;
    if constexpr (PAGED)
      vpg = RPV == 1 ? __builtin_amdgcn_readlane(pg_lane, v) : __shfl(pg_lane, RPV * v + lane / LPV, 64);
    vr[v] = KvN<KE, EPL>::raw(Vp + row_of(vt[v] >= 0 ? vt[v] : 0, vpg) + EPL * (lane % LPV));
  }

  // logits on the matrix cores, softmax statistics per head in the
  // accumulator layout, probabilities to the wave's LDS table
  f32x4_t acc[NT];
#pragma unroll
  for (int u = 0; u < NT; u++) {
    acc[u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[ks]), as_bf16x8(Kv8<KE>::bf16(kr[u][ks])), acc[u], 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; r++) {
    const int h = 4 * (lane >> 4) + r;
    float sc[NT];
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < NT; u++) {
      sc[u] = kt[u] >= 0 ? acc[u][r] * a.scale : -INFINITY;
      m = fmaxf(m, sc[u]);
    }
    m = fmaxf(m, dpp_mov<kDppXor1>(m));
    m = fmaxf(m, dpp_mov<kDppXor2>(m));
    m = fmaxf(m, dpp_mov<kDppHalfMirror>(m));
    m = fmaxf(m, dpp_mov<kDppMirror>(m));
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < NT; u++) {
      const float e = sc[u] == -INFINITY ? 0.f : __expf(sc[u] - m);
      l += e;
      const int sl = 16 * u + (lane & 15);
      // WIDE: slot sl at (sl % RPV) * NV + sl / RPV, a row group's slots contiguous
      if (h < GMAX) pw[wave][h][WIDE ? (sl % RPV) * NV + sl / RPV : sl] = e;
    }
    l = group_sum<16>(l);
    if ((lane & 15) == 0 && h < s.G) { wm[wave][h] = m; wl[wave][h] = l; }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // P.V: lane owns dimensions EPL*(lane % LPV) .. +EPL-1 over the wave's
  // slots (WIDE: over its row group's slots)
  float o[GMAX][EPL];
#pragma unroll
  for (int h = 0; h < GMAX; h++)
#pragma unroll
    for (int e = 0; e < EPL; e++) o[h][e] = 0.f;
  if constexpr (WIDE) {
    constexpr int C = NV < 4 ? NV : 4;  // slots per probability read
    const int rg = lane / LPV;
#pragma unroll
    for (int v0 = 0; v0 < NV; v0 += C) {
      float pv[GMAX][C];
#pragma unroll
      for (int h = 0; h < GMAX; h++) {
        const float *src = &pw[wave][h][rg * NV + v0];
        if constexpr (C == 4) {
          const float4 t = *reinterpret_cast<const float4 *>(src);
          pv[h][0] = t.x; pv[h][1] = t.y; pv[h][2] = t.z; pv[h][3] = t.w;
        } else if constexpr (C == 2) {
          const float2 t = *reinterpret_cast<const float2 *>(src);
          pv[h][0] = t.x; pv[h][1] = t.y;
        } else {
          pv[h][0] = *src;
        }
      }
#pragma unroll
      for (int c = 0; c < C; c++) {
        float vx[EPL];
        KvN<KE, EPL>::widen(vr[v0 + c], vt[v0 + c] >= 0, vx);
        // every one of the GMAX heads is computed (see below)
#pragma unroll
        for (int h = 0; h < GMAX; h++)
#pragma unroll
          for (int e = 0; e < EPL; e++) o[h][e] = fmaf(pv[h][c], vx[e], o[h][e]);
      }
    }
#pragma unroll
    for (int h = 0; h < GMAX; h++)
#pragma unroll
      for (int e = 0; e < EPL; e++) o[h][e] = across_sum<LPV>(o[h][e]);
  } else {
  constexpr int VPG = 4 / RPV;  // V loads per group of 4 slots
  const int half = lane / LPV;  // RPV = 2: which of the two rows of a load
#pragma unroll
  for (int g4 = 0; g4 < TPW / 4; g4++) {
    // every one of the GMAX heads is computed (heads past the group have
    // finite probabilities and are never stored): a per-head test inside
    // this loop would become a select on every accumulator update
    float4 p4[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; h++) p4[h] = *reinterpret_cast<const float4 *>(&pw[wave][h][4 * g4]);
#pragma unroll
    for (int vv = 0; vv < VPG; vv++) {
      const int v = g4 * VPG + vv;
      float vx[EPL];
      KvN<KE, EPL>::widen(vr[v], vt[v] >= 0, vx);
#pragma unroll
      for (int h = 0; h < GMAX; h++) {
        float pj;
        if (RPV == 1) pj = vv == 0 ? p4[h].x : vv == 1 ? p4[h].y : vv == 2 ? p4[h].z : p4[h].w;
        else pj = vv == 0 ? (half ? p4[h].y : p4[h].x) : (half ? p4[h].w : p4[h].z);
#pragma unroll
        for (int e = 0; e < EPL; e++) o[h][e] = fmaf(pj, vx[e], o[h][e]);
      }
    }
  }
  if (RPV == 2) {  // the two halves of the wave took alternate rows
#pragma unroll
    for (int h = 0; h < GMAX; h++)
#pragma unroll
      for (int e = 0; e < EPL; e++) o[h][e] = xor32_sum(o[h][e]);
  }
  }
  if (lane < LPV) {
#pragma unroll
    for (int h = 0; h < GMAX; h++) {
      if (h >= s.G) continue;
      if constexpr (EPL == 8) {
        *reinterpret_cast<float4 *>(&wo[wave][h][8 * lane]) = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
        *reinterpret_cast<float4 *>(&wo[wave][h][8 * lane + 4]) = make_float4(o[h][4], o[h][5], o[h][6], o[h][7]);
      } else if constexpr (EPL == 4)
        *reinterpret_cast<float4 *>(&wo[wave][h][4 * lane]) = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
      else
        *reinterpret_cast<float2 *>(&wo[wave][h][2 * lane]) = make_float2(o[h][0], o[h][1]);
    }
  }
  __syncthreads();

  // merge the four waves (log-sum-exp weights); partials to the workspace, or
  // with a single split the normalised bf16 output itself (no merge launch)
  float *mine = a.ws + ((int64_t)(prob * S + split) * s.G) * (D + 2);
  for (int oi = tid; oi < s.G * D; oi += 256) {
    const int h = oi / D, x = oi % D;
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
      uint16_t *out = reinterpret_cast<uint16_t *>(a.out) + ((int64_t)(b * s.Hq + g * s.G + h) * Tq + i) * D;
      store_elem(out + x, L > 0.f ? O / L : 0.f);
    } else {
      float *dst = mine + (int64_t)h * (D + 2);
      if constexpr (COHERENT) {  // agent-scope stores: visible to the merging workgroup
        __hip_atomic_store(dst + 2 + x, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (x == 0) {
          __hip_atomic_store(dst, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(dst + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        dst[2 + x] = O;
        if (x == 0) { dst[0] = M; dst[1] = L; }
      }
    }
  }
}

// Merge of the S split partials (max m, sum l, unnormalised output o[D]) of
// one (problem, query head) for the NX output dimensions x[], partial s at
// ph + s * sstride: every load of a batch of CH partials (m and l once, o for
// each x) is issued before any is used; per batch the maximum is a tree and
// the weights are independent exponentials, so the dependent chain is one
// step per batch rather than one per partial.  Each output takes the same
// operations in the same order whatever NX.  load(p) reads one float of the
// workspace.
template <int CH, int NX, typename Load>
__device__ __forceinline__ void merge_partials_nx(const float *ph, int S, int64_t sstride, const int (&x)[NX],
                                                  Load load, float (&res)[NX]) {
  float M = -INFINITY, L = 0.f, acc[NX];
#pragma unroll
  for (int j = 0; j < NX; j++) acc[j] = 0.f;
  int s0 = 0;
  do {
    float mm[CH], ll[CH], oo[CH][NX];
#pragma unroll
    for (int u = 0; u < CH; u++) {
      const int sp = min(s0 + u, S - 1);
      mm[u] = s0 + u < S ? load(ph + sp * sstride) : -INFINITY;
      ll[u] = load(ph + sp * sstride + 1);
#pragma unroll
      for (int j = 0; j < NX; j++) oo[u][j] = load(ph + sp * sstride + 2 + x[j]);
    }
    // batch max as a tree, then independent weights
    float bm[CH];
#pragma unroll
    for (int u = 0; u < CH; u++) bm[u] = mm[u];
#pragma unroll
    for (int w = CH / 2; w >= 1; w /= 2)
#pragma unroll
      for (int u = 0; u < w; u++) bm[u] = fmaxf(bm[u], bm[u + w]);
    const float Mn = fmaxf(M, bm[0]);
    const float c0 = M == -INFINITY ? 0.f : __expf(M - Mn);
    float Lb = 0.f, Ab[NX];
#pragma unroll
    for (int j = 0; j < NX; j++) Ab[j] = 0.f;
#pragma unroll
    for (int u = 0; u < CH; u++) {
      const float c = mm[u] == -INFINITY ? 0.f : __expf(mm[u] - Mn);
      Lb = fmaf(c, ll[u], Lb);
#pragma unroll
      for (int j = 0; j < NX; j++) Ab[j] = fmaf(c, oo[u][j], Ab[j]);
    }
    L = fmaf(L, c0, Lb);
#pragma unroll
    for (int j = 0; j < NX; j++) acc[j] = fmaf(acc[j], c0, Ab[j]);
    M = Mn;
    s0 += CH;
  } while (s0 < S);
#pragma unroll
  for (int j = 0; j < NX; j++) res[j] = L > 0.f ? acc[j] / L : 0.f;
}

template <int CH, typename Load>
__device__ __forceinline__ float merge_partials(const float *ph, int S, int64_t sstride, int x, Load load) {
  const int xs[1] = {x};
  float r[1];
  merge_partials_nx<CH, 1>(ph, S, sstride, xs, load, r);
  return r[0];
}

}  // namespace hipsa
