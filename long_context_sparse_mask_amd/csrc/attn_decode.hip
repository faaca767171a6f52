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

// Split workgroup on the matrix cores for a bf16 query, with bf16 or fp8
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
template <typename KE, int D, int GMAX, int TOK, bool PAGED, bool WIDE>
__global__ __launch_bounds__(256) void attn_decode_mfma(AttnArgs a) {
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
      dst[2 + x] = O;
      if (x == 0) { dst[0] = M; dst[1] = L; }
    }
  }
}

// Merge the S partials of one (problem, query head): one workgroup of D lanes,
// every load of a batch issued before any is used.  Per batch of CH partials
// the maximum is a tree and the weights are independent exponentials, so the
// dependent chain is one step per batch rather than one per partial.  CH is
// 16 or 32, chosen so that up to 32 partials take one memory round trip.
// The merge takes its arguments one by one, 36 bytes in all: the library is
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
  float M = -INFINITY, L = 0.f, acc = 0.f;
  int s0 = 0;
  do {  // S >= 2: launched only for several splits
    float mm[CH], ll[CH], oo[CH];
#pragma unroll
    for (int u = 0; u < CH; u++) {
      const int sp = min(s0 + u, S - 1);
      mm[u] = s0 + u < S ? ph_[sp * sstride] : -INFINITY;
      ll[u] = ph_[sp * sstride + 1];
      oo[u] = ph_[sp * sstride + 2 + x];
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
    float Lb = 0.f, Ab = 0.f;
#pragma unroll
    for (int u = 0; u < CH; u++) {
      const float c = mm[u] == -INFINITY ? 0.f : __expf(mm[u] - Mn);
      Lb = fmaf(c, ll[u], Lb);
      Ab = fmaf(c, oo[u], Ab);
    }
    L = fmaf(L, c0, Lb);
    acc = fmaf(acc, c0, Ab);
    M = Mn;
    s0 += CH;
  } while (s0 < S);
  const float v = L > 0.f ? acc / L : 0.f;
  store_elem(out + x, v);
}

// Tokens per split workgroup: 128 or 64, the larger when it still gives
// >= 512 workgroups, or when it covers a row's whole key sequence (one split:
// the split workgroup then writes the output and no merge is launched).  64
// for fp32 at d = 128 (a lane's K and V rows must fit in registers) and for
// groups of more than 8 query heads (the per-head probabilities and outputs
// of a lane must fit); a bf16 wave also has at most 63 loads in flight, which
// caps its slots at 32.
template <typename E, int D>
constexpr int max_tokens() { return (std::is_same<E, float>::value && D == 128) ? 64 : 128; }

template <typename E, int D>
int tokens_per_split(const Shape &s) {
  const int64_t total = entry_tokens(s);
  if (max_tokens<E, D>() >= 128 && s.G <= 8 && (total <= 128 || s.problems * ((total + 127) / 128) >= 512))
    return 128;
  return 64;
}

int tokens_for(const Shape &s) {
  if (s.dtype != HIPSA_F32)  // bf16 query: the matrix-core kernel, for either K/V type
    return s.d == 64 ? tokens_per_split<uint16_t, 64>(s) : tokens_per_split<uint16_t, 128>(s);
  return s.d == 64 ? tokens_per_split<float, 64>(s) : tokens_per_split<float, 128>(s);
}

// E: query / output element type; KE: K/V element type (E itself, or E5M2
// codes under a bf16 query).
// Split workgroups from which the bf16 kernel reads V rows 16 bytes per lane
// (about four per CU and more); below, 2-4 bytes per lane.
constexpr int64_t kWideGrid = 1024;

template <typename KE, int D, int GMAX, bool PAGED, bool WIDE>
void launch_mfma(const AttnArgs &a, dim3 grid, hipStream_t st, int tok) {
  if (GMAX <= 8 && tok == 128) hipLaunchKernelGGL((attn_decode_mfma<KE, D, (GMAX <= 8 ? GMAX : 8), 128, PAGED, WIDE>), grid, dim3(256), 0, st, a);
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
  if (e != hipSuccess || a.splits == 1) return e;  // one split wrote the output itself
  const dim3 cgrid((unsigned)(a.s.problems * G));
  const int32_t Tq = (int32_t)a.s.Tq, Hkv = (int32_t)a.s.Hkv, Hq = (int32_t)a.s.Hq;
  if (a.splits <= 16)
    hipLaunchKernelGGL((attn_decode_combine<E, D, 16>), cgrid, dim3(D), 0, st, a.ws, a.out, a.splits, a.s.G, Tq, Hkv, Hq);
  else
    hipLaunchKernelGGL((attn_decode_combine<E, D, 32>), cgrid, dim3(D), 0, st, a.ws, a.out, a.splits, a.s.G, Tq, Hkv, Hq);
  return hipGetLastError();
}

}  // namespace

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
