// Block-sparse attention for query blocks of 64 rows (chunked prefill: bf16
// queries, bf16 or fp8 E5M2 K/V).
//
// Input contract: per (b, kv head, query block) a list of key-block ids and
// its length nnz (rebuttal page "A Training-free Sub-quadratic Cost
// Transformer Model Serving Framework With Hierarchically Pruned Attention",
// reviewer NLBm, W2).  Exact causal softmax over the listed blocks' tokens.
//
// Prefill attention is a dense contraction per selected key tile, so it runs
// on the matrix cores (v_mfma_f32_32x32x16_bf16).  One workgroup of 8 wave64s
// serves one (b, kv head, query block) and four query heads of the group:
// wave w takes head w/2 and query rows 32*(w%2) .. +31, so every K/V tile
// fetched from memory feeds four heads, and at ~210 registers per lane two
// waves share each SIMD (one's softmax VALU work overlaps the other's
// MFMAs).  (Giving each wave both query tiles of its head halves the LDS
// operand reads per MFMA, but needs ~500 registers, leaves one wave per SIMD
// and measured slower.)  Per tile of 64 keys:
//   - the workgroup stages K and V row-major in a double-buffered LDS slot
//     (16-byte stores of bf16; fp8 slices are loaded as 8 bytes and widened
//     exactly to bf16 on the way in); the global loads run two tiles ahead
//     (two register sets), so a tile's rows have a whole tile of math to
//     arrive before they are stored to LDS, and one barrier per tile suffices;
//   - each wave forms S^T = K . Q^T (keys down the rows, its 32 queries
//     across the columns), so a query's 64 scores sit in one lane pair and
//     the online-softmax max and sum need one cross-half exchange; the two
//     32-key halves of the tile are independent accumulation chains,
//     interleaved (a dependent 32x32x16 MFMA issues ~45 cycles after its
//     predecessor, an independent one after 32); tiles that need no causal or
//     validity mask (the loader flags them) skip the per-element mask;
//   - P^T is rounded to bf16 in registers and used directly as the B operand
//     of O^T += V^T . P^T.  The register order of S^T fixes which keys form
//     each k-step; the V^T operand for those keys comes from the row-major V
//     tile through gfx950's transposing LDS read (ds_read_b64_tr_b16: within
//     each 16 lanes, lane i receives element i of the four 4-element row
//     pieces the group addresses), so V needs no transposing stores;
//   - the running output is rescaled only when some lane's running max moved.
// The tiles walk a row's key sequence: its dense part (sink and window
// blocks, if any) followed by the listed blocks (entry_block()).  With a
// paged KV cache the page of every entry is read once, beside the list, and
// the loader addresses rows through it (a page holds whole key blocks).
// LDS rows are padded (K: D+8, V: D+32 elements) so that the operand reads
// of a 256-byte LDS pass fall in distinct banks.
#include "hipsa_internal.h"

namespace hipsa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 8.f;  // log2 of the largest weight before the running max moves

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// 4 consecutive 16-bit elements of row-major LDS, transposed across each
// group of 16 lanes (see above).
__device__ inline uint2 lds_read_tr16(const uint16_t *p) {
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t *)(p));
  return __builtin_bit_cast(uint2, v);
}

// Online softmax of one query tile over one key tile.  sacc[kt][r] holds the
// score of key kt*32 + 8*(r/4) + 4*half + r%4 for this lane's query.  The
// scores are copied to plain registers and masked there with selects (a
// variant that masked the accumulator vectors in place, under divergent
// control flow, failed the parity tests; the cause was not isolated).
// Produces P^T in bf16 as MFMA B operands and updates the running max m,
// sum l and output o.
template <int DT>
__device__ inline void online_softmax(const f32x16_t (&sacc)[2], bool masked, const int32_t *tokrow,
                                      bool qvalid, int32_t qpos, bool causal, int half, float sl2,
                                      float &m, float &l, f32x16_t (&o)[DT], bf16x8_t (&pf)[4]) {
  float sv[2][16];
#pragma unroll
  for (int kt = 0; kt < 2; kt++)
#pragma unroll
    for (int r = 0; r < 16; r++) sv[kt][r] = sacc[kt][r];
  if (masked) {  // uniform: some key of this tile is invalid or after a query of the block
#pragma unroll
    for (int kt = 0; kt < 2; kt++)
#pragma unroll
      for (int gq = 0; gq < 4; gq++) {
        const int4 t4 = *reinterpret_cast<const int4 *>(&tokrow[kt * 32 + 8 * gq + 4 * half]);
        const int32_t tt[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
          const bool ok = qvalid & (tt[e] >= 0) & (!causal | (tt[e] <= qpos));
          sv[kt][4 * gq + e] = ok ? sv[kt][4 * gq + e] : -INFINITY;
        }
      }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; kt++)
#pragma unroll
    for (int r = 0; r < 16; r++) mx = fmaxf(mx, sv[kt][r]);
  mx = xor32_max(mx) * sl2;  // scale > 0: max commutes
  // The reference max m moves only when a tile's max exceeds it by more than
  // kLazy (log2 units): until then the weights exp2(s - m) stay <= 2^kLazy,
  // harmless in fp32 and in bf16, and since l and o always share the same m
  // the normalised result is the same, while the rescale of o (DT*16
  // multiplies) runs on few tiles.  m = -inf: any finite max moves it.
  const bool upd = mx > m + kLazy;
  const float mnew = upd ? mx : m;
  const float alpha = upd ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;  // exp2(-inf) = 0
  const float msub = mnew == -INFINITY ? 0.f : mnew;
  float ps4[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: short dependency chains
#pragma unroll
  for (int kt = 0; kt < 2; kt++)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sv[kt][r], sl2, -msub));  // exp2(-inf) = 0
      ps4[r & 3] += p;
      pf[kt * 2 + (r >> 3)][r & 7] = (__bf16)p;
    }
  l = fmaf(l, alpha, (ps4[0] + ps4[1]) + (ps4[2] + ps4[3]));
  m = mnew;
  if (__builtin_amdgcn_ballot_w64(upd)) {
#pragma unroll
    for (int dt = 0; dt < DT; dt++) o[dt] *= alpha;
  }
}

template <typename KE, int D, bool PAGED>
__global__ __launch_bounds__(512) void attn_prefill_kernel(AttnArgs a) {
  constexpr int KS = D / 16;   // k-steps of S^T over the head dim
  constexpr int DT = D / 32;   // 32-row tiles of O^T
  constexpr int BQ = 64, KT = 64;
  constexpr int KPAD = D + 8;  // K tile row stride (elements)
  constexpr int VPAD = D + 32; // V tile row stride (elements)
  constexpr int TPR = D / 8;   // loader: lanes per K row
  constexpr int RPP = 512 / TPR;
  constexpr int KP = KT / RPP; // loader: K rows (and V rows) per lane
  const Shape &s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;

  // query blocks of one KV head share an L2 (their key sets overlap)
  const uint32_t item = xcd_swizzle(blockIdx.x, gridDim.x);
  const uint32_t hchunks = (uint32_t)(s.G + 3) / 4;
  const uint32_t prob = item / hchunks, hc = item % hchunks;
  const uint32_t nqb = (uint32_t)s.nqb, Hkv = (uint32_t)s.Hkv, Tq = (uint32_t)s.Tq;
  const uint32_t qb = prob % nqb, g = (prob / nqb) % Hkv, b = prob / (nqb * Hkv);
  const int h = (int)hc * 4 + (wave >> 1);
  const int qt = wave & 1;
  const bool active = h < s.G;  // uniform per wave
  const int32_t r0 = (int32_t)qb * BQ;
  const int32_t r1 = min(r0 + BQ, (int32_t)Tq);
  const int32_t pos0 = (int32_t)(s.T - s.Tq) + r0;
  const int32_t Tp = s.causal ? pos0 + (r1 - r0) : (int32_t)s.T;
  const int32_t Np = (Tp + s.bk - 1) >> s.bk_shift;
  const int32_t cnt = min(max(a.nnz[prob], 0), s.Kb);
  const Dense dn(s, Np);
  const int nent = s.sink_b + s.window_b + cnt;  // entries of the key sequence
  const int bpt = KT >> s.bk_shift;  // key blocks per tile
  const int ntiles = (nent + bpt - 1) / bpt;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KT * KPAD];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][KT * VPAD];
  __shared__ __attribute__((aligned(16))) int32_t tok[2][KT];
  __shared__ int32_t tmask[2];
  // block of every entry of the tiles (-1: none), and with a paged cache its page
  __shared__ int32_t ent[kMaxKb + kMaxDenseBlocks + 8];
  __shared__ int32_t lpg[PAGED ? kMaxKb + kMaxDenseBlocks : 1];

  const int64_t kvoff = PAGED ? 0 : (int64_t)(b * Hkv + g) * s.T_cap * D;
  const KE *Kg = reinterpret_cast<const KE *>(a.K);
  const KE *Vg = reinterpret_cast<const KE *>(a.V);
  const int hq = min(h, s.G - 1);
  const uint16_t *Qg = reinterpret_cast<const uint16_t *>(a.q) + ((int64_t)(b * s.Hq + g * s.G + hq) * Tq + r0) * D;

  // B operand of S^T: Q[query qt*32 + col][16ks + 8*half .. +7]
  uint4 qf[KS];
  {
    const int row = min(qt * 32 + col, r1 - r0 - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
      qf[ks] = *reinterpret_cast<const uint4 *>(Qg + (int64_t)row * D + 16 * ks + 8 * half);
  }

  // The entries are read up to the largest possible count, not up to nent,
  // so the list loads do not wait for nnz: q, nnz and the list arrive in one
  // memory round trip.  Entries past nent come out as -1.
  const int32_t *list = a.indices + (int64_t)prob * s.Kb;
  const int nmax = ((s.sink_b + s.window_b + s.Kb + bpt - 1) / bpt) * bpt;  // >= ntiles * bpt
  for (int j = tid; j < nmax; j += 512) {
    const int32_t blk = entry_block(j, list, cnt, s, Np, dn);
    ent[j] = blk;
    if constexpr (PAGED)  // a skipped entry: any page will do
      if (j < nent) lpg[j] = page_at(a.pg, b, ((blk >= 0 ? blk : 0) << s.bk_shift) >> a.pg.ps_shift);
  }
  __syncthreads();  // ent ready

  // loader state: this lane's K and V rows of two tiles in flight (sets 0, 1)
  typename Kv8<KE>::raw_t kreg0[KP], vreg0[KP], kreg1[KP], vreg1[KP];
  int32_t vtok0 = -1, vtok1 = -1;
  const int krow0 = tid / TPR, kcol = (tid % TPR) * 8;
  // token of slot J of tile TL, or -1 (branch-free so the loads stay in flight)
#define HIPSA_TOKEN(TL, J, OUT)                                              \
  do {                                                                       \
    const int32_t blk_ = ent[(TL) * bpt + ((J) >> s.bk_shift)];              \
    const bool okb_ = blk_ >= 0;                                             \
    const int32_t t_ = ((okb_ ? blk_ : 0) << s.bk_shift) + ((J) & (s.bk - 1)); \
    OUT = (okb_ && t_ < Tp) ? t_ : -1;                                       \
  } while (0)
  // element offset of the K/V row for slot J of tile TL holding token T (or -1)
  auto row_of = [&](int tl, int j, int32_t t) -> int64_t {
    const int32_t ts = t >= 0 ? t : 0;
    if constexpr (PAGED) {
      const int n = min(tl * bpt + (j >> s.bk_shift), nent - 1);
      return paged_row(lpg[n], g, Hkv, ts, a.pg.ps_shift) * D;
    } else {
      return kvoff + (int64_t)ts * D;
    }
  };
#define HIPSA_GLOAD(TL, KREG, VREG, VTOK)                                                      \
  do {                                                                                         \
    _Pragma("unroll") for (int u = 0; u < KP; u++) {                                           \
      int32_t t;                                                                               \
      HIPSA_TOKEN(TL, u * RPP + krow0, t);                                                     \
      const int64_t off_ = row_of(TL, u * RPP + krow0, t) + kcol;                              \
      KREG[u] = Kv8<KE>::raw(Kg + off_);                                                       \
      VREG[u] = Kv8<KE>::raw(Vg + off_);                                                       \
    }                                                                                          \
    HIPSA_TOKEN(TL, lane, VTOK);                                                               \
  } while (0)
#define HIPSA_LSTORE(BUF, KREG, VREG, VTOK)                                                    \
  do {                                                                                         \
    _Pragma("unroll") for (int u = 0; u < KP; u++) {                                           \
      *reinterpret_cast<uint4 *>(&Ks[BUF][(u * RPP + krow0) * KPAD + kcol]) = Kv8<KE>::bf16(KREG[u]); \
      *reinterpret_cast<uint4 *>(&Vs[BUF][(u * RPP + krow0) * VPAD + kcol]) = Kv8<KE>::bf16(VREG[u]); \
    }                                                                                          \
    if (wave == 0) {                                                                           \
      const int32_t vtok = VTOK;                                                               \
      tok[BUF][lane] = vtok;                                                                   \
      const bool bad_ = vtok < 0 || (s.causal && vtok > pos0);                                 \
      const uint64_t any_ = __builtin_amdgcn_ballot_w64(bad_);                                 \
      if (lane == 0) tmask[BUF] = any_ != 0;                                                   \
    }                                                                                          \
  } while (0)

  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; dt++) o[dt] = f32x16_t{};
  float m = -INFINITY, l = 0.f;
  const float sl2 = a.scale * kLog2e;
  const int qq = qt * 32 + col;  // this lane's query row in the block
  const bool qvalid = r0 + qq < r1;
  const int32_t qpos = pos0 + qq;

  // the math of one tile, held in LDS slot BUF_
  auto tile = [&](const int BUF_) {
    if (active) {
      // S^T: keys kt*32 + 8*(r/4) + 4*half + r%4, queries qt*32 + col; the two
      // key halves are independent accumulation chains, interleaved
      f32x16_t sacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
#pragma unroll
        for (int kt = 0; kt < 2; kt++) {
          const uint4 kf = *reinterpret_cast<const uint4 *>(&Ks[BUF_][(kt * 32 + col) * KPAD + 16 * ks + 8 * half]);
          sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[ks]), sacc[kt], 0, 0, 0);
        }
      }
      bf16x8_t pf[4];
      online_softmax<DT>(sacc, tmask[BUF_] != 0, tok[BUF_], qvalid, qpos, s.causal != 0, half, sl2, m, l, o, pf);
      // O^T += V^T . P^T over 4 k-steps of 16 keys.  Lane l (group g = l/16,
      // L = l%16) names V row 16ks + 4*(g/2) + L/4 (+8 for the upper half of
      // the fragment), columns dt*32 + 16*(g%2) + 4*(L%4) .. +3, and receives
      // MFMA row dt*32 + l%32 for keys 16ks + 4*half (+8) .. +3.
      const int vg = lane >> 4, vl = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 4; ks++)
#pragma unroll
        for (int dt = 0; dt < DT; dt++) {
          const uint16_t *vp = &Vs[BUF_][(16 * ks + 4 * (vg >> 1) + (vl >> 2)) * VPAD + dt * 32 + 16 * (vg & 1) + 4 * (vl & 3)];
          const uint2 lo = lds_read_tr16(vp);
          const uint2 hi = lds_read_tr16(vp + 8 * VPAD);
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)),
                                                          pf[ks], o[dt], 0, 0, 0);
        }
    }
  };

  const int last = ntiles - 1;
  if (ntiles > 0) {
    HIPSA_GLOAD(0, kreg0, vreg0, vtok0);
    HIPSA_LSTORE(0, kreg0, vreg0, vtok0);
    HIPSA_GLOAD(min(1, last), kreg1, vreg1, vtok1);
  }
  __syncthreads();

  // tile tl sits in LDS slot tl & 1; register set (tl + 1) & 1 holds tile
  // tl + 1 (in flight since the previous tile), and set tl & 1, free again,
  // takes tile tl + 2.  Tiles past the last reload the last one, unused,
  // which keeps this code free of branches.
  for (int tl = 0; tl < ntiles; tl += 2) {
    HIPSA_GLOAD(min(tl + 2, last), kreg0, vreg0, vtok0);
    tile(0);
    HIPSA_LSTORE(1, kreg1, vreg1, vtok1);
    __syncthreads();
    if (tl + 1 >= ntiles) break;  // uniform
    HIPSA_GLOAD(min(tl + 3, last), kreg1, vreg1, vtok1);
    tile(1);
    HIPSA_LSTORE(0, kreg0, vreg0, vtok0);
    __syncthreads();
  }
#undef HIPSA_LSTORE
#undef HIPSA_GLOAD
#undef HIPSA_TOKEN

  if (!active) return;
  const float lt = xor32_sum(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (!qvalid) return;
  uint16_t *Og = reinterpret_cast<uint16_t *>(a.out) + ((int64_t)(b * s.Hq + g * s.G + h) * Tq + r0 + qq) * D;
#pragma unroll
  for (int dt = 0; dt < DT; dt++)
#pragma unroll
    for (int gq = 0; gq < 4; gq++) {
      const int d = dt * 32 + 8 * gq + 4 * half;
      uint2 w;
      w.x = (uint32_t)f32_to_bf16(o[dt][4 * gq] * inv) | ((uint32_t)f32_to_bf16(o[dt][4 * gq + 1] * inv) << 16);
      w.y = (uint32_t)f32_to_bf16(o[dt][4 * gq + 2] * inv) | ((uint32_t)f32_to_bf16(o[dt][4 * gq + 3] * inv) << 16);
      *reinterpret_cast<uint2 *>(Og + d) = w;
    }
}

template <bool PAGED>
void launch_kv(const AttnArgs &a, dim3 grid, dim3 block, hipStream_t st) {
  if (a.s.dtype == HIPSA_BF16_E5M2) {
    if (a.s.d == 64) hipLaunchKernelGGL((attn_prefill_kernel<uint8_t, 64, PAGED>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_prefill_kernel<uint8_t, 128, PAGED>), grid, block, 0, st, a);
  } else {
    if (a.s.d == 64) hipLaunchKernelGGL((attn_prefill_kernel<uint16_t, 64, PAGED>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_prefill_kernel<uint16_t, 128, PAGED>), grid, block, 0, st, a);
  }
}

}  // namespace

hipError_t launch_attn_prefill(const AttnArgs &a, hipStream_t st) {
  const unsigned hchunks = (unsigned)(a.s.G + 3) / 4;
  const dim3 grid((unsigned)(a.s.problems * hchunks)), block(512);
  if (a.pg.table) launch_kv<true>(a, grid, block, st);
  else launch_kv<false>(a, grid, block, st);
  return hipGetLastError();
}

}  // namespace hipsa
