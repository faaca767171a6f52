// Host entry points of libhipsa: argument checks, workspace sizing, dispatch.
//
// Every check runs before the first HIP call, so a rejected call has no
// effect on the device.  Messages are kept per host thread.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "hipsa_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return HIPSA_OK;
}

bool pow2_in(int64_t v, int64_t lo, int64_t hi) {
  return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

// Checks shared by every entry point; fills `s` on success.
int check_shape(const hipsa_desc *d, int64_t k, int64_t block_k, int64_t block_q,
                hipsa::Shape *s) {
  if (!d) return fail(HIPSA_ERR_NULL, "desc is NULL");
  if (d->B < 0 || d->Hq < 1 || d->Hkv < 1 || d->Tq < 0)
    return fail(HIPSA_ERR_SHAPE, "need B >= 0, Hq >= 1, Hkv >= 1, Tq >= 0 (got B=%lld Hq=%lld "
                "Hkv=%lld Tq=%lld)", (long long)d->B, (long long)d->Hq, (long long)d->Hkv,
                (long long)d->Tq);
  if (d->Hq % d->Hkv != 0)
    return fail(HIPSA_ERR_SHAPE, "Hq=%lld is not a multiple of Hkv=%lld", (long long)d->Hq,
                (long long)d->Hkv);
  if (d->Hq / d->Hkv > hipsa::kMaxGroup)
    return fail(HIPSA_ERR_SHAPE, "Hq/Hkv=%lld exceeds %d", (long long)(d->Hq / d->Hkv),
                hipsa::kMaxGroup);
  if (d->T < 1) return fail(HIPSA_ERR_SHAPE, "T=%lld must be >= 1", (long long)d->T);
  if (d->Tq > d->T)
    return fail(HIPSA_ERR_SHAPE, "Tq=%lld exceeds T=%lld", (long long)d->Tq, (long long)d->T);
  if (d->T_cap < d->T || d->T_cap > (int64_t(1) << 30))
    return fail(HIPSA_ERR_SHAPE, "need T <= T_cap <= 2^30 (T=%lld T_cap=%lld)", (long long)d->T,
                (long long)d->T_cap);
  if (d->d != 64 && d->d != 128)
    return fail(HIPSA_ERR_SHAPE, "head dim d=%lld unsupported (64 or 128)", (long long)d->d);
  if (d->dtype != HIPSA_F32 && d->dtype != HIPSA_BF16 && d->dtype != HIPSA_BF16_E5M2)
    return fail(HIPSA_ERR_DTYPE, "dtype=%d unsupported", (int)d->dtype);
  if (!pow2_in(block_k, 8, 64))
    return fail(HIPSA_ERR_BLOCK, "block_k=%lld unsupported (8, 16, 32 or 64)",
                (long long)block_k);
  if (k < block_k || k % block_k != 0)
    return fail(HIPSA_ERR_BLOCK, "k=%lld must be a positive multiple of block_k=%lld",
                (long long)k, (long long)block_k);
  if (k / block_k > hipsa::kMaxKb)
    return fail(HIPSA_ERR_BLOCK, "k/block_k=%lld exceeds %d", (long long)(k / block_k),
                hipsa::kMaxKb);
  if (block_q != 1 && block_q != 64)
    return fail(HIPSA_ERR_BLOCK, "block_q=%lld unsupported (1 or 64)", (long long)block_q);
  if (block_q == 64 && d->dtype == HIPSA_F32)
    return fail(HIPSA_ERR_DTYPE, "block_q=64 (prefill) needs a bf16 query (HIPSA_BF16 or "
                "HIPSA_BF16_E5M2)");
  s->B = d->B; s->Hq = d->Hq; s->Hkv = d->Hkv; s->Tq = d->Tq; s->T = d->T; s->T_cap = d->T_cap;
  s->d = d->d;
  s->G = (int32_t)(d->Hq / d->Hkv);
  s->Kb = (int32_t)(k / block_k);
  s->bk = (int32_t)block_k;
  s->bk_shift = __builtin_ctzll((unsigned long long)block_k);
  s->bq = (int32_t)block_q;
  s->causal = d->causal != 0;
  s->dtype = d->dtype;
  s->nqb = (d->Tq + block_q - 1) / block_q;
  s->problems = d->B * d->Hkv * s->nqb;
  s->sink_b = s->window_b = 0;
  // largest grid: decode attention launches problems x splits x G workgroups at most
  const int64_t splits = ((int64_t)s->Kb * s->bk + 63) / 64;
  if (s->problems * splits * s->G >= (int64_t(1) << 31))
    return fail(HIPSA_ERR_SHAPE, "too many problems (%lld) for one launch",
                (long long)s->problems);
  return HIPSA_OK;
}

size_t workspace_for(const hipsa::Shape &s) {
  if (s.problems == 0) return 0;
  if (s.bq == 1) return hipsa::attn_decode_workspace(s);
  return 0;
}

// Vector loads and stores of 16 bytes need 16-byte aligned bases.
int check_aligned(const void *const *p, const char *const *names, int n) {
  for (int i = 0; i < n; i++)
    if (reinterpret_cast<uintptr_t>(p[i]) % 16 != 0)
      return fail(HIPSA_ERR_ALIGN, "%s at %p is not 16-byte aligned", names[i], p[i]);
  return HIPSA_OK;
}

int hip_fail(hipError_t e, const char *what) {
  return fail(HIPSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Shape checks for a paged call: desc->T_cap is not used, so it is replaced
// by T before the shared checks.  `mask`: the mask kernels keep a sequence's
// page numbers on chip, which bounds ceil(T / page_size).
int check_paged(const hipsa_desc *desc, const hipsa_pages *pg, int64_t k, int64_t block_k,
                int64_t block_q, bool mask, hipsa::Shape *s, hipsa::Pages *out) {
  if (!desc || !pg) return fail(HIPSA_ERR_NULL, "desc and pages must be non-NULL");
  hipsa_desc d = *desc;
  d.T_cap = d.T;
  int rc = check_shape(&d, k, block_k, block_q, s);
  if (rc) return rc;
  if (!pow2_in(pg->page_size, 1, 65536) || pg->page_size < block_k)
    return fail(HIPSA_ERR_PAGES, "page_size=%lld must be a power of two in [block_k=%lld, 65536]",
                (long long)pg->page_size, (long long)block_k);
  const int64_t need = (d.T + pg->page_size - 1) / pg->page_size;
  if (pg->max_pages < need)
    return fail(HIPSA_ERR_PAGES, "max_pages=%lld is below ceil(T/page_size)=%lld",
                (long long)pg->max_pages, (long long)need);
  if (pg->num_pages < 1 || pg->num_pages > INT32_MAX)
    return fail(HIPSA_ERR_PAGES, "num_pages=%lld must be in [1, 2^31)", (long long)pg->num_pages);
  if (mask && need > hipsa::kMaxSeqPagesOnChip)
    return fail(HIPSA_ERR_PAGES, "ceil(T/page_size)=%lld exceeds %d for mask estimation",
                (long long)need, hipsa::kMaxSeqPagesOnChip);
  out->table = pg->table;
  out->max_pages = pg->max_pages;
  out->ps_shift = __builtin_ctzll((unsigned long long)pg->page_size);
  out->last_page = (int32_t)(pg->num_pages - 1);
  out->seq_pages = (int32_t)(need < INT32_MAX ? need : INT32_MAX);
  return HIPSA_OK;
}

// The contiguous layout: no table (max_pages 0 marks "not paged").
constexpr hipsa::Pages kContiguous{nullptr, 0, -1, 0, 0};

// Checks of every call: the shape, the paged layout when ext->pages is set,
// and the dense part (sink, window).
int prepare(const hipsa_desc *desc, const hipsa_ext *ext, int64_t k, int64_t block_k,
            int64_t block_q, bool mask, hipsa::Shape *s, hipsa::Pages *pg) {
  int rc;
  if (ext && ext->pages) {
    rc = check_paged(desc, ext->pages, k, block_k, block_q, mask, s, pg);
  } else {
    rc = check_shape(desc, k, block_k, block_q, s);
    *pg = kContiguous;
  }
  if (rc || !ext) return rc;
  if (ext->sink < 0 || ext->window < 0 || ext->sink % block_k != 0 || ext->window % block_k != 0)
    return fail(HIPSA_ERR_BLOCK, "sink=%lld and window=%lld must be non-negative multiples of "
                "block_k=%lld", (long long)ext->sink, (long long)ext->window, (long long)block_k);
  if ((ext->sink + ext->window) / block_k > hipsa::kMaxDenseBlocks)
    return fail(HIPSA_ERR_BLOCK, "(sink + window) / block_k = %lld exceeds %d",
                (long long)((ext->sink + ext->window) / block_k), hipsa::kMaxDenseBlocks);
  s->sink_b = (int32_t)(ext->sink / block_k);
  s->window_b = (int32_t)(ext->window / block_k);
  // largest grid: decode attention launches problems x splits x G workgroups at most
  if (s->problems * ((hipsa::entry_tokens(*s) + 63) / 64) * s->G >= (int64_t(1) << 31))
    return fail(HIPSA_ERR_SHAPE, "too many problems (%lld) for one launch", (long long)s->problems);
  return HIPSA_OK;
}

int mask_impl(const hipsa::Shape &s, const hipsa::Pages &pg, const void *q, const void *K,
              int32_t *indices, int32_t *nnz, void *stream) {
  if (s.problems == 0) return ok();
  if (!q || !K || !indices || !nnz)
    return fail(HIPSA_ERR_NULL, "q, K, indices and nnz must be non-NULL");
  if (pg.max_pages > 0 && !pg.table)  // a paged call (max_pages >= 1) without a table
    return fail(HIPSA_ERR_NULL, "pages->table must be non-NULL");
  int rc;
  {
    const void *p[] = {q, K};
    const char *nm[] = {"q", "K"};
    if ((rc = check_aligned(p, nm, 2))) return rc;
  }
  hipsa::MaskArgs a{q, K, indices, nnz, s, pg};
  hipError_t e = s.bq == 1 ? hipsa::launch_mask_decode(a, (hipStream_t)stream)
                           : hipsa::launch_mask_prefill(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mask estimation launch");
  return ok();
}

int attn_impl(const hipsa::Shape &s, const hipsa::Pages &pg, const void *q, const void *K,
              const void *V, const int32_t *indices, const int32_t *nnz, void *out,
              void *workspace, size_t workspace_bytes, void *stream) {
  int rc;
  if (s.problems == 0) return ok();
  if (!q || !K || !V || !indices || !nnz || !out)
    return fail(HIPSA_ERR_NULL, "q, K, V, indices, nnz and out must be non-NULL");
  if (pg.max_pages > 0 && !pg.table)  // a paged call (max_pages >= 1) without a table
    return fail(HIPSA_ERR_NULL, "pages->table must be non-NULL");
  {
    const void *p[] = {q, K, V, out};
    const char *nm[] = {"q", "K", "V", "out"};
    if ((rc = check_aligned(p, nm, 4))) return rc;
  }
  const size_t need = workspace_for(s);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(HIPSA_ERR_WORKSPACE, "workspace of %zu bytes at %p is too small: need %zu",
                workspace_bytes, workspace, need);
  hipsa::AttnArgs a{};
  a.q = q; a.K = K; a.V = V; a.indices = indices; a.nnz = nnz; a.out = out;
  a.ws = static_cast<float *>(workspace);
  a.s = s;
  a.pg = pg;
  a.scale = (float)(1.0 / __builtin_sqrt((double)s.d));
  hipError_t e;
  if (s.bq == 1) {
    a.splits = hipsa::attn_decode_splits(s);
    e = hipsa::launch_attn_decode(a, (hipStream_t)stream);
  } else {
    a.splits = 1;
    e = hipsa::launch_attn_prefill(a, (hipStream_t)stream);
  }
  if (e != hipSuccess) return hip_fail(e, "sparse attention launch");
  return ok();
}

}  // namespace

extern "C" {

int hip_mask_estimate(const hipsa_desc *desc, const void *q, const void *K, int64_t k,
                      int64_t block_k, int64_t block_q, int32_t *indices, int32_t *nnz,
                      void *workspace, size_t workspace_bytes, void *stream) {
  (void)workspace;
  (void)workspace_bytes;
  hipsa::Shape s;
  int rc = check_shape(desc, k, block_k, block_q, &s);
  if (rc) return rc;
  return mask_impl(s, kContiguous, q, K, indices, nnz, stream);
}

int hip_mask_estimate_ex(const hipsa_desc *desc, const hipsa_ext *ext, const void *q,
                         const void *K, int64_t k, int64_t block_k, int64_t block_q,
                         int32_t *indices, int32_t *nnz, void *workspace, size_t workspace_bytes,
                         void *stream) {
  (void)workspace;
  (void)workspace_bytes;
  hipsa::Shape s;
  hipsa::Pages pg;
  int rc = prepare(desc, ext, k, block_k, block_q, true, &s, &pg);
  if (rc) return rc;
  return mask_impl(s, pg, q, K, indices, nnz, stream);
}

int hip_mask_estimate_paged(const hipsa_desc *desc, const hipsa_pages *pages, const void *q,
                            const void *K, int64_t k, int64_t block_k, int64_t block_q,
                            int32_t *indices, int32_t *nnz, void *workspace,
                            size_t workspace_bytes, void *stream) {
  if (!pages) return fail(HIPSA_ERR_NULL, "desc and pages must be non-NULL");
  const hipsa_ext ext{pages, 0, 0};
  return hip_mask_estimate_ex(desc, &ext, q, K, k, block_k, block_q, indices, nnz, workspace,
                              workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Checks of a stage list and the shape; fills `a` (all but the pointers) and
// returns the workspace bytes in *ws.
int prepare_stages(const hipsa_desc *desc, const hipsa_ext *ext, const hipsa_stage *stages,
                   int32_t nstages, int64_t block_k, hipsa::StageArgs *a, size_t *ws) {
  if (!stages) return fail(HIPSA_ERR_NULL, "stages is NULL");
  if (nstages < 2 || nstages > hipsa::kMaxStages)
    return fail(HIPSA_ERR_STAGES, "nstages=%d must be in [2, %d]", (int)nstages, hipsa::kMaxStages);
  if (block_k < 1) return fail(HIPSA_ERR_BLOCK, "block_k=%lld must be positive", (long long)block_k);
  *a = hipsa::StageArgs{};
  a->nst = nstages;
  int64_t cap = 0;
  for (int32_t j = 0; j < nstages; j++) {
    const int64_t c = stages[j].chunk_size, k = stages[j].k;
    if (c < block_k || c % block_k != 0)
      return fail(HIPSA_ERR_STAGES, "stage %d: chunk_size=%lld must be a positive multiple of "
                  "block_k=%lld", (int)j, (long long)c, (long long)block_k);
    if (j > 0 && c >= stages[j - 1].chunk_size)
      return fail(HIPSA_ERR_STAGES, "stage %d: chunk_size=%lld must be below the previous "
                  "stage's %lld", (int)j, (long long)c, (long long)stages[j - 1].chunk_size);
    if (j == 0 && k != 0)
      return fail(HIPSA_ERR_STAGES, "stage 0 keeps every chunk: its k must be 0 (got %lld)",
                  (long long)k);
    if (j > 0 && (k < c || k % c != 0 || k / c > hipsa::kMaxStageChunks))
      return fail(HIPSA_ERR_STAGES, "stage %d: k=%lld must be a multiple of chunk_size=%lld "
                  "keeping 1 to %d chunks", (int)j, (long long)k, (long long)c,
                  hipsa::kMaxStageChunks);
    if (c / block_k > INT32_MAX)
      return fail(HIPSA_ERR_STAGES, "stage %d: chunk_size=%lld is too large", (int)j, (long long)c);
    a->chunk[j] = (int32_t)(c / block_k);
    a->keep[j] = j > 0 ? (int32_t)(k / c) : 0;
    if (a->keep[j] > cap) cap = a->keep[j];
  }
  if (stages[nstages - 1].chunk_size != block_k)
    return fail(HIPSA_ERR_STAGES, "the last stage's chunk_size=%lld must be block_k=%lld",
                (long long)stages[nstages - 1].chunk_size, (long long)block_k);
  hipsa::Pages pg;
  int rc = prepare(desc, ext, stages[nstages - 1].k, block_k, 1, true, &a->m.s, &pg);
  if (rc) return rc;
  a->m.pg = pg;
  const int64_t blocks = (a->m.s.T + block_k - 1) / block_k;
  const int64_t n0 = (blocks + a->chunk[0] - 1) / a->chunk[0];
  if (n0 > hipsa::kMaxStageChunks)
    return fail(HIPSA_ERR_STAGES, "stage 0 cuts up to %lld chunks of %lld tokens; at most %d "
                "are supported", (long long)n0, (long long)stages[0].chunk_size,
                hipsa::kMaxStageChunks);
  if (n0 > cap) cap = n0;
  a->cap = (int32_t)cap;
  *ws = hipsa::mask_stages_plan(a);
  return HIPSA_OK;
}

}  // namespace

extern "C" {

int hip_mask_estimate_stages(const hipsa_desc *desc, const hipsa_ext *ext,
                             const hipsa_stage *stages, int32_t nstages, const void *q,
                             const void *K, int64_t block_k, int32_t *indices, int32_t *nnz,
                             void *workspace, size_t workspace_bytes, void *stream) {
  hipsa::StageArgs a;
  size_t need = 0;
  int rc = prepare_stages(desc, ext, stages, nstages, block_k, &a, &need);
  if (rc) return rc;
  if (a.m.s.problems == 0) return ok();
  if (!q || !K || !indices || !nnz)
    return fail(HIPSA_ERR_NULL, "q, K, indices and nnz must be non-NULL");
  if (a.m.pg.max_pages > 0 && !a.m.pg.table)
    return fail(HIPSA_ERR_NULL, "pages->table must be non-NULL");
  {
    const void *p[] = {q, K};
    const char *nm[] = {"q", "K"};
    if ((rc = check_aligned(p, nm, 2))) return rc;
  }
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(HIPSA_ERR_WORKSPACE, "workspace of %zu bytes at %p is too small: need %zu",
                  workspace_bytes, workspace, need);
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
      return fail(HIPSA_ERR_ALIGN, "workspace at %p is not 16-byte aligned", workspace);
    a.keys = static_cast<uint64_t *>(workspace);
    a.arrived = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + need -
                                             (size_t)a.m.s.problems * sizeof(uint32_t));
  }
  a.m.q = q;
  a.m.K = K;
  a.m.indices = indices;
  a.m.nnz = nnz;
  hipError_t e = hipsa::launch_mask_stages(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "multi-stage mask estimation launch");
  return ok();
}

size_t hipsa_stages_workspace_bytes(const hipsa_desc *desc, const hipsa_ext *ext,
                                    const hipsa_stage *stages, int32_t nstages, int64_t block_k) {
  hipsa::StageArgs a;
  size_t need = 0;
  if (prepare_stages(desc, ext, stages, nstages, block_k, &a, &need)) return SIZE_MAX;
  g_err.clear();
  return need;
}

int hip_sparse_attn(const hipsa_desc *desc, const void *q, const void *K, const void *V,
                    const int32_t *indices, const int32_t *nnz, int64_t k, int64_t block_k,
                    int64_t block_q, void *out, void *workspace, size_t workspace_bytes,
                    void *stream) {
  hipsa::Shape s;
  int rc = check_shape(desc, k, block_k, block_q, &s);
  if (rc) return rc;
  return attn_impl(s, kContiguous, q, K, V, indices, nnz, out, workspace, workspace_bytes, stream);
}

int hip_sparse_attn_ex(const hipsa_desc *desc, const hipsa_ext *ext, const void *q, const void *K,
                       const void *V, const int32_t *indices, const int32_t *nnz, int64_t k,
                       int64_t block_k, int64_t block_q, void *out, void *workspace,
                       size_t workspace_bytes, void *stream) {
  hipsa::Shape s;
  hipsa::Pages pg;
  int rc = prepare(desc, ext, k, block_k, block_q, false, &s, &pg);
  if (rc) return rc;
  return attn_impl(s, pg, q, K, V, indices, nnz, out, workspace, workspace_bytes, stream);
}

int hip_sparse_attn_paged(const hipsa_desc *desc, const hipsa_pages *pages, const void *q,
                          const void *K, const void *V, const int32_t *indices,
                          const int32_t *nnz, int64_t k, int64_t block_k, int64_t block_q,
                          void *out, void *workspace, size_t workspace_bytes, void *stream) {
  if (!pages) return fail(HIPSA_ERR_NULL, "desc and pages must be non-NULL");
  const hipsa_ext ext{pages, 0, 0};
  return hip_sparse_attn_ex(desc, &ext, q, K, V, indices, nnz, k, block_k, block_q, out,
                            workspace, workspace_bytes, stream);
}

int hip_decode_step(const hipsa_desc *desc, const hipsa_ext *ext, const void *q, const void *K,
                    const void *V, int64_t k, int64_t block_k, int32_t *indices, int32_t *nnz,
                    void *out, void *workspace, size_t workspace_bytes, void *stream) {
  hipsa::Shape s;
  hipsa::Pages pg;
  int rc = prepare(desc, ext, k, block_k, 1, true, &s, &pg);
  if (rc) return rc;
  if (s.problems == 0) return ok();
  if (!q || !K || !V || !indices || !nnz || !out)
    return fail(HIPSA_ERR_NULL, "q, K, V, indices, nnz and out must be non-NULL");
  if (pg.max_pages > 0 && !pg.table)
    return fail(HIPSA_ERR_NULL, "pages->table must be non-NULL");
  {
    const void *p[] = {q, K, V, out};
    const char *nm[] = {"q", "K", "V", "out"};
    if ((rc = check_aligned(p, nm, 4))) return rc;
  }
  const size_t need = hipsa::decode_step_workspace(s);
  if (!workspace || workspace_bytes < need)
    return fail(HIPSA_ERR_WORKSPACE, "workspace of %zu bytes at %p is too small: need %zu",
                workspace_bytes, workspace, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(HIPSA_ERR_ALIGN, "workspace at %p is not 16-byte aligned", workspace);
  hipsa::StepArgs a{};
  a.at.q = q; a.at.K = K; a.at.V = V; a.at.out = out;
  a.at.ws = static_cast<float *>(workspace);
  a.at.s = s;
  a.at.pg = pg;
  a.at.scale = (float)(1.0 / __builtin_sqrt((double)s.d));
  a.at.splits = hipsa::attn_decode_splits(s);
  a.indices = indices;
  a.nnz = nnz;
  a.arrived = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + need -
                                           (size_t)s.problems * sizeof(uint32_t));
  hipError_t e = hipsa::launch_decode_step(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode step launch");
  return ok();
}

int hip_sparse_attn_noalloc(const hipsa_desc *desc, const void *q, const void *K, const void *V,
                            const int32_t *indices, const int32_t *nnz, int64_t k, int64_t block_k,
                            int64_t block_q, void *out, void *stream) {
  hipsa::Shape s;
  int rc = check_shape(desc, k, block_k, block_q, &s);
  if (rc) return rc;
  if (s.problems == 0) return ok();
  if (!q || !K || !V || !indices || !nnz || !out)
    return fail(HIPSA_ERR_NULL, "q, K, V, indices, nnz and out must be non-NULL");
  {
    const void *p[] = {q, K, V, out};
    const char *nm[] = {"q", "K", "V", "out"};
    if ((rc = check_aligned(p, nm, 4))) return rc;
  }
  const size_t need = workspace_for(s);
  if (need > hipsa::kNoAllocScratchBytes)
    return fail(HIPSA_ERR_WORKSPACE, "this shape needs %zu bytes of split partials; the "
                "library's scratch holds %zu (use hip_sparse_attn with a workspace)", need,
                hipsa::kNoAllocScratchBytes);
  void *scratch = nullptr;
  hipError_t e = hipsa::noalloc_scratch((hipStream_t)stream, &scratch);
  if (e != hipSuccess) return hip_fail(e, "scratch lookup");
  return attn_impl(s, kContiguous, q, K, V, indices, nnz, out, scratch,
                   hipsa::kNoAllocScratchBytes, stream);
}

size_t hipsa_decode_step_workspace_bytes(const hipsa_desc *desc, const hipsa_ext *ext, int64_t k,
                                         int64_t block_k) {
  hipsa::Shape s;
  hipsa::Pages pg;
  if (prepare(desc, ext, k, block_k, 1, true, &s, &pg)) return SIZE_MAX;
  g_err.clear();
  return hipsa::decode_step_workspace(s);
}

size_t hipsa_workspace_bytes(const hipsa_desc *desc, int64_t k, int64_t block_k,
                             int64_t block_q) {
  return hipsa_workspace_bytes_ex(desc, nullptr, k, block_k, block_q);
}

size_t hipsa_workspace_bytes_ex(const hipsa_desc *desc, const hipsa_ext *ext, int64_t k,
                                int64_t block_k, int64_t block_q) {
  hipsa::Shape s;
  hipsa::Pages pg;
  if (prepare(desc, ext, k, block_k, block_q, false, &s, &pg)) return SIZE_MAX;
  g_err.clear();
  return workspace_for(s);
}

const char *hipsa_last_error(void) { return g_err.c_str(); }

}  // extern "C"
