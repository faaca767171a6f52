"""The C ABI on the host: the library loads, exports every function that
include/hipsa.h declares, and rejects invalid arguments before any HIP call
(so these run without a GPU: no compute call is made)."""
import ctypes as C
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hipsa.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(["hip_mask_estimate", "hip_sparse_attn", "hip_mask_estimate_paged",
                                  "hip_sparse_attn_paged", "hip_mask_estimate_ex",
                                  "hip_sparse_attn_ex", "hip_sparse_attn_noalloc", "hip_decode_step",
                                  "hipsa_decode_step_workspace_bytes", "hip_mask_estimate_stages",
                                  "hipsa_stages_workspace_bytes",
                                  "hipsa_workspace_bytes", "hipsa_workspace_bytes_ex",
                                  "hipsa_last_error"])


def test_library_exports_every_declared_symbol():
    import long_context_sparse_mask_amd as hs
    for name in _declared():
        assert hasattr(hs.lib, name), name


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-fsyntax-only", "-x", "c", "-std=c99", "-Wall", "-Werror", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _desc(**kw):
    import long_context_sparse_mask_amd as hs
    base = dict(B=1, Hq=32, Hkv=8, Tq=1, T=32768, T_cap=32768, d=128, causal=1, dtype=1)
    base.update(kw)
    return hs.Desc(**base)


FAKE = C.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


def _mask(desc, k=2048, bk=64, bq=1, ptrs=(FAKE, FAKE, FAKE, FAKE)):
    import long_context_sparse_mask_amd as hs
    q, K, idx, nnz = ptrs
    return hs.lib.hip_mask_estimate(C.byref(desc), q, K, k, bk, bq, idx, nnz, None, 0, None)


ERR_NULL, ERR_SHAPE, ERR_BLOCK, ERR_DTYPE, ERR_WS, ERR_ALIGN, ERR_PAGES = -1, -2, -3, -4, -5, -7, -8
ERR_STAGES = -9


@pytest.mark.parametrize("kw,k,bk,bq,code", [
    (dict(Hq=30), 2048, 64, 1, ERR_SHAPE),          # Hq % Hkv != 0
    (dict(Hq=34, Hkv=2), 2048, 64, 1, ERR_SHAPE),   # group of 17 > 16
    (dict(T=0, T_cap=0), 2048, 64, 1, ERR_SHAPE),
    (dict(Tq=5, T=4, T_cap=4), 64, 64, 1, ERR_SHAPE),
    (dict(T_cap=100), 2048, 64, 1, ERR_SHAPE),      # T > T_cap
    (dict(T_cap=(1 << 30) + 1), 2048, 64, 1, ERR_SHAPE),
    (dict(d=96), 2048, 64, 1, ERR_SHAPE),
    (dict(dtype=7), 2048, 64, 1, ERR_DTYPE),
    (dict(), 2048, 48, 1, ERR_BLOCK),               # block_k not a power of two
    (dict(), 2048, 128, 1, ERR_BLOCK),
    (dict(), 2000, 64, 1, ERR_BLOCK),               # k % block_k
    (dict(), 32, 64, 1, ERR_BLOCK),                 # k < block_k
    (dict(), 64 * 513, 64, 1, ERR_BLOCK),           # K_b > 512
    (dict(), 2048, 64, 32, ERR_BLOCK),              # block_q
    (dict(dtype=0), 2048, 64, 64, ERR_DTYPE),       # fp32 prefill
    (dict(B=-1), 2048, 64, 1, ERR_SHAPE),
])
def test_mask_rejects_invalid_arguments(kw, k, bk, bq, code):
    import long_context_sparse_mask_amd as hs
    assert _mask(_desc(**kw), k, bk, bq) == code
    assert hs.lib.hipsa_last_error().decode() != ""


def test_null_pointers_rejected():
    import long_context_sparse_mask_amd as hs
    assert _mask(_desc(), ptrs=(None, FAKE, FAKE, FAKE)) == ERR_NULL
    assert hs.lib.hip_mask_estimate(None, FAKE, FAKE, 2048, 64, 1, FAKE, FAKE, None, 0, None) == ERR_NULL
    d = _desc()
    rc = hs.lib.hip_sparse_attn(C.byref(d), FAKE, FAKE, None, FAKE, FAKE, 2048, 64, 1, FAKE,
                                FAKE, 1 << 30, None)
    assert rc == ERR_NULL


def test_workspace_query_and_undersized_workspace():
    import long_context_sparse_mask_amd as hs
    d = _desc(B=4, T=131072, T_cap=131072)
    need = hs.lib.hipsa_workspace_bytes(C.byref(d), 2048, 64, 1)
    # 32 problems x 8 splits of 256 tokens x 4 heads x (d + 2) floats
    assert need == 32 * 8 * 4 * 130 * 4
    rc = hs.lib.hip_sparse_attn(C.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 64, 1, FAKE,
                                FAKE, need - 1, None)
    assert rc == ERR_WS and "too small" in hs.lib.hipsa_last_error().decode()
    bad = _desc(Hq=31)
    assert hs.lib.hipsa_workspace_bytes(C.byref(bad), 2048, 64, 1) == hs.SIZE_MAX


def test_fp8_kv_dtype_is_accepted_for_decode_and_prefill():
    """HIPSA_BF16_E5M2 (bf16 q, E5M2 K/V) passes validation for block_q 1 and 64
    (checked through the workspace query, which launches nothing); fp32 prefill
    stays rejected."""
    import long_context_sparse_mask_amd as hs
    d = _desc(B=4, T=131072, T_cap=131072, dtype=hs.HIPSA_BF16_E5M2)
    assert hs.lib.hipsa_workspace_bytes(C.byref(d), 2048, 64, 1) == 32 * 8 * 4 * 130 * 4
    p = _desc(Tq=4096, dtype=hs.HIPSA_BF16_E5M2)
    assert hs.lib.hipsa_workspace_bytes(C.byref(p), 2048, 64, 64) == 0
    assert hs.lib.hipsa_workspace_bytes(C.byref(_desc(Tq=4096, dtype=0)), 2048, 64, 64) == hs.SIZE_MAX
    assert hs.lib.hipsa_workspace_bytes(C.byref(_desc(dtype=3)), 2048, 64, 1) == hs.SIZE_MAX


def test_one_split_when_it_covers_the_key_sequence():
    """Decode splits a row's key sequence over workgroups of 64 to 256 tokens
    (the largest giving one workgroup per CU); a sequence that one workgroup
    covers gets a single split (its workgroup writes the output, no merge
    follows).  Seen through the workspace size, problems x splits x G x
    (d + 2) floats."""
    import long_context_sparse_mask_amd as hs
    # bf16, 128 listed tokens, 32 problems of G = 4: one split each
    d = _desc(B=1, T=8192, T_cap=8192)
    assert hs.lib.hipsa_workspace_bytes(C.byref(d), 128, 64, 1) == 8 * 1 * 4 * 130 * 4
    # 256 tokens: one split of 256
    assert hs.lib.hipsa_workspace_bytes(C.byref(d), 256, 64, 1) == 8 * 1 * 4 * 130 * 4
    # 512 tokens on 8 problems: 64-token splits give 64 workgroups (larger ones fewer)
    assert hs.lib.hipsa_workspace_bytes(C.byref(d), 512, 64, 1) == 8 * 8 * 4 * 130 * 4
    # 128k x 4 (32 problems, 2048 tokens): 256-token splits already give 256 workgroups
    d4 = _desc(B=4, T=131072, T_cap=131072)
    assert hs.lib.hipsa_workspace_bytes(C.byref(d4), 2048, 64, 1) == 32 * 8 * 4 * 130 * 4
    # groups of more than 8 query heads: 64-token splits
    d16 = _desc(B=4, Hq=32, Hkv=2, T=131072, T_cap=131072)
    assert hs.lib.hipsa_workspace_bytes(C.byref(d16), 2048, 64, 1) == 8 * 32 * 16 * 130 * 4
    # fp32 at d = 128 takes at most 64 tokens per split
    d32 = _desc(B=1, T=8192, T_cap=8192, dtype=0)
    assert hs.lib.hipsa_workspace_bytes(C.byref(d32), 64, 64, 1) == 8 * 1 * 4 * 130 * 4
    assert hs.lib.hipsa_workspace_bytes(C.byref(d32), 128, 64, 1) == 8 * 2 * 4 * 130 * 4


def test_misaligned_pointers_rejected():
    import long_context_sparse_mask_amd as hs
    odd = C.c_void_p(0x1008)
    for i in range(2):  # q, K
        ptrs = [FAKE] * 4
        ptrs[i] = odd
        assert _mask(_desc(), ptrs=tuple(ptrs)) == ERR_ALIGN
        assert "aligned" in hs.lib.hipsa_last_error().decode()
    d = _desc()
    for i in (0, 1, 2, 9):  # q, K, V, out
        args = [FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 64, 1, FAKE, FAKE, 1 << 30, None]
        args[i if i < 5 else 8] = odd
        assert hs.lib.hip_sparse_attn(C.byref(d), *args) == ERR_ALIGN


def test_binding_element_type_pairs():
    import torch
    import long_context_sparse_mask_amd as hs
    q16, q32 = torch.empty(1, dtype=torch.bfloat16), torch.empty(1)
    k8 = torch.empty(1, dtype=torch.float8_e5m2)
    assert hs._dtype_code(q16, k8) == hs.HIPSA_BF16_E5M2
    assert hs._dtype_code(q16, q16) == hs.HIPSA_BF16 and hs._dtype_code(q32, q32) == hs.HIPSA_F32
    for q, k in ((q32, k8), (q32, q16), (q16, q32), (k8, k8)):
        with pytest.raises(TypeError):
            hs._dtype_code(q, k)


def _pages(**kw):
    import long_context_sparse_mask_amd as hs
    base = dict(table=0x2000, max_pages=512, page_size=64, num_pages=4096)
    base.update(kw)
    return hs.Pages(**base)


def _mask_paged(desc, pages, k=2048, bk=64, bq=1, ptrs=(FAKE, FAKE, FAKE, FAKE)):
    import long_context_sparse_mask_amd as hs
    q, K, idx, nnz = ptrs
    return hs.lib.hip_mask_estimate_paged(C.byref(desc), C.byref(pages) if pages else None, q, K,
                                          k, bk, bq, idx, nnz, None, 0, None)


@pytest.mark.parametrize("pkw,dkw,bk,code", [
    (dict(page_size=48), {}, 64, ERR_PAGES),               # not a power of two
    (dict(page_size=32), {}, 64, ERR_PAGES),               # smaller than block_k
    (dict(page_size=1 << 17), {}, 64, ERR_PAGES),          # too large
    (dict(max_pages=511), {}, 64, ERR_PAGES),              # 32768 / 64 = 512 pages needed
    (dict(num_pages=0), {}, 64, ERR_PAGES),
    (dict(num_pages=1 << 31), {}, 64, ERR_PAGES),
    (dict(page_size=8, max_pages=20000), dict(T=16385 * 8), 8, ERR_PAGES),  # > 16384 pages on chip
    (dict(table=None), {}, 64, ERR_NULL),
    ({}, dict(Hq=30), 64, ERR_SHAPE),                      # the shared shape checks still apply
])
def test_paged_mask_rejects_invalid_pages(pkw, dkw, bk, code):
    import long_context_sparse_mask_amd as hs
    d = _desc(T_cap=0, **dkw)  # T_cap is not used by the paged calls
    assert _mask_paged(d, _pages(**pkw), k=32 * bk, bk=bk) == code
    assert hs.lib.hipsa_last_error().decode() != ""


def test_paged_calls_null_and_alignment():
    import long_context_sparse_mask_amd as hs
    assert _mask_paged(_desc(), None) == ERR_NULL
    assert _mask_paged(_desc(), _pages(), ptrs=(FAKE, C.c_void_p(0x1008), FAKE, FAKE)) == ERR_ALIGN
    d = _desc()
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 64, 1, FAKE, FAKE, 1 << 30, None]
    bad = _pages(page_size=12)
    assert hs.lib.hip_sparse_attn_paged(C.byref(d), C.byref(bad), *args) == ERR_PAGES
    args_v = list(args)
    args_v[2] = C.c_void_p(0x1008)  # V
    assert hs.lib.hip_sparse_attn_paged(C.byref(d), C.byref(_pages()), *args_v) == ERR_ALIGN
    args_ws = list(args)
    args_ws[10] = 0  # no workspace
    assert hs.lib.hip_sparse_attn_paged(C.byref(d), C.byref(_pages()), *args_ws) == ERR_WS
    # the attention call keeps no page numbers on chip: many pages are fine up to the checks
    # (exercised here only through the workspace check that precedes any launch)
    d2 = _desc(T=16385 * 8, T_cap=0)
    assert hs.lib.hip_sparse_attn_paged(C.byref(d2), C.byref(_pages(page_size=8, max_pages=20000)),
                                        FAKE, FAKE, FAKE, FAKE, FAKE, 256, 8, 1, FAKE, FAKE, 0,
                                        None) == ERR_WS


def test_dense_part_validation_and_workspace():
    """sink / window: non-negative multiples of block_k, at most 256 blocks
    together; the decode workspace grows with the dense entries."""
    import long_context_sparse_mask_amd as hs
    d = _desc(B=4, T=131072, T_cap=131072)

    def ws(sink, window, bk=64, k=2048):
        return hs.lib.hipsa_workspace_bytes_ex(C.byref(d), C.byref(hs.Ext(None, sink, window)), k,
                                               bk, 1)
    plain = hs.lib.hipsa_workspace_bytes(C.byref(d), 2048, 64, 1)
    assert ws(0, 0) == plain == 32 * 8 * 4 * 130 * 4
    # 1 sink + 64 window + 32 listed blocks = 6208 tokens: 25 splits of 256 tokens
    assert ws(64, 4096) == 32 * 25 * 4 * 130 * 4
    for sink, window in ((-64, 0), (32, 0), (0, 100), (64 * 200, 64 * 57)):
        assert ws(sink, window) == hs.SIZE_MAX
    assert ws(64 * 200, 64 * 56) != hs.SIZE_MAX  # exactly 256 blocks
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 64, 1, FAKE, FAKE, 0, None]
    assert hs.lib.hip_sparse_attn_ex(C.byref(d), C.byref(hs.Ext(None, 32, 0)), *args) == ERR_BLOCK
    assert hs.lib.hip_mask_estimate_ex(C.byref(d), C.byref(hs.Ext(None, 0, 64 * 300)), FAKE, FAKE,
                                       2048, 64, 1, FAKE, FAKE, None, 0, None) == ERR_BLOCK


def _stage_arr(stages):
    import long_context_sparse_mask_amd as hs
    return (hs.Stage * max(len(stages), 1))(*[hs.Stage(c, k) for c, k in stages])


def _stages(desc, stages, bk=64, ext=None, ptrs=(FAKE, FAKE, FAKE, FAKE), ws=None, ws_bytes=0):
    import long_context_sparse_mask_amd as hs
    q, K, idx, nnz = ptrs
    return hs.lib.hip_mask_estimate_stages(C.byref(desc), ext, _stage_arr(stages), len(stages), q,
                                           K, bk, idx, nnz, ws, ws_bytes, None)


GOOD_STAGES = [(512, 0), (128, 8192), (64, 2048)]


@pytest.mark.parametrize("stages,bk,dkw,code", [
    ([(512, 0)], 64, {}, ERR_STAGES),                              # one stage
    ([(4096 >> j, 0 if j == 0 else 64) for j in range(9)], 16, {}, ERR_STAGES),  # nine stages
    ([(512, 64), (64, 2048)], 64, {}, ERR_STAGES),                 # stage 0 keeps a count
    ([(512, 0), (512, 2048), (64, 2048)], 64, {}, ERR_STAGES),     # chunk size not decreasing
    ([(512, 0), (96, 2048), (64, 2048)], 64, {}, ERR_STAGES),      # not a multiple of block_k
    ([(512, 0), (128, 8000), (64, 2048)], 64, {}, ERR_STAGES),     # k not a multiple of the chunk
    ([(512, 0), (128, 0), (64, 2048)], 64, {}, ERR_STAGES),        # a later stage keeps nothing
    ([(512, 0), (128, 128 * 2049), (64, 2048)], 64, {}, ERR_STAGES),  # keeps over 2048 chunks
    ([(512, 0), (128, 8192)], 64, {}, ERR_STAGES),                 # last chunk is not block_k
    ([(128, 0), (64, 2048)], 64, dict(T=64 * 4097, T_cap=64 * 4097), ERR_STAGES),  # 2049 stage-0 chunks
    ([(512, 0), (128, 8192), (64, 64 * 513)], 64, {}, ERR_BLOCK),  # K_b above 512
    (GOOD_STAGES, 48, {}, ERR_STAGES),                             # chunk sizes vs block_k 48
    (GOOD_STAGES, 64, dict(Hq=30), ERR_SHAPE),                     # the shared checks still apply
])
def test_stages_reject_invalid_lists(stages, bk, dkw, code):
    import long_context_sparse_mask_amd as hs
    assert _stages(_desc(**dkw), stages, bk) == code, hs.lib.hipsa_last_error().decode()


def test_stages_null_alignment_and_empty_problems():
    import long_context_sparse_mask_amd as hs
    d = _desc()
    assert _stages(d, GOOD_STAGES, ptrs=(None, FAKE, FAKE, FAKE)) == ERR_NULL
    assert _stages(d, GOOD_STAGES, ptrs=(C.c_void_p(0x1008), FAKE, FAKE, FAKE)) == ERR_ALIGN
    assert hs.lib.hip_mask_estimate_stages(C.byref(d), None, None, 3, FAKE, FAKE, 64, FAKE, FAKE,
                                           None, 0, None) == ERR_NULL
    # exactly 2048 stage-0 chunks is accepted as far as the pointers (NULL q here)
    big = _desc(T=64 * 4096, T_cap=64 * 4096)
    assert _stages(big, [(128, 0), (64, 2048)], ptrs=(None, FAKE, FAKE, FAKE)) == ERR_NULL
    for e in (_desc(B=0), _desc(Tq=0)):
        assert _stages(e, GOOD_STAGES, ptrs=(None, None, None, None)) == 0
    # the dense part's checks apply (sink not a multiple of block_k)
    assert _stages(d, GOOD_STAGES, ext=C.byref(hs.Ext(None, 32, 0))) == ERR_BLOCK


def test_stages_workspace():
    """A first round of more than 1024 candidates is spread over workgroups
    (at most one per CU, at least 128 slots each), whose keys and arrival
    counters need a workspace; narrower first rounds need none."""
    import long_context_sparse_mask_amd as hs

    def ws(d, stages, bk=64):
        return hs.lib.hipsa_stages_workspace_bytes(C.byref(d), None, _stage_arr(stages),
                                                   len(stages), bk)
    assert ws(_desc(B=4, T=131072, T_cap=131072), GOOD_STAGES) == 0   # 512 first-round slots
    one_m = _desc(T=1 << 20, T_cap=1 << 20)
    st = [(512, 0), (128, 16384), (64, 4096)]
    # 2048 stage-0 chunks: 4096 slots per row, 8 rows, keys 8 B each, then 8 counters
    assert ws(one_m, st) == 8 * 4096 * 8 + 8 * 4
    assert ws(one_m, [(512, 0)]) == hs.SIZE_MAX
    rc = _stages(one_m, st, ptrs=(FAKE, FAKE, FAKE, FAKE), ws=FAKE, ws_bytes=8 * 4096 * 8)
    assert rc == ERR_WS and "too small" in hs.lib.hipsa_last_error().decode()
    assert _stages(one_m, st, ws=None, ws_bytes=0) == ERR_WS
    assert _stages(one_m, st, ws=C.c_void_p(0x1008), ws_bytes=1 << 20) == ERR_ALIGN


def test_paged_empty_problem_is_a_no_op():
    import long_context_sparse_mask_amd as hs
    for d in (_desc(B=0, T_cap=0), _desc(Tq=0, T_cap=0)):
        assert _mask_paged(d, _pages(table=None), ptrs=(None, None, None, None)) == 0
        assert hs.lib.hip_sparse_attn_paged(C.byref(d), C.byref(_pages(table=None)), None, None,
                                            None, None, None, 2048, 64, 1, None, None, 0,
                                            None) == 0


def test_empty_problem_is_a_no_op():
    import long_context_sparse_mask_amd as hs
    # B = 0 or Tq = 0: OK without reading any pointer (NULLs are fine)
    for d in (_desc(B=0), _desc(Tq=0)):
        assert _mask(d, ptrs=(None, None, None, None)) == 0
        assert hs.lib.hip_sparse_attn(C.byref(d), None, None, None, None, None, 2048, 64, 1, None,
                                      None, 0, None) == 0
        assert hs.lib.hipsa_workspace_bytes(C.byref(d), 2048, 64, 1) == 0


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "long_context_sparse_mask_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.lower(), os.path.join(dirpath, f)


def test_binding_fails_loudly_without_the_library(tmp_path):
    """A copy of the binding beside no libhipsa.so must refuse to import (no fallback)."""
    import shutil
    pkg = tmp_path / "long_context_sparse_mask_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "long_context_sparse_mask_amd", "__init__.py"), pkg)
    code = "import sys; sys.path.insert(0, %r); import long_context_sparse_mask_amd" % str(tmp_path)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode != 0 and "not built" in r.stderr
    # the command the message names runs the build script by path, which
    # loads without the library (loaded here without building)
    shutil.copy(os.path.join(ROOT, "long_context_sparse_mask_amd", "build.py"), pkg)
    hint = r.stderr.strip().splitlines()[-1]
    assert "long_context_sparse_mask_amd/build.py" in hint
    code = "import runpy; runpy.run_path(%r, run_name='check')" % str(pkg / "build.py")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _cpu(shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("case", ["K_batch", "K_dim", "V_shape", "V_dtype", "out_shape", "out_dtype",
                                  "idx_shape", "nnz_dtype", "q_rank"])
def test_binding_rejects_mismatched_tensors(case):
    """Shape, element-type and device mismatches are caught in the binding
    before any pointer reaches the library: a K with another batch or head
    dim, a V unlike K, or a caller's `out` unlike q would otherwise send the
    kernels past the end of an allocation."""
    import torch
    import long_context_sparse_mask_amd as hs
    B, Hq, Hkv, T, d = 2, 8, 2, 256, 128
    q, K, V = _cpu((B, Hq, 1, d)), _cpu((B, Hkv, T, d)), _cpu((B, Hkv, T, d))
    idx = torch.zeros((B, Hkv, 1, 2), dtype=torch.int32)
    nnz = torch.zeros((B, Hkv, 1), dtype=torch.int32)
    out = _cpu((B, Hq, 1, d))
    if case == "K_batch":
        K = _cpu((B + 1, Hkv, T, d))
    elif case == "K_dim":
        K = _cpu((B, Hkv, T, 64))
    elif case == "V_shape":
        V = _cpu((B, Hkv, T - 1, d))
    elif case == "V_dtype":
        V = _cpu((B, Hkv, T, d), torch.float8_e5m2)
    elif case == "out_shape":
        out = _cpu((B, Hq, 1, 64))
    elif case == "out_dtype":
        out = _cpu((B, Hq, 1, d), torch.float32)
    elif case == "idx_shape":
        idx = torch.zeros((B, Hkv, 1, 3), dtype=torch.int32)
    elif case == "nnz_dtype":
        nnz = torch.zeros((B, Hkv, 1), dtype=torch.int64)
    elif case == "q_rank":
        q = _cpu((B, Hq, d))
    with pytest.raises(ValueError):
        hs.hip_sparse_attn(q, K, V, idx, nnz, 128, 64, 1, out=out)
    with pytest.raises(ValueError):
        hs.hip_sparse_attn_ex(q, K, V, idx, nnz, 128, 64, 1, out=out, sink=64)
    if case in ("K_batch", "K_dim", "idx_shape", "nnz_dtype", "q_rank"):
        with pytest.raises(ValueError):
            hs.hip_mask_estimate(q, K, 128, 64, 1, indices=idx, nnz=nnz)


def test_binding_rejects_mismatched_paged_tensors():
    import torch
    import long_context_sparse_mask_amd as hs
    B, Hq, Hkv, d, ps = 2, 8, 2, 128, 64
    q = _cpu((B, Hq, 1, d))
    Kp, Vp = _cpu((8, Hkv, ps, d)), _cpu((8, Hkv, ps, d))
    table = torch.zeros((B, 4), dtype=torch.int32)
    idx = torch.zeros((B, Hkv, 1, 2), dtype=torch.int32)
    nnz = torch.zeros((B, Hkv, 1), dtype=torch.int32)
    with pytest.raises(ValueError):  # V pool unlike K's
        hs.hip_sparse_attn_paged(q, Kp, _cpu((8, Hkv, ps, 64)), table, idx, nnz, 256, 128, 64)
    with pytest.raises(ValueError):  # out unlike q
        hs.hip_sparse_attn_paged(q, Kp, Vp, table, idx, nnz, 256, 128, 64, out=_cpu((B, Hq, 2, d)))
    with pytest.raises(ValueError):  # table for another batch
        hs.hip_mask_estimate_paged(q, Kp, torch.zeros((B + 1, 4), dtype=torch.int32), 256, 128, 64)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """hip_sparse_attn_noalloc keeps split partials in an 8 MiB library
    scratch: a shape needing more is refused before any HIP call, with the
    same argument checks as hip_sparse_attn before that."""
    import long_context_sparse_mask_amd as hs
    assert hs.NOALLOC_SCRATCH_BYTES == 8 << 20
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 2048, 64, 1, FAKE, None]
    # 128k x 4 decode: 32 problems x 16 splits x 4 heads x 130 floats = 1 MiB: fits, but the
    # invalid variants below fail first
    assert hs.lib.hip_sparse_attn_noalloc(C.byref(_desc(Hq=30)), *args) == ERR_SHAPE
    bad = list(args)
    bad[0] = None
    assert hs.lib.hip_sparse_attn_noalloc(C.byref(_desc()), *bad) == ERR_NULL
    bad = list(args)
    bad[8] = C.c_void_p(0x1008)  # out
    assert hs.lib.hip_sparse_attn_noalloc(C.byref(_desc()), *bad) == ERR_ALIGN
    # 64 query rows x 8 KV heads x 64 splits (k = 8192 keys) x 4 heads x 130 floats: 68 MB
    big = _desc(Tq=64, T=65536, T_cap=65536)
    need = hs.lib.hipsa_workspace_bytes(C.byref(big), 8192, 64, 1)
    assert need > hs.NOALLOC_SCRATCH_BYTES
    big_args = list(args)
    big_args[5] = 8192
    assert hs.lib.hip_sparse_attn_noalloc(C.byref(big), *big_args) == ERR_WS
    assert "scratch" in hs.lib.hipsa_last_error().decode()
    # empty problems: no pointer is read
    assert hs.lib.hip_sparse_attn_noalloc(C.byref(_desc(B=0)), None, None, None, None, None, 2048,
                                          64, 1, None, None) == 0


def test_decode_step_rejects_invalid_arguments():
    """hip_decode_step runs the checks of both calls before any HIP call."""
    import long_context_sparse_mask_amd as hs

    def step(desc, ext=None, k=2048, bk=64, ptrs=None, ws=1 << 30):
        q, K, V, idx, nnz, out, wsp = ptrs or (FAKE,) * 7
        return hs.lib.hip_decode_step(C.byref(desc), C.byref(ext) if ext else None, q, K, V, k, bk,
                                      idx, nnz, out, wsp, ws, None)
    assert step(_desc(Hq=30)) == ERR_SHAPE
    assert step(_desc(), k=2000) == ERR_BLOCK
    assert step(_desc(dtype=9)) == ERR_DTYPE
    assert step(_desc(), ext=hs.Ext(None, 32, 0)) == ERR_BLOCK  # sink not a multiple of block_k
    assert step(_desc(), ptrs=(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE)) == ERR_NULL
    assert step(_desc(), ptrs=(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE)) == ERR_NULL
    odd = C.c_void_p(0x1008)
    assert step(_desc(), ptrs=(FAKE, FAKE, FAKE, FAKE, FAKE, odd, FAKE)) == ERR_ALIGN
    assert step(_desc(), ws=0) == ERR_WS
    big = _desc(B=4, T=131072, T_cap=131072)
    need = hs.lib.hipsa_decode_step_workspace_bytes(C.byref(big), None, 2048, 64)
    # 32 problems x 8 splits x 4 heads x 130 floats of partials, then 32 arrival counters
    assert need == 32 * 8 * 4 * 130 * 4 + 32 * 4
    assert step(big, ws=need - 1) == ERR_WS
    assert step(_desc(), ptrs=(FAKE,) * 6 + (C.c_void_p(0x1008),)) == ERR_ALIGN  # workspace
    pages = _pages(page_size=48)
    assert step(_desc(T_cap=0), ext=hs.Ext(C.pointer(pages), 0, 0)) == ERR_PAGES
    # empty problems read no pointer
    assert hs.lib.hip_decode_step(C.byref(_desc(B=0)), None, None, None, None, 2048, 64, None,
                                  None, None, None, 0, None) == 0
