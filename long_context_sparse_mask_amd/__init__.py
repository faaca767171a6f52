"""Python binding of libhipsa: HiP mask estimation and block-sparse attention on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libhipsa.so; torch supplies device memory and the current stream.
There is no fallback: importing this package fails if the library is not
built (``python long_context_sparse_mask_amd/build.py``).

Layouts (contiguous): q [B,Hq,Tq,d]; K, V [B,Hkv,T_cap,d] with the first T
rows valid; indices [B,Hkv,NQB,k/block_k] int32; nnz [B,Hkv,NQB] int32.
Element types (q, K/V): (float32, float32), (bfloat16, bfloat16), or
(bfloat16, float8_e5m2) for an fp8 KV cache; out has q's type.
Paged KV cache (the *_paged calls): K, V [num_pages, Hkv, page_size, d] and
block_table int32 [B, max_pages]; position t of sequence b is row
t % page_size of page block_table[b, t // page_size].
Dense part (the *_ex calls): `sink` first tokens and the last `window`
tokens' blocks are attended by every row and left out of the search.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # loads the HIP runtime first, so libhipsa binds to the same one

__all__ = ["hip_mask_estimate", "hip_sparse_attn", "hip_mask_estimate_paged",
           "hip_sparse_attn_paged", "hip_mask_estimate_ex", "hip_sparse_attn_ex",
           "hip_sparse_attn_noalloc", "hip_decode_step", "hip_mask_estimate_stages",
           "hipsa_stages_workspace_bytes", "hipsa_decode_step_workspace_bytes",
           "hipsa_workspace_bytes", "hipsa_workspace_bytes_ex",
           "HipsaError", "LIB_PATH", "lib", "NOALLOC_SCRATCH_BYTES"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhipsa.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python long_context_sparse_mask_amd/build.py`")

lib = C.CDLL(LIB_PATH)

HIPSA_F32, HIPSA_BF16, HIPSA_BF16_E5M2 = 0, 1, 2
SIZE_MAX = (1 << (8 * C.sizeof(C.c_size_t))) - 1
NOALLOC_SCRATCH_BYTES = 8 << 20  # HIPSA_NOALLOC_SCRATCH_BYTES


class Desc(C.Structure):
    _fields_ = [("B", C.c_int64), ("Hq", C.c_int64), ("Hkv", C.c_int64), ("Tq", C.c_int64),
                ("T", C.c_int64), ("T_cap", C.c_int64), ("d", C.c_int64), ("causal", C.c_int32),
                ("dtype", C.c_int32)]


class Pages(C.Structure):
    _fields_ = [("table", C.c_void_p), ("max_pages", C.c_int64), ("page_size", C.c_int64),
                ("num_pages", C.c_int64)]


class Ext(C.Structure):
    _fields_ = [("pages", C.POINTER(Pages)), ("sink", C.c_int64), ("window", C.c_int64)]


class Stage(C.Structure):
    _fields_ = [("chunk_size", C.c_int64), ("k", C.c_int64)]


_P, _I64, _SZ = C.c_void_p, C.c_int64, C.c_size_t
lib.hip_mask_estimate.argtypes = [C.POINTER(Desc), _P, _P, _I64, _I64, _I64, _P, _P, _P, _SZ, _P]
lib.hip_mask_estimate.restype = C.c_int
lib.hip_sparse_attn.argtypes = [C.POINTER(Desc), _P, _P, _P, _P, _P, _I64, _I64, _I64, _P, _P,
                                _SZ, _P]
lib.hip_sparse_attn.restype = C.c_int
lib.hip_mask_estimate_paged.argtypes = [C.POINTER(Desc), C.POINTER(Pages), _P, _P, _I64, _I64, _I64,
                                        _P, _P, _P, _SZ, _P]
lib.hip_mask_estimate_paged.restype = C.c_int
lib.hip_sparse_attn_paged.argtypes = [C.POINTER(Desc), C.POINTER(Pages), _P, _P, _P, _P, _P, _I64,
                                      _I64, _I64, _P, _P, _SZ, _P]
lib.hip_sparse_attn_paged.restype = C.c_int
lib.hip_mask_estimate_ex.argtypes = [C.POINTER(Desc), C.POINTER(Ext), _P, _P, _I64, _I64, _I64, _P,
                                     _P, _P, _SZ, _P]
lib.hip_mask_estimate_ex.restype = C.c_int
lib.hip_sparse_attn_ex.argtypes = [C.POINTER(Desc), C.POINTER(Ext), _P, _P, _P, _P, _P, _I64, _I64,
                                   _I64, _P, _P, _SZ, _P]
lib.hip_sparse_attn_ex.restype = C.c_int
lib.hip_mask_estimate_stages.argtypes = [C.POINTER(Desc), C.POINTER(Ext), C.POINTER(Stage),
                                         C.c_int32, _P, _P, _I64, _P, _P, _P, _SZ, _P]
lib.hip_mask_estimate_stages.restype = C.c_int
lib.hipsa_stages_workspace_bytes.argtypes = [C.POINTER(Desc), C.POINTER(Ext), C.POINTER(Stage),
                                             C.c_int32, _I64]
lib.hipsa_stages_workspace_bytes.restype = _SZ
lib.hip_decode_step.argtypes = [C.POINTER(Desc), C.POINTER(Ext), _P, _P, _P, _I64, _I64, _P, _P, _P,
                                _P, _SZ, _P]
lib.hip_decode_step.restype = C.c_int
lib.hipsa_decode_step_workspace_bytes.argtypes = [C.POINTER(Desc), C.POINTER(Ext), _I64, _I64]
lib.hipsa_decode_step_workspace_bytes.restype = C.c_size_t
lib.hip_sparse_attn_noalloc.argtypes = [C.POINTER(Desc), _P, _P, _P, _P, _P, _I64, _I64, _I64, _P,
                                        _P]
lib.hip_sparse_attn_noalloc.restype = C.c_int
lib.hipsa_workspace_bytes_ex.argtypes = [C.POINTER(Desc), C.POINTER(Ext), _I64, _I64, _I64]
lib.hipsa_workspace_bytes_ex.restype = C.c_size_t
lib.hipsa_workspace_bytes.argtypes = [C.POINTER(Desc), _I64, _I64, _I64]
lib.hipsa_workspace_bytes.restype = C.c_size_t
lib.hipsa_last_error.argtypes = []
lib.hipsa_last_error.restype = C.c_char_p


class HipsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"hipsa error {code}: {msg}")
        self.code = code


def _check(rc: int):
    if rc != 0:
        raise HipsaError(rc, lib.hipsa_last_error().decode())


_TYPE_PAIRS = {(torch.float32, torch.float32): HIPSA_F32,
               (torch.bfloat16, torch.bfloat16): HIPSA_BF16,
               (torch.bfloat16, torch.float8_e5m2): HIPSA_BF16_E5M2}


def _dtype_code(q: torch.Tensor, K: torch.Tensor) -> int:
    code = _TYPE_PAIRS.get((q.dtype, K.dtype))
    if code is None:
        raise TypeError(f"unsupported element types q={q.dtype}, K={K.dtype}")
    return code


def make_desc(q: torch.Tensor, K: torch.Tensor, T: int | None = None, causal: bool = True) -> Desc:
    if q.dim() != 4 or K.dim() != 4:
        raise ValueError("q must be [B, Hq, Tq, d] and K [B, Hkv, T_cap, d]")
    B, Hq, Tq, d = q.shape
    Bk, Hkv, T_cap, dk = K.shape
    if Bk != B or dk != d:
        raise ValueError(f"K {tuple(K.shape)} does not match q {tuple(q.shape)} in batch or "
                         "head dim")
    return Desc(B, Hq, Hkv, Tq, T_cap if T is None else T, T_cap, d, int(bool(causal)),
                _dtype_code(q, K))


def _check_v(K: torch.Tensor, V: torch.Tensor):
    """V must match K exactly (shape, element type, device): the kernels read
    both through one row layout."""
    if V.dtype != K.dtype or V.shape != K.shape or V.device != K.device:
        raise ValueError(f"V {tuple(V.shape)} {V.dtype} must have K's shape, dtype and device "
                         f"({tuple(K.shape)} {K.dtype})")


def _check_out(out: torch.Tensor, q: torch.Tensor):
    """A caller-supplied output must be exactly what the kernels write: q's
    shape, element type and device (a smaller buffer would be overrun)."""
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device:
        raise ValueError(f"out {tuple(out.shape)} {out.dtype} on {out.device} must have q's shape, "
                         f"dtype and device ({tuple(q.shape)} {q.dtype} on {q.device})")


def _check_lists(indices: torch.Tensor, nnz: torch.Tensor, desc: Desc, nqb: int, kb: int,
                 dev: torch.device):
    if tuple(indices.shape) != (desc.B, desc.Hkv, nqb, kb) or indices.dtype != torch.int32:
        raise ValueError("indices must be int32 [B, Hkv, NQB, k/block_k]")
    if tuple(nnz.shape) != (desc.B, desc.Hkv, nqb) or nnz.dtype != torch.int32:
        raise ValueError("nnz must be int32 [B, Hkv, NQB]")
    if indices.device != dev or nnz.device != dev:
        raise ValueError("indices and nnz must be on q's device")


def _on(dev: torch.device):
    """Marshaller of device pointers for one call: every tensor must sit on `dev`."""
    return lambda t, name: _dev_ptr(t, name, dev)


def _stream(dev: torch.device, stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev_ptr(t: torch.Tensor, name: str, dev: torch.device | None = None) -> int:
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, q on {dev}: every tensor of a call must be on "
                         "one device")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def hipsa_workspace_bytes(q, K, k: int, block_k: int, block_q: int = 1, *, T=None,
                          causal=True) -> int:
    n = lib.hipsa_workspace_bytes(C.byref(make_desc(q, K, T, causal)), k, block_k, block_q)
    if n == SIZE_MAX:
        raise HipsaError(-2, lib.hipsa_last_error().decode())
    return n


def hip_mask_estimate(q, K, k: int, block_k: int, block_q: int = 1, *, T=None, causal=True,
                      indices=None, nnz=None, stream=None):
    """Per (batch, kv head, query block): the ids of the selected key blocks
    (ascending, -1 padded) and their count.  Returns (indices, nnz)."""
    p = _on(q.device)  # device pointer of a tensor on q's device
    desc = make_desc(q, K, T, causal)
    nqb = -(-desc.Tq // block_q)
    kb = k // block_k if block_k > 0 else 0
    if indices is None:
        indices = torch.empty((desc.B, desc.Hkv, nqb, kb), dtype=torch.int32, device=q.device)
    if nnz is None:
        nnz = torch.empty((desc.B, desc.Hkv, nqb), dtype=torch.int32, device=q.device)
    _check_lists(indices, nnz, desc, nqb, kb, q.device)
    if desc.B * desc.Tq == 0:
        return indices, nnz
    _check(lib.hip_mask_estimate(C.byref(desc), p(q, "q"), p(K, "K"), k, block_k, block_q,
                                 p(indices, "indices"), p(nnz, "nnz"), None, 0,
                                 _stream(q.device, stream)))
    return indices, nnz


def hip_sparse_attn(q, K, V, indices, nnz, k: int, block_k: int, block_q: int = 1, *, T=None,
                    causal=True, out=None, workspace=None, stream=None):
    """Softmax attention of every query row over the tokens of its listed key
    blocks.  Returns out [B,Hq,Tq,d] in q's dtype."""
    p = _on(q.device)  # device pointer of a tensor on q's device
    desc = make_desc(q, K, T, causal)
    _check_v(K, V)
    nqb = -(-desc.Tq // block_q)
    kb = k // block_k if block_k > 0 else 0
    _check_lists(indices, nnz, desc, nqb, kb, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q)
    if desc.B * desc.Tq == 0:
        return out
    need = hipsa_workspace_bytes(q, K, k, block_k, block_q, T=T, causal=causal)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = p(workspace, "workspace") if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hip_sparse_attn(C.byref(desc), p(q, "q"), p(K, "K"), p(V, "V"),
                               p(indices, "indices"), p(nnz, "nnz"), k, block_k, block_q,
                               p(out, "out"), ws_ptr, ws_len, _stream(q.device, stream)))
    return out


def hip_sparse_attn_noalloc(q, K, V, indices, nnz, k: int, block_k: int, block_q: int = 1, *,
                            T=None, causal=True, out=None, stream=None):
    """hip_sparse_attn with the split partials in the library's own per-GPU
    scratch (no workspace).  `out` must be given (the call allocates nothing;
    pass out=None only outside graph capture, to let torch allocate it here).
    Calls on one GPU must be ordered on one stream."""
    p = _on(q.device)  # device pointer of a tensor on q's device
    desc = make_desc(q, K, T, causal)
    _check_v(K, V)
    nqb = -(-desc.Tq // block_q)
    kb = k // block_k if block_k > 0 else 0
    _check_lists(indices, nnz, desc, nqb, kb, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q)
    if desc.B * desc.Tq == 0:
        return out
    _check(lib.hip_sparse_attn_noalloc(C.byref(desc), p(q, "q"), p(K, "K"), p(V, "V"),
                                       p(indices, "indices"), p(nnz, "nnz"), k, block_k, block_q,
                                       p(out, "out"), _stream(q.device, stream)))
    return out


# ------------------------------------------------------------------ paged KV cache

def _paged_desc(q, K_pages, block_table, T, causal):
    p = _on(q.device)  # device pointer of a tensor on q's device
    if (q.dim() != 4 or K_pages.dim() != 4 or block_table.dim() != 2
            or block_table.dtype != torch.int32):
        raise ValueError("q must be [B, Hq, Tq, d], K and V [num_pages, Hkv, page_size, d] and "
                         "block_table int32 [B, max_pages]")
    B, Hq, Tq, d = q.shape
    num_pages, Hkv, page_size, dk = K_pages.shape
    if dk != d or block_table.shape[0] != B:
        raise ValueError("K's head dim or block_table's batch does not match q")
    desc = Desc(B, Hq, Hkv, Tq, T, T, d, int(bool(causal)), _dtype_code(q, K_pages))
    pages = Pages(p(block_table, "block_table"), block_table.shape[1], page_size,
                  num_pages)
    return desc, pages


def hip_mask_estimate_paged(q, K_pages, block_table, T: int, k: int, block_k: int,
                            block_q: int = 1, *, causal=True, indices=None, nnz=None, stream=None):
    """hip_mask_estimate on a paged KV cache.  Returns (indices, nnz)."""
    p = _on(q.device)  # device pointer of a tensor on q's device
    desc, pages = _paged_desc(q, K_pages, block_table, T, causal)
    nqb = -(-desc.Tq // block_q)
    kb = k // block_k if block_k > 0 else 0
    if indices is None:
        indices = torch.empty((desc.B, desc.Hkv, nqb, kb), dtype=torch.int32, device=q.device)
    if nnz is None:
        nnz = torch.empty((desc.B, desc.Hkv, nqb), dtype=torch.int32, device=q.device)
    _check_lists(indices, nnz, desc, nqb, kb, q.device)
    if desc.B * desc.Tq == 0:
        return indices, nnz
    _check(lib.hip_mask_estimate_paged(C.byref(desc), C.byref(pages), p(q, "q"),
                                       p(K_pages, "K"), k, block_k, block_q,
                                       p(indices, "indices"), p(nnz, "nnz"), None, 0,
                                       _stream(q.device, stream)))
    return indices, nnz


def hip_sparse_attn_paged(q, K_pages, V_pages, block_table, indices, nnz, T: int, k: int,
                          block_k: int, block_q: int = 1, *, causal=True, out=None, workspace=None,
                          stream=None):
    """hip_sparse_attn on a paged KV cache.  Returns out [B,Hq,Tq,d] in q's dtype."""
    p = _on(q.device)  # device pointer of a tensor on q's device
    desc, pages = _paged_desc(q, K_pages, block_table, T, causal)
    _check_v(K_pages, V_pages)
    nqb = -(-desc.Tq // block_q)
    kb = k // block_k if block_k > 0 else 0
    _check_lists(indices, nnz, desc, nqb, kb, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q)
    if desc.B * desc.Tq == 0:
        return out
    need = lib.hipsa_workspace_bytes(C.byref(desc), k, block_k, block_q)
    if need == SIZE_MAX:
        raise HipsaError(-2, lib.hipsa_last_error().decode())
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = p(workspace, "workspace") if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hip_sparse_attn_paged(C.byref(desc), C.byref(pages), p(q, "q"),
                                     p(K_pages, "K"),
                                     p(V_pages, "V"),
                                     p(indices, "indices"), p(nnz, "nnz"), k, block_k,
                                     block_q, p(out, "out"), ws_ptr, ws_len,
                                     _stream(q.device, stream)))
    return out


# ------------------------------------------------------------------ dense part and layout options

def _ext_desc(q, K, T, causal, sink, window, block_table):
    """(desc, ext, pages): the paged layout when block_table is given (T required)."""
    if block_table is not None:
        if T is None:
            raise ValueError("T is required with a block_table")
        desc, pages = _paged_desc(q, K, block_table, T, causal)
        return desc, Ext(C.pointer(pages), sink, window), pages
    return make_desc(q, K, T, causal), Ext(None, sink, window), None


def hipsa_workspace_bytes_ex(q, K, k: int, block_k: int, block_q: int = 1, *, T=None, causal=True,
                             sink=0, window=0, block_table=None) -> int:
    desc, ext, _pages = _ext_desc(q, K, T, causal, sink, window, block_table)
    n = lib.hipsa_workspace_bytes_ex(C.byref(desc), C.byref(ext), k, block_k, block_q)
    if n == SIZE_MAX:
        raise HipsaError(-2, lib.hipsa_last_error().decode())
    return n


def hip_mask_estimate_ex(q, K, k: int, block_k: int, block_q: int = 1, *, T=None, causal=True,
                         sink=0, window=0, block_table=None, indices=None, nnz=None, stream=None):
    """hip_mask_estimate with a dense part (sink, window tokens) and optionally a
    paged KV cache (block_table).  Returns (indices, nnz) of the searched blocks."""
    p = _on(q.device)  # device pointer of a tensor on q's device
    desc, ext, _pages = _ext_desc(q, K, T, causal, sink, window, block_table)
    nqb = -(-desc.Tq // block_q)
    kb = k // block_k if block_k > 0 else 0
    if indices is None:
        indices = torch.empty((desc.B, desc.Hkv, nqb, kb), dtype=torch.int32, device=q.device)
    if nnz is None:
        nnz = torch.empty((desc.B, desc.Hkv, nqb), dtype=torch.int32, device=q.device)
    _check_lists(indices, nnz, desc, nqb, kb, q.device)
    if desc.B * desc.Tq == 0:
        return indices, nnz
    _check(lib.hip_mask_estimate_ex(C.byref(desc), C.byref(ext), p(q, "q"),
                                    p(K, "K"),
                                    k, block_k, block_q, p(indices, "indices"),
                                    p(nnz, "nnz"), None, 0, _stream(q.device, stream)))
    return indices, nnz


def _stage_array(stages):
    return (Stage * max(len(stages), 1))(*[Stage(c, 0 if k is None else k) for c, k in stages])


def hipsa_stages_workspace_bytes(q, K, stages, block_k: int, *, T=None, causal=True, sink=0,
                                 window=0, block_table=None) -> int:
    desc, ext, _pages = _ext_desc(q, K, T, causal, sink, window, block_table)
    n = lib.hipsa_stages_workspace_bytes(C.byref(desc), C.byref(ext), _stage_array(stages),
                                         len(stages), block_k)
    if n == SIZE_MAX:
        raise HipsaError(-9, lib.hipsa_last_error().decode())
    return n


def hip_mask_estimate_stages(q, K, stages, block_k: int, *, T=None, causal=True, sink=0, window=0,
                             block_table=None, indices=None, nnz=None, workspace=None,
                             stream=None):
    """Multi-stage search for per-row problems (block_q = 1).  stages: a list of
    (chunk_size, k) in tokens, the first k None (stage 0 keeps every chunk), the
    last chunk_size block_k.  Returns (indices, nnz) with k = stages[-1][1].
    `workspace`: hipsa_stages_workspace_bytes() bytes, zero-filled before its
    first use (allocated, zeroed, when None and needed)."""
    p = _on(q.device)  # device pointer of a tensor on q's device
    desc, ext, _pages = _ext_desc(q, K, T, causal, sink, window, block_table)
    arr = _stage_array(stages)
    k_last = stages[-1][1] if stages and stages[-1][1] is not None else 0
    kb = k_last // block_k if block_k > 0 else 0
    if indices is None:
        indices = torch.empty((desc.B, desc.Hkv, desc.Tq, kb), dtype=torch.int32, device=q.device)
    if nnz is None:
        nnz = torch.empty((desc.B, desc.Hkv, desc.Tq), dtype=torch.int32, device=q.device)
    _check_lists(indices, nnz, desc, desc.Tq, kb, q.device)
    if desc.B * desc.Tq == 0:
        return indices, nnz
    need = lib.hipsa_stages_workspace_bytes(C.byref(desc), C.byref(ext), arr, len(stages), block_k)
    if workspace is None and 0 < need < SIZE_MAX:
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device)
    ws_ptr = p(workspace, "workspace") if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hip_mask_estimate_stages(C.byref(desc), C.byref(ext), arr, len(stages), p(q, "q"),
                                        p(K, "K"), block_k, p(indices, "indices"),
                                        p(nnz, "nnz"), ws_ptr, ws_len, _stream(q.device, stream)))
    return indices, nnz


def hip_sparse_attn_ex(q, K, V, indices, nnz, k: int, block_k: int, block_q: int = 1, *, T=None,
                       causal=True, sink=0, window=0, block_table=None, out=None, workspace=None,
                       stream=None):
    """hip_sparse_attn over the dense part and the listed blocks, optionally on a
    paged KV cache.  Returns out [B,Hq,Tq,d] in q's dtype."""
    p = _on(q.device)  # device pointer of a tensor on q's device
    desc, ext, _pages = _ext_desc(q, K, T, causal, sink, window, block_table)
    _check_v(K, V)
    nqb = -(-desc.Tq // block_q)
    kb = k // block_k if block_k > 0 else 0
    _check_lists(indices, nnz, desc, nqb, kb, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q)
    if desc.B * desc.Tq == 0:
        return out
    need = lib.hipsa_workspace_bytes_ex(C.byref(desc), C.byref(ext), k, block_k, block_q)
    if need == SIZE_MAX:
        raise HipsaError(-2, lib.hipsa_last_error().decode())
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_ptr = p(workspace, "workspace") if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.hip_sparse_attn_ex(C.byref(desc), C.byref(ext), p(q, "q"),
                                  p(K, "K"),
                                  p(V, "V"), p(indices, "indices"),
                                  p(nnz, "nnz"), k, block_k, block_q, p(out, "out"),
                                  ws_ptr, ws_len, _stream(q.device, stream)))
    return out


# ------------------------------------------------------------------ one decode step

def hipsa_decode_step_workspace_bytes(q, K, k: int, block_k: int, *, T=None, causal=True, sink=0,
                                      window=0, block_table=None) -> int:
    desc, ext, _pages = _ext_desc(q, K, T, causal, sink, window, block_table)
    n = lib.hipsa_decode_step_workspace_bytes(C.byref(desc), C.byref(ext), k, block_k)
    if n == SIZE_MAX:
        raise HipsaError(-2, lib.hipsa_last_error().decode())
    return n


def hip_decode_step(q, K, V, k: int, block_k: int, *, T=None, causal=True, sink=0, window=0,
                    block_table=None, indices=None, nnz=None, out=None, workspace=None,
                    stream=None):
    """hip_mask_estimate then hip_sparse_attn (block_q = 1) in one call.
    Returns (out, indices, nnz), bit for bit the two calls' results.  A
    caller's `workspace` (hipsa_decode_step_workspace_bytes bytes) must be
    zero-filled before its first use; every call leaves it reusable."""
    p = _on(q.device)  # device pointer of a tensor on q's device
    desc, ext, _pages = _ext_desc(q, K, T, causal, sink, window, block_table)
    _check_v(K, V)
    kb = k // block_k if block_k > 0 else 0
    if indices is None:
        indices = torch.empty((desc.B, desc.Hkv, desc.Tq, kb), dtype=torch.int32, device=q.device)
    if nnz is None:
        nnz = torch.empty((desc.B, desc.Hkv, desc.Tq), dtype=torch.int32, device=q.device)
    _check_lists(indices, nnz, desc, desc.Tq, kb, q.device)
    if out is None:
        out = torch.empty_like(q)
    _check_out(out, q)
    if desc.B * desc.Tq == 0:
        return out, indices, nnz
    if workspace is None:  # zero-filled: it holds the arrival counters
        workspace = torch.zeros(hipsa_decode_step_workspace_bytes(
            q, K, k, block_k, T=T, causal=causal, sink=sink, window=window,
            block_table=block_table), dtype=torch.uint8, device=q.device)
    ws_ptr = p(workspace, "workspace")
    ws_len = workspace.numel() * workspace.element_size()
    _check(lib.hip_decode_step(C.byref(desc), C.byref(ext), p(q, "q"), p(K, "K"), p(V, "V"), k,
                               block_k, p(indices, "indices"), p(nnz, "nnz"), p(out, "out"),
                               ws_ptr, ws_len, _stream(q.device, stream)))
    return out, indices, nnz
