"""ctypes front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the bench's
CPU-baseline leg may import this package; the product library never does.

Inputs are CPU torch tensors in the library's layouts: q [B,Hq,Tq,d], K and V
[B,Hkv,T_cap,d].  q is float32 or bfloat16; K and V share one type, float32,
bfloat16 or float8_e5m2 (the C code decodes every one of them to double
exactly).  Outputs are numpy arrays; attention rows are float64.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc: -O2, OpenMP over independent problems, no fast-math."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"],
                   check=True)
    os.replace(tmp, out)
    return out


class Shape(C.Structure):
    _fields_ = [("B", C.c_int64), ("Hq", C.c_int64), ("Hkv", C.c_int64), ("Tq", C.c_int64),
                ("T", C.c_int64), ("T_cap", C.c_int64), ("d", C.c_int64), ("k", C.c_int64),
                ("block_k", C.c_int64), ("block_q", C.c_int64), ("causal", C.c_int32),
                ("dtype", C.c_int32), ("kv_dtype", C.c_int32), ("sink", C.c_int64),
                ("window", C.c_int64)]


class Stage(C.Structure):
    _fields_ = [("chunk", C.c_int64), ("keep", C.c_int64)]


class Trace(C.Structure):
    _fields_ = [("max_rounds", C.c_int32), ("cap", C.c_int32), ("rounds", C.c_int32),
                ("n_cand", C.c_void_p), ("cand_start", C.c_void_p), ("cand_end", C.c_void_p),
                ("cand_centre", C.c_void_p), ("cand_score", C.c_void_p),
                ("cand_kept", C.c_void_p), ("rel_margin", C.c_void_p)]


def load(path: str | None = None):
    """Load the oracle library (building it first if it is not there).

    `path` selects another build of the same source (the mutation tests use it).
    """
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if path is None and not os.path.exists(p):
        build()
    lib = C.CDLL(p)
    P, I64, I32 = C.c_void_p, C.c_int64, C.c_int32
    lib.or_mask_one.argtypes = [C.POINTER(Shape), P, P, I64, I64, I64, P, P, P, C.POINTER(Trace)]
    lib.or_mask_all.argtypes = [C.POINTER(Shape), P, P, P, P, P, I32]
    lib.or_attn_row.argtypes = [C.POINTER(Shape), P, P, P, P, P, I64, I64, I64, P]
    lib.or_attn_all.argtypes = [C.POINTER(Shape), P, P, P, P, P, P, I32]
    for f in (lib.or_mask_one, lib.or_mask_all, lib.or_attn_row, lib.or_attn_all):
        f.restype = C.c_int
    lib.or_mask_reach.argtypes = [C.POINTER(Shape), P, P, I64, I64, I64, C.c_double, P, P, I64, I64]
    lib.or_mask_reach.restype = C.c_int64
    SP = C.POINTER(Stage)
    lib.or_mask_stages_one.argtypes = [C.POINTER(Shape), SP, I32, P, P, I64, I64, I64, P, P, P,
                                       C.POINTER(Trace)]
    lib.or_mask_stages_one.restype = C.c_int
    lib.or_mask_stages_all.argtypes = [C.POINTER(Shape), SP, I32, P, P, P, P, P, I32]
    lib.or_mask_stages_all.restype = C.c_int
    lib.or_mask_stages_reach.argtypes = [C.POINTER(Shape), SP, I32, P, P, I64, I64, I64, C.c_double,
                                         P, P, I64, I64]
    lib.or_mask_stages_reach.restype = C.c_int64
    lib.or_e5m2_value.argtypes = [C.c_uint8]
    lib.or_e5m2_value.restype = C.c_double
    if path is None:
        _lib = lib
    return lib


def _ptr(t) -> int:
    if isinstance(t, np.ndarray):
        assert t.flags["C_CONTIGUOUS"]
        return t.ctypes.data
    assert t.device.type == "cpu" and t.is_contiguous(), "oracle inputs are contiguous CPU tensors"
    return t.data_ptr()


_CODES = {torch.float32: 0, torch.bfloat16: 1, torch.float8_e5m2: 2}


def _dtype_code(t: torch.Tensor, kv: bool = False) -> int:
    code = _CODES.get(t.dtype)
    if code is None or (code == 2 and not kv):
        raise TypeError(f"oracle does not take {t.dtype} for {'K/V' if kv else 'q'}")
    return code


def shape(q, K, *, T, k, block_k, block_q, causal=1, sink=0, window=0) -> Shape:
    B, Hq, Tq, d = q.shape
    assert K.shape[0] == B and K.shape[3] == d
    return Shape(B, Hq, K.shape[1], Tq, T, K.shape[2], d, k, block_k, block_q, int(causal),
                 _dtype_code(q), _dtype_code(K, kv=True), sink, window)


def e5m2_values(lib=None) -> np.ndarray:
    """The oracle's decoding of all 256 E5M2 codes, float64 [256]."""
    lib = lib or load()
    return np.array([lib.or_e5m2_value(c) for c in range(256)], np.float64)


def nthreads(n: int | None = None) -> int:
    if n is not None:
        return n
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def mask_all(q, K, *, T, k, block_k, block_q, causal=1, sink=0, window=0, threads=None, lib=None):
    """Indices [B,Hkv,NQB,K_b], nnz [B,Hkv,NQB] and the min relative cut margin per problem."""
    lib = lib or load()
    s = shape(q, K, T=T, k=k, block_k=block_k, block_q=block_q, causal=causal, sink=sink,
              window=window)
    nqb = -(-s.Tq // block_q)
    kb = k // block_k
    idx = np.full((s.B, s.Hkv, nqb, kb), -1, np.int32)
    nnz = np.zeros((s.B, s.Hkv, nqb), np.int32)
    margin = np.zeros((s.B, s.Hkv, nqb), np.float64)
    rc = lib.or_mask_all(C.byref(s), _ptr(q), _ptr(K), idx.ctypes.data, nnz.ctypes.data,
                         margin.ctypes.data, nthreads(threads))
    assert rc == 0
    return idx, nnz, margin


def mask_one(q, K, b, g, qb, *, T, k, block_k, block_q, causal=1, sink=0, window=0, trace=False,
             lib=None, max_rounds=64):
    """One problem; with trace=True also the per-round candidates (sorted by rank)."""
    lib = lib or load()
    s = shape(q, K, T=T, k=k, block_k=block_k, block_q=block_q, causal=causal, sink=sink,
              window=window)
    kb = k // block_k
    idx = np.full(kb, -1, np.int32)
    nnz = np.zeros(1, np.int32)
    margin = np.zeros(1, np.float64)
    tr_ptr = None
    bufs = None
    if trace:
        cap = 2 * kb
        bufs = dict(n_cand=np.zeros(max_rounds, np.int32),
                    cand_start=np.zeros((max_rounds, cap), np.int64),
                    cand_end=np.zeros((max_rounds, cap), np.int64),
                    cand_centre=np.zeros((max_rounds, cap), np.int64),
                    cand_score=np.zeros((max_rounds, cap), np.float64),
                    cand_kept=np.zeros((max_rounds, cap), np.int32),
                    rel_margin=np.zeros(max_rounds, np.float64))
        tr = Trace(max_rounds, cap, 0, *(bufs[n].ctypes.data for n in
                                         ("n_cand", "cand_start", "cand_end", "cand_centre",
                                          "cand_score", "cand_kept", "rel_margin")))
        tr_ptr = C.byref(tr)
    rc = lib.or_mask_one(C.byref(s), _ptr(q), _ptr(K), b, g, qb, idx.ctypes.data,
                         nnz.ctypes.data, margin.ctypes.data, tr_ptr)
    assert rc == 0
    out = {"indices": idx, "nnz": int(nnz[0]), "margin": float(margin[0])}
    if trace:
        R = tr.rounds
        rounds = []
        for r in range(R):
            n = int(bufs["n_cand"][r])
            rounds.append({
                "start": bufs["cand_start"][r, :n].copy(), "end": bufs["cand_end"][r, :n].copy(),
                "centre": bufs["cand_centre"][r, :n].copy(),
                "score": bufs["cand_score"][r, :n].copy(),
                "kept": bufs["cand_kept"][r, :n].astype(bool),
                "rel_margin": float(bufs["rel_margin"][r])})
        out["rounds"] = rounds
    return out


def attn_all(q, K, V, indices, nnz, *, T, k, block_k, block_q, causal=1, sink=0, window=0, threads=None, lib=None):
    """Exact attention over the listed blocks, float64 [B,Hq,Tq,d]."""
    lib = lib or load()
    assert K.dtype == V.dtype and K.shape == V.shape
    s = shape(q, K, T=T, k=k, block_k=block_k, block_q=block_q, causal=causal, sink=sink,
              window=window)
    indices = np.ascontiguousarray(indices, np.int32)
    nnz = np.ascontiguousarray(nnz, np.int32)
    out = np.zeros((s.B, s.Hq, s.Tq, s.d), np.float64)
    rc = lib.or_attn_all(C.byref(s), _ptr(q), _ptr(K), _ptr(V), indices.ctypes.data,
                         nnz.ctypes.data, out.ctypes.data, nthreads(threads))
    assert rc == 0
    return out


def attn_row(q, K, V, indices, nnz, b, h, i, *, T, k, block_k, block_q, causal=1, sink=0, window=0, lib=None):
    lib = lib or load()
    assert K.dtype == V.dtype and K.shape == V.shape
    s = shape(q, K, T=T, k=k, block_k=block_k, block_q=block_q, causal=causal, sink=sink,
              window=window)
    indices = np.ascontiguousarray(indices, np.int32)
    nnz = np.ascontiguousarray(nnz, np.int32)
    out = np.zeros(s.d, np.float64)
    rc = lib.or_attn_row(C.byref(s), _ptr(q), _ptr(K), _ptr(V), indices.ctypes.data,
                         nnz.ctypes.data, b, h, i, out.ctypes.data)
    assert rc == 0
    return out


def mask_reach(q, K, b, g, qb, *, T, k, block_k, block_q, causal=1, sink=0, window=0, tol=1e-4,
               target=None, max_leaves=256, max_nodes=200000, lib=None):
    """Final lists the search reaches when every candidate score may move by
    (tol/2)*|score| (near ties at a cut resolved either way).

    Without `target`: (count, lists) with every distinct reachable list
    (ascending block ids, [count, K_b]; at most max_leaves stored).  With
    `target` (K_b ascending ids): (1 or 0, lists) -- whether the target is
    reachable.  Raises if the node budget runs out."""
    lib = lib or load()
    s = shape(q, K, T=T, k=k, block_k=block_k, block_q=block_q, causal=causal, sink=sink,
              window=window)
    kb = k // block_k
    leaves = np.full((max_leaves, kb), -1, np.int32)
    tgt = None
    if target is not None:
        tgt = np.ascontiguousarray(target, np.int32)
        assert tgt.shape == (kb,)
    n = lib.or_mask_reach(C.byref(s), _ptr(q), _ptr(K), b, g, qb, tol,
                          None if tgt is None else tgt.ctypes.data, leaves.ctypes.data, max_leaves,
                          max_nodes)
    if n < 0:
        raise RuntimeError(f"or_mask_reach failed ({n}: {'node budget' if n == -1 else 'memory'})")
    return int(n), leaves[:min(n, max_leaves)]


# ------------------------------------------------------------------ multi-stage search

def stage_array(stages, block_k):
    """A stage list [(chunk_size, k), ...] in tokens, as InfiniteHiP configures it
    (the first k is None: every chunk of the initial partition is kept), as the
    oracle's C array in blocks: (chunk blocks, chunks kept per round)."""
    arr = (Stage * len(stages))()
    for j, (chunk, k) in enumerate(stages):
        assert chunk % block_k == 0, "chunk sizes are multiples of block_k"
        arr[j].chunk = chunk // block_k
        if k is None:
            arr[j].keep = 0
        else:
            assert k % chunk == 0, "k is a multiple of the stage's chunk size"
            arr[j].keep = k // chunk
    return arr


def mask_stages_all(q, K, stages, *, T, block_k, causal=1, sink=0, window=0, threads=None,
                    lib=None):
    """The multi-stage search on every problem (block_q = 1): indices
    [B,Hkv,Tq,K_b], nnz, and the min relative cut margin per problem."""
    lib = lib or load()
    kb = stages[-1][1] // block_k
    s = shape(q, K, T=T, k=kb * block_k, block_k=block_k, block_q=1, causal=causal, sink=sink,
              window=window)
    st = stage_array(stages, block_k)
    idx = np.full((s.B, s.Hkv, s.Tq, kb), -1, np.int32)
    nnz = np.zeros((s.B, s.Hkv, s.Tq), np.int32)
    margin = np.zeros((s.B, s.Hkv, s.Tq), np.float64)
    rc = lib.or_mask_stages_all(C.byref(s), st, len(stages), _ptr(q), _ptr(K), idx.ctypes.data,
                                nnz.ctypes.data, margin.ctypes.data, nthreads(threads))
    assert rc == 0, rc
    return idx, nnz, margin


def mask_stages_reach(q, K, b, g, i, stages, *, T, block_k, causal=1, sink=0, window=0, tol=1e-4,
                      target=None, max_leaves=256, max_nodes=200000, lib=None):
    """mask_reach over a stage list (problem b, KV head g, query row i)."""
    lib = lib or load()
    kb = stages[-1][1] // block_k
    s = shape(q, K, T=T, k=kb * block_k, block_k=block_k, block_q=1, causal=causal, sink=sink,
              window=window)
    st = stage_array(stages, block_k)
    leaves = np.full((max_leaves, kb), -1, np.int32)
    tgt = None if target is None else np.ascontiguousarray(target, np.int32)
    n = lib.or_mask_stages_reach(C.byref(s), st, len(stages), _ptr(q), _ptr(K), b, g, i, tol,
                                 None if tgt is None else tgt.ctypes.data, leaves.ctypes.data,
                                 max_leaves, max_nodes)
    if n < 0:
        raise RuntimeError(f"or_mask_stages_reach failed ({n})")
    return int(n), leaves[:min(n, max_leaves)]


def mask_stages_one(q, K, b, g, i, stages, *, T, block_k, causal=1, sink=0, window=0, lib=None,
                    max_rounds=64, cap=8192):
    """One problem of the multi-stage search with its per-round trace (the
    rounds of every stage after the first, in order; candidates sorted by rank)."""
    lib = lib or load()
    kb = stages[-1][1] // block_k
    s = shape(q, K, T=T, k=kb * block_k, block_k=block_k, block_q=1, causal=causal, sink=sink,
              window=window)
    st = stage_array(stages, block_k)
    idx = np.full(kb, -1, np.int32)
    nnz = np.zeros(1, np.int32)
    margin = np.zeros(1, np.float64)
    bufs = dict(n_cand=np.zeros(max_rounds, np.int32),
                cand_start=np.zeros((max_rounds, cap), np.int64),
                cand_end=np.zeros((max_rounds, cap), np.int64),
                cand_centre=np.zeros((max_rounds, cap), np.int64),
                cand_score=np.zeros((max_rounds, cap), np.float64),
                cand_kept=np.zeros((max_rounds, cap), np.int32),
                rel_margin=np.zeros(max_rounds, np.float64))
    tr = Trace(max_rounds, cap, 0, *(bufs[n].ctypes.data for n in
                                     ("n_cand", "cand_start", "cand_end", "cand_centre",
                                      "cand_score", "cand_kept", "rel_margin")))
    rc = lib.or_mask_stages_one(C.byref(s), st, len(stages), _ptr(q), _ptr(K), b, g, i,
                                idx.ctypes.data, nnz.ctypes.data, margin.ctypes.data, C.byref(tr))
    assert rc == 0, rc
    rounds = []
    for r in range(tr.rounds):
        n = int(bufs["n_cand"][r])
        rounds.append({"start": bufs["cand_start"][r, :n].copy(), "end": bufs["cand_end"][r, :n].copy(),
                       "centre": bufs["cand_centre"][r, :n].copy(),
                       "score": bufs["cand_score"][r, :n].copy(),
                       "kept": bufs["cand_kept"][r, :n].astype(bool),
                       "rel_margin": float(bufs["rel_margin"][r])})
    return {"indices": idx, "nnz": int(nnz[0]), "margin": float(margin[0]), "rounds": rounds}
