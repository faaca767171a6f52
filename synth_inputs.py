"""Seeded synthetic inputs for HiP decode and chunked-prefill attention.

Both the CPU oracle and the GPU library consume what this module makes; it
holds none of the method's arithmetic (no scoring, no selection, no softmax).
It only draws random numbers, shapes keys along the sequence with an AR(1)
recurrence, scales the key rows of "needle" blocks, and rounds to the
workload's element types.

Why AR(1) keys: the HiP summary page ("A Training-Free Sub-quadratic Cost
Transformer Model Serving Framework with Hierarchically Pruned Attention",
Approach) rests the method on attention locality, i.e. nearby keys score
alike.  A stationary AR(1) process along the sequence axis is the plainest
synthetic stand-in for that property; it says nothing about model accuracy.

Recipe (per workload, seed s):
  * numpy SeedSequence(s).spawn(4) -> independent PCG64 streams for q, K, V
    and the needle draw; the K and V streams are spawned again per
    (batch, kv-head) slice, so results do not depend on thread count.
  * q, V ~ i.i.d. N(0, 1).
  * K[b, g, :, x] is AR(1) along the sequence: x_0 = e_0 / sqrt(1 - rho^2)
    (stationary start), x_t = rho * x_{t-1} + e_t, e_t ~ N(0, 1).
  * needle workloads: `needles` distinct block ids drawn from the needle
    stream; the K rows of those blocks (all batch entries and kv heads) are
    multiplied by `needle_scale`.
  * everything is drawn in float32 and, for bf16 workloads, rounded once to
    bf16 with round-to-nearest-even (torch's CPU cast).  "bf16_e5m2"
    workloads (an fp8 KV cache) round q to bf16 and K, V to fp8 E5M2, also
    once and to nearest even, from the same float32 draws.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, asdict, replace

import numpy as np
import scipy.signal as _signal
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    dtype: str          # "f32", "bf16" or "bf16_e5m2" (bf16 q, fp8 E5M2 K/V)
    T: int              # keys per sequence
    Tq: int             # query rows (1 = decode)
    block_k: int
    k: int              # selected keys per query block (multiple of block_k)
    block_q: int
    causal: int
    rho: float
    needles: int = 0
    needle_scale: float = 8.0
    seed: int = 1000

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def kb(self) -> int:
        return self.k // self.block_k

    @property
    def nqb(self) -> int:
        return -(-self.Tq // self.block_q)

    def as_dict(self) -> dict:
        return asdict(self)


# The five workloads: a tiny fp32 decode, Llama-3.1-8B-shaped decode at 32k and
# 128k (batch 4), a 4096-token causal prefill chunk at the end of a 32k
# sequence, and a 1M-token decode with 16 needle blocks.
WORKLOADS = {
    "tiny_decode": Workload("tiny_decode", B=1, Hq=1, Hkv=1, d=64, dtype="f32", T=1024, Tq=1,
                            block_k=8, k=128, block_q=1, causal=1, rho=0.95, seed=1000),
    "decode_32k": Workload("decode_32k", B=1, Hq=32, Hkv=8, d=128, dtype="bf16", T=32768, Tq=1,
                           block_k=64, k=2048, block_q=1, causal=1, rho=0.9, seed=1001),
    "decode_128k_b4": Workload("decode_128k_b4", B=4, Hq=32, Hkv=8, d=128, dtype="bf16", T=131072,
                               Tq=1, block_k=64, k=2048, block_q=1, causal=1, rho=0.9, seed=1002),
    "prefill_32k_chunk4k": Workload("prefill_32k_chunk4k", B=1, Hq=32, Hkv=8, d=128, dtype="bf16",
                                    T=32768, Tq=4096, block_k=64, k=2048, block_q=64, causal=1,
                                    rho=0.9, seed=1003),
    "decode_1m_needles": Workload("decode_1m_needles", B=1, Hq=32, Hkv=8, d=128, dtype="bf16",
                                  T=1048576, Tq=1, block_k=64, k=4096, block_q=1, causal=1,
                                  rho=0.9, needles=16, needle_scale=8.0, seed=1004),
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (e.g. a smaller T)."""
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def _threads() -> int:
    return max(1, min(16, len(_affinity())))


def _affinity():
    try:
        import os
        return os.sched_getaffinity(0)
    except Exception:  # pragma: no cover
        return range(8)


def _normal(seq: np.random.SeedSequence, shape) -> np.ndarray:
    return np.random.Generator(np.random.PCG64(seq)).standard_normal(shape, dtype=np.float32)


def _ar1_slice(seq: np.random.SeedSequence, T: int, d: int, rho: float) -> np.ndarray:
    """One [T, d] key slice: d independent stationary AR(1) series along T."""
    e = _normal(seq, (d, T))
    e[:, 0] /= np.float32(math.sqrt(1.0 - rho * rho))
    x = _signal.lfilter(np.array([1.0], np.float32), np.array([1.0, -rho], np.float32), e, axis=1)
    return np.ascontiguousarray(x.T, dtype=np.float32)


_Q_TYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "bf16_e5m2": torch.bfloat16}
_KV_TYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "bf16_e5m2": torch.float8_e5m2}


def _to_dtype(a: np.ndarray, tdt: torch.dtype) -> torch.Tensor:
    t = torch.from_numpy(a)
    return t.clone() if tdt == torch.float32 else t.to(tdt)


def needle_blocks(w: Workload) -> list[int]:
    if w.needles <= 0:
        return []
    seq = np.random.SeedSequence(w.seed).spawn(4)[3]
    nblk = -(-w.T // w.block_k)
    rng = np.random.Generator(np.random.PCG64(seq))
    return sorted(int(x) for x in rng.choice(nblk, size=w.needles, replace=False))


def make_inputs(w: Workload, T_cap: int | None = None) -> dict:
    """Seeded q [B,Hq,Tq,d], K and V [B,Hkv,T_cap,d] as CPU torch tensors.

    Rows T..T_cap-1 of K and V (spare cache capacity) are zero.
    """
    T_cap = w.T if T_cap is None else T_cap
    assert T_cap >= w.T
    s_q, s_k, s_v, _ = np.random.SeedSequence(w.seed).spawn(4)
    qdt, kvdt = _Q_TYPE[w.dtype], _KV_TYPE[w.dtype]
    q = _to_dtype(_normal(s_q, (w.B, w.Hq, w.Tq, w.d)), qdt)
    K = torch.zeros((w.B, w.Hkv, T_cap, w.d), dtype=kvdt)
    V = torch.zeros((w.B, w.Hkv, T_cap, w.d), dtype=kvdt)
    k_seqs = s_k.spawn(w.B * w.Hkv)
    v_seqs = s_v.spawn(w.B * w.Hkv)
    needles = needle_blocks(w)

    def fill(i):
        b, g = divmod(i, w.Hkv)
        ks = _ar1_slice(k_seqs[i], w.T, w.d, w.rho)
        for blk in needles:
            ks[blk * w.block_k:(blk + 1) * w.block_k] *= np.float32(w.needle_scale)
        K[b, g, :w.T] = _to_dtype(ks, kvdt)
        del ks
        V[b, g, :w.T] = _to_dtype(_normal(v_seqs[i], (w.T, w.d)), kvdt)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(w.B * w.Hkv)))
    return {"q": q, "K": K, "V": V, "T_cap": T_cap, "needles": needles, "workload": w}
