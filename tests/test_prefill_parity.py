"""GPU parity of the chunked-prefill path (block_q = 64, bf16) against the CPU oracle.

Every case compares every problem and every output row, the 4096-token
chunk at the end of a 32k sequence included (at full size, in the bench's
launch configuration).
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from parity_util import compare_attention, full_parity, run_gpu

pytestmark = pytest.mark.gpu


def _report(name, r):
    print(f"[parity] {name}: problems={r['problems']} exempt={r['exempt']} "
          f"max_err={r['max_err']:.3e}", flush=True)


SMALL = {
    # several query blocks, causal, the last one ragged; T not a multiple of 64
    "ragged_causal": dict(T=3000, Tq=200, Hq=8, Hkv=2, k=512),
    # a chunk whose early query blocks see fewer than K_b blocks (dense rows)
    "dense_early_blocks": dict(T=1100, Tq=1000, Hq=4, Hkv=1, k=512),
    "bk8": dict(T=4096, Tq=128, Hq=4, Hkv=1, block_k=8, k=256),
    "bk16": dict(T=4096, Tq=128, Hq=4, Hkv=1, block_k=16, k=256),
    "bk32": dict(T=4096, Tq=192, Hq=4, Hkv=1, block_k=32, k=512),
    "d64": dict(T=4096, Tq=128, Hq=8, Hkv=2, d=64, k=512),
    "group1": dict(T=4096, Tq=128, Hq=2, Hkv=2, k=512),
    "group2": dict(T=4096, Tq=128, Hq=4, Hkv=2, k=512),
    "group8": dict(T=4096, Tq=128, Hq=8, Hkv=1, k=512),
    "group16": dict(T=4096, Tq=64, Hq=16, Hkv=1, k=512),
    # groups that are not a power of two: idle waves in the last 4-head chunk
    "group3": dict(T=4096, Tq=128, Hq=6, Hkv=2, k=512),
    "group6": dict(T=4096, Tq=128, Hq=6, Hkv=1, k=512),
    "group12_ragged": dict(T=3001, Tq=100, Hq=12, Hkv=1, k=512),
    "noncausal": dict(T=4096, Tq=130, Hq=4, Hkv=1, k=512, causal=0),
    "batch2": dict(B=2, T=2048, Tq=128, Hq=4, Hkv=2, k=512),
    "kb_odd": dict(T=4096, Tq=128, Hq=4, Hkv=1, k=7 * 64),
}


@pytest.mark.parametrize("case", sorted(SMALL))
def test_small_full(case):
    w = si.workload("prefill_32k_chunk4k", **SMALL[case])
    print(f"[case] {case} {w}", flush=True)
    x = si.make_inputs(w)
    r = full_parity(x, w)
    _report(case, r)


def test_spare_capacity_rows():
    """K/V allocated beyond T (cache capacity): the unused rows hold huge
    values and must never be read, neither as centres nor as keys."""
    w = si.workload("prefill_32k_chunk4k", T=3000, Tq=200, Hq=8, Hkv=2, k=512)
    x = dict(si.make_inputs(w, T_cap=3500))
    x["K"][:, :, w.T:] = 1e4
    x["V"][:, :, w.T:] = 1e4
    r = full_parity(x, w)
    _report("spare_capacity", r)


def test_chunk_is_whole_sequence():
    """Tq = T: the chunk starts at position 0, so its first query blocks see
    fewer than K_b blocks (dense) and the rest are searched."""
    w = si.workload("prefill_32k_chunk4k", T=1536, Tq=1536, Hq=4, Hkv=1, k=512)
    r = full_parity(si.make_inputs(w), w)
    _report("whole_sequence", r)


def test_zero_query_ties_exact():
    w = si.workload("prefill_32k_chunk4k", T=4096, Tq=128, Hq=4, Hkv=1, k=512)
    x = dict(si.make_inputs(w))
    x["q"] = torch.zeros_like(x["q"])
    idx, nnz, out = run_gpu(x, w)
    assert (idx == np.arange(w.kb)).all() and (nnz == w.kb).all()
    kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal)
    ref = oracle.attn_all(x["q"], x["K"], x["V"], idx, nnz, **kw)
    compare_attention(out, ref)


def test_attention_with_oracle_indices():
    import long_context_sparse_mask_amd as hs
    w = si.workload("prefill_32k_chunk4k", T=3000, Tq=256, Hq=8, Hkv=2, k=512)
    x = si.make_inputs(w)
    kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal)
    o_idx, o_nnz, _ = oracle.mask_all(x["q"], x["K"], **kw)
    o_idx = o_idx.copy()
    o_nnz = o_nnz.copy()
    o_idx[0, 0, 0, :2] = [-1, 10 ** 6]  # out-of-range ids are skipped
    o_nnz[0, 1, 1] = 0                  # nothing to attend: zeros
    q, K, V = (x[n].cuda() for n in ("q", "K", "V"))
    out = hs.hip_sparse_attn(q, K, V, torch.from_numpy(o_idx).cuda(), torch.from_numpy(o_nnz).cuda(),
                             w.k, w.block_k, w.block_q, T=w.T)
    ref = oracle.attn_all(x["q"], x["K"], x["V"], o_idx, o_nnz, **kw)
    compare_attention(out, ref)


def test_determinism():
    w = si.workload("prefill_32k_chunk4k", T=4096, Tq=256, Hq=8, Hkv=2, k=512)
    x = si.make_inputs(w)
    a = run_gpu(x, w)
    b = run_gpu(x, w)
    assert (a[0] == b[0]).all() and torch.equal(a[2], b[2])


@pytest.mark.timeout(900)
def test_full_size_chunk():
    """The 4096-token chunk at the end of a 32k sequence, 32/8 heads, k=2048,
    in the bench's launch configuration: every one of the 512 index lists
    against the oracle's search (or, for a near tie, its tolerant search) and
    every one of the 131072 output rows against the oracle's attention."""
    w = si.workload("prefill_32k_chunk4k")
    print(f"[case] prefill_32k_chunk4k full {w}", flush=True)
    r = full_parity(si.make_inputs(w), w)
    _report("prefill_32k_chunk4k", r)
    assert r["problems"] == 512
