"""GPU: hip_sparse_attn_noalloc against hip_sparse_attn, through the C ABI.

The no-alloc call runs the same kernels with the split partials in the
library's per-GPU scratch instead of a caller workspace, so its outputs must
equal hip_sparse_attn's bit for bit.  Two calls in a row, the second on a
smaller input (fewer problems and splits: it reuses the scratch the first
call left behind), then a decode step captured in a HIP graph and replayed.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from parity_util import compare_attention

pytestmark = pytest.mark.gpu


def _lists(w, x):
    import long_context_sparse_mask_amd as hs
    q, K = x["q"].cuda(), x["K"].cuda()
    return hs.hip_mask_estimate(q, K, w.k, w.block_k, w.block_q, T=w.T, causal=bool(w.causal))


def _both(w, x):
    import long_context_sparse_mask_amd as hs
    q, K, V = (x[n].cuda() for n in ("q", "K", "V"))
    idx, nnz = _lists(w, x)
    kw = dict(T=w.T, causal=bool(w.causal))
    ref = hs.hip_sparse_attn(q, K, V, idx, nnz, w.k, w.block_k, w.block_q, **kw)
    out = torch.full_like(q, float("nan"))
    hs.hip_sparse_attn_noalloc(q, K, V, idx, nnz, w.k, w.block_k, w.block_q, out=out, **kw)
    torch.cuda.synchronize()
    return ref, out, idx, nnz


def test_noalloc_matches_workspace_call_twice():
    # first: the 32k decode at batch 2 (8 x 2 problems x 16 splits); second: a smaller,
    # ragged shape (2 problems, 5 splits) over the partials the first one left
    cases = [si.workload("decode_32k", B=2, seed=41),
             si.workload("decode_32k", Hq=8, Hkv=2, T=3001, k=640, seed=42)]
    for w in cases:
        print(f"[case] noalloc {w}", flush=True)
        x = si.make_inputs(w)
        ref, out, idx, nnz = _both(w, x)
        assert torch.equal(out, ref)
        kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal)
        o = oracle.attn_all(x["q"], x["K"], x["V"], idx.cpu().numpy(), nnz.cpu().numpy(), **kw)
        err = compare_attention(out, o)
        print(f"[parity] noalloc {w.name} B={w.B} T={w.T}: bitwise equal, max_err={err:.3e}",
              flush=True)


def test_noalloc_in_a_graph():
    """A decode step with the no-alloc attention captured in a HIP graph (no
    allocation inside the capture), replayed several times with eager work
    between replays; every replay must equal the eager result."""
    import long_context_sparse_mask_amd as hs
    w = si.workload("decode_32k", Hq=16, Hkv=4, T=8192, k=1024, seed=43)
    x = si.make_inputs(w)
    q, K, V = (x[n].cuda() for n in ("q", "K", "V"))
    kw = dict(T=w.T, causal=bool(w.causal))
    idx = torch.empty((w.B, w.Hkv, 1, w.kb), dtype=torch.int32, device="cuda")
    nnz = torch.empty((w.B, w.Hkv, 1), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)

    def step():
        hs.hip_mask_estimate(q, K, w.k, w.block_k, w.block_q, indices=idx, nnz=nnz, **kw)
        hs.hip_sparse_attn_noalloc(q, K, V, idx, nnz, w.k, w.block_k, w.block_q, out=out, **kw)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.fill_(float("nan"))
        # other eager work on the same GPU between replays (uses the scratch too)
        y = hs.hip_sparse_attn_noalloc(q, K, V, idx, nnz, w.k, w.block_k, w.block_q, **kw)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), r
        assert torch.equal(y, eager), r
    print("[parity] noalloc graph: 4 replays equal the eager step", flush=True)
