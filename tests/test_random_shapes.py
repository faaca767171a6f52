"""GPU parity on seeded random configurations spread over the parameter space.

Each case draws, from its own seed:
* decode (block_q 1, one to five rows) or prefill (block_q 64, a ragged chunk);
* the element types: bf16, bf16 query with fp8 E5M2 K/V, or fp32 (decode);
* head dim 64 or 128; 1-3 KV heads; groups of 1-16 query heads;
* block_k 8-64 and K_b 1-64; a ragged T; causal or not; batch 1-3;
* sometimes a dense part (sink and window blocks);
* sometimes a paged cache with shuffled pages.

It is checked against the oracle with the usual bar: index sets exact where
the oracle's cut margin is at least 1e-4; outputs within 2e-2, against the
oracle run on the lists the GPU produced.  Every list must be a valid
selection (ascending, in the searched range, the right count).  A
paged case must also equal the contiguous call bit for bit.

An exempt problem (a near tie at some cut) must still produce a list that
the oracle's near-tie-tolerant search reaches.  The share of exempt problems
is a property of the inputs, not of the GPU: a chunk's score is a maximum
over up to 16 heads x 64 rows, and such maxima lie close together.  Over the
64 cases 14 of 579 problems (2.4%) are exempt, but a case has only 1 to 30
problems, so the usual cap (10%, at least one) becomes at least two here.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from parity_util import compare_attention, compare_masks

pytestmark = pytest.mark.gpu

N_CASES = 64


def draw(seed):
    """Workload fields, sink, window and page size (0: contiguous) of case `seed`."""
    rng = np.random.default_rng(1000 + seed)
    prefill = rng.random() < 0.45
    dtypes = ["bf16", "bf16_e5m2"] + ([] if prefill else ["f32"])
    dtype = str(rng.choice(dtypes))
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
    bk = int(rng.choice([8, 16, 32, 64]))
    Kb = int(rng.integers(1, 65))
    T = int(rng.integers(64, 6001))
    if prefill:
        Tq = int(rng.integers(1, min(T, 300) + 1))
    else:
        Tq = int(rng.choice([1, 1, 2, 5]))
    B = int(rng.integers(1, 4))
    causal = int(rng.random() < 0.8)
    sink = window = 0
    if rng.random() < 0.3:
        sink = bk * int(rng.integers(0, 3))
        window = bk * int(rng.integers(0, 24))
    page = 0
    if rng.random() < 0.3:
        page = bk << int(rng.integers(0, 4))
    base = "prefill_32k_chunk4k" if prefill else "decode_32k"
    fields = dict(B=B, Hq=G * Hkv, Hkv=Hkv, d=d, dtype=dtype, T=T, Tq=Tq, block_k=bk, k=Kb * bk,
                  causal=causal, seed=5000 + seed)
    return si.workload(base, **fields), sink, window, page


def run_ex(x, w, sink, window, table=None, K=None, V=None):
    import long_context_sparse_mask_amd as hs
    q = x["q"].cuda()
    K = (x["K"] if K is None else K).cuda()
    V = (x["V"] if V is None else V).cuda()
    bt = None if table is None else table.cuda()
    kw = dict(T=w.T, causal=bool(w.causal), sink=sink, window=window, block_table=bt)
    idx, nnz = hs.hip_mask_estimate_ex(q, K, w.k, w.block_k, w.block_q, **kw)
    out = hs.hip_sparse_attn_ex(q, K, V, idx, nnz, w.k, w.block_k, w.block_q, **kw)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), nnz.cpu().numpy(), out


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(seed):
    w, sink, window, page = draw(seed)
    print(f"[case] seed={seed} sink={sink} window={window} page={page} {w}", flush=True)
    x = si.make_inputs(w)
    idx, nnz, out = run_ex(x, w, sink, window)
    okw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal, sink=sink,
               window=window)
    o_idx, o_nnz, o_margin = oracle.mask_all(x["q"], x["K"], **okw)
    from test_dense_part_parity import check_lists
    check_lists(idx, nnz, w, sink, window)
    exempt = compare_masks(idx, nnz, o_idx, o_nnz, o_margin, x, w, sink, window)
    assert exempt <= max(2, o_margin.size // 10), (exempt, o_margin.size)
    ref = oracle.attn_all(x["q"], x["K"], x["V"], idx, nnz, **okw)
    err = compare_attention(out, ref)
    if page:
        from test_paged_kv_parity import to_pages
        Kp, Vp, table = to_pages(x, w, page, seed=seed)
        p_idx, p_nnz, p_out = run_ex(x, w, sink, window, table=table, K=Kp, V=Vp)
        assert (p_idx == idx).all() and (p_nnz == nnz).all() and torch.equal(p_out, out)
    print(f"[parity] seed={seed}: problems={o_margin.size} exempt={exempt} max_err={err:.3e}",
          flush=True)
