"""GPU parity of hip_decode_step (one call: mask estimation then attention).

Every case runs the step through the C ABI and requires (1) bit-for-bit
equality with hip_mask_estimate followed by hip_sparse_attn on the same
inputs (the one-launch kernel runs the same search, split assignment and
merge), and (2) the oracle's acceptance: index lists equal to the oracle's
or, for near ties, reachable by its tolerant search; outputs within 2e-2 of
the oracle's attention on the GPU's lists.  Cases cover the one-launch form
(bf16 query, bf16 or fp8 K/V, contiguous or paged, K_b <= 64) and the cases
that run the two calls' kernels in turn (fp32, K_b > 64, more than 16 splits
or workgroups beyond one per CU, page numbers that do not fit in LDS beside
the kernel's own arrays).
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from parity_util import compare_attention, compare_masks, exempt_cap

pytestmark = pytest.mark.gpu


def _two_calls(x, w, sink, window, table=None, K=None, V=None):
    import long_context_sparse_mask_amd as hs
    q = x["q"].cuda()
    K = (x["K"] if K is None else K).cuda()
    V = (x["V"] if V is None else V).cuda()
    bt = None if table is None else table.cuda()
    kw = dict(T=w.T, causal=bool(w.causal), sink=sink, window=window, block_table=bt)
    idx, nnz = hs.hip_mask_estimate_ex(q, K, w.k, w.block_k, 1, **kw)
    out = hs.hip_sparse_attn_ex(q, K, V, idx, nnz, w.k, w.block_k, 1, **kw)
    step_out, s_idx, s_nnz = hs.hip_decode_step(q, K, V, w.k, w.block_k, **kw)
    torch.cuda.synchronize()
    return (idx.cpu().numpy(), nnz.cpu().numpy(), out), (s_idx.cpu().numpy(), s_nnz.cpu().numpy(),
                                                         step_out)


def check_step(name, w, sink=0, window=0, page=0, x=None):
    print(f"[case] step {name} sink={sink} window={window} page={page} {w}", flush=True)
    x = x if x is not None else si.make_inputs(w)
    table = Kp = Vp = None
    if page:
        from test_paged_kv_parity import to_pages
        Kp, Vp, table = to_pages(x, w, page)
    (idx, nnz, out), (s_idx, s_nnz, s_out) = _two_calls(x, w, sink, window, table, Kp, Vp)
    assert (s_idx == idx).all() and (s_nnz == nnz).all(), "lists differ from the two calls"
    assert torch.equal(s_out, out), "output differs from the two calls"
    okw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=1, causal=w.causal, sink=sink,
               window=window)
    o_idx, o_nnz, o_margin = oracle.mask_all(x["q"], x["K"], **okw)
    exempt = compare_masks(s_idx, s_nnz, o_idx, o_nnz, o_margin, x, w, sink, window)
    assert exempt <= exempt_cap(o_margin.size)
    ref = oracle.attn_all(x["q"], x["K"], x["V"], s_idx, s_nnz, **okw)
    err = compare_attention(s_out, ref)
    print(f"[parity] step {name}: problems={o_margin.size} exempt={exempt} max_err={err:.3e} "
          "(bitwise equal to the two calls)", flush=True)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny_decode", "decode_32k", "decode_128k_b4",
                                  "decode_1m_needles"])
def test_step_workload(name):
    check_step(name, si.workload(name))


CASES = {
    # one-launch form
    "bf16_d64_bk16_g2": dict(base="decode_32k", Hq=4, Hkv=2, d=64, T=5000, block_k=16, k=256),
    "bk32_kb7": dict(base="decode_32k", Hq=4, Hkv=1, T=9000, block_k=32, k=224),
    "dense_k_ge_T": dict(base="decode_32k", Hq=4, Hkv=2, T=500, block_k=32, k=512),
    "multi_row_causal": dict(base="decode_32k", Hq=8, Hkv=2, Tq=5, T=3000, k=512),
    "multi_row_noncausal": dict(base="decode_32k", Hq=8, Hkv=2, Tq=3, T=3000, k=512, causal=0),
    "group1": dict(base="decode_32k", Hq=4, Hkv=4, T=4096, k=1024),
    "group3": dict(base="decode_32k", Hq=6, Hkv=2, T=4096, k=1024),
    "group8": dict(base="decode_32k", Hq=16, Hkv=2, T=4096, k=1024),
    "group16": dict(base="decode_32k", Hq=16, Hkv=1, T=4096, k=1024),
    "one_split": dict(base="decode_32k", Hq=8, Hkv=2, Tq=2, T=3000, k=128),
    "ragged_batch3": dict(base="decode_32k", B=3, Hq=8, Hkv=2, T=7001, k=1024),
    "wide_grid": dict(base="decode_32k", Hq=32, Hkv=8, Tq=16, T=4096, k=1024),
    "wide_grid_d64_ragged": dict(base="decode_32k", Hq=16, Hkv=8, Tq=16, T=4001, d=64, k=1024),
    "e5m2": dict(base="decode_32k", dtype="bf16_e5m2", Hq=8, Hkv=2, T=9000, k=1024),
    "e5m2_d64_group8": dict(base="decode_32k", dtype="bf16_e5m2", Hq=16, Hkv=2, d=64, T=7000, k=1024),
    # K_b = 64: two tiles per wave and round in the search
    "kb64": dict(base="decode_32k", Hq=8, Hkv=2, T=20000, k=4096),
    # the two calls' kernels in turn
    "f32_d128": dict(base="decode_32k", dtype="f32", B=2, Hq=4, Hkv=2, T=6000, k=1024),
    "bk8_kb512": dict(base="decode_32k", Hq=8, Hkv=2, T=20000, block_k=8, k=4096),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_step_case(case):
    kw = dict(CASES[case])
    check_step(case, si.workload(kw.pop("base"), **kw))


def test_step_dense_part():
    """A sink and sliding window beside the search (one-launch form)."""
    check_step("dense_part", si.workload("decode_32k", Hq=8, Hkv=2, T=20000, k=1024), sink=64,
               window=2048)


def test_step_dense_part_128k():
    check_step("dense_part_128k_b4", si.workload("decode_128k_b4"), sink=64, window=4096)


def test_step_paged():
    """A paged KV cache (one launch; the search stages the page numbers in LDS)."""
    check_step("paged", si.workload("decode_32k", Hq=8, Hkv=2, T=8192, k=1024), page=128)


def test_step_paged_fp8():
    check_step("paged_fp8", si.workload("decode_32k", dtype="bf16_e5m2", B=2, Hq=8, Hkv=2, T=7000,
                                        k=1024), page=64)


def test_step_paged_pages_fill_lds():
    """16384 pages of 16 tokens beside a 16-head group's arrays: more than a
    workgroup's LDS, so the two calls' kernels run in turn (same results)."""
    check_step("paged_pages_fill_lds", si.workload("decode_32k", Hq=16, Hkv=1, T=262144,
                                                   block_k=16, k=1024), page=16)


def test_step_zero_query_ties_exact():
    """q = 0: every score ties, so the lowest block ids are kept and each
    output row is the mean of V over them, exactly as the two calls give."""
    w = si.workload("decode_32k", Hq=8, Hkv=2, T=8192, k=1024)
    x = dict(si.make_inputs(w))
    x["q"] = torch.zeros_like(x["q"])
    (idx, nnz, out), (s_idx, s_nnz, s_out) = _two_calls(x, w, 0, 0)
    assert (s_idx == np.arange(w.kb)).all() and (s_nnz == w.kb).all()
    assert torch.equal(s_out, out)


def test_step_reused_mask():
    """The step's lists serve a later hip_sparse_attn call (mask reuse): the
    next step's query attends over the previous step's lists."""
    import long_context_sparse_mask_amd as hs
    w = si.workload("decode_32k", B=2, Hq=8, Hkv=2, T=8192, k=1024)
    x = si.make_inputs(w)
    q, K, V = (x[n].cuda() for n in ("q", "K", "V"))
    _, idx, nnz = hs.hip_decode_step(q, K, V, w.k, w.block_k, T=w.T)
    q2 = torch.randn(q.shape, generator=torch.Generator().manual_seed(5)).to(q.dtype)
    out2 = hs.hip_sparse_attn(q2.cuda(), K, V, idx, nnz, w.k, w.block_k, 1, T=w.T)
    torch.cuda.synchronize()
    kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=1, causal=w.causal)
    ref = oracle.attn_all(q2, x["K"], x["V"], idx.cpu().numpy(), nnz.cpu().numpy(), **kw)
    compare_attention(out2, ref)


def test_step_workspace_reused():
    """One zero-filled workspace serves consecutive steps: each call's last
    split workgroups return the arrival counters to zero, so every call equals
    the two calls bit for bit and the counters end at zero."""
    import long_context_sparse_mask_amd as hs
    w = si.workload("decode_32k", B=2, Hq=16, Hkv=4, T=20000, k=1024)
    x = si.make_inputs(w)
    q, K, V = (x[n].cuda() for n in ("q", "K", "V"))
    need = hs.hipsa_decode_step_workspace_bytes(q, K, w.k, w.block_k, T=w.T)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    P = w.B * w.Hkv
    g = torch.Generator().manual_seed(11)
    for r in range(3):
        qr = q if r == 0 else torch.randn(q.shape, generator=g).to(q.dtype).cuda()
        out, idx, nnz = hs.hip_decode_step(qr, K, V, w.k, w.block_k, T=w.T, workspace=ws)
        i2, n2 = hs.hip_mask_estimate(qr, K, w.k, w.block_k, 1, T=w.T)
        o2 = hs.hip_sparse_attn(qr, K, V, i2, n2, w.k, w.block_k, 1, T=w.T)
        torch.cuda.synchronize()
        assert torch.equal(idx, i2) and torch.equal(nnz, n2) and torch.equal(out, o2), r
        assert (ws[need - 4 * P:] == 0).all(), "arrival counters not back at zero"


def _tied_scores(x):
    """Scores with many exact ties: q is zero but for dimension 0, and K's
    dimension 0 holds small integers, so every score is an exact integer on
    both sides and a round's cut falls inside a group of equal scores (the
    lower start wins)."""
    g = torch.Generator().manual_seed(5)
    q = torch.zeros_like(x["q"])
    q[..., 0] = 1
    K = x["K"].clone()
    K[..., 0] = torch.randint(-2, 3, K.shape[:-1], generator=g).to(K.dtype)
    return dict(x, q=q, K=K)


TIE_INPUTS = {"zero_query": lambda x: dict(x, q=torch.zeros_like(x["q"])), "tied_scores": _tied_scores}
TIE_SHAPES = {
    "decode_128k_b4": dict(base="decode_128k_b4"),
    "kb64": dict(base="decode_32k", Hq=8, Hkv=2, T=20000, k=4096),
    "e5m2_ragged": dict(base="decode_32k", dtype="bf16_e5m2", B=3, Hq=8, Hkv=2, T=7001, k=1024),
}


@pytest.mark.timeout(600)
@pytest.mark.parametrize("inputs", sorted(TIE_INPUTS))
@pytest.mark.parametrize("shape", sorted(TIE_SHAPES))
def test_step_exact_ties(shape, inputs):
    """Exact score ties at the cuts: the one-launch step equals the two calls
    bit for bit, and its lists equal the oracle's exactly (scores are exact
    integers on both sides, so the lower-start rule decides every tie)."""
    kw = dict(TIE_SHAPES[shape])
    w = si.workload(kw.pop("base"), **kw)
    print(f"[case] step ties {shape} {inputs} {w}", flush=True)
    x = TIE_INPUTS[inputs](si.make_inputs(w))
    (idx, nnz, out), (s_idx, s_nnz, s_out) = _two_calls(x, w, 0, 0)
    assert (s_idx == idx).all() and (s_nnz == nnz).all(), "lists differ from the two calls"
    assert torch.equal(s_out, out), "output differs from the two calls"
    o_idx, o_nnz, _ = oracle.mask_all(x["q"], x["K"], T=w.T, k=w.k, block_k=w.block_k, block_q=1,
                                      causal=w.causal)
    assert (s_idx == o_idx).all() and (s_nnz == o_nnz).all(), "lists differ from the oracle"
