"""GPU parity of the decode path (block_q = 1) against the CPU oracle.

Every case runs hip_mask_estimate then hip_sparse_attn through the C ABI on
seeded synthetic inputs and compares every problem and every output row with
the oracle on the same bits.  The four decode workloads run at full size.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from parity_util import (ATOL, check_valid_lists, compare_attention, compare_masks, full_parity,
                         run_gpu)

pytestmark = pytest.mark.gpu

_cache = {}


def _inputs(w, T_cap=None):
    key = (w, T_cap)
    if key not in _cache:
        _cache.clear()  # keep at most one large workload in host memory
        _cache[key] = si.make_inputs(w, T_cap=T_cap)
    return _cache[key]


def _report(name, r):
    print(f"[parity] {name}: problems={r['problems']} exempt={r['exempt']} "
          f"max_err={r['max_err']:.3e}", flush=True)


FULL = ["tiny_decode", "decode_32k", "decode_128k_b4", "decode_1m_needles"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_workload_full(name):
    w = si.workload(name)
    print(f"[case] {name} {w}", flush=True)
    r = full_parity(_inputs(w), w)
    _report(name, r)


EDGE = {
    # ragged last block, fp32, d=64
    "f32_d64_ragged": dict(base="tiny_decode", T=1000),
    # bf16 d=64, block_k=16, GQA 2, ragged
    "bf16_d64_bk16_g2": dict(base="decode_32k", Hq=4, Hkv=2, d=64, T=5000, block_k=16, k=256),
    # the largest K_b (512) with block_k=8
    "bk8_kb512": dict(base="decode_32k", Hq=8, Hkv=2, T=20000, block_k=8, k=4096),
    # block_k = 32, K_b = 7 (odd)
    "bk32_kb7": dict(base="decode_32k", Hq=4, Hkv=1, T=9000, block_k=32, k=224),
    # k >= T: dense attention over every block
    "dense_k_ge_T": dict(base="decode_32k", Hq=4, Hkv=2, T=500, block_k=32, k=512),
    # several query rows, each its own causal problem
    "multi_row_causal": dict(base="decode_32k", Hq=8, Hkv=2, Tq=5, T=3000, k=512),
    "multi_row_noncausal": dict(base="decode_32k", Hq=8, Hkv=2, Tq=3, T=3000, k=512, causal=0),
    # group sizes 1, 8 and 16
    "group1": dict(base="decode_32k", Hq=4, Hkv=4, T=4096, k=1024),
    "group8": dict(base="decode_32k", Hq=16, Hkv=2, T=4096, k=1024),
    "group16": dict(base="decode_32k", Hq=16, Hkv=1, T=4096, k=1024),
    # groups that are not a power of two (padded head rows in the matrix ops)
    "group3": dict(base="decode_32k", Hq=6, Hkv=2, T=4096, k=1024),
    "group5": dict(base="decode_32k", Hq=5, Hkv=1, T=4096, k=1024),
    "group12_f32": dict(base="decode_32k", dtype="f32", Hq=12, Hkv=1, T=3000, k=512),
    # fp32 at d=128, batch 3
    "f32_d128_b3": dict(base="decode_32k", dtype="f32", B=3, Hq=4, Hkv=2, T=6000, k=1024),
    # 128 listed tokens: one split workgroup writes the output, no merge launch
    "one_split_bf16": dict(base="decode_32k", Hq=8, Hkv=2, Tq=2, T=3000, k=128),
    "one_split_f32_d128": dict(base="decode_32k", dtype="f32", Hq=4, Hkv=2, T=3000, k=64),
    # 16 or more problems with a bf16 query: the mask kernel runs 8 (or 2) workgroups per
    # problem, each prefetching its share of the next round's rows; split 0 writes the list
    "split_mask_16_ragged": dict(base="decode_32k", B=2, Hq=16, Hkv=8, T=7001, k=1024),
    "split_mask_e5m2_kb64": dict(base="decode_32k", dtype="bf16_e5m2", B=2, Hq=32, Hkv=8, T=30000,
                                 k=4096),
    "split_mask_rows_causal": dict(base="decode_32k", Hq=16, Hkv=4, Tq=4, T=9000, k=512),
    "split_mask_d64_g1": dict(base="decode_32k", B=4, Hq=8, Hkv=8, d=64, T=5000, k=1024),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge(case):
    kw = dict(EDGE[case])
    w = si.workload(kw.pop("base"), **kw)
    print(f"[case] {case} {w}", flush=True)
    r = full_parity(_inputs(w), w)
    _report(case, r)


# Cases where the bf16-query split kernel reads V rows 16 bytes per lane:
# 256-token splits, or grids of >= 1024 split workgroups (many query rows
# make many problems; with groups of more than 8 heads, 64-token splits).
WIDE = {
    "wide_bf16_d128": dict(base="decode_32k", Hq=32, Hkv=8, Tq=16, T=4096, k=1024),
    "wide_e5m2_d128": dict(base="decode_32k", Hq=32, Hkv=8, Tq=16, T=4096, k=1024, dtype="bf16_e5m2"),
    "wide_bf16_d64_g2": dict(base="decode_32k", Hq=16, Hkv=8, Tq=16, T=4096, d=64, k=1024),
    "wide_e5m2_d64_ragged": dict(base="decode_32k", Hq=16, Hkv=8, Tq=16, T=4001, d=64, k=1024,
                                 dtype="bf16_e5m2"),
    "wide_group8": dict(base="decode_32k", Hq=64, Hkv=8, Tq=16, T=4096, k=1024),
    "wide_group16_noncausal": dict(base="decode_32k", Hq=32, Hkv=2, Tq=32, T=4096, k=1024, causal=0),
}


def split_workgroups(w):
    """Split workgroups of the decode attention launch, from the workspace size
    (problems x splits x G x (d + 2) floats)."""
    import long_context_sparse_mask_amd as hs
    q = torch.empty((w.B, w.Hq, w.Tq, w.d), dtype=torch.bfloat16)
    K = torch.empty((w.B, w.Hkv, w.T, w.d), dtype=q.dtype)
    ws = hs.hipsa_workspace_bytes_ex(q, K, w.k, w.block_k, w.block_q, T=w.T, causal=bool(w.causal))
    return ws // ((w.Hq // w.Hkv) * (w.d + 2) * 4)


def wide_v_reads(w):
    """Whether the split kernel takes 16-byte V reads for this (bf16 query)
    workload: 256-token splits, or at least 1024 split workgroups."""
    grid = split_workgroups(w)
    splits = grid // (w.B * w.Hkv * w.Tq)
    return grid >= 1024 or (w.k > 256 and splits == -(-w.k // 256))


@pytest.mark.parametrize("case", sorted(WIDE))
def test_wide_grid(case):
    kw = dict(WIDE[case])
    w = si.workload(kw.pop("base"), **kw)
    assert wide_v_reads(w)
    print(f"[case] {case} {w}", flush=True)
    r = full_parity(_inputs(w), w)
    _report(case, r)


def test_spare_capacity_rows():
    w = si.workload("decode_32k", Hq=8, Hkv=2, T=3000, k=512)
    x = _inputs(w, T_cap=3333)
    # poison the unused rows: they must never be read
    x["K"][:, :, w.T:] = 1e4
    x["V"][:, :, w.T:] = 1e4
    r = full_parity(x, w)
    _report("spare_capacity", r)


def test_mask_reuse_across_steps():
    """A mask estimated for one step's queries drives attention for the next
    step's queries (mask refresh every r_m steps): the attention is exact
    over the reused lists."""
    import long_context_sparse_mask_amd as hs
    w = si.workload("decode_32k", Hq=8, Hkv=2, T=6000, k=512)
    x = _inputs(w)
    q1 = torch.randn(x["q"].shape, generator=torch.Generator().manual_seed(7)).to(x["q"].dtype)
    q0, q1d, K, V = x["q"].cuda(), q1.cuda(), x["K"].cuda(), x["V"].cuda()
    idx, nnz = hs.hip_mask_estimate(q0, K, w.k, w.block_k, 1, T=w.T)
    out = hs.hip_sparse_attn(q1d, K, V, idx, nnz, w.k, w.block_k, 1, T=w.T)
    kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=1, causal=w.causal)
    ref = oracle.attn_all(q1, x["K"], x["V"], idx.cpu().numpy(), nnz.cpu().numpy(), **kw)
    compare_attention(out, ref)


def test_zero_query_ties_exact():
    """q = 0: every score is exactly 0 in any precision; the tie rule keeps the
    lowest block ids and the output is the mean of V over them."""
    w = si.workload("decode_32k", T=8192, k=1024)
    x = dict(_inputs(w))
    x["q"] = torch.zeros_like(x["q"])
    idx, nnz, out = run_gpu(x, w)
    assert (idx == np.arange(w.kb)).all() and (nnz == w.kb).all()
    Vm = x["V"][:, :, :w.kb * w.block_k].double().mean(dim=2)  # [B,Hkv,d]
    want = Vm.repeat_interleave(w.G, dim=1)[:, :, None, :].numpy()
    compare_attention(out, want)


def test_mask_scale_invariance_and_determinism():
    w = si.workload("decode_32k", T=16384, k=1024)
    x = _inputs(w)
    a = run_gpu(x, w)
    b = run_gpu(x, w)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()
    assert torch.equal(a[2], b[2])
    x2 = dict(x)
    x2["q"] = x["q"] * 2  # exact in bf16
    c = run_gpu(x2, w)
    assert (a[0] == c[0]).all()


def test_attention_with_oracle_indices_and_bad_lists():
    """hip_sparse_attn on lists it did not make: the oracle's own, and lists with
    out-of-range ids, negative ids and nnz outside [0, K_b]."""
    import long_context_sparse_mask_amd as hs
    w = si.workload("decode_32k", Hq=8, Hkv=2, T=4000, k=512)
    x = _inputs(w)
    kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal)
    o_idx, o_nnz, _ = oracle.mask_all(x["q"], x["K"], **kw)
    rng = np.random.default_rng(3)
    bad_idx = o_idx.copy()
    bad_idx[0, 0, 0, :3] = [-5, 10 ** 6, 63]       # 63 >= N_p = 63 -> skipped
    bad_nnz = o_nnz.copy()
    bad_nnz[0, 1, 0] = 99                          # clamped to K_b
    bad_nnz[1 % w.B, 0, 0] = -3 if w.B > 1 else 0  # nothing to attend: zeros
    bad_idx[0, 1, 0] = rng.permutation(62)[:w.kb]  # unsorted is fine
    for I, N in ((o_idx, o_nnz), (bad_idx, bad_nnz)):
        q, K, V = (x[n].cuda() for n in ("q", "K", "V"))
        out = hs.hip_sparse_attn(q, K, V, torch.from_numpy(I).cuda(), torch.from_numpy(N).cuda(),
                                 w.k, w.block_k, w.block_q, T=w.T)
        ref = oracle.attn_all(x["q"], x["K"], x["V"], I, N, **kw)
        compare_attention(out, ref)


def test_empty_batch():
    import long_context_sparse_mask_amd as hs
    q = torch.zeros(0, 4, 1, 128, dtype=torch.bfloat16, device="cuda")
    K = torch.zeros(0, 1, 256, 128, dtype=torch.bfloat16, device="cuda")
    idx, nnz = hs.hip_mask_estimate(q, K, 128, 64, 1)
    out = hs.hip_sparse_attn(q, K, K, idx, nnz, 128, 64, 1)
    assert out.shape == q.shape
