"""GPU parity of the dense part (sink and sliding-window blocks beside the HiP
search; hip_mask_estimate_ex / hip_sparse_attn_ex) against the CPU oracle run
with the same sink and window.  The usual bar: index sets exact where the
oracle's cut margin is at least 1e-4, outputs within 2e-2."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from parity_util import compare_attention, compare_masks, exempt_cap

pytestmark = pytest.mark.gpu


def run_ex(x, w, sink, window, block_table=None, K=None, V=None, dev="cuda"):
    import long_context_sparse_mask_amd as hs
    q = x["q"].to(dev)
    K = (x["K"] if K is None else K).to(dev)
    V = (x["V"] if V is None else V).to(dev)
    bt = None if block_table is None else block_table.to(dev)
    kw = dict(T=w.T, causal=bool(w.causal), sink=sink, window=window, block_table=bt)
    idx, nnz = hs.hip_mask_estimate_ex(q, K, w.k, w.block_k, w.block_q, **kw)
    out = hs.hip_sparse_attn_ex(q, K, V, idx, nnz, w.k, w.block_k, w.block_q, **kw)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), nnz.cpu().numpy(), out


def check_lists(idx, nnz, w, sink, window):
    """Valid searched lists: ascending, in the searched range, nnz = min(K_b, M)."""
    B, Hkv, nqb, kb = idx.shape
    for qb in range(nqb):
        last = min((qb + 1) * w.block_q, w.Tq) - 1
        Tp = (w.T - w.Tq + last + 1) if w.causal else w.T
        Np = -(-Tp // w.block_k)
        sb = min(sink // w.block_k, Np)
        wb = min(window // w.block_k, Np - sb)
        M = Np - sb - wb
        n = min(kb, M)
        for b in range(B):
            for g in range(Hkv):
                row = idx[b, g, qb]
                assert nnz[b, g, qb] == n
                assert (row[n:] == -1).all()
                if n:
                    assert (np.diff(row[:n]) > 0).all() and row[0] >= sb and row[n - 1] < Np - wb


def check_dense(name, w, sink, window, x=None, **kw):
    print(f"[case] {name} sink={sink} window={window} {w}", flush=True)
    x = x if x is not None else si.make_inputs(w)
    idx, nnz, out = run_ex(x, w, sink, window, **kw)
    check_lists(idx, nnz, w, sink, window)
    okw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal, sink=sink,
               window=window)
    o_idx, o_nnz, o_margin = oracle.mask_all(x["q"], x["K"], **okw)
    exempt = compare_masks(idx, nnz, o_idx, o_nnz, o_margin, x, w, sink, window)
    assert exempt <= exempt_cap(o_margin.size)
    ref = oracle.attn_all(x["q"], x["K"], x["V"], idx, nnz, **okw)
    err = compare_attention(out, ref)
    print(f"[parity] {name}: problems={o_margin.size} exempt={exempt} max_err={err:.3e}", flush=True)
    return idx, nnz, out


CASES = {
    # a window of 4096 tokens and one sink block, as a serving configuration would use
    "decode_32k": ("decode_32k", 64, 4096, dict(B=2, Hq=8, Hkv=2)),
    # block_k 8, K_b 512 (eight candidate tiles per wave and round)
    "decode_bk8_kb512": ("decode_32k", 8, 512, dict(Hq=8, Hkv=2, T=20000, block_k=8, k=4096)),
    # the dense part covers every block (no search, nnz 0)
    "decode_all_dense": ("decode_32k", 64, 256, dict(Hq=4, Hkv=1, T=300, k=512)),
    # the search range just above K_b
    "decode_search_range_tight": ("decode_32k", 128, 640, dict(Hq=4, Hkv=1, T=3000, k=1920)),
    "decode_multi_row": ("decode_32k", 64, 512, dict(Hq=8, Hkv=2, Tq=5, T=3000, k=512)),
    "decode_group16": ("decode_32k", 192, 1024, dict(Hq=16, Hkv=1, T=8192, k=1024)),
    "decode_f32_d64": ("tiny_decode", 16, 64, dict(T=1000)),
    "decode_e5m2": ("decode_32k", 64, 2048, dict(Hq=8, Hkv=2, T=20000, dtype="bf16_e5m2")),
    "prefill_ragged": ("prefill_32k_chunk4k", 64, 512, dict(T=3000, Tq=200, Hq=8, Hkv=2, k=512)),
    "prefill_whole_sequence": ("prefill_32k_chunk4k", 64, 256, dict(T=1536, Tq=1536, Hq=4, Hkv=1, k=512)),
    "prefill_bk16": ("prefill_32k_chunk4k", 32, 256, dict(T=4096, Tq=128, Hq=4, Hkv=1, block_k=16, k=256)),
    "prefill_e5m2_d64": ("prefill_32k_chunk4k", 64, 1024, dict(T=4500, Tq=128, Hq=8, Hkv=2, d=64, k=512,
                                                             dtype="bf16_e5m2")),
    # the largest dense part the calls accept: (sink + window) / block_k = 256 blocks
    "decode_dense_256_blocks": ("decode_32k", 64, 16320, dict(Hq=8, Hkv=2, T=32768, k=2048)),
    "prefill_dense_256_blocks": ("prefill_32k_chunk4k", 64, 16320, dict(T=20000, Tq=128, Hq=4, Hkv=1,
                                                                     k=512)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_dense_part(case):
    base, sink, window, kw = CASES[case]
    check_dense(case, si.workload(base, **kw), sink, window)


@pytest.mark.timeout(900)
def test_dense_part_decode_128k_b4_full():
    """The 128k x4 decode at full size with a 4096-token window and a sink block."""
    check_dense("decode_128k_b4", si.workload("decode_128k_b4"), 64, 4096)


def test_dense_part_paged():
    """Dense part on a paged KV cache (shuffled 128-token pages): the oracle's
    result on the logical K/V, and bit for bit the contiguous call's."""
    from test_paged_kv_parity import to_pages
    for base, kw in (("decode_32k", dict(B=2, Hq=8, Hkv=2, T=20000)),
                     ("prefill_32k_chunk4k", dict(T=3000, Tq=200, Hq=8, Hkv=2, k=512))):
        w = si.workload(base, **kw)
        x = si.make_inputs(w)
        Kp, Vp, table = to_pages(x, w, 128, seed=3)
        idx, nnz, out = check_dense(base + "_paged", w, 64, 1024, x=x, block_table=table, K=Kp, V=Vp)
        c_idx, c_nnz, c_out = run_ex(x, w, 64, 1024)
        assert (c_idx == idx).all() and (c_nnz == nnz).all() and torch.equal(c_out, out)


def test_dense_part_with_malformed_lists():
    """hip_sparse_attn_ex on lists that name dense blocks, repeat a block, or
    hold out-of-range ids: the union rule of the oracle."""
    import long_context_sparse_mask_amd as hs
    for base, kw in (("decode_32k", dict(Hq=8, Hkv=2, T=4000, k=512)),
                     ("prefill_32k_chunk4k", dict(T=3000, Tq=256, Hq=8, Hkv=2, k=512))):
        w = si.workload(base, **kw)
        x = si.make_inputs(w)
        sink, window = 128, 640
        okw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal, sink=sink,
                   window=window)
        o_idx, o_nnz, _ = oracle.mask_all(x["q"], x["K"], **okw)
        bad = o_idx.copy()
        nnz = o_nnz.copy()
        bad[0, 0, 0, :4] = [0, 1, 10 ** 6, -3]    # sink blocks and bad ids
        bad[0, 1, -1, :3] = [bad[0, 1, -1, 3]] * 3  # a repeated block
        nnz[0, 0, 0] = w.kb
        nnz[0, 1, -1] = w.kb
        q, K, V = (x[n].cuda() for n in ("q", "K", "V"))
        out = hs.hip_sparse_attn_ex(q, K, V, torch.from_numpy(bad).cuda(), torch.from_numpy(nnz).cuda(),
                                    w.k, w.block_k, w.block_q, T=w.T, sink=sink, window=window)
        ref = oracle.attn_all(x["q"], x["K"], x["V"], bad, nnz, **okw)
        compare_attention(out, ref)
