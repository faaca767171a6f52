"""GPU parity of the paged KV cache calls (hip_mask_estimate_paged,
hip_sparse_attn_paged) against the CPU oracle.

The oracle computes the method on the logical K/V of a seeded workload.  The
test stores that same K/V in a page pool [num_pages, Hkv, page_size, d]: the
pages of every sequence are scattered over the pool in a random order, the
unused pages and the tail of each sequence's last page hold large poison
values, and the table has spare columns of garbage.  A paged call must then
give the oracle's result (the usual bar: index sets exact where the margin is
safe, outputs within 2e-2) and, since it does the same arithmetic on the same
values, exactly the contiguous call's result.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from parity_util import check_valid_lists, compare_attention, compare_masks, exempt_cap, run_gpu

pytestmark = pytest.mark.gpu


def to_pages(x, w, page_size, seed=0, spare_pages=3, share_prefix_pages=0):
    """Scatter K, V [B,Hkv,T,d] into a shuffled page pool.  With
    share_prefix_pages = n, sequence 1 (when its first n pages equal sequence
    0's) reuses sequence 0's physical pages for them."""
    K, V = x["K"], x["V"]
    B, Hkv, _, d = K.shape
    n_log = -(-w.T // page_size)
    shared = share_prefix_pages if B > 1 else 0
    n_phys = B * n_log - shared + spare_pages
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_phys)
    table = np.full((B, n_log + 2), -7, np.int32)  # spare columns: garbage, never read
    nxt = 0
    for b in range(B):
        for j in range(n_log):
            if b == 1 and j < shared:
                table[b, j] = table[0, j]
            else:
                table[b, j] = perm[nxt]
                nxt += 1
    poison = 1e4
    bytes_view = K.element_size() == 1
    Kp = torch.full((n_phys, Hkv, page_size, d), poison).to(K.dtype)
    Vp = torch.full((n_phys, Hkv, page_size, d), poison).to(K.dtype)
    for b in range(B):
        for j in range(n_log):
            r = min(page_size, w.T - j * page_size)
            src_k, src_v = K[b, :, j * page_size:j * page_size + r], V[b, :, j * page_size:j * page_size + r]
            if bytes_view:  # fp8 copies go through the code bytes
                Kp.view(torch.uint8)[table[b, j], :, :r] = src_k.view(torch.uint8)
                Vp.view(torch.uint8)[table[b, j], :, :r] = src_v.view(torch.uint8)
            else:
                Kp[table[b, j], :, :r] = src_k
                Vp[table[b, j], :, :r] = src_v
    return Kp, Vp, torch.from_numpy(table)


def run_paged(x, w, Kp, Vp, table, dev="cuda"):
    import long_context_sparse_mask_amd as hs
    q = x["q"].to(dev)
    Kd, Vd, td = Kp.to(dev), Vp.to(dev), table.to(dev)
    idx, nnz = hs.hip_mask_estimate_paged(q, Kd, td, w.T, w.k, w.block_k, w.block_q,
                                          causal=bool(w.causal))
    out = hs.hip_sparse_attn_paged(q, Kd, Vd, td, idx, nnz, w.T, w.k, w.block_k, w.block_q,
                                   causal=bool(w.causal))
    torch.cuda.synchronize()
    return idx.cpu().numpy(), nnz.cpu().numpy(), out


def check_paged(w, page_size, x=None, **kw):
    print(f"[case] paged ps={page_size} {w}", flush=True)
    x = x if x is not None else si.make_inputs(w)
    Kp, Vp, table = to_pages(x, w, page_size, **kw)
    idx, nnz, out = run_paged(x, w, Kp, Vp, table)
    check_valid_lists(idx, nnz, w)
    okw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal)
    o_idx, o_nnz, o_margin = oracle.mask_all(x["q"], x["K"], **okw)
    exempt = compare_masks(idx, nnz, o_idx, o_nnz, o_margin, x, w)
    assert exempt <= exempt_cap(o_margin.size)
    ref = oracle.attn_all(x["q"], x["K"], x["V"], idx, nnz, **okw)
    err = compare_attention(out, ref)
    # the same arithmetic on the same values as the contiguous layout
    c_idx, c_nnz, c_out = run_gpu(x, w)
    assert (c_idx == idx).all() and (c_nnz == nnz).all()
    assert torch.equal(c_out, out)
    print(f"[parity] paged ps={page_size}: problems={o_margin.size} exempt={exempt} max_err={err:.3e}",
          flush=True)


CASES = {
    # page = key block, 32k decode, batch 2
    "decode_ps64": ("decode_32k", 64, dict(B=2, Hq=8, Hkv=2)),
    # pages of 4 key blocks, ragged tail page
    "decode_ps256_ragged": ("decode_32k", 256, dict(Hq=8, Hkv=2, T=30001)),
    # block_k 8 with pages of 8, several rows per call, K_b = 512 (eight tiles per wave and round)
    "decode_bk8_kb512": ("decode_32k", 8, dict(Hq=8, Hkv=2, T=20000, block_k=8, k=4096)),
    "decode_multi_row": ("decode_32k", 64, dict(Hq=8, Hkv=2, Tq=5, T=3000, k=512)),
    # fp32 path, d = 64
    "decode_f32_d64": ("tiny_decode", 16, dict(T=1000)),
    # 256-token splits (16-byte V reads), pages of 2 blocks
    "decode_wide_grid_ps128": ("decode_32k", 128, dict(Hq=32, Hkv=8, Tq=16, T=4096, k=1024)),
    # fp8 KV cache, paged
    "decode_e5m2_ps128": ("decode_32k", 128, dict(B=2, Hq=8, Hkv=2, T=20000, dtype="bf16_e5m2")),
    # group 16
    "decode_group16": ("decode_32k", 64, dict(Hq=16, Hkv=1, T=8192, k=1024)),
    # prefill, pages of 2 blocks, ragged causal chunk
    "prefill_ps128": ("prefill_32k_chunk4k", 128, dict(T=3000, Tq=200, Hq=8, Hkv=2, k=512)),
    "prefill_e5m2_ps64": ("prefill_32k_chunk4k", 64, dict(T=4096, Tq=256, Hq=8, Hkv=2, k=512,
                                                          dtype="bf16_e5m2")),
    "prefill_d64_ps1024": ("prefill_32k_chunk4k", 1024, dict(T=4500, Tq=128, Hq=8, Hkv=2, d=64,
                                                             k=512)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_paged(case):
    base, ps, kw = CASES[case]
    check_paged(si.workload(base, **kw), ps, seed=sorted(CASES).index(case))


@pytest.mark.timeout(900)
def test_paged_max_pages_per_sequence():
    """A 1M-token sequence in 64-token pages: 16384 pages, the most a sequence
    may have in the mask calls (its page numbers fill 64 KiB of LDS)."""
    check_paged(si.workload("decode_32k", Hq=4, Hkv=1, T=1 << 20, k=4096), 64, seed=13)


@pytest.mark.timeout(900)
def test_paged_decode_128k_b4_full():
    """The 128k x4 decode at full size, pages of one key block, shuffled."""
    check_paged(si.workload("decode_128k_b4"), 64, seed=11)


def test_shared_prefix_pages():
    """Two sequences whose first 40 pages are the same physical pages (a shared
    prompt): both read them, and the results equal the contiguous layout's,
    where sequence 1 holds a copy of sequence 0's prefix."""
    w = si.workload("decode_32k", B=2, Hq=8, Hkv=2, T=8192, k=1024)
    x = dict(si.make_inputs(w))
    K, V = x["K"].clone(), x["V"].clone()
    K[1, :, :40 * 64] = K[0, :, :40 * 64]
    V[1, :, :40 * 64] = V[0, :, :40 * 64]
    x["K"], x["V"] = K, V
    check_paged(w, 64, x=x, seed=5, share_prefix_pages=40)
