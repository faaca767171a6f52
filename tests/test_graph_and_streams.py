"""The library under HIP graph capture and on several streams.

Every call only enqueues kernels on the caller's stream (no allocation, no
synchronisation, no memset), so a captured graph replays it.  Each graph here
is replayed three times with other eager work of the library in between, and
every replay must equal the eager result bit for bit; two problems run on two
streams at once must each equal their eager result.
"""
import pytest
import torch

import synth_inputs as si

pytestmark = pytest.mark.gpu


def _setup(w, ext=None):
    import long_context_sparse_mask_amd as hs
    x = si.make_inputs(w)
    dev = "cuda"
    q, K, V = (x[n].to(dev) for n in ("q", "K", "V"))
    kw = dict(T=w.T, causal=bool(w.causal), **(ext or {}))
    nqb = -(-w.Tq // w.block_q)
    idx = torch.empty((w.B, w.Hkv, nqb, w.kb), dtype=torch.int32, device=dev)
    nnz = torch.empty((w.B, w.Hkv, nqb), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    need = hs.hipsa_workspace_bytes_ex(q, K, w.k, w.block_k, w.block_q, **kw)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def step(stream=None):
        hs.hip_mask_estimate_ex(q, K, w.k, w.block_k, w.block_q, indices=idx, nnz=nnz,
                                stream=stream, **kw)
        hs.hip_sparse_attn_ex(q, K, V, idx, nnz, w.k, w.block_k, w.block_q, out=out, workspace=ws,
                              stream=stream, **kw)
    return step, idx, nnz, out


CASES = {
    "decode": (dict(name="decode_32k", B=2, Hq=8, Hkv=2, T=20000), None),
    "prefill": (dict(name="prefill_32k_chunk4k", T=3000, Tq=200, Hq=8, Hkv=2, k=512), None),
    "decode_e5m2_dense": (dict(name="decode_32k", Hq=8, Hkv=2, T=12000, dtype="bf16_e5m2"),
                          dict(sink=64, window=1024)),
    # 1024 split workgroups: the 16-byte V reads of the split kernel
    "decode_wide_grid": (dict(name="decode_32k", Hq=32, Hkv=8, Tq=16, T=4096, k=1024), None),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_graph_replays_match_eager(case):
    wkw, ext = CASES[case]
    wkw = dict(wkw)
    w = si.workload(wkw.pop("name"), **wkw)
    step, idx, nnz, out = _setup(w, ext)
    other, _, _, other_out = _setup(si.workload("decode_32k", Hq=4, Hkv=1, T=5000, seed=77))
    step()
    torch.cuda.synchronize()
    want = (idx.clone(), nnz.clone(), out.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        idx.fill_(-5)
        out.zero_()
        other()  # eager work of the library between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want[0]) and torch.equal(nnz, want[1]), (case, rep)
        assert torch.equal(out, want[2]), (case, rep)


def test_paged_graph_replay():
    from test_paged_kv_parity import to_pages
    import long_context_sparse_mask_amd as hs
    w = si.workload("decode_32k", B=2, Hq=8, Hkv=2, T=10000)
    x = si.make_inputs(w)
    Kp, Vp, table = to_pages(x, w, 128, seed=4)
    q, Kp, Vp, table = x["q"].cuda(), Kp.cuda(), Vp.cuda(), table.cuda()
    idx = torch.empty((w.B, w.Hkv, 1, w.kb), dtype=torch.int32, device="cuda")
    nnz = torch.empty((w.B, w.Hkv, 1), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)

    def step():
        hs.hip_mask_estimate_paged(q, Kp, table, w.T, w.k, w.block_k, 1, indices=idx, nnz=nnz)
        hs.hip_sparse_attn_paged(q, Kp, Vp, table, idx, nnz, w.T, w.k, w.block_k, 1, out=out)
    step()
    torch.cuda.synchronize()
    want = (idx.clone(), out.clone())
    g = torch.cuda.CUDAGraph()
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")  # workspace made outside capture

    def step_ws():
        hs.hip_mask_estimate_paged(q, Kp, table, w.T, w.k, w.block_k, 1, indices=idx, nnz=nnz)
        hs.hip_sparse_attn_paged(q, Kp, Vp, table, idx, nnz, w.T, w.k, w.block_k, 1, out=out,
                                 workspace=ws)
    step_ws()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step_ws()
    for rep in range(3):
        out.zero_()
        idx.fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, want[0]) and torch.equal(out, want[1]), rep


def test_two_streams_at_once():
    """Two independent problems enqueued on two streams without waiting: each
    result equals its eager single-stream result."""
    a_step, a_idx, a_nnz, a_out = _setup(si.workload("decode_32k", B=2, Hq=8, Hkv=2, T=20000))
    b_step, b_idx, b_nnz, b_out = _setup(si.workload("prefill_32k_chunk4k", T=3000, Tq=256, Hq=8,
                                                     Hkv=2, k=512))
    a_step()
    b_step()
    torch.cuda.synchronize()
    want = [t.clone() for t in (a_idx, a_out, b_idx, b_out)]
    for t in (a_idx, b_idx):
        t.fill_(-5)
    a_out.zero_()
    b_out.zero_()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        a_step(s1)
        b_step(s2)
    torch.cuda.synchronize()
    for got, exp in zip((a_idx, a_out, b_idx, b_out), want):
        assert torch.equal(got, exp)
