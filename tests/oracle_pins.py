"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each check takes a loaded oracle library (so the mutation test can run the
same checks against deliberately broken builds) and raises AssertionError on
failure.  Nothing here calls the GPU library.

Kinds of pin used (no check re-derives the oracle's own formulas):
  * hand-traced worked examples (tests/golden/*.json);
  * dense reduction: with k >= the visible keys the method is dense softmax
    attention, compared with torch's scaled_dot_product_attention in float64;
  * exact top-k on tiny inputs when a trace certificate holds (brute force);
  * closed forms: all-zero queries give ties everywhere, so the kept blocks
    are the prefix and the output is the mean of V;
  * invariants: convex combinations of V, constant V, a dominant key,
    scale invariance of the mask, equivariance under batch / head permutation,
    the chunk tree structure and the round count;
  * fp8 (E5M2) K/V: the oracle's decoding of all 256 codes against a
    hand-derived table, torch's float8_e5m2 conversion and the identity
    "E5M2 is the upper byte of IEEE binary16"; the fp8 path against dense
    attention on torch-decoded values and against the float32 path.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _line_inputs(s, *, d=64, Hq=1, Hkv=1, Tq=1, T_cap=None, q_scale=None, seed=0):
    """q rows = scale * e_0, K[t] = s(t) * e_0 in every KV head: score(t) = scale * s(t) exactly."""
    T = len(s)
    T_cap = T if T_cap is None else T_cap
    q = torch.zeros(1, Hq, Tq, d)
    scales = q_scale if q_scale is not None else [1.0] * Tq
    for i in range(Tq):
        q[0, :, i, 0] = scales[i]
    K = torch.zeros(1, Hkv, T_cap, d)
    K[0, :, :T, 0] = torch.tensor(s, dtype=torch.float32)
    g = torch.Generator().manual_seed(seed)
    V = torch.randn(1, Hkv, T_cap, d, generator=g)
    return q, K, V


def _s_from(g, T):
    if "s" in g:
        return [float(x) for x in g["s"]]
    s = [0.0] * T
    for t, v in g["s_sparse"].items():
        s[int(t)] = float(v)
    return s


def _check_trace(got_rounds, want_rounds):
    assert len(got_rounds) == len(want_rounds), (len(got_rounds), len(want_rounds))
    for r, (got, want) in enumerate(zip(got_rounds, want_rounds)):
        cands = sorted(zip(got["start"].tolist(), got["end"].tolist(), got["centre"].tolist()))
        assert cands == sorted(tuple(c) for c in want["candidates"]), (r, cands, want["candidates"])
        kept = sorted((int(a), int(e)) for a, e, k in zip(got["start"], got["end"], got["kept"]) if k)
        assert kept == sorted(tuple(c) for c in want["kept"]), (r, kept, want["kept"])


def _run_golden(lib, name):
    g = _golden(name)
    sh = g["shape"]
    T = sh["T"]
    q, K, _ = _line_inputs(_s_from(g, T), Hq=sh["Hq"], Hkv=sh["Hkv"], Tq=sh["Tq"],
                           T_cap=sh.get("T_cap"), q_scale=g.get("q_scale_per_row"))
    res = oracle.mask_one(q, K, 0, 0, 0, T=T, k=sh["k"], block_k=sh["block_k"],
                          block_q=sh["block_q"], causal=sh["causal"], trace=True, lib=lib)
    assert res["indices"].tolist() == g["expected_indices"], (name, res["indices"].tolist())
    assert res["nnz"] == len(g["expected_indices"])
    _check_trace(res["rounds"], g["trace"])
    return g, res


# ---------------------------------------------------------------- golden traces

def pin_monotone_counterexample(lib):
    g, res = _run_golden(lib, "monotone_counterexample.json")
    s = np.array(g["s"], np.float32)
    top2 = sorted(np.argsort(-s, kind="stable")[:2].tolist())
    assert top2 == g["brute_force_top2"]
    assert res["indices"].tolist() != top2
    # the reported margin is the smallest relative gap at a cut (values as fp32)
    rels = [(np.float64(np.float32(a)) - np.float64(np.float32(b))) / abs(np.float64(np.float32(a)))
            for a, b in g["cut_pairs"]]
    assert math.isclose(res["margin"], min(rels), rel_tol=1e-12), (res["margin"], rels)


def pin_centre_tokens(lib):
    _run_golden(lib, "centre_rule_tokens.json")


def pin_centre_blocks(lib):
    _run_golden(lib, "centre_rule_blocks.json")


def pin_centre_partial_block(lib):
    _run_golden(lib, "centre_partial_block.json")


def pin_uneven_partition(lib):
    g, res = _run_golden(lib, "uneven_partition.json")
    rels = [(a - b) / abs(a) for a, b in g["cut_pairs"]]
    assert math.isclose(res["margin"], min(rels), rel_tol=1e-12)


def pin_causal_vote(lib):
    _run_golden(lib, "causal_vote.json")


# ---------------------------------------------------------------- group maximum

def pin_group_max(lib):
    """Hq=4, Hkv=2: head h reads unit direction e_h, KV head g carries two score
    series; the chunk score must be the max over the group's two heads only."""
    T, d = 32, 64
    rng = np.random.default_rng(7)
    q = torch.zeros(1, 4, 1, d)
    for h in range(4):
        q[0, h, 0, h] = 1.0
    series = rng.permutation(4 * T).astype(np.float32).reshape(4, T) / 7.0  # distinct values
    K = torch.zeros(1, 2, T, d)
    for h in range(4):
        K[0, h // 2, :, h] = torch.from_numpy(series[h])
    for g in range(2):
        res = oracle.mask_one(q, K, 0, g, 0, T=T, k=4, block_k=1, block_q=1, trace=True, lib=lib)
        for rnd in res["rounds"]:
            for t, sc in zip(rnd["centre"], rnd["score"]):
                want = max(series[2 * g][t], series[2 * g + 1][t])
                assert sc == want, (g, t, sc, want)


# ---------------------------------------------------------------- dense reduction

def _dense_reference(q, K, V, T, causal):
    """Dense softmax attention in float64 with torch SDPA (GQA by head expansion)."""
    B, Hq, Tq, d = q.shape
    G = Hq // K.shape[1]
    q64 = q.double()
    K64 = K[:, :, :T].double().repeat_interleave(G, dim=1)
    V64 = V[:, :, :T].double().repeat_interleave(G, dim=1)
    mask = None
    if causal:
        pos = torch.arange(Tq) + (T - Tq)
        mask = torch.arange(T)[None, :] <= pos[:, None]
    return F.scaled_dot_product_attention(q64, K64, V64, attn_mask=mask).numpy()


def pin_dense_reduction(lib):
    rng = torch.Generator().manual_seed(3)
    cases = [  # (B, Hq, Hkv, Tq, T, d, block_k, block_q, causal)
        (2, 4, 2, 1, 100, 64, 8, 1, 1),
        (1, 4, 2, 40, 100, 64, 8, 16, 1),
        (1, 2, 1, 7, 37, 32, 4, 1, 1),
        (1, 4, 2, 24, 70, 64, 16, 8, 0),
    ]
    for (B, Hq, Hkv, Tq, T, d, bk, bq, causal) in cases:
        q = torch.randn(B, Hq, Tq, d, generator=rng)
        K = torch.randn(B, Hkv, T, d, generator=rng)
        V = torch.randn(B, Hkv, T, d, generator=rng)
        nblk = -(-T // bk)
        k = nblk * bk  # k >= T: every block is visible to the search
        idx, nnz, margin = oracle.mask_all(q, K, T=T, k=k, block_k=bk, block_q=bq, causal=causal,
                                           threads=2, lib=lib)
        nqb = -(-Tq // bq)
        for qb in range(nqb):
            last = min((qb + 1) * bq, Tq) - 1
            Tp = (T - Tq + last + 1) if causal else T
            Np = -(-Tp // bk)
            assert (nnz[:, :, qb] == Np).all()
            assert (idx[:, :, qb, :Np] == np.arange(Np)).all()
            assert (idx[:, :, qb, Np:] == -1).all()
        assert np.isinf(margin).all()
        out = oracle.attn_all(q, K, V, idx, nnz, T=T, k=k, block_k=bk, block_q=bq, causal=causal,
                              threads=2, lib=lib)
        ref = _dense_reference(q, K, V, T, causal)
        err = np.abs(out - ref).max()
        assert err < 1e-10, (B, Hq, Hkv, Tq, T, err)


# ---------------------------------------------------------------- exact top-k

def _topk_run(lib, s, k):
    q, K, _ = _line_inputs(list(s))
    return oracle.mask_one(q, K, 0, 0, 0, T=len(s), k=k, block_k=1, block_q=1, trace=True, lib=lib)


def pin_exact_topk_monotone(lib):
    for T in (8, 64, 256):
        for k in (1, 2, 4):
            if k >= T:
                continue
            inc = np.arange(T, dtype=np.float32)
            assert _topk_run(lib, inc, k)["indices"].tolist() == list(range(T - k, T))
            dec = inc[::-1].copy()
            assert _topk_run(lib, dec, k)["indices"].tolist() == list(range(k))


def pin_exact_topk_disjoint_chunks(lib):
    """Increasing inside each initial chunk, value ranges of chunks disjoint."""
    rng = np.random.default_rng(11)
    for trial in range(40):
        k = int(rng.choice([2, 4]))
        T = k * int(rng.choice([4, 8, 16]))
        chunk = T // k
        order = rng.permutation(k)
        s = np.zeros(T, np.float32)
        for c in range(k):
            s[c * chunk:(c + 1) * chunk] = order[c] * 1000 + np.sort(rng.choice(900, chunk, replace=False))
        got = _topk_run(lib, s, k)["indices"].tolist()
        want = sorted(np.argsort(-s, kind="stable")[:k].tolist())
        assert got == want, (trial, got, want)


def pin_exact_topk_certified(lib):
    """Random distinct scores: whenever the trace shows every kept chunk's maximum
    at least every dropped chunk's maximum, in every round, the result is the
    exact top-k (induction on rounds)."""
    rng = np.random.default_rng(5)
    certified = 0
    for trial in range(400):
        k = int(rng.choice([1, 2, 3]))
        T = int(rng.choice([8, 12, 16, 24]))
        s = rng.permutation(T).astype(np.float32)
        res = _topk_run(lib, s, k)
        ok = True
        for rnd in res["rounds"]:
            mx = [s[a:e].max() for a, e in zip(rnd["start"], rnd["end"])]
            kept = [m for m, kp in zip(mx, rnd["kept"]) if kp]
            dropped = [m for m, kp in zip(mx, rnd["kept"]) if not kp]
            if dropped and min(kept) < max(dropped):
                ok = False
                break
        if ok:
            certified += 1
            want = sorted(np.argsort(-s, kind="stable")[:k].tolist())
            assert res["indices"].tolist() == want, (trial, s, res["indices"])
    assert certified >= 50, certified


# ---------------------------------------------------------------- structure

def pin_tree_structure(lib):
    """Round count, candidate count, and the chunk tree: the candidates of a round
    tile exactly the chunks kept by the previous round, each chunk splits into at
    most two halves, and final blocks lie in a kept chunk of every round."""
    import synth_inputs as si
    w = si.workload("tiny_decode")
    x = si.make_inputs(w)
    res = oracle.mask_one(x["q"], x["K"], 0, 0, 0, T=w.T, k=w.k, block_k=w.block_k,
                          block_q=w.block_q, trace=True, lib=lib)
    Np, Kb = w.T // w.block_k, w.kb
    R = int(math.ceil(math.log2(Np / Kb)))
    assert len(res["rounds"]) == R == 3
    for rnd in res["rounds"]:
        assert len(rnd["start"]) == 2 * Kb and int(rnd["kept"].sum()) == Kb
    # uneven cases: causal prefill-like block counts
    rng = torch.Generator().manual_seed(9)
    for T in (449 * 8, 500 * 8, 37 * 8 + 3):
        q = torch.randn(1, 2, 1, 64, generator=rng)
        K = torch.randn(1, 1, T + 64, 64, generator=rng)  # spare capacity rows past T
        Kb = 32 if T > 1000 else 5
        res = oracle.mask_one(q, K, 0, 0, 0, T=T, k=Kb * 8, block_k=8, block_q=1, trace=True,
                              lib=lib)
        Np = -(-T // 8)
        prev = [(i * Np // Kb, (i + 1) * Np // Kb) for i in range(Kb)]
        assert len(res["rounds"]) <= math.ceil(math.log2(-(-Np // Kb)))
        final = res["indices"].tolist()
        assert len(set(final)) == Kb and all(0 <= b < Np for b in final)
        for rnd in res["rounds"]:
            cands = sorted(zip(rnd["start"].tolist(), rnd["end"].tolist()))
            tiles = []
            for a, e in sorted(prev):
                kids = [c for c in cands if a <= c[0] and c[1] <= e]
                assert 1 <= len(kids) <= 2 and kids[0][0] == a and kids[-1][1] == e
                if len(kids) == 2:
                    assert kids[0][1] == kids[1][0] == a + (e - a) // 2
                else:
                    assert e - a == 1
                tiles += kids
            assert tiles == cands
            prev = [(int(a), int(e)) for a, e, kp in zip(rnd["start"], rnd["end"], rnd["kept"]) if kp]
            for b in final:
                assert any(a <= b < e for a, e in prev)
        assert all(e - a == 1 for a, e in prev)


# ---------------------------------------------------------------- closed forms

def pin_zero_query_ties(lib):
    """q = 0: every score is exactly 0, ties go to the lower start, the kept
    blocks are the prefix 0..K_b-1 and attention is the mean of V over them."""
    rng = torch.Generator().manual_seed(1)
    for (Tq, bq, T, bk, k) in ((1, 1, 200, 8, 48), (20, 4, 150, 8, 40), (33, 16, 301, 16, 64)):
        q = torch.zeros(1, 4, Tq, 64)
        K = torch.randn(1, 2, T + 64, 64, generator=rng)  # spare capacity rows past T
        V = torch.randn(1, 2, T + 64, 64, generator=rng)
        idx, nnz, margin = oracle.mask_all(q, K, T=T, k=k, block_k=bk, block_q=bq, threads=2, lib=lib)
        Kb = k // bk
        assert (idx == np.arange(Kb)).all() and (nnz == Kb).all()
        assert (margin == 0).all()
        out = oracle.attn_all(q, K, V, idx, nnz, T=T, k=k, block_k=bk, block_q=bq, threads=2, lib=lib)
        Vn = V.double().numpy()
        for h in range(4):
            for i in range(Tq):
                pos = T - Tq + i
                hi = min(Kb * bk, pos + 1)
                want = Vn[0, h // 2, :hi].mean(axis=0)
                assert np.abs(out[0, h, i] - want).max() < 1e-12


# ---------------------------------------------------------------- attention invariants

def pin_attention_invariants(lib):
    import synth_inputs as si
    w = si.workload("tiny_decode")
    x = si.make_inputs(w)
    kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal, lib=lib)
    idx, nnz, _ = oracle.mask_all(x["q"], x["K"], threads=2, **kw)
    out = oracle.attn_all(x["q"], x["K"], x["V"], idx, nnz, threads=2, **kw)
    toks = np.concatenate([np.arange(b * w.block_k, (b + 1) * w.block_k) for b in idx[0, 0, 0]])
    Vsel = x["V"][0, 0, toks].double().numpy()
    assert (out[0, 0, 0] >= Vsel.min(0) - 1e-12).all() and (out[0, 0, 0] <= Vsel.max(0) + 1e-12).all()
    # constant V
    Vc = torch.full_like(x["V"], 0.375)
    oc = oracle.attn_all(x["q"], x["K"], Vc, idx, nnz, threads=2, **kw)
    assert np.abs(oc - 0.375).max() < 1e-12
    # one dominant key: its V row comes out (margin of 60 in the logit)
    q = torch.zeros_like(x["q"])
    q[0, 0, 0, 0] = 1.0
    K = torch.zeros_like(x["K"])
    t_star = int(toks[len(toks) // 2])
    K[0, 0, t_star, 0] = 60.0 * math.sqrt(w.d)
    od = oracle.attn_all(q, K, x["V"], idx, nnz, threads=2, **kw)
    # the other weights are e^-60 each, far below one ulp of the result
    assert np.abs(od[0, 0, 0] - x["V"][0, 0, t_star].double().numpy()).max() < 1e-14


def pin_mask_invariances(lib):
    """Doubling q leaves the mask unchanged (exact in binary floating point);
    permuting batch entries or KV heads (with their query groups) permutes it."""
    import synth_inputs as si
    w = si.workload("decode_32k", T=4096, k=512, B=2)
    x = si.make_inputs(w)
    kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal, threads=4, lib=lib)
    q = x["q"].float()
    K = x["K"].float()
    idx, nnz, _ = oracle.mask_all(q, K, **kw)
    idx2, _, _ = oracle.mask_all(q * 2, K, **kw)
    assert (idx == idx2).all()
    G = w.G
    perm_g = [3, 0, 7, 1, 6, 2, 5, 4]
    perm_h = [g * G + j for g in perm_g for j in range(G)]
    qp = q[[1, 0]][:, perm_h].contiguous()
    Kp = K[[1, 0]][:, perm_g].contiguous()
    idxp, _, _ = oracle.mask_all(qp, Kp, **kw)
    assert (idxp == idx[[1, 0]][:, perm_g]).all()


# ---------------------------------------------------------------- fp8 (E5M2) K/V

def pin_e5m2_codes(lib):
    got = oracle.e5m2_values(lib)
    table = _golden("e5m2_codes.json")["values"]
    for code, want in table.items():
        c = int(code, 16)
        if want == "nan":
            assert math.isnan(got[c]), (code, got[c])
        else:
            w = float(want)
            assert got[c] == w and math.copysign(1.0, got[c]) == math.copysign(1.0, w), (code, got[c])
    codes = torch.arange(256, dtype=torch.uint8)
    via_torch = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    via_half = (codes.numpy().astype(np.uint16) << 8).view(np.float16).astype(np.float64)
    for ref in (via_torch, via_half):
        assert np.array_equal(np.isnan(got), np.isnan(ref))
        fin = ~np.isnan(ref)
        assert np.array_equal(got[fin], ref[fin])
        assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))


def pin_e5m2_kv(lib):
    """fp8 K/V: dense reduction against torch on torch-decoded values, and the
    same mask and outputs as the float32 path on those values."""
    rng = torch.Generator().manual_seed(11)
    B, Hq, Hkv, d, T, bk = 1, 4, 2, 64, 200, 8
    q = torch.randn(B, Hq, 1, d, generator=rng).to(torch.bfloat16)
    K8 = (torch.randn(B, Hkv, T, d, generator=rng) * 2).to(torch.float8_e5m2)
    V8 = torch.randn(B, Hkv, T, d, generator=rng).to(torch.float8_e5m2)
    Kf, Vf = K8.float(), V8.float()
    nblk = -(-T // bk)
    kw = dict(T=T, block_k=bk, block_q=1, causal=1, threads=2, lib=lib)
    idx, nnz, _ = oracle.mask_all(q, K8, k=nblk * bk, **kw)
    out = oracle.attn_all(q, K8, V8, idx, nnz, k=nblk * bk, **kw)
    ref = _dense_reference(q.float(), Kf, Vf, T, 1)
    assert np.abs(out - ref).max() < 1e-10
    k = 5 * bk  # sparse: 5 of 25 blocks
    idx8, nnz8, m8 = oracle.mask_all(q, K8, k=k, **kw)
    idxf, nnzf, mf = oracle.mask_all(q, Kf, k=k, **kw)
    assert (idx8 == idxf).all() and (nnz8 == nnzf).all() and np.array_equal(m8, mf)
    o8 = oracle.attn_all(q, K8, V8, idx8, nnz8, k=k, **kw)
    of = oracle.attn_all(q, Kf, Vf, idx8, nnz8, k=k, **kw)
    assert np.array_equal(o8, of)
    assert not np.array_equal(o8, out)  # the sparse result differs from the dense one


# ---------------------------------------------------------------- dense part (sink + window)

def pin_dense_part_trace(lib):
    """Hand-traced search with sink and window blocks, and attention over the
    union of the dense blocks and the list (softmax over the named tokens)."""
    g = _golden("dense_part.json")
    sh = g["shape"]
    T = sh["T"]
    q, K, V = _line_inputs(g["s"])
    kw = dict(T=T, k=sh["k"], block_k=sh["block_k"], block_q=1, causal=1, sink=sh["sink"],
              window=sh["window"], lib=lib)
    res = oracle.mask_one(q, K, 0, 0, 0, trace=True, **kw)
    assert res["indices"].tolist() == g["expected_indices"], res["indices"].tolist()
    _check_trace(res["rounds"], g["trace"])
    assert math.isclose(res["margin"], g["expected_margin"], rel_tol=1e-12), res["margin"]
    idx = res["indices"].reshape(1, 1, 1, -1)
    nnz = np.array([[[res["nnz"]]]], np.int32)
    out = oracle.attn_row(q, K, V, idx, nnz, 0, 0, 0, **kw)
    toks = g["attended_tokens"]
    logit = np.array([g["s"][t] for t in toks]) / math.sqrt(q.shape[-1])
    w = np.exp(logit - logit.max())
    want = (w[:, None] * V[0, 0, toks].double().numpy()).sum(0) / w.sum()
    assert np.abs(out - want).max() < 1e-12


def pin_dense_part_reduction(lib):
    """sink + window + k covering every visible block: dense attention (torch SDPA)."""
    rng = torch.Generator().manual_seed(21)
    for (B, Hq, Hkv, Tq, T, d, bk, bq, sink, window) in [(1, 4, 2, 1, 100, 64, 8, 1, 16, 40),
                                                         (1, 4, 2, 40, 100, 64, 8, 16, 8, 24)]:
        q = torch.randn(B, Hq, Tq, d, generator=rng)
        K = torch.randn(B, Hkv, T, d, generator=rng)
        V = torch.randn(B, Hkv, T, d, generator=rng)
        nblk = -(-T // bk)
        k = (nblk - (sink + window) // bk) * bk  # the search sees every middle block
        kw = dict(T=T, k=k, block_k=bk, block_q=bq, causal=1, sink=sink, window=window, threads=2,
                  lib=lib)
        idx, nnz, margin = oracle.mask_all(q, K, **kw)
        assert np.isinf(margin).all()
        out = oracle.attn_all(q, K, V, idx, nnz, **kw)
        assert np.abs(out - _dense_reference(q, K, V, T, 1)).max() < 1e-10


def pin_dense_part_search_range(lib):
    """For a decode row the search with sink S and window W equals the plain
    search on the keys between them (same scores, centres and ranking), its
    block ids shifted by S_b."""
    import synth_inputs as si
    w = si.workload("decode_32k", T=3000, Hq=4, Hkv=1, block_k=16, k=256)
    x = si.make_inputs(w)
    q, K = x["q"].float(), x["K"].float()
    S, W = 5 * 16, 9 * 16
    Np = -(-w.T // 16)
    hi = (Np - W // 16) * 16  # first token of the window
    kw = dict(k=w.k, block_k=16, block_q=1, causal=1, threads=2, lib=lib)
    idx, nnz, m = oracle.mask_all(q, K, T=w.T, sink=S, window=W, **kw)
    Kc = K[:, :, S:hi].contiguous()
    idx_c, nnz_c, m_c = oracle.mask_all(q, Kc, T=hi - S, **kw)
    assert (nnz == nnz_c).all() and np.array_equal(m, m_c)
    assert (idx == np.where(idx_c >= 0, idx_c + S // 16, -1)).all()


def pin_dense_part_union(lib):
    """Attention with a dense part equals attention over the explicit list of
    the dense blocks followed by the listed blocks outside them; listed ids
    inside a dense range add nothing."""
    rng = torch.Generator().manual_seed(22)
    T, d, bk, sink, window, kb = 700, 32, 8, 24, 40, 12
    q = torch.randn(1, 2, 3, d, generator=rng)
    K = torch.randn(1, 1, T, d, generator=rng)
    V = torch.randn(1, 1, T, d, generator=rng)
    Np = -(-T // bk)
    lst = np.array([0, 2, 5, 40, 41, 41, 80, Np - 1, Np - 3, 500, -1, 63], np.int32)  # dense ids, a repeat, bad ids
    idx = lst.reshape(1, 1, 1, kb)
    nnz = np.array([[[kb]]], np.int32)
    kw = dict(T=T, k=kb * bk, block_k=bk, block_q=3, causal=1, threads=2, lib=lib)
    out = oracle.attn_all(q, K, V, idx, nnz, sink=sink, window=window, **kw)
    sb, wb = sink // bk, window // bk
    dense = list(range(sb)) + list(range(Np - wb, Np))
    rest = [int(b) for b in lst if 0 <= b < Np and not (b < sb or b >= Np - wb)]
    full = np.array(dense + rest, np.int32)
    kb2 = len(full)
    out2 = oracle.attn_all(q, K, V, full.reshape(1, 1, 1, kb2), np.array([[[kb2]]], np.int32),
                           T=T, k=kb2 * bk, block_k=bk, block_q=3, causal=1, threads=2, lib=lib)
    assert np.array_equal(out, out2)



# ---------------------------------------------------------------- near-tie-tolerant search

def pin_reach_branch_golden(lib):
    """Hand-traced: a near tie at the first cut branches into two final lists."""
    g = _golden("near_tie_branch.json")
    sh = g["shape"]
    q, K, _ = _line_inputs(_s_from(g, sh["T"]))
    kw = dict(T=sh["T"], k=sh["k"], block_k=sh["block_k"], block_q=sh["block_q"], causal=sh["causal"])
    r = oracle.mask_one(q, K, 0, 0, 0, lib=lib, **kw)
    assert r["indices"].tolist() == g["exact_indices"]
    n, lists = oracle.mask_reach(q, K, 0, 0, 0, tol=g["tol"], lib=lib, **kw)
    assert n == len(g["reachable"]) and sorted(l.tolist() for l in lists) == g["reachable"], lists
    for t in g["reachable"]:
        assert oracle.mask_reach(q, K, 0, 0, 0, tol=g["tol"], target=t, lib=lib, **kw)[0] == 1, t
    for t in g["unreachable"]:
        assert oracle.mask_reach(q, K, 0, 0, 0, tol=g["tol"], target=t, lib=lib, **kw)[0] == 0, t
    n, lists = oracle.mask_reach(q, K, 0, 0, 0, tol=g["tol_below_gap"], lib=lib, **kw)
    assert n == 1 and [l.tolist() for l in lists] == g["reachable_below_gap"]


def pin_reach_identity(lib):
    """Without near ties the tolerant search has exactly one result, the exact
    search's; with them the exact search's result is always among its results.
    Seeded AR(1) decode and prefill problems, several group sizes."""
    import synth_inputs as si
    cases = [si.workload("decode_32k", T=6000, Hq=8, Hkv=2, Tq=8, k=512, seed=77),
             si.workload("decode_32k", T=3000, Hq=16, Hkv=1, Tq=8, block_k=16, k=256, seed=78),
             si.workload("prefill_32k_chunk4k", T=1500, Tq=640, Hq=8, Hkv=2, k=256, block_k=32,
                         seed=79)]
    tol = 1e-4
    seen_exempt = seen_safe = 0
    for w in cases:
        x = si.make_inputs(w)
        kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal)
        idx, _, margin = oracle.mask_all(x["q"], x["K"], lib=lib, **kw)
        for b, g, qb in np.ndindex(*margin.shape):
            n, lists = oracle.mask_reach(x["q"], x["K"], b, g, qb, tol=tol, lib=lib, **kw)
            exact = idx[b, g, qb].tolist()
            if margin[b, g, qb] > tol:
                seen_safe += 1
                assert n == 1 and lists[0].tolist() == exact, (w.name, b, g, qb, n)
            elif margin[b, g, qb] < tol:
                seen_exempt += 1
                assert exact in [l.tolist() for l in lists], (w.name, b, g, qb)
    assert seen_safe >= 30, seen_safe


def pin_reach_target_agrees(lib):
    """Target mode answers exactly the membership question of the enumeration."""
    g = _golden("near_tie_branch.json")
    sh = g["shape"]
    q, K, _ = _line_inputs(_s_from(g, sh["T"]))
    kw = dict(T=sh["T"], k=sh["k"], block_k=sh["block_k"], block_q=sh["block_q"], causal=sh["causal"])
    n, lists = oracle.mask_reach(q, K, 0, 0, 0, tol=g["tol"], lib=lib, **kw)
    reach = {tuple(l.tolist()) for l in lists}
    T = sh["T"]
    for a in range(T):
        for b in range(a + 1, T):
            got = oracle.mask_reach(q, K, 0, 0, 0, tol=g["tol"], target=[a, b], lib=lib, **kw)[0]
            assert got == ((a, b) in reach), (a, b)


# ---------------------------------------------------------------- multi-stage search

def _stages_golden(lib, name):
    g = _golden(name)
    sh = g["shape"]
    q, K, _ = _line_inputs(_s_from(g, sh["T"]))
    stages = [(c, k) for c, k in g["stages"]]
    r = oracle.mask_stages_one(q, K, 0, 0, 0, stages, T=sh["T"], block_k=sh["block_k"],
                               causal=sh["causal"], lib=lib)
    rounds = [t for t in g["trace"] if t["stage"] > 0]
    _check_trace(r["rounds"], rounds)
    assert r["indices"].tolist() == g["expected_indices"] + [-1] * (len(r["indices"]) -
                                                                  len(g["expected_indices"]))
    assert r["nnz"] == len(g["expected_indices"])
    assert abs(r["margin"] - g["expected_margin"]) < 1e-12, r["margin"]


def pin_stages_three_golden(lib):
    """Hand-traced: fixed-size stage 0 with a partial chunk, a pass-through."""
    _stages_golden(lib, "stages_three.json")


def pin_stages_two_rounds_golden(lib):
    """Hand-traced: a stage that needs two rounds, a tie broken by start."""
    _stages_golden(lib, "stages_two_rounds.json")


def pin_stages_fit_first_round_golden(lib):
    """Hand-traced: a stage whose incoming chunks already fit still ranks them."""
    _stages_golden(lib, "stages_fit_first_round.json")


def pin_stages_identity(lib):
    """A stage list whose stage 0 is the uniform partition (M a multiple of
    K_b) and whose one later stage keeps K_b single blocks is the one-stage
    search: indices, counts and margins equal or_mask_one's exactly, over
    several shapes (query rows, groups, block sizes, a dense part)."""
    import synth_inputs as si
    cases = [(si.workload("decode_32k", T=8192, Hq=8, Hkv=2, Tq=1, k=512, seed=81), 0, 0),
             (si.workload("decode_32k", T=4096, Hq=16, Hkv=1, Tq=1, block_k=16, k=256, seed=82), 0, 0),
             (si.workload("decode_32k", T=8192 + 64 * 12, Hq=4, Hkv=4, Tq=1, k=256, seed=83), 64 * 4,
              64 * 8)]
    for w, sink, window in cases:
        x = si.make_inputs(w)
        kw = dict(T=w.T, causal=w.causal, sink=sink, window=window)
        idx, nnz, margin = oracle.mask_all(x["q"], x["K"], k=w.k, block_k=w.block_k, block_q=1,
                                           lib=lib, **kw)
        M = -(-w.T // w.block_k) - sink // w.block_k - window // w.block_k
        assert M % w.kb == 0, (w, M)
        stages = [((M // w.kb) * w.block_k, None), (w.block_k, w.k)]
        s_idx, s_nnz, s_margin = oracle.mask_stages_all(x["q"], x["K"], stages, block_k=w.block_k,
                                                        lib=lib, **kw)
        assert (s_idx == idx).all() and (s_nnz == nnz).all(), w
        assert np.array_equal(s_margin, margin), w


def pin_stages_structure(lib):
    """Counts and tree structure of a multi-stage search on seeded data: each
    round keeps min(stage keep, candidates); a candidate is a half of a kept
    chunk larger than the stage's size or such a chunk itself; the result
    lists the last stage's single blocks, each inside a chunk kept in every
    round; every stage-0 block range is covered by the first round."""
    import synth_inputs as si
    w = si.workload("decode_32k", T=5000, Hq=8, Hkv=2, Tq=1, block_k=8, k=256, seed=84)
    x = si.make_inputs(w)
    stages = [(128, None), (32, 2048), (16, 1024), (8, 256)]  # chunks 16 -> 4 -> 2 -> 1 blocks
    keeps = [None, 64, 64, 32]
    M = -(-w.T // 8)
    r = oracle.mask_stages_one(x["q"], x["K"], 0, 0, 0, stages, T=w.T, block_k=8, lib=lib)
    rounds = r["rounds"]
    # stage 1 from 16-block chunks to 4: two rounds; stage 2 (4 -> 2): one; stage 3 (2 -> 1): one
    assert len(rounds) == 4, len(rounds)
    first = rounds[0]
    assert sorted(first["start"].tolist())[0] == 0 and max(first["end"]) == M
    covered = sorted(zip(first["start"].tolist(), first["end"].tolist()))
    assert all(a == b for (_, a), (b, _) in zip(covered, covered[1:]))  # the halves tile [0, M)
    stage_of_round = [1, 1, 2, 3]
    prev = None
    for ri, rd in enumerate(rounds):
        keep = keeps[stage_of_round[ri]]
        assert rd["kept"].sum() == min(keep, len(rd["kept"]))
        if prev is not None:
            tb = {1: 4, 2: 2, 3: 1}[stage_of_round[ri]]  # this round's stage chunk size
            kept_prev = [(a, e) for a, e, k in zip(prev["start"], prev["end"], prev["kept"]) if k]
            for a, e in zip(rd["start"], rd["end"]):
                assert any(pa <= a and e <= pe and (e - a == pe - pa if pe - pa <= tb
                                                    else e - a in ((pe - pa) // 2, pe - pa - (pe - pa) // 2))
                           for pa, pe in kept_prev), (ri, a, e)
        prev = rd
    final = [a for a, k in zip(rounds[-1]["start"], rounds[-1]["kept"]) if k]
    assert sorted(final) == r["indices"][:r["nnz"]].tolist() and r["nnz"] == 32
    for rd in rounds:
        kept = [(a, e) for a, e, k in zip(rd["start"], rd["end"], rd["kept"]) if k]
        assert all(any(a <= t < e for a, e in kept) for t in final)


def pin_stages_reach_identity(lib):
    """The tolerant search over a stage list: without near ties exactly the
    greedy result; with them the greedy result is among its results."""
    import synth_inputs as si
    w = si.workload("decode_32k", T=6000, Hq=8, Hkv=2, Tq=6, block_k=16, k=256, seed=85)
    x = si.make_inputs(w)
    stages = [(256, None), (64, 1024), (16, 256)]
    idx, nnz, margin = oracle.mask_stages_all(x["q"], x["K"], stages, T=w.T, block_k=16, lib=lib)
    safe = 0
    for b, g, i in np.ndindex(*margin.shape):
        n, lists = oracle.mask_stages_reach(x["q"], x["K"], b, g, i, stages, T=w.T, block_k=16,
                                            lib=lib)
        exact = idx[b, g, i].tolist()
        if margin[b, g, i] > 1e-4:
            safe += 1
            assert n == 1 and lists[0].tolist() == exact, (b, g, i, n)
        else:
            assert exact in [l.tolist() for l in lists]
    assert safe >= 6


def pin_stages_exact_topk(lib):
    """block_k = 1, exact scores increasing inside each stage-0 chunk with
    pairwise disjoint value ranges between chunks: every stage keeps the
    chunks holding the largest scores, so the result is the brute-force top."""
    rng = np.random.default_rng(7)
    for trial in range(20):
        T = int(rng.integers(40, 200))
        c0 = int(rng.choice([8, 16]))
        n0 = -(-T // c0)
        base = rng.permutation(n0) * 10.0  # chunk value ranges [10 j, 10 j + 1)
        s = [float(base[t // c0] + (t % c0) / (2 * c0)) for t in range(T)]
        keep_last = int(rng.integers(1, 5))
        stages = [(c0, None), (c0 // 4, (c0 // 4) * keep_last), (1, keep_last)]
        q, K, _ = _line_inputs(s)
        r = oracle.mask_stages_one(q, K, 0, 0, 0, stages, T=T, block_k=1, lib=lib)
        brute = sorted(np.argsort(s)[::-1][:keep_last].tolist())
        assert r["indices"][:r["nnz"]].tolist() == brute, (trial, r["indices"], brute)


ALL_PINS = [
    pin_monotone_counterexample, pin_centre_tokens, pin_centre_blocks, pin_centre_partial_block,
    pin_uneven_partition, pin_causal_vote, pin_group_max, pin_dense_reduction,
    pin_exact_topk_monotone, pin_exact_topk_disjoint_chunks, pin_exact_topk_certified,
    pin_tree_structure, pin_zero_query_ties, pin_attention_invariants, pin_mask_invariances,
    pin_e5m2_codes, pin_e5m2_kv, pin_dense_part_trace, pin_dense_part_reduction,
    pin_dense_part_search_range, pin_dense_part_union, pin_reach_branch_golden,
    pin_reach_identity, pin_reach_target_agrees, pin_stages_three_golden,
    pin_stages_two_rounds_golden, pin_stages_fit_first_round_golden, pin_stages_identity, pin_stages_structure,
    pin_stages_reach_identity, pin_stages_exact_topk,
]
