#!/usr/bin/env python3
"""Benchmark of the HiP hot path on one MI355X: mask estimation + block-sparse
attention per step, on seeded synthetic Llama-3.1-8B-shaped inputs.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  Default workload: decode at 128k context, batch 4,
32 query / 8 KV heads, d=128, bf16, block_k=64, k=2048 (decode_128k_b4).
A step = one hip_decode_step call (mask estimation then sparse attention) for
the whole batch; the value is microseconds per step (lower is better).  With
the default workload the line also carries the 32k and 1M-token decodes
(`decode_32k`, `decode_1m_needles`, the latter with needle recall), the step
as two calls, the chunked-prefill throughput (4096-token chunk at the end of
a 32k sequence, `prefill`), the fp8, paged and dense-part variants, and the
multi-stage search (`multi_stage`: a stage list per workload, alone and
followed by the sparse attention).

Timing: the K timed steps (and the W warm-up steps) are captured as HIP
graphs of C-ABI launches on torch's capture stream and replayed, so host
call overhead is not in the figure; HIP events on that stream bracket the
replay.  Consecutive steps rotate over 8 rolled copies of the layer's K/V
and 16 query sets, so the selected blocks differ from step to step and come
from HBM, not from the 256 MB last-level cache.  The attention-only and
mask-reuse legs (`mask_reuse`: the mask re-estimated every r_m steps,
attention every step) attend each step over the lists that step's own mask
selected, so they read as many distinct bytes as full steps do.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
N_LAYER_COPIES = 8   # defaults; --layer-copies / --query-sets override
N_QUERY_SETS = 16


def rounds_of(Np: int, Kb: int) -> int:
    """Rounds of the search when every chunk halves evenly (power-of-two ratio)."""
    return 0 if Np <= Kb else int(math.ceil(math.log2(Np / Kb)))


# bytes per element of (q and out, K and V) for each workload element type
ELEM_BYTES = {"f32": (4, 4), "bf16": (2, 2), "bf16_e5m2": (2, 1)}


def decode_bytes(w) -> dict:
    """Algorithmic HBM bytes of one decode step (what the method must move)."""
    qsz, kvsz = ELEM_BYTES[w.dtype]
    row = w.d * kvsz
    P = w.B * w.Hkv * w.Tq
    Np = -(-w.T // w.block_k)
    R = rounds_of(Np, w.kb)
    centre = P * R * 2 * w.kb * row
    kv = P * 2 * min(w.kb, Np) * w.block_k * row
    q = w.B * w.Hq * w.Tq * w.d * qsz
    idx = P * (w.kb + 1) * 4
    return {"centre": centre, "kv": kv, "q": q, "out": q, "indices": idx, "rounds": R,
            "mask": centre + q + idx, "attn": kv + 2 * q + idx, "step": centre + kv + 3 * q + 2 * idx}


def prefill_flops(w) -> dict:
    """Algorithmic FLOPs of one prefill chunk: mask scoring (per round a
    [G*b_q x d] . [d x 2K_b] product per problem) and attention (QK^T and PV
    over the visible selected keys)."""
    nqb = -(-w.Tq // w.block_q)
    mask = 0
    attn = 0
    for qb in range(nqb):
        r1 = min((qb + 1) * w.block_q, w.Tq)
        rows = r1 - qb * w.block_q
        Tp = w.T - w.Tq + r1
        Np = -(-Tp // w.block_k)
        ncand = 0
        if Np > w.kb:
            sizes = [(i + 1) * Np // w.kb - i * Np // w.kb for i in range(w.kb)]
            while max(sizes) > 1:  # worst case: the widest chunks survive every round
                ncand += sum(2 if s > 1 else 1 for s in sizes)
                halves = []
                for s in sizes:
                    halves += [s // 2, s - s // 2] if s > 1 else [s]
                sizes = sorted(halves, reverse=True)[:w.kb]
        mask += w.B * w.Hkv * 2 * w.G * rows * w.d * ncand
        keys = min(w.kb, Np) * w.block_k
        attn += w.B * w.Hq * rows * keys * w.d * 4
    return {"mask": mask, "attn": attn, "total": mask + attn}


# kernels behind each call, for matching the committed HBM counter summary
CALL_KERNELS = {
    # the one-launch form (the workloads measured here fit it: contiguous bf16
    # or fp8 K/V, K_b <= 64, at most 16 splits and one split workgroup per CU)
    ("decode", "hip_decode_step"): ("decode_step_kernel",),
    ("decode", "hip_sparse_attn"): ("attn_decode_mfma", "attn_decode_kernel", "attn_decode_combine"),
    ("decode", "hip_mask_estimate"): ("mask_decode",),
    ("prefill", "hip_sparse_attn"): ("attn_prefill_kernel",),
    ("prefill", "hip_mask_estimate"): ("mask_prefill_kernel",),
}


# string and character literals (kept) or comments (dropped), in source order
_LITERAL_OR_COMMENT = re.compile(r'"(?:\\.|[^"\\])*"|\'(?:\\.|[^\'\\])*\'|//[^\n]*|/\*.*?\*/', re.S)


def code_text(src: str) -> str:
    """The code of a C/C++/HIP source without comments, whitespace runs collapsed."""
    src = _LITERAL_OR_COMMENT.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", src)
    return re.sub(r"\s+", " ", src).strip()


def kernel_source_sha(d: str | None = None) -> str:
    """Hash of the library's sources, comments and layout aside: the measured
    traffic stays valid across comment edits and is dropped on any code change."""
    import hashlib
    d = d or os.path.join(ROOT, "long_context_sparse_mask_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        h.update(f.encode() + b"\0" + code_text(open(os.path.join(d, f)).read()).encode() + b"\0")
    return h.hexdigest()[:16]


def kernel_matches(kernel: str, dtype: str) -> bool:
    """Whether a profiled instantiation (name with template arguments) serves a
    workload of element type `dtype`: kernels that read K/V by their K/V type
    (unsigned char = E5M2 codes, unsigned short = bf16, float), the decode
    combine (which never reads K/V) by its output type."""
    args = kernel.split("<", 1)[1] if "<" in kernel else ""
    if kernel.startswith("attn_decode_combine"):
        return ("float" in args) == (dtype == "f32")
    if "unsigned char" in args:
        return dtype == "bf16_e5m2"
    if "unsigned short" in args:
        return dtype == "bf16"
    return dtype == "f32"


def measured_traffic(kind: str, call: str, dtype: str = "bf16"):
    """HBM bytes per launch from profiles/hbm_traffic.md (FETCH_SIZE + WRITE_SIZE,
    copy-calibrated), or None when the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    try:
        txt = open(path).read()
        blob = json.loads(txt.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if blob.get("source_sha") != kernel_source_sha():
        return None
    names = CALL_KERNELS.get((kind, call, dtype), CALL_KERNELS[(kind, call)])
    hits = [v["traffic_bytes"] for k, v in blob["kernels"].items()
            if k.startswith(names) and kernel_matches(k, dtype)]
    return sum(hits) if hits else None


def _time_oracle(fn, budget_s: float, min_runs: int, max_runs: int) -> list:
    """Wall-clock seconds of repeated fn() calls: at least min_runs, then
    until budget_s is spent (at most max_runs)."""
    times = []
    t_start = time.perf_counter()
    while len(times) < min_runs or (time.perf_counter() - t_start < budget_s
                                    and len(times) < max_runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return times


def cpu_baseline(x, w, budget_s: float) -> dict:
    """The CPU oracle (mask + attention) on one whole decode step of the
    workload (the first query set and layer copy): with every host thread,
    and with one thread."""
    import oracle
    kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal)
    nt = oracle.nthreads()

    def step(threads):
        idx, nnz, _ = oracle.mask_all(x["q"], x["K"], threads=threads, **kw)
        oracle.attn_all(x["q"], x["K"], x["V"], idx, nnz, threads=threads, **kw)
    all_t = _time_oracle(lambda: step(nt), budget_s, 3, 2000)
    one_t = _time_oracle(lambda: step(1), budget_s / 2, 1, 200)
    med, med1 = statistics.median(all_t), statistics.median(one_t)
    return {"value": round(med * 1e6, 1), "unit": "us/step", "cores": nt, "kind": "oracle",
            "sample": f"whole {w.name} step (first query set and layer copy), median of "
                      f"{len(all_t)} runs ({sum(all_t):.1f} s), fp64 C + OpenMP",
            "single_thread": {"value": round(med1 * 1e6, 1), "unit": "us/step", "cores": 1,
                              "sample": f"the same step, median of {len(one_t)} runs "
                                        f"({sum(one_t):.1f} s)"},
            "cpu_model": host_cpu_model()}


def cpu_baseline_prefill(si, budget_s: float) -> dict:
    """The CPU oracle (mask + attention) on the whole 4096-row prefill chunk
    with every host thread; with one thread on its last 256 rows (4 of its 64
    query blocks, each with the same 32 selected blocks per KV head as every
    block of the chunk), the time scaled by 16."""
    import oracle
    full = si.workload("prefill_32k_chunk4k")
    xf = si.make_inputs(full)
    nt = oracle.nthreads()

    def chunk(w, x, threads):
        kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal)
        idx, nnz, _ = oracle.mask_all(x["q"], x["K"], threads=threads, **kw)
        oracle.attn_all(x["q"], x["K"], x["V"], idx, nnz, threads=threads, **kw)
    all_t = _time_oracle(lambda: chunk(full, xf, nt), budget_s, 2, 5)
    part = si.workload("prefill_32k_chunk4k", Tq=256)
    xp = si.make_inputs(part)
    one_t = _time_oracle(lambda: chunk(part, xp, 1), budget_s / 2, 1, 5)
    med = statistics.median(all_t)
    scale = full.Tq / part.Tq
    med1 = statistics.median(one_t) * scale
    return {"value": round(full.Tq / med, 1), "unit": "tok/s", "cores": nt, "kind": "oracle",
            "sample": f"whole 4096-row chunk at T={full.T}, fp64 C + OpenMP, median of "
                      f"{len(all_t)} runs ({sum(all_t):.1f} s)", "s_per_chunk": round(med, 2),
            "single_thread": {"value": round(full.Tq / med1, 1), "unit": "tok/s", "cores": 1,
                              "sample": f"last {part.Tq} rows of the chunk, median of "
                                        f"{len(one_t)} runs, time scaled x{scale:g}",
                              "s_per_chunk": round(med1, 1)}}


def host_cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def graph_of(fn, n, torch):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in range(n):
            fn(j)
    return g


def time_graph(g, reps, torch):
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1)  # ms


def setup(w, x, torch, dev, n_layers=N_LAYER_COPIES, n_q=N_QUERY_SETS):
    """Device copies: n_layers rolled K/V layers and n_q query sets."""
    K0, V0 = x["K"].to(dev), x["V"].to(dev)
    kvdt = K0.dtype
    if K0.element_size() == 1:  # fp8 codes: roll the bytes
        K0, V0 = K0.view(torch.uint8), V0.view(torch.uint8)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    shifts = [0] + [int(s) for s in torch.randint(1, w.T, (n_layers - 1,), generator=gen,
                                                   device=dev).tolist()]
    layers = [(torch.roll(K0, s, dims=2).contiguous().view(kvdt),
               torch.roll(V0, s, dims=2).contiguous().view(kvdt)) for s in shifts]
    del K0, V0
    tdt = x["q"].dtype
    qs = [x["q"].to(dev)]
    for _ in range(n_q - 1):
        qs.append(torch.randn(x["q"].shape, generator=gen, device=dev, dtype=torch.float32).to(tdt))
    return layers, qs, shifts


def page_pool(K, V, T, page_size, gen, torch):
    """K, V [B,Hkv,T_cap,d] as a page pool [B*n, Hkv, page_size, d] (n = T/page_size pages per
    sequence) whose pages are placed in a random order, and the table [B, n] that finds them."""
    B, Hkv, _, d = K.shape
    n = T // page_size
    perm = torch.randperm(B * n, generator=gen, device=K.device)

    def pool(X):
        X = X[:, :, :n * page_size].reshape(B, Hkv, n, page_size, d).permute(0, 2, 1, 3, 4)
        X = X.reshape(B * n, Hkv, page_size, d)
        out = torch.empty_like(X)
        out[perm] = X  # logical page i of the flattened order lands at physical page perm[i]
        return out
    table = perm.view(B, n).to(torch.int32).contiguous()
    return pool(K), pool(V), table


def run_workload(w, steps, warmup, torch, hs, si, n_layers=N_LAYER_COPIES, n_q=N_QUERY_SETS,
                 page_size=0, dense=(0, 0), legs=True, x=None):
    """Times one workload on cuda:0.

    Decode (block_q 1): the timed step is one hip_decode_step call.  With
    `legs`: also the step as two calls (hip_mask_estimate + hip_sparse_attn),
    the mask call alone, the attention call alone on each step's own lists,
    and mask reuse every r_m steps.  Prefill: the step is the two calls; with
    `legs` each call alone as well.  Returns milliseconds per step of each
    and the lists of the eager step on the first query set and layer copy."""
    dev = torch.device("cuda:0")
    x = x if x is not None else si.make_inputs(w)
    layers, qs, shifts = setup(w, x, torch, dev, n_layers, n_q)
    if page_size:  # the same layer copies held in shuffled page pools
        assert w.T % page_size == 0
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed + 1)
        pooled = []
        for K, V in layers:
            if K.element_size() == 1:
                Kp, Vp, tab = page_pool(K.view(torch.uint8), V.view(torch.uint8), w.T, page_size, gen,
                                        torch)
                Kp, Vp = Kp.view(K.dtype), Vp.view(K.dtype)
            else:
                Kp, Vp, tab = page_pool(K, V, w.T, page_size, gen, torch)
            pooled.append((Kp, Vp, tab))
        del layers
        layers = pooled
    decode = w.block_q == 1
    nqb = -(-w.Tq // w.block_q)
    idx = torch.empty((w.B, w.Hkv, nqb, w.kb), dtype=torch.int32, device=dev)
    nnz = torch.empty((w.B, w.Hkv, nqb), dtype=torch.int32, device=dev)
    out = torch.empty_like(qs[0])
    sink, window = dense
    wsb = hs.hipsa_workspace_bytes_ex(qs[0], x["K"], w.k, w.block_k, w.block_q, T=w.T, sink=sink,
                                      window=window)
    if decode:  # the step's workspace (partials, then its zeroed arrival counters) covers both
        wsb = max(wsb, hs.hipsa_decode_step_workspace_bytes(qs[0], x["K"], w.k, w.block_k, T=w.T,
                                                            sink=sink, window=window))
    ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=dev)
    ckw = dict(T=w.T, causal=bool(w.causal), sink=sink, window=window)

    def table(L):
        return L[2] if page_size else None

    def mask(j, idx=idx, nnz=nnz):
        q, L = qs[j % len(qs)], layers[j % len(layers)]
        hs.hip_mask_estimate_ex(q, L[0], w.k, w.block_k, w.block_q, block_table=table(L),
                                indices=idx, nnz=nnz, **ckw)

    def attn(j, idx=idx, nnz=nnz):
        q, L = qs[j % len(qs)], layers[j % len(layers)]
        hs.hip_sparse_attn_ex(q, L[0], L[1], idx, nnz, w.k, w.block_k, w.block_q,
                              block_table=table(L), out=out, workspace=ws, **ckw)

    def fused(j):
        q, L = qs[j % len(qs)], layers[j % len(layers)]
        hs.hip_decode_step(q, L[0], L[1], w.k, w.block_k, block_table=table(L), indices=idx,
                           nnz=nnz, out=out, workspace=ws, **ckw)

    def two_calls(j):
        mask(j)
        attn(j)

    step = fused if decode else two_calls
    # the lists and output of the eager step on the first query set and layer copy
    step(0)
    torch.cuda.synchronize()
    first = {"indices": idx.cpu().numpy(), "nnz": nnz.cpu().numpy(), "out": out.float().cpu()}
    if decode:  # the one-call step equals the two calls bit for bit
        two_calls(0)
        torch.cuda.synchronize()
        assert (idx.cpu().numpy() == first["indices"]).all() and torch.equal(out.float().cpu(),
                                                                              first["out"])
    # eager reference of the last timed step, to check the graph replays against
    step(steps - 1)
    torch.cuda.synchronize()
    eager = (idx.clone(), out.clone())

    g_warm = graph_of(step, max(warmup, 1), torch)
    g_step = graph_of(step, steps, torch)
    if warmup > 0:
        g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_graph(g_step, 1, torch)
    wall = time.perf_counter() - t0
    assert torch.equal(idx, eager[0]) and torch.equal(out, eager[1]), "graph replay differs from eager"
    del g_warm, g_step
    res = {"ms_per_step": ms / steps, "wall_s": wall, "shifts": shifts, "first": first}
    if not legs:
        return res

    def timed(fn, n):
        g = graph_of(fn, n, torch)
        g.replay()  # warm-up replay
        t = time_graph(g, 1, torch) / n
        del g
        return t

    res["ms_mask"] = timed(mask, steps)
    # attention alone, each step over the lists its own mask selected
    lists = []
    for j in range(steps):
        mask(j)
        lists.append((idx.clone(), nnz.clone()))
    torch.cuda.synchronize()
    res["ms_attn"] = timed(lambda j: attn(j, *lists[j]), steps)
    if decode:
        res["ms_two_calls"] = timed(two_calls, steps)
        reuse = {}
        for r_m in (2, 4, 8):
            def step_r(j, r_m=r_m):
                if j % r_m == 0:
                    fused(j)  # new lists, and the attention over them
                else:
                    attn(j)   # the lists of the last refresh
            reuse[r_m] = timed(step_r, steps)
        res["ms_reuse"] = reuse
    del layers, qs, lists
    torch.cuda.empty_cache()
    return res


# Stage lists (tokens) of the multi-stage leg: stage 0 chunks of 8 blocks, a
# middle stage keeping four times the final keys in 2-block chunks, then
# single blocks; the same shape as the PR page's 128 -> 32 -> 8 chunks with
# stage_k falling by 4.
STAGES = {"decode_128k_b4": [(512, None), (128, 8192), (64, 2048)],
          "decode_1m_needles": [(512, None), (128, 16384), (64, 4096)]}


def run_stages(w, stages, steps, warmup, torch, hs, si, n_layers=N_LAYER_COPIES,
               n_q=N_QUERY_SETS, x=None):
    """The multi-stage search (hip_mask_estimate_stages) alone, and followed by
    hip_sparse_attn over its lists, timed like the step; the lists of the
    first query set and layer copy, and their overlap with the one-stage
    search's."""
    dev = torch.device("cuda:0")
    x = x if x is not None else si.make_inputs(w)
    layers, qs, _ = setup(w, x, torch, dev, n_layers, n_q)
    idx = torch.empty((w.B, w.Hkv, w.Tq, w.kb), dtype=torch.int32, device=dev)
    nnz = torch.empty((w.B, w.Hkv, w.Tq), dtype=torch.int32, device=dev)
    out = torch.empty_like(qs[0])
    ws = torch.zeros(max(hs.hipsa_workspace_bytes(qs[0], x["K"], w.k, w.block_k, 1, T=w.T), 1),
                     dtype=torch.uint8, device=dev)

    def mask(j):
        q, L = qs[j % len(qs)], layers[j % len(layers)]
        hs.hip_mask_estimate_stages(q, L[0], stages, w.block_k, T=w.T, indices=idx, nnz=nnz)

    def step(j):
        mask(j)
        q, L = qs[j % len(qs)], layers[j % len(layers)]
        hs.hip_sparse_attn(q, L[0], L[1], idx, nnz, w.k, w.block_k, 1, T=w.T, out=out,
                           workspace=ws)

    mask(0)
    torch.cuda.synchronize()
    first = idx.cpu().numpy()
    one, _ = hs.hip_mask_estimate(qs[0], layers[0][0], w.k, w.block_k, 1, T=w.T)
    one = one.cpu().numpy()
    common = sum(len(set(a.tolist()) & set(b.tolist()))
                 for a, b in zip(first.reshape(-1, w.kb), one.reshape(-1, w.kb)))

    def timed(fn, n):
        g = graph_of(fn, max(warmup, 1), torch)
        g.replay()
        del g
        g = graph_of(fn, n, torch)
        t = time_graph(g, 1, torch) / n
        del g
        return t
    res = {"ms_mask": timed(mask, steps), "ms_step": timed(step, steps), "first": first,
           "shared_with_one_stage": round(common / first.size, 4)}
    del layers, qs
    torch.cuda.empty_cache()
    return res


def stage_candidates(w, stages) -> list:
    """Candidates scored per round by the multi-stage search on a row that
    sees all ceil(T / block_k) blocks, when every chunk of a round has the
    same width (the workloads' sizes divide evenly): stage 0 cuts chunks of
    its size; each later stage halves the chunks wider than its size, at
    least once per stage and until they fit, keeping k / chunk_size."""
    Np = -(-w.T // w.block_k)
    c0 = stages[0][0] // w.block_k
    nk, width = -(-Np // c0), c0
    counts = []
    for chunk, k in stages[1:]:
        tb, keep = chunk // w.block_k, k // chunk
        fresh = True
        while fresh or width > tb:
            fresh = False
            halve = width > tb
            n = nk * (2 if halve else 1)
            counts.append(n)
            width = width - width // 2 if halve else width  # the larger half
            nk = min(keep, n)
    return counts


def stage_mask_bytes(w, stages) -> int:
    """Algorithmic HBM bytes of one multi-stage search over every problem:
    the centre rows of every round's candidates, the query rows, the lists."""
    qsz, kvsz = ELEM_BYTES[w.dtype]
    P = w.B * w.Hkv * w.Tq
    return P * (sum(stage_candidates(w, stages)) * w.d * kvsz + w.G * w.d * qsz + 4 * (w.kb + 1))


def stages_line(w, stages, r) -> dict:
    nb = decode_bytes(w)
    mb = stage_mask_bytes(w, stages)
    d = {"workload": w.name, "stages": [[c, k] for c, k in stages],
         "candidates_per_round": stage_candidates(w, stages),
         "mask_us": round(r["ms_mask"] * 1e3, 3), "step_us": round(r["ms_step"] * 1e3, 3),
         "mask_bytes": mb, "mask_frac": round(mb / (r["ms_mask"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
         "step_frac": round((mb + nb["attn"]) / (r["ms_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
         "blocks_shared_with_one_stage": r["shared_with_one_stage"]}
    if "cpu_baseline" in r:
        d["cpu_baseline"] = r["cpu_baseline"]
    return d


def cpu_baseline_stages(x, w, stages, budget_s: float) -> dict:
    """The CPU oracle's multi-stage search plus the attention over its lists on
    one whole decode step of the workload (first query set and layer copy),
    with every host thread."""
    import oracle
    nt = oracle.nthreads()
    kw = dict(T=w.T, block_k=w.block_k, causal=w.causal)

    def step():
        idx, nnz, _ = oracle.mask_stages_all(x["q"], x["K"], stages, threads=nt, **kw)
        oracle.attn_all(x["q"], x["K"], x["V"], idx, nnz, k=w.k, block_q=1, threads=nt, **kw)
    t = _time_oracle(step, budget_s, 2, 500)
    return {"value": round(statistics.median(t) * 1e6, 1), "unit": "us/step", "cores": nt,
            "kind": "oracle", "sample": f"whole {w.name} step with the stage list, median of "
                                        f"{len(t)} runs ({sum(t):.1f} s), fp64 C + OpenMP"}


def needle_recall(x, indices):
    """Needle recall of the GPU's lists (`indices`) on the first query set and
    layer copy (no roll, so the needles sit where drawn)."""
    return {"gpu": needle_share(x, indices), "needles": len(x["needles"])}


def needle_share(x, lists):
    """Share of (problem, needle block) pairs with the needle block in the
    problem's list (query row 0)."""
    import numpy as np
    needles = np.array(x["needles"])
    B, Hkv = lists.shape[:2]
    hits = [np.isin(needles, lists[b, g, 0]).sum() for b in range(B) for g in range(Hkv)]
    return round(float(sum(hits)) / (len(hits) * len(needles)), 4)


def decode_line(w, r) -> dict:
    """Figures of one decode workload: µs per step and the step's roofline."""
    nb = decode_bytes(w)
    us = r["ms_per_step"] * 1e3
    gbs = nb["step"] / (r["ms_per_step"] * 1e-3) / 1e9
    d = {"workload": w.name, "us_per_step": round(us, 3), "algorithmic_bytes": nb["step"],
         "achieved_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4), "rounds": nb["rounds"]}
    for key, name in (("ms_two_calls", "two_calls_us"), ("ms_mask", "mask_us"),
                      ("ms_attn", "attn_us")):
        if key in r:
            d[name] = round(r[key] * 1e3, 3)
    return d


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_128k_b4")
    ap.add_argument("--kv", choices=["native", "e5m2"], default="native",
                    help="e5m2: run the workload with an fp8 (E5M2) KV cache")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 KV cache leg")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged KV cache leg")
    ap.add_argument("--page-size", type=int, default=64, help="tokens per page of the paged leg")
    ap.add_argument("--no-dense", action="store_true", help="skip the sink + window leg")
    ap.add_argument("--sink", type=int, default=64, help="sink tokens of the dense-part leg")
    ap.add_argument("--window", type=int, default=4096, help="window tokens of the dense-part leg")
    ap.add_argument("--no-other-decodes", action="store_true",
                    help="skip the 32k and 1M-token decode legs")
    ap.add_argument("--no-stages", action="store_true", help="skip the multi-stage search leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--only-step", action="store_true",
                    help="time the headline step only (no legs): for kernel profiles of the step")
    ap.add_argument("--cpu-budget", type=float, default=8.0)
    ap.add_argument("--layer-copies", type=int, default=N_LAYER_COPIES,
                    help="rolled K/V copies rotated over the steps (1 = one layer, cache-warm)")
    ap.add_argument("--query-sets", type=int, default=N_QUERY_SETS,
                    help="query sets rotated over the steps (1 = same selection every step)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: the library runs on exactly one GPU (no multi-GPU path); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.only_step:
        args.no_fp8 = args.no_paged = args.no_dense = args.no_other_decodes = args.no_stages = True
        args.no_prefill = args.no_cpu_baseline = True

    import torch
    import long_context_sparse_mask_amd as hs
    import synth_inputs as si

    w = si.workload(args.workload)
    if args.kv == "e5m2":
        w = si.workload(args.workload, dtype="bf16_e5m2")
    is_decode = w.block_q == 1
    x = si.make_inputs(w)
    r = run_workload(w, args.steps, args.warmup, torch, hs, si, args.layer_copies,
                     args.query_sets, legs=not args.only_step, x=x)
    us = r["ms_per_step"] * 1e3
    line = {"metric": "decode attn us/step/layer at 128k (mask+sparse) & % HBM peak; prefill tok/s",
            "value": round(us, 3) if is_decode else None, "unit": "us/step",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": r["ms_per_step"], "higher_is_better": False, "scaling": "weak",
            "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded AR(1) keys, N(0,1) q/V)",
            "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "T": w.T,
                       "Tq": w.Tq, "block_k": w.block_k, "block_q": w.block_q, "k": w.k,
                       "seed": w.seed, "layer_copies": args.layer_copies,
                       "query_sets": args.query_sets}}
    if is_decode:
        nb = decode_bytes(w)

        def hbm_roof(call, t_ms, byt, kernels):
            ach = byt / (t_ms * 1e-3) / 1e9
            return {"bound": "hbm", "kernel": call, "launches": kernels, "achieved": round(ach, 1),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic("decode", call, w.dtype), "algorithmic_bytes": byt,
                    "launch_us": round(t_ms * 1e3, 3)}
        # the step is one call: its kernels (the one-launch search + attention, then the
        # merge of the splits) carry every byte of the step
        line["roofline"] = hbm_roof("hip_decode_step", r["ms_per_step"], nb["step"],
                                    list(CALL_KERNELS.get(("decode", "hip_decode_step", w.dtype),
                                                          CALL_KERNELS[("decode", "hip_decode_step")])))
        if "ms_attn" in r:
            line["roofline_other"] = {
                "hip_sparse_attn": hbm_roof("hip_sparse_attn", r["ms_attn"], nb["attn"],
                                            list(CALL_KERNELS[("decode", "hip_sparse_attn")])),
                "hip_mask_estimate": hbm_roof("hip_mask_estimate", r["ms_mask"], nb["mask"],
                                              list(CALL_KERNELS[("decode", "hip_mask_estimate")]))}
            line["mask_reuse"] = {"r_m": [1] + sorted(r["ms_reuse"]),
                                  "us_per_step": [round(us, 3)] + [round(r["ms_reuse"][k] * 1e3, 3)
                                                                   for k in sorted(r["ms_reuse"])],
                                  "attention_only_us": round(r["ms_attn"] * 1e3, 3)}
        line["step_roofline"] = decode_line(w, r)
    else:
        fl = prefill_flops(w)
        tflops = fl["total"] / (r["ms_per_step"] * 1e-3) / 1e12
        line["value"] = round(w.B * w.Tq / (r["ms_per_step"] * 1e-3), 1)
        line["unit"] = "tok/s"
        line["higher_is_better"] = True
        if "ms_attn" in r:
            kern = {"hip_mask_estimate": (r["ms_mask"], fl["mask"]),
                    "hip_sparse_attn": (r["ms_attn"], fl["attn"])}

            def mfma_roof(k):
                t_ms, f = kern[k]
                ach = f / (t_ms * 1e-3) / 1e12
                return {"bound": "mfma", "kernel": k, "achieved": round(ach, 2),
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": measured_traffic("prefill", k, w.dtype),
                        "algorithmic_flops": f, "launch_us": round(t_ms * 1e3, 3)}
            line["roofline"] = mfma_roof("hip_sparse_attn")
            line["roofline_other"] = mfma_roof("hip_mask_estimate")
        line["step_roofline"] = {"algorithmic_flops": fl["total"], "achieved_tflops": round(tflops, 2),
                                 "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = (cpu_baseline(x, w, args.cpu_budget) if is_decode
                                else cpu_baseline_prefill(si, args.cpu_budget))
    del x
    headline = is_decode and args.workload == "decode_128k_b4" and args.kv == "native"
    small = dict(steps=max(10, args.steps // 2), warmup=max(2, args.warmup // 2))
    if headline and not args.no_other_decodes:
        w1 = si.workload("decode_32k")
        r1 = run_workload(w1, small["steps"], small["warmup"], torch, hs, si, args.layer_copies,
                          args.query_sets)
        line["decode_32k"] = decode_line(w1, r1)
        w4 = si.workload("decode_1m_needles")
        x4 = si.make_inputs(w4)
        r4 = run_workload(w4, small["steps"], small["warmup"], torch, hs, si, 4, args.query_sets,
                          x=x4)
        line["decode_1m_needles"] = decode_line(w4, r4)
        line["decode_1m_needles"]["needle_recall"] = needle_recall(x4, r4["first"]["indices"])
        if not args.no_stages:
            st4 = STAGES[w4.name]
            rs4 = run_stages(w4, st4, small["steps"], small["warmup"], torch, hs, si, 4,
                             args.query_sets, x=x4)
            line.setdefault("multi_stage", {})[w4.name] = dict(
                stages_line(w4, st4, rs4), needle_recall_gpu=needle_share(x4, rs4["first"]))
        del x4
    if headline and not args.no_stages:
        # the multi-stage search on the headline shape, then attention over its lists
        st = STAGES[w.name]
        rs = run_stages(w, st, args.steps, args.warmup, torch, hs, si, args.layer_copies,
                        args.query_sets)
        if not args.no_cpu_baseline:
            xs = si.make_inputs(w)
            rs["cpu_baseline"] = cpu_baseline_stages(xs, w, st, args.cpu_budget / 2)
            del xs
        line.setdefault("multi_stage", {})[w.name] = stages_line(w, st, rs)
    if headline and not args.no_fp8:
        # the same step with an fp8 (E5M2) KV cache: half the K/V bytes
        w8 = si.workload(args.workload, dtype="bf16_e5m2")
        r8 = run_workload(w8, args.steps, args.warmup, torch, hs, si, args.layer_copies,
                          args.query_sets)
        nb8 = decode_bytes(w8)
        a_gbs = nb8["attn"] / (r8["ms_attn"] * 1e-3) / 1e9
        line["fp8_kv"] = decode_line(w8, r8)
        line["fp8_kv"]["attn_roofline"] = {
            "algorithmic_bytes": nb8["attn"], "achieved": round(a_gbs, 1),
            "frac": round(a_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode", "hip_sparse_attn", w8.dtype)}
        line["fp8_kv"]["mask_reuse_us"] = {str(k): round(v * 1e3, 3)
                                           for k, v in sorted(r8["ms_reuse"].items())}
    if headline and not args.no_paged:
        # the same step with K/V in a page pool: pages of page_size tokens in a random order
        rpg = run_workload(w, small["steps"], small["warmup"], torch, hs, si, args.layer_copies,
                           args.query_sets, page_size=args.page_size)
        line["paged_kv"] = dict(decode_line(w, rpg), page_size=args.page_size,
                                pages="shuffled over the pool")
    if headline and not args.no_dense:
        # the same step with a dense part: sink and sliding-window blocks beside the search
        rd = run_workload(w, small["steps"], small["warmup"], torch, hs, si, args.layer_copies,
                          args.query_sets, dense=(args.sink, args.window))
        line["dense_part"] = dict(decode_line(w, rd), sink=args.sink, window=args.window,
                                  keys_per_row=args.sink + args.window + w.k)
    if headline and not args.no_prefill:
        wp = si.workload("prefill_32k_chunk4k")
        # 40 chunks per timed graph at the default 200 steps: replays of short graphs
        # measured slower per call (10 attention calls: 190-200 us each; 30 or more,
        # eager calls and kernel traces: 155-163 us)
        psteps, pwarm = max(8, args.steps // 5), max(2, args.warmup // 5)
        rp = run_workload(wp, psteps, pwarm, torch, hs, si, 4)
        fl = prefill_flops(wp)
        line["prefill"] = {"workload": wp.name,
                           "tok_per_s": round(wp.Tq / (rp["ms_per_step"] * 1e-3), 1),
                           "ms_per_chunk": round(rp["ms_per_step"], 4),
                           "mask_us": round(rp["ms_mask"] * 1e3, 2),
                           "attn_us": round(rp["ms_attn"] * 1e3, 2),
                           "mfma_frac": round(fl["total"] / (rp["ms_per_step"] * 1e-3) / 1e12
                                              / MFMA_BF16_PEAK_TFLOPS, 4),
                           "attn_mfma_frac": round(fl["attn"] / (rp["ms_attn"] * 1e-3) / 1e12
                                                   / MFMA_BF16_PEAK_TFLOPS, 4),
                           "algorithmic_flops": fl["total"]}
        if not args.no_fp8:
            wp8 = si.workload("prefill_32k_chunk4k", dtype="bf16_e5m2")
            rp8 = run_workload(wp8, psteps, pwarm, torch, hs, si, 4)
            line["prefill"]["fp8_kv"] = {"tok_per_s": round(wp8.Tq / (rp8["ms_per_step"] * 1e-3), 1),
                                         "mask_us": round(rp8["ms_mask"] * 1e3, 2),
                                         "attn_us": round(rp8["ms_attn"] * 1e3, 2)}
        if not args.no_cpu_baseline:
            line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(si, args.cpu_budget)
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = 1 << 30
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
