#!/usr/bin/env python3
"""Benchmark of the HiP hot path on one MI355X: mask estimation + block-sparse
attention per step, on seeded synthetic Llama-3.1-8B-shaped inputs.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Prints ONE JSON line.  Default workload: decode at 128k context, batch 4,
32 query / 8 KV heads, d=128, bf16, block_k=64, k=2048 (decode_128k_b4).
A step = hip_mask_estimate + hip_sparse_attn for the whole batch; the value
is microseconds per step (lower is better).  With the default workload the
line also carries the chunked-prefill throughput (4096-token chunk at the end
of a 32k sequence) as `prefill`.

Timing: the K timed steps (and the W warm-up steps) are captured as HIP
graphs of C-ABI launches on torch's capture stream and replayed, so host
call overhead is not in the figure.  Consecutive steps rotate over 4 rolled
copies of the layer's K/V and 16 query sets, so selected blocks differ from
step to step and the selected bytes come from HBM, not from the 256 MB
last-level cache.  Per-kernel launch durations for the roofline are taken the
same way from graphs of one kernel each, with HIP events on the stream that
the kernels run on.  Decode lines also carry `mask_reuse`: µs per step when
the mask is re-estimated only every r_m steps (attention every step).
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
N_LAYER_COPIES = 4   # defaults; --layer-copies / --query-sets override
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
    names = CALL_KERNELS[(kind, call)]
    hits = [v["traffic_bytes"] for k, v in blob["kernels"].items()
            if k.startswith(names) and kernel_matches(k, dtype)]
    return sum(hits) if hits else None


def cpu_baseline(x, w, budget_s: float) -> dict:
    """The CPU oracle on the same seeded step, all host threads."""
    import oracle
    kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal)
    nt = oracle.nthreads()
    times = []
    t_start = time.perf_counter()
    # whole steps, repeated until about budget_s of CPU time is spent (at least 3)
    while len(times) < 3 or (time.perf_counter() - t_start < budget_s and len(times) < 2000):
        t0 = time.perf_counter()
        idx, nnz, _ = oracle.mask_all(x["q"], x["K"], threads=nt, **kw)
        oracle.attn_all(x["q"], x["K"], x["V"], idx, nnz, threads=nt, **kw)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > 4 * budget_s:
            break
    return times, nt


def cpu_baseline_prefill(si, budget_s: float) -> dict:
    """The CPU oracle on a bounded sample of the prefill chunk: the last 1024
    query rows (16 of the 64 query blocks, each seeing 32 selected blocks like
    every block of the chunk) at the same T, same shapes and distributions,
    repeated until about budget_s of CPU time is spent; the time is scaled to
    the 4096-row chunk."""
    import oracle
    ws = si.workload("prefill_32k_chunk4k", Tq=1024)
    xs = si.make_inputs(ws)
    kw = dict(T=ws.T, k=ws.k, block_k=ws.block_k, block_q=ws.block_q, causal=ws.causal)
    nt = oracle.nthreads()
    times = []
    t_start = time.perf_counter()
    while len(times) < 1 or (time.perf_counter() - t_start < budget_s and len(times) < 50):
        t0 = time.perf_counter()
        idx, nnz, _ = oracle.mask_all(xs["q"], xs["K"], threads=nt, **kw)
        oracle.attn_all(xs["q"], xs["K"], xs["V"], idx, nnz, threads=nt, **kw)
        times.append(time.perf_counter() - t0)
    full = si.workload("prefill_32k_chunk4k")
    scale = full.Tq / ws.Tq
    t = statistics.median(times) * scale
    return {"value": round(full.Tq / t, 1), "unit": "tok/s", "cores": nt, "kind": "oracle",
            "sample": f"last {ws.Tq} query rows of the 4096-row chunk at T={ws.T} "
                      f"({ws.Tq // ws.block_q} of 64 query blocks, 32 heads), fp64 C + OpenMP, "
                      f"median of {len(times)} runs ({sum(times):.1f} s in all), time scaled x{scale:g}",
            "s_per_chunk": round(t, 2)}


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


def run_workload(w, steps, warmup, torch, hs, si, with_cpu, cpu_budget,
                 n_layers=N_LAYER_COPIES, n_q=N_QUERY_SETS, page_size=0, dense=(0, 0)):
    dev = torch.device("cuda:0")
    x = si.make_inputs(w)
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
    nqb = -(-w.Tq // w.block_q)
    idx = torch.empty((w.B, w.Hkv, nqb, w.kb), dtype=torch.int32, device=dev)
    nnz = torch.empty((w.B, w.Hkv, nqb), dtype=torch.int32, device=dev)
    out = torch.empty_like(qs[0])
    sink, window = dense
    wsb = hs.hipsa_workspace_bytes_ex(qs[0], x["K"], w.k, w.block_k, w.block_q, T=w.T, sink=sink,
                                      window=window)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    kw = dict(T=w.T, causal=bool(w.causal))

    def mask(j):
        q, L = qs[j % len(qs)], layers[j % len(layers)]
        if sink or window:
            hs.hip_mask_estimate_ex(q, L[0], w.k, w.block_k, w.block_q, T=w.T, causal=bool(w.causal),
                                    sink=sink, window=window, indices=idx, nnz=nnz)
        elif page_size:
            hs.hip_mask_estimate_paged(q, L[0], L[2], w.T, w.k, w.block_k, w.block_q, indices=idx,
                                       nnz=nnz, causal=bool(w.causal))
        else:
            hs.hip_mask_estimate(q, L[0], w.k, w.block_k, w.block_q, indices=idx, nnz=nnz, **kw)

    def attn(j):
        q, L = qs[j % len(qs)], layers[j % len(layers)]
        if sink or window:
            hs.hip_sparse_attn_ex(q, L[0], L[1], idx, nnz, w.k, w.block_k, w.block_q, T=w.T,
                                  causal=bool(w.causal), sink=sink, window=window, out=out,
                                  workspace=ws)
        elif page_size:
            hs.hip_sparse_attn_paged(q, L[0], L[1], L[2], idx, nnz, w.T, w.k, w.block_k, w.block_q,
                                     causal=bool(w.causal), out=out, workspace=ws)
        else:
            hs.hip_sparse_attn(q, L[0], L[1], idx, nnz, w.k, w.block_k, w.block_q, out=out,
                               workspace=ws, **kw)

    def step(j):
        mask(j)
        attn(j)

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

    # per-kernel launch durations (graphs of one kernel kind)
    g_mask = graph_of(mask, steps, torch)
    g_attn = graph_of(attn, steps, torch)
    g_mask.replay(); g_attn.replay()
    ms_mask = time_graph(g_mask, 1, torch) / steps
    ms_attn = time_graph(g_attn, 1, torch) / steps

    res = {"ms_per_step": ms / steps, "wall_s": wall, "ms_mask": ms_mask, "ms_attn": ms_attn,
           "shifts": shifts}
    if w.block_q == 1:
        # mask reuse: the mask estimated every r_m steps, attention every step
        reuse = {}
        for r_m in (2, 4, 8):
            def step_r(j, r_m=r_m):
                if j % r_m == 0:
                    mask(j)
                attn(j)
            g_r = graph_of(step_r, steps, torch)
            g_r.replay()
            reuse[r_m] = time_graph(g_r, 1, torch) / steps
            del g_r
        res["ms_reuse"] = reuse
    if with_cpu:
        times, nt = cpu_baseline(x, w, cpu_budget)
        res["cpu"] = {"times": times, "threads": nt}
    del layers, qs
    torch.cuda.empty_cache()
    return res


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
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
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

    import torch
    import long_context_sparse_mask_amd as hs
    import synth_inputs as si

    w = si.workload(args.workload)
    if args.kv == "e5m2":
        w = si.workload(args.workload, dtype="bf16_e5m2")
    is_decode = w.block_q == 1
    r = run_workload(w, args.steps, args.warmup, torch, hs, si, not args.no_cpu_baseline,
                     args.cpu_budget, args.layer_copies, args.query_sets)
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
        kern = {"hip_mask_estimate": (r["ms_mask"], nb["mask"]),
                "hip_sparse_attn": (r["ms_attn"], nb["attn"])}
        def hbm_roof(k):
            t_ms, byt = kern[k]
            ach = byt / (t_ms * 1e-3) / 1e9
            return {"bound": "hbm", "kernel": k, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic("decode", k, w.dtype), "algorithmic_bytes": byt,
                    "launch_us": round(t_ms * 1e3, 3)}
        dom = max(kern, key=lambda k: kern[k][0])  # the longer launch
        line["roofline"] = hbm_roof(dom)
        line["roofline_other"] = hbm_roof(min(kern, key=lambda k: kern[k][0]))
        line["mask_reuse"] = {"r_m": [1] + sorted(r["ms_reuse"]),
                              "us_per_step": [round(us, 3)] + [round(r["ms_reuse"][k] * 1e3, 3)
                                                               for k in sorted(r["ms_reuse"])],
                              "attention_only_us": round(r["ms_attn"] * 1e3, 3)}
        step_gbs = nb["step"] / (r["ms_per_step"] * 1e-3) / 1e9
        line["step_roofline"] = {"algorithmic_bytes": nb["step"], "achieved": round(step_gbs, 1),
                                 "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                                 "mask_us": round(r["ms_mask"] * 1e3, 3),
                                 "attn_us": round(r["ms_attn"] * 1e3, 3), "rounds": nb["rounds"]}
    else:
        fl = prefill_flops(w)
        tflops = fl["total"] / (r["ms_per_step"] * 1e-3) / 1e12
        line["value"] = round(w.B * w.Tq / (r["ms_per_step"] * 1e-3), 1)
        line["unit"] = "tok/s"
        line["higher_is_better"] = True
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
        dom = max(kern, key=lambda k: kern[k][0])  # the longer launch
        line["roofline"] = mfma_roof(dom)
        line["roofline_other"] = mfma_roof(min(kern, key=lambda k: kern[k][0]))
        line["step_roofline"] = {"algorithmic_flops": fl["total"], "achieved_tflops": round(tflops, 2),
                                 "mask_us": round(r["ms_mask"] * 1e3, 3),
                                 "attn_us": round(r["ms_attn"] * 1e3, 3)}
    if "cpu" in r:
        med = statistics.median(r["cpu"]["times"])
        if is_decode:
            cv, cu = med * 1e6, "us/step"
        else:
            cv, cu = w.B * w.Tq / med, "tok/s"
        line["cpu_baseline"] = {"value": round(cv, 1), "unit": cu, "cores": r["cpu"]["threads"],
                                "kind": "oracle",
                                "sample": f"whole {w.name} step on the first query set and layer copy, "
                                          f"median of {len(r['cpu']['times'])} runs "
                                          f"({sum(r['cpu']['times']):.1f} s in all), fp64 C + OpenMP",
                                "cpu_model": host_cpu_model()}
    headline = is_decode and args.workload == "decode_128k_b4" and args.kv == "native"
    if headline and not args.no_fp8:
        # the same step with an fp8 (E5M2) KV cache: half the K/V bytes
        w8 = si.workload(args.workload, dtype="bf16_e5m2")
        r8 = run_workload(w8, args.steps, args.warmup, torch, hs, si, False, 0,
                          args.layer_copies, args.query_sets)
        nb8 = decode_bytes(w8)
        a_gbs = nb8["attn"] / (r8["ms_attn"] * 1e-3) / 1e9
        s_gbs = nb8["step"] / (r8["ms_per_step"] * 1e-3) / 1e9
        line["fp8_kv"] = {"workload": w8.name, "dtype": w8.dtype,
                          "us_per_step": round(r8["ms_per_step"] * 1e3, 3),
                          "mask_us": round(r8["ms_mask"] * 1e3, 3),
                          "attn_us": round(r8["ms_attn"] * 1e3, 3),
                          "attn_roofline": {"algorithmic_bytes": nb8["attn"], "achieved": round(a_gbs, 1),
                                            "frac": round(a_gbs / HBM_PEAK_GBS, 4),
                                            "traffic": measured_traffic("decode", "hip_sparse_attn",
                                                                        w8.dtype)},
                          "step_roofline": {"algorithmic_bytes": nb8["step"], "achieved": round(s_gbs, 1),
                                            "frac": round(s_gbs / HBM_PEAK_GBS, 4)},
                          "mask_reuse_us": {str(k): round(v * 1e3, 3)
                                            for k, v in sorted(r8["ms_reuse"].items())}}
    if headline and not args.no_paged:
        # the same step with K/V in a page pool: pages of page_size tokens in a random order
        rpg = run_workload(w, args.steps, args.warmup, torch, hs, si, False, 0,
                           args.layer_copies, args.query_sets, page_size=args.page_size)
        line["paged_kv"] = {"page_size": args.page_size, "pages": "shuffled over the pool",
                            "us_per_step": round(rpg["ms_per_step"] * 1e3, 3),
                            "mask_us": round(rpg["ms_mask"] * 1e3, 3),
                            "attn_us": round(rpg["ms_attn"] * 1e3, 3)}
    if headline and not args.no_dense:
        # the same step with a dense part: sink and sliding-window blocks beside the search
        rd = run_workload(w, args.steps, args.warmup, torch, hs, si, False, 0, args.layer_copies,
                          args.query_sets, dense=(args.sink, args.window))
        line["dense_part"] = {"sink": args.sink, "window": args.window,
                              "keys_per_row": args.sink + args.window + w.k,
                              "us_per_step": round(rd["ms_per_step"] * 1e3, 3),
                              "mask_us": round(rd["ms_mask"] * 1e3, 3),
                              "attn_us": round(rd["ms_attn"] * 1e3, 3)}
    if headline and not args.no_prefill:
        wp = si.workload("prefill_32k_chunk4k")
        rp = run_workload(wp, max(4, args.steps // 20), max(1, args.warmup // 10), torch, hs, si,
                          False, 0)
        fl = prefill_flops(wp)
        line["prefill"] = {"workload": wp.name,
                           "tok_per_s": round(wp.Tq / (rp["ms_per_step"] * 1e-3), 1),
                           "ms_per_chunk": round(rp["ms_per_step"], 4),
                           "mask_us": round(rp["ms_mask"] * 1e3, 2),
                           "attn_us": round(rp["ms_attn"] * 1e3, 2),
                           "mfma_frac": round(fl["total"] / (rp["ms_per_step"] * 1e-3) / 1e12
                                              / MFMA_BF16_PEAK_TFLOPS, 4),
                           "algorithmic_flops": fl["total"]}
        if not args.no_fp8:
            wp8 = si.workload("prefill_32k_chunk4k", dtype="bf16_e5m2")
            rp8 = run_workload(wp8, max(4, args.steps // 20), max(1, args.warmup // 10), torch, hs,
                               si, False, 0)
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
