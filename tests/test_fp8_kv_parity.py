"""GPU parity of the fp8 KV cache path (bf16 queries, K and V as OCP E5M2
codes; dtype HIPSA_BF16_E5M2) against the CPU oracle, which decodes every
code exactly in fp64.

The GPU widens each code exactly to bf16 (every E5M2 value is a bf16 value),
so the comparison bar is the bf16 one: index sets exact where the oracle's
cut margin is at least 1e-4, outputs within 2e-2 absolute; a row that
attends to one key must reproduce that key's value row bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from parity_util import full_parity, run_gpu

pytestmark = pytest.mark.gpu

# every finite E5M2 code (exponent field 31 holds the infinities and NaNs)
FINITE_CODES = np.array([c for c in range(256) if (c >> 2) & 31 != 31], np.uint8)


def _report(name, r):
    print(f"[parity] {name}: problems={r['problems']} exempt={r['exempt']} "
          f"max_err={r['max_err']:.3e}", flush=True)


def _fp8(name, **kw):
    return si.workload(name, dtype="bf16_e5m2", **kw)


def _check(name, w, x=None):
    print(f"[case] {name} {w}", flush=True)
    r = full_parity(x if x is not None else si.make_inputs(w), w)
    _report(name, r)


# ------------------------------------------------------------------ decode

@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode_32k", "decode_128k_b4"])
def test_decode_workload_full(name):
    _check(name + "_e5m2", _fp8(name))


DECODE_EDGE = {
    # d = 64: V rows of 2 codes per lane
    "d64_bk16_g2": dict(Hq=4, Hkv=2, d=64, T=5000, block_k=16, k=256),
    # K_b = 512: eight candidate tiles per wave and round
    "bk8_kb512": dict(Hq=8, Hkv=2, T=20000, block_k=8, k=4096),
    "bk32_kb7": dict(Hq=4, Hkv=1, T=9000, block_k=32, k=224),
    "dense_k_ge_T": dict(Hq=4, Hkv=2, T=500, block_k=32, k=512),
    "multi_row_causal": dict(Hq=8, Hkv=2, Tq=5, T=3000, k=512),
    "group1": dict(Hq=4, Hkv=4, T=4096, k=1024),
    "group8": dict(Hq=16, Hkv=2, T=4096, k=1024),
    "group16": dict(Hq=16, Hkv=1, T=4096, k=1024),
    "batch3_ragged": dict(B=3, Hq=8, Hkv=2, T=6001, k=1024),
}


@pytest.mark.parametrize("case", sorted(DECODE_EDGE))
def test_decode_edge(case):
    _check(case, _fp8("decode_32k", **DECODE_EDGE[case]))


def test_decode_spare_capacity_rows():
    w = _fp8("decode_32k", Hq=8, Hkv=2, T=3000, k=512)
    x = dict(si.make_inputs(w, T_cap=3333))
    big = torch.tensor(1e4).to(torch.float8_e5m2)  # finite, far above any real key
    x["K"][:, :, w.T:] = big
    x["V"][:, :, w.T:] = big
    _check("spare_capacity_e5m2", w, x)


def _codes_tensor(shape, gen):
    """Every finite code at least once (in order), then random finite codes."""
    n = int(np.prod(shape))
    fill = gen.choice(FINITE_CODES, size=n)
    fill[:len(FINITE_CODES)] = FINITE_CODES
    return torch.from_numpy(fill.reshape(shape)).view(torch.float8_e5m2)


@pytest.mark.parametrize("d", [64, 128])
def test_every_code_decodes_exactly(d):
    """A decode row that sees a single key returns that key's V row exactly:
    its softmax weight is 1, so the output is the decoded code rounded to
    bf16, which is the decoded code itself.  V row 0 holds every finite code."""
    w = _fp8("decode_32k", B=1, Hq=4, Hkv=4, d=d, T=1, k=64)
    x = dict(si.make_inputs(w))
    x["V"] = _codes_tensor(tuple(x["V"].shape), np.random.default_rng(5))
    idx, nnz, out = run_gpu(x, w)
    kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=1, causal=1)
    ref = oracle.attn_all(x["q"], x["K"], x["V"], idx, nnz, **kw)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref)
    vals = oracle.e5m2_values()
    assert set(np.unique(ref)) == set(vals[FINITE_CODES])  # all 248 values came through


def test_keys_over_every_finite_code():
    """K drawn over all finite codes (2^-16 .. 57344, both signs, subnormals
    included) with a query scaled by 2^-14, so the logits stay moderate and
    every code matters to the ranking and the softmax."""
    w = _fp8("decode_32k", B=2, Hq=8, Hkv=2, T=4096, k=512)
    x = dict(si.make_inputs(w))
    x["K"] = _codes_tensor(tuple(x["K"].shape), np.random.default_rng(6))
    x["q"] = (x["q"].float() * 2.0 ** -14).to(torch.bfloat16)
    _check("keys_all_codes", w, x)


# ------------------------------------------------------------------ prefill

PREFILL = {
    "ragged_causal": dict(T=3000, Tq=200, Hq=8, Hkv=2, k=512),
    "dense_early_blocks": dict(T=1100, Tq=1000, Hq=4, Hkv=1, k=512),
    "bk16": dict(T=4096, Tq=128, Hq=4, Hkv=1, block_k=16, k=256),
    "d64": dict(T=4096, Tq=128, Hq=8, Hkv=2, d=64, k=512),
    "group8": dict(T=4096, Tq=128, Hq=8, Hkv=1, k=512),
    "group16": dict(T=4096, Tq=64, Hq=16, Hkv=1, k=512),
    "noncausal": dict(T=4096, Tq=130, Hq=4, Hkv=1, k=512, causal=0),
    "kb_odd": dict(T=4096, Tq=128, Hq=4, Hkv=1, k=7 * 64),
}


@pytest.mark.parametrize("case", sorted(PREFILL))
def test_prefill_small(case):
    _check("prefill_" + case, _fp8("prefill_32k_chunk4k", **PREFILL[case]))


def test_prefill_every_code_first_row():
    """Chunk = whole sequence: query row 0 sees key 0 alone, so its output is
    V row 0 exactly; V row 0 of the four KV heads holds every finite code.
    The other rows mix that row (values up to 57344) with ordinary ones.  The
    matrix cores take the probabilities in bf16 (8 significant bits: relative
    error up to 2^-8) and the output is rounded to bf16 (2^-8 again), so those
    rows are held to 2e-2 + 1.01 * 2^-7 * A per element, A = sum_t p_t |V_t|
    (the oracle's attention over |V|, exact since attention is linear in V);
    a wrongly decoded code would be off by a multiple of A."""
    w = _fp8("prefill_32k_chunk4k", T=128, Tq=128, Hq=4, Hkv=4, k=512)
    x = dict(si.make_inputs(w))
    V = x["V"].view(torch.uint8).clone()
    V[:, :, 0] = _codes_tensor(tuple(V[:, :, 0].shape), np.random.default_rng(7)).view(torch.uint8)
    x["V"] = V.view(torch.float8_e5m2)
    idx, nnz, out = run_gpu(x, w)
    kw = dict(T=w.T, k=w.k, block_k=w.block_k, block_q=w.block_q, causal=w.causal)
    ref = oracle.attn_all(x["q"], x["K"], x["V"], idx, nnz, **kw)
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got[:, :, 0], ref[:, :, 0])
    Vabs = (x["V"].view(torch.uint8) & 0x7F).view(torch.float8_e5m2)  # sign bit cleared
    A = oracle.attn_all(x["q"], x["K"], Vabs, idx, nnz, **kw)
    excess = np.abs(got - ref) - (2e-2 + 1.01 * 2.0 ** -7 * A)
    assert (excess <= 0).all(), float(excess.max())


@pytest.mark.timeout(900)
def test_prefill_full_size_chunk():
    """The 4096-token chunk at the end of a 32k sequence with an fp8 KV cache:
    every index list and every output row against the oracle."""
    w = _fp8("prefill_32k_chunk4k")
    print(f"[case] prefill_32k_chunk4k_e5m2 full {w}", flush=True)
    r = full_parity(si.make_inputs(w), w)
    _report("prefill_32k_chunk4k_e5m2", r)
    assert r["problems"] == 512
