"""CPU checks of bench.py: the algorithmic byte and FLOP counts behind its
roofline figures, and its command-line contract."""
import os
import re
import subprocess
import sys

import torch

import bench
import synth_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_rounds_of():
    assert bench.rounds_of(2048, 32) == 6      # 64-block chunks halve six times
    assert bench.rounds_of(32, 32) == 0        # dense: nothing to search
    assert bench.rounds_of(10, 32) == 0
    assert bench.rounds_of(100, 8) == 4        # chunks of 12-13 blocks: 13 -> 7 -> 4 -> 2 -> 1


def test_decode_bytes_128k_b4():
    """32 problems (4 sequences x 8 KV heads); 2048 blocks of 64 keys, 32 kept."""
    nb = bench.decode_bytes(si.workload("decode_128k_b4"))
    assert nb["rounds"] == 6
    assert nb["centre"] == 3 * 2 ** 20         # 32 x 6 rounds x 64 centre rows x 256 B
    assert nb["kv"] == 32 * 2 ** 20            # 32 x 2048 selected tokens x (K + V) 512 B
    assert nb["q"] == 4 * 32 * 256
    assert nb["step"] == 36_806_912
    assert nb["step"] == nb["mask"] + nb["attn"] + nb["out"] - nb["q"]


def test_decode_bytes_fp8_kv():
    """An E5M2 KV cache halves the centre-row and K/V bytes; q and out stay bf16."""
    nb = bench.decode_bytes(si.workload("decode_128k_b4", dtype="bf16_e5m2"))
    assert nb["centre"] == 3 * 2 ** 19 and nb["kv"] == 16 * 2 ** 20
    assert nb["q"] == nb["out"] == 4 * 32 * 256
    assert nb["step"] == 3 * 2 ** 19 + 16 * 2 ** 20 + 3 * 4 * 32 * 256 + 2 * 32 * 33 * 4


def test_traffic_lookup_separates_element_types():
    m = bench.kernel_matches
    bf = "attn_decode_mfma<unsigned short, 128, 4, 128>"
    f8 = "attn_decode_mfma<unsigned char, 128, 4, 128>"
    assert m(bf, "bf16") and not m(bf, "bf16_e5m2") and m(f8, "bf16_e5m2") and not m(f8, "bf16")
    mk8 = "mask_decode_kernel<unsigned short, unsigned char, 128, 4, 2>"
    assert m(mk8, "bf16_e5m2") and not m(mk8, "bf16")
    comb = "attn_decode_combine<unsigned short, 128>"
    assert m(comb, "bf16") and m(comb, "bf16_e5m2") and not m(comb, "f32")
    assert m("attn_decode_kernel<float, 64, 1, 64>", "f32")
    st = "decode_step_kernel<unsigned short, 128, 4, 1, 256, true, false>"
    st8 = "decode_step_kernel<unsigned char, 128, 4, 1, 256, true, false>"
    assert m(st, "bf16") and not m(st, "bf16_e5m2") and m(st8, "bf16_e5m2") and not m(st8, "bf16")


def test_decode_bytes_dense_case():
    """k >= T: no search rounds, every block attended."""
    w = si.workload("tiny_decode", k=1024)
    nb = bench.decode_bytes(w)
    assert nb["rounds"] == 0 and nb["centre"] == 0
    assert nb["kv"] == 1 * 1 * 2 * 1024 * 64 * 4


def test_prefill_flops_chunk():
    fl = bench.prefill_flops(si.workload("prefill_32k_chunk4k"))
    # every 64-row block of the chunk sees >= 32 blocks: 2048 selected keys,
    # QK^T and PV at 2 flops per multiply-add
    assert fl["attn"] == 64 * 32 * 64 * 2048 * 128 * 4
    assert abs(fl["mask"] / 8.59e9 - 1) < 0.01


def test_prefill_mask_flops_power_of_two():
    """N_p = K_b * 2^R: every round scores exactly 2 K_b candidates."""
    w = si.workload("prefill_32k_chunk4k", B=1, Hq=1, Hkv=1, T=4096, Tq=64, k=8 * 64)
    fl = bench.prefill_flops(w)
    ncand = 3 * 2 * 8                          # 64 blocks, 8 kept: 8 -> 4 -> 2 -> 1
    assert fl["mask"] == 2 * 64 * 128 * ncand


def test_call_kernels_name_real_kernels():
    src = ""
    d = os.path.join(ROOT, "long_context_sparse_mask_amd", "csrc")
    for f in os.listdir(d):
        src += open(os.path.join(d, f)).read()
    kernels = set(re.findall(r"__global__.*?void\s+(\w+)\s*\(", src))
    for names in bench.CALL_KERNELS.values():
        for n in names:
            assert any(k.startswith(n) for k in kernels), n


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_page_pool_addressing():
    """The bench's page pool: position t of sequence b is row t % page_size of
    page table[b, t // page_size], pages shuffled over the pool."""
    g = torch.Generator().manual_seed(0)
    B, Hkv, T, d, ps = 2, 3, 256, 4, 64
    K, V = torch.randn(B, Hkv, T, d), torch.randn(B, Hkv, T, d)
    Kp, Vp, tab = bench.page_pool(K, V, T, ps, g, torch)
    assert Kp.shape == (B * T // ps, Hkv, ps, d) and tab.dtype == torch.int32
    assert sorted(tab.flatten().tolist()) == list(range(B * T // ps))
    t = torch.arange(T)
    for b in range(B):
        assert torch.equal(Kp[tab[b, t // ps].long(), :, t % ps].permute(1, 0, 2), K[b])
        assert torch.equal(Vp[tab[b, t // ps].long(), :, t % ps].permute(1, 0, 2), V[b])


def test_source_hash_ignores_comments_only(tmp_path):
    """The hash that gates the measured traffic survives comment and layout
    edits and changes with any code edit."""
    src = 'int f(int a) { // add one\n  return a + 1; /* done */ }\nconst char *s = "// kept";\n'
    (tmp_path / "k.hip").write_text(src)
    base = bench.kernel_source_sha(str(tmp_path))
    (tmp_path / "k.hip").write_text(src.replace("// add one", "// increment").replace("  return", "return"))
    assert bench.kernel_source_sha(str(tmp_path)) == base
    (tmp_path / "k.hip").write_text(src.replace('"// kept"', '"// changed"'))
    assert bench.kernel_source_sha(str(tmp_path)) != base
    (tmp_path / "k.hip").write_text(src.replace("a + 1", "a + 2"))
    assert bench.kernel_source_sha(str(tmp_path)) != base


def test_needle_share():
    """Needle recall counts (KV head, needle) pairs whose block is listed."""
    import numpy as np
    x = {"needles": [5, 9]}
    lists = np.full((1, 2, 1, 4), -1, np.int32)
    lists[0, 0, 0, :2] = [5, 9]   # head 0 finds both
    lists[0, 1, 0, :2] = [1, 9]   # head 1 finds one
    assert bench.needle_share(x, lists) == 0.75
    assert bench.needle_recall(x, lists) == {"gpu": 0.75, "needles": 2}


def test_stage_lists_end_at_the_workload_k():
    """The multi-stage leg's lists keep the workload's k in single blocks."""
    for name, stages in bench.STAGES.items():
        w = si.workload(name)
        assert stages[0][1] is None and stages[-1] == (w.block_k, w.k)
        assert all(a[0] > b[0] for a, b in zip(stages, stages[1:]))


def test_stage_candidates():
    """Rounds of the bench's stage lists, traced by hand: 128k x 4 has 2048
    blocks, 256 stage-0 chunks of 8; stage 1 (2-block chunks, keep 64) halves
    them twice (512, then 128 candidates), stage 2 (single blocks, keep 32)
    once (128).  1M: 16384 blocks, 2048 chunks: 4096, 256, 256."""
    assert bench.stage_candidates(si.workload("decode_128k_b4"), bench.STAGES["decode_128k_b4"]) == [512, 128, 128]
    assert bench.stage_candidates(si.workload("decode_1m_needles"), bench.STAGES["decode_1m_needles"]) == [4096, 256, 256]
    # 40 blocks in 8 stage-0 chunks of 5: stage 1 (4-block chunks, keep 8)
    # halves once (16 candidates, widths 3); stage 2 (3-block chunks, keep 6)
    # finds them fitting and still ranks them (8); stage 3 (single blocks,
    # keep 4) halves twice (12, then 8)
    w = si.workload("tiny_decode", T=320, block_k=8, k=32)
    assert bench.stage_candidates(w, [(40, None), (32, 256), (24, 144), (8, 32)]) == [16, 8, 12, 8]
    nb = bench.stage_mask_bytes(si.workload("decode_128k_b4"), bench.STAGES["decode_128k_b4"])
    assert nb == 32 * (768 * 256 + 4 * 256 + 4 * 33)


def test_stage_candidates_match_the_oracle_trace():
    """The bench's round counts equal the candidates the oracle's stage search
    scores per round (trace of one problem)."""
    import oracle
    w = si.workload("decode_32k", Hq=4, Hkv=1)
    x = si.make_inputs(w)
    st = bench.STAGES["decode_128k_b4"]
    tr = oracle.mask_stages_one(x["q"], x["K"], 0, 0, 0, st, T=w.T, block_k=w.block_k)
    assert [len(r["start"]) for r in tr["rounds"]] == bench.stage_candidates(w, st) == [128, 128, 128]
