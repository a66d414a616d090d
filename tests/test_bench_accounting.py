"""The bench's algorithmic work per gate/up launch, the numerator of its
roofline figure, against sums written out by hand from the layer shapes:
every weight of an expert that received rows read once (plus its fp8 block
scales), every dispatched row read once and every SwiGLU output written once,
the shared experts' weights and rows likewise, 2 flops per multiply-add."""
import numpy as np

import bench
import workloads as W


def test_decode_gate_up_work_by_hand():
    cfg = W.get_config(2)                  # H 2048, 64 experts top-6, I 1408, 2 shared of 1408, bf16
    counts = np.full(64, 12)               # 768 pairs of a 128-token microbatch, every expert hit
    (nbytes, flops), = bench.gateup_work(cfg, [counts], [128])
    weights = 64 * (2 * 1408) * 2048 * 2
    rows = 768 * 2048 * 2
    h = 768 * 1408 * 2
    shared = (2 * 2816) * 2048 * 2 + 128 * 2048 * 2 + 128 * 2816 * 2
    assert nbytes == weights + rows + h + shared == 767_819_776
    assert flops == 2 * 768 * 2048 * (2 * 1408) + 2 * 128 * 2048 * (2 * 2816) == 11_811_160_064


def test_prefill_fp8_gate_up_work_by_hand():
    cfg = W.get_config(3)                  # H 2048, 128 experts top-8, I 768, fp8 weights, no shared
    counts = np.full(128, 256)             # 32768 pairs of a 4096-token microbatch
    counts[5] = 0                          # an expert without rows reads no weights
    counts[6] = 512
    (nbytes, flops), = bench.gateup_work(cfg, [counts], [4096])
    weights = 127 * (2 * 768) * 2048 * 1 + 127 * (2 * 768 // 128) * (2048 // 128) * 4
    rows = 32768 * 2048 * 2
    h = 32768 * 768 * 2
    assert nbytes == weights + rows + h
    assert flops == 2 * 32768 * 2048 * (2 * 768)
    # fp8 activations: rows and h one byte per element plus one scale byte per 128
    (nb8, fl8), = bench.gateup_work(cfg, [counts], [4096], fp8_act=True)
    assert nb8 == weights + 32768 * 2048 * (1 + 1 / 128) + 32768 * 768 * (1 + 1 / 128)
    assert fl8 == flops


def test_shared_slabs_match_the_chunk_rule():
    # two shared experts of I = 1408 beside routed experts of I = 1408: the
    # down projection (K = 2816) is cut into two chunks of 1408
    assert bench.shared_slabs(W.get_config(2)) == 2
    assert bench.shared_slabs(W.get_config(3)) == 0


def test_per_expert_roof_by_hand():
    """Sum over experts of max(flops / 2.5 PFLOP/s, bytes / 8 TB/s): with 256
    rows each, the Qwen3-shaped gate/up experts are MFMA-bound (644 ns of
    flops against 574 ns of bytes each); the down experts HBM-bound."""
    cfg = W.get_config(3)
    counts = np.full(128, 256)
    counts[0] = 0
    t, fl, by, t_mfma, t_hbm = bench.ffn_expert_roof(cfg, counts, 4096, "gate_up")
    f_e = 4 * 256 * 2048 * 768
    b_e = 2 * 768 * 2048 + 256 * 2048 * 2 + 256 * 768 * 2 + 12 * 16 * 4
    assert f_e / 2.5e15 > b_e / 8e12
    assert abs(t - 127 * f_e / 2.5e15) < 1e-12 and t_hbm == 0.0
    assert fl == 127 * f_e and by == 127 * b_e
    t, fl, by, t_mfma, t_hbm = bench.ffn_expert_roof(cfg, counts, 4096, "down")
    f_e = 2 * 256 * 2048 * 768
    b_e = 2048 * 768 + 256 * 768 * 2 + 256 * 2048 * 2 + 16 * 6 * 4
    assert b_e / 8e12 > f_e / 2.5e15
    assert abs(t - 127 * b_e / 8e12) < 1e-12 and t_mfma == 0.0
    # decode: the shared experts count as one dense expert over the microbatch
    cfg2 = W.get_config(2)
    t2, _, by2, _, _ = bench.ffn_expert_roof(cfg2, np.full(64, 12), 128, "gate_up")
    shared = 2 * 2816 * 2048 * 2 + 128 * 2048 * 2 + 128 * 2816 * 2
    routed = 64 * (2 * 1408 * 2048 * 2 + 12 * 2048 * 2 + 12 * 1408 * 2)
    assert by2 == routed + shared and abs(t2 - (routed + shared) / 8e12) < 1e-12
