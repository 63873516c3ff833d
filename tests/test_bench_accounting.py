"""Host-side checks of bench.py's roofline accounting (no GPU).

The algorithmic work of each step at the PixArt-2048 shape (16 384 tokens,
C = 1152, 16 heads x 72, r = 4) against figures derived here from the
layer's definition: a Linear over M tokens is 2 M N K flops and reads its
input and weights once and writes its output once; the 3x3 conv is a
Linear with K = 9 C; the depthwise stride-2 conv reads kv0 once and writes
the compressed keys and values.
"""
import pytest

import bench
from seeded_inputs import CONFIGS

S = CONFIGS["pixart2048"]
M, C, CR = S.B * S.N, S.C, S.C // 4
NC = S.B * ((S.H + 1) // 2) * ((S.W + 1) // 2)
BF = 2   # bytes per bf16 element


@pytest.fixture(scope="module")
def work():
    return bench.algorithmic_work(S)


def test_projection_flops_exact(work):
    assert work["kv_proj"][0] == 2 * M * (2 * C) * C
    assert work["out_proj"][0] == 2 * M * C * C
    # the query Linear over [x | act] with the restore folded into its weights: K = C + C/r
    assert work["q_proj"][0] == 2 * M * C * (C + CR)


def test_projection_bytes(work):
    # x in, kv0 out, both weights
    assert work["kv_proj"][1] == BF * (M * C + M * 2 * C + 2 * C * C + 2 * C)
    assert work["out_proj"][1] == BF * (M * C + M * C + C * C + C)


def test_conv_flops(work):
    # the implicit GEMM (K = 9 C) plus, in the same launch, the restore fold W_q [W_cf2 | b_cf2]
    conv = 2 * M * CR * 9 * C
    fold = 2 * C * C * (CR + 1)
    assert work["cf_conv3x3"][0] == pytest.approx(conv + fold, rel=1e-3)


def test_memory_bound_bytes(work):
    # bf16: kv0 in, K' and V' out, the depthwise weights, the per-head state out (K', V' not read back)
    st = S.B * S.heads * (S.head_dim ** 2 + S.head_dim) * 4
    assert work["sc_dwconv"][1] == BF * (M * 2 * C + 2 * NC * C) + BF * 2 * (9 * C + C) + st
    # q in, y out; the per-head operand and z are a rounding error beside them
    assert work["linattn_apply"][1] == pytest.approx(BF * 2 * M * C, rel=0.01)
    # the merge of the 16 chunk partials (80 x 80 fp32 each) of the 16 heads, and the state out
    assert work["kv_state"][1] == 16 * 16 * 80 * 80 * 4 + st
    # fp32: the two passes of the design (K', V' written, then read by the state)
    w32 = bench.algorithmic_work(CONFIGS["tiny"])
    t = CONFIGS["tiny"]
    nc = t.B * t.Nc
    assert w32["kv_state"][1] == 4 * 2 * nc * t.C + t.B * t.heads * (t.head_dim ** 2 + t.head_dim) * 4


def test_layer_floor():
    """The layer at the published peaks (2.5 PFLOP/s bf16 MFMA, 8 TB/s HBM):
    ~140 us, i.e. ~117 M image tokens/s per layer at 100%."""
    w = bench.algorithmic_work(S)
    floor_us = sum(max(f / (bench.PEAK_MFMA_TFLOPS["bf16"] * 1e6), b / (bench.PEAK_HBM_GBS * 1e3))
                   for f, b in w.values())
    assert 130.0 < floor_us < 150.0


def test_statistics_tile_rows():
    # 256-row statistics tiles unless they would fill fewer than half the CUs
    assert bench.gn_tile_rows(CONFIGS["pixart2048"]) == 256
    assert bench.gn_tile_rows(CONFIGS["pixart1024"]) == 256   # W = 64: the kernel-row conv
    assert bench.stats_in_conv(CONFIGS["pixart1024"]) and bench.stats_in_conv(CONFIGS["pixart2048"])
    assert not bench.stats_in_conv(CONFIGS["tiny"])   # fp32: the separate statistics pass
