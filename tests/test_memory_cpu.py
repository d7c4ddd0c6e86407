"""CPU checks of the per-rank memory accounting (long_context_transformer_amd.memory).

The workspace terms must equal the library's own size queries byte for byte, so the TSP
counts are the buffers the library really asks for. The layout comparison then checks the
qualitative memory results the pages report for the 7B layer at 16K-128K tokens: TSP holds
the least of the compared layouts at every length; TP's activations grow with the whole
sequence, so its gap to TSP widens with S; SP keeps every weight ("Folding Tensor and Sequence
Parallelism for Memory-Efficient Transformer Training & Inference", gist.science
2604.26294, §2 unified sharding, §4 memory efficiency and larger micro-batches).
"""

import os

import pytest

from long_context_transformer_amd import memory as mm
from long_context_transformer_amd import synth, tsp

needs_lib = pytest.mark.skipif(not os.path.exists(tsp.LIB_PATH), reason="libtsp.so not built")

SHAPES = [  # B, S, D, d, H, hd, F
    (1, 256, 4, 256, 4, 64, 688),        # tiny workload, F/D = 172 (padded stride 176)
    (2, 1200, 3, 384, 6, 64, 1032),
    (1, 512, 8, 512, 8, 64, 2304),
    (1, 256, 1, 256, 2, 128, 512),       # D = 1
    (1, 256, 4, 512, 8, 64, 696),        # F/D = 174
    (1, 131072, 8, 4096, 32, 128, 11008),
    (4, 65536, 8, 4096, 32, 128, 11008),
]


@needs_lib
@pytest.mark.parametrize("B,S,D,d,H,hd,F", SHAPES)
def test_workspace_terms_equal_the_library(B, S, D, d, H, hd, F):
    s = mm.Shape(B, S, D, d, H, hd, F)
    desc = tsp.make_desc(B, S, D, 0, d, H, hd, F)
    assert mm.layer_workspace(s) == tsp.layer_workspace_size(desc)
    assert mm.streamed_workspace(s) == tsp.layer_streamed_workspace_size(desc)


@pytest.mark.parametrize("B,S,D,d,H,hd,F", SHAPES)
def test_layout_identities(B, S, D, d, H, hd, F):
    s = mm.Shape(B, S, D, d, H, hd, F)
    ts, tr, tp_, sp_ = mm.tsp_streamed(s), mm.tsp_resident(s), mm.tp(s), mm.sp(s)
    full_w = (4 * d * d + 3 * d * F) * 2
    assert tr["weights"] == sp_["weights"] == full_w
    assert tp_["weights"] * D == full_w
    # the rank's own packed shards are 1/D of the weights, plus the W2 stride padding
    pad = d * (s.Fp - s.Fs) * 2
    assert ts["weights"] * D == full_w + D * pad
    # tokens: TSP holds 1/D of what TP holds, K/V over the whole sequence like SP
    assert ts["x"] * D == tp_["x"] and ts["mlp_out"] * D == tp_["mlp_out"]
    assert ts["kv"] == sp_["kv"] == 2 * B * S * d * 2
    if D == 1:
        assert tp_["hidden"] == sp_["hidden"]


def test_pages_memory_results_at_7b():
    """TSP is the lowest of TSP/TP/SP at 16K-128K; TP's excess over TSP grows with S; SP's
    excess is its full weights; TSP fits the largest micro-batch."""
    names = ["7b_s16k_d8", "7b_s32k_d8", "7b_s128k_d8"]
    ratios = []
    for n in names:
        s = mm.shape_of(synth.WORKLOADS[n])
        for per in (mm.per_rank_bytes(s), mm.model_peak_bytes(s, 32)):
            assert per["tsp_streamed"] < min(per["tp"], per["sp"]), (n, per)
        peak = mm.model_peak_bytes(s, 32)
        ratios.append(peak["tp"] / peak["tsp_streamed"])
        bmax = {k: mm.max_batch(s, 32, 288 * 10**9, k) for k in ("tsp_streamed", "tp", "sp")}
        assert bmax["tsp_streamed"] > max(bmax["tp"], bmax["sp"]), (n, bmax)
    assert ratios == sorted(ratios) and ratios[-1] > ratios[0], ratios
    assert ratios[0] < 1.1  # short sequences: TSP and TP are close (weights dominate)


def test_max_batch_is_the_largest_fit():
    s = mm.shape_of(synth.WORKLOADS["7b_s128k_d8"])
    cap = 40 * 10**9
    for layout in mm.LAYOUTS:
        b = mm.max_batch(s, 32, cap, layout)
        fit = lambda x: mm.model_peak_bytes(mm.Shape(x, s.S, s.D, s.d, s.H, s.hd, s.F), 32)[layout] <= cap
        assert b == 0 or fit(b)
        assert not fit(b + 1)
