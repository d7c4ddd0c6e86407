"""GPU parity of the weight-streamed layer (tsp_layer_fwd_streamed) against the fp64 oracle.

The rank holds two receive slots per weight kind; the layer runs as a loop over head
groups (QKV of the group, attention of its heads, the group's W_O partial added to an fp32
sum) and the MLP ring over shards, each shard copied into a slot on a copy stream while
the previous one computes (summary of "Folding Tensor and Sequence Parallelism for
Memory-Efficient Transformer Training & Inference", gist.science 2604.26294, §2 attention
and MLP layers, §3 overlap of weight transfers). The per-rank outputs are those of the
unsharded layer at the rank's positions, as for tsp_layer_fwd.
Tolerance: max-abs <= 2e-2 max|ref|, mean-abs <= 2e-3 max|ref| per tensor; the run on
four streams and the run on one stream must agree bit for bit (same launches, same
accumulation order, only the overlap differs).
"""

import numpy as np
import pytest
import torch

from long_context_transformer_amd import synth, tsp
from oracle import tsp_oracle as O

from _gpu_helpers import check_close, dev_bf16, fill_peer_kv, host_f64, nan_bf16, shard_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsp.load()


def run_streamed(w, inputs, rank, overlap=True, calls=1):
    B, S, D, H, hd, d, F = w.B, w.S, w.D, w.n_heads, w.head_dim, w.d_model, w.ffn
    x_full = dev_bf16(inputs["x_full"])
    w_qkv, w_o = dev_bf16(inputs["w_qkv"]), dev_bf16(inputs["w_o"])
    w1, w3, w2 = dev_bf16(inputs["w1"]), dev_bf16(inputs["w3"]), dev_bf16(inputs["w2"])
    pa = tsp.pack_attn_shards(w_qkv, w_o, D)
    pm = tsp.pack_mlp_shards(w1, w3, w2, D)
    kf, vf = nan_bf16((B, S, d)), nan_bf16((B, S, d))
    fill_peer_kv(x_full, w_qkv, kf, vf, B, S, D, rank, H, hd)
    xs = shard_rows(x_full, S, D, rank)
    desc = tsp.make_desc(B, S, D, rank, d, H, hd, F)
    ws = torch.full((tsp.layer_streamed_workspace_size(desc),), 0xFF, dtype=torch.uint8, device="cuda")
    a = nan_bf16((B, S // D, d))
    y = torch.full((B, S // D, d), float("nan"), dtype=torch.float32, device="cuda")
    streams = [torch.cuda.Stream() for _ in range(3)] if overlap else None
    torch.cuda.synchronize()
    for _ in range(calls):
        tsp.layer_fwd_streamed(desc, xs, pa, pm, kf, vf, a, y, ws, streams=streams)
    torch.cuda.synchronize()
    idx = torch.from_numpy(tsp.zigzag_index(S, D, rank)).cuda()
    assert bool(torch.isfinite(kf[:, idx]).all()) and bool(torch.isfinite(vf[:, idx]).all())
    return a, y


STREAMED_MID = [  # B, S, D, rank, H, hd, F
    (2, 2048, 4, 1, 4, 128, 1376),  # Fs = 344, one head per group
    (1, 1200, 3, 2, 6, 64, 1032),   # odd D (last W_O step on the caller's stream), C = 200
    (1, 512, 8, 5, 8, 64, 2304),    # D = 8, ring wraps at rank 5
    (1, 768, 2, 1, 4, 64, 1040),    # D = 2: both slots in use from the start, no refill
    (1, 256, 4, 2, 8, 64, 696),     # Fs = 174: padded W2 stride in the packed shard
    (1, 256, 1, 0, 2, 128, 512),    # D = 1: one group, its W_O step is also the last
]


@pytest.mark.parametrize("B,S,D,rank,H,hd,F", STREAMED_MID)
def test_streamed_layer_parity(B, S, D, rank, H, hd, F):
    print(f"streamed layer B={B} S={S} D={D} rank={rank} H={H} hd={hd} F={F}", flush=True)
    w = synth.Workload(110 + S % 7, "mid", B, S, D, rank, H * hd, H, hd, F)
    inputs = synth.layer_inputs(w)
    a, y = run_streamed(w, inputs, rank, overlap=True, calls=2)
    a1, y1 = run_streamed(w, inputs, rank, overlap=False)
    f64 = {k: synth.to_f64(v) for k, v in inputs.items()}
    ref = O.rank_layer(f64["x_full"], f64["w_qkv"], f64["w_o"], f64["w1"], f64["w3"], f64["w2"],
                       S, D, rank, H)
    check_close("attn_out", host_f64(a), ref["attn_out"])
    check_close("mlp_out", host_f64(y), ref["mlp_out"])
    assert torch.equal(a, a1), "four-stream and one-stream runs differ (attn_out)"
    assert torch.equal(y, y1), "four-stream and one-stream runs differ (mlp_out)"


def test_streamed_tiny_all_ranks_glued():
    """The tiny workload, every rank: the ranks' outputs glued in position order equal
    the unsharded layer."""
    w = synth.WORKLOADS["tiny_s256_d4"]
    inputs = synth.layer_inputs(w)
    f64 = {k: synth.to_f64(v) for k, v in inputs.items()}
    full = O.rank_layer(f64["x_full"], f64["w_qkv"], f64["w_o"], f64["w1"], f64["w3"], f64["w2"],
                        w.S, 1, 0, w.n_heads)
    glued_a = np.zeros_like(full["attn_out"])
    glued_y = np.zeros_like(full["mlp_out"])
    for r in range(w.D):
        print(f"streamed tiny rank {r}", flush=True)
        a, y = run_streamed(w, inputs, r)
        idx = O.zigzag_index(w.S, w.D, r)
        glued_a[:, idx] = host_f64(a)
        glued_y[:, idx] = host_f64(y)
    check_close("glued attn_out", glued_a, full["attn_out"])
    check_close("glued mlp_out", glued_y, full["mlp_out"])


@pytest.mark.parametrize("name", ["tiny_s256_d4", "7b_s16k_d8", "7b_s128k_d8"])
def test_streamed_memory_footprint(name):
    """The rank's buffers for tsp_layer_fwd_streamed are exactly the analytic per-rank count,
    and a call changes neither the device's free memory nor the allocator's peak: the library
    allocates nothing. (The allocator's own count of those tensors may exceed their sizes by
    up to 1 MiB each: it rounds to 512 bytes and does not split a cached block when less than
    1 MiB would remain.)"""
    from long_context_transformer_amd import memory
    print(f"memory footprint {name}", flush=True)
    r = memory.measure_streamed(synth.WORKLOADS[name], 0)
    print(f"  owned {r['measured_owned_bytes']} tensors {r['owned_tensor_bytes']} "
          f"analytic {r['analytic_tsp_streamed_bytes']} free change {r['free_bytes_change_during_call']}", flush=True)
    assert r["owned_tensor_bytes"] == r["analytic_tsp_streamed_bytes"]
    assert 0 <= r["measured_owned_bytes"] - r["owned_tensor_bytes"] <= 8 * (1 << 20)
    assert r["free_bytes_change_during_call"] == 0
    assert r["allocator_peak_growth_during_call"] == 0
