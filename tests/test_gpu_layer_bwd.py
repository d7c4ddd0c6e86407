"""GPU parity of the layer backward (tsp_layer_bwd_attn_mlp, tsp_layer_bwd_qkv) against the
fp64 oracle (layer_bwd: the derivative of the unsharded layer, pinned by torch autograd and
finite differences in the CPU suite).

Every rank of a mid-size workload runs on the one GPU: its forward (QKV, attention with the
log-sum-exp), part 1 of the backward on its rows of the output gradient, then, after its
dk/dv contributions are summed over the ranks (the one-GPU stand-in for the reduce-scatter),
part 2 on its rows. The ranks' dx rows, glued in position order, must equal the oracle's dx,
and every weight gradient summed over the ranks the oracle's. The pages name training but do
not describe the backward ("Folding Tensor and Sequence Parallelism for Memory-Efficient
Transformer Training & Inference", gist.science 2604.26294, title; §2 for the forward).
Tolerance: max-abs <= 2e-2 max|ref|, mean-abs <= 2e-3 max|ref| per tensor.
"""

import numpy as np
import pytest
import torch

from long_context_transformer_amd import synth, tsp
from oracle import tsp_oracle as O

from _gpu_helpers import check_close, dev_bf16, host_f64, shard_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsp.load()


LAYER_BWD_CASES = [  # B, S, D, H, hd, F
    (1, 512, 4, 4, 64, 688),     # F/D = 172: the GEMMs' ragged-K path
    (1, 1024, 2, 4, 128, 1024),
    (2, 768, 3, 3, 64, 1032),    # odd D, two sequences
]


@pytest.mark.parametrize("B,S,D,H,hd,F", LAYER_BWD_CASES)
def test_layer_bwd_all_ranks(B, S, D, H, hd, F):
    print(f"layer backward B={B} S={S} D={D} H={H} hd={hd} F={F}", flush=True)
    d = H * hd
    Fs = F // D
    w = synth.Workload(120 + S % 7, "mid", B, S, D, 0, d, H, hd, F)
    inputs = synth.layer_inputs(w)
    dy_bits = synth.normal_bf16((B, S, d), 130 + S % 7, std=1.0)
    f64 = {k: synth.to_f64(v) for k, v in inputs.items()}
    ref = O.layer_bwd(f64["x_full"], f64["w_qkv"], f64["w_o"], f64["w1"], f64["w3"], f64["w2"], H,
                      synth.to_f64(dy_bits))

    x_full = dev_bf16(inputs["x_full"])
    w_qkv, w_o = dev_bf16(inputs["w_qkv"]), dev_bf16(inputs["w_o"])
    w1, w3, w2 = dev_bf16(inputs["w1"]), dev_bf16(inputs["w3"]), dev_bf16(inputs["w2"])
    packed = tsp.pack_mlp_shards(w1, w3, w2, D)
    dy_full = torch.from_numpy(synth.to_f64(dy_bits).astype(np.float32)).cuda()
    kf = torch.empty((B, S, d), dtype=torch.bfloat16, device="cuda")
    vf = torch.empty_like(kf)
    R = S // D
    qs, xs_all = [], []
    for r in range(D):  # every rank's projections: its own K/V rows and its Q
        xs = shard_rows(x_full, S, D, r)
        q = torch.empty((B, R, d), dtype=torch.bfloat16, device="cuda")
        tsp.qkv_fwd(xs, w_qkv, q, kf, vf, B, S, D, r, H, hd)
        qs.append(q)
        xs_all.append(xs)
    desc0 = tsp.make_desc(B, S, D, 0, d, H, hd, F)
    ws = torch.empty(tsp.layer_bwd_workspace_size(desc0), dtype=torch.uint8, device="cuda")
    f32 = lambda *shape: torch.full(shape, float("nan"), dtype=torch.float32, device="cuda")
    dk_sum, dv_sum = torch.zeros((B, S, d), device="cuda"), torch.zeros((B, S, d), device="cuda")
    dwo_sum = torch.zeros((d, d), device="cuda")
    dw13_sum = [torch.zeros((2 * Fs, d), device="cuda") for _ in range(D)]
    dw2_sum = [torch.zeros((d, Fs), device="cuda") for _ in range(D)]
    dqs = []
    for r in range(D):
        desc = tsp.make_desc(B, S, D, r, d, H, hd, F)
        o = torch.empty((B, R, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, H, R), dtype=torch.float32, device="cuda")
        tsp.attn_fwd(qs[r], kf, vf, o, lse, B, S, D, r, H, hd)
        idx = torch.from_numpy(tsp.zigzag_index(S, D, r)).cuda()
        dy = dy_full.index_select(1, idx).contiguous()
        dq, dk, dv, dwo = f32(B, R, d), f32(B, S, d), f32(B, S, d), f32(d, d)
        dw13 = [f32(2 * Fs, d) for _ in range(D)]
        dw2 = [f32(d, Fs) for _ in range(D)]
        tsp.layer_bwd_attn_mlp(desc, qs[r], o, lse, kf, vf, w_o, packed, dy, dq, dk, dv, dwo, dw13, dw2, ws)
        dk_sum += dk
        dv_sum += dv
        dwo_sum += dwo
        for j in range(D):
            dw13_sum[j] += dw13[j]
            dw2_sum[j] += dw2[j]
        dqs.append(dq)
    dx_full = np.zeros((B, S, d))
    dwqkv_sum = torch.zeros((3 * d, d), device="cuda")
    for r in range(D):
        desc = tsp.make_desc(B, S, D, r, d, H, hd, F)
        idx = torch.from_numpy(tsp.zigzag_index(S, D, r)).cuda()
        dk_own = dk_sum.index_select(1, idx).contiguous()
        dv_own = dv_sum.index_select(1, idx).contiguous()
        dx, dwqkv = f32(B, R, d), f32(3 * d, d)
        tsp.layer_bwd_qkv(desc, xs_all[r], w_qkv, dqs[r], dk_own, dv_own, dx, dwqkv, ws)
        dwqkv_sum += dwqkv
        dx_full[:, tsp.zigzag_index(S, D, r)] = host_f64(dx)
    torch.cuda.synchronize()
    check_close("dx (glued over ranks)", dx_full, ref["dx"])
    check_close("dW_qkv (sum over ranks)", host_f64(dwqkv_sum), ref["dw_qkv"])
    check_close("dW_o (sum over ranks)", host_f64(dwo_sum), ref["dw_o"])
    dw1 = np.concatenate([host_f64(dw13_sum[j])[:Fs] for j in range(D)])
    dw3 = np.concatenate([host_f64(dw13_sum[j])[Fs:] for j in range(D)])
    dw2 = np.concatenate([host_f64(dw2_sum[j]) for j in range(D)], axis=1)
    check_close("dW1 (sum over ranks)", dw1, ref["dw1"])
    check_close("dW3 (sum over ranks)", dw3, ref["dw3"])
    check_close("dW2 (sum over ranks)", dw2, ref["dw2"])
