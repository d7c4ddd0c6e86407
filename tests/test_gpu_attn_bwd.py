"""GPU parity of the attention backward (tsp_attn_bwd) against the fp64 oracle.

The oracle is causal_attention_bwd: the derivative of the forward definition (pinned by
finite differences and by torch autograd in the CPU suite). The pages name training but do
not describe the backward pass ("Folding Tensor and Sequence Parallelism for
Memory-Efficient Transformer Training & Inference", gist.science 2604.26294, title; §2 for
the forward it differentiates).

Inputs are bf16 q, k, v, d_o; o and lse come from tsp_attn_fwd on the GPU (as a training
step would use them) or, in a second check, from the oracle. Tolerance: the contract's
max-abs <= 2e-2 max|ref| and mean-abs <= 2e-3 max|ref| per tensor (per head at full size).
At full size, dq is checked on sampled rows; dk and dv through properties that hold at any
size: summed over the keys, dk vanishes (each softmax row's ds sums to zero) and dv equals
the sum of d_o over the rank's rows (each P row sums to one).
"""

import numpy as np
import pytest
import torch

from long_context_transformer_amd import synth, tsp
from oracle import tsp_oracle as O

from _gpu_helpers import BF16_NAN, check_close, dev_bf16, host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsp.load()


def run_bwd(q, k, v, g, B, S, D, rank, H, hd, lse_host=None):
    """Forward on the GPU (o, lse), then the backward; lse_host replaces the forward's lse."""
    R = S // D
    qd, kd, vd, gd = dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(g)
    o = torch.empty((B, R, H, hd), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, R), dtype=torch.float32, device="cuda")
    tsp.attn_fwd(qd, kd, vd, o, lse, B, S, D, rank, H, hd)
    if lse_host is not None:
        lse = torch.from_numpy(lse_host.astype(np.float32)).cuda()
    nan = float("nan")
    dq = torch.full((B, R, H, hd), nan, dtype=torch.float32, device="cuda")
    dk = torch.full((B, S, H, hd), nan, dtype=torch.float32, device="cuda")
    dv = torch.full((B, S, H, hd), nan, dtype=torch.float32, device="cuda")
    ws = torch.empty(tsp.attn_bwd_workspace_size(B, S, D, H), dtype=torch.uint8, device="cuda")
    tsp.attn_bwd(qd, kd, vd, o, lse, gd, dq, dk, dv, B, S, D, rank, H, hd, ws)
    torch.cuda.synchronize()
    return dq, dk, dv


BWD_CASES = [  # B, S, D, rank, H, hd
    (1, 256, 4, 0, 2, 64),
    (1, 256, 4, 3, 2, 128),
    (2, 1200, 3, 1, 3, 128),   # C = 200: tiles and stages end mid-chunk
    (1, 4096, 2, 1, 2, 128),
    (1, 640, 1, 0, 2, 64),     # D = 1: ordinary causal attention
    (1, 96, 3, 2, 1, 64),      # C = 16: fewer rows than one tile
]


@pytest.mark.parametrize("B,S,D,rank,H,hd", BWD_CASES)
def test_attn_bwd_parity(B, S, D, rank, H, hd):
    print(f"attention backward B={B} S={S} D={D} rank={rank} H={H} hd={hd}", flush=True)
    seed = 700 + S % 97 + rank
    q = synth.normal_bf16((B, S // D, H, hd), seed, std=1.0)
    k = synth.normal_bf16((B, S, H, hd), seed + 1, std=1.0)
    v = synth.normal_bf16((B, S, H, hd), seed + 2, std=1.0)
    g = synth.normal_bf16((B, S // D, H, hd), seed + 3, std=1.0)
    idx = O.zigzag_index(S, D, rank)
    qf, kf, vf, gf = (synth.to_f64(x) for x in (q, k, v, g))
    rq, rk, rv = O.causal_attention_bwd(qf, idx, kf, vf, gf)
    _, ref_lse = O.causal_attention(qf, idx, kf, vf)
    for label, lse_host in (("forward kernel lse", None), ("oracle lse", ref_lse)):
        dq, dk, dv = run_bwd(q, k, v, g, B, S, D, rank, H, hd, lse_host=lse_host)
        check_close(f"{label} dq", host_f64(dq), rq)
        check_close(f"{label} dk", host_f64(dk), rk)
        check_close(f"{label} dv", host_f64(dv), rv)
        last = int(idx.max())
        assert torch.all(dk[:, last + 1:] == 0) and torch.all(dv[:, last + 1:] == 0), "keys no row sees"


@pytest.mark.parametrize("B,S,D,rank,H,hd", [(2, 1200, 3, 1, 3, 128), (1, 1320, 3, 2, 2, 64)])
def test_attn_bwd_unfilled_keys(B, S, D, rank, H, hd):
    """K/V rows after the rank's last position hold NaN (the forward never reads them, so a
    caller need not fill them). With C = 200 and C = 220 the rank's last position is not a
    multiple of 32, so a 32-key wave of the key-stationary kernel straddles it; its gradients
    must stay finite, match the oracle, and be exactly zero at keys no query of the rank sees."""
    print(f"attention backward, NaN past the last position: B={B} S={S} D={D} rank={rank}", flush=True)
    seed = 760 + rank
    q = synth.normal_bf16((B, S // D, H, hd), seed, std=1.0)
    k = synth.normal_bf16((B, S, H, hd), seed + 1, std=1.0)
    v = synth.normal_bf16((B, S, H, hd), seed + 2, std=1.0)
    g = synth.normal_bf16((B, S // D, H, hd), seed + 3, std=1.0)
    idx = O.zigzag_index(S, D, rank)
    last = int(idx.max())
    assert last + 1 < S and (last + 1) % 32 != 0
    k_nan, v_nan = k.copy(), v.copy()
    k_nan[:, last + 1:] = BF16_NAN
    v_nan[:, last + 1:] = BF16_NAN
    rq, rk, rv = O.causal_attention_bwd(synth.to_f64(q), idx, synth.to_f64(k), synth.to_f64(v), synth.to_f64(g))
    dq, dk, dv = run_bwd(q, k_nan, v_nan, g, B, S, D, rank, H, hd)
    check_close("dq", host_f64(dq), rq)
    check_close("dk", host_f64(dk), rk)
    check_close("dv", host_f64(dv), rv)
    assert torch.all(dk[:, last + 1:] == 0) and torch.all(dv[:, last + 1:] == 0), "keys no row sees"


def test_attn_bwd_errors_and_empty():
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    f = torch.empty(0, dtype=torch.float32, device="cuda")
    tsp.attn_bwd(e, e, e, e, f, e, f, f, f, 0, 256, 4, 1, 2, 64, None, 0)
    with pytest.raises(tsp.TspError) as ex:
        tsp.attn_bwd(e, e, e, e, f, e, f, f, f, 1, 256, 4, 1, 2, 64, None, 0)
    assert ex.value.code == 1
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    t = torch.zeros(64, dtype=torch.bfloat16, device="cuda")
    tf = torch.zeros(64, dtype=torch.float32, device="cuda")
    with pytest.raises(tsp.TspError) as ex:
        tsp.attn_bwd(t, t, t, t, tf, t, tf, tf, tf, 1, 256, 4, 1, 2, 64, ws)
    assert ex.value.code == 5


@pytest.mark.parametrize("name,rank", [("7b_s128k_d8", 0), ("7b_s32k_d8", 5)])
def test_attn_bwd_fullsize(name, rank):
    """Full size, one rank: dq on sampled rows per head against the oracle; dk and dv per
    head through their sums over the keys."""
    w = synth.WORKLOADS[name].with_rank(rank)
    B, S, D, H, hd, C = w.B, w.S, w.D, w.n_heads, w.head_dim, w.C
    R = S // D
    print(f"full-size attention backward {name} rank {rank}", flush=True)
    std = float(np.sqrt(4096) * 0.02)
    q = synth.normal_bf16((B, R, H, hd), 9100 + rank, std=std)
    k = synth.normal_bf16((B, S, H, hd), 9101, std=std)
    v = synth.normal_bf16((B, S, H, hd), 9102, std=1.0)
    g = synth.normal_bf16((B, R, H, hd), 9103 + rank, std=1.0)
    dq, dk, dv = run_bwd(q, k, v, g, B, S, D, rank, H, hd)
    dq_h = host_f64(dq)
    # sums over keys, per (sequence, head), in float64 on the GPU
    sk = dk.double().sum(dim=1).cpu().numpy()          # [B, H, hd]
    ak = dk.double().abs().sum(dim=1).cpu().numpy()    # [B, H, hd]
    sv = dv.double().sum(dim=1).cpu().numpy()
    del dk, dv, dq
    torch.cuda.empty_cache()
    gsum = synth.to_f64(g).sum(axis=1)  # [B, H, hd]
    for h in range(H):
        # sum_j dk_j = scale sum_i (sum_j ds_ij) q_i vanishes: the sum cancels to a small
        # fraction of the sum of magnitudes (rounding, and the forward's lse error)
        frac = float(np.abs(sk[0, h]).max() / ak[0, h].max())
        assert frac < 2e-2, (h, frac)
        check_close(f"h{h} sum_j dv_j vs sum_i do_i", sv[0, h], gsum[0, h])
    idx = O.zigzag_index(S, D, rank)
    rng = np.random.default_rng(9200 + rank)
    rows = np.unique(np.concatenate([[0, C - 1, C, 2 * C - 1], rng.choice(2 * C, 6, replace=False)]))
    kmax = int(idx[rows].max()) + 1
    rq, _, _ = O.causal_attention_bwd(synth.to_f64(q[:, rows]), idx[rows], synth.to_f64(k[:, :kmax]),
                                      synth.to_f64(v[:, :kmax]), synth.to_f64(g[:, rows]))
    for h in range(H):
        check_close(f"dq h{h}", dq_h[0, rows, h], rq[0, :, h])
