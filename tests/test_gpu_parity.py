"""GPU parity of every C-ABI entry point against the fp64 CPU oracle, at sizes the oracle
finishes in seconds that still span several tiles and ragged tails, plus the method's
edge cases (D = 1, the diagonal, keys after the rank's last position never read).

Method: summary of "Folding Tensor and Sequence Parallelism for Memory-Efficient
Transformer Training & Inference" (gist.science 2604.26294), §2. Tolerance: max-abs
<= 2e-2 max|ref|, mean-abs <= 2e-3 max|ref|; zigzag maps and untouched rows bit-exact.
"""

import numpy as np
import pytest
import torch

from long_context_transformer_amd import synth, tsp
from oracle import tsp_oracle as O

from _gpu_helpers import (RAMP_SCALE, BF16_NAN, ramp_inputs, check_close, check_lse, dev_bf16, fill_peer_kv, host_bits, host_f64,
                          nan_bf16, shard_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsp.load()


# ------------------------------------------------------------------------------- a2 QKV
QKV_CASES = [  # B, S, D, rank, H, hd
    (1, 256, 4, 0, 4, 64),
    (1, 256, 4, 3, 4, 64),
    (2, 1200, 3, 1, 4, 128),   # C = 200: ragged row tiles
    (1, 640, 1, 0, 2, 128),    # D = 1
    (1, 4096, 2, 1, 32, 128),  # M = 2048, N = 12288: 384 tiles of 256 x 256 (the large-tile kernel)
    (1, 8192, 2, 0, 32, 128),  # M = 4096, N = 12288: 768 tiles of 256 x 256 in one launch
    (1, 8192, 8, 3, 32, 128),  # M = 1024, N = 12288: 384 tiles of 256 x 128 (the narrow persistent tile)
]


@pytest.mark.parametrize("B,S,D,rank,H,hd", QKV_CASES)
def test_qkv_parity(B, S, D, rank, H, hd):
    print(f"qkv B={B} S={S} D={D} rank={rank} H={H} hd={hd}", flush=True)
    d = H * hd
    x_full = synth.normal_bf16((B, S, d), 7001 + S)
    w_qkv = synth.normal_bf16((3 * d, d), 7002 + S, 0.02)
    xs = shard_rows(dev_bf16(x_full), S, D, rank)
    q = torch.empty((B, S // D, d), dtype=torch.bfloat16, device="cuda")
    kf, vf = nan_bf16((B, S, d)), nan_bf16((B, S, d))
    tsp.qkv_fwd(xs, dev_bf16(w_qkv), q, kf, vf, B, S, D, rank, H, hd)
    torch.cuda.synchronize()
    idx = O.zigzag_index(S, D, rank)
    qr, kr, vr = O.qkv_rows(synth.to_f64(x_full)[:, idx], synth.to_f64(w_qkv), H)
    check_close("q", host_f64(q), qr.reshape(B, -1, d))
    kb, vb = host_bits(kf), host_bits(vf)
    check_close("k rows", synth.to_f64(kb[:, idx]), kr.reshape(B, -1, d))
    check_close("v rows", synth.to_f64(vb[:, idx]), vr.reshape(B, -1, d))
    others = np.setdiff1d(np.arange(S), idx)
    assert np.all(kb[:, others] == BF16_NAN) and np.all(vb[:, others] == BF16_NAN)


# ------------------------------------------------------------------------- a3 attention
ATTN_CASES = [  # B, S, D, rank, H, hd
    (1, 256, 4, 0, 4, 64),      # the tiny workload, every rank
    (1, 256, 4, 1, 4, 64),
    (1, 256, 4, 2, 4, 64),
    (1, 256, 4, 3, 4, 64),
    (1, 256, 4, 0, 2, 128),
    (2, 1200, 3, 1, 3, 128),    # C = 200: tiles straddle chunks, ragged key stages
    (1, 1200, 3, 2, 2, 64),
    (2, 4096, 2, 1, 2, 128),    # C = 1024: many full stages
    (1, 640, 1, 0, 2, 128),     # D = 1: plain causal attention
    (1, 96, 3, 2, 1, 64),       # C = 16, one tile holding both chunks
    # B*H a multiple of the 8 XCDs and few tiles: longest tile first across an XCD's heads
    (1, 2048, 2, 1, 8, 64),     # 4 tiles per head
    (2, 1536, 3, 2, 4, 128),    # two sequences, 2 tiles per head
]


@pytest.mark.parametrize("B,S,D,rank,H,hd", ATTN_CASES)
def test_attn_parity(B, S, D, rank, H, hd):
    print(f"attn B={B} S={S} D={D} rank={rank} H={H} hd={hd}", flush=True)
    C = S // (2 * D)
    rows = 2 * C
    q = synth.normal_bf16((B, rows, H, hd), 7101 + S + rank)
    k = synth.normal_bf16((B, S, H, hd), 7102 + S + rank)
    v = synth.normal_bf16((B, S, H, hd), 7103 + S + rank)
    end = (2 * D - rank) * C
    # rows after the rank's last position hold NaN: the kernel must never read them
    k[:, end:] = BF16_NAN
    v[:, end:] = BF16_NAN
    o = torch.empty((B, rows, H, hd), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, rows), dtype=torch.float32, device="cuda")
    tsp.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), o, lse, B, S, D, rank, H, hd)
    torch.cuda.synchronize()
    idx = O.zigzag_index(S, D, rank)
    ref_o, ref_lse = O.causal_attention(synth.to_f64(q), idx, synth.to_f64(k[:, :end]),
                                        synth.to_f64(v[:, :end]))
    check_close("o", host_f64(o), ref_o)
    check_lse("lse", host_f64(lse), ref_lse)
    # per (chunk, head) so a small-valued late chunk cannot hide behind an early one
    got = host_f64(o)
    for c0 in (0, C):
        for h in range(H):
            check_close(f"o chunk{c0 // C} head{h}", got[:, c0:c0 + C, h], ref_o[:, c0:c0 + C, h])


RAMP_CASES = [  # B, S, D, rank, H, hd
    (1, 2048, 2, 1, 4, 128),
    (2, 1024, 4, 2, 4, 128),
    (1, 512, 1, 0, 4, 128),    # D = 1: plain causal attention
    (1, 1200, 3, 1, 4, 64),
]


@pytest.mark.parametrize("B,S,D,rank,H,hd", RAMP_CASES)
def test_attn_reference_moves(B, S, D, rank, H, hd):
    """Scores that climb, creep, fall or wander along the keys: the online softmax's
    reference moves at every block, every few blocks or never, and each case must still
    match the oracle (O per head, and the log-sum-exp)."""
    print(f"attn reference moves B={B} S={S} D={D} rank={rank} H={H} hd={hd}", flush=True)
    rows = S // D
    q, k, v = ramp_inputs(B, S, rows, H, hd, 7300 + S + rank)
    o = torch.empty((B, rows, H, hd), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, rows), dtype=torch.float32, device="cuda")
    tsp.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), o, lse, B, S, D, rank, H, hd, scale=RAMP_SCALE)
    torch.cuda.synchronize()
    idx = O.zigzag_index(S, D, rank)
    ref_o, ref_lse = O.causal_attention(synth.to_f64(q), idx, synth.to_f64(k), synth.to_f64(v), scale=RAMP_SCALE)
    got = host_f64(o)
    for h in range(H):
        check_close(f"o head{h}", got[:, :, h], ref_o[:, :, h])
    check_lse("lse", host_f64(lse), ref_lse)


def test_attn_scale_argument():
    B, S, D, rank, H, hd = 1, 256, 2, 1, 2, 64
    rows = S // D
    q = synth.normal_bf16((B, rows, H, hd), 7201)
    k = synth.normal_bf16((B, S, H, hd), 7202)
    v = synth.normal_bf16((B, S, H, hd), 7203)
    o = torch.empty((B, rows, H, hd), dtype=torch.bfloat16, device="cuda")
    tsp.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), o, None, B, S, D, rank, H, hd, scale=0.3)
    torch.cuda.synchronize()
    ref, _ = O.causal_attention(synth.to_f64(q), O.zigzag_index(S, D, rank), synth.to_f64(k),
                                synth.to_f64(v), scale=0.3)
    check_close("o scale=0.3", host_f64(o), ref)


def test_attn_position_zero_is_v0():
    """Rank 0's first row sits at position 0 and sees only key 0: its output is V_0
    rounded to bf16, whatever Q and K hold."""
    B, S, D, H, hd = 1, 512, 4, 2, 128
    rows = S // D
    q = synth.normal_bf16((B, rows, H, hd), 7301, 3.0)
    k = synth.normal_bf16((B, S, H, hd), 7302, 3.0)
    v = synth.normal_bf16((B, S, H, hd), 7303)
    o = torch.empty((B, rows, H, hd), dtype=torch.bfloat16, device="cuda")
    tsp.attn_fwd(dev_bf16(q), dev_bf16(k), dev_bf16(v), o, None, B, S, D, 0, H, hd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(o)[0, 0], v[0, 0])


# ------------------------------------------------------------------------------- a5 MLP
MLP_CASES = [  # M, d, Fs, ld_w2 (0 = Fs)
    (64, 256, 172, 0),       # the tiny workload's shard: odd K, 8-byte-aligned W2 rows
    (64, 256, 172, 688),     # W2 shard as a column block of the full W2
    (300, 512, 344, 0),      # ragged M and N
    (1000, 256, 1376, 0),    # the 7B shard width: K tail of 32 in the down projection
    # the large-tile kernels: gate/up 256 x 128 per weight (512 tiles), down 256 x 256 (256 tiles)
    (4096, 4096, 4096, 0),
    (4000, 4096, 4104, 0),   # ragged: M tail 160, gate/up N tail 8, down K tail 8
    # down 256 x 128 (M = 2048, N = 4096: 256 x 256 tiles would fill half the CUs)
    (2048, 4096, 1376, 0),   # the narrow persistent tile, a half stage at the end of K
    (1950, 4096, 1024, 0),   # the narrow persistent tile, ragged M (tail 158)
    (1900, 4096, 1000, 0),   # ragged: M tail 108, down K tail 40 (8-wave kernel)
]


@pytest.mark.parametrize("M,d,Fs,ld", MLP_CASES)
def test_mlp_shard_accum_parity(M, d, Fs, ld):
    print(f"mlp M={M} d={d} Fs={Fs} ld={ld}", flush=True)
    D = 2
    x = synth.normal_bf16((M, d), 7401 + Fs)
    w1 = synth.normal_bf16((D * Fs, d), 7402 + Fs, 0.02)
    w3 = synth.normal_bf16((D * Fs, d), 7403 + Fs, 0.02)
    w2 = synth.normal_bf16((d, D * Fs), 7404 + Fs, 0.02)
    xd = dev_bf16(x)
    acc = torch.full((M, d), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(tsp.mlp_workspace_size(M, Fs), dtype=torch.uint8, device="cuda")
    w2d = dev_bf16(w2)
    for j in range(D):
        w1j = dev_bf16(np.ascontiguousarray(w1[j * Fs:(j + 1) * Fs]))
        w3j = dev_bf16(np.ascontiguousarray(w3[j * Fs:(j + 1) * Fs]))
        if ld:
            w2j = w2d.view(-1)[j * Fs:].data_ptr()  # column block of the full [d, D*Fs] W2
            ldw2 = D * Fs
        else:
            w2j = dev_bf16(np.ascontiguousarray(w2[:, j * Fs:(j + 1) * Fs]))
            ldw2 = Fs
        if ld and (j * Fs * 2) % 16:
            continue  # the ABI requires 16-byte aligned shard pointers
        tsp.mlp_shard_accum(xd, w1j, w3j, w2j, ldw2, acc, M, d, Fs, j > 0, ws)
        torch.cuda.synchronize()
        parts = [O.mlp_shard_partial(synth.to_f64(x), synth.to_f64(w1), synth.to_f64(w3),
                                     synth.to_f64(w2), jj, D) for jj in range(j + 1)]
        check_close(f"acc after shard {j}", host_f64(acc), sum(parts))


def test_mlp_ring_sum_equals_unsharded():
    """D ring steps accumulated in fp32 reproduce the unsharded SwiGLU MLP."""
    M, d, D, Fs = 256, 256, 4, 96
    x = synth.normal_bf16((M, d), 7501)
    w1 = synth.normal_bf16((D * Fs, d), 7502, 0.02)
    w3 = synth.normal_bf16((D * Fs, d), 7503, 0.02)
    w2 = synth.normal_bf16((d, D * Fs), 7504, 0.02)
    acc = torch.empty((M, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(tsp.mlp_workspace_size(M, Fs), dtype=torch.uint8, device="cuda")
    xd = dev_bf16(x)
    for t in range(D):
        j = (2 - t) % D
        tsp.mlp_shard_accum(xd, dev_bf16(np.ascontiguousarray(w1[j * Fs:(j + 1) * Fs])),
                            dev_bf16(np.ascontiguousarray(w3[j * Fs:(j + 1) * Fs])),
                            dev_bf16(np.ascontiguousarray(w2[:, j * Fs:(j + 1) * Fs])), Fs, acc, M, d,
                            Fs, t > 0, ws)
    torch.cuda.synchronize()
    ref = O.swiglu_mlp(synth.to_f64(x), synth.to_f64(w1), synth.to_f64(w3), synth.to_f64(w2))
    check_close("ring sum", host_f64(acc), ref)


# ---------------------------------------------------------------------------- the layer
def run_layer(w, inputs, rank, w2_view=False):
    """Upload inputs, emulate the K/V all-gather for the peers, run tsp_layer_fwd.

    w2_view: False (W1/W3 shards are row blocks of one tensor, W2 shards contiguous
    copies), True (W2 shards are column views of the full W2, row stride F), or
    "separate" (every shard of W1/W3/W2 its own allocation, made in reverse shard order)."""
    B, S, D, H, hd, d, F = w.B, w.S, w.D, w.n_heads, w.head_dim, w.d_model, w.ffn
    Fs = F // D
    x_full = dev_bf16(inputs["x_full"])
    w_qkv, w_o = dev_bf16(inputs["w_qkv"]), dev_bf16(inputs["w_o"])
    w1, w3, w2 = dev_bf16(inputs["w1"]), dev_bf16(inputs["w3"]), dev_bf16(inputs["w2"])
    w1s = [w1[j * Fs:(j + 1) * Fs] for j in range(D)]
    w3s = [w3[j * Fs:(j + 1) * Fs] for j in range(D)]
    if w2_view == "separate":
        order = list(range(D))[::-1]
        sep = {j: (w1s[j].clone(), w3s[j].clone(), w2[:, j * Fs:(j + 1) * Fs].contiguous()) for j in order}
        w1s = [sep[j][0] for j in range(D)]
        w3s = [sep[j][1] for j in range(D)]
        w2s = [sep[j][2] for j in range(D)]
        w2_view = False
    elif w2_view:
        w2s = [w2.view(-1)[j * Fs:].data_ptr() for j in range(D)]
    else:
        w2s = [w2[:, j * Fs:(j + 1) * Fs].contiguous() for j in range(D)]
    kf, vf = nan_bf16((B, S, d)), nan_bf16((B, S, d))
    fill_peer_kv(x_full, w_qkv, kf, vf, B, S, D, rank, H, hd)
    xs = shard_rows(x_full, S, D, rank)
    desc = tsp.make_desc(B, S, D, rank, d, H, hd, F, w2_ld=F if w2_view else 0)
    ws = torch.empty(tsp.layer_workspace_size(desc), dtype=torch.uint8, device="cuda")
    a = torch.empty((B, S // D, d), dtype=torch.bfloat16, device="cuda")
    y = torch.full((B, S // D, d), float("nan"), dtype=torch.float32, device="cuda")
    tsp.layer_fwd(desc, xs, w_qkv, w_o, w1s, w3s, w2s, kf, vf, a, y, ws)
    torch.cuda.synchronize()
    return a, y, kf, vf


def test_layer_tiny_all_ranks():
    """The tiny workload (S=256, D=4, d=256, 4x64 heads, F=688): every rank, and the four
    ranks' outputs glued in position order equal the unsharded layer."""
    w = synth.WORKLOADS["tiny_s256_d4"]
    inputs = synth.layer_inputs(w)
    f64 = {k: synth.to_f64(v) for k, v in inputs.items()}
    full = O.rank_layer(f64["x_full"], f64["w_qkv"], f64["w_o"], f64["w1"], f64["w3"], f64["w2"],
                        w.S, 1, 0, w.n_heads)
    glued_a = np.zeros_like(full["attn_out"])
    glued_y = np.zeros_like(full["mlp_out"])
    for r in range(w.D):
        print(f"layer tiny rank {r}", flush=True)
        a, y, kf, vf = run_layer(w, inputs, r)
        ref = O.rank_layer(f64["x_full"], f64["w_qkv"], f64["w_o"], f64["w1"], f64["w3"], f64["w2"],
                           w.S, w.D, r, w.n_heads)
        check_close(f"attn_out r{r}", host_f64(a), ref["attn_out"])
        check_close(f"mlp_out r{r}", host_f64(y), ref["mlp_out"])
        idx = ref["idx"]
        assert np.all(np.isfinite(host_f64(kf)[:, idx])) and np.all(np.isfinite(host_f64(vf)[:, idx]))
        glued_a[:, idx] = host_f64(a)
        glued_y[:, idx] = host_f64(y)
    check_close("glued attn_out", glued_a, full["attn_out"])
    check_close("glued mlp_out", glued_y, full["mlp_out"])


# Fs % 8 == 0 takes the two-launch MLP ring (gated hidden of all shards, then one down
# projection over the shards in ring order); the tiny workload (Fs = 172) takes the
# per-shard steps.
LAYER_MID = [  # B, S, D, rank, H, hd, F, w2_view
    (2, 2048, 4, 1, 4, 128, 1376, False),     # Fs = 344: 24-column k tail in every shard
    (1, 1200, 3, 2, 4, 64, 1032, True),       # C = 200, Fs = 344, W2 shards as views
    (1, 512, 8, 5, 8, 64, 2304, False),       # D = 8, ring wraps at rank 5, Fs = 288
    (1, 768, 2, 1, 4, 64, 1040, "separate"),  # Fs = 520, shards in separate allocations
    (1, 256, 4, 2, 4, 64, 696, False),        # Fs = 174: per-shard steps (Fs % 8 != 0)
    # at most one query tile per CU: the later chunk's tiles run as two key halves beside the
    # earlier chunk's whole tiles, in one launch
    (1, 4096, 4, 0, 4, 64, 1024, False),      # split at D C + 128 = 2176; heads do not divide over 8 XCDs
    (1, 4096, 4, 2, 4, 64, 2048, False),      # split at 2176
    (1, 1024, 1, 0, 2, 128, 1024, False),     # D = 1: split at the chunk boundary (position C)
    (1, 2048, 4, 1, 8, 64, 1024, False),      # one head per XCD, split at 1152
    (1, 2048, 4, 3, 8, 128, 2048, False),     # one head per XCD, split at the later chunk's start 1024
]


@pytest.mark.parametrize("B,S,D,rank,H,hd,F,w2_view", LAYER_MID)
def test_layer_mid(B, S, D, rank, H, hd, F, w2_view):
    print(f"layer B={B} S={S} D={D} rank={rank} H={H} hd={hd} F={F} view={w2_view}", flush=True)
    w = synth.Workload(90 + S % 7, "mid", B, S, D, rank, H * hd, H, hd, F)
    inputs = synth.layer_inputs(w)
    a, y, _, _ = run_layer(w, inputs, rank, w2_view=w2_view)
    f64 = {k: synth.to_f64(v) for k, v in inputs.items()}
    ref = O.rank_layer(f64["x_full"], f64["w_qkv"], f64["w_o"], f64["w1"], f64["w3"], f64["w2"],
                       S, D, rank, H)
    check_close("attn_out", host_f64(a), ref["attn_out"])
    check_close("mlp_out", host_f64(y), ref["mlp_out"])


def test_empty_problems_on_device():
    """B = 0 with empty device tensors: every entry point returns OK and writes nothing."""
    e = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    tsp.attn_fwd(e, e, e, e, None, 0, 256, 4, 1, 4, 64)
    tsp.qkv_fwd(e, e, None, e, e, 0, 256, 4, 1, 4, 64)
    sentinel = torch.full((4, 8), 7.0, device="cuda")
    tsp.mlp_shard_accum(e, e, e, e, 172, sentinel, 0, 256, 172, 0, torch.empty(0, device="cuda"))
    desc = tsp.make_desc(0, 256, 4, 1, 256, 4, 64, 688)
    assert tsp.layer_workspace_size(desc) == 0
    tsp.layer_fwd(desc, e, e, e, [e] * 4, [e] * 4, [e] * 4, e, e, e,
                  torch.empty(0, device="cuda"), torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(sentinel == 7.0)


def test_phase_timing_hook():
    """The library's phase events: armed for 2 calls, 3 calls made, 2 read back, every
    phase positive; disarmed afterwards (a further read returns nothing)."""
    w = synth.WORKLOADS["tiny_s256_d4"]
    inputs = synth.layer_inputs(w)
    run_layer(w, inputs, 1)
    tsp.timing_start(2)
    for _ in range(3):
        run_layer(w, inputs, 1)
    calls = tsp.timing_read(2)
    assert len(calls) == 2
    assert all(c[p] > 0 for c in calls for p in tsp.PHASES), calls
    assert tsp.timing_read(2) == []


def test_layer_deterministic():
    w = synth.WORKLOADS["tiny_s256_d4"]
    inputs = synth.layer_inputs(w)
    a1, y1, _, _ = run_layer(w, inputs, 2)
    a2, y2, _, _ = run_layer(w, inputs, 2)
    assert torch.equal(a1, a2) and torch.equal(y1, y2)
