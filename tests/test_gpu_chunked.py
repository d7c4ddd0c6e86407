"""GPU parity of chunked-arrival attention: attention over a key range (tsp_attn_fwd_range)
and the log-sum-exp merge of partial attentions (tsp_attn_merge), against the fp64 oracle.

The all-gather of K/V delivers the sequence chunk by chunk; attention over each arrived
chunk, merged by log-sum-exp, must equal attention over the whole sequence (summary of
"Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer Training &
Inference", gist.science 2604.26294, §2 attention layers, §3 implementation and overlap).
Tolerance: the contract's max-abs <= 2e-2 max|ref|, mean-abs <= 2e-3 max|ref| per tensor
(per (chunk, head) at full size); rows that see no key of a range must be exactly
(0, -inf).
"""

import numpy as np
import pytest
import torch

from long_context_transformer_amd import synth, tsp
from oracle import tsp_oracle as O

from _gpu_helpers import RAMP_SCALE, check_close, check_lse, dev_bf16, host_f64, ramp_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsp.load()


def qkv_inputs(B, S, D, H, hd, seed):
    R = S // D
    q = synth.normal_bf16((B, R, H, hd), seed, std=1.0)
    k = synth.normal_bf16((B, S, H, hd), seed + 1, std=1.0)
    v = synth.normal_bf16((B, S, H, hd), seed + 2, std=1.0)
    return q, k, v


def arrival_order(D, r):
    """All-gather arrival order of the 2D chunks: the rank's own two chunks, then the
    chunk pairs of ranks r-1, r-2, ... around the ring."""
    order = [r, 2 * D - 1 - r]
    for t in range(1, D):
        p = (r - t) % D
        order += [p, 2 * D - 1 - p]
    return order


def run_range(qd, kd, vd, B, S, D, r, H, hd, lo, hi):
    R = S // D
    o = torch.full((B, R, H, hd), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, H, R), float("nan"), dtype=torch.float32, device="cuda")
    tsp.attn_fwd_range(qd, kd, vd, o, lse, B, S, D, r, H, hd, lo, hi)
    return o, lse


def nan_outside(t, lo, hi):
    """Copy of a [B, S, H, hd] bf16 K or V buffer whose rows outside [lo, hi) are NaN: the
    chunks the all-gather has not delivered yet may hold anything."""
    out = torch.full_like(t, float("nan"))
    out[:, lo:hi] = t[:, lo:hi]
    return out


def check_range(name, o, lse, ref_o, ref_lse):
    o_h = o.cpu().numpy().astype(np.float64)
    l_h = lse.cpu().numpy().astype(np.float64)
    empty = ~np.isfinite(ref_lse)  # [B, H, n]
    assert np.array_equal(~np.isfinite(l_h), empty), f"{name}: rows without keys differ"
    assert np.all(l_h[empty] == -np.inf)
    rows_empty = np.transpose(empty, (0, 2, 1))  # [B, n, H]
    assert np.all(o_h[rows_empty] == 0.0), f"{name}: O of rows without keys is not 0"
    if np.any(~empty):
        check_close(f"{name} O", o_h[~rows_empty], ref_o[~rows_empty])
        check_lse(f"{name} lse", l_h[~empty], ref_lse[~empty])


RAMP_RANGE_CASES = [  # B, S, D, rank, H, hd, ranges
    (1, 2048, 2, 1, 4, 128, [(0, 2048), (700, 1500), (1500, 2048), (33, 1000)]),
    (1, 1200, 3, 2, 4, 64, [(100, 900), (0, 1200)]),
]


@pytest.mark.parametrize("B,S,D,rank,H,hd,ranges", RAMP_RANGE_CASES)
def test_attn_range_reference_moves(B, S, D, rank, H, hd, ranges):
    """Key ranges over scores that climb, creep, fall or wander along the keys (see
    ramp_inputs): rows that see no key of the range until late, or at all, next to rows
    whose reference moves at every block."""
    print(f"range attention, reference moves B={B} S={S} D={D} rank={rank} H={H} hd={hd}", flush=True)
    R = S // D
    q, k, v = ramp_inputs(B, S, R, H, hd, 7400 + S + rank)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    idx = O.zigzag_index(S, D, rank)
    for lo, hi in ranges:
        o = torch.full((B, R, H, hd), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, H, R), float("nan"), dtype=torch.float32, device="cuda")
        tsp.attn_fwd_range(qd, nan_outside(kd, lo, hi), nan_outside(vd, lo, hi), o, lse, B, S, D, rank, H, hd,
                           lo, hi, scale=RAMP_SCALE)
        torch.cuda.synchronize()
        ref_o, ref_lse = O.attention_range(synth.to_f64(q), idx, synth.to_f64(k), synth.to_f64(v), lo, hi,
                                           scale=RAMP_SCALE)
        check_range(f"[{lo},{hi})", o, lse, ref_o, ref_lse)


RANGE_CASES = [  # B, S, D, rank, H, hd, ranges
    (1, 256, 4, 0, 4, 64, [(0, 256), (0, 32), (224, 256), (64, 128), (5, 71), (100, 101), (0, 0), (250, 256)]),
    (2, 1200, 3, 1, 3, 128, [(0, 1200), (200, 400), (333, 777), (1000, 1200), (0, 64), (1199, 1200)]),
    (1, 4096, 2, 1, 2, 128, [(1024, 2048), (0, 3000), (2047, 2049), (3072, 4096)]),
]


@pytest.mark.parametrize("B,S,D,rank,H,hd,ranges", RANGE_CASES)
def test_attn_range_parity(B, S, D, rank, H, hd, ranges):
    print(f"range attention B={B} S={S} D={D} rank={rank} H={H} hd={hd}", flush=True)
    q, k, v = qkv_inputs(B, S, D, H, hd, 300 + S % 97)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    idx = O.zigzag_index(S, D, rank)
    qf, kf, vf = synth.to_f64(q), synth.to_f64(k), synth.to_f64(v)
    for lo, hi in ranges:
        # K/V rows outside the range are NaN: the kernel must read only [lo, hi)
        o, lse = run_range(qd, nan_outside(kd, lo, hi), nan_outside(vd, lo, hi), B, S, D, rank, H, hd, lo, hi)
        torch.cuda.synchronize()
        ref_o, ref_lse = O.attention_range(qf, idx, kf, vf, lo, hi)
        check_range(f"[{lo},{hi})", o, lse, ref_o, ref_lse)
    # o_out without accumulation: the bf16 of the range's own O, for every row
    lo, hi = ranges[-1]
    o2 = torch.empty((B, S // D, H, hd), dtype=torch.float32, device="cuda")
    l2 = torch.empty((B, H, S // D), dtype=torch.float32, device="cuda")
    ob = torch.full((B, S // D, H, hd), float("nan"), dtype=torch.bfloat16, device="cuda")
    tsp.attn_fwd_range(qd, kd, vd, o2, l2, B, S, D, rank, H, hd, lo, hi, o_out=ob)
    torch.cuda.synchronize()
    assert torch.equal(ob, o2.to(torch.bfloat16))


def test_merge_parity():
    """The merge kernel against the oracle's lse_merge, with rows of -inf on either side."""
    B, S, D, H, hd = 2, 256, 4, 3, 128
    R = S // D
    rng = np.random.default_rng(41)
    oa = rng.standard_normal((B, R, H, hd)).astype(np.float32)
    ob = rng.standard_normal((B, R, H, hd)).astype(np.float32)
    la = (rng.standard_normal((B, H, R)) * 3).astype(np.float32)
    lb = (rng.standard_normal((B, H, R)) * 3).astype(np.float32)
    la[0, 0, :5] = -np.inf
    oa[0, :5, 0] = 0
    lb[1, 2, 7:12] = -np.inf
    ob[1, 7:12, 2] = 0
    la[0, 1, 20:23] = lb[0, 1, 20:23] = -np.inf
    oa[0, 20:23, 1] = ob[0, 20:23, 1] = 0
    d = lambda x: torch.from_numpy(x).cuda()
    o_acc, l_acc = d(oa.copy()), d(la.copy())
    out = torch.empty((B, R, H, hd), dtype=torch.bfloat16, device="cuda")
    tsp.attn_merge(o_acc, l_acc, d(ob), d(lb), out, B, S, D, H, hd)
    torch.cuda.synchronize()
    ref_o, ref_l = O.lse_merge(oa, la, ob, lb)
    got_l = l_acc.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isfinite(got_l), np.isfinite(ref_l))
    fin = np.isfinite(ref_l)
    np.testing.assert_allclose(got_l[fin], ref_l[fin], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(o_acc.cpu().numpy(), ref_o, rtol=1e-5, atol=1e-5)
    check_close("merged bf16 O", host_f64(out), ref_o)


def test_range_accumulate_leaves_earlier_rows():
    """Merging one key range into the accumulator: rows whose position precedes the range are
    left bit-for-bit as they were (whole query tiles of them are not launched at all), and the
    other rows equal the oracle's log-sum-exp merge of the accumulator with the range."""
    B, S, D, r, H, hd = 1, 4096, 2, 1, 2, 128  # C = 1024, 8 query tiles of 256 rows
    R = S // D
    q, k, v = qkv_inputs(B, S, D, H, hd, 977)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    idx = O.zigzag_index(S, D, r)
    qf, kf, vf = synth.to_f64(q), synth.to_f64(k), synth.to_f64(v)
    rng = np.random.default_rng(43)
    oa = rng.standard_normal((B, R, H, hd)).astype(np.float32)
    la = (rng.standard_normal((B, H, R)) * 3).astype(np.float32)
    d = lambda x: torch.from_numpy(x).cuda()
    # (first key past four whole tiles and inside the fifth, a single key, the last position
    # only, a range that starts inside the second tile)
    for lo, hi in [(2100, 3000), (2048, 2049), (3071, 4096), (1500, 2600)]:
        print(f"accumulate range [{lo},{hi})", flush=True)
        acc_o, acc_l = d(oa.copy()), d(la.copy())
        tsp.attn_fwd_range(qd, kd, vd, acc_o, acc_l, B, S, D, r, H, hd, lo, hi, accumulate=True)
        torch.cuda.synchronize()
        got_o, got_l = acc_o.cpu().numpy(), acc_l.cpu().numpy()
        before = idx < lo
        assert np.array_equal(got_o[:, before], oa[:, before]), f"[{lo},{hi}): O of earlier rows changed"
        assert np.array_equal(got_l[:, :, before], la[:, :, before]), f"[{lo},{hi}): lse of earlier rows changed"
        part_o, part_l = O.attention_range(qf, idx, kf, vf, lo, hi)
        ref_o, ref_l = O.lse_merge(oa, la, part_o, part_l)
        after = ~before
        check_lse(f"[{lo},{hi}) merged lse", got_l[:, :, after], ref_l[:, :, after])
        check_close(f"[{lo},{hi}) merged O", got_o[:, after].astype(np.float64), ref_o[:, after])


PIPE_CASES = [  # B, S, D, rank, H, hd
    (1, 256, 4, 2, 4, 64),
    (2, 2048, 4, 0, 2, 128),
    (1, 1200, 3, 1, 3, 128),
]


def chunked_attention(qd, kd, vd, B, S, D, r, H, hd, bounds, fused=True):
    """Attention per arrived chunk merged into an fp32 accumulator, bf16 O at the end:
    fused (each range launch merges into the accumulator itself) or as range launches
    followed by merge launches."""
    R = S // D
    acc_o = torch.zeros((B, R, H, hd), dtype=torch.float32, device="cuda")
    acc_l = torch.full((B, H, R), float("-inf"), dtype=torch.float32, device="cuda")
    out = torch.full((B, R, H, hd), float("nan"), dtype=torch.bfloat16, device="cuda")
    po = torch.empty_like(acc_o)
    pl = torch.empty_like(acc_l)
    for n, (lo, hi) in enumerate(bounds):
        last = out if n == len(bounds) - 1 else None
        if fused:
            tsp.attn_fwd_range(qd, kd, vd, acc_o, acc_l, B, S, D, r, H, hd, lo, hi, accumulate=True, o_out=last)
        else:
            tsp.attn_fwd_range(qd, kd, vd, po, pl, B, S, D, r, H, hd, lo, hi)
            tsp.attn_merge(acc_o, acc_l, po, pl, last, B, S, D, H, hd)
    return out, acc_l


@pytest.mark.parametrize("B,S,D,rank,H,hd", PIPE_CASES)
def test_chunked_pipeline(B, S, D, rank, H, hd):
    """The 2D zigzag chunks in all-gather arrival order, merged, equal full causal attention
    (oracle) and the single-launch kernel; so does an unaligned split in reverse order."""
    print(f"chunked pipeline B={B} S={S} D={D} rank={rank} H={H} hd={hd}", flush=True)
    q, k, v = qkv_inputs(B, S, D, H, hd, 500 + S % 89)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    idx = O.zigzag_index(S, D, rank)
    ref_o, ref_lse = O.causal_attention(synth.to_f64(q), idx, synth.to_f64(k), synth.to_f64(v))
    C = S // (2 * D)
    splits = {"arrival": [(c * C, (c + 1) * C) for c in arrival_order(D, rank)],
              "unaligned": [(S - S // 3, S), (37, S - S // 3), (0, 37)]}
    mono = torch.empty((B, S // D, H, hd), dtype=torch.bfloat16, device="cuda")
    tsp.attn_fwd(qd, kd, vd, mono, None, B, S, D, rank, H, hd)
    for name, bounds in splits.items():
        for fused in (True, False):
            tag = f"{name} {'fused' if fused else 'range+merge'}"
            out, lse = chunked_attention(qd, kd, vd, B, S, D, rank, H, hd, bounds, fused=fused)
            torch.cuda.synchronize()
            check_close(f"{tag} O vs oracle", host_f64(out), ref_o)
            check_lse(f"{tag} lse vs oracle", lse.cpu().numpy().astype(np.float64), ref_lse)
            check_close(f"{tag} O vs single launch", host_f64(out), host_f64(mono))


ARRIVAL_CASES = [  # B, S, D, rank, H, hd: C = 32 (half the chunk starts off the 64-key stage) and C = 200
    (1, 256, 4, 0, 4, 64),
    (1, 256, 4, 1, 4, 64),
    (1, 256, 4, 2, 4, 64),
    (1, 256, 4, 3, 4, 64),
    (2, 1200, 3, 1, 3, 128),
    (1, 1200, 3, 2, 2, 64),
]


@pytest.mark.parametrize("B,S,D,rank,H,hd", ARRIVAL_CASES)
def test_chunked_pipeline_as_delivered(B, S, D, rank, H, hd):
    """K/V as the all-gather delivers it: every row starts as NaN and each chunk's rows are
    written just before its range launch, in arrival order. A range launch that read a row
    of a chunk still to come would carry NaN into the accumulator (a masked score gives
    P = 0, but 0 * NaN is NaN), so a finite result that matches the oracle shows that each
    launch reads only its own chunk."""
    print(f"chunked pipeline as delivered B={B} S={S} D={D} rank={rank} H={H} hd={hd}", flush=True)
    q, k, v = qkv_inputs(B, S, D, H, hd, 600 + S % 83 + rank)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    idx = O.zigzag_index(S, D, rank)
    ref_o, ref_lse = O.causal_attention(synth.to_f64(q), idx, synth.to_f64(k), synth.to_f64(v))
    C = S // (2 * D)
    R = S // D
    for fused in (True, False):
        kbuf, vbuf = torch.full_like(kd, float("nan")), torch.full_like(vd, float("nan"))
        acc_o = torch.zeros((B, R, H, hd), dtype=torch.float32, device="cuda")
        acc_l = torch.full((B, H, R), float("-inf"), dtype=torch.float32, device="cuda")
        out = torch.full((B, R, H, hd), float("nan"), dtype=torch.bfloat16, device="cuda")
        po, pl = torch.empty_like(acc_o), torch.empty_like(acc_l)
        order = arrival_order(D, rank)
        for n, c in enumerate(order):
            lo, hi = c * C, (c + 1) * C
            kbuf[:, lo:hi] = kd[:, lo:hi]  # this chunk arrives (same stream as the launches)
            vbuf[:, lo:hi] = vd[:, lo:hi]
            last = out if n == len(order) - 1 else None
            if fused:
                tsp.attn_fwd_range(qd, kbuf, vbuf, acc_o, acc_l, B, S, D, rank, H, hd, lo, hi, accumulate=True,
                                   o_out=last)
            else:
                tsp.attn_fwd_range(qd, kbuf, vbuf, po, pl, B, S, D, rank, H, hd, lo, hi)
                tsp.attn_merge(acc_o, acc_l, po, pl, last, B, S, D, H, hd)
        torch.cuda.synchronize()
        tag = "fused" if fused else "range+merge"
        assert bool(torch.isfinite(acc_o).all()), f"{tag}: non-finite accumulator"
        check_close(f"{tag} O vs oracle", host_f64(out), ref_o)
        check_lse(f"{tag} lse vs oracle", acc_l.cpu().numpy().astype(np.float64), ref_lse)


@pytest.mark.parametrize("name,rank", [("7b_s128k_d8", 0), ("7b_s32k_d8", 5)])
def test_chunked_pipeline_fullsize(name, rank):
    """Full size: the 16 zigzag chunks in arrival order, sampled rows checked per (chunk, head)."""
    w = synth.WORKLOADS[name].with_rank(rank)
    B, S, D, H, hd, C = w.B, w.S, w.D, w.n_heads, w.head_dim, w.C
    print(f"full-size chunked pipeline {name} rank {rank}", flush=True)
    std = float(np.sqrt(4096) * 0.02)
    q = synth.normal_bf16((B, S // D, H, hd), 8200 + rank, std=std)
    k = synth.normal_bf16((B, S, H, hd), 8201, std=std)
    v = synth.normal_bf16((B, S, H, hd), 8202, std=1.0)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    out, _ = chunked_attention(qd, kd, vd, B, S, D, rank, H, hd,
                               [(c * C, (c + 1) * C) for c in arrival_order(D, rank)])
    torch.cuda.synchronize()
    o_h = host_f64(out)
    del qd, kd, vd
    idx = O.zigzag_index(S, D, rank)
    rng = np.random.default_rng(8300 + rank)
    rows = np.unique(np.concatenate([[0, C - 1, C, 2 * C - 1], rng.choice(2 * C, 12, replace=False)]))
    kmax = int(idx[rows].max()) + 1
    ref_o, _ = O.causal_attention(synth.to_f64(q[:, rows]), idx[rows], synth.to_f64(k[:, :kmax]),
                                  synth.to_f64(v[:, :kmax]))
    for chunk, sel in (("early", rows < C), ("mirror", rows >= C)):
        for h in range(H):
            check_close(f"{chunk} h{h}", o_h[0, rows[sel], h], ref_o[0, sel, h])
