"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Method source: summary of "Folding Tensor and Sequence Parallelism for Memory-Efficient
Transformer Training & Inference" (gist.science 2604.26294), §2 (unified sharding,
zigzag partitioning, all-gathered K/V + FlashAttention, gated-MLP ring with local
accumulation and no all-reduce). The pages print no numeric example, so the pins are:
closed forms, invariants the method states, special cases that reduce to textbook or
library routines, and a scalar-loop brute force on tiny inputs. The last test plants
plausible mistakes in the oracle and checks that some pin catches each one.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import tsp_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _read_ranges(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split("-")
            out.extend(range(int(a), int(b) + 1))
    return np.array(out, dtype=np.int64)


# ----------------------------------------------------------------------------- pins
# Each pin is a plain function that raises AssertionError on failure, so the planted
# mistake test at the end can run all of them against a broken oracle.

def pin_zigzag_golden():
    """S=256, D=4, rank 0 -> chunks 0 and 7 (hand-written fixture)."""
    np.testing.assert_array_equal(O.zigzag_index(256, 4, 0), _read_ranges("zigzag_s256_d4_r0.txt"))


def pin_zigzag_partition():
    """Over all ranks the maps partition 0..S-1; each map ascends and has S/D rows."""
    for S, D in [(256, 4), (48, 3), (16384, 8), (16, 1), (40, 5)]:
        seen = np.zeros(S, dtype=np.int64)
        for r in range(D):
            idx = O.zigzag_index(S, D, r)
            assert idx.shape == (S // D,)
            assert np.all(np.diff(idx) > 0)
            seen[idx] += 1
        assert np.all(seen == 1), (S, D)


def pin_zigzag_balance():
    """Every rank sees exactly C(S+1) causal (query, key) pairs: sum of (pos+1).

    Chunk r contributes C(rC) + C(C+1)/2 and chunk 2D-1-r contributes
    C(2D-1-r)C + C(C+1)/2, which add to C(2DC + C... ) = C(S+1) for every r; a
    contiguous split instead grows linearly with r.
    """
    for S, D in [(256, 4), (131072, 8), (48, 3)]:
        C = S // (2 * D)
        for r in range(D):
            assert int((O.zigzag_index(S, D, r) + 1).sum()) == C * (S + 1), (S, D, r)


def pin_zigzag_identity():
    np.testing.assert_array_equal(O.zigzag_index(64, 1, 0), np.arange(64))


def pin_attention_vs_brute():
    """Oracle attention equals scalar loops on a tiny input, for every rank of a fold."""
    rng = _rng(11)
    B, S, H, hd, D = 1, 16, 2, 4, 2
    k = rng.standard_normal((B, S, H, hd))
    v = rng.standard_normal((B, S, H, hd))
    for r in range(D):
        pos = brute.zigzag_positions(S, D, r)
        q = rng.standard_normal((B, len(pos), H, hd))
        o, lse = O.causal_attention(q, O.zigzag_index(S, D, r), k, v)
        for i, p in enumerate(pos):
            for h in range(H):
                ob, lb = brute.attention_row(list(q[0, i, h]), p, k[0, :, h].tolist(),
                                             v[0, :, h].tolist(), 1.0 / math.sqrt(hd))
                np.testing.assert_allclose(o[0, i, h], ob, rtol=1e-12, atol=1e-12)
                assert abs(lse[0, h, i] - lb) < 1e-12


def _sdpa(q, k, v, scale=None):
    """torch's fp64 CPU causal SDPA on [B, S, H, hd] tensors (a library routine)."""
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def pin_attention_vs_library():
    """D = 1 is textbook causal attention: torch SDPA in fp64 on the CPU."""
    rng = _rng(12)
    B, S, H, hd = 2, 96, 3, 16
    q, k, v = (rng.standard_normal((B, S, H, hd)) for _ in range(3))
    o, _ = O.causal_attention(q, O.zigzag_index(S, 1, 0), k, v, row_block=40)
    np.testing.assert_allclose(o, _sdpa(q, k, v), rtol=1e-10, atol=1e-12)


def pin_attention_concat_ranks():
    """All D ranks' outputs, put back in position order, equal full causal attention."""
    rng = _rng(13)
    B, S, H, hd, D = 2, 64, 2, 8, 4
    q, k, v = (rng.standard_normal((B, S, H, hd)) for _ in range(3))
    full = _sdpa(q, k, v)
    glued = np.zeros_like(full)
    for r in range(D):
        idx = O.zigzag_index(S, D, r)
        o, _ = O.causal_attention(q[:, idx], idx, k, v)
        glued[:, idx] = o
    np.testing.assert_allclose(glued, full, rtol=1e-10, atol=1e-12)


def pin_attention_special_cases():
    """Rows sum to one; constant V; zero keys give the prefix mean; position 0 gives V_0."""
    rng = _rng(14)
    B, S, H, hd, D, r = 1, 48, 2, 8, 3, 1
    idx = O.zigzag_index(S, D, r)
    q = rng.standard_normal((B, len(idx), H, hd))
    k = rng.standard_normal((B, S, H, hd))
    ones = np.ones((B, S, H, hd))
    o, _ = O.causal_attention(q, idx, k, ones)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-13)
    c = rng.standard_normal(hd)
    o, _ = O.causal_attention(q, idx, k, np.broadcast_to(c, (B, S, H, hd)))
    np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-13)
    v = rng.standard_normal((B, S, H, hd))
    o, lse = O.causal_attention(q, idx, np.zeros((B, S, H, hd)), v)
    for i, p in enumerate(idx):
        np.testing.assert_allclose(o[0, i], v[0, :p + 1].mean(axis=0), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[0, :, i], math.log(p + 1), rtol=1e-13)
    idx0 = O.zigzag_index(S, D, 0)
    o, _ = O.causal_attention(q, idx0, k, v)
    assert idx0[0] == 0
    np.testing.assert_array_equal(o[0, 0], v[0, 0])


def pin_attention_scale():
    """The default scale is 1/sqrt(hd): doubling q equals scale 2/sqrt(hd) (SDPA agrees)."""
    rng = _rng(15)
    B, S, H, hd = 1, 32, 1, 16
    q, k, v = (rng.standard_normal((B, S, H, hd)) for _ in range(3))
    o, _ = O.causal_attention(q, np.arange(S), k, v)
    np.testing.assert_allclose(o, _sdpa(q, k, v, scale=1.0 / math.sqrt(hd)), rtol=1e-10, atol=1e-12)
    o2, _ = O.causal_attention(2 * q, np.arange(S), k, v)
    np.testing.assert_allclose(o2, _sdpa(q, k, v, scale=2.0 / math.sqrt(hd)), rtol=1e-10, atol=1e-12)


def pin_silu_closed_form():
    """silu(0)=0, silu(1)=e/(1+e), silu(-1)=-1/(1+e), silu(x)->x for large x."""
    e = math.e
    got = O.silu(np.array([0.0, 1.0, -1.0, 40.0, -40.0]))
    want = np.array([0.0, e / (1 + e), -1 / (1 + e), 40.0, -40.0 * math.exp(-40.0)])
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-300)


def pin_mlp_vs_brute():
    rng = _rng(16)
    d, F = 6, 10
    x = rng.standard_normal((3, d))
    w1, w3 = rng.standard_normal((F, d)), rng.standard_normal((F, d))
    w2 = rng.standard_normal((d, F))
    y = O.swiglu_mlp(x, w1, w3, w2)
    for i in range(3):
        np.testing.assert_allclose(y[i], brute.mlp_row(list(x[i]), w1.tolist(), w3.tolist(), w2.tolist()),
                                   rtol=1e-12, atol=1e-12)


def pin_mlp_shards_sum():
    """Summing the D ffn-shard partials gives the unsharded MLP (no all-reduce needed)."""
    rng = _rng(17)
    d, F = 8, 24
    x = rng.standard_normal((5, d))
    w1, w3 = rng.standard_normal((F, d)), rng.standard_normal((F, d))
    w2 = rng.standard_normal((d, F))
    full = O.swiglu_mlp(x, w1, w3, w2)
    for D in (1, 2, 3, 4, 8):
        parts = [O.mlp_shard_partial(x, w1, w3, w2, j, D) for j in range(D)]
        np.testing.assert_allclose(sum(parts), full, rtol=1e-12, atol=1e-12)
        # a single shard is not the whole (unless D = 1)
        if D > 1:
            assert np.abs(parts[0] - full).max() > 1e-6
    np.testing.assert_array_equal(O.swiglu_mlp(np.zeros((2, d)), w1, w3, w2), 0.0)


def _tiny_layer(seed, S=16, D=2, d=8, H=2, F=12):
    rng = _rng(seed)
    x = rng.standard_normal((1, S, d))
    w_qkv = rng.standard_normal((3 * d, d)) * 0.3
    w_o = rng.standard_normal((d, d)) * 0.3
    w1, w3 = rng.standard_normal((F, d)) * 0.3, rng.standard_normal((F, d)) * 0.3
    w2 = rng.standard_normal((d, F)) * 0.3
    return x, w_qkv, w_o, w1, w3, w2


def pin_layer_vs_brute():
    S, D, H = 16, 2, 2
    x, w_qkv, w_o, w1, w3, w2 = _tiny_layer(18, S=S, D=D, H=H)
    for r in range(D):
        got = O.rank_layer(x, w_qkv, w_o, w1, w3, w2, S, D, r, H)
        want = brute.rank_layer(x[0].tolist(), w_qkv.tolist(), w_o.tolist(), w1.tolist(),
                                w3.tolist(), w2.tolist(), S, D, r, H)
        np.testing.assert_array_equal(got["pos"], want["pos"])
        np.testing.assert_allclose(got["o"][0], np.array(want["o"]), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(got["attn_out"][0], np.array(want["attn_out"]), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(got["mlp_out"][0], np.array(want["mlp_out"]), rtol=1e-11, atol=1e-12)


def pin_layer_concat_ranks():
    """Every rank's layer rows, glued in position order, equal the unsharded layer."""
    S, D, H = 32, 4, 2
    x, w_qkv, w_o, w1, w3, w2 = _tiny_layer(19, S=S, D=D, H=H)
    full = O.rank_layer(x, w_qkv, w_o, w1, w3, w2, S, 1, 0, H)
    glued = np.zeros_like(full["mlp_out"])
    for r in range(D):
        got = O.rank_layer(x, w_qkv, w_o, w1, w3, w2, S, D, r, H)
        glued[:, got["idx"]] = got["mlp_out"]
    np.testing.assert_allclose(glued, full["mlp_out"], rtol=1e-11, atol=1e-12)


def pin_layer_rows_subset():
    """Evaluating a subset of rows gives the same values as the full shard at those rows."""
    S, D, H = 32, 2, 2
    x, w_qkv, w_o, w1, w3, w2 = _tiny_layer(20, S=S, D=D, H=H)
    full = O.rank_layer(x, w_qkv, w_o, w1, w3, w2, S, D, 1, H)
    rows = np.array([0, 3, 9, 15])
    sub = O.rank_layer(x, w_qkv, w_o, w1, w3, w2, S, D, 1, H, rows=rows)
    np.testing.assert_allclose(sub["mlp_out"], full["mlp_out"][:, rows], rtol=1e-12, atol=1e-13)


def pin_layer_flops():
    """Closed-form FLOPs equal an explicit count over causal pairs and GEMM shapes."""
    for (B, S, D, d, H, hd, F) in [(1, 256, 4, 256, 4, 64, 688), (2, 48, 3, 16, 2, 8, 12)]:
        pairs = 0
        for r in [0]:
            pairs = sum(p + 1 for p in brute.zigzag_positions(S, D, r))
        M = B * S // D
        count = 2 * M * d * 3 * d + B * H * pairs * 2 * hd * 2 + 2 * M * d * d + 3 * 2 * M * d * F
        assert O.layer_flops(B, S, D, d, H, hd, F) == count
    assert O.layer_flops(1, 256, 4, 256, 4, 64, 688) == 109_608_960


def pin_range_vs_brute():
    """Attention over a key range equals the scalar-loop brute force: ranges that start and
    end inside a block, cut through the query rows, or leave rows with no key at all."""
    rng = _rng(21)
    B, S, H, hd, D, r = 1, 40, 2, 8, 2, 1
    idx = O.zigzag_index(S, D, r)
    q = rng.standard_normal((B, len(idx), H, hd))
    k = rng.standard_normal((B, S, H, hd))
    v = rng.standard_normal((B, S, H, hd))
    scale = 1.0 / math.sqrt(hd)
    for lo, hi in [(0, S), (3, 17), (11, 12), (25, 40), (35, 36), (0, 0), (38, 60)]:
        o, lse = O.attention_range(q, idx, k, v, lo, hi, row_block=7)
        for i, p in enumerate(idx):
            for h in range(H):
                ob, lb = brute.attention_row_range(q[0, i, h].tolist(), int(p), k[0, :, h].tolist(),
                                                   v[0, :, h].tolist(), scale, lo, hi)
                np.testing.assert_allclose(o[0, i, h], ob, rtol=1e-12, atol=1e-13)
                if math.isinf(lb):
                    assert lse[0, h, i] == -np.inf
                else:
                    np.testing.assert_allclose(lse[0, h, i], lb, rtol=1e-12)


def pin_range_merge_equals_full():
    """Key chunks merged in all-gather arrival order (the rank's own chunks first, then the
    others around the ring) give full causal attention; so does an unaligned split merged
    in reverse order."""
    rng = _rng(22)
    B, S, H, hd, D, r = 2, 64, 2, 8, 4, 1
    C = S // (2 * D)
    idx = O.zigzag_index(S, D, r)
    q = rng.standard_normal((B, len(idx), H, hd))
    k = rng.standard_normal((B, S, H, hd))
    v = rng.standard_normal((B, S, H, hd))
    full_o, full_lse = O.causal_attention(q, idx, k, v)
    own = [r, 2 * D - 1 - r]
    order = own + [c for t in range(1, D) for c in ((r - t) % D, 2 * D - 1 - (r - t) % D)]
    assert sorted(order) == list(range(2 * D))
    for bounds in ([(c * C, (c + 1) * C) for c in order], [(23, 64), (5, 23), (0, 5)]):
        acc_o = np.zeros_like(full_o)
        acc_lse = np.full_like(full_lse, -np.inf)
        for lo, hi in bounds:
            po, pl = O.attention_range(q, idx, k, v, lo, hi)
            acc_o, acc_lse = O.lse_merge(acc_o, acc_lse, po, pl)
        np.testing.assert_allclose(acc_o, full_o, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(acc_lse, full_lse, rtol=1e-12)


def pin_merge_identity():
    """(0, -inf) is neutral for lse_merge, the merge is symmetric, and the range [0, S)
    is causal attention itself."""
    rng = _rng(23)
    B, S, H, hd = 1, 24, 2, 4
    pos = np.arange(S)
    q, k, v = (rng.standard_normal((B, S, H, hd)) for _ in range(3))
    o, lse = O.attention_range(q, pos, k, v, 0, S)
    fo, fl = O.causal_attention(q, pos, k, v)
    np.testing.assert_allclose(o, fo, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, fl, rtol=1e-13)
    zo, zl = np.zeros_like(o), np.full_like(lse, -np.inf)
    mo, ml = O.lse_merge(zo, zl, o, lse)
    np.testing.assert_array_equal(mo, o)
    np.testing.assert_array_equal(ml, lse)
    o1, l1 = O.attention_range(q, pos, k, v, 0, 9)
    o2, l2 = O.attention_range(q, pos, k, v, 9, S)
    a = O.lse_merge(o1, l1, o2, l2)
    b = O.lse_merge(o2, l2, o1, l1)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(a[0], fo, rtol=1e-10, atol=1e-12)
    eo, el = O.lse_merge(zo, zl, zo, zl)
    assert np.all(eo == 0) and np.all(el == -np.inf)


def _attn_loss(q, pos, k, v, g):
    o, _ = O.causal_attention(q, pos, k, v)
    return float((o * g).sum())


def pin_attention_bwd_finite_differences():
    """Every gradient entry of causal_attention_bwd against a central difference of the
    forward oracle's loss sum(o * d_o), on zigzag rows of a tiny sequence."""
    rng = _rng(31)
    B, S, D, r, H, hd = 1, 16, 2, 1, 2, 4
    pos = O.zigzag_index(S, D, r)
    q = rng.standard_normal((B, S // D, H, hd))
    k, v = rng.standard_normal((B, S, H, hd)), rng.standard_normal((B, S, H, hd))
    g = rng.standard_normal((B, S // D, H, hd))
    dq, dk, dv = O.causal_attention_bwd(q, pos, k, v, g)
    eps = 1e-6
    for name, x, dx in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[i] += eps
            xm[i] -= eps
            args = {"q": q, "k": k, "v": v}
            lp = _attn_loss(**{**args, name: xp}, pos=pos, g=g)
            lm = _attn_loss(**{**args, name: xm}, pos=pos, g=g)
            num[i] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(dx, num, rtol=1e-6, atol=1e-8, err_msg=name)


def pin_attention_bwd_vs_autograd():
    """Against torch autograd (CPU, float64) through an explicit masked softmax, with a
    scale argument and two rank maps; and the invariants: the keys' dk sum to zero per
    (sequence, head) (softmax rows sum to one), and the keys' dv sum equals the queries'
    d_o sum."""
    import torch
    rng = _rng(37)
    B, S, D, H, hd = 2, 32, 4, 3, 8
    for r, scale in ((0, None), (3, 0.7)):
        pos = O.zigzag_index(S, D, r)
        q = rng.standard_normal((B, S // D, H, hd))
        k, v = rng.standard_normal((B, S, H, hd)), rng.standard_normal((B, S, H, hd))
        g = rng.standard_normal((B, S // D, H, hd))
        dq, dk, dv = O.causal_attention_bwd(q, pos, k, v, g, scale=scale)
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        sc = (1.0 / np.sqrt(hd)) if scale is None else scale
        s = torch.einsum("bihd,bjhd->bhij", tq, tk) * sc
        mask = torch.tensor(np.arange(S)[None, :] <= pos[:, None])
        s = s.masked_fill(~mask, float("-inf"))
        o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), tv)
        (o * torch.tensor(g)).sum().backward()
        np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-10)
        np.testing.assert_allclose(dv.sum(axis=1), g.sum(axis=1), rtol=1e-10, atol=1e-10)
        assert np.all(dk[:, pos.max() + 1:] == 0) and np.all(dv[:, pos.max() + 1:] == 0)


def pin_attention_bwd_ranks_sum():
    """Summed over the D ranks, the ranks' dk and dv equal those of the whole sequence at
    D = 1, and the ranks' dq, placed at their positions, equal its dq."""
    rng = _rng(41)
    B, S, D, H, hd = 1, 24, 3, 2, 4
    q_all = rng.standard_normal((B, S, H, hd))
    k, v = rng.standard_normal((B, S, H, hd)), rng.standard_normal((B, S, H, hd))
    g_all = rng.standard_normal((B, S, H, hd))
    fq, fk, fv = O.causal_attention_bwd(q_all, np.arange(S), k, v, g_all)
    sk, sv, sq = np.zeros_like(fk), np.zeros_like(fv), np.zeros_like(fq)
    for r in range(D):
        idx = O.zigzag_index(S, D, r)
        dq, dk, dv = O.causal_attention_bwd(q_all[:, idx], idx, k, v, g_all[:, idx])
        sk += dk
        sv += dv
        sq[:, idx] = dq
    np.testing.assert_allclose(sk, fk, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(sv, fv, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(sq, fq, rtol=1e-10, atol=1e-12)


def _torch_layer(x, w_qkv, w_o, w1, w3, w2, H):
    """The layer in torch ops (an independent implementation for the autograd pin)."""
    import torch
    B, S, d = x.shape
    hd = d // H
    q, k, v = (x @ w_qkv[i * d:(i + 1) * d].T for i in range(3))
    sh = lambda t: t.reshape(B, S, H, hd)
    s = torch.einsum("bihd,bjhd->bhij", sh(q), sh(k)) / np.sqrt(hd)
    s = s.masked_fill(~torch.ones(S, S, dtype=torch.bool).tril(), float("-inf"))
    o = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, dim=-1), sh(v)).reshape(B, S, d)
    a = o @ w_o.T
    return (torch.nn.functional.silu(a @ w1.T) * (a @ w3.T)) @ w2.T


def pin_layer_bwd_vs_autograd():
    """layer_bwd against torch autograd (CPU, float64) of an independent torch layer, and
    one finite difference per weight."""
    import torch
    rng = _rng(43)
    B, S, d, H, F = 2, 12, 16, 2, 24
    arrs = {"x": rng.standard_normal((B, S, d)), "w_qkv": 0.3 * rng.standard_normal((3 * d, d)),
            "w_o": 0.3 * rng.standard_normal((d, d)), "w1": 0.3 * rng.standard_normal((F, d)),
            "w3": 0.3 * rng.standard_normal((F, d)), "w2": 0.3 * rng.standard_normal((d, F))}
    dy = rng.standard_normal((B, S, d))
    ref = O.layer_bwd(arrs["x"], arrs["w_qkv"], arrs["w_o"], arrs["w1"], arrs["w3"], arrs["w2"], H, dy)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in arrs.items()}
    y = _torch_layer(t["x"], t["w_qkv"], t["w_o"], t["w1"], t["w3"], t["w2"], H)
    (y * torch.tensor(dy)).sum().backward()
    names = {"x": "dx", "w_qkv": "dw_qkv", "w_o": "dw_o", "w1": "dw1", "w3": "dw3", "w2": "dw2"}
    for k, r in names.items():
        np.testing.assert_allclose(ref[r], t[k].grad.numpy(), rtol=1e-9, atol=1e-11, err_msg=k)
    eps = 1e-6
    for k, r in names.items():
        i = tuple(int(rng.integers(n)) for n in arrs[k].shape)
        plus, minus = {**arrs}, {**arrs}
        plus[k], minus[k] = arrs[k].copy(), arrs[k].copy()
        plus[k][i] += eps
        minus[k][i] -= eps
        f = lambda z: float((O.swiglu_mlp(O.project(O.causal_attention(
            *O.qkv_rows(z["x"], z["w_qkv"], H)[:1], np.arange(S), *O.qkv_rows(z["x"], z["w_qkv"], H)[1:])[0]
            .reshape(B, S, d), z["w_o"]), z["w1"], z["w3"], z["w2"]) * dy).sum())
        num = (f(plus) - f(minus)) / (2 * eps)
        np.testing.assert_allclose(ref[r][i], num, rtol=1e-5, atol=1e-7, err_msg=k)


PINS = [pin_zigzag_golden, pin_zigzag_partition, pin_zigzag_balance, pin_zigzag_identity,
        pin_attention_vs_brute, pin_attention_vs_library, pin_attention_concat_ranks,
        pin_attention_special_cases, pin_attention_scale, pin_silu_closed_form,
        pin_mlp_vs_brute, pin_mlp_shards_sum, pin_layer_vs_brute, pin_layer_concat_ranks,
        pin_layer_rows_subset, pin_layer_flops, pin_range_vs_brute, pin_range_merge_equals_full,
        pin_merge_identity, pin_attention_bwd_finite_differences, pin_attention_bwd_vs_autograd,
        pin_attention_bwd_ranks_sum, pin_layer_bwd_vs_autograd]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_zigzag_rejects_bad_shapes():
    with pytest.raises(ValueError):
        O.zigzag_index(100, 8, 0)  # S not a multiple of 2D
    with pytest.raises(ValueError):
        O.zigzag_index(64, 4, 4)   # rank out of range


# ---------------------------------------------------------------- planted mistakes

def _bad_zigzag(S, D, rank):
    C = S // (2 * D)
    late = 2 * D - rank  # off by one in the mirror chunk
    return np.concatenate([np.arange(rank * C, rank * C + C),
                           np.arange((late % (2 * D)) * C, (late % (2 * D)) * C + C)])


def _bad_mask(q_pos, n_keys):
    keys = np.arange(n_keys)
    return keys[None, :] < np.asarray(q_pos)[:, None]  # drops the diagonal


def _bad_mask_off(q_pos, n_keys):
    keys = np.arange(n_keys)
    return keys[None, :] <= np.asarray(q_pos)[:, None] + 1  # one key too many


def _bad_project(x, w):
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64)  # transposed operand


def _bad_silu(g):
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(g))  # wrong sign


def _bad_split_heads(t, n_heads):
    # interleaves heads instead of giving head h a contiguous block of features
    return t.reshape(*t.shape[:-1], t.shape[-1] // n_heads, n_heads).swapaxes(-1, -2)


_good_range = O.attention_range
_good_merge = O.lse_merge


def _bad_range(q, q_pos, k, v, key_lo, key_hi, scale=None, row_block=512):
    return _good_range(q, q_pos, k, v, key_lo + 1, key_hi, scale, row_block)  # lower bound one key late


def _bad_merge(o_a, lse_a, o_b, lse_b):
    o, lse = _good_merge(o_b, lse_a, o_a, lse_b)  # outputs paired with the other side's weight
    return o, lse


_good_bwd = O.causal_attention_bwd


def _bad_bwd_no_rowsum(q, q_pos, k, v, d_o, scale=None, row_block=512):
    # drops the softmax Jacobian's row term: ds = P dP
    q, k, v, d_o = (np.asarray(a, dtype=np.float64) for a in (q, k, v, d_o))
    B, n, H, hd = q.shape
    sc = 1.0 / np.sqrt(hd) if scale is None or scale <= 0 else scale
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            s = (q[b, :, h] @ k[b, :, h].T) * sc
            s = np.where(O.causal_scores_mask(q_pos, k.shape[1]), s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dv[b, :, h] = p.T @ d_o[b, :, h]
            ds = p * (d_o[b, :, h] @ v[b, :, h].T)
            dq[b, :, h] = sc * ds @ k[b, :, h]
            dk[b, :, h] = sc * ds.T @ q[b, :, h]
    return dq, dk, dv


def _bad_bwd_unscaled_dk(q, q_pos, k, v, d_o, scale=None, row_block=512):
    dq, dk, dv = _good_bwd(q, q_pos, k, v, d_o, scale, row_block)
    hd = np.asarray(q).shape[-1]
    return dq, dk * np.sqrt(hd), dv  # the scale left out of dk


_good_layer_bwd = O.layer_bwd


def _bad_layer_bwd(x_full, w_qkv, w_o, w1, w3, w2, n_heads, d_y, scale=None):
    # silu'(g) taken as sigmoid(g) alone: the gate's gradient loses its g (1 - s) term
    saved = O.causal_attention_bwd
    r = _good_layer_bwd(x_full, w_qkv, w_o, w1, w3, w2, n_heads, d_y, scale)
    x = np.asarray(x_full, dtype=np.float64)
    B, S, d = x.shape
    q, k, v = O.qkv_rows(x, w_qkv, n_heads)
    o, _ = O.causal_attention(q, np.arange(S), k, v, scale=scale)
    a = O.project(o.reshape(B, S, d), w_o)
    g, u = O.project(a, w1), O.project(a, w3)
    sg = 1.0 / (1.0 + np.exp(-g))
    dhh = np.asarray(d_y, dtype=np.float64) @ np.asarray(w2, dtype=np.float64)
    r["dw1"] = (dhh * u * sg).reshape(-1, g.shape[-1]).T @ a.reshape(-1, d)
    assert saved is O.causal_attention_bwd
    return r


MUTANTS = {
    "layer_bwd_silu_derivative": ("layer_bwd", _bad_layer_bwd),
    "bwd_softmax_row_term_dropped": ("causal_attention_bwd", _bad_bwd_no_rowsum),
    "bwd_dk_unscaled": ("causal_attention_bwd", _bad_bwd_unscaled_dk),
    "range_lower_bound_late": ("attention_range", _bad_range),
    "merge_weights_swapped": ("lse_merge", _bad_merge),
    "zigzag_mirror_off_by_one": ("zigzag_index", _bad_zigzag),
    "mask_drops_diagonal": ("causal_scores_mask", _bad_mask),
    "mask_one_key_late": ("causal_scores_mask", _bad_mask_off),
    "weight_not_transposed": ("project", _bad_project),
    "silu_sign": ("silu", _bad_silu),
    "heads_interleaved": ("split_heads", _bad_split_heads),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTANTS[name]
    monkeypatch.setattr(O, attr, bad)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
