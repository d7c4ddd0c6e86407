"""Pure-Python brute force for tiny TSP layer inputs (test infrastructure only).

Test infrastructure: only the test suite imports this. It evaluates the same
definitions as tsp_oracle with explicit scalar loops and the math module, no numpy,
so that a vectorisation slip in the oracle (a transposed operand, a broadcast along
the wrong axis, a wrong mask index) shows up as a disagreement on tiny inputs.

Method source: summary of "Folding Tensor and Sequence Parallelism for
Memory-Efficient Transformer Training & Inference" (gist.science 2604.26294), §2:
the rank's outputs are those of the unsharded causal layer at its zigzag rows.
Inputs are nested Python lists (or anything indexable) of floats.
"""

import math


def zigzag_positions(S, D, rank):
    """Rank r owns chunks r and 2D-1-r of 2D equal chunks, listed in that order."""
    C = S // (2 * D)
    out = []
    for chunk in (rank, 2 * D - 1 - rank):
        for t in range(C):
            out.append(chunk * C + t)
    return out


def matvec_t(w, x):
    """y[o] = sum_i w[o][i] * x[i] for w stored [out][in]."""
    return [sum(w[o][i] * x[i] for i in range(len(x))) for o in range(len(w))]


def attention_row(q_row, pos, k_seq, v_seq, scale):
    """One query row of causal attention for one head.

    q_row [hd]; k_seq, v_seq [S][hd] in position order; keys 0..pos are visible.
    Returns (o [hd], lse).
    """
    scores = []
    for j in range(pos + 1):
        scores.append(scale * sum(q_row[c] * k_seq[j][c] for c in range(len(q_row))))
    mx = max(scores)
    ex = [math.exp(s - mx) for s in scores]
    z = sum(ex)
    hd = len(v_seq[0])
    o = [sum(ex[j] * v_seq[j][c] for j in range(pos + 1)) / z for c in range(hd)]
    return o, mx + math.log(z)


def attention_row_range(q_row, pos, k_seq, v_seq, scale, key_lo, key_hi):
    """One query row attending the keys j with key_lo <= j < key_hi and j <= pos.

    Returns (o [hd], lse); a row that sees no key gives ([0]*hd, -inf).
    """
    keys = [j for j in range(key_lo, min(key_hi, pos + 1))]
    hd = len(v_seq[0])
    if not keys:
        return [0.0] * hd, -math.inf
    scores = [scale * sum(q_row[c] * k_seq[j][c] for c in range(len(q_row))) for j in keys]
    mx = max(scores)
    ex = [math.exp(s - mx) for s in scores]
    z = sum(ex)
    o = [sum(ex[t] * v_seq[j][c] for t, j in enumerate(keys)) / z for c in range(hd)]
    return o, mx + math.log(z)


def silu(g):
    return g / (1.0 + math.exp(-g))


def mlp_row(x_row, w1, w3, w2):
    """(silu(x W1^T) * (x W3^T)) W2^T for one row; w1, w3 [F][d], w2 [d][F]."""
    g = matvec_t(w1, x_row)
    u = matvec_t(w3, x_row)
    h = [silu(g[f]) * u[f] for f in range(len(g))]
    return matvec_t(w2, h)


def rank_layer(x_full, w_qkv, w_o, w1, w3, w2, S, D, rank, n_heads, scale=None):
    """All outputs of one rank's layer for one sequence, by scalar loops.

    x_full [S][d]. Returns dict of lists: pos, o [n][H][hd], lse [H][n],
    attn_out [n][d], mlp_out [n][d].
    """
    d = len(x_full[0])
    hd = d // n_heads
    if scale is None:
        scale = 1.0 / math.sqrt(hd)
    wq, wk, wv = w_qkv[0:d], w_qkv[d:2 * d], w_qkv[2 * d:3 * d]
    kk = [matvec_t(wk, x_full[t]) for t in range(S)]
    vv = [matvec_t(wv, x_full[t]) for t in range(S)]
    pos_list = zigzag_positions(S, D, rank)
    o_all, lse_all, a_all, y_all = [], [], [], []
    lse_all = [[0.0] * len(pos_list) for _ in range(n_heads)]
    for i, p in enumerate(pos_list):
        qrow = matvec_t(wq, x_full[p])
        o_row = []
        for h in range(n_heads):
            sl = slice(h * hd, (h + 1) * hd)
            k_h = [kk[t][sl] for t in range(S)]
            v_h = [vv[t][sl] for t in range(S)]
            o_h, l_h = attention_row(qrow[sl], p, k_h, v_h, scale)
            o_row.append(o_h)
            lse_all[h][i] = l_h
        o_all.append(o_row)
        flat = [val for head in o_row for val in head]
        a = matvec_t(w_o, flat)
        a_all.append(a)
        y_all.append(mlp_row(a, w1, w3, w2))
    return {"pos": pos_list, "o": o_all, "lse": lse_all, "attn_out": a_all,
            "mlp_out": y_all}
