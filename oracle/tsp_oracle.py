"""Reference oracle for one rank's share of a TSP transformer layer (test infrastructure only).

This module is test infrastructure. Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it. The product path (the HIP library
and its Python binding) never imports, calls or links anything here, and nothing
here imports the product path.

Source of the method: the two summaries (Arabic and Japanese) of "Folding Tensor and
Sequence Parallelism for Memory-Efficient Transformer Training & Inference"
(gist.science, paper 2604.26294), cited below as [TSP §n] for section n of that
summary. The facts used:

* [TSP §2, unified sharding] each of D ranks holds 1/D of the tokens and sees the
  weights as D shards.
* [TSP §2, attention layers] every rank projects its own tokens with the packed
  W_Q/W_K/W_V shards, the K/V of the whole sequence is gathered, and FlashAttention
  runs the rank's queries against it; zigzag partitioning balances causal work.
* [TSP §2, gated MLP layers] the W1/W2/W3 shards travel round a ring and every rank
  sums the partial outputs of the shards it sees, with no all-reduce.

TSP changes where the work runs, not what is computed: a rank's outputs are the
unsharded layer's outputs at that rank's rows. So this oracle is the plain
definition of that layer, written out in float64:

    idx      = zigzag rows of the rank                       (zigzag_index)
    Q,K,V    = X W_q^T, X W_k^T, X W_v^T                     (project)
    O[i]     = sum_{j <= idx[i]} softmax_j(q_i.k_j * scale) v_j   (causal_attention)
    A        = O W_o^T                                        (project)
    Y        = (silu(A W1^T) * (A W3^T)) W2^T                 (swiglu_mlp)
    Y        = sum_j  partial of ffn shard j                  (mlp_shard_partial)

Readings taken where the pages say nothing (each also listed in the design notes):
  - chunking: 2D equal chunks of C = S/(2D) tokens; rank r owns chunks r and
    2D-1-r; its local rows run over chunk r then chunk 2D-1-r, ascending.
  - softmax scale 1/sqrt(head_dim); the causal mask keeps key j for query position
    p when j <= p (the diagonal is visible).
  - no positional encoding, norm, residual, bias or dropout: the layer is exactly
    QKV -> attention -> W_O -> gated MLP, and the MLP input is the W_O output.
  - the gated MLP is SwiGLU: silu on the W1 branch, W3 the "up" branch, W2 "down";
    silu(g) = g * sigmoid(g).
  - the ffn dimension is cut into D contiguous shards of F/D; shard j is rows
    [j F/D, (j+1) F/D) of W1 and W3 and the same columns of W2.
  - weights are stored [out_features, in_features]; W_qkv rows are [W_q; W_k; W_v],
    head h owning rows h*hd .. h*hd+hd-1 of each.

Every function computes in float64 on whatever values it is given. Inputs that the
GPU consumes as bf16 are handed over already rounded to bf16 values by the seeded
generator, so both sides see identical numbers.
"""

import numpy as np

__all__ = [
    "zigzag_index",
    "project",
    "split_heads",
    "causal_scores_mask",
    "causal_attention",
    "silu",
    "swiglu_mlp",
    "mlp_shard_partial",
    "qkv_rows",
    "rank_layer",
    "layer_flops",
    "attention_range",
    "lse_merge",
    "causal_attention_bwd",
    "layer_bwd",
]


def zigzag_index(S, D, rank):
    """Global sequence positions of a rank's local rows. [TSP §2, zigzag partitioning]

    The sequence of S tokens is cut into 2D chunks of C = S/(2D). Rank r owns chunk
    r and its mirror chunk 2D-1-r, so an early (cheap) chunk is paired with a late
    (expensive) one under the causal mask. Local rows list chunk r first, then
    chunk 2D-1-r, each in ascending order.
    """
    S, D, rank = int(S), int(D), int(rank)
    if D < 1 or S % (2 * D) != 0:
        raise ValueError("S must be a positive multiple of 2D")
    if not 0 <= rank < D:
        raise ValueError("rank must be in [0, D)")
    C = S // (2 * D)
    early = np.arange(rank * C, (rank + 1) * C, dtype=np.int64)
    mirror = 2 * D - 1 - rank
    late = np.arange(mirror * C, (mirror + 1) * C, dtype=np.int64)
    return np.concatenate([early, late])


def project(x, w):
    """Linear map with a weight stored [out_features, in_features]: x @ w^T. [TSP §2]"""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def split_heads(t, n_heads):
    """[..., H*hd] -> [..., H, hd]; head h owns features h*hd .. h*hd+hd-1."""
    return t.reshape(*t.shape[:-1], n_heads, t.shape[-1] // n_heads)


def causal_scores_mask(q_pos, n_keys):
    """Boolean [n_q, n_keys] mask, True where key j may be attended from query position p.

    Causal attention keeps the keys at positions not after the query (j <= p).
    """
    keys = np.arange(n_keys, dtype=np.int64)
    return keys[None, :] <= np.asarray(q_pos, dtype=np.int64)[:, None]


def causal_attention(q, q_pos, k, v, scale=None, row_block=512):
    """Causal softmax attention of queries at given global positions. [TSP §2, attention layers]

    q      [B, n, H, hd]  queries of the rank's rows
    q_pos  [n]            global position of each query row
    k, v   [B, S, H, hd]  keys and values of the whole sequence, natural order
    Returns (o [B, n, H, hd], lse [B, H, n]) with lse the natural-log sum of the
    exponentiated scaled scores over the visible keys.

    The definition is per query row: o_i = sum_{j <= p_i} softmax_j(scale * q_i.k_j) v_j.
    Rows are evaluated in blocks only to bound memory; keys after the block's last
    position are masked for every row of the block, so they are not materialised.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    B, n, H, hd = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(hd)
    o = np.zeros((B, n, H, hd), dtype=np.float64)
    lse = np.zeros((B, H, n), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, n, row_block):
                r1 = min(n, r0 + row_block)
                pos = q_pos[r0:r1]
                kmax = int(pos.max()) + 1
                kk = k[b, :kmax, h, :]
                vv = v[b, :kmax, h, :]
                s = (q[b, r0:r1, h, :] @ kk.T) * scale
                s = np.where(causal_scores_mask(pos, kmax), s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                z = e.sum(axis=1, keepdims=True)
                o[b, r0:r1, h, :] = (e / z) @ vv
                lse[b, h, r0:r1] = (m + np.log(z))[:, 0]
    return o, lse


def causal_attention_bwd(q, q_pos, k, v, d_o, scale=None, row_block=512):
    """Gradients of causal_attention with respect to q, k and v, given the gradient d_o of
    its output o. [TSP title: training; the pages do not describe the backward pass, so
    this is the derivative of the forward definition above]

    With s_ij = scale q_i.k_j over the visible keys (j <= p_i) and P_i = softmax_j(s_ij),
    o_i = sum_j P_ij v_j. Differentiating:
      dv_j  = sum_i P_ij do_i                       (v enters o linearly)
      dP_ij = do_i . v_j
      ds_ij = P_ij (dP_ij - sum_l P_il dP_il)        (Jacobian of the softmax of row i)
      dq_i  = scale sum_j ds_ij k_j,   dk_j = scale sum_i ds_ij q_i
    q, q_pos, k, v as in causal_attention; d_o [B, n, H, hd].
    Returns (dq [B, n, H, hd], dk [B, S, H, hd], dv [B, S, H, hd]); keys after every
    query's position get zero gradient. For one rank, dk and dv are its contributions:
    the gradient of the whole sequence's K and V is their sum over the ranks.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_o = np.asarray(d_o, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    B, n, H, hd = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(hd)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, n, row_block):
                r1 = min(n, r0 + row_block)
                pos = q_pos[r0:r1]
                kmax = int(pos.max()) + 1
                kk = k[b, :kmax, h, :]
                vv = v[b, :kmax, h, :]
                qq = q[b, r0:r1, h, :]
                g = d_o[b, r0:r1, h, :]
                s = (qq @ kk.T) * scale
                s = np.where(causal_scores_mask(pos, kmax), s, -np.inf)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
                dv[b, :kmax, h, :] += p.T @ g
                dp = g @ vv.T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, r0:r1, h, :] = scale * (ds @ kk)
                dk[b, :kmax, h, :] += scale * (ds.T @ qq)
    return dq, dk, dv


def attention_range(q, q_pos, k, v, key_lo, key_hi, scale=None, row_block=512):
    """Causal attention restricted to the keys at positions [key_lo, key_hi).

    [TSP §2, attention layers] The all-gather delivers the K/V of the sequence chunk by
    chunk; attention over each arrived chunk, merged by log-sum-exp (lse_merge), equals
    attention over the whole sequence. For a query at position p the visible keys are j
    with key_lo <= j < key_hi and j <= p.
    Returns (o [B, n, H, hd], lse [B, H, n]): the softmax-weighted mean of V over the
    visible keys and the natural log of sum_j exp(scale * q.k_j) over them. A row that
    sees no key gets o = 0 and lse = -inf (the neutral element of lse_merge).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    B, n, H, hd = q.shape
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(hd)
    key_lo, key_hi = int(key_lo), int(key_hi)
    o = np.zeros((B, n, H, hd), dtype=np.float64)
    lse = np.full((B, H, n), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, n, row_block):
                r1 = min(n, r0 + row_block)
                pos = q_pos[r0:r1]
                hi = min(key_hi, int(pos.max()) + 1)
                if hi <= key_lo:
                    continue
                keys = np.arange(key_lo, hi, dtype=np.int64)
                s = (q[b, r0:r1, h, :] @ k[b, key_lo:hi, h, :].T) * scale
                visible = keys[None, :] <= pos[:, None]
                s = np.where(visible, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                seen = np.isfinite(m[:, 0])
                m_safe = np.where(np.isfinite(m), m, 0.0)
                e = np.exp(s - m_safe)
                z = e.sum(axis=1, keepdims=True)
                z_safe = np.where(z > 0, z, 1.0)
                o[b, r0:r1, h, :] = np.where(seen[:, None], (e / z_safe) @ v[b, key_lo:hi, h, :], 0.0)
                lse[b, h, r0:r1] = np.where(seen, (m_safe + np.log(z_safe))[:, 0], -np.inf)
    return o, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Attention over the union of two disjoint key sets, from the attention over each.

    With lse = log(exp(lse_a) + exp(lse_b)), the merged output is
    exp(lse_a - lse) o_a + exp(lse_b - lse) o_b (each o a softmax-weighted mean over its
    own keys). o: [B, n, H, hd], lse: [B, H, n]. (0, -inf) is the neutral element.
    """
    o_a, o_b = np.asarray(o_a, dtype=np.float64), np.asarray(o_b, dtype=np.float64)
    lse_a, lse_b = np.asarray(lse_a, dtype=np.float64), np.asarray(lse_b, dtype=np.float64)
    lse = np.logaddexp(lse_a, lse_b)
    fin = np.isfinite(lse)
    ref = np.where(fin, lse, 0.0)
    w_a = np.where(fin, np.exp(lse_a - ref), 0.0)  # [B, H, n]
    w_b = np.where(fin, np.exp(lse_b - ref), 0.0)
    to_rows = lambda w: np.transpose(w, (0, 2, 1))[..., None]  # [B, n, H, 1]
    return to_rows(w_a) * o_a + to_rows(w_b) * o_b, lse


def silu(g):
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)), the SwiGLU gate activation."""
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def swiglu_mlp(x, w1, w3, w2):
    """Unsharded gated MLP: (silu(x W1^T) * (x W3^T)) W2^T. [TSP §2, gated MLP layers]

    x [..., d]; w1, w3 [F, d]; w2 [d, F].
    """
    return project(silu(project(x, w1)) * project(x, w3), w2)


def mlp_shard_partial(x, w1, w3, w2, j, D):
    """Partial MLP output of ffn shard j out of D. [TSP §2, gated MLP ring]

    Shard j holds ffn features [j F/D, (j+1) F/D): those rows of W1 and W3 and those
    columns of W2. Summing the D partials gives swiglu_mlp's output exactly in exact
    arithmetic, which is why the ring needs no all-reduce.
    """
    F = np.asarray(w1).shape[0]
    if F % D != 0:
        raise ValueError("F must be a multiple of D")
    Fs = F // D
    sl = slice(j * Fs, (j + 1) * Fs)
    return swiglu_mlp(x, np.asarray(w1)[sl], np.asarray(w3)[sl], np.asarray(w2)[:, sl])


def qkv_rows(x_rows, w_qkv, n_heads):
    """Q, K, V of the given token rows, each [..., H, hd]. [TSP §2, local projections]

    w_qkv [3d, d] stacks W_q, W_k, W_v.
    """
    w_qkv = np.asarray(w_qkv, dtype=np.float64)
    d = w_qkv.shape[1]
    q = project(x_rows, w_qkv[0:d])
    k = project(x_rows, w_qkv[d:2 * d])
    v = project(x_rows, w_qkv[2 * d:3 * d])
    return split_heads(q, n_heads), split_heads(k, n_heads), split_heads(v, n_heads)


def rank_layer(x_full, w_qkv, w_o, w1, w3, w2, S, D, rank, n_heads, rows=None,
               scale=None):
    """One rank's layer outputs, as the unsharded layer's outputs at the rank's rows.

    x_full [B, S, d] holds every rank's tokens (the peers' K/V derive from them).
    rows   optional subset of local row indices (0 .. 2C-1) to evaluate.
    Returns dict with idx, q [B,n,H,hd], o [B,n,H,hd], lse [B,H,n],
    attn_out [B,n,d] (A = O W_o^T) and mlp_out [B,n,d] (the SwiGLU of A).
    """
    x_full = np.asarray(x_full, dtype=np.float64)
    B, S_, d = x_full.shape
    assert S_ == S
    idx = zigzag_index(S, D, rank)
    if rows is None:
        rows = np.arange(idx.shape[0])
    rows = np.asarray(rows, dtype=np.int64)
    pos = idx[rows]
    kmax = int(pos.max()) + 1
    # K/V of the prefix every selected row can see (the all-gathered context).
    w_qkv = np.asarray(w_qkv, dtype=np.float64)
    k = split_heads(project(x_full[:, :kmax], w_qkv[d:2 * d]), n_heads)
    v = split_heads(project(x_full[:, :kmax], w_qkv[2 * d:3 * d]), n_heads)
    q = split_heads(project(x_full[:, pos], w_qkv[0:d]), n_heads)
    o, lse = causal_attention(q, pos, k, v, scale=scale)
    attn_out = project(o.reshape(B, len(rows), d), w_o)
    mlp_out = swiglu_mlp(attn_out, w1, w3, w2)
    return {"idx": idx, "pos": pos, "q": q, "o": o, "lse": lse,
            "attn_out": attn_out, "mlp_out": mlp_out}


def layer_bwd(x_full, w_qkv, w_o, w1, w3, w2, n_heads, d_y, scale=None):
    """Gradients of the unsharded layer (QKV -> causal attention -> W_O -> SwiGLU MLP) given
    the gradient d_y [B, S, d] of its output. [TSP title: training; the backward is the
    derivative of the forward defined above]

    With A = O W_o^T, G = A W1^T, U = A W3^T, Hh = silu(G) * U, Y = Hh W2^T:
      dW2 = dY^T Hh,  dHh = dY W2,
      dG = dHh * U * silu'(G)  (silu'(g) = s(g) (1 + g (1 - s(g))), s the sigmoid),
      dU = dHh * silu(G),  dW1 = dG^T A,  dW3 = dU^T A,  dA = dG W1 + dU W3,
      dW_o = dA^T O,  dO = dA W_o,  (dQ, dK, dV) = causal_attention_bwd(..., dO),
      dW_qkv = [dQ; dK; dV]^T X,  dX = dQ W_q + dK W_k + dV W_v.
    Returns a dict with dx [B, S, d], dw_qkv [3d, d], dw_o [d, d], dw1, dw3 [F, d], dw2 [d, F].
    On D ranks every term is a sum over tokens: a rank's share of a weight gradient is the
    same expression over its own rows, and the shares add up to these.
    """
    x = np.asarray(x_full, dtype=np.float64)
    w_qkv, w_o = np.asarray(w_qkv, dtype=np.float64), np.asarray(w_o, dtype=np.float64)
    w1, w3, w2 = (np.asarray(w, dtype=np.float64) for w in (w1, w3, w2))
    dy = np.asarray(d_y, dtype=np.float64)
    B, S, d = x.shape
    pos = np.arange(S)
    q, k, v = qkv_rows(x, w_qkv, n_heads)
    o, _ = causal_attention(q, pos, k, v, scale=scale)
    of = o.reshape(B, S, d)
    a = project(of, w_o)
    g, u = project(a, w1), project(a, w3)
    sg = 1.0 / (1.0 + np.exp(-g))
    hh = g * sg * u
    flat = lambda t: t.reshape(-1, t.shape[-1])
    dw2 = flat(dy).T @ flat(hh)
    dhh = dy @ w2
    dg = dhh * u * sg * (1.0 + g * (1.0 - sg))
    du = dhh * g * sg
    dw1, dw3 = flat(dg).T @ flat(a), flat(du).T @ flat(a)
    da = dg @ w1 + du @ w3
    dw_o = flat(da).T @ flat(of)
    do = (da @ w_o).reshape(o.shape)
    dq, dk, dv = causal_attention_bwd(q, pos, k, v, do, scale=scale)
    dqkv = np.concatenate([dq.reshape(B, S, d), dk.reshape(B, S, d), dv.reshape(B, S, d)], axis=-1)
    dw_qkv = flat(dqkv).T @ flat(x)
    dx = dqkv @ w_qkv
    return {"dx": dx, "dw_qkv": dw_qkv, "dw_o": dw_o, "dw1": dw1, "dw3": dw3, "dw2": dw2}


def layer_flops(B, S, D, d, n_heads, head_dim, F):
    """Algorithmic FLOPs of one rank's layer forward (exact causal pairs).

    2*M*d*3d (QKV) + 4*B*H*hd*C*(S+1) (QK^T and PV over C(S+1) causal pairs per
    (sequence, head)) + 2*M*d*d (W_O) + 6*M*d*F (SwiGLU over all D shards), with
    C = S/(2D) and M = B*S/D. Zigzag pairing gives every rank the same pair count
    C(S+1): sum over chunk r and 2D-1-r of (position + 1).
    """
    C = S // (2 * D)
    M = B * 2 * C
    pairs = C * (S + 1)
    return (2 * M * d * 3 * d + 4 * B * n_heads * head_dim * pairs
            + 2 * M * d * d + 6 * M * d * F)
