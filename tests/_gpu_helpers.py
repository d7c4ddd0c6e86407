"""Shared helpers of the GPU parity tests (device upload/download, tolerance check, the
one-GPU stand-in for the K/V all-gather)."""

import numpy as np
import torch

from long_context_transformer_amd import synth, tsp

# Contract for floating-point parity against the fp64 oracle (bf16 inputs and stored
# intermediates, fp32 accumulation): max-abs <= 2e-2 * max|ref| and
# mean-abs <= 2e-3 * max|ref|.
MAX_REL = 2e-2
MEAN_REL = 2e-3

# The log-sum-exp output has no tolerance in the contract; its error is an absolute error
# in log space. The kernel forms scores from Q * scale * log2(e) rounded to bf16 (relative
# error <= 2^-9 per element), which moves a score by at most 2^-9 * scale * sum_d |q_d k_d|
# (<= about 0.015 in natural-log units for unit-to-1.3 spreads and head_dim <= 128, about
# 0.002 on average); the LSE, a smooth max of the scores, inherits errors of that size
# (exactly that size for a row that sees a single key).
LSE_MAX_ABS = 0.02
LSE_MEAN_ABS = 3e-3

BF16_NAN = 0x7FC0


# Softmax scale 1/(8 log2 e): the kernel's pre-scaled Q (q / 8) is then exact in bf16, so its
# scores differ from the oracle's only by fp32 rounding even where they reach thousands.
RAMP_SCALE = float(1.0 / (8.0 * np.log2(np.e)))


def ramp_inputs(B, S, rows, H, hd, seed):
    """Per head, scores (log2 units) that rise by 12 per key position (the running max moves
    at every 32-key block, so every block takes the reference-move path and the next block's
    scores were started from the old reference), rise by 0.2 per key (a move every few
    blocks), fall by 0.5 per key (no move after the first block), or are random (head 3)."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal(hd).astype(np.float32)
    u /= np.linalg.norm(u)
    q = rng.standard_normal((B, rows, H, hd)).astype(np.float32)
    k = rng.standard_normal((B, S, H, hd)).astype(np.float32)
    v = rng.standard_normal((B, S, H, hd)).astype(np.float32)
    pos = np.arange(S, dtype=np.float32)[:, None]
    for h, slope in ((0, 12.0), (1, 0.2), (2, -0.5)):
        q[:, :, h] = u + 0.05 * q[:, :, h]
        k[:, :, h] = 8.0 * slope * pos * u + 0.05 * k[:, :, h]
    return tuple(synth.round_bf16_bits(x) for x in (q, k, v))


def dev_bf16(bits):
    return synth.to_torch(bits).cuda()


def host_f64(t):
    """bf16 or f32 device tensor -> float64 numpy."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return synth.to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def host_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def nan_bf16(shape):
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")


def check_close(name, got, ref, max_rel=MAX_REL, mean_rel=MEAN_REL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    scale = float(np.abs(ref).max())
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    print(f"  {name}: max|ref|={scale:.4g} max_err={mx:.3g} ({mx / scale:.2e}) "
          f"mean_err={mean:.3g} ({mean / scale:.2e})", flush=True)
    assert mx <= max_rel * scale, f"{name}: max-abs {mx:.4g} > {max_rel} * {scale:.4g}"
    assert mean <= mean_rel * scale, f"{name}: mean-abs {mean:.4g} > {mean_rel} * {scale:.4g}"
    return mx / scale, mean / scale


def check_lse(name, got, ref):
    """Absolute log-space bounds for the log-sum-exp output; -inf entries must match."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{name}: -inf pattern differs"
    err = np.abs(got[fin] - ref[fin])
    mx, mean = float(err.max()), float(err.mean())
    print(f"  {name}: max_err={mx:.3g} mean_err={mean:.3g} (absolute, natural log)", flush=True)
    assert mx <= LSE_MAX_ABS, f"{name}: max-abs {mx:.4g} > {LSE_MAX_ABS}"
    assert mean <= LSE_MEAN_ABS, f"{name}: mean-abs {mean:.4g} > {LSE_MEAN_ABS}"


def shard_rows(x_full_dev, S, D, rank):
    """The rank's tokens [B, 2C, d] in local row order (gathered with the library's map)."""
    idx = torch.from_numpy(tsp.zigzag_index(S, D, rank)).cuda()
    return x_full_dev.index_select(1, idx).contiguous()


def fill_peer_kv(x_full_dev, w_qkv_dev, k_full, v_full, B, S, D, rank, H, hd):
    """Stand-in for the K/V all-gather on one GPU: every other rank's rows of k_full and
    v_full are written by that rank's own QKV projection."""
    for r in range(D):
        if r == rank:
            continue
        xs = shard_rows(x_full_dev, S, D, r)
        tsp.qkv_fwd(xs, w_qkv_dev, None, k_full, v_full, B, S, D, r, H, hd)
