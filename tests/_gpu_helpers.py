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

# The log-sum-exp output has no tolerance in the contract. The kernel forms scores from
# Q * scale * log2(e) rounded to bf16 (relative error <= 2^-9 per element), which moves a
# score by about 3e-3 (log2 units) at the spreads of the 7B workloads; the LSE, a smooth
# max of the scores, carries errors of that size (about 2e-3 in natural-log units). Bounds
# of 2e-3 (max) and 3e-4 (mean) of max|lse| (about 11 at S=128K) leave a margin of 2-3x.
LSE_MAX_REL = 2e-3
LSE_MEAN_REL = 3e-4

BF16_NAN = 0x7FC0


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
