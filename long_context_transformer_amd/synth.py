"""Seeded synthetic inputs for the TSP rank-shard layer (shared by tests, smoke and bench).

This module draws numbers and rounds them to bf16; it holds none of the layer's
arithmetic, so both the HIP path and the CPU oracle can take their inputs from it
without sharing any of the computation under test.

Recipe (stated once, used everywhere):
  * generator: numpy PCG64 ``default_rng(seed)``, ``standard_normal`` in float32,
    multiplied by the standard deviation, rounded to bf16 with round-to-nearest-even;
  * seed = 1000 * workload_id + t, with t = 1 for X_full, 2 for W_qkv, 3 for W_o,
    4 for W1, 5 for W3, 6 for W2 (7.. for extra tensors a test draws);
  * activations ~ N(0, 1), weights ~ N(0, 0.02^2);
  * X_full [B, S, d] holds every rank's tokens: the peers' keys and values are
    projections of it.
Arrays are returned as uint16 bf16 bit patterns; ``to_f64`` and ``to_torch`` turn
them into exact float64 values or a CPU bf16 tensor.
"""

from dataclasses import dataclass

import numpy as np

_CHUNK = 1 << 24  # draw in fixed chunks so the stream is identical for any size


@dataclass(frozen=True)
class Workload:
    """Sizes of one rank-shard layer workload."""
    wid: int
    name: str
    B: int
    S: int
    D: int
    rank: int
    d_model: int
    n_heads: int
    head_dim: int
    ffn: int

    @property
    def C(self):
        return self.S // (2 * self.D)

    @property
    def rows(self):
        """Local rows per sequence (two zigzag chunks)."""
        return 2 * self.C

    @property
    def M(self):
        return self.B * self.rows

    @property
    def Fs(self):
        return self.ffn // self.D

    def with_rank(self, rank):
        return Workload(self.wid, self.name, self.B, self.S, self.D, rank, self.d_model,
                        self.n_heads, self.head_dim, self.ffn)


# The five workloads: a tiny shard for exhaustive checks, then a 7B-style dense layer
# (d_model 4096, 32 heads of 128, SwiGLU ffn 11008) folded D = 8 ways.
WORKLOADS = {
    "tiny_s256_d4": Workload(0, "tiny_s256_d4", 1, 256, 4, 0, 256, 4, 64, 688),
    "7b_s16k_d8": Workload(1, "7b_s16k_d8", 1, 16384, 8, 0, 4096, 32, 128, 11008),
    "7b_s32k_d8": Workload(2, "7b_s32k_d8", 1, 32768, 8, 0, 4096, 32, 128, 11008),
    "7b_s128k_d8": Workload(3, "7b_s128k_d8", 1, 131072, 8, 0, 4096, 32, 128, 11008),
    "7b_b4_s64k_d8": Workload(4, "7b_b4_s64k_d8", 4, 65536, 8, 0, 4096, 32, 128, 11008),
}


def round_bf16_bits(f32):
    """float32 array -> uint16 bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def normal_bf16(shape, seed, std=1.0):
    """Seeded N(0, std^2) draws rounded to bf16, as uint16 bit patterns."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        draw = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            draw *= np.float32(std)
        out[s:e] = round_bf16_bits(draw)
    return out.reshape(shape)


def to_f64(bits):
    """bf16 bit patterns -> exact float64 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f32(bits):
    """bf16 bit patterns -> exact float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_torch(bits):
    """bf16 bit patterns -> CPU torch.bfloat16 tensor sharing the values."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def layer_inputs(w, std_w=0.02):
    """All inputs of a workload: X_full and the full weights, as bf16 bit arrays.

    Shapes: x_full [B,S,d]; w_qkv [3d,d]; w_o [d,d]; w1, w3 [F,d]; w2 [d,F].
    """
    d, F = w.d_model, w.ffn
    base = 1000 * w.wid
    return {
        "x_full": normal_bf16((w.B, w.S, d), base + 1, 1.0),
        "w_qkv": normal_bf16((3 * d, d), base + 2, std_w),
        "w_o": normal_bf16((d, d), base + 3, std_w),
        "w1": normal_bf16((F, d), base + 4, std_w),
        "w3": normal_bf16((F, d), base + 5, std_w),
        "w2": normal_bf16((d, F), base + 6, std_w),
    }
