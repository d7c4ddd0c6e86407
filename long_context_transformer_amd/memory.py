"""Per-rank device memory of one layer's forward pass, by layout, in bytes.

Accounting of what one rank holds while it runs one transformer layer forward on D ranks,
for four layouts on the same D:

  tsp_streamed  this library's tsp_layer_fwd_streamed: the rank's own 1/D of the weights
                (its packed attention shard and its packed MLP shard), two receive slots per
                weight kind, 1/D of the tokens, the gathered K/V, and the workspace;
  tsp_resident  this library's tsp_layer_fwd on one GPU: every weight shard resident;
  tp            tensor parallelism alone: 1/D of the weights, every token;
  sp            sequence parallelism alone: every weight, 1/D of the tokens, the gathered K/V.

The pages frame memory as parameter memory plus activation memory, and state that TSP
cuts both by 1/D on one device axis, where TP leaves activations whole and SP leaves
weights whole; the measured result is the lowest peak memory of all strategies at 16K to
128K tokens, equal to TP at short sequences ("Folding Tensor and Sequence Parallelism for
Memory-Efficient Transformer Training & Inference", gist.science 2604.26294, §1 problem
statement, §2 unified sharding, §4 memory efficiency). The pages give no equations, so
every layout here counts the buffers of this library's layer, with its precisions: bf16
weights and activations, fp32 mlp_out, attention that never materialises the S x S
scores. Forward only (no gradients or optimizer state: the pages do not describe the
backward pass).

The tsp_* counts are exact: the workspace terms reproduce tsp_layer_workspace_size and
tsp_layer_streamed_workspace_size byte for byte (a CPU test checks both against the
library).
"""

from dataclasses import dataclass

BF16 = 2
F32 = 4
ALIGN = 256  # the library's workspace carve alignment


def _rup(x, a):
    return (x + a - 1) // a * a


@dataclass(frozen=True)
class Shape:
    B: int
    S: int
    D: int
    d: int
    H: int
    hd: int
    F: int

    @property
    def M(self):
        """Local tokens of one rank: B * S / D."""
        return self.B * self.S // self.D

    @property
    def Fs(self):
        return self.F // self.D

    @property
    def Fp(self):
        """F/D rounded up to a multiple of 8 (W2 row stride in a packed MLP shard)."""
        return _rup(self.Fs, 8)

    @property
    def Fh(self):
        """F/D rounded up to a multiple of 64 (row stride of one shard's gated hidden)."""
        return _rup(self.Fs, 64)

    @property
    def weight_elems(self):
        """All weights of the layer: W_qkv [3d, d], W_o [d, d], W1, W3 [F, d], W2 [d, F]."""
        return 4 * self.d * self.d + 3 * self.d * self.F


def shape_of(w):
    """Shape of a synth.Workload."""
    return Shape(w.B, w.S, w.D, w.d_model, w.n_heads, w.head_dim, w.ffn)


def layer_workspace(s):
    """tsp_layer_workspace_size: Q, O bf16 [M, d]; gated hidden of all D shards; with D even and
    at most 128 output tiles of 256 x 256 in the down projection, an fp32 [M, d] partial sum."""
    act = _rup(s.M * s.d * BF16, ALIGN)
    split = s.D % 2 == 0 and -(-s.M // 256) * -(-s.d // 256) <= 128
    return 2 * act + _rup(s.M * s.D * s.Fh * BF16, ALIGN) + (_rup(s.M * s.d * F32, ALIGN) if split else 0)


def streamed_workspace(s):
    """tsp_layer_streamed_workspace_size: Q, O, the gated hidden of two shards (one if D = 1),
    two attention slots, two MLP slots and, when D is odd, the two fp32 key halves of the lone
    last head group's O and log-sum-exp (pairs of groups write O directly)."""
    dg = s.d // s.D
    hg = s.H // s.D
    act = _rup(s.M * s.d * BF16, ALIGN)
    hid = _rup(s.M * (2 if s.D >= 2 else 1) * s.Fh * BF16, ALIGN)
    slot_a = _rup(4 * dg * s.d * BF16, ALIGN)
    slot_m = _rup((2 * s.Fs + s.Fp) * s.d * BF16, ALIGN)
    part = _rup(2 * s.M * dg * F32, ALIGN) + _rup(2 * s.M * hg * F32, ALIGN)
    return 2 * act + hid + 2 * slot_a + 2 * slot_m + (part if s.D % 2 else 0)


def _io(s):
    """Inputs and outputs every TSP layout holds: x_shard bf16 [M, d], the gathered K and V
    bf16 [B, S, d] each, attn_out bf16 [M, d], mlp_out fp32 [M, d]."""
    return {"x": s.M * s.d * BF16, "kv": 2 * s.B * s.S * s.d * BF16,
            "attn_out": s.M * s.d * BF16, "mlp_out": s.M * s.d * F32}


def tsp_streamed(s):
    own_attn = 4 * (s.d // s.D) * s.d * BF16          # packed attention shard of this rank
    own_mlp = (2 * s.Fs + s.Fp) * s.d * BF16          # packed MLP shard of this rank
    parts = {"weights": own_attn + own_mlp, **_io(s), "workspace": streamed_workspace(s)}
    return parts


def tsp_resident(s):
    parts = {"weights": s.weight_elems * BF16, **_io(s), "workspace": layer_workspace(s)}
    return parts


def tp(s):
    """Tensor parallelism over D: 1/D of every weight, all B*S tokens; the rank's heads' Q, K,
    V and O, the all-reduced attn_out, its F/D columns of the gated hidden, mlp_out."""
    T = s.B * s.S
    return {"weights": s.weight_elems * BF16 // s.D, "x": T * s.d * BF16,
            "qkv": 3 * T * (s.d // s.D) * BF16, "o": T * (s.d // s.D) * BF16,
            "attn_out": T * s.d * BF16, "hidden": T * s.Fs * BF16, "mlp_out": T * s.d * F32}


def sp(s):
    """Sequence parallelism over D: every weight, the rank's M tokens; Q and O of its tokens,
    K and V gathered over the whole sequence, the full-width gated hidden, mlp_out."""
    return {"weights": s.weight_elems * BF16, "x": s.M * s.d * BF16, "q": s.M * s.d * BF16,
            "kv": 2 * s.B * s.S * s.d * BF16, "o": s.M * s.d * BF16, "attn_out": s.M * s.d * BF16,
            "hidden": s.M * s.F * BF16, "mlp_out": s.M * s.d * F32}


LAYOUTS = {"tsp_streamed": tsp_streamed, "tsp_resident": tsp_resident, "tp": tp, "sp": sp}


def per_rank_bytes(s):
    """{layout: total bytes} for one rank of one layer."""
    return {name: sum(fn(s).values()) for name, fn in LAYOUTS.items()}


def model_peak_bytes(s, n_layers):
    """Peak of a forward pass through n_layers identical layers, one at a time: every layer's
    resident weights stay, one layer's activations and workspace are live at once."""
    out = {}
    for name, fn in LAYOUTS.items():
        parts = fn(s)
        out[name] = n_layers * parts["weights"] + sum(v for k, v in parts.items() if k != "weights")
    return out


def max_batch(s, n_layers, capacity, layout):
    """Largest B whose model_peak_bytes fits in `capacity` bytes (0 if even B = 1 does not)."""
    def fits(b):
        t = Shape(b, s.S, s.D, s.d, s.H, s.hd, s.F)
        return model_peak_bytes(t, n_layers)[layout] <= capacity
    if not fits(1):
        return 0
    hi = 1
    while fits(2 * hi):
        hi *= 2
    lo, hi = hi, 2 * hi  # fits(lo), not fits(hi)
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if fits(mid) else (lo, mid)
    return lo


def measure_streamed(w, rank):
    """Device memory of one rank running tsp_layer_fwd_streamed: the buffers the rank owns
    (its tokens, its own packed shards, the gathered K/V, outputs, workspace) as the caching
    allocator counts them, against the analytic count; and the device's free memory across
    a call (after a warmup call), which the library must leave unchanged. The other ranks'
    packed shards (the broadcast and ring sources) are allocated too, but not counted."""
    import torch
    from long_context_transformer_amd import tsp
    s = shape_of(w)
    B, S, D, d = w.B, w.S, w.D, w.d_model
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    desc = tsp.make_desc(B, S, D, rank, d, w.n_heads, w.head_dim, w.ffn)
    shard_a = 4 * (d // D) * d
    shard_m = (2 * s.Fs + s.Fp) * d
    bf = torch.bfloat16
    own = {
        "x": torch.zeros((B, S // D, d), dtype=bf, device="cuda"),
        "attn_shard": torch.zeros(shard_a, dtype=bf, device="cuda"),
        "mlp_shard": torch.zeros(shard_m, dtype=bf, device="cuda"),
        "k": torch.zeros((B, S, d), dtype=bf, device="cuda"),
        "v": torch.zeros((B, S, d), dtype=bf, device="cuda"),
        "attn_out": torch.empty((B, S // D, d), dtype=bf, device="cuda"),
        "mlp_out": torch.empty((B, S // D, d), dtype=torch.float32, device="cuda"),
        "ws": torch.empty(tsp.layer_streamed_workspace_size(desc), dtype=torch.uint8, device="cuda"),
    }
    torch.cuda.synchronize()
    owned = torch.cuda.memory_allocated() - base
    exact = sum(t.numel() * t.element_size() for t in own.values())
    peers_a = [own["attn_shard"] if j == rank else torch.zeros(shard_a, dtype=bf, device="cuda") for j in range(D)]
    peers_m = [own["mlp_shard"] if j == rank else torch.zeros(shard_m, dtype=bf, device="cuda") for j in range(D)]
    streams = [torch.cuda.Stream() for _ in range(3)]

    def call():
        tsp.layer_fwd_streamed(desc, own["x"], peers_a, peers_m, own["k"], own["v"], own["attn_out"],
                               own["mlp_out"], own["ws"], streams=streams)
        torch.cuda.synchronize()

    call()  # warmup: the library creates its events on first use
    free0 = torch.cuda.mem_get_info()[0]
    alloc0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    call()
    free1 = torch.cuda.mem_get_info()[0]
    peak_growth = torch.cuda.max_memory_allocated() - alloc0
    analytic = per_rank_bytes(s)
    res = {"workload": w.name, "rank": rank,
           "measured_owned_bytes": owned, "owned_tensor_bytes": exact,
           "analytic_tsp_streamed_bytes": analytic["tsp_streamed"],
           "free_bytes_change_during_call": free0 - free1, "allocator_peak_growth_during_call": peak_growth,
           "analytic_per_layer_bytes": analytic,
           "analytic_model_peak_bytes_32_layers": model_peak_bytes(s, 32),
           "max_batch_in_288GB_32_layers": {k: max_batch(s, 32, 288 * 10**9, k) for k in LAYOUTS}}
    del own, peers_a, peers_m
    torch.cuda.empty_cache()
    return res
