"""Python binding of libtsp.so (the C ABI in include/tsp.h): argument marshalling only.

Every function takes device tensors (torch, on a ROCm GPU) or raw integer device
addresses, passes pointers and sizes to the library, and raises TspError on a non-OK
status. No arithmetic of the layer happens here; every step runs in the library's
HIP kernels. If libtsp.so is missing the import of this module still works, but the
first call raises: there is no fallback path.
"""

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# TSP_LIBRARY selects another build of the same library (the sanitized host build of the CPU
# tests); by default the in-tree libtsp.so.
LIB_PATH = os.environ.get("TSP_LIBRARY") or os.path.join(_PKG, "libtsp.so")

TSP_OK = 0
STATUS_NAMES = {0: "TSP_OK", 1: "TSP_ERR_NULL", 2: "TSP_ERR_SHAPE", 3: "TSP_ERR_RANK",
                4: "TSP_ERR_UNSUPPORTED", 5: "TSP_ERR_WORKSPACE", 6: "TSP_ERR_ALIGN",
                7: "TSP_ERR_HIP"}


class TspError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {msg}")
        self.code = code


class LayerDesc(ctypes.Structure):
    """Mirror of tsp_layer_desc."""
    _fields_ = [("batch", ctypes.c_int32), ("fold", ctypes.c_int32), ("seq_len", ctypes.c_int64),
                ("rank", ctypes.c_int32), ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("w2_ld", ctypes.c_int64), ("scale", ctypes.c_float)]


_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SIGS = {
    "tsp_version": (_I32, []),
    "tsp_last_error": (ctypes.c_char_p, []),
    "tsp_zigzag_index": (_I32, [_I64, _I32, _I32, _VP, _I64]),
    "tsp_qkv_fwd": (_I32, [_VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I32, _I32, _VP]),
    "tsp_attn_fwd": (_I32, [_VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I32, _I32,
                            ctypes.c_float, _VP]),
    "tsp_mlp_workspace_size": (ctypes.c_size_t, [_I64, _I32]),
    "tsp_mlp_shard_accum": (_I32, [_VP, _VP, _VP, _VP, _I64, _VP, _I64, _I32, _I32, _I32, _VP,
                                   ctypes.c_size_t, _VP]),
    "tsp_mlp_noalloc_max_bytes": (ctypes.c_size_t, []),
    "tsp_mlp_shard_accum_noalloc": (_I32, [_VP, _VP, _VP, _VP, _I64, _VP, _I64, _I32, _I32, _I32, _VP]),
    "tsp_layer_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc)]),
    "tsp_layer_fwd": (_I32, [ctypes.POINTER(LayerDesc), _VP, _VP, _VP, ctypes.POINTER(_VP),
                             ctypes.POINTER(_VP), ctypes.POINTER(_VP), _VP, _VP, _VP, _VP, _VP,
                             ctypes.c_size_t, _VP]),
    "tsp_attn_fwd_range": (_I32, [_VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I32, _I32,
                                  ctypes.c_float, _I64, _I64, _I32, _VP, _VP]),
    "tsp_attn_merge": (_I32, [_VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I32, _VP]),
    "tsp_layer_streamed_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc)]),
    "tsp_layer_fwd_streamed": (_I32, [ctypes.POINTER(LayerDesc), _VP, ctypes.POINTER(_VP),
                                      ctypes.POINTER(_VP), _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t,
                                      ctypes.POINTER(_VP), _I32]),
    "tsp_attn_bwd_workspace_size": (ctypes.c_size_t, [_I32, _I64, _I32, _I32]),
    "tsp_attn_bwd": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I64, _I32, _I32, _I32, _I32,
                            ctypes.c_float, _VP, ctypes.c_size_t, _VP]),
    "tsp_layer_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(LayerDesc)]),
    "tsp_layer_bwd_attn_mlp": (_I32, [ctypes.POINTER(LayerDesc), _VP, _VP, _VP, _VP, _VP, _VP,
                                      ctypes.POINTER(_VP), _VP, _VP, _VP, _VP, _VP, ctypes.POINTER(_VP),
                                      ctypes.POINTER(_VP), _VP, ctypes.c_size_t, _VP]),
    "tsp_layer_bwd_qkv": (_I32, [ctypes.POINTER(LayerDesc), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                 ctypes.c_size_t, _VP]),
    "tsp_timing_start": (_I32, [_I32]),
    "tsp_timing_read": (_I32, [ctypes.POINTER(ctypes.c_float), _I32, ctypes.POINTER(_I32)]),
}

_lib = None


def load(path=None):
    """Load libtsp.so (once). Raises OSError if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} not found: build it with `python -m long_context_transformer_amd.build`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(code):
    if code != TSP_OK:
        raise TspError(code, load().tsp_last_error().decode())


def _ptr(t):
    """Device address of a tensor (must live on a GPU) or pass through an int / None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not getattr(t, "is_cuda", False):
        raise TypeError("expected a GPU tensor (or a raw device address)")
    if not t.is_contiguous():
        raise TypeError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    for t in tensors:
        if getattr(t, "is_cuda", False):
            import torch
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def version():
    return load().tsp_version()


def zigzag_index(S, D, rank):
    """Global positions of a rank's local rows (host computation, int64 numpy)."""
    out = np.empty(S // D if D > 0 else 0, dtype=np.int64)
    _check(load().tsp_zigzag_index(S, D, rank, out.ctypes.data if out.size else None, out.size))
    return out


def qkv_fwd(x, w_qkv, q_out, k_full, v_full, B, S, D, rank, n_heads, head_dim, stream=None):
    _check(load().tsp_qkv_fwd(_ptr(x), _ptr(w_qkv), _ptr(q_out), _ptr(k_full), _ptr(v_full), B, S, D,
                              rank, n_heads, head_dim, _stream(stream, x)))


def attn_fwd(q, k_full, v_full, o, lse, B, S, D, rank, n_heads, head_dim, scale=0.0, stream=None):
    _check(load().tsp_attn_fwd(_ptr(q), _ptr(k_full), _ptr(v_full), _ptr(o), _ptr(lse), B, S, D, rank,
                               n_heads, head_dim, scale, _stream(stream, q)))


def attn_fwd_range(q, k_full, v_full, o_part, lse_part, B, S, D, rank, n_heads, head_dim, key_lo,
                   key_hi, scale=0.0, accumulate=False, o_out=None, stream=None):
    """Attention of the rank's queries against key positions [key_lo, key_hi): fp32 o_part
    [B, 2C, H, hd] and lse_part [B, H, 2C] (0 and -inf for rows with no visible key), or
    merged into them when accumulate; o_out (bf16 or None) receives the resulting O."""
    _check(load().tsp_attn_fwd_range(_ptr(q), _ptr(k_full), _ptr(v_full), _ptr(o_part), _ptr(lse_part), B, S,
                                     D, rank, n_heads, head_dim, scale, key_lo, key_hi, 1 if accumulate else 0,
                                     _ptr(o_out), _stream(stream, q)))


def attn_merge(o_acc, lse_acc, o_part, lse_part, o_out, B, S, D, n_heads, head_dim, stream=None):
    """(o_acc, lse_acc) <- log-sum-exp merge with (o_part, lse_part); o_out (bf16 or None)
    receives the merged O."""
    _check(load().tsp_attn_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part), _ptr(o_out), B, S, D,
                                 n_heads, head_dim, _stream(stream, o_acc)))


def attn_bwd_workspace_size(B, S, D, n_heads):
    return int(load().tsp_attn_bwd_workspace_size(int(B), int(S), int(D), int(n_heads)))


def attn_bwd(q, k_full, v_full, o, lse, d_o, dq, dk_full, dv_full, B, S, D, rank, n_heads, head_dim, ws,
             ws_bytes=None, scale=0.0, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None and not isinstance(ws, int) else 0
    _check(load().tsp_attn_bwd(_ptr(q), _ptr(k_full), _ptr(v_full), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq),
                               _ptr(dk_full), _ptr(dv_full), B, S, D, rank, n_heads, head_dim, float(scale),
                               _ptr(ws), ws_bytes, _stream(stream, q)))


def mlp_workspace_size(M, Fs):
    return int(load().tsp_mlp_workspace_size(M, Fs))


def mlp_shard_accum(x, w1_j, w3_j, w2_j, ld_w2, acc, M, d, Fs, accumulate, ws, ws_bytes=None,
                    stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load().tsp_mlp_shard_accum(_ptr(x), _ptr(w1_j), _ptr(w3_j), _ptr(w2_j), ld_w2, _ptr(acc), M,
                                      d, Fs, 1 if accumulate else 0, _ptr(ws), ws_bytes,
                                      _stream(stream, x)))


def mlp_noalloc_max_bytes():
    return int(load().tsp_mlp_noalloc_max_bytes())


def mlp_shard_accum_noalloc(x, w1_j, w3_j, w2_j, ld_w2, acc, M, d, Fs, accumulate, stream=None):
    _check(load().tsp_mlp_shard_accum_noalloc(_ptr(x), _ptr(w1_j), _ptr(w3_j), _ptr(w2_j), ld_w2, _ptr(acc), M,
                                              d, Fs, 1 if accumulate else 0, _stream(stream, x)))


def make_desc(B, S, D, rank, d_model, n_heads, head_dim, ffn, w2_ld=0, scale=0.0):
    return LayerDesc(B, D, S, rank, d_model, n_heads, head_dim, ffn, 0, w2_ld, scale)


def layer_workspace_size(desc):
    return int(load().tsp_layer_workspace_size(ctypes.byref(desc)))


def layer_fwd(desc, x_shard, w_qkv, w_o, w1, w3, w2, k_full, v_full, attn_out, mlp_out, ws,
              ws_bytes=None, stream=None):
    """w1, w3, w2: sequences of D shard tensors (or addresses), indexed by shard id."""
    D = desc.fold
    arr = _VP * D
    a1 = arr(*[_ptr(t) for t in w1])
    a3 = arr(*[_ptr(t) for t in w3])
    a2 = arr(*[_ptr(t) for t in w2])
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(load().tsp_layer_fwd(ctypes.byref(desc), _ptr(x_shard), _ptr(w_qkv), _ptr(w_o), a1, a3, a2,
                                _ptr(k_full), _ptr(v_full), _ptr(attn_out), _ptr(mlp_out), _ptr(ws),
                                ws_bytes, _stream(stream, x_shard)))


def layer_streamed_workspace_size(desc):
    return int(load().tsp_layer_streamed_workspace_size(ctypes.byref(desc)))


def layer_fwd_streamed(desc, x_shard, w_attn, w_mlp, k_full, v_full, attn_out, mlp_out, ws,
                       ws_bytes=None, stream=None, streams=None):
    """w_attn, w_mlp: sequences of D packed shards (pack_attn_shards / pack_mlp_shards).
    streams: None (everything on `stream`, no overlap) or three more streams: the second
    attention stream, the W_O stream and the copy stream."""
    D = desc.fold
    arr = _VP * D
    aa = arr(*[_ptr(t) for t in w_attn])
    am = arr(*[_ptr(t) for t in w_mlp])
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    st = _stream(stream, x_shard)
    if streams is None:
        sv, n = (_VP * 1)(st), 1
    else:
        if len(streams) != 3:
            raise ValueError("streams: the second attention stream, the W_O stream, the copy stream")
        sv, n = (_VP * 4)(st, *[_stream(x) for x in streams]), 4
    _check(load().tsp_layer_fwd_streamed(ctypes.byref(desc), _ptr(x_shard), aa, am, _ptr(k_full),
                                         _ptr(v_full), _ptr(attn_out), _ptr(mlp_out), _ptr(ws),
                                         ws_bytes, sv, n))


def pack_attn_shards(w_qkv, w_o, D):
    """Weight layout helper: the D packed attention shards of a [3d, d] W_qkv (Q, K, V row
    blocks) and a [d, d] W_o, as contiguous bf16 tensors of 4 (d/D) d elements each: the
    group's W_q, W_k, W_v rows, then its W_o columns as a [d, d/D] row-major block."""
    import torch
    d = w_o.shape[0]
    dg = d // D
    out = []
    for j in range(D):
        rows = [w_qkv[p * d + j * dg:p * d + (j + 1) * dg] for p in range(3)]
        cols = w_o[:, j * dg:(j + 1) * dg].contiguous()
        out.append(torch.cat([r.reshape(-1) for r in rows] + [cols.reshape(-1)]).contiguous())
    return out


def pack_mlp_shards(w1, w3, w2, D):
    """Weight layout helper: the D packed MLP shards of W1, W3 [F, d] and W2 [d, F], as
    contiguous bf16 tensors: shard j's W1 rows, W3 rows ([F/D, d] each), then its W2
    columns as [d, F/D] with row stride round_up(F/D, 8) (pad columns zero)."""
    import torch
    F, d = w1.shape
    Fs = F // D
    fp = (Fs + 7) // 8 * 8
    out = []
    for j in range(D):
        sl = slice(j * Fs, (j + 1) * Fs)
        w2p = torch.zeros((d, fp), dtype=w2.dtype, device=w2.device)
        w2p[:, :Fs] = w2[:, sl]
        out.append(torch.cat([w1[sl].reshape(-1), w3[sl].reshape(-1), w2p.reshape(-1)]).contiguous())
    return out


def layer_bwd_workspace_size(desc):
    return int(load().tsp_layer_bwd_workspace_size(ctypes.byref(desc)))


def layer_bwd_attn_mlp(desc, q, o, lse, k_full, v_full, w_o, w_mlp, d_y, dq, dk_full, dv_full, dw_o, dw13, dw2,
                       ws, ws_bytes=None, stream=None):
    """w_mlp, dw13, dw2: sequences of D tensors (or addresses) indexed by shard id."""
    D = desc.fold
    arr = _VP * D
    am, a13, a2 = (arr(*[_ptr(t) for t in seq]) for seq in (w_mlp, dw13, dw2))
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None and not isinstance(ws, int) else 0
    _check(load().tsp_layer_bwd_attn_mlp(ctypes.byref(desc), _ptr(q), _ptr(o), _ptr(lse), _ptr(k_full),
                                         _ptr(v_full), _ptr(w_o), am, _ptr(d_y), _ptr(dq), _ptr(dk_full),
                                         _ptr(dv_full), _ptr(dw_o), a13, a2, _ptr(ws), ws_bytes,
                                         _stream(stream, q)))


def layer_bwd_qkv(desc, x_shard, w_qkv, dq, dk_own, dv_own, dx, dw_qkv, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size() if ws is not None and not isinstance(ws, int) else 0
    _check(load().tsp_layer_bwd_qkv(ctypes.byref(desc), _ptr(x_shard), _ptr(w_qkv), _ptr(dq), _ptr(dk_own),
                                    _ptr(dv_own), _ptr(dx), _ptr(dw_qkv), _ptr(ws), ws_bytes,
                                    _stream(stream, x_shard)))


PHASES = ("qkv", "attention", "w_o", "mlp")


def timing_start(max_calls):
    """Arm the library's phase timing for the next `max_calls` layer_fwd calls."""
    _check(load().tsp_timing_start(int(max_calls)))


def timing_read(max_calls):
    """Per-call phase durations (ms) of the armed calls: list of dicts keyed by PHASES."""
    buf = (ctypes.c_float * (4 * max(int(max_calls), 1)))()
    n = _I32(0)
    _check(load().tsp_timing_read(buf, int(max_calls), ctypes.byref(n)))
    return [{p: float(buf[4 * i + k]) for k, p in enumerate(PHASES)} for i in range(n.value)]
