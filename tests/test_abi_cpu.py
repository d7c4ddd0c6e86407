"""CPU checks of the C ABI: every declared symbol is exported, the host-only zigzag map is
bit-exact against the oracle, and invalid arguments return the documented status before
any HIP call. No test here launches a kernel: every compute entry point is called with
arguments its host-side checks reject."""

import ctypes
import os
import re

import numpy as np
import pytest

from long_context_transformer_amd import tsp
from oracle import tsp_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(tsp.LIB_PATH),
                                reason="libtsp.so not built (python -m long_context_transformer_amd.build)")

# Fake device addresses: 16-byte aligned, never dereferenced (every call below fails a
# host check first).
A = 0x7F0000000000
MIS = A + 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tsp_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_contract_entry_points():
    names = declared_functions()
    for required in ("tsp_zigzag_index", "tsp_attn_fwd", "tsp_mlp_shard_accum", "tsp_layer_fwd"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tsp.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_clean_error():
    assert tsp.version() >> 16 == 1
    tsp.zigzag_index(64, 2, 1)
    assert tsp.load().tsp_last_error() == b""


@pytest.mark.parametrize("S,D", [(256, 4), (16384, 8), (131072, 8), (48, 3), (64, 1), (40, 5)])
def test_zigzag_bit_exact_vs_oracle(S, D):
    for r in range(D):
        np.testing.assert_array_equal(tsp.zigzag_index(S, D, r), tsp_oracle.zigzag_index(S, D, r))


def _code(fn, *args):
    with pytest.raises(tsp.TspError) as e:
        fn(*args)
    return e.value.code


def test_zigzag_errors():
    lib = tsp.load()
    buf = np.zeros(64, dtype=np.int64)
    assert lib.tsp_zigzag_index(256, 4, 0, None, 64) == 1
    assert lib.tsp_zigzag_index(250, 4, 0, buf.ctypes.data, 64) == 2
    assert lib.tsp_zigzag_index(256, 4, 4, buf.ctypes.data, 64) == 3
    assert lib.tsp_zigzag_index(256, 4, -1, buf.ctypes.data, 64) == 3
    assert lib.tsp_zigzag_index(256, 4, 0, buf.ctypes.data, 63) == 2
    assert lib.tsp_zigzag_index(256, 0, 0, buf.ctypes.data, 64) == 2
    assert b"rank" in lib.tsp_last_error() or b"idx_len" in lib.tsp_last_error() or lib.tsp_last_error()


def test_attn_errors():
    f = tsp.attn_fwd
    assert _code(f, None, A, A, A, None, 1, 256, 4, 0, 4, 64, 0.0, 0) == 1
    assert _code(f, A, A, A, A, None, 1, 250, 4, 0, 4, 64, 0.0, 0) == 2
    assert _code(f, A, A, A, A, None, -1, 256, 4, 0, 4, 64, 0.0, 0) == 2
    assert _code(f, A, A, A, A, None, 1, 256, 4, 5, 4, 64, 0.0, 0) == 3
    assert _code(f, A, A, A, A, None, 1, 256, 4, 0, 4, 96, 0.0, 0) == 4
    assert _code(f, A, MIS, A, A, None, 1, 256, 4, 0, 4, 64, 0.0, 0) == 6
    assert _code(f, A, A, A, A, A + 2, 1, 256, 4, 0, 4, 64, 0.0, 0) == 6
    assert _code(f, A, A, A, A, None, 1, 256, 4, 0, 4, 64, float("nan"), 0) == 2


def test_attn_range_and_merge_errors():
    f = tsp.attn_fwd_range
    args = (A, A, A, A, A + 16)
    assert _code(f, *args, 1, 256, 4, 0, 4, 64, -1, 10, 0.0, 0) == 2     # key_lo < 0
    assert _code(f, *args, 1, 256, 4, 0, 4, 64, 20, 10, 0.0, 0) == 2     # key_lo > key_hi
    assert _code(f, *args, 1, 256, 4, 0, 4, 64, 0, 257, 0.0, 0) == 2     # key_hi > S
    assert _code(f, *args, 1, 256, 4, 9, 4, 64, 0, 256, 0.0, 0) == 3
    assert _code(f, None, A, A, A, A, 1, 256, 4, 0, 4, 64, 0, 256, 0.0, 0) == 1
    assert _code(f, A, A, A, MIS, A, 1, 256, 4, 0, 4, 64, 0, 256, 0.0, 0) == 6
    assert _code(f, A, A, A, A, A + 2, 1, 256, 4, 0, 4, 64, 0, 256, 0.0, 0) == 6
    f(None, None, None, None, None, 0, 256, 4, 0, 4, 64, 0, 256)          # empty batch: no-op
    m = tsp.attn_merge
    assert _code(m, A, A + 16, A + 32, A + 48, None, 1, 250, 4, 4, 64) == 2
    assert _code(m, None, A, A, A, None, 1, 256, 4, 4, 64) == 1
    assert _code(m, A, A + 16, A, A + 48, None, 1, 256, 4, 4, 64) == 2   # partial aliases accumulator
    assert _code(m, A, A + 16, A + 32, A + 48, MIS, 1, 256, 4, 4, 64) == 6
    m(None, None, None, None, None, 0, 256, 4, 4, 64)


def test_qkv_errors():
    f = tsp.qkv_fwd
    assert _code(f, A, None, None, A, A, 1, 256, 4, 0, 4, 64, 0) == 1
    assert _code(f, A, A, None, A, A, 1, 256, 3, 0, 4, 64, 0) == 2
    assert _code(f, A, A, None, A, A, 1, 256, 4, 0, 4, 32, 0) == 4
    assert _code(f, A, A, MIS, A, A, 1, 256, 4, 0, 4, 64, 0) == 6


def test_mlp_errors():
    f = tsp.mlp_shard_accum
    need = tsp.mlp_workspace_size(64, 172)
    assert need >= 64 * 176 * 2
    assert _code(f, A, A, A, None, 172, A, 64, 256, 172, 0, A, need, 0) == 1
    assert _code(f, A, A, A, A, 171, A, 64, 256, 172, 0, A, need, 0) == 2
    assert _code(f, A, A, A, A, 172, A, -1, 256, 172, 0, A, need, 0) == 2
    assert _code(f, A, A, A, A, 172, A, 64, 256, 0, 0, A, need, 0) == 2
    assert _code(f, A, A, A, A, 172, MIS, 64, 256, 172, 0, A, need, 0) == 6
    assert _code(f, A, A, A, A, 172, A, 64, 256, 172, 0, A, need - 1, 0) == 5
    assert tsp.mlp_workspace_size(0, 172) == 0


def test_mlp_noalloc_errors():
    """The allocation-free MLP step: the same argument checks as the workspace form, and a
    call whose gated hidden exceeds the scratch maximum is refused before any HIP call."""
    f = tsp.load().tsp_mlp_shard_accum_noalloc
    cap = tsp.mlp_noalloc_max_bytes()
    assert cap == 64 << 20
    assert f(A, A, A, None, 172, A, 64, 256, 172, 0, None) == 1
    assert f(A, A, A, A, 171, A, 64, 256, 172, 0, None) == 2
    assert f(A, A, A, A, 172, A, -1, 256, 172, 0, None) == 2
    assert f(A, A, A, A, 172, MIS, 64, 256, 172, 0, None) == 6
    rows = cap // (1408 * 2)                         # 23831 rows of the 7B shard width fit (stride 1408)
    assert tsp.mlp_workspace_size(rows, 1376) <= cap < tsp.mlp_workspace_size(rows + 1, 1376)
    assert f(A, A, A, A, 1376, A, rows + 1, 4096, 1376, 0, None) == 5
    assert b"maximum" in tsp.load().tsp_last_error()
    assert f(None, None, None, None, 1376, None, 0, 4096, 1376, 0, None) == 0  # empty: no device access


def _desc(**kw):
    base = dict(B=1, S=256, D=4, rank=0, d_model=256, n_heads=4, head_dim=64, ffn=688)
    base.update(kw)
    return tsp.make_desc(**base)


def test_layer_desc_and_workspace():
    assert ctypes.sizeof(tsp.LayerDesc) == 56
    good = _desc()
    M = 64
    ws = tsp.layer_workspace_size(good)
    assert ws >= 2 * M * 256 * 2 + M * 176 * 2
    assert tsp.layer_workspace_size(_desc(ffn=690)) == 0      # F % D != 0
    assert tsp.layer_workspace_size(_desc(d_model=250)) == 0  # d != H*hd
    assert tsp.layer_workspace_size(_desc(head_dim=80, d_model=320)) == 0
    assert tsp.layer_workspace_size(_desc(rank=4)) == 0
    assert tsp.layer_workspace_size(_desc(S=2**31, D=8, ffn=1024)) == 0  # key positions beyond 32 bits
    assert tsp.layer_workspace_size(_desc(S=2**29, D=8, ffn=1024)) > 0


def test_layer_errors():
    good = _desc()
    ws = tsp.layer_workspace_size(good)
    sh = [A] * 4
    f = tsp.layer_fwd
    assert _code(f, _desc(S=100), A, A, A, sh, sh, sh, A, A, A, A, A, ws, 0) == 2
    assert _code(f, _desc(rank=7), A, A, A, sh, sh, sh, A, A, A, A, A, ws, 0) == 3
    assert _code(f, good, None, A, A, sh, sh, sh, A, A, A, A, A, ws, 0) == 1
    assert _code(f, good, A, A, A, [A, A, None, A], sh, sh, A, A, A, A, A, ws, 0) == 1
    assert _code(f, good, A, A, A, sh, [A, MIS, A, A], sh, A, A, A, A, A, ws, 0) == 6
    assert _code(f, good, A, A, A, sh, sh, sh, A, A, A, A, A, ws - 16, 0) == 5
    assert _code(f, _desc(w2_ld=100), A, A, A, sh, sh, sh, A, A, A, A, A, ws, 0) == 2
    bad = _desc()
    bad.reserved = 1
    assert _code(f, bad, A, A, A, sh, sh, sh, A, A, A, A, A, ws, 0) == 2


def test_attn_bwd_errors():
    f = tsp.attn_bwd
    ws = tsp.attn_bwd_workspace_size(1, 256, 4, 2)
    assert ws == 1 * 2 * 64 * 4 and tsp.attn_bwd_workspace_size(1, 250, 4, 2) == 0
    good = [A] * 9
    shape = (1, 256, 4, 0, 2, 64)  # B, S, D, rank, H, hd
    assert _code(f, *good, 1, 250, 4, 0, 2, 64, A, ws) == 2
    assert _code(f, *good, 1, 256, 4, 4, 2, 64, A, ws) == 3
    assert _code(f, *good, 1, 256, 4, 0, 2, 80, A, ws) == 4
    assert _code(f, *([A] * 4 + [None] + [A] * 4), *shape, A, ws) == 1   # lse
    assert _code(f, *([A] * 6 + [MIS] + [A] * 2), *shape, A, ws) == 6    # dq
    assert _code(f, *good, *shape, A, ws - 4) == 5
    f(*[None] * 9, 0, 256, 4, 1, 2, 64, None, 0)              # empty problem: OK, nothing read


def test_layer_bwd_errors():
    good = _desc()
    ws = tsp.layer_bwd_workspace_size(good)
    assert ws > 0 and tsp.layer_bwd_workspace_size(_desc(ffn=690)) == 0
    sh = [A] * 4
    f1, f2 = tsp.layer_bwd_attn_mlp, tsp.layer_bwd_qkv
    p1 = [A] * 6  # q, o, lse, k_full, v_full, w_o
    assert _code(f1, _desc(S=100), *p1, sh, A, A, A, A, A, sh, sh, A, ws, 0) == 2
    assert _code(f1, _desc(rank=4), *p1, sh, A, A, A, A, A, sh, sh, A, ws, 0) == 3
    assert _code(f1, good, *p1, [A, None, A, A], A, A, A, A, A, sh, sh, A, ws, 0) == 1
    assert _code(f1, good, *p1, sh, A, A, A, A, A, sh, [A, A, MIS, A], A, ws, 0) == 6
    assert _code(f1, good, *p1, sh, A, A, A, A, A, sh, sh, A, ws - 1, 0) == 5
    assert _code(f2, good, A, A, A, A, A, A, A, A, ws - 1, 0) == 5
    assert _code(f2, good, A, A, None, A, A, A, A, A, ws, 0) == 1
    assert _code(f2, good, A, A, A, A, A, MIS, A, A, ws, 0) == 6
    e = _desc(B=0)
    f1(e, *[None] * 6, [None] * 4, None, None, None, None, None, [None] * 4, [None] * 4, None, 0)
    f2(e, *[None] * 8, 0)


def test_streamed_layer_workspace_and_errors():
    rup = lambda x: (x + 255) // 256 * 256

    def want(M, d, Fs, fp, fh, dg, hg, odd):
        act = M * d * 2
        # the lone last head group of an odd D: two key halves, fp32 O and lse
        part = rup(2 * M * dg * 4) + rup(2 * M * hg * 4) if odd else 0
        hid = rup(M * (1 if odd and dg == d else 2) * fh * 2)   # two shards' gated hidden (one if D = 1)
        return (2 * rup(act) + hid + 2 * rup(4 * dg * d * 2) + 2 * rup((2 * Fs + fp) * d * 2) + part)

    good = _desc()
    ws = tsp.layer_streamed_workspace_size(good)
    assert ws == want(64, 256, 172, 176, 192, 64, 1, False)   # D = 4: pairs of groups only
    assert tsp.layer_streamed_workspace_size(_desc(D=1, rank=0)) == want(256, 256, 688, 688, 704, 256, 4, True)
    # H % D != 0: a head group must hold whole heads
    assert tsp.layer_streamed_workspace_size(_desc(n_heads=2, head_dim=128)) == 0
    sh = [A] * 4
    f = tsp.layer_fwd_streamed
    assert _code(f, _desc(n_heads=2, head_dim=128), A, sh, sh, A, A, A, A, A, ws, 0) == 2
    assert _code(f, _desc(S=100), A, sh, sh, A, A, A, A, A, ws, 0) == 2
    assert _code(f, _desc(rank=5), A, sh, sh, A, A, A, A, A, ws, 0) == 3
    assert _code(f, good, A, [A, None, A, A], sh, A, A, A, A, A, ws, 0) == 1
    assert _code(f, good, A, sh, [A, A, A, MIS], A, A, A, A, A, ws, 0) == 6
    assert _code(f, good, A, sh, sh, A, A, MIS, A, A, ws, 0) == 6
    assert _code(f, good, A, sh, sh, A, A, A, None, A, ws, 0) == 1
    assert _code(f, good, A, sh, sh, A, A, A, A, A, ws - 1, 0) == 5
    with pytest.raises(ValueError):  # the binding takes exactly three extra streams
        f(good, A, sh, sh, A, A, A, A, A, ws, 0, [0, 0])
    lib = tsp.load()
    arr = (ctypes.c_void_p * 4)()
    aa = (ctypes.c_void_p * 4)(*([A] * 4))
    for n in (0, 2, 3, 5):
        assert lib.tsp_layer_fwd_streamed(ctypes.byref(good), A, aa, aa, A, A, A, A, A, ws, arr, n) == 2
    assert lib.tsp_layer_fwd_streamed(ctypes.byref(good), A, aa, aa, A, A, A, A, A, ws, None, 1) == 1
    tsp.layer_fwd_streamed(_desc(B=0), None, [None] * 4, [None] * 4, None, None, None, None, None, 0)


def test_empty_problems_are_noops():
    """B = 0, S = 0 or M = 0: shape checks still apply, then TSP_OK with no pointer read
    (NULL pointers, as torch gives for empty tensors) and no launch (none can happen here:
    there is no GPU)."""
    lib = tsp.load()
    assert lib.tsp_zigzag_index(0, 4, 1, None, 0) == 0
    assert lib.tsp_zigzag_index(0, 4, 4, None, 0) == 3
    assert tsp.zigzag_index(0, 4, 1).shape == (0,)
    tsp.attn_fwd(None, None, None, None, None, 0, 256, 4, 0, 4, 64)
    tsp.attn_fwd(None, None, None, None, None, 2, 0, 4, 3, 4, 64)
    assert _code(tsp.attn_fwd, None, None, None, None, None, 0, 250, 4, 0, 4, 64, 0.0, 0) == 2
    assert _code(tsp.attn_fwd, None, None, None, None, None, 0, 256, 4, 0, 4, 80, 0.0, 0) == 4
    tsp.qkv_fwd(None, None, None, None, None, 0, 256, 4, 0, 4, 64)
    tsp.mlp_shard_accum(None, None, None, None, 172, None, 0, 256, 172, 0, None, 0)
    empty = _desc(B=0)
    assert tsp.layer_workspace_size(empty) == 0
    tsp.layer_fwd(empty, None, None, None, [None] * 4, [None] * 4, [None] * 4, None, None, None,
                  None, None, 0)
    assert _code(tsp.layer_fwd, _desc(B=0, rank=4), None, None, None, [None] * 4, [None] * 4,
                 [None] * 4, None, None, None, None, None, 0, 0) == 3


def test_timing_hook_errors():
    lib = tsp.load()
    n = ctypes.c_int32(5)
    assert lib.tsp_timing_start(-1) == 2
    assert lib.tsp_timing_start(0) == 0
    assert lib.tsp_timing_read(None, 4, ctypes.byref(n)) == 1
    assert lib.tsp_timing_read(None, 0, None) == 1
    assert lib.tsp_timing_read(None, 0, ctypes.byref(n)) == 0 and n.value == 0


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(4, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        tsp.attn_fwd(x, x, x, x, None, 1, 256, 4, 0, 4, 64)
