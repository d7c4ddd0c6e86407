"""GPU check of the allocation-free MLP ring step (tsp_mlp_shard_accum_noalloc) against the
workspace form (tsp_mlp_shard_accum), through the C ABI.

Two calls in a row on one stream, the second with a smaller, different input (so the scratch
still holds the first call's larger hidden): each must equal the workspace form's output
bit for bit (the same kernels on the same inputs), the second must also match the fp64
oracle within the contract (max-abs <= 2e-2 max|ref|, mean-abs <= 2e-3 max|ref|), and after
the one-time set-up of the first call on the device, a call must not change the device's free
memory. One ring step of the gated MLP: summary of
"Folding Tensor and Sequence Parallelism for Memory-Efficient Transformer Training &
Inference" (gist.science 2604.26294), §2 gated MLP layers.
"""

import numpy as np
import pytest
import torch

from long_context_transformer_amd import synth, tsp
from oracle import tsp_oracle as O

from _gpu_helpers import check_close, dev_bf16, host_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tsp.load()


def shard_inputs(M, d, Fs, seed):
    x = synth.normal_bf16((M, d), seed)
    w1 = synth.normal_bf16((Fs, d), seed + 1, 0.02)
    w3 = synth.normal_bf16((Fs, d), seed + 2, 0.02)
    w2 = synth.normal_bf16((d, Fs), seed + 3, 0.02)
    acc0 = np.random.default_rng(seed + 4).standard_normal((M, d)).astype(np.float32)
    return x, w1, w3, w2, acc0


def test_noalloc_matches_workspace_form_twice():
    # The first call on a device looks up the device's scratch address; the HIP runtime
    # materialises the library's device global then (once per device, held until the process
    # ends). After that set-up, calls change no device memory.
    x0 = torch.zeros((16, 256), dtype=torch.bfloat16, device="cuda")
    w0 = torch.zeros((64, 256), dtype=torch.bfloat16, device="cuda")
    w20 = torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda")
    a0 = torch.zeros((16, 256), device="cuda")
    tsp.mlp_shard_accum_noalloc(x0, w0, w0, w20, 64, a0, 16, 256, 64, 0)
    torch.cuda.synchronize()
    assert bool((a0 == 0).all())
    calls = [  # M, d, Fs, accumulate, seed: the 7B shard width; the second call smaller
        (8192, 4096, 1376, 0, 9500),
        (3000, 4096, 1376, 1, 9600),
    ]
    for n, (M, d, Fs, accum, seed) in enumerate(calls):
        print(f"no-alloc MLP step, call {n}: M={M} d={d} Fs={Fs} accumulate={accum}", flush=True)
        assert tsp.mlp_workspace_size(M, Fs) <= tsp.mlp_noalloc_max_bytes()
        x, w1, w3, w2, acc0 = shard_inputs(M, d, Fs, seed)
        xd, w1d, w3d, w2d = dev_bf16(x), dev_bf16(w1), dev_bf16(w3), dev_bf16(w2)
        ref = torch.from_numpy(acc0).cuda()
        got = ref.clone()
        ws = torch.empty(tsp.mlp_workspace_size(M, Fs), dtype=torch.uint8, device="cuda")
        tsp.mlp_shard_accum(xd, w1d, w3d, w2d, Fs, ref, M, d, Fs, accum, ws)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        tsp.mlp_shard_accum_noalloc(xd, w1d, w3d, w2d, Fs, got, M, d, Fs, accum)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0, "the allocation-free call changed free device memory"
        assert bool(torch.isfinite(got).all())
        assert torch.equal(got, ref), f"call {n}: differs from the workspace form"
        if n == len(calls) - 1:
            part = O.mlp_shard_partial(synth.to_f64(x), synth.to_f64(w1), synth.to_f64(w3), synth.to_f64(w2), 0, 1)
            check_close(f"call {n} vs oracle", host_f64(got), acc0.astype(np.float64) * accum + part)


def test_noalloc_refuses_oversized_call():
    """A call whose hidden exceeds the scratch maximum fails with TSP_ERR_WORKSPACE and
    launches nothing (the output is untouched)."""
    d, Fs = 256, 1376
    M = tsp.mlp_noalloc_max_bytes() // (Fs * 2) + 1
    x = torch.zeros((M, d), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((Fs, d), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((d, Fs), dtype=torch.bfloat16, device="cuda")
    acc = torch.full((M, d), 3.0, device="cuda")
    with pytest.raises(tsp.TspError) as ex:
        tsp.mlp_shard_accum_noalloc(x, w, w, w2, Fs, acc, M, d, Fs, 0)
    assert ex.value.code == 5
    torch.cuda.synchronize()
    assert bool((acc == 3.0).all())
