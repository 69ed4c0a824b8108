"""The allocation-free split-K call (w8a8_gemm_splitk_noalloc) through the C ABI: the same
bits as w8a8_gemm_splitk with a caller workspace, on two calls in a row (the second with a
smaller problem, so stale partial results of the first sit in the scratch), per-channel and
per-group; the single pass when the plan does not split; a clear error when the plan needs
more than the scratch holds."""
import sys

import numpy as np
import pytest
import torch

from synth_inputs import linear_inputs

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20


def note(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def w8a8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_activation_quantized_amd as w
    assert w.w8a8_is_available(0), w.w8a8_last_error()
    w.w8a8_debug_force_config(-1)
    w.w8a8_debug_force_splitk(-1)
    return w


def operands(w8a8, M, N, K, bits, gs, seed):
    x, W = linear_inputs(M, N, K, seed=seed)
    xq, sx = w8a8.quantize_per_token(torch.from_numpy(x).cuda())
    wq, sw = w8a8.quantize_weight(torch.from_numpy(W).cuda(), bits, gs)
    torch.cuda.synchronize()
    return xq, sx, wq, sw


def with_workspace(w8a8, ops, bits, gs, out):
    xq, sx, wq, sw = ops
    M, K = xq.shape
    n = w8a8.w8a8_gemm_splitk_workspace(M, wq.shape[0], K, bits, gs, out)
    ws = torch.empty(max(n, 16) // 4, dtype=torch.int32, device="cuda")
    y = w8a8.w8a8_gemm_splitk(xq, sx, wq, sw, bits, gs, out, workspace=ws)
    torch.cuda.synchronize()
    return n, y


@pytest.mark.parametrize("bits,gs", [(8, 0), (8, 128), (4, 128)])
def test_noalloc_equals_workspace_call_twice(w8a8, bits, gs):
    N, K = 2560, 10240
    for M in (1000, 160):  # second call smaller: the scratch still holds the first call's partials
        ops = operands(w8a8, M, N, K, bits, gs, seed=M + bits + gs)
        for out in (torch.float16, torch.float32):
            n, ref = with_workspace(w8a8, ops, bits, gs, out)
            note(f"noalloc bits={bits} gs={gs} M={M} {out}: split workspace {n} bytes")
            assert 0 < n <= SCRATCH_BYTES, "expected a split plan within the scratch"
            y = torch.full_like(ref, 3.0)
            w8a8.w8a8_gemm_splitk_noalloc(*ops, bits, gs, out, y=y)
            torch.cuda.synchronize()
            assert (y.view(torch.int32) == ref.view(torch.int32)).all(), f"M={M} {out}: differs from the workspace call"


def test_noalloc_single_pass_and_too_large(w8a8):
    # a plan without a split (wide N, short K at M = 4096): the single-pass kernels run
    ops = operands(w8a8, 512, 10240, 2560, 8, 0, seed=3)
    n, ref = with_workspace(w8a8, ops, 8, 0, torch.float16)
    assert n == 0
    y = w8a8.w8a8_gemm_splitk_noalloc(*ops, 8, 0, torch.float16)
    torch.cuda.synchronize()
    assert (y.view(torch.int16) == ref.view(torch.int16)).all()
    # a plan whose partial results exceed the scratch: a clear error, nothing enqueued
    ops = operands(w8a8, 4096, 2560, 10240, 8, 128, seed=4)
    need = w8a8.w8a8_gemm_splitk_workspace(4096, 2560, 10240, 8, 128, torch.float16)
    note(f"noalloc too large: plan needs {need} bytes")
    assert need > SCRATCH_BYTES
    y = torch.zeros((4096, 2560), dtype=torch.float16, device="cuda")
    with pytest.raises(w8a8.W8A8Error, match="scratch"):
        w8a8.w8a8_gemm_splitk_noalloc(*ops, 8, 128, torch.float16, y=y)
    torch.cuda.synchronize()
    assert (y == 0).all()
