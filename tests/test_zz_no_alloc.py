"""GPU: forge_dgrad_split_noalloc, the allocation-free variant of
forge_dgrad_split (for callers that cannot allocate), through the C ABI
against forge_dgrad_split with a caller workspace.  Both run the same
kernels with the same splits and reduction order, so dX must be identical
bit for bit.  Two calls in a row, the second on a smaller input, so that
partial sums left in the static scratch array by the first call would show
up in the second if they leaked; a third on a shape with no split (the
scratch is not used) and a rejected one (more scratch than the array
holds), which must leave dX untouched.  dX is also checked against the
oracle's fp64 product on sampled rows, within the fp32 summation bound.
"""

import sys

import numpy as np
import pytest
import torch

import backward_weight_gradient_amd as F
import oracle as O
import synth

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _operands(BT, N, K, extra):
    dY = synth.normal((BT, N), 1e-3, "cuda", 60, 1, synth.T_DY, extra).to(torch.bfloat16)
    W = synth.normal((N, K), 0.02, "cuda", 60, 1, synth.T_W, extra).to(torch.bfloat16)
    return dY, W


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _check_oracle(dY, W, dX, rows):
    dYh, Wh = synth.host(dY), synth.host(W)
    ref = O.input_grad(dYh, Wh, rows)
    bound = O.input_grad_error_bound(dYh, Wh, rows)
    got = synth.host(dX)[rows]
    got = O.bf16_bits_to_f64(got) if dX.dtype == torch.bfloat16 else got.astype(np.float64)
    if dX.dtype == torch.bfloat16:   # one more rounding: half a bf16 ulp of the value
        bound = bound + np.abs(ref) * 2.0 ** -8
    assert np.all(np.abs(got - ref) <= bound * (1 + 1e-6) + 1e-30)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_dgrad_equals_workspace_variant(out_dtype):
    # 64 MiB of partials (the maximum, 256 x 256 tiles), then 8 MiB (128-token
    # tiles), then no split, then too much
    for i, (BT, N, K) in enumerate(((512, 14336, 4096), (256, 4096, 2048), (512, 1024, 4096))):
        _say(f"case: noalloc dX {BT}x{N}x{K} {out_dtype}")
        need = F.forge_dgrad_workspace_bytes(BT, N, K)
        assert need <= F.FORGE_DGRAD_SCRATCH_BYTES
        dY, W = _operands(BT, N, K, i)
        ws = torch.empty(max(1, need // 4), device="cuda", dtype=torch.float32)
        ref = torch.empty((BT, K), device="cuda", dtype=out_dtype)
        got = torch.full((BT, K), float("nan"), device="cuda", dtype=out_dtype)
        F.forge_dgrad_split(dY, W, ref, ws if need else None)
        F.forge_dgrad_split_noalloc(dY, W, got)
        torch.cuda.synchronize()
        assert torch.equal(_bits(ref), _bits(got)), f"{BT}x{N}x{K}: dX differs from the workspace variant"
        _check_oracle(dY, W, got, np.array([0, 1, BT // 2, BT - 1]))
        del dY, W, ws, ref, got
    _say("case: noalloc dX beyond the scratch")
    BT, N, K = 512, 8192, 12288
    assert F.forge_dgrad_workspace_bytes(BT, N, K) > F.FORGE_DGRAD_SCRATCH_BYTES
    dY, W = _operands(BT, N, K, 9)
    dX = torch.full((BT, K), 3.0, device="cuda", dtype=out_dtype)
    torch.cuda.synchronize()
    assert F.forge_dgrad_split_noalloc(dY, W, dX, check=False) == F.FORGE_E_SCRATCH
    torch.cuda.synchronize()
    assert bool((dX == 3.0).all()), "a rejected call wrote dX"
