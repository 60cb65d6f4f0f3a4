"""GPU: the measurement hooks bench.py takes its ceilings from.

forge_debug_copy must copy bit for bit (random bytes, a size that is not a
multiple of the kernel's four-request unroll, and one that spans several
grid strides); forge_debug_mfma_peak must leave 64 * iters in every output
element (all-ones operands: each round adds exactly 16 per accumulator), so
the flops it is credited with were really issued.
"""

import sys

import pytest
import torch

import backward_weight_gradient_amd as F

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("n16", [1, 5, 1000003, 16 * 1024 * 1024 + 7])
def test_copy_is_exact(n16):
    _say(f"case: debug copy {n16 * 16} bytes")
    g = torch.Generator(device="cuda").manual_seed(n16)
    src = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), device="cuda", dtype=torch.int32, generator=g)
    dst = torch.zeros_like(src)
    F.forge_debug_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


@pytest.mark.parametrize("blocks,iters", [(1, 1), (300, 37), (2048, 500)])
def test_mfma_loop_result(blocks, iters):
    _say(f"case: debug mfma {blocks} blocks x {iters} rounds")
    out = torch.full((256 * blocks,), float("nan"), device="cuda")
    F.forge_debug_mfma_peak(out, blocks, iters)
    torch.cuda.synchronize()
    assert torch.all(out == 64.0 * iters)
