"""GPU: the fused epilogue's 8-bit block quantiser on its own
(forge_debug_quant: the same device function and thread mapping as the S8 /
U8 / E4M3 state store), bit for bit against the oracle's quantize_signed,
quantize_unsigned and quantize_e4m3 on identical fp32 inputs.  This is the
"codes bit-exact given identical inputs" half of the int8 tolerance; the
fused step itself is checked in the parity tests, where the kernel's fp32
pre-quantisation values differ from the oracle's by the summation order.

The inputs are built so that a plausible mistake fails: exact ties (the
reciprocal exactly 1 or 8, values k + 1/2), all-zero blocks, positive values
below half a step (the U8 floor to code 1), the absmax element, negative
zero, a lone outlier, blocks whose absmax is below 2^-64, in the fp32
subnormal range, near or above 2^126 and up to the fp32 maximum, and
ragged row / column counts against the 16-row, 128-column work unit of the
kernel.  The fast scale / reciprocal quotients the quantiser uses are
checked against IEEE division for every fp32 absmax in their range.
"""

import sys

import numpy as np
import pytest
import torch

import backward_weight_gradient_amd as F
import oracle as O

pytestmark = pytest.mark.gpu

RULES = {  # name -> (forge dtype, second-moment rule, oracle quantiser, QMAX)
    "s8": (F.FORGE_S8, False, O.quantize_signed, 127.0),
    "u8": (F.FORGE_U8, True, O.quantize_unsigned, 255.0),
    "e4m3_m": (F.FORGE_E4M3, False, lambda x, b: O.quantize_e4m3(x, b, False), O.E4M3_MAX),
    "e4m3_v": (F.FORGE_E4M3, True, lambda x, b: O.quantize_e4m3(x, b, True), O.E4M3_MAX),
}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _inputs(rows: int, cols: int, block: int, qmax: float, positive: bool, seed: int) -> np.ndarray:
    """rows x cols fp32 with one kind of block per row (cycling through the kinds)."""
    rng = np.random.default_rng(seed)
    x = np.zeros((rows, cols), dtype=np.float32)
    nb = cols // block
    grid = O.e4m3_to_f64(np.arange(0x7F))
    for r in range(rows):
        kind = r % 13
        for b in range(nb):
            blk = np.zeros(block, dtype=np.float64)
            if kind == 0:                                   # plain normal values
                blk = rng.standard_normal(block) * 1e-3
            elif kind == 1:                                 # exact ties, reciprocal exactly 1
                blk = rng.integers(0, int(qmax) - 1, block) + 0.5
                if qmax == O.E4M3_MAX:                      # E4M3: midpoints of the grid
                    i = rng.integers(0, 0x7D, block)
                    blk = (grid[i] + grid[i + 1]) / 2
                blk[0] = qmax
                blk *= np.where(rng.random(block) < 0.5, -1.0, 1.0)
                blk[0] = qmax
            elif kind == 2:                                 # exact ties with reciprocal 8
                blk = (rng.integers(0, int(qmax) - 1, block) + 0.5) / 8.0
                blk[0] = qmax / 8.0
            elif kind == 3:                                 # all zero (kept)
                pass
            elif kind == 4:                                 # sub-half-step positives and the absmax
                blk = np.abs(rng.standard_normal(block)) * 1e-3
                blk[0] = 1.0
                blk[1:6] = [1e-9, 0.3 / qmax, 0.49 / qmax, 0.5 / qmax, 0.51 / qmax]
            elif kind == 5:                                 # zeros and negative zeros among values
                blk = rng.standard_normal(block)
                blk[::3] = 0.0
                blk[1::7] = -0.0
            elif kind == 6:                                 # a lone outlier
                blk = rng.standard_normal(block) * 1e-4
                blk[block // 2] = 3.0
            elif kind == 7:                                 # absmax below 2^-64
                blk = rng.standard_normal(block) * 1e-25
            elif kind == 8:                                 # absmax near the fp32 subnormal range
                blk = rng.standard_normal(block) * 1e-38
            elif kind == 9:                                 # subnormal values only
                blk = rng.integers(-50, 50, block) * 2.0 ** -149
            elif kind == 10:                                # huge values
                blk = rng.standard_normal(block) * 1e37
            elif kind == 11:                                # absmax at or above 2^126
                blk = rng.uniform(-3.4e38, 3.4e38, block)
                blk[0] = 2.0 ** 126
            else:                                           # exactly on the code grid
                blk = rng.integers(-int(qmax), int(qmax) + 1, block) * (0.37 / qmax)
            x[r, b * block:(b + 1) * block] = blk.astype(np.float32)
    if positive:
        x = np.abs(x)
    return x


@pytest.mark.parametrize("rule", list(RULES))
@pytest.mark.parametrize("rows,cols,block", [(37, 384, 128), (21, 192, 64), (16, 96, 32), (50, 512, 32),
                                             (1, 128, 128), (33, 320, 64)])
def test_quantiser_bit_exact_against_oracle(rule, rows, cols, block):
    dtype, second, quant, qmax = RULES[rule]
    _say(f"case: quantiser {rule} {rows}x{cols} block {block}")
    x = _inputs(rows, cols, block, qmax, second, seed=rows * cols + block)
    ref_q, ref_s = quant(x, block)
    xin = torch.from_numpy(x).cuda()
    codes = torch.full((rows, cols), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows, cols // block), -1.0, dtype=torch.float32, device="cuda")
    F.forge_debug_quant(xin, codes, scales, dtype, second, block)
    torch.cuda.synchronize()
    got_q = codes.cpu().numpy()
    got_s = scales.cpu().numpy()
    np.testing.assert_array_equal(got_q, ref_q.view(np.uint8), err_msg=f"{rule} codes")
    np.testing.assert_array_equal(got_s.view(np.uint32), ref_s.view(np.uint32), err_msg=f"{rule} scales")


def test_quantiser_empty_and_rejected_calls_touch_nothing():
    _say("case: quantiser empty / rejected")
    xin = torch.ones((4, 128), device="cuda")
    codes = torch.full((4, 128), 7, dtype=torch.uint8, device="cuda")
    scales = torch.full((4, 1), 5.0, device="cuda")
    assert F.forge_debug_quant(xin[:0], codes[:0], scales[:0], F.FORGE_S8, False, 128) == F.FORGE_OK
    assert F.forge_debug_quant(xin, codes, scales, F.FORGE_S8, True, 128, check=False) == F.FORGE_E_DTYPE
    torch.cuda.synchronize()
    assert int(codes.sum()) == 7 * 512 and float(scales.sum()) == 20.0


def test_quantiser_quotients_equal_ieee_division_exhaustively():
    """The block scale a / QMAX and reciprocal QMAX / a from short fma
    sequences, compared with IEEE division for every fp32 a in [2^-64,
    2^126) and QMAX in {127, 255, 448} (outside that range the quantiser
    divides with IEEE division)."""
    _say("case: quantiser quotients, exhaustive")
    counts = torch.zeros(F.FORGE_QUOTIENT_COUNTS, dtype=torch.int64, device="cuda")
    F.forge_debug_quotients(counts)
    torch.cuda.synchronize()
    c = counts.cpu().numpy().reshape(-1, 8)
    assert int(c[:, 6].sum()) == 0x7E800000 - 0x1F800000          # every a in the range checked
    names = ["a/127", "127/a", "a/255", "255/a", "a/448", "448/a"]
    bad = {n: int(c[:, k].sum()) for k, n in enumerate(names)}
    assert all(v == 0 for v in bad.values()), bad
