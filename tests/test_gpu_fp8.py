"""GPU: FP8 E4M3 moment storage (the paper's FP8 moment quantization,
section 3.6; format and scale rule as documented in forge.h).

The device's E4M3 rounding is checked bit for bit against the oracle's on
every grid point, every midpoint and its neighbours, subnormals and
saturation; the fused step with E4M3 moments (AdamW m and v, Lion / SGD-m m,
every block size) against the oracle element by element (codes within one
grid step, 99% identical; scales within 1e-5 or the hull of the block
absmax); fused against unfused bit for bit, in a grouped call, and at the
full gate_proj size on sampled rows.
"""

import sys

import numpy as np
import pytest
import torch

import backward_weight_gradient_amd as F
import oracle as O
import synth
from forge_testlib import assert_ok, check_against_oracle, make_layer, run_fused, run_unfused, sample_rows, snapshot

pytestmark = pytest.mark.gpu
SEED = 1337


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _spec(opt, block=128, w="bf16"):
    return synth.LayerSpec("bf16", w, "e4m3", "e4m3" if opt == "adamw" else None, block=block)


def _hyper(opt):
    return F.hyper(opt, lr=1e-4 if opt == "lion" else 1e-3, beta2=0.99 if opt == "lion" else None)


def _bytes(t):
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


def test_e4m3_device_rounding_bit_exact():
    _say("case: E4M3 rounding hook")
    grid = O.e4m3_to_f64(np.arange(0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(12)
    x = np.concatenate([grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), [448.0, 460.0, 1e30, 2.0 ** -10],
                        rng.uniform(0, 448, 200000), 10.0 ** rng.uniform(-12, 3, 200000)]).astype(np.float32)
    x = np.concatenate([x, -x, np.float32([0.0, -0.0])])
    xin = torch.from_numpy(x).cuda()
    out = torch.empty(x.size, device="cuda", dtype=torch.uint8)
    F.forge_debug_e4m3(xin, out)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), O.f32_to_e4m3_rne(x))


@pytest.mark.parametrize("opt", ["adamw", "lion", "sgdm"])
@pytest.mark.parametrize("block,w", [(128, "bf16"), (64, "f32"), (32, "bf16")])
def test_e4m3_states_verification_shape(opt, block, w):
    _say(f"case: E4M3 {opt} 512x512 BT256 block {block} W {w}")
    L = make_layer(40, 512, 512, 256, 1, _spec(opt, block, w), outlier_p=0.01)
    h = _hyper(opt)
    for t in (1, 2, 3):
        X, dY = synth.activations(40, 256, 512, 512, t, in_dtype="bf16", outlier_p=0.01)
        L.X, L.dY = X.cuda(), dY.cuda()
        snap = snapshot(L)
        run_fused(L, h, t, SEED)
        torch.cuda.synchronize()
        assert_ok(check_against_oracle(snap, L, h, t, SEED), f"E4M3 {opt} t={t}")


@pytest.mark.parametrize("opt", ["adamw", "lion"])
@pytest.mark.parametrize("N,K,BT", [(130, 256, 77), (1, 128, 1), (264, 384, 129)])
def test_e4m3_states_ragged(opt, N, K, BT):
    _say(f"case: E4M3 {opt} ragged {N}x{K} BT{BT}")
    L = make_layer(41, N, K, BT, 4, _spec(opt))
    h = _hyper(opt)
    snap = snapshot(L)
    run_fused(L, h, 4, SEED)
    torch.cuda.synchronize()
    assert_ok(check_against_oracle(snap, L, h, 4, SEED), f"E4M3 {opt} {N}x{K}")


@pytest.mark.parametrize("N,K,BT", [(600, 1024, 300), (1000, 1408, 4100)])   # the second takes the 256 x 256 kernel
def test_e4m3_fused_equals_unfused(N, K, BT):
    _say(f"case: E4M3 fused vs unfused {N}x{K} BT{BT}")
    L = make_layer(42, N, K, BT, 6, _spec("adamw"), gen_device="cuda")
    U = L.clone()
    h = F.hyper("adamw")
    run_fused(L, h, 6, SEED)
    run_unfused(U, h, 6, SEED, torch.float32)
    torch.cuda.synchronize()
    for name in ("W", "m", "v", "ms", "vs"):
        assert torch.equal(_bytes(getattr(L, name)), _bytes(getattr(U, name))), f"{name} differs"


def test_e4m3_grouped_call():
    _say("case: E4M3 grouped q/k/v")
    layers = [make_layer(43, N, 1024, 300, 5, _spec("adamw"), extra=i) for i, N in enumerate((512, 128, 128))]
    ref = [L.clone() for L in layers]
    h = F.hyper("adamw")
    F.forge_wgrad_step_group([(L.X, L.dY, L.W, L.forge_m(), L.forge_v(), SEED + i) for i, L in enumerate(layers)],
                             h, 5)
    for i, R in enumerate(ref):
        F.forge_wgrad_step(R.X, R.dY, R.W, R.forge_m(), R.forge_v(), h, 5, SEED + i)
    torch.cuda.synchronize()
    for L, R in zip(layers, ref):
        for name in ("W", "m", "v", "ms", "vs"):
            assert torch.equal(_bytes(getattr(L, name)), _bytes(getattr(R, name))), f"{name} differs"


def test_e4m3_full_size_gate_proj():
    _say("case: E4M3 gate_proj 14336x4096 BT512")
    N, K, BT = 14336, 4096, 512
    L = make_layer(44, N, K, BT, 10, _spec("adamw"), gen_device="cuda", outlier_p=0.01)
    h = F.hyper("adamw")
    rows = sample_rows(N, 40, 44)
    snap = snapshot(L, rows)
    run_fused(L, h, 10, SEED)
    torch.cuda.synchronize()
    assert_ok(check_against_oracle(snap, L, h, 10, SEED, col_ranges=[(0, 128), (2048, 2176), (K - 128, K)]),
              "E4M3 gate_proj")
