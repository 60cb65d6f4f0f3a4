"""GPU: FP8 (E4M3) weight storage (the paper's FP8 weight quantization
folded into the per-tile kernel, section 3.6 and Figure 7; format, scale
and rounding as documented in forge.h).

forge_wgrad_step_fp8w against the oracle element by element: codes that the
fp32 uncertainty of the new weight cannot change must be identical (for
stochastic rounding: with the weight's own SR bits), the others within one
grid step; scales within 1e-5 or the hull of the block absmax; moments as in
the other parity tests.  AdamW with every moment format, Lion and SGD-m,
both rounding modes, blocks of 128, 64 and 32, several steps, ragged shapes,
the 256 x 256 kernel (BT >= 2048) and gate_proj at full size on sampled
rows.  The device's E4M3 stochastic rounding on its own, bit for bit
(forge_debug_e4m3_sr).  forge_dgrad_fp8w against the oracle's fp64 product
with the decoded weight.  Unsupported combinations and shapes are refused before anything
is enqueued.
"""

import sys

import numpy as np
import pytest
import torch

import backward_weight_gradient_amd as F
import oracle as O
import synth
from forge_testlib import assert_ok, assert_rejected, check_against_oracle, make_layer, run_fused, sample_rows, \
    snapshot

pytestmark = pytest.mark.gpu
SEED = 1337


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _hyper(opt, round_):
    if opt == "lion":
        return F.hyper("lion", lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01, round=round_)
    return F.hyper(opt, round=round_)


def _spec(opt, state, block=128):
    m = None if opt not in F.KEEPS_M else ("s8" if state == "int8" else state)
    v = None if opt not in F.KEEPS_V else ("u8" if state == "int8" else state)
    return synth.LayerSpec("bf16", "e4m3", m, v, block=block)


def test_e4m3_stochastic_rounding_hook_bit_exact():
    """The device's E4M3 stochastic rounding (the FP8 weight store) against
    the oracle's definition, bit for bit, element i with the SR bits of flat
    index i under the weight's key: every grid point, midpoint and its
    neighbours, the subnormal range densely, values just below and above the
    normal/subnormal boundary 2^-6, saturation, signed zeros, random
    magnitudes over the whole range."""
    _say("case: E4M3 SR hook")
    grid = O.e4m3_to_f64(np.arange(0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(21)
    sub = rng.integers(0, 0x3C800000, 300000, dtype=np.int64).astype(np.uint32).view(np.float32)
    x = np.concatenate([grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        [448.0, 449.0, 464.0, 480.0, 1e30, 2.0 ** -6, np.nextafter(np.float32(2.0 ** -6), 0),
                         2.0 ** -9, 2.0 ** -10, 2.0 ** -149],
                        sub, rng.uniform(0, 448, 200000), 10.0 ** rng.uniform(-12, 3, 200000)]).astype(np.float32)
    x = np.concatenate([x, -x, np.float32([0.0, -0.0])])
    for seed, step in ((SEED, 1), (2**63 + 12345, 7)):
        xin = torch.from_numpy(x).cuda()
        out = torch.empty(x.size, device="cuda", dtype=torch.uint8)
        F.forge_debug_e4m3_sr(xin, out, seed, step)
        torch.cuda.synchronize()
        r16 = O.sr_bits(O.sr_key(seed, step, 0), np.arange(x.size, dtype=np.uint64))
        np.testing.assert_array_equal(out.cpu().numpy(), O.f32_to_e4m3_sr(x, r16))


CASES = [("adamw", "f32"), ("adamw", "bf16"), ("adamw", "int8"), ("adamw", "e4m3"), ("lion", "f32"),
         ("lion", "e4m3"), ("sgdm", "bf16"), ("sgdm", "e4m3")]


@pytest.mark.parametrize("opt,state", CASES)
@pytest.mark.parametrize("round_", ["sr", "rne"])
def test_fp8_weight_verification_shape(opt, state, round_):
    _say(f"case: FP8 W {opt} {state} {round_} 512x512 BT256")
    L = make_layer(70, 512, 512, 256, 1, _spec(opt, state), outlier_p=0.01 if state == "int8" else 0.0)
    h = _hyper(opt, round_)
    for t in (1, 2, 3):
        X, dY = synth.activations(70, 256, 512, 512, t, outlier_p=0.01 if state == "int8" else 0.0)
        L.X, L.dY = X.cuda(), dY.cuda()
        snap = snapshot(L)
        run_fused(L, h, t, SEED)
        torch.cuda.synchronize()
        assert_ok(check_against_oracle(snap, L, h, t, SEED), f"FP8 W {opt} {state} {round_} t={t}")


@pytest.mark.parametrize("block", [64, 32])
@pytest.mark.parametrize("N,K,BT", [(130, 256, 77), (264, 384, 129), (1, 128, 1), (200, 512, 0)])
def test_fp8_weight_ragged(block, N, K, BT):
    _say(f"case: FP8 W ragged {N}x{K} BT{BT} block {block}")
    L = make_layer(71, N, K, BT, 5, _spec("adamw", "e4m3", block))
    h = _hyper("adamw", "sr")
    snap = snapshot(L)
    run_fused(L, h, 5, SEED)
    torch.cuda.synchronize()
    assert_ok(check_against_oracle(snap, L, h, 5, SEED), f"FP8 W {N}x{K}x{BT}")


@pytest.mark.parametrize("state", ["f32", "e4m3"])
def test_fp8_weight_wide_kernel(state):
    """BT >= 2048: the 256 x 256 macro-tile kernel with the E4M3 weight."""
    _say(f"case: FP8 W wide kernel {state}")
    L = make_layer(72, 520, 384, 2080, 4, _spec("adamw", state), gen_device="cuda")
    h = _hyper("adamw", "sr")
    snap = snapshot(L)
    run_fused(L, h, 4, SEED)
    torch.cuda.synchronize()
    assert_ok(check_against_oracle(snap, L, h, 4, SEED), f"FP8 W wide {state}")


@pytest.mark.parametrize("state", ["f32", "e4m3"])
def test_fp8_weight_gate_proj_full_size(state):
    """gate_proj [14336, 4096] at BT = 512 on sampled rows and column blocks."""
    _say(f"case: FP8 W gate_proj BT512 {state}")
    N, K = synth.LLAMA8B_LAYERS["gate_proj"]
    L = make_layer(73, N, K, 512, 10, _spec("adamw", state), gen_device="cuda")
    h = _hyper("adamw", "sr")
    rows = sample_rows(N, 24, seed=73)
    snap = snapshot(L, rows)
    run_fused(L, h, 10, SEED)
    torch.cuda.synchronize()
    cols = [(0, 128), (1280, 1408), (K - 128, K)]
    assert_ok(check_against_oracle(snap, L, h, 10, SEED, col_ranges=cols), f"FP8 W gate_proj {state}")
    del L
    torch.cuda.empty_cache()


# bf16 dY with N % 8 == 0 and aligned rows takes the bf16 matrix-core kernel
# (three bf16 terms per decoded weight): (512, 512, 256), (14336, 4096, 512),
# (1000, 1056, 77) (64-token tiles, ragged tokens, reduction chunk and column
# tile, blocks of 32), (520, 2048, 2048) (128-token tiles, blocks of 64),
# (136, 2016, 2048) (128-token tiles, a partial last column tile, blocks of
# 32), (264, 384, 300); N % 8 != 0 takes the fp32 matrix-core kernel: (130,
# 256, 77); fp32 dY the plain kernel: (97, 384, 130).
@pytest.mark.parametrize("N,K,BT,dx,dy32,block", [(512, 512, 256, torch.bfloat16, False, 128),
                                                  (130, 256, 77, torch.float32, False, 128),
                                                  (97, 384, 130, torch.bfloat16, True, 128),
                                                  (14336, 4096, 512, torch.bfloat16, False, 128),
                                                  (1000, 1056, 77, torch.bfloat16, False, 32),
                                                  (520, 2048, 2048, torch.float32, False, 64),
                                                  (136, 2016, 2048, torch.bfloat16, False, 32),
                                                  (264, 384, 300, torch.float32, False, 128)])
def test_fp8_weight_dgrad(N, K, BT, dx, dy32, block):
    _say(f"case: FP8 W dX {N}x{K} BT{BT} {dx} dY {'f32' if dy32 else 'bf16'} block {block}")
    L = make_layer(75, N, K, BT, 2, _spec("adamw", "f32", block), gen_device="cuda" if N > 4096 else "cpu")
    if dy32:
        L.dY = L.dY.float()
    dX = torch.full((BT, K), float("nan"), device="cuda", dtype=dx)
    F.forge_dgrad_fp8w(L.dY, L.forge_w(), dX)
    torch.cuda.synchronize()
    rows = np.unique(np.array([0, 1, BT // 2, BT - 1] + list(np.random.default_rng(N).integers(0, BT, 12))))
    Wst = O.Stored("e4m3", synth.host(L.W), L.wsc.cpu().numpy(), block)
    Wdec = O.decode(Wst).astype(np.float32)         # the stored weight, exactly (fp32)
    dYh = synth.host(L.dY)
    ref = O.input_grad(dYh, Wdec, rows)
    bound = O.input_grad_error_bound(dYh, Wdec, rows)
    got = synth.host(dX)[rows]
    got = O.bf16_bits_to_f64(got) if dx == torch.bfloat16 else got.astype(np.float64)
    if dx == torch.bfloat16:
        bound = bound + np.abs(ref) * 2.0 ** -8
    bad = np.abs(got - ref) > bound * (1 + 1e-6) + 1e-30
    assert not bad.any(), f"{int(bad.sum())} dX elements outside the fp32 bound"
    del L
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wpad", [16, 8])
def test_fp8_weight_dgrad_strided(wpad):
    """Row pitches above the row length on dY, the codes and dX: a code pitch that is a multiple of 16
    (K + 16) takes the bf16 matrix-core kernel, K + 8 the fp32 one; dX columns past K stay untouched."""
    N, K, BT, block = 264, 256, 130, 64
    _say(f"case: FP8 W dX strided, code pitch K + {wpad}")
    L = make_layer(77, N, K, BT, 2, _spec("adamw", "f32", block))
    codes = torch.zeros((N, K + wpad), dtype=torch.uint8)
    codes[:, :K] = L.W.view(torch.uint8).cpu()
    codes = codes.to("cuda")
    Wv = codes[:, :K].view(torch.float8_e4m3fn)
    dYb = torch.zeros((BT, N + 8), device="cuda", dtype=torch.bfloat16)
    dYb[:, :N] = L.dY.to("cuda")
    dY = dYb[:, :N]
    big = torch.full((BT, K + 24), float("nan"), device="cuda", dtype=torch.bfloat16)
    dX = big[:, :K]
    wsc = L.wsc.to("cuda")
    W = F.state(Wv, wsc, block)
    F.forge_dgrad_fp8w(dY, W, dX)
    torch.cuda.synchronize()
    rows = np.arange(BT)
    Wst = O.Stored("e4m3", synth.host(L.W), L.wsc.cpu().numpy(), block)
    Wdec = O.decode(Wst).astype(np.float32)
    dYh = synth.host(L.dY)
    ref = O.input_grad(dYh, Wdec, rows)
    bound = O.input_grad_error_bound(dYh, Wdec, rows) + np.abs(ref) * 2.0 ** -8
    got = O.bf16_bits_to_f64(synth.host(dX.contiguous()))
    bad = np.abs(got - ref) > bound * (1 + 1e-6) + 1e-30
    assert not bad.any(), f"{int(bad.sum())} dX elements outside the fp32 bound"
    assert torch.isnan(big[:, K:].float()).all(), "dX columns past K were written"


def test_fp8_weight_rejections_leave_everything_untouched():
    _say("case: FP8 W rejected calls")
    h = _hyper("adamw", "sr")
    # K not a multiple of the block
    L = make_layer(76, 64, 200, 32, 1, synth.LayerSpec("bf16", "e4m3", "f32", "f32", block=128))
    assert_rejected(L, lambda: F.forge_wgrad_step_fp8w(L.X, L.dY, L.forge_w(), L.forge_m(), L.forge_v(), h, 1,
                                                         SEED, check=False))
    # a combination without an FP8-weight kernel (NAdam), and fp32 inputs
    L = make_layer(76, 64, 256, 32, 1, synth.LayerSpec("bf16", "e4m3", "f32", "f32", block=128))
    assert_rejected(L, lambda: F.forge_wgrad_step_fp8w(L.X, L.dY, L.forge_w(), L.forge_m(), L.forge_v(),
                                                         F.hyper("nadam"), 1, SEED, check=False),
                    code=F.FORGE_E_UNSUPPORTED)
    X32, dY32 = L.X.float(), L.dY.float()
    assert_rejected(L, lambda: F.forge_wgrad_step_fp8w(X32, dY32, L.forge_w(), L.forge_m(), L.forge_v(), h, 1,
                                                         SEED, check=False), code=F.FORGE_E_UNSUPPORTED)
    # a bf16 weight passed as the E4M3 state
    Wb = torch.zeros((64, 256), device="cuda", dtype=torch.bfloat16)
    bad = F.forge_state(F.mat(Wb), L.wsc.data_ptr(), 128)
    assert_rejected(L, lambda: F.forge_wgrad_step_fp8w(L.X, L.dY, bad, L.forge_m(), L.forge_v(), h, 1, SEED,
                                                         check=False), code=F.FORGE_E_DTYPE)
