"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Workloads follow the fp32 single-layer case, the Llama-3.1-8B layer shapes at
BT = 512 (fp32 / bf16 / int8 state), and the compute-bound BT = 2048 / 8192
sweep with AdamW, Lion and SGD-momentum; small and ragged shapes are checked
element by element, full sizes on sampled rows and column blocks.
"""

import sys

import numpy as np
import pytest
import torch

import backward_weight_gradient_amd as F
import oracle as O
import synth
from forge_testlib import (Layer, assert_ok, assert_rejected, check_against_oracle, make_layer, run_fused,
                           run_unfused, sample_rows, snapshot)

pytestmark = pytest.mark.gpu
SEED = 1337

SPEC_F32 = synth.LayerSpec(in_dtype="f32", w_fmt="f32", m_fmt="f32", v_fmt="f32")
SPEC_CFG1 = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="f32", v_fmt="f32")
SPEC_CFG2 = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="bf16", v_fmt="bf16")
SPEC_CFG3 = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="s8", v_fmt="u8", block=128)


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _full_check(L: Layer, h, step, seed=SEED, **kw):
    snap = snapshot(L)
    run_fused(L, h, step, seed)
    torch.cuda.synchronize()
    rep = check_against_oracle(snap, L, h, step, seed, **kw)
    return rep


# ---------------------------------------------------------------------------
# fp32 everywhere, BT 64, 256 x 256, AdamW t = 1..3 with fresh inputs
# ---------------------------------------------------------------------------
def test_fp32_layer_three_steps():
    _say("case: fp32 256x256 BT64 t=1..3")
    L = make_layer(0, 256, 256, 64, 1, SPEC_F32, dy_std=0.01, v_zero=True)
    h = F.hyper("adamw")
    for t in (1, 2, 3):
        X, dY = synth.activations(0, 64, 256, 256, t, in_dtype="f32", dy_std=0.01)
        L.X, L.dY = X.cuda(), dY.cuda()
        rep = _full_check(L, h, t)
        assert_ok(rep, f"fp32 t={t}")
        _say(f"  t={t}: {rep.checked} elements, hull-only {rep.clause2}")


# ---------------------------------------------------------------------------
# Small and ragged shapes, every state layout
# ---------------------------------------------------------------------------
SHAPES = [(256, 256, 64), (300, 200, 100), (129, 131, 65), (1, 1, 1), (130, 136, 511), (64, 130, 63),
          (512, 512, 256)]


@pytest.mark.parametrize("N,K,BT", SHAPES)
@pytest.mark.parametrize("round_", ["sr", "rne"])
def test_bf16_w_fp32_state(N, K, BT, round_):
    _say(f"case: bf16/f32 state {N}x{K} BT{BT} {round_}")
    L = make_layer(1, N, K, BT, 10, SPEC_CFG1)
    assert_ok(_full_check(L, F.hyper("adamw", round=round_), 10), f"{N}x{K}x{BT}")


@pytest.mark.parametrize("N,K,BT", SHAPES)
def test_bf16_everywhere(N, K, BT):
    _say(f"case: bf16 everywhere {N}x{K} BT{BT}")
    L = make_layer(2, N, K, BT, 10, SPEC_CFG2)
    assert_ok(_full_check(L, F.hyper("adamw", round="sr"), 10), f"{N}x{K}x{BT}")


@pytest.mark.parametrize("N,K,BT,block", [(256, 256, 64, 128), (300, 384, 100, 128), (129, 256, 65, 64),
                                          (64, 96, 63, 32), (512, 512, 256, 128)])
def test_int8_moments(N, K, BT, block):
    _say(f"case: int8 state {N}x{K} BT{BT} block{block}")
    spec = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="s8", v_fmt="u8", block=block)
    L = make_layer(3, N, K, BT, 10, spec, outlier_p=0.01, v_init="quantized")
    h = F.hyper("adamw", round="sr")
    assert_ok(_full_check(L, h, 10), f"int8 {N}x{K}")
    # a second step from the quantised state the first one wrote
    L.X, L.dY = (t.cuda() for t in synth.activations(3, BT, N, K, 11, outlier_p=0.01))
    assert_ok(_full_check(L, h, 11), f"int8 {N}x{K} second step")


@pytest.mark.parametrize("opt,m_fmt,w_fmt", [("lion", "f32", "bf16"), ("lion", "bf16", "bf16"),
                                             ("lion", "s8", "bf16"), ("sgdm", "f32", "bf16"),
                                             ("sgdm", "bf16", "f32"), ("sgdm", "s8", "bf16"),
                                             ("adamw", "f32", "f32")])
@pytest.mark.parametrize("N,K,BT", [(300, 256, 100), (512, 512, 256)])
def test_other_optimizers(opt, m_fmt, w_fmt, N, K, BT):
    _say(f"case: {opt} m={m_fmt} W={w_fmt} {N}x{K} BT{BT}")
    spec = synth.LayerSpec(in_dtype="bf16", w_fmt=w_fmt, m_fmt=m_fmt, v_fmt="f32" if opt == "adamw" else None)
    L = make_layer(4, N, K, BT, 10, spec)
    if opt == "lion":
        h = F.hyper("lion", lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01)
    elif opt == "sgdm":
        h = F.hyper("sgdm", lr=1e-3, beta1=0.9, weight_decay=0.01)
    else:
        h = F.hyper("adamw")
    # momentum that is not zero, so that the state update is exercised
    for t in (1, 2):
        L.X, L.dY = (x.cuda() for x in synth.activations(4, BT, N, K, t))
        assert_ok(_full_check(L, h, t), f"{opt} step {t}")


def test_fp32_inputs_bf16_weight():
    _say("case: fp32 inputs, bf16 W, fp32 state")
    spec = synth.LayerSpec(in_dtype="f32", w_fmt="bf16", m_fmt="f32", v_fmt="f32")
    L = make_layer(0, 200, 136, 70, 2, spec, dy_std=0.01)
    assert_ok(_full_check(L, F.hyper("adamw"), 2), "f32 in, bf16 W")


def test_empty_token_axis_applies_decay():
    """BT = 0: G = 0, the step still applies decoupled decay."""
    _say("case: BT=0")
    L = make_layer(1, 256, 128, 0, 10, SPEC_CFG1)
    assert L.X.shape == (0, 128)
    assert_ok(_full_check(L, F.hyper("adamw", round="rne"), 10), "BT=0")


def test_empty_layer_is_noop():
    W = torch.zeros((0, 64), device="cuda", dtype=torch.bfloat16)
    m = torch.zeros((0, 64), device="cuda")
    v = torch.zeros((0, 64), device="cuda")
    X = torch.zeros((16, 64), device="cuda", dtype=torch.bfloat16)
    dY = torch.zeros((16, 0), device="cuda", dtype=torch.bfloat16)
    assert F.forge_wgrad_step(X, dY, W, F.state(m), F.state(v), F.hyper(), 1, 1) == F.FORGE_OK


def test_strided_leading_dimension():
    """Rows with ld > cols (a column slice of a wider buffer)."""
    _say("case: ld > cols")
    N, K, BT = 200, 136, 80
    big = make_layer(1, N, 160, BT, 10, SPEC_CFG1)
    L = Layer(N, K, BT, SPEC_CFG1, big.X[:, :K], big.dY, big.W[:, :K], big.m[:, :K], big.v[:, :K])
    assert L.W.stride(0) == 160
    assert_ok(_full_check(L, F.hyper("adamw"), 10), "strided")
    # the columns outside the view are untouched
    ref = make_layer(1, N, 160, BT, 10, SPEC_CFG1)
    assert torch.equal(big.W[:, K:], ref.W[:, K:]) and torch.equal(big.m[:, K:], ref.m[:, K:])


# ---------------------------------------------------------------------------
# Fused == unfused (fp32 dW), bit for bit (Corollary 1(a)); resume exactness
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("spec,opt", [(SPEC_F32, "adamw"), (SPEC_CFG1, "adamw"), (SPEC_CFG2, "adamw"),
                                      (SPEC_CFG3, "adamw"),
                                      (synth.LayerSpec("bf16", "bf16", "f32", None), "lion"),
                                      (synth.LayerSpec("bf16", "bf16", "s8", None), "sgdm")])
def test_fused_equals_unfused_fp32_dw(spec, opt):
    _say(f"case: fused vs unfused {spec} {opt}")
    L = make_layer(1, 300, 384, 130, 10, spec)
    U = L.clone()
    h = F.hyper(opt, lr=1e-4 if opt == "lion" else 1e-3, beta2=0.99 if opt == "lion" else 0.999)
    run_fused(L, h, 10, SEED)
    dW = run_unfused(U, h, 10, SEED, torch.float32)
    torch.cuda.synchronize()
    for a, b in ((L.W, U.W), (L.m, U.m), (L.v, U.v), (L.ms, U.ms), (L.vs, U.vs)):
        if a is not None:
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b)
    # the materialised gradient itself is the oracle's G to fp32 accuracy
    snap_G = O.weight_grad(synth.host(L.X), synth.host(L.dY))
    E = O.grad_error_bound(synth.host(L.X), synth.host(L.dY))
    assert np.all(np.abs(dW.cpu().numpy().astype(np.float64) - snap_G) <= E)


def test_unfused_bf16_dw_runs_and_rounds_g():
    """The bf16-gradient baseline reads G rounded to bf16 (the pages' standard
    pipeline), so it differs from the fused step by that rounding only."""
    L = make_layer(1, 256, 256, 64, 10, SPEC_CFG1)
    snapG = O.weight_grad(synth.host(L.X), synth.host(L.dY))
    dW = run_unfused(L, F.hyper(), 10, SEED, torch.bfloat16)
    torch.cuda.synchronize()
    g = O.bf16_bits_to_f64(synth.host(dW))
    assert np.all(np.abs(g - snapG) <= 2.0 ** -8 * np.abs(snapG) + 1e-30)


def test_resume_is_bit_exact():
    """Three steps in a row == two steps, copy state out and back, one step."""
    L = make_layer(2, 256, 256, 64, 1, SPEC_CFG2)
    R = L.clone()
    h = F.hyper()
    for t in (1, 2, 3):
        run_fused(L, h, t, SEED)
    for t in (1, 2):
        run_fused(R, h, t, SEED)
    saved = [x.cpu() for x in (R.W, R.m, R.v)]
    R.W, R.m, R.v = (x.cuda() for x in saved)
    run_fused(R, h, 3, SEED)
    torch.cuda.synchronize()
    for a, b in ((L.W, R.W), (L.m, R.m), (L.v, R.v)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---------------------------------------------------------------------------
# Stochastic rounding through the device SR function
# ---------------------------------------------------------------------------
def test_debug_sr_matches_oracle_and_is_unbiased():
    n = 1_000_000
    x = torch.full((n,), 1 + 2 ** -10, dtype=torch.float32, device="cuda")
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    F.forge_debug_sr_bf16(x, out, SEED, 1, 0)
    torch.cuda.synchronize()
    got = synth.host(out)
    ref = O.f32_to_bf16_sr(x.cpu().numpy(), O.sr_bits(O.sr_key(SEED, 1, 0), np.arange(n)))
    np.testing.assert_array_equal(got, ref)
    up = np.mean(O.bf16_bits_to_f64(got) > 1.0)
    assert abs(up - 0.125) < 5 * np.sqrt(0.125 * 0.875 / n)
    # random values, negative and tiny ones, every tensor id
    xr = (torch.randn(1 << 16, device="cuda") * torch.logspace(-30, 30, 1 << 16, device="cuda")).float()
    for tid in (0, 1, 2):
        F.forge_debug_sr_bf16(xr, out[: xr.numel()], 99, 12345, tid)
        torch.cuda.synchronize()
        ref = O.f32_to_bf16_sr(xr.cpu().numpy(), O.sr_bits(O.sr_key(99, 12345, tid), np.arange(xr.numel())))
        np.testing.assert_array_equal(synth.host(out[: xr.numel()]), ref)


def test_debug_sr_special_values():
    """Infinities keep their pattern, NaNs come out quiet (signalling ones too), values at the edge of
    the bf16 range may round up to infinity, zeros keep their sign, denormals round stochastically."""
    bits = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001, 0xFF800123, 0x7FFFFFFF, 0xFFFFFFFF,
                     0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x00000000, 0x80000000, 0x00000001, 0x807FFFFF,
                     0x3F800001, 0xBF80FFFF], dtype=np.uint32)
    x = np.tile(bits, 4096).view(np.float32)
    out = torch.empty(x.size, dtype=torch.bfloat16, device="cuda")
    for tid in (0, 2):
        F.forge_debug_sr_bf16(torch.from_numpy(x).cuda(), out, 7, 3, tid)
        torch.cuda.synchronize()
        ref = O.f32_to_bf16_sr(x, O.sr_bits(O.sr_key(7, 3, tid), np.arange(x.size)))
        np.testing.assert_array_equal(synth.host(out), ref)


# ---------------------------------------------------------------------------
# Full sizes (sampled rows and column blocks)
# ---------------------------------------------------------------------------
LLAMA_BT512 = [("q_proj", 4096, 4096), ("k_proj", 1024, 4096), ("gate_proj", 14336, 4096),
               ("down_proj", 4096, 14336)]


def _sampled(L: Layer, h, step, nrows=40, ncolblocks=3, seed=SEED, **kw):
    rows = sample_rows(L.N, nrows, seed=L.N + L.K)
    snap = snapshot(L, rows)
    run_fused(L, h, step, seed)
    torch.cuda.synchronize()
    rng = np.random.default_rng(L.K)
    nb = -(-L.K // 128)
    blocks = sorted({0, nb - 1} | set(int(b) for b in rng.choice(nb, size=min(nb, ncolblocks), replace=False)))
    cols = [(b * 128, min(L.K, b * 128 + 128)) for b in blocks]
    return check_against_oracle(snap, L, h, step, seed, col_ranges=cols, **kw)


@pytest.mark.parametrize("name,N,K", LLAMA_BT512)
def test_llama_bt512_fp32_state_full_size(name, N, K):
    _say(f"case: {name} BT512 fp32 state")
    L = make_layer(1, N, K, 512, 10, SPEC_CFG1, gen_device="cuda")
    assert_ok(_sampled(L, F.hyper("adamw", round="sr"), 10), name)


@pytest.mark.parametrize("name,N,K", LLAMA_BT512[2:])
def test_llama_bt512_bf16_state_full_size(name, N, K):
    _say(f"case: {name} BT512 bf16 state")
    L = make_layer(2, N, K, 512, 10, SPEC_CFG2, gen_device="cuda")
    assert_ok(_sampled(L, F.hyper("adamw", round="sr"), 10), name)


@pytest.mark.parametrize("name,N,K", LLAMA_BT512[2:])
def test_llama_bt512_int8_state_full_size(name, N, K):
    _say(f"case: {name} BT512 int8 state")
    L = make_layer(3, N, K, 512, 10, SPEC_CFG3, gen_device="cuda", outlier_p=0.01)
    assert_ok(_sampled(L, F.hyper("adamw", round="sr"), 10), name)


@pytest.mark.parametrize("BT", [2048, 8192])
@pytest.mark.parametrize("name,N,K", [("down_proj", 4096, 14336), ("lm_head", 128256, 4096)])
@pytest.mark.parametrize("opt", ["adamw", "lion", "sgdm"])
def test_compute_bound_sweep_full_size(BT, name, N, K, opt):
    _say(f"case: {name} BT{BT} {opt}")
    spec = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="f32", v_fmt="f32" if opt == "adamw" else None)
    L = make_layer(4, N, K, BT, 10, spec, gen_device="cuda")
    if opt == "lion":
        h = F.hyper("lion", lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01)
    elif opt == "sgdm":
        h = F.hyper("sgdm", lr=1e-3, beta1=0.9, weight_decay=0.01)
    else:
        h = F.hyper("adamw")
    assert_ok(_sampled(L, h, 10, nrows=24, ncolblocks=2), f"{name} BT{BT} {opt}")
    del L
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Aligned (direct-to-LDS, vector epilogue) path on many tiles with ragged N
# and BT, every optimizer and state layout; bit-equal to the unfused baseline
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("spec,opt", [(SPEC_CFG1, "adamw"), (SPEC_CFG2, "adamw"), (SPEC_CFG3, "adamw"),
                                      (synth.LayerSpec("bf16", "bf16", "e4m3", "e4m3", block=128), "adamw"),
                                      (synth.LayerSpec("bf16", "bf16", "f32", None), "lion"),
                                      (synth.LayerSpec("bf16", "f32", "bf16", None), "sgdm")])
# 1024 x 2048 is whole tiles (the epilogue without per-segment bounds checks,
# for every state but bf16 moments); the next three are ragged; the last two
# take the 256 x 256 macro-tile kernel used for long token axes (ragged
# against 256 in both W dimensions and in the token chunks).
@pytest.mark.parametrize("N,K,BT", [(1024, 2048, 300), (2000, 4096, 300), (4104, 1024, 520), (600, 17152, 256),
                                    (1000, 1408, 4100), (2048, 1664, 4128)])
def test_aligned_multi_tile(spec, opt, N, K, BT):
    _say(f"case: aligned multi-tile {spec} {opt} {N}x{K} BT{BT}")
    L = make_layer(5, N, K, BT, 7, spec, gen_device="cuda", outlier_p=0.01 if spec.m_fmt == "s8" else 0.0)
    h = F.hyper(opt, lr=1e-4 if opt == "lion" else 1e-3, beta2=0.99 if opt == "lion" else 0.999)
    rows = np.array(sorted({0, 1, 127, 128, 255, 256, N // 2, N - 9, N - 1} |
                           set(int(r) for r in np.random.default_rng(N).choice(N, 40, replace=False))))
    snap = snapshot(L, rows)
    U = L.clone()
    run_fused(L, h, 7, SEED)
    run_unfused(U, h, 7, SEED, torch.float32)
    torch.cuda.synchronize()
    nb = K // 128
    cols = [(0, 128), (128, 256), ((nb // 2) * 128, (nb // 2) * 128 + 128), (K - 128, K)]
    assert_ok(check_against_oracle(snap, L, h, 7, SEED, col_ranges=cols), f"aligned {N}x{K}x{BT}")
    for a, b in ((L.W, U.W), (L.m, U.m), (L.v, U.v), (L.ms, U.ms), (L.vs, U.vs)):
        if a is not None:
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b)


# ---------------------------------------------------------------------------
# The 256 x 256 kernel (BT >= 2048) at small and ragged shapes: sub-tiles
# outside the matrix, a single partial macro tile, BT at the switch and one
# below it (the 128 x 128 kernel), every element against the oracle and bit
# for bit against the unfused baseline
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,BT", [(136, 72, 2100), (8, 8, 2049), (264, 520, 2048), (264, 512, 2047),
                                    (520, 256, 2080)])
@pytest.mark.parametrize("state", ["f32", "e4m3"])
def test_wide_kernel_edge_shapes(N, K, BT, state):
    _say(f"case: wide-kernel edge {N}x{K} BT{BT} state {state}")
    spec = synth.LayerSpec("bf16", "bf16", state, state, block=128)
    L = make_layer(8, N, K, BT, 4, spec, gen_device="cuda")
    if state == "e4m3" and K % 128:
        # block-scaled states need K % block == 0: rejected before any launch
        assert_rejected(L, lambda: F.forge_wgrad_step(L.X, L.dY, L.W, L.forge_m(), L.forge_v(), F.hyper("adamw"),
                                                      4, SEED, check=False))
        return
    h = F.hyper("adamw")
    snap = snapshot(L)
    U = L.clone()
    run_fused(L, h, 4, SEED)
    run_unfused(U, h, 4, SEED, torch.float32)
    torch.cuda.synchronize()
    assert_ok(check_against_oracle(snap, L, h, 4, SEED), f"wide edge {N}x{K}x{BT}")
    for a, b in ((L.W, U.W), (L.m, U.m), (L.v, U.v), (L.ms, U.ms), (L.vs, U.vs)):
        if a is not None:
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b)
