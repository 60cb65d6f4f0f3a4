"""GPU parity of the optimizer families beyond AdamW, Lion and SGD-momentum:
NAdam, RAdam, RMSprop, AdaGrad and plain SGD (FORGE paper, Appendix N, the
"fully fused" list).

Each family runs at the pages' verification shape (D_in = D_out = 512,
BT = 256, Appendix N "Numerical verification") over several steps against
the oracle element by element (RAdam past its switch to the rectified step
at t = 6), on ragged shapes through both mainloops, fused against the
unfused baseline bit for bit, through the 256 x 256 kernel and a grouped
call, and at the full gate_proj size on sampled rows.
"""

import sys

import numpy as np
import pytest
import torch

import backward_weight_gradient_amd as F
import synth
from forge_testlib import (assert_ok, check_against_oracle, make_layer, run_fused, run_unfused, sample_rows,
                           snapshot)

pytestmark = pytest.mark.gpu
SEED = 1337
FAMILIES = ("nadam", "radam", "rmsprop", "adagrad", "sgd")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _spec(opt, state="f32", w="bf16", in_dtype="bf16"):
    m = state if opt in F.KEEPS_M else None
    v = state if opt in F.KEEPS_V else None
    return synth.LayerSpec(in_dtype=in_dtype, w_fmt=w, m_fmt=m, v_fmt=v)


def _hyper(opt, round="sr"):
    # the pages' sweep values for the eps of AdaGrad (1e-10) and the others (1e-8), wd 1e-2
    return F.hyper(opt, lr=1e-3, weight_decay=0.01, round=round)


def _bytes(t):
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


@pytest.mark.parametrize("opt", FAMILIES)
@pytest.mark.parametrize("state,w", [("f32", "bf16"), ("bf16", "bf16"), ("f32", "f32")])
def test_family_verification_shape(opt, state, w):
    steps = 7 if opt == "radam" else 3
    _say(f"case: {opt} 512x512 BT256 state {state} W {w}, t=1..{steps}")
    spec = _spec(opt, state, w)
    L = make_layer(10, 512, 512, 256, 1, spec)
    h = _hyper(opt)
    for t in range(1, steps + 1):
        X, dY = synth.activations(10, 256, 512, 512, t, in_dtype="bf16")
        L.X, L.dY = X.cuda(), dY.cuda()
        snap = snapshot(L)
        run_fused(L, h, t, SEED)
        torch.cuda.synchronize()
        assert_ok(check_against_oracle(snap, L, h, t, SEED), f"{opt} t={t}")


@pytest.mark.parametrize("opt", FAMILIES)
@pytest.mark.parametrize("N,K,BT,in_dtype,round", [(129, 131, 65, "bf16", "sr"), (130, 136, 511, "bf16", "rne"),
                                                    (64, 200, 97, "f32", "sr"), (1, 1, 1, "bf16", "sr")])
def test_family_ragged(opt, N, K, BT, in_dtype, round):
    _say(f"case: {opt} ragged {N}x{K} BT{BT} {in_dtype} {round}")
    L = make_layer(11, N, K, BT, 3, _spec(opt, "f32", "bf16", in_dtype))
    h = _hyper(opt, round)
    snap = snapshot(L)
    run_fused(L, h, 3, SEED)
    torch.cuda.synchronize()
    assert_ok(check_against_oracle(snap, L, h, 3, SEED), f"{opt} {N}x{K}x{BT}")


@pytest.mark.parametrize("opt", FAMILIES)
@pytest.mark.parametrize("N,K,BT", [(600, 1024, 300), (1000, 1408, 4100)])   # the second takes the 256 x 256 kernel
def test_family_fused_equals_unfused(opt, N, K, BT):
    _say(f"case: {opt} fused vs unfused {N}x{K} BT{BT}")
    spec = _spec(opt, "bf16", "bf16")
    L = make_layer(12, N, K, BT, 7, spec, gen_device="cuda")
    U = L.clone()
    h = _hyper(opt)
    rows = sample_rows(N, 24, N + BT)
    snap = snapshot(L, rows)
    run_fused(L, h, 7, SEED)
    run_unfused(U, h, 7, SEED, torch.float32)
    torch.cuda.synchronize()
    for name in ("W", "m", "v"):
        a, b = getattr(L, name), getattr(U, name)
        if a is not None:
            assert torch.equal(_bytes(a), _bytes(b)), f"{opt}: fused {name} differs from the unfused baseline"
    assert_ok(check_against_oracle(snap, L, h, 7, SEED, col_ranges=[(0, 128), (K - 128, K)]), f"{opt} {N}x{K}")


@pytest.mark.parametrize("opt", FAMILIES)
def test_family_group(opt):
    _say(f"case: {opt} grouped q/k/v")
    spec = _spec(opt, "f32", "bf16")
    layers = [make_layer(13, N, 1024, 300, 5, spec, extra=i) for i, N in enumerate((512, 128, 128))]
    for L in layers[1:]:
        L.X = layers[0].X
    ref = [L.clone() for L in layers]
    h = _hyper(opt)
    F.forge_wgrad_step_group([(L.X, L.dY, L.W, L.forge_m(), L.forge_v(), SEED + i) for i, L in enumerate(layers)],
                             h, 5)
    for i, R in enumerate(ref):
        F.forge_wgrad_step(R.X, R.dY, R.W, R.forge_m(), R.forge_v(), h, 5, SEED + i)
    torch.cuda.synchronize()
    for L, R in zip(layers, ref):
        for name in ("W", "m", "v"):
            a, b = getattr(L, name), getattr(R, name)
            if a is not None:
                assert torch.equal(_bytes(a), _bytes(b)), f"{opt}: grouped {name} differs"


@pytest.mark.parametrize("opt", FAMILIES)
def test_family_full_size_gate_proj(opt):
    """gate_proj [14336, 4096] at BT = 512 (the benchmark's layer), sampled rows."""
    _say(f"case: {opt} gate_proj 14336x4096 BT512")
    N, K, BT = 14336, 4096, 512
    L = make_layer(14, N, K, BT, 10, _spec(opt, "f32", "bf16"), gen_device="cuda")
    h = _hyper(opt)
    rows = sample_rows(N, 40, 14)
    snap = snapshot(L, rows)
    run_fused(L, h, 10, SEED)
    torch.cuda.synchronize()
    cols = [(0, 128), (2048, 2176), (K - 128, K)]
    assert_ok(check_against_oracle(snap, L, h, 10, SEED, col_ranges=cols), f"{opt} gate_proj")
