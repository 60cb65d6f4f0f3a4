"""GPU: exact gradient accumulation (FORGE paper, Appendix L).

Micro-steps add their weight gradient into an fp32 accumulator
(forge_wgrad_accumulate); the final micro-step runs the fused step on
accumulator + its own gradient (forge_wgrad_step_accumulated).  The oracle
sees one batch made of all micro-batches' tokens: the summed gradient is the
gradient of the concatenated batch (Eq. 3 is a sum over tokens), and the
fp32 error bound grows by one addition per micro-batch.  Both final-step
paths are covered (the fused kernel that reads the accumulator for aligned
bf16 inputs, accumulate-then-step for the others) and checked against each
other bit for bit.
"""

import sys

import numpy as np
import pytest
import torch

import backward_weight_gradient_amd as F
import oracle as O
import synth
from forge_testlib import assert_ok, assert_rejected, check_against_oracle, make_layer, snapshot

pytestmark = pytest.mark.gpu
SEED = 1337


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _micro(cfg, bts, N, K, in_dtype, extra=0):
    """Seeded micro-batches (X_i, dY_i) on the GPU."""
    out = []
    for i, bt in enumerate(bts):
        X, dY = synth.activations(cfg, bt, N, K, 1, in_dtype=in_dtype, extra=100 * extra + i)
        out.append((X.cuda(), dY.cuda()))
    return out


def _spec(opt, state="f32", in_dtype="bf16", w="bf16"):
    if state == "int8":
        return synth.LayerSpec(in_dtype=in_dtype, w_fmt=w, m_fmt="s8" if opt in F.KEEPS_M else None,
                               v_fmt="u8" if opt in F.KEEPS_V else None, block=128)
    if state == "e4m3":
        return synth.LayerSpec(in_dtype=in_dtype, w_fmt=w, m_fmt="e4m3" if opt in F.KEEPS_M else None,
                               v_fmt="e4m3" if opt in F.KEEPS_V else None, block=128)
    return synth.LayerSpec(in_dtype=in_dtype, w_fmt=w, m_fmt=state if opt in F.KEEPS_M else None,
                           v_fmt=state if opt in F.KEEPS_V else None)


@pytest.mark.parametrize("N,K,bts,in_dtype", [(300, 260, (100, 64, 200, 1), "bf16"),
                                               (512, 1024, (128, 128, 256), "bf16"),
                                               (136, 72, (33, 0, 70), "f32")])
def test_accumulator_is_the_summed_gradient(N, K, bts, in_dtype):
    _say(f"case: accumulate {N}x{K} micro-batches {bts} {in_dtype}")
    mb = _micro(20, bts, N, K, in_dtype)
    acc = torch.full((N, K), float("nan"), device="cuda")       # first=True must overwrite everything
    for i, (X, dY) in enumerate(mb):
        F.forge_wgrad_accumulate(X, dY, acc, first=(i == 0))
    torch.cuda.synchronize()
    Xc = synth.host(torch.cat([X for X, _ in mb]))
    dYc = synth.host(torch.cat([dY for _, dY in mb]))
    G = O.weight_grad(Xc, dYc)
    E = O.grad_error_bound(Xc, dYc, extra_terms=len(bts))
    got = acc.cpu().numpy().astype(np.float64)
    bad = np.abs(got - G) > E + 1e-30
    assert not bad.any(), f"{int(bad.sum())} accumulator elements outside the fp32 bound"


def test_accumulator_strided_and_first_with_no_tokens():
    """An accumulator with ld > K; a first micro-step with BT = 0 clears it."""
    N, K = 200, 136
    big = torch.full((N, K + 24), float("nan"), device="cuda")
    acc = big[:, :K]
    X0, dY0 = torch.empty((0, K), device="cuda", dtype=torch.bfloat16), torch.empty((0, N), device="cuda",
                                                                                    dtype=torch.bfloat16)
    F.forge_wgrad_accumulate(X0, dY0, acc, first=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(acc).item() == 0
    assert torch.isnan(big[:, K:]).all(), "columns past K of the accumulator were written"
    (X, dY), = _micro(21, (77,), N, K, "bf16")
    F.forge_wgrad_accumulate(X, dY, acc, first=False)
    torch.cuda.synchronize()
    G = O.weight_grad(synth.host(X), synth.host(dY))
    E = O.grad_error_bound(synth.host(X), synth.host(dY), extra_terms=2)
    assert np.all(np.abs(acc.cpu().numpy() - G) <= E + 1e-30)
    assert torch.isnan(big[:, K:]).all()


CASES = [("adamw", "f32"), ("adamw", "bf16"), ("adamw", "int8"), ("adamw", "e4m3"), ("lion", "f32"),
         ("lion", "e4m3"), ("sgdm", "bf16"), ("sgdm", "e4m3"), ("nadam", "f32"), ("radam", "bf16"),
         ("rmsprop", "f32"), ("adagrad", "bf16"), ("sgd", None)]


@pytest.mark.parametrize("opt,state", CASES)
@pytest.mark.parametrize("N,K,bts,in_dtype", [(384, 512, (96, 160, 64), "bf16"),     # fused final step
                                               (130, 136, (65, 33, 100), "bf16"),    # unaligned: accumulate, then step
                                               (128, 256, (50, 70), "f32")])         # fp32 inputs: accumulate, then step
def test_step_accumulated_matches_oracle(opt, state, N, K, bts, in_dtype):
    _say(f"case: accumulated step {opt} {state} {N}x{K} {bts} {in_dtype}")
    spec = _spec(opt, state or "f32", in_dtype)
    L = make_layer(22, N, K, 1, 8, spec, outlier_p=0.0)
    mb = _micro(22, bts, N, K, in_dtype, extra=1)
    acc = torch.empty((N, K), device="cuda")
    for i, (X, dY) in enumerate(mb[:-1]):
        F.forge_wgrad_accumulate(X, dY, acc, first=(i == 0))
    h = F.hyper(opt, lr=1e-4 if opt == "lion" else 1e-3, beta2=0.99 if opt == "lion" else None)
    if state in ("int8", "e4m3") and K % 128:
        # block-scaled states need K % block == 0: the final step is rejected
        # before any launch, and the accumulator is left as it was
        Xl, dYl = mb[-1]
        assert_rejected(L, lambda: F.forge_wgrad_step_accumulated(Xl, dYl, acc, L.W, L.forge_m(), L.forge_v(), h, 8,
                                                                  SEED, check=False), extra=(acc,))
        return
    # the oracle's batch: all micro-batches' tokens
    L.X = torch.cat([X for X, _ in mb])
    L.dY = torch.cat([dY for _, dY in mb])
    snap = snapshot(L)
    snap.extra_terms = len(bts)
    Xl, dYl = mb[-1]
    F.forge_wgrad_step_accumulated(Xl, dYl, acc, L.W, L.forge_m(), L.forge_v(), h, 8, SEED)
    torch.cuda.synchronize()
    assert_ok(check_against_oracle(snap, L, h, 8, SEED), f"accumulated {opt} {state}")


@pytest.mark.parametrize("opt,state", [("adamw", "f32"), ("adamw", "int8"), ("adamw", "e4m3"), ("nadam", "bf16"),
                                       ("sgd", None)])
def test_fused_final_step_equals_accumulate_then_step(opt, state):
    """Fused kernel reading the accumulator == adding the last micro-batch
    into the accumulator first and stepping with no further tokens."""
    _say(f"case: fused accumulator read vs accumulate-then-step {opt} {state}")
    N, K = 640, 1024
    spec = _spec(opt, state or "f32")
    A = make_layer(23, N, K, 1, 4, spec, gen_device="cuda")
    B = A.clone()
    mb = _micro(23, (200, 312), N, K, "bf16")
    acc_a = torch.empty((N, K), device="cuda")
    F.forge_wgrad_accumulate(*mb[0], acc_a, first=True)
    acc_b = acc_a.clone()
    h = F.hyper(opt)
    F.forge_wgrad_step_accumulated(*mb[1], acc_a, A.W, A.forge_m(), A.forge_v(), h, 4, SEED)
    F.forge_wgrad_accumulate(*mb[1], acc_b, first=False)
    X0 = torch.empty((0, K), device="cuda", dtype=torch.bfloat16)
    dY0 = torch.empty((0, N), device="cuda", dtype=torch.bfloat16)
    F.forge_wgrad_step_accumulated(X0, dY0, acc_b, B.W, B.forge_m(), B.forge_v(), h, 4, SEED)
    torch.cuda.synchronize()
    for name in ("W", "m", "v", "ms", "vs"):
        a, b = getattr(A, name), getattr(B, name)
        if a is not None:
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b), f"{name} differs"
