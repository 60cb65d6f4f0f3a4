"""GPU: forge_wgrad_step_group.

The grouped call must equal separate forge_wgrad_step calls bit for bit
(same arithmetic per element, same SR keys), and the oracle checks a group's
layers element by element.  Groups cover the q/k/v pattern (three layers
reading one X), eight layers of mixed shapes and token counts (ragged tiles,
BT = 0, an empty layer, a layer that needs its own launch because its rows
are not 16-byte aligned, one long enough for the wide kernel), and every
state format and optimizer.  At full size, the seven linear layers of a
Llama-3.1-8B decoder layer at BT = 512 go through one call, the launch the
throughput figure times.
"""

import sys

import numpy as np
import pytest
import torch

import backward_weight_gradient_amd as F
import synth
from forge_testlib import assert_ok, check_against_oracle, make_layer, sample_rows, snapshot

pytestmark = pytest.mark.gpu
SEED = 1337

SPEC_CFG1 = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="f32", v_fmt="f32")
SPEC_CFG2 = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="bf16", v_fmt="bf16")
SPEC_CFG3 = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="s8", v_fmt="u8", block=128)
SPEC_F32W = synth.LayerSpec(in_dtype="bf16", w_fmt="f32", m_fmt="f32", v_fmt="f32")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _hyper(opt):
    if opt == "lion":
        return F.hyper("lion", lr=1e-4, beta2=0.99)
    return F.hyper(opt)


def _args(L, seed):
    return (L.X, L.dY, L.W, L.forge_m(), L.forge_v(), seed)


def _bytes(t):
    return t.view(torch.uint8) if t.dtype != torch.uint8 else t


def _assert_same_state(a, b, what):
    for name in ("W", "m", "v", "ms", "vs"):
        x, y = getattr(a, name), getattr(b, name)
        if x is None:
            assert y is None
            continue
        assert torch.equal(_bytes(x), _bytes(y)), f"{what}: {name} differs from the separate call"


def _group_vs_separate(layers, h, step, seeds):
    ref = [L.clone() for L in layers]
    F.forge_wgrad_step_group([_args(L, s) for L, s in zip(layers, seeds)], h, step)
    for R, s in zip(ref, seeds):
        F.forge_wgrad_step(R.X, R.dY, R.W, R.forge_m(), R.forge_v(), h, step, s)
    torch.cuda.synchronize()
    for i, (L, R) in enumerate(zip(layers, ref)):
        _assert_same_state(L, R, f"layer {i} ({L.N}x{L.K}, BT {L.BT})")


@pytest.mark.parametrize("spec,opt", [(SPEC_CFG1, "adamw"), (SPEC_CFG2, "adamw"), (SPEC_CFG3, "adamw"),
                                      (SPEC_F32W, "adamw"),
                                      (synth.LayerSpec("bf16", "bf16", "f32", None), "lion"),
                                      (synth.LayerSpec("bf16", "bf16", "s8", None, block=128), "sgdm")])
def test_group_qkv_pattern(spec, opt):
    """q, k, v of one attention block: one X, three dY, one launch."""
    _say(f"case: group q/k/v {spec} {opt}")
    BT, K = 300, 1024
    shapes = [(512, K), (128, K), (128, K)]
    layers = [make_layer(6, N, K, BT, 4, spec, extra=i, outlier_p=0.01 if spec.m_fmt == "s8" else 0.0)
              for i, (N, K) in enumerate(shapes)]
    for L in layers[1:]:
        L.X = layers[0].X
    h = _hyper(opt)
    seeds = [SEED + 11 * i for i in range(3)]
    snaps = [snapshot(L) if L.N <= 128 else snapshot(L, np.array([0, 1, 127, 128, 255, 256, 383, 384, 511]))
             for L in layers]
    _group_vs_separate(layers, h, 4, seeds)      # `layers` now hold the grouped result
    for i, (L, snap, s) in enumerate(zip(layers, snaps, seeds)):
        assert_ok(check_against_oracle(snap, L, h, 4, s), f"group q/k/v layer {i}")


# Block-scaled moments at each block size: 128 takes the grouped kernel with
# the block fixed at compile time, 32 and 64 the one that reads it per layer.
@pytest.mark.parametrize("block", [32, 64, 128])
@pytest.mark.parametrize("m_fmt,v_fmt", [("s8", "u8"), ("e4m3", "e4m3")])
def test_group_block_sizes(m_fmt, v_fmt, block):
    _say(f"case: group q/k/v, {m_fmt}/{v_fmt} moments, block {block}")
    spec = synth.LayerSpec("bf16", "bf16", m_fmt, v_fmt, block=block)
    BT, K = 300, 1024
    layers = [make_layer(10, N, K, BT, 5, spec, extra=i, outlier_p=0.01)
              for i, N in enumerate((384, 128, 136))]
    for L in layers[1:]:
        L.X = layers[0].X
    h = F.hyper("adamw")
    seeds = [SEED + 5 * i for i in range(3)]
    snaps = [snapshot(L) for L in layers]
    _group_vs_separate(layers, h, 5, seeds)      # `layers` now hold the grouped result
    for i, (L, snap, s) in enumerate(zip(layers, snaps, seeds)):
        assert_ok(check_against_oracle(snap, L, h, 5, s), f"group block {block} layer {i}")


@pytest.mark.parametrize("spec", [SPEC_CFG1, SPEC_CFG2])
def test_group_eight_mixed_layers(spec):
    """Eight layers of different shapes and token counts in one call."""
    _say(f"case: group of eight mixed layers {spec}")
    cases = [(256, 256, 64), (136, 520, 100), (1024, 128, 512), (8, 8, 1),
             (264, 1001, 77),     # K % 8 != 0: rows not 16-byte aligned, runs as its own launch
             (256, 512, 4100),    # long token axis: the wide kernel, its own launch
             (0, 256, 64),        # empty: nothing to do
             (128, 128, 0)]       # BT = 0: the step with G = 0
    layers = [make_layer(7, N, K, BT, 2, spec, extra=i) for i, (N, K, BT) in enumerate(cases)]
    h = F.hyper("adamw")
    seeds = [SEED * (i + 1) for i in range(len(layers))]
    snaps = [snapshot(L) if L.N else None for L in layers]
    _group_vs_separate(layers, h, 2, seeds)      # `layers` now hold the grouped result
    for i, (L, snap, s) in enumerate(zip(layers, snaps, seeds)):
        if snap is not None:
            assert_ok(check_against_oracle(snap, L, h, 2, s), f"group layer {i} {cases[i]}")


def test_group_of_one_equals_the_single_call():
    _say("case: group of one")
    L = make_layer(8, 392, 776, 333, 3, SPEC_CFG1)
    _group_vs_separate([L], F.hyper("adamw"), 3, [SEED])


def test_group_repeated_steps_bit_equal():
    """Three steps of a two-layer group equal three steps of separate calls."""
    _say("case: group, three steps")
    a = [make_layer(9, 384, 640, 128, 1, SPEC_CFG2, extra=i) for i in range(2)]
    b = [L.clone() for L in a]
    h = F.hyper("adamw")
    for t in (1, 2, 3):
        F.forge_wgrad_step_group([_args(L, SEED + i) for i, L in enumerate(a)], h, t)
        for i, L in enumerate(b):
            F.forge_wgrad_step(L.X, L.dY, L.W, L.forge_m(), L.forge_v(), h, t, SEED + i)
    torch.cuda.synchronize()
    for L, R in zip(a, b):
        _assert_same_state(L, R, "three steps")


# The seven layers of a Llama-3.1-8B decoder layer at BT = 512 in one call, in
# the order the throughput figure launches them: bf16 X, dY and W, AdamW with
# SR on W at t = 10; fp32 m and v (the timed configuration), bf16 m and v, and
# int8 m and v with 1% gradient outliers.  Every element of every layer is compared
# with separate single-layer calls (bit for bit), and sampled rows and column
# blocks of each layer with the oracle.
DECODER_LAYER = ("gate_proj", "up_proj", "down_proj", "q_proj", "k_proj", "v_proj", "o_proj")


@pytest.mark.parametrize("cfg,spec", [(1, SPEC_CFG1), (2, SPEC_CFG2), (3, SPEC_CFG3)])
def test_llama_decoder_layer_group_full_size(cfg, spec):
    _say(f"case: group, Llama-3.1-8B decoder layer, BT 512, full size, {spec}")
    step, BT = 10, 512
    h = F.hyper("adamw", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, round="sr")
    layers, snaps, cols = [], [], []
    for i, name in enumerate(DECODER_LAYER):
        N, K = synth.LLAMA8B_LAYERS[name]
        L = make_layer(cfg, N, K, BT, step, spec, gen_device="cuda", extra=i,
                       outlier_p=0.01 if spec.m_fmt == "s8" else 0.0)
        rows = sample_rows(N, 24, seed=N + K + i)
        nb = K // 128
        rng = np.random.default_rng(K + i)
        blocks = sorted({0, nb - 1} | set(int(b) for b in rng.choice(nb, size=2, replace=False)))
        layers.append(L)
        snaps.append(snapshot(L, rows))
        cols.append([(b * 128, b * 128 + 128) for b in blocks])
    torch.cuda.synchronize()
    _group_vs_separate(layers, h, step, [SEED] * len(layers))   # `layers` now hold the grouped result
    for name, L, snap, c in zip(DECODER_LAYER, layers, snaps, cols):
        assert_ok(check_against_oracle(snap, L, h, step, SEED, col_ranges=c), name)
    del layers
    torch.cuda.empty_cache()
