"""GPU: the input gradient dX = dY W (Remark 1's upstream GEMM) and
forge_backward_step (dX from the pre-update W, then the fused step).

dX is compared with the oracle's fp64 product element by element: fp32
outputs within the fp32 summation bound 2 gamma_{N+1} sum |dY W| (any
order), bf16 outputs within one bf16 ULP more (round to nearest even of a
value inside that interval).  Shapes cover the MFMA kernel (aligned bf16,
ragged against its 128-token tiles, 32-element reduction chunks and
128-column tiles) and the plain kernel (unaligned, fp32 and mixed dtypes,
strided buffers), the empty reduction, and full Llama layers on sampled
token rows.
"""

import sys

import numpy as np
import pytest
import torch

import backward_weight_gradient_amd as F
import oracle as O
import synth
from forge_testlib import assert_rejected, make_layer

pytestmark = pytest.mark.gpu
SEED = 1337


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _bf16_ulp(x):
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def _check(dX, dY, W, rows=None, what=""):
    dYh, Wh = synth.host(dY), synth.host(W)
    ref = O.input_grad(dYh, Wh, rows)
    E = O.input_grad_error_bound(dYh, Wh, rows)
    idx = slice(None) if rows is None else torch.as_tensor(rows, device=dX.device)
    g = synth.host(dX[idx])
    if dX.dtype == torch.bfloat16:
        got = O.bf16_bits_to_f64(g)
        tol = E + _bf16_ulp(np.abs(ref) + E)
    else:
        got = g.astype(np.float64)
        tol = E + 1e-30
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} dX elements off, e.g. "
                           f"{tuple(np.argwhere(bad)[0])} got {got[tuple(np.argwhere(bad)[0])]!r} "
                           f"ref {ref[tuple(np.argwhere(bad)[0])]!r}")


def _operands(BT, N, K, dy_dtype, w_dtype, cfg=30):
    X, dY = synth.activations(cfg, BT, N, K, 1, in_dtype=dy_dtype, dy_std=1.0)
    W = synth.normal((N, K), 0.02, "cpu", cfg, 0, synth.T_W, 0)
    W = W.to(torch.bfloat16) if w_dtype == "bf16" else W
    return dY.cuda(), W.cuda()


DT = {"bf16": torch.bfloat16, "f32": torch.float32}


# (200, 520, 264): four reduction groups over 17 chunks (the last iteration of groups 1-3 reads a
# chunk past the end, which must contribute zero); (130, 4360, 264): two groups over 137 chunks
@pytest.mark.parametrize("BT,N,K", [(300, 136, 264), (1, 8, 8), (130, 1000, 520), (512, 1024, 1024),
                                    (64, 32, 128), (200, 520, 264), (130, 4360, 264)])
@pytest.mark.parametrize("dx_dtype", ["bf16", "f32"])
def test_dgrad_mfma_kernel(BT, N, K, dx_dtype):
    _say(f"case: dgrad MFMA {BT}x{N}x{K} dX {dx_dtype}")
    dY, W = _operands(BT, N, K, "bf16", "bf16")
    dX = torch.full((BT, K), float("nan"), device="cuda", dtype=DT[dx_dtype])
    F.forge_dgrad(dY, W, dX)
    torch.cuda.synchronize()
    _check(dX, dY, W, what=f"{BT}x{N}x{K}")


@pytest.mark.parametrize("BT,N,K,dy,w", [(129, 131, 65, "bf16", "bf16"), (64, 200, 97, "f32", "f32"),
                                         (100, 64, 72, "bf16", "f32"), (70, 48, 40, "f32", "bf16"),
                                         (3, 1, 5, "bf16", "bf16")])
@pytest.mark.parametrize("dx_dtype", ["bf16", "f32"])
def test_dgrad_plain_kernel(BT, N, K, dy, w, dx_dtype):
    _say(f"case: dgrad plain {BT}x{N}x{K} {dy}/{w} dX {dx_dtype}")
    dY, W = _operands(BT, N, K, dy, w)
    dX = torch.full((BT, K), float("nan"), device="cuda", dtype=DT[dx_dtype])
    F.forge_dgrad(dY, W, dX)
    torch.cuda.synchronize()
    _check(dX, dY, W, what=f"{BT}x{N}x{K} {dy}/{w}")


def test_dgrad_strided_buffers_and_empty_reduction():
    _say("case: dgrad strided, N = 0")
    BT, N, K = 200, 264, 136
    dYb, Wb = _operands(BT, N + 8, K + 16, "bf16", "bf16")
    dY, W = dYb[:, :N], Wb[:N, :K]                     # ld > cols for both (still 16-byte aligned rows)
    big = torch.full((BT, K + 24), float("nan"), device="cuda")
    dX = big[:, :K]
    F.forge_dgrad(dY, W, dX)
    torch.cuda.synchronize()
    _check(dX, dY.contiguous(), W.contiguous(), what="strided")
    assert torch.isnan(big[:, K:]).all(), "dX columns past K were written"
    dY0 = torch.empty((BT, 0), device="cuda", dtype=torch.bfloat16)
    W0 = torch.empty((0, K), device="cuda", dtype=torch.bfloat16)
    dX0 = torch.full((BT, K), float("nan"), device="cuda")
    F.forge_dgrad(dY0, W0, dX0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dX0).item() == 0


@pytest.mark.parametrize("name", ["q_proj", "gate_proj", "down_proj"])
def test_dgrad_full_size_llama_bt512(name):
    N, K = synth.LLAMA8B_LAYERS[name]
    _say(f"case: dgrad {name} {N}x{K} BT512")
    dY, W = _operands(512, N, K, "bf16", "bf16")
    dX = torch.empty((512, K), device="cuda", dtype=torch.bfloat16)
    F.forge_dgrad(dY, W, dX)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 127, 128, 255, 256, 511} | set(np.random.default_rng(3).choice(512, 20).tolist())))
    _check(dX, dY, W, rows, what=name)


@pytest.mark.parametrize("opt,spec", [("adamw", synth.LayerSpec("bf16", "bf16", "f32", "f32")),
                                      ("rmsprop", synth.LayerSpec("bf16", "f32", None, "bf16")),
                                      ("adamw", synth.LayerSpec("bf16", "bf16", "s8", "u8", block=128)),
                                      ("lion", synth.LayerSpec("bf16", "bf16", "e4m3", None, block=64))])
@pytest.mark.parametrize("N,K,BT", [(512, 1024, 300), (130, 136, 65)])
def test_backward_step_orders_dgrad_before_the_update(opt, spec, N, K, BT):
    """dX comes from the weight before the step; the step is forge_wgrad_step's, bit for bit."""
    _say(f"case: backward step {opt} {N}x{K} BT{BT}")
    L = make_layer(31, N, K, BT, 6, spec)
    R = L.clone()
    W_before = L.W.clone()
    dX = torch.empty((BT, K), device="cuda", dtype=torch.bfloat16)
    h = F.hyper(opt)
    if spec.m_fmt in ("s8", "e4m3") and K % spec.block:
        # block-scaled states need K % block == 0: rejected before anything
        # (the dX GEMM included) is enqueued
        dX.fill_(3.0)
        assert_rejected(L, lambda: F.forge_backward_step(L.X, L.dY, L.W, L.forge_m(), L.forge_v(), h, 6, SEED, dX,
                                                         check=False), extra=(dX,))
        return
    F.forge_backward_step(L.X, L.dY, L.W, L.forge_m(), L.forge_v(), h, 6, SEED, dX)
    dX_ref = torch.empty_like(dX)
    F.forge_dgrad(R.dY, W_before, dX_ref)
    F.forge_wgrad_step(R.X, R.dY, R.W, R.forge_m(), R.forge_v(), h, 6, SEED)
    torch.cuda.synchronize()
    assert torch.equal(dX.view(torch.int16), dX_ref.view(torch.int16)), "dX did not use the pre-update weight"
    for name in ("W", "m", "v", "ms", "vs"):
        a, b = getattr(L, name), getattr(R, name)
        if a is not None:
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b), f"{name} differs"


# ---------------------------------------------------------------------------
# forge_dgrad_split: the reduction split across workgroups into a workspace
# ---------------------------------------------------------------------------
# (130, 2056, 520): ragged token and column tiles, two splits of 33 and 32 chunks, the last one partial
# (300, 2048, 1024), (130, 2056, 520), (64, 4096, 128), (512, 8192, 2048):
# 128-token tiles; (512, 8192, 3072), (520, 8200, 2056), (300, 8192, 4104):
# 256 x 256 tiles (k_dgrad_wide), the last two ragged in tokens, reduction
# and columns
@pytest.mark.parametrize("BT,N,K", [(300, 2048, 1024), (130, 2056, 520), (64, 4096, 128), (512, 8192, 2048),
                                    (512, 8192, 3072), (520, 8200, 2056), (300, 8192, 4104)])
@pytest.mark.parametrize("dx_dtype", ["bf16", "f32"])
def test_dgrad_split_matches_oracle(BT, N, K, dx_dtype):
    _say(f"case: dgrad split {BT}x{N}x{K} dX {dx_dtype}")
    need = F.forge_dgrad_workspace_bytes(BT, N, K)
    assert need > 0, "these shapes take the split"
    dY, W = _operands(BT, N, K, "bf16", "bf16")
    ws = torch.full((need // 4,), float("nan"), device="cuda")
    dX = torch.full((BT, K), float("nan"), device="cuda", dtype=DT[dx_dtype])
    F.forge_dgrad_split(dY, W, dX, ws)
    torch.cuda.synchronize()
    _check(dX, dY, W, what=f"split {BT}x{N}x{K}")
    again = torch.full_like(dX, float("nan"))
    F.forge_dgrad_split(dY, W, again, ws)
    torch.cuda.synchronize()
    assert torch.equal(dX.view(torch.uint8), again.view(torch.uint8)), "split result differs between calls"


@pytest.mark.parametrize("name", ["q_proj", "gate_proj", "down_proj"])
def test_dgrad_split_full_size_llama_bt512(name):
    N, K = synth.LLAMA8B_LAYERS[name]
    _say(f"case: dgrad split {name} {N}x{K} BT512")
    need = F.forge_dgrad_workspace_bytes(512, N, K)
    # q_proj: 64-token tiles fill the chip unsplit, no workspace; gate: 8
    # splits of 256 x 256 tiles; down: 2 splits
    assert (need == 0) == (name == "q_proj")
    dY, W = _operands(512, N, K, "bf16", "bf16")
    ws = torch.empty((need // 4,), device="cuda") if need else None
    dX = torch.empty((512, K), device="cuda", dtype=torch.bfloat16)
    F.forge_dgrad_split(dY, W, dX, ws)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 127, 128, 255, 256, 511} | set(np.random.default_rng(5).choice(512, 20).tolist())))
    _check(dX, dY, W, rows, what=f"split {name}")


def test_dgrad_split_where_it_does_not_apply_is_dgrad():
    _say("case: dgrad split not applicable")
    # enough 128-token tiles: no split, no workspace, bit-equal to forge_dgrad
    BT, N, K = 2048, 256, 2048
    assert F.forge_dgrad_workspace_bytes(BT, N, K) == 0
    dY, W = _operands(BT, N, K, "bf16", "bf16")
    a = torch.empty((BT, K), device="cuda", dtype=torch.bfloat16)
    b = torch.empty_like(a)
    F.forge_dgrad(dY, W, a)
    F.forge_dgrad_split(dY, W, b, None)
    # fp32 operands take the plain kernel: the workspace is not touched
    BT, N, K = 300, 2048, 1024
    need = F.forge_dgrad_workspace_bytes(BT, N, K)
    dY32, W32 = _operands(BT, N, K, "f32", "f32")
    ws = torch.full((need // 4,), float("nan"), device="cuda")
    c = torch.empty((BT, K), device="cuda")
    d = torch.empty_like(c)
    F.forge_dgrad(dY32, W32, c)
    F.forge_dgrad_split(dY32, W32, d, ws)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c, d)
    assert torch.isnan(ws).all(), "the workspace was written on the plain path"


def test_backward_step_split_orders_split_dgrad_before_the_update():
    """forge_backward_step_split = forge_dgrad_split on the weight before the step, then forge_wgrad_step."""
    BT, N, K = 300, 2048, 1024
    _say(f"case: backward step split {N}x{K} BT{BT}")
    spec = synth.LayerSpec("bf16", "bf16", "f32", "f32")
    need = F.forge_dgrad_workspace_bytes(BT, N, K)
    assert need > 0
    L = make_layer(32, N, K, BT, 6, spec)
    R = L.clone()
    W_before = L.W.clone()
    ws = torch.empty((need // 4,), device="cuda")
    dX = torch.empty((BT, K), device="cuda", dtype=torch.bfloat16)
    h = F.hyper("adamw")
    F.forge_backward_step_split(L.X, L.dY, L.W, L.forge_m(), L.forge_v(), h, 6, SEED, dX, ws)
    dX_ref = torch.empty_like(dX)
    F.forge_dgrad_split(R.dY, W_before, dX_ref, ws)
    F.forge_wgrad_step(R.X, R.dY, R.W, R.forge_m(), R.forge_v(), h, 6, SEED)
    torch.cuda.synchronize()
    assert torch.equal(dX.view(torch.int16), dX_ref.view(torch.int16)), "dX did not use the pre-update weight"
    for name in ("W", "m", "v"):
        a, b = getattr(L, name), getattr(R, name)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{name} differs"
    _check(dX, L.dY, W_before, what="backward step split")


@pytest.mark.parametrize("BT,N,K", [(200, 2048, 1024), (512, 8192, 3072)])
def test_dgrad_split_strided_buffers(BT, N, K):
    """Leading dimensions larger than the row length on dY, W and dX; dX columns past K stay untouched
    (128-token tiles, then 256 x 256 tiles)."""
    _say(f"case: dgrad split strided {BT}x{N}x{K}")
    need = F.forge_dgrad_workspace_bytes(BT, N, K)
    assert need > 0
    dYb, Wb = _operands(BT, N + 8, K + 16, "bf16", "bf16")
    dY, W = dYb[:, :N], Wb[:N, :K]                     # 16-byte aligned rows, ld > cols
    big = torch.full((BT, K + 24), float("nan"), device="cuda", dtype=torch.bfloat16)
    dX = big[:, :K]
    ws = torch.full((need // 4,), float("nan"), device="cuda")
    F.forge_dgrad_split(dY, W, dX, ws)
    torch.cuda.synchronize()
    _check(dX, dY.contiguous(), W.contiguous(), what="split strided")
    assert torch.isnan(big[:, K:].float()).all(), "dX columns past K were written"
