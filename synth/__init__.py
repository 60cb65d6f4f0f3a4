"""Seeded synthetic inputs for the weight-gradient + optimizer step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the tests (for the oracle and the HIP path alike)
and the benchmark take their inputs from here, so the two sides always see the
same bytes.

Recipe: every tensor is drawn from its own ``torch.Generator`` whose seed is
derived from (1337, config, step, tensor code) by NumPy's ``SeedSequence``;
normals are drawn in float32 and cast to bfloat16 with torch's own cast where
a bf16 tensor is wanted.  Generators on "cpu" and on "cuda" give different
(each deterministic) streams, so a test that checks a GPU result against the
oracle draws once and hands the same tensors to both.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

SEED_BASE = 1337
T_X, T_DY, T_W, T_M, T_V, T_OUTLIER = range(6)

# Llama-3.1-8B linear layers: name -> (D_out = N, D_in = K)
LLAMA8B_LAYERS = {
    "q_proj": (4096, 4096),
    "k_proj": (1024, 4096),
    "v_proj": (1024, 4096),
    "o_proj": (4096, 4096),
    "gate_proj": (14336, 4096),
    "up_proj": (14336, 4096),
    "down_proj": (4096, 14336),
}
LM_HEAD = (128256, 4096)


def seed_for(cfg: int, step: int, tensor: int, extra: int = 0) -> int:
    ss = np.random.SeedSequence([SEED_BASE, cfg, step, tensor, extra])
    return int(ss.generate_state(1, np.uint64)[0] & np.uint64(0x7FFFFFFFFFFFFFFF))


def _gen(device, cfg, step, tensor, extra=0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(cfg, step, tensor, extra))
    return g


def normal(shape, std, device, cfg, step, tensor, extra=0) -> torch.Tensor:
    """float32 N(0, std^2) draws (std is the standard deviation)."""
    g = _gen(device, cfg, step, tensor, extra)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def uniform_int(shape, lo, hi, device, cfg, step, tensor, extra=0, dtype=torch.uint8):
    g = _gen(device, cfg, step, tensor, extra)
    return torch.randint(lo, hi, shape, generator=g, device=device, dtype=torch.int64).to(dtype)


def bernoulli(shape, p, device, cfg, step, tensor, extra=0) -> torch.Tensor:
    g = _gen(device, cfg, step, tensor, extra)
    return torch.rand(shape, generator=g, device=device) < p


@dataclass
class LayerSpec:
    """Formats of one layer's tensors."""
    in_dtype: str = "bf16"   # X, dY: "bf16" | "f32"
    w_fmt: str = "bf16"      # "bf16" | "f32"
    m_fmt: Optional[str] = "f32"   # "f32" | "bf16" | "s8" | "e4m3" | None
    v_fmt: Optional[str] = "f32"   # "f32" | "bf16" | "u8" | "e4m3" | None
    block: int = 128


def _cast(x: torch.Tensor, fmt: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if fmt == "bf16" else x.to(torch.float32)


def activations(cfg, BT, N, K, step, *, in_dtype="bf16", x_std=1.0, dy_std=1e-3,
                outlier_p=0.0, outlier_scale=50.0, device="cpu", extra=0):
    """X [BT, K] ~ N(0, x_std^2) and dY [BT, N] ~ N(0, dy_std^2), fresh per step;
    with ``outlier_p`` > 0 a Bernoulli(outlier_p) subset of dY is multiplied by
    ``outlier_scale`` before the cast."""
    X = normal((BT, K), x_std, device, cfg, step, T_X, extra)
    dY = normal((BT, N), dy_std, device, cfg, step, T_DY, extra)
    if outlier_p > 0:
        mask = bernoulli((BT, N), outlier_p, device, cfg, step, T_OUTLIER, extra)
        dY = torch.where(mask, dY * outlier_scale, dY)
    return _cast(X, in_dtype), _cast(dY, in_dtype)


def state(cfg, N, K, spec: LayerSpec, *, w_std=0.02, v_std=1e-6, v_zero=False,
          device="cpu", extra=0, step=0):
    """W ~ N(0, w_std^2); m = 0; v = |N(0, v_std^2)| (or 0 with ``v_zero``).

    int8 moments: m starts as all-zero codes with zero scales; v (when not
    zero) starts as uniform random codes in 1..255 with one scale per block
    equal to 3.5*v_std/255, a stand-in for a quantised |N(0, v_std^2)| state.
    Returns dict W, m, v, m_scale, v_scale (absent entries are None).
    """
    out = {"W": _cast(normal((N, K), w_std, device, cfg, step, T_W, extra), spec.w_fmt),
           "m": None, "v": None, "m_scale": None, "v_scale": None}
    nb = K // spec.block if spec.block else 0
    if spec.m_fmt in ("f32", "bf16"):
        out["m"] = torch.zeros((N, K), device=device, dtype=torch.float32 if spec.m_fmt == "f32" else torch.bfloat16)
    elif spec.m_fmt == "s8":
        out["m"] = torch.zeros((N, K), device=device, dtype=torch.int8)
        out["m_scale"] = torch.zeros((N, nb), device=device, dtype=torch.float32)
    elif spec.m_fmt == "e4m3":
        out["m"] = torch.zeros((N, K), device=device, dtype=torch.uint8).view(torch.float8_e4m3fn)
        out["m_scale"] = torch.zeros((N, nb), device=device, dtype=torch.float32)
    if spec.v_fmt in ("f32", "bf16"):
        if v_zero:
            v = torch.zeros((N, K), device=device, dtype=torch.float32)
        else:
            v = normal((N, K), v_std, device, cfg, step, T_V, extra).abs()
        out["v"] = _cast(v, spec.v_fmt)
    elif spec.v_fmt == "u8":
        if v_zero:
            out["v"] = torch.zeros((N, K), device=device, dtype=torch.uint8)
            out["v_scale"] = torch.zeros((N, nb), device=device, dtype=torch.float32)
        else:
            out["v"] = uniform_int((N, K), 1, 256, device, cfg, step, T_V, extra)
            out["v_scale"] = torch.full((N, nb), 3.5 * v_std / 255.0, device=device, dtype=torch.float32)
    elif spec.v_fmt == "e4m3":
        if v_zero:
            out["v"] = torch.zeros((N, K), device=device, dtype=torch.uint8).view(torch.float8_e4m3fn)
            out["v_scale"] = torch.zeros((N, nb), device=device, dtype=torch.float32)
        else:
            # positive E4M3 codes 1 .. 0x7E (subnormals and normals up to 448)
            out["v"] = uniform_int((N, K), 1, 0x7F, device, cfg, step, T_V, extra).view(torch.float8_e4m3fn)
            out["v_scale"] = torch.full((N, nb), 3.5 * v_std / 448.0, device=device, dtype=torch.float32)
    return out


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """The uint16 bit patterns of a bfloat16 tensor, as a host NumPy array."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    """Host NumPy copy: bf16 as uint16 bits, everything else as-is."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    if t.dtype == torch.float8_e4m3fn:
        return t.detach().cpu().contiguous().view(torch.uint8).numpy()
    return t.detach().cpu().contiguous().numpy()
