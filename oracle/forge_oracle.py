"""Plain CPU oracle for one fused weight-gradient + optimizer step.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  The product never
imports this module.

What it computes (FORGE paper, arXiv 2606.22932):

* the weight gradient of a linear layer ``Y = X W^T``:
  ``G[p, q] = sum_t dY[t, p] * X[t, q]``  (section 2.1, Eq. 3; Appendix A,
  "Setup"), for W of shape [N = D_out, K = D_in], X [BT, K], dY [BT, N];
* one element-wise optimizer step per coordinate (Appendix A, Definition 1):
  AdamW with bias correction and decoupled decay (Algorithm 1, Phase 2),
  Lion and SGD with momentum (Appendix N, "fully fused" list);
* the write-back in the stored precision (Algorithm 1, Phase 3): fp32 with
  round-to-nearest-even, bf16 with round-to-nearest-even or stochastic
  rounding (Appendix C), or int8 block-absmax moments (section 2.3 and
  Appendix B).

By Proposition 1 (per-tile exactness) the fused per-tile schedule reaches the
same result as "materialise G, then step", so the oracle *is* that plain
definition: G from a library fp64 matmul (every bf16*bf16 and fp32*fp32
product is exact in fp64), then the textbook step in fp64 on the decoded
stored values, then one rounding to the storage format.  ``step_tiled``
additionally runs the per-tile schedule itself, so that Proposition 1 and
Corollary 1(a) can be checked on the oracle.

Readings taken where the pages leave a step open (each is repeated in the
design notes):

* Lion follows its textbook form (Chen et al. 2023): interpolate
  ``c = b1*m + (1-b1)*G``, update ``W <- (1-lr*wd)*W - lr*sign(c)`` with
  sign(0) = 0, then ``m <- b2*m + (1-b2)*G``.
* SGD with momentum follows PyTorch SGD semantics (the paper checks each
  fused family against PyTorch's own implementation, Appendix N):
  coupled L2 decay ``g = G + wd*W``, ``b <- mu*b + g`` (dampening 0, no
  Nesterov), ``W <- W - lr*b``; ``mu`` is passed as ``beta1``.
* NAdam, RAdam, RMSprop, AdaGrad and plain SGD: the pages name each family
  in one line (Appendix N, "fully fused") and verify it against a PyTorch
  reference, so each follows its textbook rule as PyTorch states it.  NAdam
  ("AdamW with Nesterov momentum correction on m_hat", Dozat 2016) uses the
  momentum schedule ``mu_i = b1 (1 - 0.5 * 0.96^(0.004 i))`` and its running
  product; RAdam ("AdamW with rectified-variance term", Liu et al. 2019)
  takes the adaptive step only once ``rho_t > 5``; both take AdamW's
  decoupled decay (the pages call them AdamW variants).  RMSprop ("second
  moment only") keeps ``v <- a v + (1-a) g^2`` with ``a = beta2``, no
  momentum, not centred; AdaGrad (a running sum of squared gradients) keeps
  ``v <- v + g^2`` with no learning-rate decay; RMSprop, AdaGrad and SGD take
  coupled L2 decay like SGD with momentum.
* The step index t is 1-based and is used directly in the bias correction.
* The SR random bits come from a counter-based hash of (seed, step, tensor,
  flat index).  The pages name only a cheap integer hash of the seed and an
  offset, of the splitmix kind, in place of Philox (Appendix C,
  Implementation; Table 3); the hash used here is the MurmurHash3 32-bit finaliser ``fmix32`` (Appleby, public
  domain), composed as documented in :func:`sr_key` and :func:`sr_bits`.
* Stochastic rounding adds 16 random bits below the bf16 cut and truncates
  (rounds |x| up with probability f = (x - x_lo)/ULP, quantised to 2^-16);
  non-finite values take the round-to-nearest-even path.
* int8 moments: per contiguous block of ``block`` elements of a row; m is
  symmetric signed (``s = absmax/127``, codes -127..127), v is unsigned with
  code 0 reserved for an exact zero (``s = absmax/255``, positive values take
  codes 1..255, which keeps v away from zero); quantisation multiplies the
  fp32 value by the correctly-rounded fp32 reciprocal ``127/a`` (``255/a``)
  and rounds half-to-even; the weight update uses the pre-quantisation
  m', v'.

Pins (tests/test_oracle_*.py): hand-worked AdamW / Lion / SGD-m values at
t = 1..3 (tests/golden), closed forms, torch.optim.AdamW / SGD in float64 as
library special cases, exact integer brute-force GEMMs, MurmurHash3 published
test vectors, SR unbiasedness over 1e6 draws and the paper's quarter-ULP
microbenchmark, bf16 RNE against torch's cast, the int8 round-off bound
(Appendix B) and the Proposition 4 drift bound, and Proposition 1 tiling
invariance.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Stored", "Hyper",
    "bf16_bits_to_f64", "f32_to_bf16_rne", "f32_to_bf16_sr",
    "fmix32", "sr_key", "sr_bits",
    "weight_grad", "weight_grad_abs", "grad_error_bound", "input_grad", "input_grad_error_bound",
    "adamw", "lion", "sgdm", "nadam", "radam", "rmsprop", "adagrad", "sgd",
    "nadam_mu", "radam_rect",
    "quantize_signed", "quantize_unsigned", "dequantize",
    "E4M3_MAX", "e4m3_to_f64", "f32_to_e4m3_rne", "f32_to_e4m3_sr", "quantize_e4m3",
    "decode", "encode", "wgrad_step", "apply_step", "step_tiled",
    "TENSOR_W", "TENSOR_M", "TENSOR_V",
]

TENSOR_W, TENSOR_M, TENSOR_V = 0, 1, 2
_M32 = 0xFFFFFFFF
_GOLDEN32 = 0x9E3779B9


# --------------------------------------------------------------------------
# Stored tensors and hyper-parameters
# --------------------------------------------------------------------------
@dataclass
class Stored:
    """A stored matrix.

    fmt  "f32": ``data`` is float32 values.
         "bf16": ``data`` is uint16 bf16 bit patterns.
         "s8" / "u8": ``data`` is int8 / uint8 codes and ``scale`` holds one
         float32 scale per ``block`` consecutive elements of a row
         (shape [rows, cols // block]).
    """
    fmt: str
    data: np.ndarray
    scale: Optional[np.ndarray] = None
    block: int = 128

    def copy(self) -> "Stored":
        return Stored(self.fmt, self.data.copy(),
                      None if self.scale is None else self.scale.copy(), self.block)


@dataclass
class Hyper:
    """Optimizer hyper-parameters (Algorithm 1 inputs: eta, beta1, beta2, eps, lambda)."""
    opt: str = "adamw"          # "adamw" | "lion" | "sgdm" | "nadam" | "radam" | "rmsprop" | "adagrad" | "sgd"
    lr: float = 1e-3
    beta1: float = 0.9          # SGD-m: momentum mu
    beta2: float = 0.999        # RMSprop: smoothing constant a
    eps: float = 1e-8
    weight_decay: float = 0.01
    round: str = "sr"           # bf16 stores: "sr" | "rne"


# --------------------------------------------------------------------------
# bf16 conversions
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values (bf16 is the top half of fp32)."""
    u32 = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):      # signalling-NaN patterns stay NaN
        return u32.view(np.float32).astype(np.float64)


def f32_to_bf16_rne(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(np.ascontiguousarray(x32, dtype=np.float32))
    quiet = ((u >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return np.where(nan, quiet, rounded)


def f32_to_bf16_sr(x32: np.ndarray, r16: np.ndarray) -> np.ndarray:
    """Stochastic rounding fp32 -> bf16 (FORGE paper, Appendix C).

    With x between adjacent bf16 values x_lo <= x <= x_hi and
    f = (x - x_lo)/ULP, the result is x_hi with probability f.  Adding a
    uniform 16-bit integer r16 to the discarded low half of the fp32 pattern
    and truncating does exactly that: the carry into bit 16 happens iff
    r16 >= 2^16 - low16, i.e. with probability low16 / 2^16 = f.  Because the
    pattern is sign-magnitude, the carry increases |x|, so negative values
    round away from zero with the same probability.  Non-finite values are
    rounded to nearest even.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    u = x32.view(np.uint32)
    r = np.asarray(r16, dtype=np.uint32) & np.uint32(0xFFFF)
    sr = ((u + r) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isfinite(x32), sr, f32_to_bf16_rne(x32))


# --------------------------------------------------------------------------
# Counter-based random bits for stochastic rounding
# --------------------------------------------------------------------------
def fmix32(h):
    """MurmurHash3 32-bit finaliser (Appleby, public domain): a bijection on
    32-bit words made of three xor-shifts (16, 13, 16) around two multiplies
    by the odd constants 0x85EBCA6B and 0xC2B2AE35.  Works on Python ints and
    on uint32 arrays."""
    if isinstance(h, np.ndarray):
        h = h.astype(np.uint32)
        h ^= h >> np.uint32(16)
        h = (h.astype(np.uint64) * np.uint64(0x85EBCA6B) & np.uint64(_M32)).astype(np.uint32)
        h ^= h >> np.uint32(13)
        h = (h.astype(np.uint64) * np.uint64(0xC2B2AE35) & np.uint64(_M32)).astype(np.uint32)
        h ^= h >> np.uint32(16)
        return h
    h = int(h) & _M32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & _M32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & _M32
    h ^= h >> 16
    return h


def sr_key(seed: int, step: int, tensor_id: int) -> int:
    """Per-(seed, step, tensor) 32-bit key.

    key = fmix32(lo(seed) ^ fmix32(hi(seed) ^ fmix32(lo(step) ^
          fmix32(hi(step) + 0x9E3779B9*(tensor_id+1)))))   (all mod 2^32)

    where lo/hi are the low/high 32 bits of the 64-bit seed and step.  The
    weight, first and second moment use tensor ids 0, 1, 2, so each stored
    tensor draws an independent stream.
    """
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    step = int(step) & 0xFFFFFFFFFFFFFFFF
    k = fmix32(((step >> 32) + _GOLDEN32 * (int(tensor_id) + 1)) & _M32)
    k = fmix32((step & _M32) ^ k)
    k = fmix32((seed >> 32) ^ k)
    k = fmix32((seed & _M32) ^ k)
    return k


def sr_bits(key: int, flat_index: np.ndarray) -> np.ndarray:
    """16 random bits for each element.  flat_index is the row-major index
    p*K + q of the element in the logical [N, K] matrix; the elements
    2j and 2j + 1 share one hash word

        h_j = fmix32(key ^ (j * 0x9E3779B9 mod 2^32)),

    element 2j taking its top half and element 2j + 1 its bottom half (the
    two halves of a finaliser output are independent uniform 16-bit values,
    so one hash serves two elements)."""
    idx = np.asarray(flat_index, dtype=np.uint64)
    pair = idx >> np.uint64(1)
    mixed = ((pair * np.uint64(_GOLDEN32)) & np.uint64(_M32)).astype(np.uint32)
    h = fmix32(np.uint32(key) ^ mixed)
    odd = (idx & np.uint64(1)).astype(bool)
    return np.where(odd, h & np.uint32(0xFFFF), h >> np.uint32(16)).astype(np.uint32)


# --------------------------------------------------------------------------
# Gradient (Eq. 3 / Eq. 5)
# --------------------------------------------------------------------------
def _as_f64(a: np.ndarray) -> np.ndarray:
    """Decode an input activation array: uint16 = bf16 bits, else float32."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return a.astype(np.float64)


def weight_grad(X: np.ndarray, dY: np.ndarray, rows=None, cols=None,
                order: str = "blas") -> np.ndarray:
    """G[p, q] = sum_t dY[t, p] * X[t, q] for p in ``rows``, q in ``cols``.

    X is [BT, K], dY is [BT, N]; both float32, or uint16 holding bf16 bits.

    order "blas":  fp64 library matmul ``dY^T X`` (the reference value:
                   products are exact in fp64, the sum is rounded in fp64).
    order "seq64": tokens added in ascending order in fp64.
    order "seq32": tokens added in ascending order in fp32 (fp32 product,
                   then fp32 add) -- an fp32 accumulator in one fixed order.
    """
    BT = X.shape[0]
    if dY.shape[0] != BT:
        raise ValueError("X and dY must have the same number of token rows")
    rows = np.arange(dY.shape[1]) if rows is None else np.asarray(rows)
    cols = np.arange(X.shape[1]) if cols is None else np.asarray(cols)
    dYs = _as_f64(dY[:, rows])
    Xs = _as_f64(X[:, cols])
    if order == "blas":
        return dYs.T @ Xs
    if order == "seq64":
        G = np.zeros((len(rows), len(cols)), dtype=np.float64)
        for t in range(BT):
            G += np.multiply.outer(dYs[t], Xs[t])
        return G
    if order == "seq32":
        dY32, X32 = dYs.astype(np.float32), Xs.astype(np.float32)
        G = np.zeros((len(rows), len(cols)), dtype=np.float32)
        for t in range(BT):
            G = G + np.multiply.outer(dY32[t], X32[t])
        return G.astype(np.float64)
    raise ValueError(f"unknown order {order!r}")


def weight_grad_abs(X, dY, rows=None, cols=None) -> np.ndarray:
    """A[p, q] = sum_t |dY[t, p] * X[t, q]| (fp64), the scale of the
    reduction-order error."""
    rows = np.arange(dY.shape[1]) if rows is None else np.asarray(rows)
    cols = np.arange(X.shape[1]) if cols is None else np.asarray(cols)
    return np.abs(_as_f64(dY[:, rows])).T @ np.abs(_as_f64(X[:, cols]))


def grad_error_bound(X, dY, rows=None, cols=None, extra_terms: int = 0) -> np.ndarray:
    """Largest deviation of an fp32-accumulated G from the exact one.

    Corollary 1(b): against any other implementation the only discrepancy is
    the summation order of the token reduction.  For any order with fp32
    accumulation the standard forward error bound is
    ``|G_hat - G| <= gamma_n * sum_t |dY X|`` with ``gamma_n = n u/(1 - n u)``,
    u = 2^-24 and n the number of terms (+1 for a rounded fp32 product).  The
    bound is doubled so that accumulators which truncate instead of rounding
    are covered too.  ``extra_terms`` counts further fp32 additions of
    partial sums (gradient accumulation over micro-batches, Appendix L: one
    per micro-batch), each of which adds at most u * sum_t |dY X|.
    """
    n = X.shape[0] + 1 + extra_terms
    u = 2.0 ** -24
    gamma = n * u / (1.0 - n * u)
    return 2.0 * gamma * weight_grad_abs(X, dY, rows, cols)


def input_grad(dY: np.ndarray, W: np.ndarray, rows=None) -> np.ndarray:
    """The input gradient dX[t, q] = sum_p dY[t, p] W[p, q] (the GEMM that
    Remark 1 orders before the in-place update) for tokens t in ``rows``;
    dY [BT, N], W [N, K], float32 or uint16 bf16 bits.  fp64 library matmul:
    every product is exact in fp64."""
    rows = np.arange(dY.shape[0]) if rows is None else np.asarray(rows)
    return _as_f64(dY[rows]) @ _as_f64(W)


def input_grad_error_bound(dY: np.ndarray, W: np.ndarray, rows=None) -> np.ndarray:
    """Largest deviation of an fp32-accumulated dX from the exact one in any
    summation order: 2 gamma_{N+1} sum_p |dY W| (as grad_error_bound)."""
    rows = np.arange(dY.shape[0]) if rows is None else np.asarray(rows)
    n = dY.shape[1] + 1
    u = 2.0 ** -24
    gamma = n * u / (1.0 - n * u)
    return 2.0 * gamma * (np.abs(_as_f64(dY[rows])) @ np.abs(_as_f64(W)))


# --------------------------------------------------------------------------
# Element-wise optimizers (Definition 1; Algorithm 1 Phase 2; Appendix N)
# --------------------------------------------------------------------------
def adamw(W, G, m, v, t, lr, beta1, beta2, eps, weight_decay):
    """AdamW, Algorithm 1 Phase 2, in fp64:
    m' = b1 m + (1-b1) G;  v' = b2 v + (1-b2) G^2;
    m_hat = m'/(1-b1^t);  v_hat = v'/(1-b2^t);
    W' = (1 - lr*wd) W - lr * m_hat / (sqrt(v_hat) + eps)."""
    m1 = beta1 * m + (1.0 - beta1) * G
    v1 = beta2 * v + (1.0 - beta2) * G * G
    m_hat = m1 / (1.0 - beta1 ** t)
    v_hat = v1 / (1.0 - beta2 ** t)
    W1 = (1.0 - lr * weight_decay) * W - lr * m_hat / (np.sqrt(v_hat) + eps)
    return W1, m1, v1


def lion(W, G, m, lr, beta1, beta2, weight_decay):
    """Lion (Appendix N: the step is the sign of an interpolated momentum,
    and one moment buffer is kept; textbook form of Chen et al. 2023), fp64."""
    c = beta1 * m + (1.0 - beta1) * G
    W1 = (1.0 - lr * weight_decay) * W - lr * np.sign(c)
    m1 = beta2 * m + (1.0 - beta2) * G
    return W1, m1


def sgdm(W, G, b, lr, mu, weight_decay):
    """SGD with momentum (Appendix N; PyTorch semantics: coupled L2 decay,
    dampening 0, no Nesterov), fp64."""
    g = G + weight_decay * W
    b1 = mu * b + g
    W1 = W - lr * b1
    return W1, b1


NADAM_PSI = 0.004   # momentum decay of the NAdam schedule


def nadam_mu(i, beta1):
    """NAdam momentum schedule mu_i = b1 (1 - 0.5 * 0.96^(psi i)) (Dozat 2016,
    as PyTorch states it), i 1-based."""
    return beta1 * (1.0 - 0.5 * 0.96 ** (i * NADAM_PSI))


def nadam(W, G, m, v, t, lr, beta1, beta2, eps, weight_decay):
    """NAdam (Appendix N: AdamW with Nesterov momentum correction on m_hat),
    decoupled decay, fp64:
    m' = b1 m + (1-b1) G;  v' = b2 v + (1-b2) G^2;
    m_hat = mu_{t+1} m' / (1 - prod_{i<=t+1} mu_i) + (1 - mu_t) G / (1 - prod_{i<=t} mu_i);
    W' = (1 - lr wd) W - lr m_hat / (sqrt(v'/(1-b2^t)) + eps)."""
    prod = 1.0
    for i in range(1, t + 1):
        prod *= nadam_mu(i, beta1)
    mu_t, mu_next = nadam_mu(t, beta1), nadam_mu(t + 1, beta1)
    m1 = beta1 * m + (1.0 - beta1) * G
    v1 = beta2 * v + (1.0 - beta2) * G * G
    m_hat = mu_next * m1 / (1.0 - prod * mu_next) + (1.0 - mu_t) * G / (1.0 - prod)
    W1 = (1.0 - lr * weight_decay) * W - lr * m_hat / (np.sqrt(v1 / (1.0 - beta2 ** t)) + eps)
    return W1, m1, v1


def radam_rect(t, beta2):
    """RAdam's rectification at step t (Liu et al. 2019): (rho_t > 5, r_t)."""
    rho_inf = 2.0 / (1.0 - beta2) - 1.0
    rho_t = rho_inf - 2.0 * t * beta2 ** t / (1.0 - beta2 ** t)
    if rho_t <= 5.0:
        return False, 0.0
    return True, np.sqrt((rho_t - 4.0) * (rho_t - 2.0) * rho_inf / ((rho_inf - 4.0) * (rho_inf - 2.0) * rho_t))


def radam(W, G, m, v, t, lr, beta1, beta2, eps, weight_decay):
    """RAdam (Appendix N: AdamW with rectified-variance term), decoupled
    decay, fp64: m', v' as AdamW, m_hat = m'/(1-b1^t); once rho_t > 5
    W' = (1 - lr wd) W - lr m_hat r_t sqrt(1-b2^t) / (sqrt(v') + eps), before
    that W' = (1 - lr wd) W - lr m_hat."""
    m1 = beta1 * m + (1.0 - beta1) * G
    v1 = beta2 * v + (1.0 - beta2) * G * G
    m_hat = m1 / (1.0 - beta1 ** t)
    on, r = radam_rect(t, beta2)
    if on:
        upd = m_hat * r * np.sqrt(1.0 - beta2 ** t) / (np.sqrt(v1) + eps)
    else:
        upd = m_hat
    W1 = (1.0 - lr * weight_decay) * W - lr * upd
    return W1, m1, v1


def rmsprop(W, G, v, lr, alpha, eps, weight_decay):
    """RMSprop (Appendix N: second moment only, no first moment), coupled
    decay, no momentum, not centred, fp64:
    g = G + wd W;  v' = a v + (1-a) g^2;  W' = W - lr g / (sqrt(v') + eps)."""
    g = G + weight_decay * W
    v1 = alpha * v + (1.0 - alpha) * g * g
    W1 = W - lr * g / (np.sqrt(v1) + eps)
    return W1, v1


def adagrad(W, G, v, lr, eps, weight_decay):
    """AdaGrad (Appendix N: the squared gradients are summed, never decayed), coupled
    decay, no learning-rate decay, fp64:
    g = G + wd W;  v' = v + g^2;  W' = W - lr g / (sqrt(v') + eps)."""
    g = G + weight_decay * W
    v1 = v + g * g
    W1 = W - lr * g / (np.sqrt(v1) + eps)
    return W1, v1


def sgd(W, G, lr, weight_decay):
    """SGD (Appendix N: vanilla gradient descent, no moment buffers), coupled
    decay, fp64: W' = W - lr (G + wd W)."""
    return W - lr * (G + weight_decay * W)


# --------------------------------------------------------------------------
# int8 block quantisation (section 2.3, Appendix B)
# --------------------------------------------------------------------------
def _blocks(x32: np.ndarray, block: int) -> np.ndarray:
    r, c = x32.shape
    if c % block:
        raise ValueError("the column count must be a multiple of the block size")
    return x32.reshape(r, c // block, block)


_TINY = np.float32(2.0 ** -64)
_BIG = np.float32(2.0 ** 64)


def _scaled_codes(xb: np.ndarray, a: np.ndarray, qmax: float):
    """fp32(x * fp32(qmax / a)) for every element of every block, and the
    scale fp32(a / qmax).  The reciprocal is the correctly rounded fp32
    quotient; for a block absmax below 2^-64 the quotient would overflow, so
    there x and a are first multiplied by 2^64 (exact in fp32), which yields
    the product as if the exponent range were unbounded and equals the plain
    formula wherever that one is finite.  a = 0 gives inv = s = 0."""
    q32 = np.float32(qmax)
    tiny = (a > 0) & (a < _TINY)
    with np.errstate(over="ignore"):       # the scaled copies are used only where the block is tiny
        a_eff = np.where(tiny, a * _BIG, a).astype(np.float32)
        x_eff = np.where(tiny[:, :, None], xb * _BIG, xb).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        s = np.where(a > 0, a / q32, np.float32(0)).astype(np.float32)
        inv = np.where(a > 0, q32 / a_eff, np.float32(0)).astype(np.float32)
    return (x_eff * inv[:, :, None]).astype(np.float32), s


def quantize_signed(x32: np.ndarray, block: int):
    """Signed block-absmax int8: a = max|x| over the block, s = fp32(a/127),
    code = clamp(rint(fp32(x * fp32(127/a))), -127, 127); a = 0 gives s = 0
    and all codes 0.  Returns (int8 codes, float32 scales)."""
    xb = _blocks(np.asarray(x32, dtype=np.float32), block)
    a = np.max(np.abs(xb), axis=2)
    y, s = _scaled_codes(xb, a, 127.0)
    q = np.clip(np.rint(y), -127, 127).astype(np.int8)
    return q.reshape(x32.shape), s


def quantize_unsigned(x32: np.ndarray, block: int):
    """Unsigned block-absmax uint8 with code 0 reserved for an exact zero:
    a = max x over the block, s = fp32(a/255), a positive x takes
    clamp(rint(fp32(x * fp32(255/a))), 1, 255), x == 0 takes code 0.
    Returns (uint8 codes, float32 scales)."""
    xb = _blocks(np.asarray(x32, dtype=np.float32), block)
    a = np.max(xb, axis=2)
    y, s = _scaled_codes(xb, a, 255.0)
    q = np.where(xb == 0, 0, np.clip(np.rint(y), 1, 255)).astype(np.uint8)
    return q.reshape(x32.shape), s


# OCP FP8 E4M3 ("fn"): sign, 4 exponent bits (bias 7), 3 mantissa bits; the
# largest finite value is 448 = 1.75 * 2^8, there are no infinities and
# S.1111.111 is NaN; exponent 0 holds the subnormals m * 2^-9.
E4M3_MAX = 448.0


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Values of E4M3 codes (uint8), exactly, in fp64."""
    c = np.asarray(codes).astype(np.int64)
    e, m = (c >> 3) & 15, c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


_E4M3_GRID = e4m3_to_f64(np.arange(0x7F))          # the 127 finite magnitudes, codes 0 .. 0x7E, ascending


def f32_to_e4m3_rne(y32: np.ndarray) -> np.ndarray:
    """The E4M3 code nearest to each fp32 value (ties to the even code, i.e.
    the even significand), saturating at +-448; the sign bit follows the
    input's (so -0.0 gives 0x80)."""
    y = np.asarray(y32, dtype=np.float32).astype(np.float64)
    ay = np.abs(y)
    hi = np.clip(np.searchsorted(_E4M3_GRID, ay, side="left"), 0, len(_E4M3_GRID) - 1)
    lo = np.clip(hi - 1, 0, len(_E4M3_GRID) - 1)
    dlo, dhi = ay - _E4M3_GRID[lo], _E4M3_GRID[hi] - ay
    pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(hi % 2 == 0, hi, lo)))
    pick = np.where(ay >= E4M3_MAX, 0x7E, pick)
    return (pick | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def f32_to_e4m3_sr(y32: np.ndarray, r16: np.ndarray) -> np.ndarray:
    """Stochastic rounding of fp32 values onto the E4M3 grid (the FP8 weight
    store with stochastic rounding; the pages give no rule, this is the
    reading): |y| is rounded to one of its two neighbouring E4M3 values,
    away from zero with probability equal to its fractional position between
    them (quantised to 2^-16), saturating at 448; the sign is kept (a result
    of zero keeps the input's sign).  With 16 random bits r:

    * |y| >= 2^-6 (the normal range, 3 fraction bits): r * 2^4 is added to
      the 20 fraction bits of |y|'s fp32 pattern that E4M3 does not keep and
      those bits are cleared (a carry moves |y| to the next grid value);
    * |y| < 2^-6 (the subnormal range, spacing 2^-9): z = floor(|y| 2^25)
      (exact), and the result is ((z + r) >> 16) * 2^-9.

    Returns uint8 codes."""
    y = np.ascontiguousarray(y32, dtype=np.float32)
    u = y.view(np.uint32)
    sign = u & np.uint32(0x80000000)
    au = u & np.uint32(0x7FFFFFFF)
    ay = au.view(np.float32)
    r = np.asarray(r16, dtype=np.uint32) & np.uint32(0xFFFF)
    with np.errstate(invalid="ignore", over="ignore"):
        normal = np.minimum(((au + (r << np.uint32(4))) & np.uint32(0xFFF00000)).view(np.float32), np.float32(448.0))
        z = np.floor(ay.astype(np.float64) * 2.0 ** 25)
        z = np.where(ay < np.float32(2.0 ** -6), z, 0.0).astype(np.uint64)
    sub = (((z + r.astype(np.uint64)) >> np.uint64(16)).astype(np.float64) * 2.0 ** -9).astype(np.float32)
    mag = np.where(ay >= np.float32(2.0 ** -6), normal, sub).astype(np.float32)
    val = (mag.view(np.uint32) | sign).view(np.float32)
    return f32_to_e4m3_rne(val)          # on the grid: the conversion is exact


def quantize_e4m3(x32: np.ndarray, block: int, positive: bool, r16: Optional[np.ndarray] = None):
    """E4M3 block quantisation (the int8 scheme with E4M3 codes; the paper's
    FP8 moment quantization, section 3.6, gives no format, this is the
    reading): a = max|x| over the block, s = fp32(a/448), code =
    f32_to_e4m3_rne(fp32(x * fp32(448/a))); with ``positive`` (the second
    moment) a positive x never takes code 0 but the smallest subnormal.
    a = 0 gives s = 0 and all codes +-0.  With ``r16`` (16 random bits per
    element, the shape of x) the code is f32_to_e4m3_sr of the same scaled
    value instead of the nearest one (the FP8 weight store with stochastic
    rounding).  Returns (uint8 codes, float32 scales)."""
    xb = _blocks(np.asarray(x32, dtype=np.float32), block)
    a = np.max(np.abs(xb), axis=2)
    y, s = _scaled_codes(xb, a, E4M3_MAX)
    if r16 is None:
        q = f32_to_e4m3_rne(y)
    else:
        q = f32_to_e4m3_sr(y, np.asarray(r16).reshape(xb.shape))
    if positive:
        q = np.where((xb > 0) & (q == 0), np.uint8(1), q).astype(np.uint8)
    return q.reshape(x32.shape), s


def dequantize(codes: np.ndarray, scales: np.ndarray, block: int) -> np.ndarray:
    """Stored value = fp32(code * scale)."""
    r, c = codes.shape
    cb = codes.astype(np.float32).reshape(r, c // block, block)
    return (cb * scales.astype(np.float32)[:, :, None]).astype(np.float32).reshape(r, c)


# --------------------------------------------------------------------------
# Decoding / encoding stored tensors
# --------------------------------------------------------------------------
def decode(st: Stored, rows=None, c0: int = 0, c1: Optional[int] = None) -> np.ndarray:
    """Exact fp64 values of the sub-block rows x [c0, c1) of a stored tensor."""
    rows = np.arange(st.data.shape[0]) if rows is None else np.asarray(rows)
    c1 = st.data.shape[1] if c1 is None else c1
    d = st.data[rows][:, c0:c1]
    if st.fmt == "f32":
        return d.astype(np.float64)
    if st.fmt == "bf16":
        return bf16_bits_to_f64(d)
    if st.fmt in ("s8", "u8", "e4m3"):
        if c0 % st.block or (c1 - c0) % st.block:
            raise ValueError("block-scaled sub-blocks must be block aligned")
        s = st.scale[rows][:, c0 // st.block:c1 // st.block]
        if st.fmt == "e4m3":
            r, c = d.shape
            vals = e4m3_to_f64(d).astype(np.float32).reshape(r, c // st.block, st.block)
            return (vals * s.astype(np.float32)[:, :, None]).astype(np.float32).reshape(r, c).astype(np.float64)
        return dequantize(d, s, st.block).astype(np.float64)
    raise ValueError(f"unknown format {st.fmt!r}")


def encode(x64: np.ndarray, fmt: str, *, round: str = "sr", key: int = 0,
           flat_index: Optional[np.ndarray] = None, block: int = 128, positive: bool = False,
           fp8_round: str = "rne") -> Stored:
    """Round fp64 results once into the storage format (Algorithm 1 Phase 3).

    fp32: round to nearest even.  bf16: the value is first rounded to fp32,
    then to bf16 by round-to-nearest-even or by stochastic rounding with the
    counter-based bits of ``key`` and ``flat_index``.  s8 / u8 / e4m3: the
    fp32 value is block-quantised (e4m3 with ``positive`` for the second
    moment); e4m3 codes are the nearest grid values, or, with
    ``fp8_round="sr"`` (the FP8 weight with stochastic rounding), drawn with
    the same counter-based bits as a bf16 store.
    """
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if fmt == "f32":
        return Stored("f32", x32)
    if fmt == "bf16":
        if round == "rne":
            return Stored("bf16", f32_to_bf16_rne(x32))
        return Stored("bf16", f32_to_bf16_sr(x32, sr_bits(key, flat_index)))
    if fmt == "s8":
        q, s = quantize_signed(x32, block)
        return Stored("s8", q, s, block)
    if fmt == "u8":
        q, s = quantize_unsigned(x32, block)
        return Stored("u8", q, s, block)
    if fmt == "e4m3":
        r16 = sr_bits(key, flat_index) if fp8_round == "sr" else None
        q, s = quantize_e4m3(x32, block, positive, r16)
        return Stored("e4m3", q, s, block)
    raise ValueError(f"unknown format {fmt!r}")


# --------------------------------------------------------------------------
# One step
# --------------------------------------------------------------------------
def apply_step(G: np.ndarray, W: Stored, m: Optional[Stored], v: Optional[Stored],
               hyper: Hyper, step: int, seed: int, rows=None, c0: int = 0,
               c1: Optional[int] = None, flat: Optional[np.ndarray] = None) -> dict:
    """Apply the optimizer to the sub-block rows x [c0, c1) given its fp64
    gradient G, and store the results.

    ``flat`` optionally gives the flat index p*K + q of every element of the
    sub-block in the logical [N, K] weight (used only to draw the SR bits);
    by default it is computed from ``rows``, the column range and the stored
    width, i.e. the arrays passed in are the whole layer.  Pass it when the
    arrays hold a gathered subset of the layer's rows.

    Returns a dict with the stored sub-blocks ``W``, ``m``, ``v`` (``None``
    where the optimizer keeps no such state) and ``pre``: the fp64 values
    before the final rounding.
    """
    if step < 1:
        raise ValueError("the step index t is 1-based")
    N, K = W.data.shape
    rows = np.arange(N) if rows is None else np.asarray(rows)
    c1 = K if c1 is None else c1
    cols = np.arange(c0, c1)
    h = hyper
    W0 = decode(W, rows, c0, c1)
    m0 = decode(m, rows, c0, c1) if m is not None else None
    v0 = decode(v, rows, c0, c1) if v is not None else None
    if h.opt == "adamw":
        W1, m1, v1 = adamw(W0, G, m0, v0, step, h.lr, h.beta1, h.beta2, h.eps, h.weight_decay)
    elif h.opt == "lion":
        W1, m1 = lion(W0, G, m0, h.lr, h.beta1, h.beta2, h.weight_decay)
        v1 = None
    elif h.opt == "sgdm":
        W1, m1 = sgdm(W0, G, m0, h.lr, h.beta1, h.weight_decay)
        v1 = None
    elif h.opt == "nadam":
        W1, m1, v1 = nadam(W0, G, m0, v0, step, h.lr, h.beta1, h.beta2, h.eps, h.weight_decay)
    elif h.opt == "radam":
        W1, m1, v1 = radam(W0, G, m0, v0, step, h.lr, h.beta1, h.beta2, h.eps, h.weight_decay)
    elif h.opt == "rmsprop":
        W1, v1 = rmsprop(W0, G, v0, h.lr, h.beta2, h.eps, h.weight_decay)
        m1 = None
    elif h.opt == "adagrad":
        W1, v1 = adagrad(W0, G, v0, h.lr, h.eps, h.weight_decay)
        m1 = None
    elif h.opt == "sgd":
        W1 = sgd(W0, G, h.lr, h.weight_decay)
        m1 = v1 = None
    else:
        raise ValueError(f"unknown optimizer {h.opt!r}")
    if flat is None:
        flat = rows.astype(np.uint64)[:, None] * np.uint64(K) + cols.astype(np.uint64)[None, :]

    def store(x, st, tid):
        if st is None:
            return None
        # an FP8 weight follows the rounding mode like a bf16 one; FP8
        # moments always take the nearest code (the int8 scheme's rule)
        return encode(x, st.fmt, round=h.round, key=sr_key(seed, step, tid),
                      flat_index=flat, block=st.block, positive=(tid == TENSOR_V),
                      fp8_round=h.round if tid == TENSOR_W else "rne")

    return {"W": store(W1, W, TENSOR_W), "m": store(m1, m, TENSOR_M),
            "v": store(v1, v, TENSOR_V), "pre": {"W": W1, "m": m1, "v": v1}}


def wgrad_step(X, dY, W: Stored, m: Optional[Stored], v: Optional[Stored], hyper: Hyper,
               step: int, seed: int, rows=None, c0: int = 0, c1: Optional[int] = None,
               order: str = "blas", flat: Optional[np.ndarray] = None) -> dict:
    """Materialise-then-step on the sub-block rows x [c0, c1): G from Eq. 3,
    then :func:`apply_step` (``flat`` as there).  With the defaults this is
    the whole layer.  The result dict also carries ``G`` (fp64)."""
    K = W.data.shape[1]
    c1 = K if c1 is None else c1
    G = weight_grad(X, dY, rows, np.arange(c0, c1), order)
    out = apply_step(G, W, m, v, hyper, step, seed, rows, c0, c1, flat)
    out["G"] = G
    return out


def _put(dst: Stored, src: Stored, rows, c0, c1):
    dst.data[rows[0]:rows[-1] + 1, c0:c1] = src.data
    if dst.scale is not None:
        dst.scale[rows[0]:rows[-1] + 1, c0 // dst.block:c1 // dst.block] = src.scale


def step_tiled(X, dY, W: Stored, m: Optional[Stored], v: Optional[Stored], hyper: Hyper,
               step: int, seed: int, tile_r: int, tile_c: int, tk: int,
               tile_order: Optional[Sequence[int]] = None, acc: str = "seq32") -> dict:
    """The per-tile fused schedule of section 2.2 / Algorithm 1, on the CPU.

    For every T_R x T_C tile (in ``tile_order``, default row-major) the tile
    gradient is accumulated over token chunks of ``tk`` rows (Eq. 5), tokens
    in ascending order in the accumulator precision ``acc`` ("seq32" fp32,
    "seq64" fp64); the optimizer is applied to that tile only and the tile is
    written back.  Returns new stored W, m, v for the whole layer.
    """
    N, K = W.data.shape
    BT = X.shape[0]
    nr, nc = -(-N // tile_r), -(-K // tile_c)
    order = list(range(nr * nc)) if tile_order is None else list(tile_order)
    if sorted(order) != list(range(nr * nc)):
        raise ValueError("tile_order must be a permutation of the tiles")
    outW = W.copy()
    outm = m.copy() if m is not None else None
    outv = v.copy() if v is not None else None
    for tile in order:
        i, j = divmod(tile, nc)
        rows = np.arange(i * tile_r, min(N, (i + 1) * tile_r))
        c0, c1 = j * tile_c, min(K, (j + 1) * tile_c)
        cols = np.arange(c0, c1)
        dYs, Xs = _as_f64(dY[:, rows]), _as_f64(X[:, cols])
        if acc == "seq32":
            Gt = np.zeros((len(rows), len(cols)), dtype=np.float32)
            dYs, Xs = dYs.astype(np.float32), Xs.astype(np.float32)
        elif acc == "seq64":
            Gt = np.zeros((len(rows), len(cols)), dtype=np.float64)
        else:
            raise ValueError(f"unknown accumulator {acc!r}")
        for k0 in range(0, BT, tk):                      # token chunks kappa
            for t in range(k0, min(BT, k0 + tk)):
                Gt = Gt + np.multiply.outer(dYs[t], Xs[t])
        res = apply_step(Gt.astype(np.float64), W, m, v, hyper, step, seed, rows, c0, c1)
        _put(outW, res["W"], rows, c0, c1)
        if outm is not None:
            _put(outm, res["m"], rows, c0, c1)
        if outv is not None:
            _put(outv, res["v"], rows, c0, c1)
    return {"W": outW, "m": outm, "v": outv}
