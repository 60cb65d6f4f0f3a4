"""Shared helpers of the GPU parity tests.

A ``Layer`` holds one linear layer's tensors on the GPU, drawn from the seeded
generators in ``synth``; ``snapshot`` copies what the oracle needs to the host
*before* the in-place GPU step; ``check_against_oracle`` runs the oracle on
the same inputs and compares every output element by element:

* fp32 outputs: ``|got - ref| <= 1e-5 S``, or ``got`` inside the hull of
  the optimizer evaluated over ``G +- E`` (E the forward error bound of an
  fp32 reduction in any order -- the only discrepancy Corollary 1(b) of the
  FORGE paper allows), widened by ``1e-5 S``; S is the larger of |ref| and
  the magnitude of the terms the output is summed from (the step evaluated
  on absolute values), so that an output which cancels -- a weight that the
  update drives through zero -- is judged against its operands' scale;
* bf16 outputs: within one bf16 ULP (+ 1e-5 S) of that hull, and bit-identical to the
  oracle's stored pattern for at least a fraction 1 - (1e-3 + 2 sqrt(BT) 2^-16)
  of the elements (the SR bits come from the same counter-based hash on both
  sides, so a stored pattern differs only where the fp32 gradient's rounding
  -- relative size about sqrt(BT) 2^-24 for a BT-term fp32 sum -- moves the
  value across the rounding decision, which happens with probability of that
  size in units of a bf16 ULP, 2^-8: about sqrt(BT) 2^-16);
* int8 and E4M3 codes: identical to the oracle's wherever the code is
  determined -- every value the fp32 pre-quantisation input can take inside
  that hull (widened as above), scaled by every reciprocal the block absmax
  can take, rounds to the same code -- and elsewhere within one code (one
  step of the grid), at least 99% identical overall; scales within 1e-5
  relative or inside the hull of the block absmax.  (The quantiser alone,
  on identical fp32 inputs, is checked bit for bit through
  forge_debug_quant.)

Counts reported per output: ``clause2`` (fp32 elements that pass only
through the hull), ``s_only`` (fp32 elements that pass only because the
tolerance is taken relative to the operand scale S rather than to |ref|),
``determined`` (the fraction of 8-bit codes that had to be exact).
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

import backward_weight_gradient_amd as F
import oracle as O
import synth

FMT_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "s8": torch.int8, "u8": torch.uint8,
             "e4m3": torch.float8_e4m3fn}


def _codes(t):
    """FP8 tensors as their uint8 codes (row gathers are done on those)."""
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


@dataclass
class Layer:
    N: int
    K: int
    BT: int
    spec: synth.LayerSpec
    X: torch.Tensor
    dY: torch.Tensor
    W: torch.Tensor
    m: Optional[torch.Tensor]
    v: Optional[torch.Tensor]
    ms: Optional[torch.Tensor] = None
    vs: Optional[torch.Tensor] = None
    wsc: Optional[torch.Tensor] = None      # block scales of an E4M3 weight

    def _state(self, t, scale):
        if t is None:
            return None
        if scale is None:
            return F.state(t)
        if self.K % self.spec.block:
            # a shape the library must reject: built without the binding's own
            # checks, so that the C ABI's validation is what is exercised
            return F.forge_state(F.mat(t), scale.data_ptr(), self.spec.block)
        return F.state(t, scale, self.spec.block)

    def forge_m(self):
        return self._state(self.m, self.ms)

    def forge_w(self):
        """The weight as the fused step takes it: a tensor, or for an E4M3
        weight a forge_state with its block scales."""
        return self._state(self.W, self.wsc) if self.wsc is not None else self.W

    def forge_v(self):
        return self._state(self.v, self.vs)

    def clone(self) -> "Layer":
        c = lambda t: None if t is None else t.clone()
        return Layer(self.N, self.K, self.BT, self.spec, self.X, self.dY, c(self.W), c(self.m), c(self.v),
                     c(self.ms), c(self.vs), c(self.wsc))


def make_layer(cfg: int, N: int, K: int, BT: int, step: int, spec: synth.LayerSpec, *, device="cuda",
               gen_device="cpu", x_std=1.0, dy_std=1e-3, outlier_p=0.0, v_zero=False, w_std=0.02,
               v_init="quantized", extra=0) -> Layer:
    """Seeded layer on `device`.  Small layers are drawn on the CPU and moved;
    large ones directly on the GPU (gen_device="cuda").  With a block-scaled
    v (U8 or E4M3) and v_init="quantized" (the default: the int8 workload's
    init), v starts as the oracle's quantisation of |N(0, 1e-6)| (the same
    codes and scales go to both sides); v_init="random" keeps synth's
    uniform stand-in codes."""
    X, dY = synth.activations(cfg, BT, N, K, step, in_dtype=spec.in_dtype, x_std=x_std, dy_std=dy_std,
                              outlier_p=outlier_p, device=gen_device, extra=extra)
    st = synth.state(cfg, N, K, spec, w_std=w_std, v_zero=v_zero, device=gen_device, extra=extra)
    # (a K that is not a multiple of the block keeps the stand-in codes: such a
    # state is only used to check that the call is rejected)
    if spec.v_fmt in ("u8", "e4m3") and v_init == "quantized" and not v_zero and K % spec.block == 0:
        v32 = synth.normal((N, K), 1e-6, "cpu", cfg, 0, synth.T_V, extra).abs().numpy()
        if spec.v_fmt == "u8":
            q, s = O.quantize_unsigned(v32, spec.block)
            st["v"] = torch.from_numpy(q)
        else:
            q, s = O.quantize_e4m3(v32, spec.block, True)
            st["v"] = torch.from_numpy(q).view(torch.float8_e4m3fn)
        st["v_scale"] = torch.from_numpy(s)
        del v32
    w_scale = None
    if spec.w_fmt == "e4m3":
        # an E4M3 weight starts as the oracle's nearest-code quantisation of
        # W ~ N(0, w_std^2) (the same codes and scales go to both sides)
        w32 = st["W"].float().cpu().numpy()
        if K % spec.block == 0:
            q, sc = O.quantize_e4m3(w32, spec.block, False)
        else:   # only used to check that the call is rejected
            q, sc = np.zeros(w32.shape, np.uint8), np.zeros((N, max(1, K // spec.block)), np.float32)
        st["W"], w_scale = torch.from_numpy(q).view(torch.float8_e4m3fn), torch.from_numpy(sc)
    mv = lambda t: None if t is None else t.to(device)
    return Layer(N, K, BT, spec, mv(X), mv(dY), mv(st["W"]), mv(st["m"]), mv(st["v"]), mv(st["m_scale"]),
                 mv(st["v_scale"]), mv(w_scale))


def run_fused(L: Layer, h, step: int, seed: int):
    if L.wsc is not None:
        F.forge_wgrad_step_fp8w(L.X, L.dY, L.forge_w(), L.forge_m(), L.forge_v(), h, step, seed)
    else:
        F.forge_wgrad_step(L.X, L.dY, L.W, L.forge_m(), L.forge_v(), h, step, seed)


def run_unfused(L: Layer, h, step: int, seed: int, dw_dtype=torch.float32):
    dW = torch.empty((L.N, L.K), device=L.W.device, dtype=dw_dtype)
    F.forge_wgrad_unfused(L.X, L.dY, L.W, L.forge_m(), L.forge_v(), h, step, seed, dW)
    return dW


def oracle_hyper(h) -> O.Hyper:
    inv_opt = {v: k for k, v in F.OPTIMIZERS.items()}
    inv_round = {v: k for k, v in F.ROUNDING.items()}
    return O.Hyper(opt=inv_opt[h.opt], lr=h.lr, beta1=h.beta1, beta2=h.beta2, eps=h.eps,
                   weight_decay=h.weight_decay, round=inv_round[h.round])


# ---------------------------------------------------------------------------
# Host snapshots
# ---------------------------------------------------------------------------
@dataclass
class Snap:
    """Host copies of the rows `rows` (global indices) of a layer, and of the
    columns of dY those rows need, taken before a step."""
    rows: np.ndarray
    X: np.ndarray
    dY: np.ndarray
    W: O.Stored
    m: Optional[O.Stored]
    v: Optional[O.Stored]
    extra_terms: int = 0      # fp32 additions of partial gradients (micro-batch accumulation)


def _stored(t, fmt, scale, block, rows):
    if t is None:
        return None
    idx = torch.as_tensor(rows, device=t.device, dtype=torch.long)
    data = synth.host(_codes(t).index_select(0, idx))
    sc = None if scale is None else scale.index_select(0, idx).cpu().numpy()
    return O.Stored(fmt, data, sc, block)


def snapshot(L: Layer, rows=None) -> Snap:
    rows = np.arange(L.N) if rows is None else np.asarray(rows)
    idx = torch.as_tensor(rows, device=L.dY.device, dtype=torch.long)
    s = L.spec
    return Snap(rows=rows, X=synth.host(L.X), dY=synth.host(L.dY.index_select(1, idx)),
                W=_stored(L.W, s.w_fmt, L.wsc, s.block, rows),
                m=_stored(L.m, s.m_fmt, L.ms, s.block, rows),
                v=_stored(L.v, s.v_fmt, L.vs, s.block, rows))


# ---------------------------------------------------------------------------
# Comparison
# ---------------------------------------------------------------------------
def _bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.abs(x)
    ax = np.where(ax < 2.0 ** -126, 2.0 ** -126, ax)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


@dataclass
class Report:
    checked: int = 0
    clause2: dict = field(default_factory=dict)     # fp32 elements passing only via the hull
    s_only: dict = field(default_factory=dict)      # fp32 elements passing only via the operand scale S
    exact_frac: dict = field(default_factory=dict)  # bf16 / int8 bit-exact fractions
    determined: dict = field(default_factory=dict)  # 8-bit codes fixed by the inputs (must be exact)
    failures: list = field(default_factory=list)

    def summary(self) -> str:
        n2 = sum(self.clause2.values())
        ns = sum(self.s_only.values())
        det = ", ".join(f"{k} {v:.5f}" for k, v in self.determined.items())
        return (f"{self.checked} elements; fp32 hull-only {n2}, S-only {ns}"
                + (f"; 8-bit codes determined: {det}" if det else ""))

    def ok(self):
        return not self.failures


def _hull(snap: Snap, hyp: O.Hyper, step: int, seed: int, c0: int, c1: int, K: int):
    rows_local = np.arange(len(snap.rows))
    cols = np.arange(c0, c1)
    G = O.weight_grad(snap.X, snap.dY, rows_local, cols)
    E = O.grad_error_bound(snap.X, snap.dY, rows_local, cols, snap.extra_terms)
    flat = snap.rows.astype(np.uint64)[:, None] * np.uint64(K) + cols.astype(np.uint64)[None, :]
    ref = O.apply_step(G, snap.W, snap.m, snap.v, hyp, step, seed, rows_local, c0, c1, flat)
    lo = {k: v.copy() for k, v in ref["pre"].items() if v is not None}
    hi = {k: v.copy() for k, v in ref["pre"].items() if v is not None}
    probes = [G - E, G - 0.5 * E, G + 0.5 * E, G + E, np.where(np.abs(G) <= E, 0.0, G)]
    for Gp in probes:
        r = O.apply_step(Gp, snap.W, snap.m, snap.v, hyp, step, seed, rows_local, c0, c1, flat)
        for k in lo:
            lo[k] = np.minimum(lo[k], r["pre"][k])
            hi[k] = np.maximum(hi[k], r["pre"][k])
    # Scale of the terms each output is summed from: the same step evaluated
    # on absolute values with the update added instead of subtracted (the
    # usual device of running a computation on |inputs| to bound its
    # rounding error).  fp32 evaluation error is a few ulps of this scale.
    absW, absm, absv = (_abs_stored(x) for x in (snap.W, snap.m, snap.v))
    ahyp = O.Hyper(opt=hyp.opt, lr=-hyp.lr, beta1=hyp.beta1, beta2=hyp.beta2, eps=hyp.eps,
                   weight_decay=hyp.weight_decay, round=hyp.round)
    ra = O.apply_step(np.abs(G) + E, absW, absm, absv, ahyp, step, seed, rows_local, c0, c1, flat)
    scale = {k: np.abs(ra["pre"][k]) for k in lo}
    return ref, lo, hi, scale


def _abs_stored(st):
    if st is None:
        return None
    if st.fmt == "f32":
        return O.Stored("f32", np.abs(st.data))
    if st.fmt == "bf16":
        return O.Stored("bf16", st.data & np.uint16(0x7FFF))
    if st.fmt == "s8":
        return O.Stored("s8", np.abs(st.data.astype(np.int16)).astype(np.int8), st.scale, st.block)
    if st.fmt == "e4m3":
        return O.Stored("e4m3", st.data & np.uint8(0x7F), st.scale, st.block)
    return st


def check_against_oracle(snap: Snap, L: Layer, h, step: int, seed: int, col_ranges=None,
                         rep: Optional[Report] = None, exact_min=None, code_exact_min=0.99) -> Report:
    """Compare the layer's current (post-step) tensors on rows snap.rows and
    the given column ranges with the oracle run on the snapshot."""
    rep = rep or Report()
    if exact_min is None:
        exact_min = 1.0 - (1e-3 + 2.0 * np.sqrt(max(1, snap.X.shape[0])) * 2.0 ** -16)
    hyp = oracle_hyper(h)
    K = L.K
    col_ranges = col_ranges or [(0, K)]
    idx = torch.as_tensor(snap.rows, device=L.W.device, dtype=torch.long)
    s = L.spec
    for c0, c1 in col_ranges:
        if c1 <= c0:
            continue
        ref, lo, hi, tscale = _hull(snap, hyp, step, seed, c0, c1, K)
        got = {"W": (L.W, s.w_fmt, L.wsc), "m": (L.m, s.m_fmt, L.ms), "v": (L.v, s.v_fmt, L.vs)}
        for name, (t, fmt, scale) in got.items():
            if t is None or fmt is None:
                continue
            g = synth.host(_codes(t).index_select(0, idx)[:, c0:c1])
            r_st = ref[name]
            r_pre = ref["pre"][name]
            where = f"{name}[{fmt}] cols {c0}:{c1}"
            rep.checked += g.size
            if fmt == "f32":
                g64 = g.astype(np.float64)
                tol = 1e-5 * np.maximum(np.abs(r_pre), tscale[name])
                c1ok = np.abs(g64 - r_pre) <= tol
                c2ok = (g64 >= lo[name] - tol) & (g64 <= hi[name] + tol)
                bad = ~(c1ok | c2ok)
                rep.clause2[where] = int(np.sum(~c1ok & c2ok))
                # passes that rely on S: outside 1e-5 |ref| of both the value and the hull
                tol_r = 1e-5 * np.abs(r_pre)
                strict = (np.abs(g64 - r_pre) <= tol_r) | ((g64 >= lo[name] - tol_r) & (g64 <= hi[name] + tol_r))
                rep.s_only[where] = int(np.sum(~strict & ~bad))
                if bad.any():
                    i = np.argwhere(bad)[0]
                    rep.failures.append(f"{where}: {int(bad.sum())} fp32 elements off, e.g. {tuple(i)} "
                                        f"got {g64[tuple(i)]!r} ref {r_pre[tuple(i)]!r} "
                                        f"hull [{lo[name][tuple(i)]!r}, {hi[name][tuple(i)]!r}]")
            elif fmt == "bf16":
                gv = O.bf16_bits_to_f64(g)
                ulp = np.maximum(_bf16_ulp(lo[name]), _bf16_ulp(hi[name])) + 1e-5 * tscale[name]
                bad = (gv < lo[name] - ulp) | (gv > hi[name] + ulp)
                exact = float(np.mean(g == r_st.data)) if g.size else 1.0
                rep.exact_frac[where] = exact
                if bad.any():
                    i = np.argwhere(bad)[0]
                    rep.failures.append(f"{where}: {int(bad.sum())} bf16 elements beyond 1 ulp, e.g. {tuple(i)} "
                                        f"got {gv[tuple(i)]!r} hull [{lo[name][tuple(i)]!r}, {hi[name][tuple(i)]!r}]")
                if exact < exact_min:
                    rep.failures.append(f"{where}: bf16 bit-exact fraction {exact:.6f} < {exact_min}")
            else:  # 8-bit codes + scales (int8, or E4M3 compared as sign-magnitude steps)
                gi = g.astype(np.int64)
                ri = r_st.data.astype(np.int64)
                if fmt == "e4m3":
                    gi = np.where(gi & 0x80, -(gi & 0x7F), gi)
                    ri = np.where(ri & 0x80, -(ri & 0x7F), ri)
                d = np.abs(gi - ri)
                exact = float(np.mean(d == 0)) if d.size else 1.0
                rep.exact_frac[where] = exact
                tol8 = 1e-5 * np.maximum(np.abs(r_pre), tscale[name])
                r16 = None
                if name == "W" and hyp.round == "sr":   # the weight's own SR bits decide its code
                    flat = snap.rows.astype(np.uint64)[:, None] * np.uint64(K) + \
                        np.arange(c0, c1, dtype=np.uint64)[None, :]
                    r16 = O.sr_bits(O.sr_key(seed, step, O.TENSOR_W), flat)
                det = _determined_codes(fmt, name == "v", lo[name] - tol8, hi[name] + tol8, s.block, r16)
                rep.determined[where] = float(np.mean(det)) if det.size else 1.0
                if (det & (d != 0)).any():
                    i = np.argwhere(det & (d != 0))[0]
                    rep.failures.append(f"{where}: {int((det & (d != 0)).sum())} determined codes differ, e.g. "
                                        f"{tuple(i)} got {gi[tuple(i)]} ref {ri[tuple(i)]}")
                if (d > 1).any():
                    i = np.argwhere(d > 1)[0]
                    rep.failures.append(f"{where}: {int((d > 1).sum())} codes off by > 1, e.g. {tuple(i)} "
                                        f"got {gi[tuple(i)]} ref {ri[tuple(i)]}")
                if exact < code_exact_min:
                    rep.failures.append(f"{where}: code exact fraction {exact:.6f} < {code_exact_min}")
                b = s.block
                gs = scale.index_select(0, idx)[:, c0 // b:c1 // b].cpu().numpy().astype(np.float64)
                rs = r_st.scale.astype(np.float64)
                qmax = {"s8": 127.0, "u8": 255.0, "e4m3": O.E4M3_MAX}[fmt]
                alo = np.where((lo[name] <= 0) & (hi[name] >= 0), 0.0, np.minimum(np.abs(lo[name]), np.abs(hi[name])))
                ahi = np.maximum(np.abs(lo[name]), np.abs(hi[name]))
                R = alo.shape[0]
                slo = alo.reshape(R, -1, b).max(axis=2) / qmax
                shi = ahi.reshape(R, -1, b).max(axis=2) / qmax
                tol = 1e-5 * rs
                sbad = ~((np.abs(gs - rs) <= tol) | ((gs >= slo - tol) & (gs <= shi + tol)))
                if sbad.any():
                    i = np.argwhere(sbad)[0]
                    rep.failures.append(f"{where}: {int(sbad.sum())} scales off, e.g. {tuple(i)} "
                                        f"got {gs[tuple(i)]!r} ref {rs[tuple(i)]!r}")
    return rep


def _determined_codes(fmt: str, second: bool, xlo: np.ndarray, xhi: np.ndarray, block: int,
                      r16: Optional[np.ndarray] = None) -> np.ndarray:
    """True where the 8-bit code is fixed by the inputs: every fp32
    pre-quantisation value in [xlo, xhi], multiplied by every reciprocal
    QMAX / a that the block absmax a can take (a over the same intervals),
    rounds to one code (the product's own fp32 rounding and the reciprocal's
    are covered by a relative widening of 2^-21).  Where this holds, the
    kernel's code and the oracle's must be identical: the quantiser is the
    same definition on both sides.  With ``r16`` (an E4M3 weight stored with
    stochastic rounding) the code is the SR code with those bits, which is
    monotone in y too."""
    qmax = {"s8": 127.0, "u8": 255.0, "e4m3": O.E4M3_MAX}[fmt]
    R, C = xlo.shape
    alo = np.where((xlo <= 0) & (xhi >= 0), 0.0, np.minimum(np.abs(xlo), np.abs(xhi)))
    ahi = np.maximum(np.abs(xlo), np.abs(xhi))
    blo = np.repeat(alo.reshape(R, -1, block).max(axis=2), block, axis=1)
    bhi = np.repeat(ahi.reshape(R, -1, block).max(axis=2), block, axis=1)
    ok = blo > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        c = [xlo * qmax / np.where(ok, blo, 1.0), xlo * qmax / np.where(ok, bhi, 1.0),
             xhi * qmax / np.where(ok, blo, 1.0), xhi * qmax / np.where(ok, bhi, 1.0)]
    ylo, yhi = np.minimum.reduce(c), np.maximum.reduce(c)
    w = 2.0 ** -21 * np.maximum(np.abs(ylo), np.abs(yhi))
    ylo, yhi = ylo - w, yhi + w

    def code(y):
        if fmt == "s8":
            return np.clip(np.rint(y), -127, 127)
        if fmt == "u8":
            return np.clip(np.rint(y), 1, 255)
        yy = np.maximum(y, 2.0 ** -9) if second else y
        yy = np.clip(yy, -3e38, 3e38).astype(np.float32)
        # stochastic rounding with fixed bits is monotone in y, like the nearest code
        cc = (O.f32_to_e4m3_rne(yy) if r16 is None else O.f32_to_e4m3_sr(yy, r16)).astype(np.int64)
        return np.where(cc & 0x80, -(cc & 0x7F), cc)

    det = ok & (code(ylo) == code(yhi))
    if fmt == "u8" or (fmt == "e4m3" and second):
        det &= xlo > 0            # an exact zero (or a value that may be zero) takes its own rule
    elif fmt == "e4m3":
        det &= (xlo > 0) | (xhi < 0)   # the sign of a zero code follows the input's
    return det


def assert_ok(rep: Report, label: str = ""):
    print(f"  {label}: {rep.summary()}", flush=True)
    if not rep.ok():
        raise AssertionError(f"{label}: " + "\n".join(rep.failures[:10]))


def assert_rejected(L: Layer, call, extra=(), code=None):
    """`call()` (a binding call with check=False) must return `code`
    (FORGE_E_SHAPE by default) and leave every tensor of the layer, and the
    tensors in `extra`, unchanged: validation happens before anything is
    enqueued."""
    code = F.FORGE_E_SHAPE if code is None else code
    ts = [t for t in (L.W, L.m, L.v, L.ms, L.vs, L.wsc, *extra) if t is not None]
    before = [_codes(t).clone() for t in ts]
    torch.cuda.synchronize()
    rc = call()
    torch.cuda.synchronize()
    assert rc == code, f"expected {F.forge_status_str(code)}, got {F.forge_status_str(rc)}"
    for a, b in zip(ts, before):
        assert torch.equal(_codes(a), b), "a rejected call modified its arguments"


def sample_rows(N: int, n: int, seed: int) -> np.ndarray:
    """First, last and tile-boundary rows plus random ones, sorted."""
    rng = np.random.default_rng(seed)
    base = {0, N - 1, min(N - 1, 127), min(N - 1, 128)}
    extra = rng.choice(N, size=min(N, n), replace=False)
    return np.array(sorted(base | set(int(x) for x in extra)))
