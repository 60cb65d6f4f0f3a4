"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: values
worked by hand (tests/golden), closed forms, library routines that the
definition reduces to in special cases (torch.optim in float64, torch's bf16
cast), exact integer arithmetic, published hash test vectors, and the
statistical statements of the FORGE paper's Appendices B and C.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hyper(opt, d):
    return O.Hyper(opt=opt, **d)


# ---------------------------------------------------------------------------
# Element-wise optimizers
# ---------------------------------------------------------------------------
def _run_scalar(case):
    h = case["hyper"]
    W, m, v = case["W0"], 0.0, 0.0
    out = {"W": [], "m": [], "v": []}
    for t, G in enumerate(case["G"], 1):
        if case["opt"] == "adamw":
            W, m, v = O.adamw(W, G, m, v, t, h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"])
        elif case["opt"] == "lion":
            W, m = O.lion(W, G, m, h["lr"], h["beta1"], h["beta2"], h["weight_decay"])
        else:
            W, m = O.sgdm(W, G, m, h["lr"], h["beta1"], h["weight_decay"])
        out["W"].append(W)
        out["m"].append(m)
        out["v"].append(v)
    return out


def test_hand_worked_trajectories():
    """Algorithm 1 Phase 2 (AdamW), Lion and SGD-m against values worked by hand."""
    with open(os.path.join(GOLDEN, "hand_worked_steps.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        got = _run_scalar(case)
        for key in ("W", "m", "v"):
            if key not in case:
                continue
            for t, (a, r) in enumerate(zip(got[key], case[key]), 1):
                assert a == pytest.approx(r, rel=1e-12, abs=1e-18), (case["opt"], key, t, a, r)


def test_adamw_first_step_closed_form():
    """t = 1 from m = v = 0: m_hat = G and v_hat = G^2, so
    W1 = (1 - lr wd) W0 - lr G/(|G| + eps)."""
    rng = np.random.default_rng(0)
    W0, G = rng.normal(0, 0.02, 1000), rng.normal(0, 1e-2, 1000)
    lr, b1, b2, eps, wd = 1e-3, 0.9, 0.999, 1e-8, 0.01
    W1, m1, v1 = O.adamw(W0, G, np.zeros(1000), np.zeros(1000), 1, lr, b1, b2, eps, wd)
    np.testing.assert_allclose(W1, (1 - lr * wd) * W0 - lr * G / (np.abs(G) + eps), rtol=1e-13)
    np.testing.assert_allclose(m1 / (1 - b1), G, rtol=1e-13)
    np.testing.assert_allclose(v1 / (1 - b2), G * G, rtol=1e-12)


def test_adamw_constant_gradient_bias_correction():
    """A constant gradient gives m_hat = G and v_hat = G^2 at every step: the
    bias correction uses the 1-based t directly."""
    G = np.array([0.3, -2e-3, 5e-6])
    b1, b2 = 0.9, 0.999
    m = v = np.zeros(3)
    W = np.full(3, 0.1)
    for t in range(1, 30):
        W, m, v = O.adamw(W, G, m, v, t, 1e-3, b1, b2, 1e-8, 0.0)
        np.testing.assert_allclose(m / (1 - b1 ** t), G, rtol=1e-12)
        np.testing.assert_allclose(v / (1 - b2 ** t), G * G, rtol=1e-11)


def test_adamw_zero_gradient_is_pure_decay():
    W0 = np.array([0.02, -0.5, 3.0])
    W, m, v = W0, np.zeros(3), np.zeros(3)
    for t in range(1, 6):
        W, m, v = O.adamw(W, np.zeros(3), m, v, t, 1e-3, 0.9, 0.999, 1e-8, 0.01)
        np.testing.assert_allclose(W, (1 - 1e-5) ** t * W0, rtol=1e-14)


def test_adamw_matches_torch_adamw_float64():
    """torch.optim.AdamW (decoupled decay, bias correction, eps outside the
    root) is the same map; in float64 the two agree to rounding."""
    rng = np.random.default_rng(1)
    n = 4096
    W = rng.normal(0, 0.02, n)
    m, v = np.zeros(n), np.zeros(n)
    p = torch.tensor(W.copy(), dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([p], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    for t in range(1, 8):
        G = rng.normal(0, 1e-2, n)
        W, m, v = O.adamw(W, G, m, v, t, 1e-3, 0.9, 0.999, 1e-8, 0.01)
        p.grad = torch.tensor(G, dtype=torch.float64)
        opt.step()
    st = opt.state[p]
    np.testing.assert_allclose(W, p.detach().numpy(), rtol=1e-13, atol=1e-18)
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-20)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-24)


def test_sgdm_matches_torch_sgd_float64():
    rng = np.random.default_rng(2)
    n = 2048
    W = rng.normal(0, 0.02, n)
    b = np.zeros(n)
    p = torch.tensor(W.copy(), dtype=torch.float64, requires_grad=True)
    opt = torch.optim.SGD([p], lr=1e-3, momentum=0.9, weight_decay=0.01)
    for _ in range(5):
        G = rng.normal(0, 1e-2, n)
        W, b = O.sgdm(W, G, b, 1e-3, 0.9, 0.01)
        p.grad = torch.tensor(G, dtype=torch.float64)
        opt.step()
    np.testing.assert_allclose(W, p.detach().numpy(), rtol=1e-14)
    np.testing.assert_allclose(b, opt.state[p]["momentum_buffer"].numpy(), rtol=1e-12)


def test_lion_sign_and_zero():
    """Lion moves every coordinate by exactly lr (plus decay) in the direction
    of -sign(c); where c == 0 only the decay acts.  (b1 = 0.5 keeps c exact.)"""
    W0 = np.array([0.5, 0.5, 0.5, -0.25])
    m0 = np.array([0.0, 1.0, -1.0, 0.0])
    G = np.array([0.0, -1.0, 3.0, -3.0])       # c = 0, 0, 1, -1.5
    W1, m1 = O.lion(W0, G, m0, 1e-4, 0.5, 0.99, 0.01)
    dec = (1 - 1e-6) * W0
    np.testing.assert_allclose(W1, dec - 1e-4 * np.array([0, 0, 1, -1]), rtol=1e-15)
    np.testing.assert_allclose(m1, 0.99 * m0 + 0.01 * G, rtol=1e-15)


# ---------------------------------------------------------------------------
# Gradient (Eq. 3)
# ---------------------------------------------------------------------------
def _int_inputs(BT, N, K, rng, in_dtype):
    """Integer-valued inputs exact in bf16: X in {-2..2}, dY in {-2..2} * 2^-10."""
    Xi = rng.integers(-2, 3, (BT, K))
    dYi = rng.integers(-2, 3, (BT, N))
    Xt = torch.tensor(Xi, dtype=torch.float32)
    dYt = torch.tensor(dYi, dtype=torch.float32) * 2.0 ** -10
    if in_dtype == "bf16":
        X = Xt.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        dY = dYt.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        X, dY = Xt.numpy(), dYt.numpy()
    return Xi, dYi, X, dY


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("BT,N,K", [(1, 1, 1), (2, 3, 9), (3, 9, 3), (7, 5, 130), (64, 130, 7)])
def test_weight_grad_brute_force(BT, N, K, in_dtype):
    """G[p, q] = sum_t dY[t, p] X[t, q] against an exact integer triple loop.
    Non-square shapes make a transposed operand fail."""
    rng = np.random.default_rng(BT * 1000 + N * 10 + K)
    Xi, dYi, X, dY = _int_inputs(BT, N, K, rng, in_dtype)
    exact = np.zeros((N, K), dtype=object)
    for p in range(N):
        for q in range(K):
            s = 0
            for t in range(BT):
                s += int(dYi[t, p]) * int(Xi[t, q])
            exact[p, q] = Fraction(s, 1024)
    ref = np.array([[float(x) for x in row] for row in exact])
    for order in ("blas", "seq64", "seq32"):
        G = O.weight_grad(X, dY, order=order)
        assert G.shape == (N, K)
        np.testing.assert_array_equal(G, ref)


def test_weight_grad_sub_block_indexing():
    """A sub-block (rows, cols) of G equals the same entries of the full G,
    computed independently with math.fsum."""
    rng = np.random.default_rng(5)
    X = rng.normal(size=(33, 21)).astype(np.float32)
    dY = rng.normal(size=(33, 17)).astype(np.float32)
    rows, cols = np.array([16, 3, 0]), np.array([20, 1])
    G = O.weight_grad(X, dY, rows, cols)
    for a, p in enumerate(rows):
        for b, q in enumerate(cols):
            ref = math.fsum(float(dY[t, p]) * float(X[t, q]) for t in range(33))
            assert G[a, b] == pytest.approx(ref, rel=1e-14, abs=1e-14)


def test_grad_error_bound_covers_fp32_orders():
    """The fp32 sequential accumulation lies within the stated bound of the
    fp64 value (Corollary 1(b): only the reduction order differs)."""
    rng = np.random.default_rng(6)
    X = rng.normal(size=(512, 40)).astype(np.float32)
    dY = (rng.normal(size=(512, 30)) * 1e-3).astype(np.float32)
    G64 = O.weight_grad(X, dY)
    G32 = O.weight_grad(X, dY, order="seq32")
    E = O.grad_error_bound(X, dY)
    assert np.all(np.abs(G32 - G64) <= E)
    # ... and the bound is far tighter than dropping a single token would be
    G_drop = O.weight_grad(X[1:], dY[1:])
    assert np.mean(np.abs(G_drop - G64) > E) > 0.95


# ---------------------------------------------------------------------------
# Counter-based random bits
# ---------------------------------------------------------------------------
def test_fmix32_published_vectors():
    """MurmurHash3_x86_32 of the empty input is fmix32(seed); its published test
    vectors for seeds 0, 1 and 0xFFFFFFFF are 0, 0x514E28B7, 0x81F16F39."""
    assert O.fmix32(0) == 0
    assert O.fmix32(1) == 0x514E28B7
    assert O.fmix32(0xFFFFFFFF) == 0x81F16F39
    arr = O.fmix32(np.array([0, 1, 0xFFFFFFFF], dtype=np.uint32))
    assert list(map(int, arr)) == [0, 0x514E28B7, 0x81F16F39]


def test_sr_bits_uniform_and_independent():
    n = 1 << 20
    idx = np.arange(n, dtype=np.uint64)
    r = O.sr_bits(O.sr_key(1337, 10, 0), idx).astype(np.int64)
    assert r.min() >= 0 and r.max() < 65536
    # mean of U{0..65535} is 32767.5, sd 18918.6 -> 5 sigma of the mean ~ 92
    assert abs(r.mean() - 32767.5) < 5 * 18918.6 / math.sqrt(n)
    for bit in range(16):
        frac = ((r >> bit) & 1).mean()
        assert abs(frac - 0.5) < 5 * 0.5 / math.sqrt(n)
    hist = np.bincount(r >> 8, minlength=256)
    chi2 = ((hist - n / 256) ** 2 / (n / 256)).sum()
    assert chi2 < 400  # 255 dof: mean 255, sd 22.6
    # the two halves of a pair's hash (even and odd elements), and
    # neighbouring pairs, are uncorrelated
    for a, b in ((r[0::2], r[1::2]), (r[1::2][:-1], r[2::2])):
        assert abs(np.corrcoef(a, b)[0, 1]) < 5 / math.sqrt(n / 2)
    # different tensor / step / seed -> uncorrelated streams
    for key in (O.sr_key(1337, 10, 1), O.sr_key(1337, 11, 0), O.sr_key(1338, 10, 0)):
        r2 = O.sr_bits(key, idx).astype(np.int64)
        c = np.corrcoef(r, r2)[0, 1]
        assert abs(c) < 5 / math.sqrt(n)
    # keys are all distinct across the three tensors
    assert len({O.sr_key(7, 3, t) for t in range(3)}) == 3


def test_sr_key_and_bits_hand_worked():
    """The key derivation and the per-element bits against values worked by
    hand from the written specification (tests/golden/sr_key_worked.json:
    every fmix32 call with its intermediate words).  A swapped hi/lo fold, an
    addition in place of an xor, a wrong tensor offset or a different index
    multiplier changes these words."""
    with open(os.path.join(GOLDEN, "sr_key_worked.json")) as f:
        doc = json.load(f)
    n_calls = 0
    for case in doc["cases"]:
        seed, step, tid = int(case["seed"], 16), int(case["step"], 16), case["tensor_id"]
        for w in case["key_working"]:
            assert O.fmix32(int(w["in"], 16)) == int(w["out"], 16)
            n_calls += 1
        assert O.sr_key(seed, step, tid) == int(case["key"], 16), case
        key = int(case["key"], 16)
        for b in case["sr_bits"]:
            assert O.fmix32(int(b["fmix32"]["in"], 16)) == int(b["fmix32"]["out"], 16)
            # the worked word is the stated half of the pair's hash
            out = int(b["fmix32"]["out"], 16)
            assert b["pair_index"] == b["flat_index"] >> 1
            assert int(b["r16"], 16) == ((out & 0xFFFF) if b["half"] == "bottom" else (out >> 16))
            got = O.sr_bits(key, np.array([b["flat_index"]], dtype=np.uint64))
            assert int(got[0]) == int(b["r16"], 16), (case["seed"], b["flat_index"])
    assert n_calls == 4 * len(doc["cases"]) and len(doc["cases"]) >= 5


# ---------------------------------------------------------------------------
# bf16 rounding (Appendix C)
# ---------------------------------------------------------------------------
def test_bf16_rne_matches_torch_cast():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.normal(size=100000).astype(np.float32),
        (rng.normal(size=1000) * 1e-40).astype(np.float32),           # subnormals
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0, np.inf, -np.inf,
                  3.3895314e38, 1e-45], dtype=np.float32),           # ties, specials, overflow
    ])
    ours = O.f32_to_bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    nan = O.f32_to_bf16_rne(np.array([np.nan], dtype=np.float32))
    assert np.isnan(O.bf16_bits_to_f64(nan))[0]


def test_bf16_dead_zone_and_sr_exact_values():
    """Round-to-nearest discards an update below half an ULP (Appendix C,
    dead-zone); SR leaves exactly representable values unchanged."""
    w = np.float32(0.75)                  # bf16 ULP at 0.75 is 2^-8
    x = np.full(1000, w - np.float32(1e-3), dtype=np.float32)
    assert np.all(O.bf16_bits_to_f64(O.f32_to_bf16_rne(x)) == 0.75)
    exact = O.bf16_bits_to_f64(np.arange(0, 65535, 7, dtype=np.uint16)).astype(np.float32)
    exact = exact[np.isfinite(exact)]
    r = O.sr_bits(O.sr_key(1, 1, 0), np.arange(exact.size))
    out = O.bf16_bits_to_f64(O.f32_to_bf16_sr(exact, r))
    np.testing.assert_array_equal(out, exact.astype(np.float64))


def test_sr_unbiased_1e6_draws():
    """Proposition 5: E[SR(x)] = x.  x = 1 + 2^-10 sits 1/8 ULP above 1.0, so
    SR rounds up with probability 0.125; round-to-nearest is biased by
    -2^-10 = -9.77e-4."""
    n = 1_000_000
    x = np.full(n, 1 + 2 ** -10, dtype=np.float32)
    r = O.sr_bits(O.sr_key(1337, 1, 0), np.arange(n))
    y = O.bf16_bits_to_f64(O.f32_to_bf16_sr(x, r))
    assert set(np.unique(y)) <= {1.0, 1.0 + 2 ** -7}
    up = np.mean(y > 1.0)
    sd = math.sqrt(0.125 * 0.875 / n)                   # 3.3e-4
    assert abs(up - 0.125) < 5 * sd
    err = np.mean(y) - (1 + 2 ** -10)
    assert abs(err) < 5 * sd * 2 ** -7                  # 1.3e-5
    rne = O.bf16_bits_to_f64(O.f32_to_bf16_rne(x))
    assert np.all(rne == 1.0)
    assert np.mean(rne) - (1 + 2 ** -10) == pytest.approx(-2 ** -10)


def test_sr_quarter_ulp_microbenchmark():
    """Appendix C, Implementation: 100 steps of a true update of -1e-3 at a
    quarter ULP.  Round-to-nearest reports a mean change of 0.000, stochastic
    rounding -0.100 (the fp32-master value)."""
    n, steps = 100_000, 100
    idx = np.arange(n)
    w_sr = np.full(n, 0.75, dtype=np.float32)
    w_rn = w_sr.copy()
    for t in range(1, steps + 1):
        r = O.sr_bits(O.sr_key(1337, t, 0), idx)
        w_sr = O.bf16_bits_to_f64(O.f32_to_bf16_sr(w_sr - np.float32(1e-3), r)).astype(np.float32)
        w_rn = O.bf16_bits_to_f64(O.f32_to_bf16_rne(w_rn - np.float32(1e-3))).astype(np.float32)
    assert np.mean(w_rn.astype(np.float64) - 0.75) == 0.0
    assert abs(np.mean(w_sr.astype(np.float64) - 0.75) - (-0.100)) < 5e-4


@pytest.mark.parametrize("BT", [512, 4100])
@pytest.mark.parametrize("opt", ["adamw", "nadam"])
def test_bf16_flip_fraction_is_under_the_parity_floor(BT, opt):
    """The GPU parity tests require the stored bf16 patterns to equal the
    oracle's for a fraction >= 1 - (1e-3 + 2 sqrt(BT) 2^-16) of the elements.
    Derivation: with the same SR bits on both sides a pattern differs only
    where the fp32 gradient's summation error (about sqrt(BT) 2^-24 relative
    for a BT-term fp32 sum) moves the value across its rounding decision,
    which happens with probability of that size in units of a bf16 ULP
    (2^-8): about sqrt(BT) 2^-16, doubled, plus 1e-3 for the elements whose
    gradient nearly cancels.  Checked here on the oracle itself: the step
    stochastically rounded from an fp32 gradient summed in one fixed order
    (tokens ascending, a pessimistic order for fp32) against the step from
    the exact gradient, with the bf16 W, m and v and the inputs of the
    bf16-everywhere workload."""
    import synth
    N, K, step, seed = 256, 256, 10, 1337
    spec = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="bf16", v_fmt="bf16")
    X, dY = synth.activations(2, BT, N, K, step, in_dtype="bf16")
    st = synth.state(2, N, K, spec)
    Xh, dYh = synth.host(X), synth.host(dY)
    W, m, v = (O.Stored("bf16", synth.host(st[k])) for k in ("W", "m", "v"))
    hyp = O.Hyper(opt=opt, round="sr")
    exact = O.apply_step(O.weight_grad(Xh, dYh), W, m, v, hyp, step, seed)
    fp32 = O.apply_step(O.weight_grad(Xh, dYh, order="seq32"), W, m, v, hyp, step, seed)
    floor = 1e-3 + 2.0 * math.sqrt(BT) * 2.0 ** -16
    for name in ("W", "m", "v"):
        flips = float(np.mean(exact[name].data != fp32[name].data))
        print(f"{opt} BT {BT} {name}: {flips:.6f} of the patterns differ (floor {floor:.6f})")
        assert flips <= floor, (name, flips, floor)


# ---------------------------------------------------------------------------
# int8 moments (section 2.3, Appendix B)
# ---------------------------------------------------------------------------
def test_int8_round_trip_bound():
    """|q(x) - x| <= s/2 for every element of a block (Appendix B)."""
    rng = np.random.default_rng(7)
    x = (rng.standard_t(3, size=(64, 512)) * 1e-3).astype(np.float32)
    q, s = O.quantize_signed(x, 128)
    back = O.dequantize(q, s, 128)
    half = np.repeat(s, 128, axis=1) / 2
    assert np.all(np.abs(back.astype(np.float64) - x) <= half * (1 + 1e-6))
    assert q.min() >= -127 and q.max() <= 127
    # the absmax element of every block takes code +-127 exactly
    xb = x.reshape(64, 4, 128)
    qb = q.reshape(64, 4, 128)
    arg = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(qb, arg[:, :, None], axis=2)[:, :, 0]
    assert np.all(np.abs(top) == 127)
    v = np.abs(x)
    qu, su = O.quantize_unsigned(v, 128)
    backu = O.dequantize(qu, su, 128)
    halfu = np.repeat(su, 128, axis=1) / 2
    pos = v > 0
    # positive values below half a step are floored to code 1 (one step s):
    # their error is at most s, every other value is within s/2
    lim = np.where(v < halfu, 2 * halfu, halfu)
    assert np.all(np.abs(backu.astype(np.float64) - v)[pos] <= lim[pos] * (1 + 1e-6))


def test_int8_exact_grid_values():
    """Values on the quantisation grid come back exactly."""
    s = np.float32(0.5)
    codes = np.arange(-127, 128, dtype=np.int64)
    x = np.zeros((1, 256), dtype=np.float32)
    x[0, :255] = codes.astype(np.float32) * s
    q, sc = O.quantize_signed(x, 256)
    assert sc[0, 0] == np.float32(127 * 0.5 / 127)
    np.testing.assert_array_equal(q[0, :255], codes)


def test_quantisers_round_ties_to_even():
    """Round to nearest with ties to even (reading of Appendix B, Prop. 4):
    with absmax 127 (255) the reciprocal is exactly 1, so x = k + 1/2 is a
    tie; codes worked by hand.  A kernel that rounded ties away from zero
    (roundf) would give 1, 3, -1, -3, 127 here."""
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :8] = [127.0, 0.5, 2.5, -0.5, -2.5, 126.5, -126.5, 1.5]
    q, s = O.quantize_signed(x, 32)
    assert s[0, 0] == np.float32(1.0)
    assert list(q[0, :8]) == [127, 0, 2, 0, -2, 126, -126, 2]
    u = np.zeros((1, 32), dtype=np.float32)
    u[0, :6] = [255.0, 0.5, 2.5, 3.5, 254.5, 0.25]
    qu, su = O.quantize_unsigned(u, 32)
    assert su[0, 0] == np.float32(1.0)
    # 0.5 -> 0 by the tie rule, floored to 1 (a positive value never takes code 0)
    assert list(qu[0, :6]) == [255, 1, 2, 4, 254, 1]
    # the same ties with a non-trivial exact reciprocal: absmax 127/8, inv = 8
    x2 = x / np.float32(8)
    q2, s2 = O.quantize_signed(x2, 32)
    assert s2[0, 0] == np.float32(0.125)
    np.testing.assert_array_equal(q2, q)


@pytest.mark.parametrize("shift", [-100, -70, -40, 40])
def test_quantisers_commute_with_power_of_two_scaling(shift):
    """Scaling a block by 2^k leaves every 8-bit code unchanged and scales its
    scale by 2^k (every step of the quantiser is exact under such scaling
    while no value leaves the normal range).  Shifts of -70 and -100 take the
    block absmax below 2^-64, where the reciprocal is formed on values scaled
    by 2^64; -100 also takes it below 127 / FLT_MAX, where the plain
    reciprocal would overflow."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((8, 256)) * 1e-3).astype(np.float32)
    x[0, :64] = 0.0                                   # an all-zero 64-block
    x[1, 3] = 0.25                                    # an outlier
    f = np.float32(2.0 ** shift)
    for block in (32, 64, 128):
        for quant, arr in ((O.quantize_signed, x), (O.quantize_unsigned, np.abs(x)),
                           (lambda a, b: O.quantize_e4m3(a, b, False), x),
                           (lambda a, b: O.quantize_e4m3(a, b, True), np.abs(x))):
            q0, s0 = quant(arr, block)
            q1, s1 = quant((arr * f).astype(np.float32), block)
            np.testing.assert_array_equal(q1, q0)
            np.testing.assert_array_equal(s1, (s0 * f).astype(np.float32))


def test_uint8_reserved_zero():
    """Code 0 is reserved for an exact zero: v == 0 <=> code 0; tiny positive
    values are floored to code 1; an all-zero block has scale 0."""
    v = np.zeros((3, 128), dtype=np.float32)
    v[0, :] = np.linspace(0, 1, 128, dtype=np.float32)
    v[1, 5] = 1e-30
    v[1, 6] = 1.0
    q, s = O.quantize_unsigned(v, 128)
    assert np.all((q == 0) == (v == 0))
    assert q[1, 5] == 1 and q[1, 6] == 255
    assert s[2, 0] == 0 and np.all(q[2] == 0)
    assert q[0, 127] == 255


def test_int8_state_drift_bound_prop4():
    """Proposition 4: with identical gradients the int8-stored first moment
    stays within s/(2(1-b1)) of the exact one, and its RMS deviation is about
    s/sqrt(12(1-b1^2)); same for v with b2."""
    rng = np.random.default_rng(8)
    R, C, steps = 8, 512, 200
    b1, b2 = 0.9, 0.999
    m_ex, v_ex = np.zeros((R, C)), np.zeros((R, C))
    m_st = O.Stored("s8", np.zeros((R, C), np.int8), np.zeros((R, C // 128), np.float32))
    v_st = O.Stored("u8", np.zeros((R, C), np.uint8), np.zeros((R, C // 128), np.float32))
    W_st = O.Stored("f32", np.zeros((R, C), np.float32))
    smax_m = np.zeros((R, C // 128))
    smax_v = np.zeros((R, C // 128))
    worst_m = worst_v = 0.0
    devs, scales = [], []
    hyp = O.Hyper(opt="adamw", lr=1e-3, beta1=b1, beta2=b2, eps=1e-8, weight_decay=0.0)
    for t in range(1, steps + 1):
        G = rng.normal(0, 1e-2, (R, C))
        res = O.apply_step(G, W_st, m_st, v_st, hyp, t, 1337)
        m_st, v_st = res["m"], res["v"]
        m_ex = b1 * m_ex + (1 - b1) * G
        v_ex = b2 * v_ex + (1 - b2) * G * G
        smax_m = np.maximum(smax_m, m_st.scale)
        smax_v = np.maximum(smax_v, v_st.scale)
        dm = np.abs(O.decode(m_st) - m_ex)
        dv = np.abs(O.decode(v_st) - v_ex)
        worst_m = max(worst_m, np.max(dm / np.repeat(smax_m / (2 * (1 - b1)), 128, axis=1)))
        worst_v = max(worst_v, np.max(dv / np.repeat(smax_v / (2 * (1 - b2)), 128, axis=1)))
        if t > 50:
            devs.append(O.decode(m_st) - m_ex)
            scales.append(np.repeat(m_st.scale, 128, axis=1))
    assert worst_m <= 1.0 + 1e-5
    assert worst_v <= 1.0 + 1e-5
    rms = math.sqrt(np.mean(np.square(devs)))
    pred = math.sqrt(np.mean(np.square(scales))) / math.sqrt(12 * (1 - b1 ** 2))
    assert 0.5 * pred < rms < 2.0 * pred


# ---------------------------------------------------------------------------
# Proposition 1 / Corollary 1(a): per-tile schedule == materialise-then-step
# ---------------------------------------------------------------------------
def _small_layer(N, K, BT, in_dtype, w_fmt, m_fmt, v_fmt, seed, block=32):
    rng = np.random.default_rng(seed)
    Xf = rng.normal(0, 1, (BT, K)).astype(np.float32)
    dYf = (rng.normal(0, 1e-3, (BT, N))).astype(np.float32)
    if in_dtype == "bf16":
        X, dY = O.f32_to_bf16_rne(Xf), O.f32_to_bf16_rne(dYf)
    else:
        X, dY = Xf, dYf
    W32 = rng.normal(0, 0.02, (N, K)).astype(np.float32)
    W = O.Stored("f32", W32) if w_fmt == "f32" else O.Stored("bf16", O.f32_to_bf16_rne(W32))

    def mk(fmt, signed):
        x = (rng.normal(0, 1e-4, (N, K)) if signed else np.abs(rng.normal(0, 1e-6, (N, K)))).astype(np.float32)
        if fmt is None:
            return None
        if fmt == "f32":
            return O.Stored("f32", x)
        if fmt == "bf16":
            return O.Stored("bf16", O.f32_to_bf16_rne(x))
        q, s = (O.quantize_signed if signed else O.quantize_unsigned)(x, block)
        return O.Stored(fmt, q, s, block)

    return X, dY, W, mk(m_fmt, True), mk(v_fmt, False)


def _same(a, b):
    if a is None:
        assert b is None
        return
    np.testing.assert_array_equal(a.data, b.data)
    if a.scale is not None:
        np.testing.assert_array_equal(a.scale, b.scale)


@pytest.mark.parametrize("acc", ["seq32", "seq64"])
@pytest.mark.parametrize("fmts,opt", [
    (("f32", "f32", "f32", "f32"), "adamw"),
    (("bf16", "bf16", "f32", "f32"), "adamw"),
    (("bf16", "bf16", "bf16", "bf16"), "adamw"),
    (("bf16", "bf16", "s8", "u8"), "adamw"),
    (("bf16", "bf16", "f32", None), "lion"),
    (("bf16", "f32", "bf16", None), "sgdm"),
])
def test_tiled_schedule_equals_materialise_then_step(fmts, opt, acc):
    in_dtype, w_fmt, m_fmt, v_fmt = fmts
    int8 = m_fmt == "s8"
    N, K, BT = (70, 192, 37) if int8 else (70, 45, 37)
    X, dY, W, m, v = _small_layer(N, K, BT, in_dtype, w_fmt, m_fmt, v_fmt, seed=11)
    hyp = O.Hyper(opt=opt, lr=1e-3 if opt != "lion" else 1e-4, beta1=0.9,
                  beta2=0.999 if opt != "lion" else 0.99, round="sr")
    ref = O.wgrad_step(X, dY, W, m, v, hyp, 10, 1337, order=acc)
    rng = np.random.default_rng(12)
    tilings = [(32, 32 if int8 else 16, 8), (64, 64, 13), (17, 32 if int8 else 7, 5)]
    for tr, tc, tk in tilings:
        ntiles = -(-N // tr) * -(-K // tc)
        order = rng.permutation(ntiles)
        got = O.step_tiled(X, dY, W, m, v, hyp, 10, 1337, tr, tc, tk, order, acc=acc)
        _same(ref["W"], got["W"])
        _same(ref["m"], got["m"])
        _same(ref["v"], got["v"])


def test_tiled_schedule_detects_a_dropped_chunk():
    """The invariance test has teeth: skipping one token chunk changes W."""
    X, dY, W, m, v = _small_layer(40, 40, 64, "bf16", "f32", "f32", "f32", seed=3)
    hyp = O.Hyper()
    ref = O.wgrad_step(X, dY, W, m, v, hyp, 1, 1, order="seq32")
    bad = O.step_tiled(X[:48], dY[:48], W, m, v, hyp, 1, 1, 16, 16, 16, acc="seq32")
    assert not np.array_equal(ref["m"].data, bad["m"].data)


# ---------------------------------------------------------------------------
# End-to-end composition on the fp32 single-layer workload
# ---------------------------------------------------------------------------
def test_fp32_layer_three_steps_match_torch():
    """fp32 everywhere, BT 64, 256 x 256, AdamW t = 1..3 with fresh inputs:
    the oracle equals torch (matmul + torch.optim.AdamW in float64, state
    rounded to fp32 after each step) to fp32 rounding."""
    import synth
    spec = synth.LayerSpec(in_dtype="f32", w_fmt="f32", m_fmt="f32", v_fmt="f32")
    st = synth.state(0, 256, 256, spec, v_zero=True)
    W = O.Stored("f32", synth.host(st["W"]))
    m = O.Stored("f32", synth.host(st["m"]))
    v = O.Stored("f32", synth.host(st["v"]))
    p = torch.tensor(W.data.astype(np.float64), requires_grad=True)
    opt = torch.optim.AdamW([p], lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    hyp = O.Hyper(opt="adamw")
    for t in (1, 2, 3):
        X, dY = synth.activations(0, 64, 256, 256, t, in_dtype="f32", dy_std=0.01)
        X, dY = synth.host(X), synth.host(dY)
        res = O.wgrad_step(X, dY, W, m, v, hyp, t, 1337)
        W, m, v = res["W"], res["m"], res["v"]
        p.grad = torch.from_numpy(dY.astype(np.float64)).T @ torch.from_numpy(X.astype(np.float64))
        opt.step()
        with torch.no_grad():   # fp32 storage between steps
            p.copy_(p.to(torch.float32).to(torch.float64))
            for k in ("exp_avg", "exp_avg_sq"):
                opt.state[p][k].copy_(opt.state[p][k].to(torch.float32).to(torch.float64))
        np.testing.assert_allclose(W.data, p.detach().numpy().astype(np.float32), rtol=2e-7, atol=1e-12)
        np.testing.assert_allclose(m.data, opt.state[p]["exp_avg"].numpy().astype(np.float32), rtol=2e-7, atol=1e-20)
        np.testing.assert_allclose(v.data, opt.state[p]["exp_avg_sq"].numpy().astype(np.float32), rtol=2e-7, atol=1e-30)


# ---------------------------------------------------------------------------
# The other element-wise families (Appendix N, "fully fused"): each against
# torch.optim in float64 over enough steps to cover RAdam's switch to the
# rectified step (t = 6 with beta2 = 0.999), and against closed forms.
# ---------------------------------------------------------------------------
def _torch_run(make_opt, oracle_step, n=2048, steps=9, seed=11, state_keys=()):
    rng = np.random.default_rng(seed)
    W = rng.normal(0, 0.02, n)
    st = [np.zeros(n) for _ in state_keys]
    p = torch.tensor(W.copy(), dtype=torch.float64, requires_grad=True)
    opt = make_opt([p])
    for t in range(1, steps + 1):
        G = rng.normal(0, 1e-2, n)
        W, *st = oracle_step(W, G, st, t)
        p.grad = torch.tensor(G, dtype=torch.float64)
        opt.step()
        np.testing.assert_allclose(W, p.detach().numpy(), rtol=1e-12, atol=1e-18, err_msg=f"W at t={t}")
        for k, s in zip(state_keys, st):
            # torch forms the moments with lerp; rounding differs from b m + (1-b) g
            np.testing.assert_allclose(s, opt.state[p][k].numpy(), rtol=1e-10, atol=1e-22, err_msg=f"{k} at t={t}")


def test_nadam_matches_torch_nadam_decoupled_float64():
    # torch keeps NAdam's running product of mu_i as a tensor of the default
    # dtype; float64 throughout makes it the same product as the oracle's
    old = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    try:
        _nadam_run()
    finally:
        torch.set_default_dtype(old)


def _nadam_run():
    _torch_run(lambda ps: torch.optim.NAdam(ps, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01,
                                            momentum_decay=4e-3, decoupled_weight_decay=True),
               lambda W, G, st, t: O.nadam(W, G, st[0], st[1], t, 1e-3, 0.9, 0.999, 1e-8, 0.01),
               state_keys=("exp_avg", "exp_avg_sq"))


def test_radam_matches_torch_radam_decoupled_float64():
    _torch_run(lambda ps: torch.optim.RAdam(ps, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01,
                                            decoupled_weight_decay=True),
               lambda W, G, st, t: O.radam(W, G, st[0], st[1], t, 1e-3, 0.9, 0.999, 1e-8, 0.01),
               state_keys=("exp_avg", "exp_avg_sq"))


def test_rmsprop_matches_torch_rmsprop_float64():
    _torch_run(lambda ps: torch.optim.RMSprop(ps, lr=1e-3, alpha=0.99, eps=1e-8, weight_decay=0.01),
               lambda W, G, st, t: O.rmsprop(W, G, st[0], 1e-3, 0.99, 1e-8, 0.01),
               state_keys=("square_avg",))


def test_adagrad_matches_torch_adagrad_float64():
    _torch_run(lambda ps: torch.optim.Adagrad(ps, lr=1e-3, lr_decay=0, weight_decay=0.01, eps=1e-10,
                                              initial_accumulator_value=0.0),
               lambda W, G, st, t: O.adagrad(W, G, st[0], 1e-3, 1e-10, 0.01),
               state_keys=("sum",))


def test_sgd_matches_torch_sgd_float64():
    _torch_run(lambda ps: torch.optim.SGD(ps, lr=1e-3, weight_decay=0.01),
               lambda W, G, st, t: (O.sgd(W, G, 1e-3, 0.01),))


def test_first_steps_closed_forms():
    """t = 1 from zero state, eps = 0: each rule reduces to a sign step of a
    known length (nonzero G), independent of the gradient's magnitude."""
    W = np.array([0.3, -0.2, 0.05, -0.7])
    G = np.array([2e-3, -5e-1, 7.0, -1e-6])
    lr, wd = 1e-3, 0.01
    # RMSprop: v' = (1-a) g^2 -> W - lr sign(g) / sqrt(1-a), with g = G + wd W
    g = G + wd * W
    W1, v1 = O.rmsprop(W, G, np.zeros(4), lr, 0.99, 0.0, wd)
    np.testing.assert_allclose(W1, W - lr * np.sign(g) / math.sqrt(0.01), rtol=1e-13)
    np.testing.assert_allclose(v1, 0.01 * g * g, rtol=1e-15)
    # AdaGrad: v' = g^2 -> W - lr sign(g)
    W1, v1 = O.adagrad(W, G, np.zeros(4), lr, 0.0, wd)
    np.testing.assert_allclose(W1, W - lr * np.sign(g), rtol=1e-15)
    # RAdam before rectification: W' = (1 - lr wd) W - lr m_hat, m_hat = G at t = 1
    W1, m1, v1 = O.radam(W, G, np.zeros(4), np.zeros(4), 1, lr, 0.9, 0.999, 1e-8, wd)
    np.testing.assert_allclose(W1, (1 - lr * wd) * W - lr * G, rtol=1e-15)
    # NAdam: m_hat = G (1 + mu2 (1 - b1) / (1 - mu1 mu2)), v_hat = G^2
    mu1 = 0.9 * (1 - 0.5 * 0.96 ** 0.004)
    mu2 = 0.9 * (1 - 0.5 * 0.96 ** 0.008)
    W1, m1, v1 = O.nadam(W, G, np.zeros(4), np.zeros(4), 1, lr, 0.9, 0.999, 0.0, wd)
    np.testing.assert_allclose(W1, (1 - lr * wd) * W - lr * np.sign(G) * (1 + mu2 * 0.1 / (1 - mu1 * mu2)),
                               rtol=1e-13)
    # SGD is SGD with momentum at mu = 0 from a zero buffer
    np.testing.assert_allclose(O.sgd(W, G, lr, wd), O.sgdm(W, G, np.zeros(4), lr, 0.0, wd)[0], rtol=0)


def test_radam_rectification_limits():
    """rho_t <= 5 for t <= 5 (beta2 = 0.999): plain momentum steps; the
    rectification r_t -> 1 as t -> infinity (rho_t -> rho_inf)."""
    assert [O.radam_rect(t, 0.999)[0] for t in range(1, 8)] == [False] * 5 + [True] * 2
    on, r = O.radam_rect(10 ** 7, 0.999)
    assert on and abs(r - 1.0) < 1e-6


# ---------------------------------------------------------------------------
# Input gradient dX = dY W (Remark 1's upstream GEMM)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("BT,N,K", [(1, 1, 1), (2, 3, 9), (3, 9, 4), (7, 5, 130)])
def test_input_grad_brute_force(BT, N, K, in_dtype):
    """dX[t, q] = sum_p dY[t, p] W[p, q] against an exact integer triple loop;
    non-square shapes make a transposed operand fail."""
    rng = np.random.default_rng(BT * 77 + N * 7 + K)
    dYi = rng.integers(-64, 64, size=(BT, N))
    Wi = rng.integers(-64, 64, size=(N, K))
    dYt = torch.tensor(dYi, dtype=torch.float32) * 2.0 ** -6
    Wt = torch.tensor(Wi, dtype=torch.float32) * 2.0 ** -4
    if in_dtype == "bf16":
        dY = dYt.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        W = Wt.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    else:
        dY, W = dYt.numpy(), Wt.numpy()
    exact = np.array([[float(Fraction(sum(int(dYi[t, p]) * int(Wi[p, q]) for p in range(N)), 1024))
                       for q in range(K)] for t in range(BT)])
    np.testing.assert_array_equal(O.input_grad(dY, W), exact)
    rows = np.array([BT - 1, 0])
    np.testing.assert_array_equal(O.input_grad(dY, W, rows), exact[rows])


def test_input_grad_error_bound_covers_fp32_order():
    rng = np.random.default_rng(8)
    dY = (rng.normal(size=(40, 700)) * 1e-3).astype(np.float32)
    W = (rng.normal(size=(700, 30)) * 0.02).astype(np.float32)
    ref = O.input_grad(dY, W)
    acc = np.zeros((40, 30), dtype=np.float32)
    for p in range(700):                       # one fp32 order: p ascending
        acc = acc + np.multiply.outer(dY[:, p], W[p])
    assert np.all(np.abs(acc.astype(np.float64) - ref) <= O.input_grad_error_bound(dY, W))


# ---------------------------------------------------------------------------
# FP8 E4M3 moment storage
# ---------------------------------------------------------------------------
def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert O.e4m3_to_f64(np.array([0x7E]))[0] == 448.0 and O.e4m3_to_f64(np.array([0x01]))[0] == 2.0 ** -9


def test_e4m3_round_to_nearest_even_matches_torch_in_range():
    """torch's cast to float8_e4m3fn rounds to nearest even; inside the
    finite range the two must agree everywhere, including at every midpoint
    between neighbouring codes (ties) and in the subnormal range."""
    grid = O.e4m3_to_f64(np.arange(0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(9)
    x = np.concatenate([grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(0, 448, 20000), rng.uniform(0, 2 ** -6, 5000)]).astype(np.float32)
    x = x[x < 448]
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.f32_to_e4m3_rne(x), ref)
    assert O.f32_to_e4m3_rne(np.array([448.0, 1e6, -600.0], dtype=np.float32)).tolist() == [0x7E, 0x7E, 0xFE]


def test_e4m3_block_quantisation():
    """Scale absmax/448; the block maximum maps to 448 exactly; every element
    is within half a grid step of its value; a positive second moment never
    becomes zero; an all-zero block stores scale 0."""
    rng = np.random.default_rng(10)
    x = (rng.normal(size=(6, 256)) * 10.0 ** rng.uniform(-8, 2, size=(6, 1))).astype(np.float32)
    x[5] = 0
    q, s = O.quantize_e4m3(x, 64, positive=False)
    a = np.abs(x).reshape(6, 4, 64).max(axis=2)
    np.testing.assert_array_equal(s, (a / np.float32(448)).astype(np.float32))
    back = O.e4m3_to_f64(q).reshape(6, 4, 64) * s[:, :, None].astype(np.float64)
    xb = x.reshape(6, 4, 64).astype(np.float64)
    scaled = np.abs(xb) / np.where(s[:, :, None] > 0, s[:, :, None], 1)       # position on the E4M3 grid
    step = np.where(scaled >= 2 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(scaled, 2 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(back - xb) <= (0.5 * step + 1e-6 * scaled) * s[:, :, None] + 1e-45)
    assert np.all(s[5] == 0) and np.all((q[5] & 0x7F) == 0)
    v = np.abs(x)
    v[0, :3] = [1e-30, 0.0, 1e-12]
    qv, sv = O.quantize_e4m3(v, 128, positive=True)
    assert np.all(qv[v > 0] != 0) and np.all(qv[v == 0] == 0)


# ---------------------------------------------------------------------------
# FP8 (E4M3) weight store with stochastic rounding (section 3.6; the pages
# give no rule, the reading is in forge.h and the oracle)
# ---------------------------------------------------------------------------
def _e4m3_neighbours(y):
    """The E4M3 grid values at or below |y| and at or above it (by search on
    the grid itself), with |y| >= 448 saturating."""
    grid = O.e4m3_to_f64(np.arange(0x7F))
    ay = np.minimum(np.abs(y.astype(np.float64)), 448.0)
    hi_i = np.searchsorted(grid, ay, side="left")
    lo_i = np.where(grid[np.minimum(hi_i, 126)] == ay, hi_i, hi_i - 1)
    return grid[np.clip(lo_i, 0, 126)], grid[np.clip(hi_i, 0, 126)]


def test_e4m3_sr_takes_a_neighbour_and_truncates_with_zero_bits():
    rng = np.random.default_rng(21)
    y = np.concatenate([rng.uniform(-448, 448, 20000), 10.0 ** rng.uniform(-5, 2.6, 20000),
                        -(10.0 ** rng.uniform(-5, 2.6, 20000)), [500.0, -1e9, 0.0, -0.0]]).astype(np.float32)
    lo, hi = _e4m3_neighbours(y)
    for r in (0, 1, 0x7FFF, 0x8000, 0xFFFF):
        got = O.e4m3_to_f64(O.f32_to_e4m3_sr(y, np.full(y.shape, r)))
        mag = np.abs(got)
        assert np.all((mag == lo) | (mag == hi)), r
        assert np.all(np.signbit(got) == np.signbit(y)), r
        if r == 0:                                   # no random bits: toward zero
            np.testing.assert_array_equal(mag, lo)
    # grid values are kept for every r; beyond 448 saturates
    grid = O.e4m3_to_f64(np.arange(0x7F)).astype(np.float32)
    for r in (0, 0x1234, 0xFFFF):
        np.testing.assert_array_equal(O.e4m3_to_f64(O.f32_to_e4m3_sr(grid, np.full(grid.shape, r))), grid)
    assert O.e4m3_to_f64(O.f32_to_e4m3_sr(np.float32([479.0, 1e30]), np.full(2, 0xFFFF))).tolist() == [448.0, 448.0]


@pytest.mark.parametrize("y", [1.0 + 2.0 ** -5, 0.3, 300.0, 5.1 * 2.0 ** -9, 2.0 ** -12, -0.0107])
def test_e4m3_sr_unbiased(y):
    """E[SR(y)] = y over 1e6 counter-based draws, in the normal range, the
    subnormal range and across the sign; the probability of rounding up is
    the fractional position (Appendix C's argument, applied to E4M3)."""
    n = 1 << 20
    ys = np.full(n, y, dtype=np.float32)
    r = O.sr_bits(O.sr_key(1337, 3, 0), np.arange(n))
    got = O.e4m3_to_f64(O.f32_to_e4m3_sr(ys, r))
    lo, hi = _e4m3_neighbours(np.float32([y]))
    f = (abs(np.float64(np.float32(y))) - lo[0]) / (hi[0] - lo[0])
    sd = (hi[0] - lo[0]) * math.sqrt(f * (1 - f) / n)
    assert abs(np.mean(got) - np.float64(np.float32(y))) < 5 * sd + 2.0 ** -16 * (hi[0] - lo[0])
    up = np.mean(np.abs(got) == hi[0])
    assert abs(up - f) < 5 * math.sqrt(f * (1 - f) / n) + 2.0 ** -16


def test_fp8_weight_store_follows_the_rounding_mode():
    """An E4M3 weight takes stochastic rounding when the step's mode is SR
    (with the weight's own SR bits) and the nearest code when it is RNE;
    E4M3 moments take the nearest code either way."""
    rng = np.random.default_rng(5)
    N, K = 8, 256
    W0 = rng.standard_normal((N, K)).astype(np.float32) * 0.02
    qw, sw = O.quantize_e4m3(W0, 128, False)
    W = O.Stored("e4m3", qw, sw, 128)
    m = O.Stored("e4m3", np.zeros((N, K), np.uint8), np.zeros((N, 2), np.float32), 128)
    v = O.Stored("e4m3", np.zeros((N, K), np.uint8), np.zeros((N, 2), np.float32), 128)
    G = rng.standard_normal((N, K)) * 1e-3
    for mode in ("rne", "sr"):
        hyp = O.Hyper(opt="adamw", round=mode)
        out = O.apply_step(G, W, m, v, hyp, 10, 1337)
        pre = out["pre"]
        flat = np.arange(N * K, dtype=np.uint64).reshape(N, K)
        r16 = O.sr_bits(O.sr_key(1337, 10, O.TENSOR_W), flat) if mode == "sr" else None
        qW, sW = O.quantize_e4m3(pre["W"].astype(np.float32), 128, False, r16)
        np.testing.assert_array_equal(out["W"].data, qW)
        np.testing.assert_array_equal(out["W"].scale, sW)
        qm, _ = O.quantize_e4m3(pre["m"].astype(np.float32), 128, False)
        np.testing.assert_array_equal(out["m"].data, qm)
    assert not np.array_equal(O.apply_step(G, W, m, v, O.Hyper(round="sr"), 10, 1337)["W"].data,
                              O.apply_step(G, W, m, v, O.Hyper(round="rne"), 10, 1337)["W"].data)
