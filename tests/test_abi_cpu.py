"""Host-only checks of the C ABI: the library loads, exports every declared
entry point, and validates arguments (no device call is made; the pointers
below are fake and never dereferenced)."""

import ctypes
import os
import re

import pytest

import backward_weight_gradient_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "forge.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(forge_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("forge_wgrad_step", "forge_wgrad_check", "forge_wgrad_unfused", "forge_debug_sr_bf16",
              "forge_status_str", "forge_version", "forge_last_error"):
        assert n in names


def test_header_is_plain_c(tmp_path):
    """forge.h is a C ABI: it compiles as pedantic C99 (and as C++)."""
    import shutil
    import subprocess
    src = tmp_path / "use_forge.c"
    src.write_text('#include "forge.h"\nint main(void) { return (int)sizeof(forge_mat) + (int)sizeof(forge_layer)'
                   ' + (int)sizeof(forge_hyper) + (int)sizeof(forge_state); }\n')
    inc = os.path.dirname(HEADER)
    for cc, std in (("gcc", ["-std=c99", "-pedantic", "-x", "c"]), ("g++", ["-std=c++17", "-x", "c++"])):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not installed")
        r = subprocess.run([cc, *std, "-Wall", "-Wextra", "-Werror", "-fsyntax-only", f"-I{inc}", str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(F.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in forge.h but not exported"


def test_version_and_status_strings():
    assert "gfx950" in F.forge_version()
    for code in range(11):
        assert F.forge_status_str(code).startswith(F.STATUS_NAMES[code])


# fake, well-aligned, non-overlapping device addresses
BASE = 0x7F0000000000
GAP = 1 << 36


def addr(i):
    return BASE + i * GAP


def layer(N=256, K=256, BT=64, in_dt=F.FORGE_BF16, w_dt=F.FORGE_BF16, m_dt=F.FORGE_F32, v_dt=F.FORGE_F32,
          block=128):
    X = F.mat_raw(addr(0), in_dt, BT, K)
    dY = F.mat_raw(addr(1), in_dt, BT, N)
    W = F.mat_raw(addr(2), w_dt, N, K)
    ms = addr(5) if m_dt == F.FORGE_S8 else None
    vs = addr(6) if v_dt == F.FORGE_U8 else None
    m = F.forge_state(F.mat_raw(addr(3), m_dt, N, K), ms, block if ms else 0)
    v = F.forge_state(F.mat_raw(addr(4), v_dt, N, K), vs, block if vs else 0) if v_dt is not None else None
    return X, dY, W, m, v


def check(X, dY, W, m, v, h=None, step=10):
    return F.forge_wgrad_check(X, dY, W, m, v, h or F.hyper(), step)


def test_valid_configurations_pass():
    assert check(*layer()) == F.FORGE_OK
    assert check(*layer(in_dt=F.FORGE_F32, w_dt=F.FORGE_F32)) == F.FORGE_OK
    assert check(*layer(m_dt=F.FORGE_BF16, v_dt=F.FORGE_BF16)) == F.FORGE_OK
    assert check(*layer(m_dt=F.FORGE_S8, v_dt=F.FORGE_U8)) == F.FORGE_OK
    X, dY, W, m, _ = layer(v_dt=None)
    assert check(X, dY, W, m, None, F.hyper("lion", lr=1e-4, beta2=0.99)) == F.FORGE_OK
    assert check(X, dY, W, m, None, F.hyper("sgdm")) == F.FORGE_OK
    # ragged and degenerate shapes
    assert check(*layer(N=129, K=131, BT=65)) == F.FORGE_OK
    assert check(*layer(BT=0)) == F.FORGE_OK
    assert check(*layer(N=0)) == F.FORGE_OK


def test_null_pointers():
    X, dY, W, m, v = layer()
    assert F.forge_wgrad_check(None, dY, W, m, v, F.hyper(), 1) == F.FORGE_E_NULL
    assert F.forge_wgrad_check(X, dY, W, m, v, None, 1) == F.FORGE_E_NULL
    assert check(X, dY, W, None, v) == F.FORGE_E_NULL
    assert check(X, dY, W, m, None) == F.FORGE_E_NULL           # AdamW needs v
    W0 = F.mat_raw(0, F.FORGE_BF16, 256, 256)
    assert check(X, dY, W0, m, v) == F.FORGE_E_NULL
    X, dY, W, m, v = layer(m_dt=F.FORGE_S8, v_dt=F.FORGE_U8)
    m.scale = None
    assert check(X, dY, W, m, v) == F.FORGE_E_NULL


def test_step_zero_rejected():
    assert check(*layer(), step=0) == F.FORGE_E_STEP
    assert check(*layer(), step=-3) == F.FORGE_E_STEP


def test_shape_mismatches():
    X, dY, W, m, v = layer()
    assert check(F.mat_raw(addr(0), F.FORGE_BF16, 64, 255), dY, W, m, v) == F.FORGE_E_SHAPE
    assert check(X, F.mat_raw(addr(1), F.FORGE_BF16, 63, 256), W, m, v) == F.FORGE_E_SHAPE
    assert check(X, dY, F.mat_raw(addr(2), F.FORGE_BF16, 256, 128), m, v) == F.FORGE_E_SHAPE
    bad_m = F.forge_state(F.mat_raw(addr(3), F.FORGE_F32, 255, 256), None, 0)
    assert check(X, dY, W, bad_m, v) == F.FORGE_E_SHAPE
    assert check(X, dY, F.mat_raw(addr(2), F.FORGE_BF16, 256, 256, ld=200), m, v) == F.FORGE_E_SHAPE


def test_int8_block_rules():
    # K must be a multiple of the block
    assert check(*layer(K=200, m_dt=F.FORGE_S8, v_dt=F.FORGE_U8)) == F.FORGE_E_SHAPE
    # block must divide the 128-wide tile
    assert check(*layer(m_dt=F.FORGE_S8, v_dt=F.FORGE_U8, block=96)) == F.FORGE_E_SHAPE
    assert check(*layer(K=192, m_dt=F.FORGE_S8, v_dt=F.FORGE_U8, block=64)) == F.FORGE_OK
    # signed codes are for m, unsigned for v
    assert check(*layer(m_dt=F.FORGE_U8, v_dt=F.FORGE_U8)) == F.FORGE_E_DTYPE
    assert check(*layer(m_dt=F.FORGE_S8, v_dt=F.FORGE_S8)) == F.FORGE_E_DTYPE


def test_dtype_rules():
    X, dY, W, m, v = layer()
    assert check(F.mat_raw(addr(0), F.FORGE_F32, 64, 256), dY, W, m, v) == F.FORGE_E_DTYPE   # X != dY
    assert check(*layer(in_dt=F.FORGE_S8)) == F.FORGE_E_DTYPE
    assert check(*layer(w_dt=F.FORGE_U8)) == F.FORGE_E_DTYPE
    assert check(X, dY, W, m, v) == F.FORGE_OK
    assert check(*layer(in_dt=7)) == F.FORGE_E_DTYPE
    # mixed state layouts that are not built
    assert check(*layer(m_dt=F.FORGE_F32, v_dt=F.FORGE_BF16)) == F.FORGE_E_UNSUPPORTED


def test_optimizer_state_rules():
    X, dY, W, m, v = layer()
    assert check(X, dY, W, m, v, F.hyper("lion", lr=1e-4, beta2=0.99)) == F.FORGE_E_UNSUPPORTED  # v given
    assert check(X, dY, W, m, v, F.hyper("sgdm")) == F.FORGE_E_UNSUPPORTED


def test_hyper_parameter_rules():
    base = layer()
    bad = [F.hyper(lr=float("nan")), F.hyper(lr=-1.0), F.hyper(beta1=1.0), F.hyper(beta2=1.5),
           F.hyper(eps=0.0), F.hyper(weight_decay=float("inf")), F.hyper(weight_decay=-0.1)]
    for h in bad:
        assert check(*base, h=h) == F.FORGE_E_HYPER
    h = F.hyper()
    h.opt = 9
    assert check(*base, h=h) == F.FORGE_E_HYPER
    h = F.hyper()
    h.round = 5
    assert check(*base, h=h) == F.FORGE_E_HYPER


def test_alignment():
    X, dY, W, m, v = layer()
    assert check(X, dY, F.mat_raw(addr(2) + 1, F.FORGE_BF16, 256, 256), m, v) == F.FORGE_E_ALIGN
    bad_m = F.forge_state(F.mat_raw(addr(3) + 2, F.FORGE_F32, 256, 256), None, 0)
    assert check(X, dY, W, bad_m, v) == F.FORGE_E_ALIGN


def test_aliasing_rejected():
    X, dY, W, m, v = layer()
    assert check(X, dY, F.mat_raw(addr(0), F.FORGE_BF16, 256, 256), m, v) == F.FORGE_E_ALIAS   # W == X
    assert check(X, dY, F.mat_raw(addr(1) + 512, F.FORGE_BF16, 256, 256), m, v) == F.FORGE_E_ALIAS
    m2 = F.forge_state(F.mat_raw(addr(2) + 4096, F.FORGE_F32, 256, 256), None, 0)             # m inside W
    assert check(X, dY, W, m2, v) == F.FORGE_E_ALIAS
    v2 = F.forge_state(F.mat_raw(addr(3), F.FORGE_F32, 256, 256), None, 0)                    # v == m
    assert check(X, dY, W, m, v2) == F.FORGE_E_ALIAS


def test_flat_index_limit():
    # N * K >= 2^32 cannot be addressed by the 32-bit SR index
    assert check(*layer(N=65536, K=65536)) == F.FORGE_E_SHAPE
    assert check(*layer(N=65536, K=65535)) == F.FORGE_OK


def test_debug_sr_argument_errors():
    assert F.lib.forge_debug_sr_bf16(None, None, -1, 1, 1, 0, None) == F.FORGE_E_SHAPE
    assert F.lib.forge_debug_sr_bf16(None, None, 10, 1, 1, 0, None) == F.FORGE_E_NULL
    assert F.lib.forge_debug_sr_bf16(addr(0), addr(1), 10, 1, 0, 0, None) == F.FORGE_E_STEP
    assert F.lib.forge_debug_sr_bf16(addr(0), addr(0) + 8, 10, 1, 1, 0, None) == F.FORGE_E_ALIAS
    assert F.lib.forge_debug_sr_bf16(None, None, 0, 1, 1, 0, None) == F.FORGE_OK


def test_measurement_hook_argument_errors():
    """Validation of the ceiling hooks happens on the host, before any launch."""
    c = F.lib.forge_debug_copy
    assert c(addr(0), addr(1 << 20), -16, None) == F.FORGE_E_SHAPE
    assert c(addr(0), addr(1 << 20), 24, None) == F.FORGE_E_SHAPE       # not a multiple of 16
    assert c(None, addr(1 << 20), 32, None) == F.FORGE_E_NULL
    assert c(addr(0) + 8, addr(1 << 20), 32, None) == F.FORGE_E_ALIGN
    assert c(addr(0), addr(0) + 16, 64, None) == F.FORGE_E_ALIAS
    assert c(None, None, 0, None) == F.FORGE_OK                        # nothing to do
    m = F.lib.forge_debug_mfma_peak
    assert m(addr(0), 0, 10, None) == F.FORGE_E_SHAPE
    assert m(addr(0), 4, 0, None) == F.FORGE_E_SHAPE
    assert m(addr(0), (1 << 20) + 1, 10, None) == F.FORGE_E_SHAPE
    assert m(None, 4, 10, None) == F.FORGE_E_NULL
    assert m(addr(0) + 2, 4, 10, None) == F.FORGE_E_ALIGN


def test_unfused_argument_errors():
    X, dY, W, m, v = layer()
    h = F.hyper()
    rc = F.lib.forge_wgrad_unfused(ctypes.byref(X), ctypes.byref(dY), ctypes.byref(W), ctypes.byref(m),
                                   ctypes.byref(v), ctypes.byref(h), 1, 1, addr(7), F.FORGE_S8, None)
    assert rc == F.FORGE_E_DTYPE
    rc = F.lib.forge_wgrad_unfused(ctypes.byref(X), ctypes.byref(dY), ctypes.byref(W), ctypes.byref(m),
                                   ctypes.byref(v), ctypes.byref(h), 1, 1, None, F.FORGE_F32, None)
    assert rc == F.FORGE_E_NULL
    rc = F.lib.forge_wgrad_unfused(ctypes.byref(X), ctypes.byref(dY), ctypes.byref(W), ctypes.byref(m),
                                   ctypes.byref(v), ctypes.byref(h), 1, 1, addr(2) + 64, F.FORGE_F32, None)
    assert rc == F.FORGE_E_ALIAS


def test_last_error_is_a_static_string_before_any_launch():
    # No device call has been made on this thread: the HIP error behind the
    # last FORGE_E_HIP is hipSuccess's description.
    s = F.forge_last_error()
    assert isinstance(s, str) and len(s) > 0


def test_one_hip_runtime_per_process():
    # A fresh interpreter that imports only the binding must end up with a
    # single libamdhip64 mapped (the one torch loads), whatever the order.
    import subprocess
    import sys
    code = ("import os, backward_weight_gradient_amd\n"
            "maps = open(f'/proc/{os.getpid()}/maps').read()\n"
            "print(len(set(l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l)))\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


# ---------------------------------------------------------------------------
# forge_wgrad_step_group: every error is decided before anything is enqueued,
# so these cases make no device call.
# ---------------------------------------------------------------------------
def glayer(slot, seed=0, **kw):
    """layer() at its own set of fake addresses (slot 0 == layer())."""
    X, dY, W, m, v = layer(**kw)
    shift = slot * 8 * GAP
    X.data += shift
    dY.data += shift
    W.data += shift
    m.q.data += shift
    if m.scale:
        m.scale += shift
    if v is not None:
        v.q.data += shift
        if v.scale:
            v.scale += shift
    return (X, dY, W, m, v, seed)


def group(layers, h=None, step=10):
    return F.forge_wgrad_step_group(layers, h or F.hyper(), step, stream=0, check=False)


def test_group_count_limits():
    assert group([]) == F.FORGE_E_SHAPE
    assert group([glayer(i) for i in range(F.FORGE_GROUP_MAX + 1)]) == F.FORGE_E_SHAPE


def test_group_reports_a_layers_own_error():
    bad = glayer(1, N=256, K=255)                       # W must be [N, K]: shape mismatch below
    X, dY, W, m, v, s = bad
    W.cols = 100
    assert group([glayer(0), (X, dY, W, m, v, s)]) == F.FORGE_E_SHAPE
    assert group([glayer(0), glayer(1)], step=0) == F.FORGE_E_STEP


def test_group_formats_must_agree():
    assert group([glayer(0), glayer(1, m_dt=F.FORGE_BF16, v_dt=F.FORGE_BF16)]) == F.FORGE_E_UNSUPPORTED
    assert group([glayer(0), glayer(1, w_dt=F.FORGE_F32)]) == F.FORGE_E_UNSUPPORTED
    assert group([glayer(0, m_dt=F.FORGE_S8, v_dt=F.FORGE_U8, block=128),
                  glayer(1, m_dt=F.FORGE_S8, v_dt=F.FORGE_U8, block=64)]) == F.FORGE_E_UNSUPPORTED


def test_group_layers_must_not_write_each_others_buffers():
    a = glayer(0)
    b = glayer(1)
    # layer 1's W on top of layer 0's X
    b[2].data = a[0].data
    assert group([a, b]) == F.FORGE_E_ALIAS
    # layer 1's m on top of layer 0's W
    b = glayer(1)
    b[3].q.data = a[2].data
    assert group([a, b]) == F.FORGE_E_ALIAS


def test_group_of_empty_layers_is_a_no_op():
    # N == 0 everywhere: valid and nothing to launch
    assert group([glayer(0, N=0), glayer(1, N=0)]) == F.FORGE_OK


# ---------------------------------------------------------------------------
# State and hyper-parameter rules of the eight optimizer families
# ---------------------------------------------------------------------------
def test_family_state_rules():
    X, dY, W, m, v = layer()
    for opt in ("nadam", "radam"):
        assert check(X, dY, W, m, v, F.hyper(opt)) == F.FORGE_OK
        assert check(X, dY, W, m, None, F.hyper(opt)) == F.FORGE_E_NULL
    for opt in ("rmsprop", "adagrad"):
        assert check(X, dY, W, None, v, F.hyper(opt)) == F.FORGE_OK
        assert check(X, dY, W, m, v, F.hyper(opt)) == F.FORGE_E_UNSUPPORTED    # no first moment kept
        assert check(X, dY, W, None, None, F.hyper(opt)) == F.FORGE_E_NULL
    assert check(X, dY, W, None, None, F.hyper("sgd")) == F.FORGE_OK
    assert check(X, dY, W, m, None, F.hyper("sgd")) == F.FORGE_E_UNSUPPORTED
    assert check(X, dY, W, None, v, F.hyper("sgd")) == F.FORGE_E_UNSUPPORTED
    # AdamW, Lion, SGD-m still need m
    for opt in ("adamw", "lion", "sgdm"):
        assert check(X, dY, W, None, v if opt == "adamw" else None, F.hyper(opt)) == F.FORGE_E_NULL


def test_family_formats():
    # NAdam / RAdam: fp32 or bf16 moments, no int8
    X, dY, W, m, v = layer(m_dt=F.FORGE_BF16, v_dt=F.FORGE_BF16)
    assert check(X, dY, W, m, v, F.hyper("radam")) == F.FORGE_OK
    X, dY, W, m, v = layer(m_dt=F.FORGE_S8, v_dt=F.FORGE_U8)
    assert check(X, dY, W, m, v, F.hyper("nadam")) == F.FORGE_E_UNSUPPORTED
    # RMSprop / AdaGrad: v fp32 or bf16
    X, dY, W, m, v = layer(v_dt=F.FORGE_BF16)
    assert check(X, dY, W, None, v, F.hyper("adagrad")) == F.FORGE_OK
    X, dY, W, m, v = layer(m_dt=F.FORGE_S8, v_dt=F.FORGE_U8)
    assert check(X, dY, W, None, v, F.hyper("rmsprop")) == F.FORGE_E_UNSUPPORTED


def test_family_hyper_ranges():
    X, dY, W, m, v = layer()
    assert check(X, dY, W, None, v, F.hyper("rmsprop", beta2=1.0)) == F.FORGE_E_HYPER   # smoothing constant
    assert check(X, dY, W, None, v, F.hyper("rmsprop", eps=0.0)) == F.FORGE_E_HYPER
    assert check(X, dY, W, None, v, F.hyper("adagrad", eps=0.0)) == F.FORGE_E_HYPER
    assert check(X, dY, W, m, v, F.hyper("nadam", beta1=1.0)) == F.FORGE_E_HYPER
    assert check(X, dY, W, m, v, F.hyper("radam", eps=-1.0)) == F.FORGE_E_HYPER
    # parameters an optimizer does not use are not range-checked (only finiteness)
    assert check(X, dY, W, None, v, F.hyper("adagrad", beta1=1.5, beta2=2.0)) == F.FORGE_OK
    assert check(X, dY, W, None, None, F.hyper("sgd", beta1=3.0, eps=0.0)) == F.FORGE_OK
    assert check(X, dY, W, None, None, F.hyper("sgd", beta1=float("nan"))) == F.FORGE_E_HYPER
    h = F.hyper("sgd")
    h.opt = 8
    assert check(X, dY, W, None, None, h) == F.FORGE_E_HYPER


# ---------------------------------------------------------------------------
# Gradient accumulation entry points (validation only; no device call)
# ---------------------------------------------------------------------------
def _acc(N=256, K=256, dtype=F.FORGE_F32, slot=7):
    return F.mat_raw(addr(slot), dtype, N, K)


def test_accumulate_validation():
    X, dY, W, m, v = layer()
    acc = lambda *a, **k: F.forge_wgrad_accumulate(*a, stream=0, check=False, **k)
    assert acc(X, dY, _acc(dtype=F.FORGE_BF16), True) == F.FORGE_E_DTYPE
    assert acc(X, dY, _acc(N=255), True) == F.FORGE_E_SHAPE
    bad = _acc()
    bad.data = X.data                                   # on top of X
    assert acc(X, dY, bad, False) == F.FORGE_E_ALIAS
    assert F.lib.forge_wgrad_accumulate(F._ref(X), F._ref(dY), None, 1, None) == F.FORGE_E_NULL
    Xe, dYe, *_ = layer(N=0)
    assert acc(Xe, dYe, _acc(N=0), True) == F.FORGE_OK  # nothing to do, nothing launched


def test_step_accumulated_validation():
    X, dY, W, m, v = layer()
    step = lambda a, *r, **k: F.forge_wgrad_step_accumulated(X, dY, a, W, m, v, F.hyper(), 10, 1, stream=0,
                                                              check=False)
    bad = _acc()
    bad.data = W.data                                   # on top of W
    assert step(bad) == F.FORGE_E_ALIAS
    bad = _acc()
    bad.data = m.q.data
    assert step(bad) == F.FORGE_E_ALIAS
    assert step(_acc(dtype=F.FORGE_BF16)) == F.FORGE_E_DTYPE
    assert step(_acc(K=128)) == F.FORGE_E_SHAPE
    # the step's own rules still apply
    assert F.forge_wgrad_step_accumulated(X, dY, _acc(), W, m, None, F.hyper(), 10, 1, stream=0,
                                          check=False) == F.FORGE_E_NULL
    assert F.forge_wgrad_step_accumulated(X, dY, _acc(), W, m, v, F.hyper(), 0, 1, stream=0,
                                          check=False) == F.FORGE_E_STEP


# ---------------------------------------------------------------------------
# dX = dY W and the ordered backward step (validation only)
# ---------------------------------------------------------------------------
def test_dgrad_validation():
    X, dY, W, m, v = layer()                     # dY [64, 256], W [256, 256]
    dX = F.mat_raw(addr(7), F.FORGE_BF16, 64, 256)
    dg = lambda a, b, c: F.forge_dgrad(a, b, c, stream=0, check=False)
    bad = F.mat_raw(W.data, F.FORGE_BF16, 64, 256)                     # on top of W
    assert dg(dY, W, bad) == F.FORGE_E_ALIAS
    assert dg(dY, W, F.mat_raw(addr(7), F.FORGE_S8, 64, 256)) == F.FORGE_E_DTYPE
    assert dg(dY, W, F.mat_raw(addr(7), F.FORGE_BF16, 63, 256)) == F.FORGE_E_SHAPE
    assert dg(dY, F.mat_raw(addr(2), F.FORGE_BF16, 255, 256), dX) == F.FORGE_E_SHAPE
    assert F.lib.forge_dgrad(F._ref(dY), F._ref(W), None, None) == F.FORGE_E_NULL
    # an empty output needs no launch
    assert dg(F.mat_raw(addr(1), F.FORGE_BF16, 0, 256), W, F.mat_raw(addr(7), F.FORGE_BF16, 0, 256)) == F.FORGE_OK


def test_dgrad_split_workspace_and_validation():
    # workspace sizes: splits x BT x K x 4 bytes where the reduction is split, else 0
    wb = F.forge_dgrad_workspace_bytes
    # 256 x 256 tiles: splits s <= 8 of >= 32 chunks minimising rounds x chunks per split
    assert wb(512, 14336, 4096) == 8 * 512 * 4096 * 4      # gate / up at BT 512: 32 tiles, 8 splits of 56 chunks
    assert wb(512, 4096, 14336) == 2 * 512 * 14336 * 4    # down: 112 tiles, 2 splits fill the chip once
    assert wb(300, 8192, 4104) == 7 * 300 * 4104 * 4       # 34 tiles: 7 splits (238 workgroups) of <= 37 chunks
    # 128-token tiles
    assert wb(512, 4096, 4096) == 0                        # q / o: 256 tiles of 64 tokens fill the chip unsplit
    assert wb(512, 2048, 4096) == 0
    assert wb(256, 4096, 4096) == 4 * 256 * 4096 * 4       # 128 tiles of 64 tokens: 4 splits of 32 chunks
    assert wb(512, 1024, 4096) == 0                        # k / v: 32 chunks, too short to split
    assert wb(300, 2048, 1024) == 2 * 300 * 1024 * 4       # 24 tiles: 2 splits of 32 chunks
    assert wb(2048, 4096, 4096) == 0                       # 512 tiles of 128 tokens: no split
    assert wb(0, 4096, 4096) == 0 and wb(512, 0, 4096) == 0 and wb(-1, 8, 8) == 0
    # validation (nothing reaches the device): dY [512, 2048], W [2048, 1024], dX [512, 1024]
    dY = F.mat_raw(addr(1), F.FORGE_BF16, 512, 2048)
    W = F.mat_raw(addr(2), F.FORGE_BF16, 2048, 1024)
    dX = F.mat_raw(addr(7), F.FORGE_BF16, 512, 1024)
    need = wb(512, 2048, 1024)
    assert need > 0
    sp = lambda ws, nbytes, out=dX: F.lib.forge_dgrad_split(F._ref(dY), F._ref(W), F._ref(out), ws, nbytes, None)
    assert sp(None, need) == F.FORGE_E_NULL
    assert sp(addr(8), need - 16) == F.FORGE_E_SHAPE
    assert sp(addr(8), -1) == F.FORGE_E_SHAPE
    assert sp(addr(8) + 4, need) == F.FORGE_E_ALIGN
    assert sp(addr(7), need) == F.FORGE_E_ALIAS                          # on top of dX
    assert sp(addr(2) + 1024, need) == F.FORGE_E_ALIAS                   # inside W
    assert sp(addr(8), need, F.mat_raw(addr(7), F.FORGE_BF16, 511, 1024)) == F.FORGE_E_SHAPE
    assert F.lib.forge_dgrad_split(F._ref(dY), F._ref(W), None, addr(8), need, None) == F.FORGE_E_NULL


def test_backward_step_split_validation():
    # X [300, 1024], dY [300, 2048], W [2048, 1024]: the dX reduction (N = 2048) is split in two
    X, dY, W, m, v = layer(N=2048, K=1024, BT=300)
    need = F.forge_dgrad_workspace_bytes(300, 2048, 1024)
    assert need == 2 * 300 * 1024 * 4
    dX = F.mat_raw(addr(7), F.FORGE_BF16, 300, 1024)
    bs = lambda ws, nbytes, step=10: F.lib.forge_backward_step_split(
        F._ref(X), F._ref(dY), F._ref(W), F._ref(m), F._ref(v), F._ref(F.hyper()), step, 1, F._ref(dX), ws, nbytes,
        None)
    assert bs(None, need) == F.FORGE_E_NULL
    assert bs(addr(8), need - 4) == F.FORGE_E_SHAPE
    assert bs(addr(8) + 8, need) == F.FORGE_E_ALIGN
    assert bs(m.q.data, need) == F.FORGE_E_ALIAS                          # on top of m
    assert bs(X.data, need) == F.FORGE_E_ALIAS                            # on top of X
    assert bs(addr(7), need) == F.FORGE_E_ALIAS                           # on top of dX
    assert bs(addr(8), need, step=0) == F.FORGE_E_STEP


def test_backward_step_validation():
    X, dY, W, m, v = layer()
    bs = lambda dX, **k: F.forge_backward_step(X, dY, W, m, v, F.hyper(), k.get("step", 10), 1, dX, stream=0,
                                               check=False)
    assert bs(F.mat_raw(m.q.data, F.FORGE_BF16, 64, 256)) == F.FORGE_E_ALIAS   # on top of m
    assert bs(F.mat_raw(X.data, F.FORGE_BF16, 64, 256)) == F.FORGE_E_ALIAS     # on top of X
    assert bs(F.mat_raw(addr(7), F.FORGE_BF16, 64, 256), step=0) == F.FORGE_E_STEP


# ---------------------------------------------------------------------------
# E4M3 states (validation only)
# ---------------------------------------------------------------------------
def test_e4m3_state_rules():
    E = F.FORGE_E4M3
    X, dY, W, m, v = layer(m_dt=E, v_dt=E)
    m.scale, m.block = addr(5), 128
    v.scale, v.block = addr(6), 128
    assert check(X, dY, W, m, v) == F.FORGE_OK
    assert check(X, dY, W, m, None, F.hyper("lion")) == F.FORGE_OK
    assert check(X, dY, W, m, None, F.hyper("sgdm")) == F.FORGE_OK
    assert check(X, dY, W, m, v, F.hyper("nadam")) == F.FORGE_E_UNSUPPORTED       # fp32 / bf16 only
    X2, dY2, W2, m2, v2 = layer(m_dt=F.FORGE_S8, v_dt=E)
    v2.scale, v2.block = addr(6), 128
    assert check(X2, dY2, W2, m2, v2) == F.FORGE_E_UNSUPPORTED                     # S8 with E4M3
    m.scale = None
    assert check(X, dY, W, m, v) == F.FORGE_E_NULL                                 # scales required
    m.scale, m.block = addr(5), 48
    assert check(X, dY, W, m, v) == F.FORGE_E_SHAPE                                # block 32 / 64 / 128


def test_matrix_extent_is_bounded():
    """A leading dimension whose byte extent wraps around 64 bits, or exceeds
    2^48 bytes, is a shape error (not a spurious alias, not accepted)."""
    X, dY, W, m, v = layer(N=8, K=256)
    for ld in ((1 << 63) - 1, 1 << 62, 1 << 47):
        Wbad = F.mat_raw(addr(2), F.FORGE_BF16, 8, 256, ld=ld)
        assert check(X, dY, Wbad, m, v) == F.FORGE_E_SHAPE, ld
    # just inside: the extent of W is exactly 2^48 bytes (the inputs and states
    # are placed above it)
    ld_ok = ((1 << 47) - 256) // 7
    Wok = F.mat_raw(addr(2), F.FORGE_BF16, 8, 256, ld=ld_ok)
    assert (7 * ld_ok + 256) * 2 <= 1 << 48
    far = addr(2) + (1 << 48) + (1 << 36)
    m2 = F.forge_state(F.mat_raw(far, F.FORGE_F32, 8, 256), None, 0)
    v2 = F.forge_state(F.mat_raw(far + (1 << 36), F.FORGE_F32, 8, 256), None, 0)
    assert check(X, dY, Wok, m2, v2) == F.FORGE_OK
    # the same bound for the dX GEMM's operands
    dYg = F.mat_raw(addr(0), F.FORGE_BF16, 4, 256)
    Wg = F.mat_raw(addr(1), F.FORGE_BF16, 256, 256, ld=1 << 62)
    dX = F.mat_raw(addr(2), F.FORGE_BF16, 4, 256)
    assert F.lib.forge_dgrad(ctypes.byref(dYg), ctypes.byref(Wg), ctypes.byref(dX), None) == F.FORGE_E_SHAPE


def test_debug_quant_argument_errors():
    q = F.lib.forge_debug_quant
    a, c, s = addr(0), addr(1), addr(2)
    assert q(a, c, s, 4, 128, F.FORGE_F32, 0, 128, None) == F.FORGE_E_DTYPE
    assert q(a, c, s, 4, 128, F.FORGE_S8, 1, 128, None) == F.FORGE_E_DTYPE   # signed codes: first-moment rule
    assert q(a, c, s, 4, 128, F.FORGE_U8, 0, 128, None) == F.FORGE_E_DTYPE   # unsigned: second-moment rule
    assert q(a, c, s, 4, 128, F.FORGE_E4M3, 2, 128, None) == F.FORGE_E_DTYPE
    assert q(a, c, s, 4, 128, F.FORGE_S8, 0, 96, None) == F.FORGE_E_SHAPE
    assert q(a, c, s, 4, 96, F.FORGE_S8, 0, 64, None) == F.FORGE_E_SHAPE      # cols % block
    assert q(a, c, s, 1 << 17, 1 << 15, F.FORGE_S8, 0, 128, None) == F.FORGE_E_SHAPE   # 2^32 elements
    assert q(None, c, s, 4, 128, F.FORGE_S8, 0, 128, None) == F.FORGE_E_NULL
    assert q(a, c + 2, s, 4, 128, F.FORGE_S8, 0, 128, None) == F.FORGE_E_ALIGN
    assert q(a, a + 256, s, 4, 128, F.FORGE_S8, 0, 128, None) == F.FORGE_E_ALIAS
    assert q(a, c, c + 128, 4, 128, F.FORGE_E4M3, 1, 32, None) == F.FORGE_E_ALIAS
    assert q(None, None, None, 0, 128, F.FORGE_U8, 1, 128, None) == F.FORGE_OK


def test_debug_e4m3_sr_and_quotient_hook_argument_errors():
    f = F.lib.forge_debug_e4m3_sr
    assert f(None, None, -1, 1, 1, None) == F.FORGE_E_SHAPE
    assert f(None, None, 1 << 32, 1, 1, None) == F.FORGE_E_SHAPE
    assert f(addr(0), addr(1), 10, 1, 0, None) == F.FORGE_E_STEP
    assert f(None, addr(1), 10, 1, 1, None) == F.FORGE_E_NULL
    assert f(addr(0) + 2, addr(1), 10, 1, 1, None) == F.FORGE_E_ALIGN
    assert f(addr(0), addr(0) + 36, 10, 1, 1, None) == F.FORGE_E_ALIAS
    assert f(None, None, 0, 1, 1, None) == F.FORGE_OK
    q = F.lib.forge_debug_quotients
    assert q(None, None) == F.FORGE_E_NULL
    assert q(addr(0) + 4, None) == F.FORGE_E_ALIGN
    import torch
    with pytest.raises(ValueError):
        F.forge_debug_quotients(torch.zeros(8, dtype=torch.int64))
    with pytest.raises(ValueError):
        F.forge_debug_e4m3_sr(torch.zeros(8), torch.zeros(7, dtype=torch.uint8), 1, 1)


def test_binding_state_checks_the_scale_tensor():
    """The binding forwards a scale pointer only for a float32, contiguous
    tensor of exactly rows * cols / block elements on the codes' device."""
    import torch
    codes = torch.zeros((4, 256), dtype=torch.int8)
    good = torch.zeros((4, 2), dtype=torch.float32)
    assert F.state(codes, good, 128).block == 128
    for bad, block in ((torch.zeros(1, dtype=torch.float32), 128),           # too few
                       (torch.zeros((4, 2), dtype=torch.bfloat16), 128),     # wrong dtype
                       (torch.zeros((2, 4), dtype=torch.float32).t(), 128),  # not contiguous
                       (torch.zeros((4, 2), dtype=torch.float32), 96),       # block not allowed
                       (torch.zeros((4, 4), dtype=torch.float32), 128)):     # too many
        with pytest.raises(ValueError):
            F.state(codes, bad, block)
    with pytest.raises(ValueError):
        F.state(torch.zeros((4, 200), dtype=torch.int8), torch.zeros((4, 1)), 128)


def test_dgrad_noalloc_validation():
    """The allocation-free dX call validates like forge_dgrad and rejects, on
    the host, a split that needs more than its static scratch array."""
    nd = F.lib.forge_dgrad_split_noalloc
    dY = F.mat_raw(addr(0), F.FORGE_BF16, 512, 8192)
    W = F.mat_raw(addr(1), F.FORGE_BF16, 8192, 12288)
    dX = F.mat_raw(addr(2), F.FORGE_BF16, 512, 12288)
    assert F.forge_dgrad_workspace_bytes(512, 8192, 12288) > F.FORGE_DGRAD_SCRATCH_BYTES
    assert nd(ctypes.byref(dY), ctypes.byref(W), ctypes.byref(dX), None) == F.FORGE_E_SCRATCH
    # the Llama-3.1-8B shapes at BT 512 fit (64 MiB exactly for gate / up: 8 splits)
    for N, K in ((4096, 4096), (14336, 4096), (1024, 4096), (4096, 14336)):
        assert F.forge_dgrad_workspace_bytes(512, N, K) <= F.FORGE_DGRAD_SCRATCH_BYTES
    assert F.forge_dgrad_workspace_bytes(512, 14336, 4096) == F.FORGE_DGRAD_SCRATCH_BYTES
    # errors of forge_dgrad come first
    bad = F.mat_raw(addr(2), F.FORGE_BF16, 511, 12288)
    assert nd(ctypes.byref(dY), ctypes.byref(W), ctypes.byref(bad), None) == F.FORGE_E_SHAPE
    assert nd(None, ctypes.byref(W), ctypes.byref(dX), None) == F.FORGE_E_NULL
    alias = F.mat_raw(addr(1), F.FORGE_BF16, 512, 12288)
    assert nd(ctypes.byref(dY), ctypes.byref(W), ctypes.byref(alias), None) == F.FORGE_E_ALIAS


def test_state_stream_hook_argument_errors():
    f = F.lib.forge_debug_state_stream
    assert f(addr(0), addr(1), addr(2), 128, 100, None) == F.FORGE_E_SHAPE        # K % 128
    assert f(addr(0), addr(1), addr(2), 65536, 65536, None) == F.FORGE_E_SHAPE    # 2^32 elements
    assert f(None, addr(1), addr(2), 128, 128, None) == F.FORGE_E_NULL
    assert f(addr(0) + 4, addr(1), addr(2), 128, 128, None) == F.FORGE_E_ALIGN
    assert f(addr(0), addr(0) + 1024, addr(2), 128, 128, None) == F.FORGE_E_ALIAS
    assert f(None, None, None, 0, 128, None) == F.FORGE_OK
