#!/usr/bin/env python3
"""Benchmark of the fused weight-gradient + AdamW step on one MI355X.

One step = the fused weight-gradient + AdamW update of every linear layer of
a Llama-3.1-8B decoder layer (q, k, v, o, gate, up, down) at BT = 512 tokens
(batch 1 x sequence 512): bf16 X / dY / W, fp32 m / v, AdamW with bias
correction (step t = 10), stochastic-rounding bf16 weight store.  Inputs are
seeded synthetic tensors with the real layer shapes (X ~ N(0, 1),
dY ~ N(0, 1e-3^2), W ~ N(0, 0.02^2), m = 0, v = |N(0, 1e-6^2)|), resident in
HBM before timing starts.

Launch grouping (--grouping).  A layer's update only has to follow the input
gradient dX computed from its pre-update W (FORGE, Remark 1), so its weight
step may wait until the end of the decoder layer's backward.  Default
"block": one forge_wgrad_step_group launch for all seven layers after the
decoder layer's backward (the activation gradients of the seven stay alive
until then, ~44 MB at BT = 512).  "subblock": one launch for the MLP
([gate, up, down]) and one for attention ([q, k, v, o]).  "ready": four
launches as the layer gradients become available in backward order ([down],
[gate, up], [o], [q, k, v]).  "layer": seven forge_wgrad_step launches.  The
work is the same in all four; fewer launches pay the start of a launch (all
workgroups computing G, no state streaming yet) and its drain fewer times.

Prints one JSON line: params/s over the whole step, the fused kernel's
achieved HBM bandwidth against the 8 TB/s peak (algorithmic bytes: state read
and written once plus X and dY read once, per launch, divided by the launch
time measured with HIP events on the launch stream), the CPU oracle's
throughput on a bounded sample, and the unfused baseline (G written to HBM,
then the step) for comparison.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
BT = 512
STEP_T = 10
SEED = 1337
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_wgrad_llama8b_bt512_traffic.json")
KERNEL_DIR = os.path.join(ROOT, "backward_weight_gradient_amd", "csrc")


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=100,
                   help="untimed steps before the timed ones; from an idle GPU the engine clock takes some 50 ms "
                        "of continuous load to settle, and launches in that time run 5-12%% slower, so the "
                        "default (about 80 ms of steps) covers that")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    p.add_argument("--no-unfused", action="store_true", help="skip the unfused comparison")
    p.add_argument("--no-ceilings", action="store_true", help="skip the measured HBM and MFMA ceilings")
    p.add_argument("--cpu-quick", action="store_true",
                   help="time the oracle on k_proj of the fp32-moment workload only (a short check of the output)")
    p.add_argument("--grouping", choices=["block", "subblock", "ready", "layer"], default="block",
                   help="block: one launch for the decoder layer's seven; subblock: one launch per sub-block, "
                        "[gate, up, down] and [q, k, v, o]; ready: as the gradients become available, [down] "
                        "[gate, up] [o] [q, k, v]; layer: one forge_wgrad_step launch per layer")
    p.add_argument("--no-family-sweep", action="store_true",
                   help="skip the per-optimizer timing (gate_proj, BT 512, all eight families)")
    p.add_argument("--no-state-formats", action="store_true",
                   help="skip the grouped decoder-layer step with bf16, int8 and E4M3 moments")
    p.add_argument("--no-accumulation", action="store_true",
                   help="skip the gradient-accumulation timing (gate_proj, 4 micro-batches of 128 tokens)")
    p.add_argument("--no-dgrad", action="store_true",
                   help="skip the input-gradient GEMM timing (dX = dY W for the seven layers at BT 512)")
    p.add_argument("--no-mfma-sweep", action="store_true",
                   help="skip the compute-bound sweep (down_proj, lm_head at BT 2048 / 8192)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="instead of the step, time a plain 1 GiB device copy (read 1 GiB, write 1 GiB): the "
                        "reference kernel for scaling HBM counter readings")
    return p.parse_args()


LEAD_IN_CYCLES = 400_000   # about 0.2 ms of spinning at the engine clock


def lead_in():
    """Queue a short device-side spin on the current stream ahead of a
    per-call timing: while it runs, the host records the start event and
    enqueues the timed call, so the interval between the two events is
    device time (the kernels and the gaps between them), not the binding's
    argument marshalling on the host."""
    import torch
    torch.cuda._sleep(LEAD_IN_CYCLES)


# Before a per-call timing each case runs back to back for about this long
# (at least once, at most WARM_MAX_CALLS calls): from an idle or lightly
# loaded GPU the engine clock takes some 50 ms of continuous load to settle.
WARM_MS = 80.0
WARM_MAX_CALLS = 2000


def warm_up(fn):
    """Run fn back to back for about WARM_MS of device time, then synchronize
    (the second call sizes the loop: the first may include one-time loading)."""
    import torch
    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    n = min(WARM_MAX_CALLS, int(WARM_MS / max(e0.elapsed_time(e1), 1e-3)))
    for _ in range(n):
        fn()
    torch.cuda.synchronize()


# The per-call extras time BURST calls queued back to back between one pair of
# events, as a training step would launch them, and report the mean per call:
# an event pair around a lone call also holds the call's dispatch latency
# (a few microseconds).
BURST = 6


def timed_burst(fns, reps):
    """Median over `reps` samples of the mean device time per call (ms), each
    sample BURST calls back to back, cycling over `fns` (consecutive calls
    use different buffers where the caller passes several), after a lead-in
    spin; the case is warmed up first."""
    import torch
    fns = list(fns)
    stream = torch.cuda.current_stream()
    warm_up(lambda: [fn() for fn in fns])
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        lead_in()
        e0.record(stream)
        for i in range(BURST):
            fns[i % len(fns)]()
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / BURST)
    return sorted(ts)[len(ts) // 2]


def copy_calibration(steps):
    """A plain device-to-device copy of known size, for calibrating the
    FETCH_SIZE / WRITE_SIZE counters against a kernel whose traffic is known."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    lead_in()
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": round(ms, 4),
                      "copy_gbs": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)


def layer_bytes(N, K, bt):
    """Algorithmic HBM bytes of one fused launch: W bf16 (2+2), m and v fp32
    (4+4 each) read and written once, X and dY (bf16) read once."""
    P = N * K
    return 20 * P + 2 * bt * (N + K)


# the sources the timed kernel (k_fused_group for AdamW) is built from
HEADLINE_SOURCES = ("forge_device.h", "forge_internal.h", "forge_k_adamw.hip")


def kernel_sha():
    """sha256 over the sources of the timed kernel and its launcher (a change
    to any of them voids counter readings taken before it)."""
    h = hashlib.sha256()
    for name in HEADLINE_SOURCES:
        with open(os.path.join(KERNEL_DIR, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def load_traffic(grouping):
    """HBM bytes per step measured with rocprofv3 counters, if they were taken
    on the current kernel source with the same launch grouping; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_sha() or t.get("grouping") != grouping:
        return None
    return t.get("hbm_bytes_per_step")


def mfma_sweep(F, synth, h, reps=3):
    """Compute-bound configurations: down_proj [4096, 14336] and lm_head
    [128256, 4096] at BT = 2048 and 8192 with bf16 X, dY, W and fp32 moments,
    under AdamW (the step's hyperparameters), Lion (lr 1e-4, beta1 0.9,
    beta2 0.99) and SGD-momentum 0.9 (one launch each; HIP events on the
    launch stream).  Reported as achieved bf16 MFMA TFLOP/s (2 BT N K flops)
    against the 2.5 PFLOP/s peak.  AdamW keys are `<layer>_bt<BT>`, the other
    optimizers' `<layer>_bt<BT>_<optimizer>`."""
    import torch
    stream = torch.cuda.current_stream()
    optimizers = (("adamw", h, 20),
                  ("lion", F.hyper("lion", lr=1e-4, beta1=0.9, beta2=0.99, weight_decay=0.01), 12),
                  ("sgdm", F.hyper("sgdm", lr=1e-3, beta1=0.9, weight_decay=0.01), 12))
    out = {}
    for name, (N, K) in (("down_proj", (4096, 14336)), ("lm_head", (128256, 4096))):
        for bt in (2048, 8192):
            X, dY = synth.activations(4, bt, N, K, STEP_T, device="cuda")
            for opt, hy, state_bytes in optimizers:
                spec = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="f32",
                                       v_fmt="f32" if opt == "adamw" else None)
                st = synth.state(4, N, K, spec, device="cuda")
                args = (F.mat(X), F.mat(dY), F.mat(st["W"]), F.state(st["m"]),
                        None if st["v"] is None else F.state(st["v"]))
                warm_up(lambda: F.forge_wgrad_step(*args, hy, STEP_T, SEED, stream=stream.cuda_stream))
                times = []
                for _ in range(reps):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    lead_in()
                    e0.record(stream)
                    F.forge_wgrad_step(*args, hy, STEP_T, SEED, stream=stream.cuda_stream)
                    e1.record(stream)
                    torch.cuda.synchronize()
                    times.append(e0.elapsed_time(e1))
                ms = sorted(times)[len(times) // 2]
                tflops = 2.0 * bt * N * K / (ms * 1e-3) / 1e12
                alg = state_bytes * N * K + 2 * bt * (N + K)
                key = f"{name}_bt{bt}" if opt == "adamw" else f"{name}_bt{bt}_{opt}"
                out[key] = {"us": round(1e3 * ms, 1), "tflops": round(tflops, 1),
                            "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                            "hbm_gbs_alg": round(alg / (ms * 1e-3) / 1e9, 1)}
                del st, args
                torch.cuda.empty_cache()
            del X, dY
            torch.cuda.empty_cache()
    return out


def quantized_v(F, synth, st, cfg, N, K, fmt, extra, block=128):
    """Replace the stand-in codes of a block-scaled second moment with the
    int8 workload's init: |N(0, 1e-6^2)| quantised on the device by the
    library's own block quantiser (forge_debug_quant, the epilogue's code)."""
    import torch
    v32 = synth.normal((N, K), 1e-6, "cuda", cfg, 0, synth.T_V, extra).abs()
    codes = torch.empty((N, K), device="cuda", dtype=torch.uint8)
    scales = torch.empty((N, K // block), device="cuda", dtype=torch.float32)
    F.forge_debug_quant(v32, codes, scales, F.FORGE_U8 if fmt == "u8" else F.FORGE_E4M3, True, block)
    st["v"] = codes if fmt == "u8" else codes.view(torch.float8_e4m3fn)
    st["v_scale"] = scales
    del v32


def family_sweep(F, synth, reps=5):
    """Each of the eight optimizer families on gate_proj [14336, 4096] at
    BT = 512 (bf16 X / dY / W with SR, fp32 states where the family keeps
    them), and AdamW with bf16 moments (stochastic rounding on W, m and v), with
    int8 and with E4M3 block-scaled moments; timed_burst, `reps` samples.
    Algorithmic bytes: W read + written (4 B), each fp32 state read + written
    (8 B), each bf16 state (4 B) or each 8-bit state with its block scales
    (2 + 8/128 B), X and dY read once."""
    import torch
    N, K = 14336, 4096
    stream = torch.cuda.current_stream()
    X, dY = synth.activations(1, BT, N, K, STEP_T, device="cuda", extra=40)
    out = {}
    cases = [(o, "f32") for o in ("adamw", "nadam", "radam", "lion", "sgdm", "rmsprop", "adagrad", "sgd")]
    cases += [("adamw", "bf16"), ("adamw", "int8"), ("adamw", "e4m3")]
    for opt, state in cases:
        if state in ("f32", "bf16"):
            spec = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt=state if opt in F.KEEPS_M else None,
                                   v_fmt=state if opt in F.KEEPS_V else None)
        elif state == "int8":
            spec = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="s8", v_fmt="u8", block=128)
        else:
            spec = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="e4m3", v_fmt="e4m3", block=128)
        st = synth.state(1, N, K, spec, device="cuda", extra=40)
        blocked = state in ("int8", "e4m3")
        if blocked:
            quantized_v(F, synth, st, 1, N, K, spec.v_fmt, 40)
        m = (F.state(st["m"], st["m_scale"], 128) if blocked else F.state(st["m"])) if st["m"] is not None else None
        v = (F.state(st["v"], st["v_scale"], 128) if blocked else F.state(st["v"])) if st["v"] is not None else None
        args = (F.mat(X), F.mat(dY), F.mat(st["W"]), m, v)
        h = F.hyper(opt, lr=1e-4 if opt == "lion" else 1e-3, beta2=0.99 if opt == "lion" else None)
        ms = timed_burst([lambda: F.forge_wgrad_step(*args, h, STEP_T, SEED, stream=stream.cuda_stream)], reps)
        if blocked:    # 1-byte codes + one fp32 scale per 128 elements, read and written
            bpp = 4 + 2 * (2 + 8 / 128)
        else:          # each fp32 state read and written: 8 B; each bf16 state: 4 B
            per = 8 if state == "f32" else 4
            bpp = 4 + per * (opt in F.KEEPS_M) + per * (opt in F.KEEPS_V)
        nbytes = bpp * N * K + 2 * BT * (N + K)          # X and dY (bf16) read once
        name = opt if state == "f32" else f"{opt}_{state}"
        out[name] = {"us": round(1e3 * ms, 1), "state_bytes_per_param": bpp,
                     "hbm_gbs_alg": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del st, args, m, v
    del X, dY
    torch.cuda.empty_cache()
    return out


def fp8_weight_sweep(F, synth, h, reps=5):
    """E4M3 weight with fp32 block scales (forge_wgrad_step_fp8w) on gate_proj
    [14336, 4096] at BT = 512, AdamW t = 10 with stochastic rounding of the
    weight, moments fp32, bf16 or E4M3; and dX from the E4M3 weight
    (forge_dgrad_fp8w: the bf16 matrix cores, three exact bf16 terms per
    decoded weight).  The weight starts as the
    device-quantised N(0, 0.02^2) (forge_debug_quant, nearest code).
    Algorithmic bytes: W codes read and written (2 B) plus its scales
    (8 B per 128 elements), the moments' bytes, X and dY read once."""
    import torch
    N, K = synth.LLAMA8B_LAYERS["gate_proj"]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    X, dY = synth.activations(1, BT, N, K, STEP_T, device="cuda", extra=60)
    w32 = synth.normal((N, K), 0.02, "cuda", 1, 0, synth.T_W, 60)
    wq = torch.empty((N, K), device="cuda", dtype=torch.uint8)
    ws = torch.empty((N, K // 128), device="cuda", dtype=torch.float32)
    F.forge_debug_quant(w32, wq, ws, F.FORGE_E4M3, False, 128)
    del w32
    W = F.state(wq.view(torch.float8_e4m3fn), ws, 128)
    out = {}

    def timed(fn):
        return timed_burst([fn], reps)

    for fmt, mbytes in (("f32", 16.0), ("bf16", 8.0), ("e4m3", 2 * (2 + 8 / 128))):
        spec = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt=fmt, v_fmt=fmt, block=128)
        st = synth.state(1, N, K, spec, device="cuda", extra=60)
        if fmt == "e4m3":
            quantized_v(F, synth, st, 1, N, K, "e4m3", 60)
            m, v = F.state(st["m"], st["m_scale"], 128), F.state(st["v"], st["v_scale"], 128)
        else:
            m, v = F.state(st["m"]), F.state(st["v"])
        Xm, dYm = F.mat(X), F.mat(dY)
        ms = timed(lambda: F.forge_wgrad_step_fp8w(Xm, dYm, W, m, v, h, STEP_T, SEED, stream=sp))
        bpp = 2 + 8 / 128 + mbytes
        nbytes = bpp * N * K + 2 * BT * (N + K)
        out[f"adamw_{fmt}_moments"] = {"us": round(1e3 * ms, 1), "state_bytes_per_param": bpp,
                                       "hbm_gbs_alg": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                       "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del st, m, v
    dX = torch.empty((BT, K), device="cuda", dtype=torch.bfloat16)
    ms = timed(lambda: F.forge_dgrad_fp8w(dY, W, dX, stream=sp))
    out["dgrad_fp8w_gate_proj_us"] = round(1e3 * ms, 1)
    out["dgrad_fp8w_tflops"] = round(2.0 * BT * N * K / (ms * 1e-3) / 1e12, 1)
    del X, dY, wq, ws, dX
    torch.cuda.empty_cache()
    return out


def state_format_sweep(F, synth, h, reps=10):
    """The step's grouped launch (the seven Llama-3.1-8B layers at BT = 512,
    AdamW t = 10, SR) with compact moments: bf16 W, m, v (all three rounded
    stochastically), int8 m / v with fp32 scales per 128 elements (1% x50
    gradient outliers) and E4M3 m / v with fp32 scales per 128 elements;
    median of `reps` samples of back-to-back launches (timed_burst).  Algorithmic bytes: W read
    and written (4 B), each bf16 moment 4 B, each 8-bit moment 2 + 8/128 B,
    X and dY read once."""
    import torch
    order = ("gate_proj", "up_proj", "down_proj", "q_proj", "k_proj", "v_proj", "o_proj")
    specs = {"bf16": synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="bf16", v_fmt="bf16"),
             "int8": synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="s8", v_fmt="u8", block=128),
             "e4m3": synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="e4m3", v_fmt="e4m3", block=128)}
    cfg_of = {"bf16": 2, "int8": 3, "e4m3": 3}
    stream = torch.cuda.current_stream()
    out = {}
    for fmt, spec in specs.items():
        keep, layers_arg, P_total, nbytes = [], [], 0, 0
        bpp = 4 + (8.0 if fmt == "bf16" else 2 * (2 + 8 / 128))
        for i, name in enumerate(order):
            N, K = synth.LLAMA8B_LAYERS[name]
            X, dY = synth.activations(cfg_of[fmt], BT, N, K, STEP_T, device="cuda", extra=i,
                                      outlier_p=0.01 if fmt == "int8" else 0.0)
            st = synth.state(cfg_of[fmt], N, K, spec, device="cuda", extra=i)
            blocked = fmt != "bf16"
            if blocked:
                quantized_v(F, synth, st, cfg_of[fmt], N, K, spec.v_fmt, i)
            m = F.state(st["m"], st["m_scale"], 128) if blocked else F.state(st["m"])
            v = F.state(st["v"], st["v_scale"], 128) if blocked else F.state(st["v"])
            keep.append((X, dY, st))
            layers_arg.append((F.mat(X), F.mat(dY), F.mat(st["W"]), m, v, SEED))
            P_total += N * K
            nbytes += bpp * N * K + 2 * BT * (N + K)     # X and dY (bf16) read once
        ms = timed_burst([lambda: F.forge_wgrad_step_group(layers_arg, h, STEP_T, stream=stream.cuda_stream)], reps)
        out[fmt] = {"us": round(1e3 * ms, 1), "params_per_s": round(P_total / (ms * 1e-3), 1),
                    "state_bytes_per_param": bpp, "hbm_gbs_alg": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del keep, layers_arg
        torch.cuda.empty_cache()
    return out


def accumulation_sweep(F, synth, h, micro=4, reps=5):
    """Exact gradient accumulation (Appendix L) on gate_proj [14336, 4096]:
    `micro` micro-batches of BT / micro tokens, AdamW as in the step.  Each
    micro-step but the last adds into an fp32 accumulator (first one
    overwrites); the last runs the fused step on accumulator + its gradient.
    Algorithmic bytes: accumulator written (first) or read and written (4 / 8
    B per parameter), final step 20 + 4 B per parameter, activations once."""
    import torch
    N, K = 14336, 4096
    bt = BT // micro
    stream = torch.cuda.current_stream()
    spec = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="f32", v_fmt="f32")
    st = synth.state(1, N, K, spec, device="cuda", extra=50)
    mb = [synth.activations(1, bt, N, K, STEP_T, device="cuda", extra=50 + i) for i in range(micro)]
    acc = torch.empty((N, K), device="cuda", dtype=torch.float32)
    W, m, v = F.mat(st["W"]), F.state(st["m"]), F.state(st["v"])
    sp = stream.cuda_stream
    mats = [(F.mat(X), F.mat(dY)) for X, dY in mb]
    accm = F.mat(acc)

    # each phase timed on its own, its calls back to back (timed_burst): the
    # first micro-step (overwrites), an adding one, and the fused final step
    first = lambda: F.forge_wgrad_accumulate(*mats[0], accm, first=True, stream=sp)
    adds = [lambda Xm=Xm, dYm=dYm: F.forge_wgrad_accumulate(Xm, dYm, accm, first=False, stream=sp)
            for Xm, dYm in mats[1:-1]]
    final = lambda: F.forge_wgrad_step_accumulated(*mats[-1], accm, W, m, v, h, STEP_T, SEED, stream=sp)
    t_first = timed_burst([first], reps)
    t_add = timed_burst(adds, reps) if adds else 0.0
    t_final = timed_burst([final], reps)
    med = [t_first] + [t_add] * (micro - 2) + [t_final]
    act = 2 * bt * (N + K)                                  # X and dY (bf16) read once
    nbytes = [(4 if i == 0 else 8) * N * K + act for i in range(micro - 1)] + [24 * N * K + act]
    out = {"micro_batches": micro, "tokens_per_micro_batch": bt,
           "accumulate_first_us": round(1e3 * med[0], 1),
           "accumulate_add_us": round(1e3 * sum(med[1:-1]) / max(1, micro - 2), 1),
           "final_fused_step_us": round(1e3 * med[-1], 1),
           "total_us": round(1e3 * sum(med), 1)}
    out["hbm_gbs_alg"] = round(sum(nbytes) / (sum(med) * 1e-3) / 1e9, 1)
    del st, mb, acc, mats
    torch.cuda.empty_cache()
    return out


def dgrad_sweep(F, L, layers, reps=6, sets=3):
    """dX = dY W (bf16, fp32 accumulation, bf16 dX) for each layer of the step
    at BT = 512 (timed_burst, `reps` samples): forge_dgrad_split with its
    workspace (the reduction split across workgroups where that applies) and
    forge_dgrad (never split).  The launches rotate over `sets` copies of dY
    and W (the step's own, then clones), so consecutive launches do not find
    their operands in the 256 MiB MALL (q / o W is 32 MiB, k / v W 8 MiB)."""
    import torch
    stream = torch.cuda.current_stream()
    out = {}

    def timed(fns):
        return timed_burst(fns, reps)

    for name, (N, K) in layers.items():
        d = L[name]
        ops = [(d["dY"], d["W"])] + [(d["dY"].clone(), d["W"].clone()) for _ in range(sets - 1)]
        mats = [(F.mat(a), F.mat(b)) for a, b in ops]
        dX = torch.empty((BT, K), device="cuda", dtype=torch.bfloat16)
        dXm = F.mat(dX)
        need = F.forge_dgrad_workspace_bytes(BT, N, K)
        ws = torch.empty((need // 4,), device="cuda") if need else None
        sp = stream.cuda_stream
        ms = timed([lambda a=a, b=b: F.forge_dgrad_split(a, b, dXm, ws, stream=sp) for a, b in mats])
        ms_plain = timed([lambda a=a, b=b: F.forge_dgrad(a, b, dXm, stream=sp) for a, b in mats])
        tflops = 2.0 * BT * N * K / (ms * 1e-3) / 1e12
        out[name] = {"us": round(1e3 * ms, 1), "tflops": round(tflops, 1),
                     "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4), "workspace_bytes": need,
                     "us_unsplit": round(1e3 * ms_plain, 1), "buffer_sets": sets}
        del dX, ws, ops, mats
    out["seven_layers_us"] = round(sum(v["us"] for v in out.values()), 1)
    return out


def measured_ceilings(F, reps=5):
    """The box's own ceilings through the library's measurement hooks: HBM read + write in the
    fused epilogue's access width (a 1 GiB copy, 2 GiB moved; forge_debug_copy) and the matrix
    cores in a register-only v_mfma_f32_32x32x16_bf16 loop (forge_debug_mfma_peak).  timed_burst,
    `reps` samples."""
    import torch
    n = 1 << 30
    src = torch.empty(n // 4, device="cuda", dtype=torch.int32).random_()
    dst = torch.empty_like(src)

    def timed(fn):
        return timed_burst([fn], reps) * 1e-3

    t_copy = timed(lambda: F.forge_debug_copy(src, dst))
    del src, dst
    # the fused step's own state traffic (bf16 W, fp32 m and v, 20 B per element) through the
    # epilogue's access pattern with nothing computed: gate_proj-sized, 1.17 GB moved
    N, K = 14336, 4096
    Ws = torch.zeros((N, K), device="cuda", dtype=torch.bfloat16)
    ms_ = torch.zeros((N, K), device="cuda", dtype=torch.float32)
    vs_ = torch.zeros((N, K), device="cuda", dtype=torch.float32)
    t_state = timed(lambda: F.forge_debug_state_stream(Ws, ms_, vs_))
    del Ws, ms_, vs_
    blocks, iters = 2048, 4000
    out = torch.empty(256 * blocks, device="cuda")
    t_mfma = timed(lambda: F.forge_debug_mfma_peak(out, blocks, iters))
    del out
    torch.cuda.empty_cache()
    gbs = 2 * n / t_copy / 1e9
    gbs_state = 20.0 * N * K / t_state / 1e9
    tflops = blocks * 4 * iters * 131072 / t_mfma / 1e12
    return {"hbm_copy_gbs": round(gbs, 1), "hbm_copy_frac_of_spec": round(gbs / HBM_PEAK_GBS, 4),
            "hbm_state_stream_gbs": round(gbs_state, 1),
            "hbm_state_stream_frac_of_spec": round(gbs_state / HBM_PEAK_GBS, 4),
            "state_stream": "forge_debug_state_stream: bf16 W, fp32 m, v [14336, 4096] read and written once "
                            "(20 B per element) in the epilogue's 128 x 128 tile pattern, nothing computed",
            "mfma_bf16_tflops": round(tflops, 1), "mfma_frac_of_spec": round(tflops / BF16_PEAK_TFLOPS, 4),
            "copy": "1 GiB device copy, 16-byte non-temporal loads and stores, a contiguous chunk per workgroup "
                    "(2 GiB moved)",
            "mfma": f"{blocks} workgroups x 4 waves x {iters} rounds of 4 independent 32x32x16 bf16 MFMAs"}


def library_gemm_reference(synth, L, layers, reps=5):
    """The same GEMMs through hipBLASLt (torch.mm, bf16 in, bf16 out, fp32
    accumulation), timed beside the library's kernels: dX = dY W for the
    seven layers at BT = 512, and the weight gradient dY^T X alone (no
    optimizer step, G stored) for down_proj and lm_head at BT = 8192.  Each
    operand is made contiguous in the layout torch.mm reads best
    (row-major A and B, no transposed views)."""
    import torch
    out = {}

    def timed(fn):
        return timed_burst([fn], reps)

    dx = {}
    for name in layers:
        d = L[name]
        dY, W = d["dY"], d["W"]
        o = torch.empty((dY.shape[0], W.shape[1]), device="cuda", dtype=torch.bfloat16)
        ms = timed(lambda: torch.mm(dY, W, out=o))
        dx[name] = round(1e3 * ms, 1)
        del o
    out["dgrad_bt512_us"] = dx
    out["dgrad_bt512_seven_layers_us"] = round(sum(dx.values()), 1)
    for name, (N, K) in (("down_proj", (4096, 14336)), ("lm_head", (128256, 4096))):
        bt = 8192
        X, dY = synth.activations(4, bt, N, K, STEP_T, device="cuda")
        dYt = dY.t().contiguous()                    # [N, BT]: G = dY^T X as a plain NN product
        G = torch.empty((N, K), device="cuda", dtype=torch.bfloat16)
        ms = timed(lambda: torch.mm(dYt, X, out=G))
        tf = 2.0 * bt * N * K / (ms * 1e-3) / 1e12
        out[f"wgrad_gemm_{name}_bt{bt}"] = {"us": round(1e3 * ms, 1), "tflops": round(tf, 1),
                                           "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
        del X, dY, dYt, G
        torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_cpu():
    """The host's processor: model name, logical CPUs, and the CPUs this process may use."""
    info = {"model": cpu_model(), "logical_cpus": os.cpu_count()}
    try:
        info["usable_cpus"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        info["usable_cpus"] = os.cpu_count()
    return info


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def _oracle_layer(O, synth, cfg, N, K, bt, hyp, spec, outlier_p, threads):
    """One whole-layer oracle step (G by fp64 matmul, then the step and its
    stores).  Returns (matmul seconds on 1 BLAS thread, matmul seconds on
    `threads` threads, step seconds); the step runs once."""
    from threadpoolctl import threadpool_limits
    X, dY = synth.activations(cfg, bt, N, K, STEP_T, outlier_p=outlier_p, extra=90)
    st = synth.state(cfg, N, K, spec, extra=90)
    Xh, dYh = synth.host(X), synth.host(dY)
    del X, dY

    def stored(fmt, t, sc):
        if t is None:
            return None
        return O.Stored(fmt, synth.host(t), None if sc is None else sc.numpy(), spec.block)

    W = stored(spec.w_fmt, st["W"], None)
    m = stored(spec.m_fmt, st["m"], st["m_scale"])
    v = stored(spec.v_fmt, st["v"], st["v_scale"])
    mm = []
    for n in ((1, threads) if threads > 1 else (1,)):
        with threadpool_limits(n):
            t0 = time.perf_counter()
            G = O.weight_grad(Xh, dYh)
            mm.append(time.perf_counter() - t0)
    t1 = time.perf_counter()
    O.apply_step(G, W, m, v, hyp, STEP_T, SEED)
    return mm[0], mm[-1], time.perf_counter() - t1


def oracle_cpu_times(layers, quick=False):
    """The oracle (oracle/) on the host cores, per layer, for the BT = 512
    workloads: fp32 layer (config 0 shape, 256 x 256, BT 64), bf16 W with
    fp32 m / v (config 1), bf16 W / m / v (config 2) and int8 m / v with 1%
    x50 outliers (config 3), every layer in full.  The fp64 matmul is timed
    on 1 thread and on all BLAS threads; the element-wise step is plain
    single-threaded NumPy either way, so the all-core time of a layer is the
    all-thread matmul plus the step.  Config 4 (BT 2048 / 8192): down_proj
    in full (all threads) and lm_head on a seeded sample -- 4 corner and 12
    random 128 x 128 tiles plus 4,096 random elements -- timed per checked
    element with an extrapolated full-layer time, labelled as such."""
    import numpy as np
    import oracle as O
    import synth
    threads = _blas_threads()
    specs = {1: synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="f32", v_fmt="f32"),
             2: synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="bf16", v_fmt="bf16"),
             3: synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="s8", v_fmt="u8", block=128)}
    hyp = O.Hyper(opt="adamw", round="sr")
    out = {"blas_threads": threads, "host": host_cpu()}
    t_start = time.perf_counter()
    if quick:
        specs = {1: specs[1]}
        layers = {"k_proj": layers["k_proj"]}
    # config 0: fp32 256 x 256, BT 64, one step
    spec0 = synth.LayerSpec(in_dtype="f32", w_fmt="f32", m_fmt="f32", v_fmt="f32")
    mm1, _, st1 = _oracle_layer(O, synth, 0, 256, 256, 64, hyp, spec0, 0.0, 1)
    out["cfg0_fp32_256x256_bt64"] = {"matmul_1t_s": round(mm1, 5), "step_s": round(st1, 5)}
    for cfg, spec in specs.items():
        rows, tot1, totn, params = {}, 0.0, 0.0, 0
        for name, (N, K) in layers.items():
            mm1, mmn, step = _oracle_layer(O, synth, cfg, N, K, BT, hyp, spec, 0.01 if cfg == 3 else 0.0, threads)
            rows[name] = {"matmul_1t_s": round(mm1, 3), f"matmul_{threads}t_s": round(mmn, 3),
                          "step_s": round(step, 3), "single_thread_s": round(mm1 + step, 3),
                          "all_core_s": round(mmn + step, 3)}
            tot1 += mm1 + step
            totn += mmn + step
            params += N * K
        out[f"cfg{cfg}_bt512"] = {"layers": rows, "single_thread_s": round(tot1, 2), "all_core_s": round(totn, 2),
                                  "params": params, "params_per_s_all_core": round(params / totn, 1)}
    if quick:
        out["total_s"] = round(time.perf_counter() - t_start, 1)
        return out
    # config 4: down_proj in full (all threads)
    spec4 = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="f32", v_fmt="f32")
    N, K = layers["down_proj"]
    for bt in (2048, 8192):
        _, mm, step = _oracle_layer(O, synth, 4, N, K, bt, hyp, spec4, 0.0, threads)
        out[f"cfg4_down_proj_bt{bt}"] = {f"matmul_{threads}t_s": round(mm, 3), "step_s": round(step, 3),
                                         "all_core_s": round(mm + step, 3)}
    # config 4: lm_head at BT 8192 on a seeded sample of tiles and elements
    NL, KL = synth.LM_HEAD
    bt = 8192
    rng = np.random.default_rng(4)
    ti = [(0, 0), (0, KL // 128 - 1), (NL // 128 - 1, 0), (NL // 128 - 1, KL // 128 - 1)]
    ti += [(int(a), int(b)) for a, b in zip(rng.integers(0, NL // 128, 12), rng.integers(0, KL // 128, 12))]
    X = synth.host(synth.normal((bt, KL), 1.0, "cpu", 4, STEP_T, synth.T_X, 91).to(torch_bf16()))
    t_tiles = 0.0
    for (a, b) in ti:
        dYs = synth.host(synth.normal((bt, 128), 1e-3, "cpu", 4, STEP_T, synth.T_DY, 1000 + a).to(torch_bf16()))
        Wt = O.Stored("bf16", synth.host(synth.normal((128, 128), 0.02, "cpu", 4, 0, synth.T_W, a).to(torch_bf16())))
        z = O.Stored("f32", np.zeros((128, 128), np.float32))
        t0 = time.perf_counter()
        G = O.weight_grad(X[:, b * 128:(b + 1) * 128], dYs)
        O.apply_step(G, Wt, z, z.copy(), hyp, STEP_T, SEED)
        t_tiles += time.perf_counter() - t0
    rows = rng.integers(0, NL, 4096)
    cols = rng.integers(0, KL, 4096)
    dYe = synth.host(synth.normal((bt, 4096), 1e-3, "cpu", 4, STEP_T, synth.T_DY, 2000).to(torch_bf16()))
    t0 = time.perf_counter()
    for j in range(4096):
        O.weight_grad(X[:, cols[j]:cols[j] + 1], dYe[:, j:j + 1])
    t_el = time.perf_counter() - t0
    n_tiles = len(ti) * 128 * 128
    out["cfg4_lm_head_bt8192_sample"] = {
        "sample": "4 corner + 12 random 128x128 tiles (G by fp64 matmul over 8192 tokens, then the AdamW step) "
                  "and 4096 random single elements (G by one fp64 dot product each)",
        "tile_elements": n_tiles, "tile_seconds": round(t_tiles, 3),
        "tile_us_per_element": round(1e6 * t_tiles / n_tiles, 4),
        "single_elements": 4096, "single_seconds": round(t_el, 3),
        "single_us_per_element": round(1e6 * t_el / 4096, 3),
        "extrapolated_full_layer_s_from_tiles": round(t_tiles / n_tiles * NL * KL, 1),
        "extrapolated": True}
    out["total_s"] = round(time.perf_counter() - t_start, 1)
    return out


def torch_bf16():
    import torch
    return torch.bfloat16


def cpu_baseline_from(detail):
    """cpu_baseline: the oracle's params/s on the BT = 512 step's workload
    (config 1, all seven layers in full), all-core wall time (BLAS matmul on
    every thread, the element-wise step single-threaded)."""
    c1 = detail["cfg1_bt512"]
    h = detail["host"]
    return {"value": c1["params_per_s_all_core"], "unit": "params/s", "cores": detail["blas_threads"],
            "kind": "oracle",
            "sample": f"{','.join(c1['layers'])} of the Llama-3.1-8B decoder layer at BT={BT} in full "
                      f"({c1['params']} params, "
                      f"{c1['all_core_s']} s all-core, {c1['single_thread_s']} s single-thread); fp64 BLAS matmul "
                      f"on {detail['blas_threads']} threads, element-wise step single-threaded NumPy; host "
                      f"{h['model']}, {h['logical_cpus']} logical CPUs ({h['usable_cpus']} usable)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    import torch
    import backward_weight_gradient_amd as F
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layers = synth.LLAMA8B_LAYERS
    spec = synth.LayerSpec(in_dtype="bf16", w_fmt="bf16", m_fmt="f32", v_fmt="f32")
    h = F.hyper("adamw", lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, round="sr")

    L = {}
    for i, (name, (N, K)) in enumerate(layers.items()):
        X, dY = synth.activations(1, BT, N, K, STEP_T, device="cuda", extra=i)
        st = synth.state(1, N, K, spec, device="cuda", extra=i)
        L[name] = dict(N=N, K=K, X=X, dY=dY, W=st["W"], m=st["m"], v=st["v"],
                       mst=F.state(st["m"]), vst=F.state(st["v"]), Xm=F.mat(X), dYm=F.mat(dY), Wm=F.mat(st["W"]))
    torch.cuda.synchronize()
    P_total = sum(N * K for N, K in layers.values())
    bytes_total = sum(layer_bytes(N, K, BT) for N, K in layers.values())
    flops_total = sum(2 * BT * N * K for N, K in layers.values())
    if args.grouping == "layer":
        groups = [(n,) for n in layers]
    elif args.grouping == "ready":
        groups = [("down_proj",), ("gate_proj", "up_proj"), ("o_proj",), ("q_proj", "k_proj", "v_proj")]
    elif args.grouping == "block":
        groups = [("gate_proj", "up_proj", "down_proj", "q_proj", "k_proj", "v_proj", "o_proj")]
    else:
        groups = [("gate_proj", "up_proj", "down_proj"), ("q_proj", "k_proj", "v_proj", "o_proj")]
    names = [",".join(g) for g in groups]
    group_of = dict(zip(names, groups))
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def launch(name):
        g = group_of[name]
        if args.grouping == "layer":
            d = L[g[0]]
            F.forge_wgrad_step(d["Xm"], d["dYm"], d["Wm"], d["mst"], d["vst"], h, STEP_T, SEED, stream=sptr)
        else:
            F.forge_wgrad_step_group([(L[n]["Xm"], L[n]["dYm"], L[n]["Wm"], L[n]["mst"], L[n]["vst"], SEED)
                                      for n in g], h, STEP_T, stream=sptr)

    def group_bytes(name):
        return sum(layer_bytes(*layers[n], BT) for n in group_of[name])

    def timed_steps():
        """W untimed warm-up steps, then exactly K steps back to back between
        one pair of events on the launch stream (an event recorded between two
        launches adds ~11 us of queue time to each gap, measured in the kernel
        trace); returns ms per step.  With one launch per step (grouping
        "block") the interval is the launch's own duration plus the gaps
        between consecutive launches."""
        for _ in range(args.warmup):
            for n in names:
                launch(n)
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        for _ in range(args.steps):
            for n in names:
                launch(n)
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / args.steps

    # the timed region, right after set-up
    ms_per_step = timed_steps()
    # per-launch durations (spread, and the per-launch split of "subblock" /
    # "ready" / "layer" groupings): K more steps, each launch between its own
    # pair of events
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        for j, n in enumerate(names):
            ev[s][j][0].record(stream)
            launch(n)
            ev[s][j][1].record(stream)
    torch.cuda.synchronize()
    per_layer = {n: sorted(ev[s][j][0].elapsed_time(ev[s][j][1]) for s in range(args.steps))
                 for j, n in enumerate(names)}
    med = {n: v[len(v) // 2] for n, v in per_layer.items()}
    # mean kernel time per step of the timed region: all of it when one launch
    # makes a step; else its share by the per-launch event durations
    split = sum(sum(v) for v in per_layer.values()) / args.steps
    kernel_ms = ms_per_step if len(names) == 1 else min(ms_per_step, split)
    achieved_gbs = bytes_total / (kernel_ms * 1e-3) / 1e9
    # Context, not the timed region: from an idle GPU the launches some 5 to
    # 25 into a burst run 5-12% slower than later ones (the kernel trace; the
    # chip settling under the new load).  The same K steps after 60 more
    # untimed ones shows whether W warm-up steps were enough:
    for _ in range(60):
        for n in names:
            launch(n)
    settled = timed_steps()
    extras = {"settled_ms_per_step_after_60_more_steps": round(settled, 4)}

    if not args.no_unfused:
        # unfused baseline: G (fp32) to HBM, then the step; same layers, same protocol
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base_alloc = torch.cuda.memory_allocated()
        for n in names:
            launch(n)
        torch.cuda.synchronize()
        peak_fused = torch.cuda.max_memory_allocated() - base_alloc
        dws = {}
        torch.cuda.reset_peak_memory_stats()
        for n in layers:
            dws[n] = torch.empty((L[n]["N"], L[n]["K"]), device=dev, dtype=torch.float32)
        for _ in range(max(1, args.warmup)):
            for n in layers:
                d = L[n]
                F.forge_wgrad_unfused(d["Xm"], d["dYm"], d["Wm"], d["mst"], d["vst"], h, STEP_T, SEED, dws[n],
                                      stream=sptr)
        torch.cuda.synchronize()
        peak_unfused = torch.cuda.max_memory_allocated() - base_alloc
        u0 = torch.cuda.Event(enable_timing=True)
        u1 = torch.cuda.Event(enable_timing=True)
        u0.record(stream)
        for _ in range(args.steps):
            for n in layers:
                d = L[n]
                F.forge_wgrad_unfused(d["Xm"], d["dYm"], d["Wm"], d["mst"], d["vst"], h, STEP_T, SEED, dws[n],
                                      stream=sptr)
        u1.record(stream)
        torch.cuda.synchronize()
        extras["unfused_fp32_dw_ms_per_step"] = round(u0.elapsed_time(u1) / args.steps, 4)
        extras["peak_extra_bytes_fused"] = int(peak_fused)
        extras["peak_extra_bytes_unfused_fp32_dw"] = int(peak_unfused)
        del dws
        torch.cuda.empty_cache()

    if not args.no_family_sweep:
        extras["optimizer_families_gate_proj_bt512"] = family_sweep(F, synth)
    if not args.no_state_formats:
        extras["state_formats_llama8b_bt512_grouped"] = state_format_sweep(F, synth, h)
        extras["fp8_weight_gate_proj_bt512"] = fp8_weight_sweep(F, synth, h)
    if not args.no_dgrad:
        extras["dgrad_bt512"] = dgrad_sweep(F, L, layers)
    if not args.no_accumulation:
        extras["grad_accumulation_gate_proj"] = accumulation_sweep(F, synth, h)
    if not args.no_mfma_sweep:
        extras["compute_bound_sweep"] = mfma_sweep(F, synth, h)
    if not args.no_dgrad and not args.no_mfma_sweep:
        extras["hipblaslt_reference"] = library_gemm_reference(synth, L, layers)
    c = None if args.no_ceilings else measured_ceilings(F)

    traffic_step = load_traffic(args.grouping)
    roofline = {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
                "traffic": None if traffic_step is None else round(traffic_step / len(names))}

    extras.update({
        "kernel": ("forge::k_fused<bf16 in, AdamW, bf16 W, fp32 m, fp32 v>" if args.grouping == "layer" else
                   "forge::k_fused_group<AdamW, bf16 W, fp32 m, fp32 v>"),
        "grouping": args.grouping,
        "launches": names,
        "launches_per_step": len(names),
        "algorithmic_bytes_per_step": bytes_total,
        "algorithmic_bytes_per_launch_mean": bytes_total / len(names),
        "kernel_ms_per_step_mean": round(kernel_ms, 4),
        "mfma_util": round(flops_total / (kernel_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        "per_launch_us_median": {n: round(1e3 * v, 2) for n, v in med.items()},
        "per_launch_us_iqr": {n: [round(1e3 * v[len(v) // 4], 2), round(1e3 * v[(3 * len(v)) // 4], 2)]
                              for n, v in per_layer.items()},
        "per_launch_gbs_median": {n: round(group_bytes(n) / (med[n] * 1e-3) / 1e9, 1) for n in names},
    })
    if "unfused_fp32_dw_ms_per_step" in extras:
        extras["fused_speedup_vs_unfused"] = round(extras["unfused_fp32_dw_ms_per_step"] / ms_per_step, 3)
    if c is not None:
        extras["measured_ceilings"] = c
        extras["roofline_frac_of_measured_hbm"] = round(achieved_gbs / c["hbm_copy_gbs"], 4)
        extras["roofline_frac_of_state_stream"] = round(achieved_gbs / c["hbm_state_stream_gbs"], 4)
        for v in extras.get("compute_bound_sweep", {}).values():
            v["mfma_frac_of_measured"] = round(v["tflops"] / c["mfma_bf16_tflops"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        detail = oracle_cpu_times(layers, quick=args.cpu_quick)
        extras["oracle_cpu_times"] = detail
        extras["host_cpu"] = detail["host"]
        cpu = cpu_baseline_from(detail)

    out = {
        "metric": "fused wgrad+AdamW params/s & HBM GB/s (% roofline), Llama-8B shapes, BT=512",
        "value": P_total / (ms_per_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Llama-3.1-8B decoder-layer linears q,k,v,o,gate,up,down; BT=512 (BS 1 x SEQ 512); "
                               "bf16 X/dY/W, fp32 m/v, AdamW t=10, SR bf16 W store",
                   "global_batch": 1, "seq_len": BT, "params_per_step": P_total, "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
