"""Throughput of the MXFP4 block-scaled Hadamard-32 hot path on one MI355X.

One step = the whole path of a linear layer over one synthetic batch: six operand quantizations
(32-point Hadamard with random signs, truncation-free ceil scale, Philox stochastic rounding,
each along the reduction axis of the GEMM that consumes it) and the three MXFP4 GEMMs
(Fprop Y = H W^T, Dgrad dH = dY W, Wgrad dW = dY^T H), bf16 outputs, fp32 accumulation.

Default workload: the 70B MLP down-projection, one GPU's share (T=16384 tokens, hidden 8192,
FFN 28672). Inputs are generated on the GPU before timing (seeded, synthetic).

Prints one JSON line: whole-step MXFP4 TFLOP/s (value), plus the headline components — Wgrad
GEMM TFLOP/s and Hadamard-quantize GB/s as fractions of MI355X peak — the roofline record of the
dominant kernel (the GEMM, timed with HIP events on its stream) and the CPU oracle baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MXFP4 Wgrad GEMM TFLOPS + Hadamard-quant GB/s, as % of MI355X peak"
PEAK_FP4_TFLOPS = 10100.0   # MI355X dense MXFP4 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
QUANT_BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 32.0   # bf16 read + packed code + scale byte
GEMM_SRC = os.path.join(ROOT, "mxfp4_block_scaled_hadamard32_amd", "csrc", "gemm.hip")
QUANT_SRC = os.path.join(ROOT, "mxfp4_block_scaled_hadamard32_amd", "csrc", "quant.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_llama70b_down.json")


def sha(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="llama70b_down", choices=["llama70b_down", "llama8b_up"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-gemm-rows", type=int, default=64,
                   help="random full output rows per GEMM in the CPU oracle sample")
    p.add_argument("--cpu-gemm-elements", type=int, default=1024,
                   help="random single outputs per GEMM in the CPU oracle sample")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also launch one plain 1 GiB device copy (counter calibration runs)")
    p.add_argument("--step-only", action="store_true",
                   help="skip the comparisons run after the timed steps (fused epilogue, linear "
                        "layer), so that a profile of the run holds the step's launches alone")
    p.add_argument("--with-variants", action="store_true",
                   help="with --step-only, still run the MXFP8 and tile-size variant comparisons")
    p.add_argument("--power", type=float, metavar="SECONDS",
                   help="instead of the bench: run the Wgrad GEMM, the row and the column "
                        "quantizer of the larger operand and the matrix-core probe back to back "
                        "for SECONDS each while sampling board power and clock (amdsmi, "
                        "read-only), and print one JSON record of them")
    p.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="no GPU work: turn the counter_collection.csv files of a FETCH_SIZE and "
                        "a WRITE_SIZE rocprofv3 pass over a --copy-calibration run into the "
                        "per-launch HBM traffic record that later runs report")
    return p.parse_args()


class Layer:
    """Device buffers and the six quantize + three GEMM launches of one linear-layer step."""

    def __init__(self, mx, wl, workload: str):
        import torch
        self.mx, self.torch = mx, torch
        dev = "cuda"
        if workload == "llama70b_down":
            d = wl.llama70b_down(device=dev)
            self.X, self.W, self.dY = d["H"], d["W"], d["dY"]
            mask = wl.sign_mask()
            # (hadamard, mask, rule, round, alpha) per GEMM
            self.fprop_q = self.dgrad_q = self.wgrad_q = (1, mask, 1, 1)
            self.alpha = {"fprop": -5, "dgrad": -5, "wgrad": -5}
            self.desc = ("70B MLP down-projection, one GPU's share: H 16384x28672 ~ t(3), "
                         "W 8192x28672 ~ N(0,0.01), dY 16384x8192 ~ N(0,1e-3), bf16; "
                         "Hadamard32 (random signs) + ceil scale + SR on all six operand "
                         "quantizations; Fprop/Dgrad/Wgrad bf16 out")
        else:
            d = wl.llama8b_up(device=dev)
            self.X, self.W, self.dY = d["X"], d["W"], d["dY"]
            self.fprop_q = self.dgrad_q = (0, 0, 0, 0)
            self.wgrad_q = (1, 0, 0, 0)   # deterministic Hadamard along T, floor, RNE
            self.alpha = {"fprop": 0, "dgrad": 0, "wgrad": -5}
            self.desc = ("Llama-3.1-8B MLP up-projection, one GPU's share: T=8192, K=4096, "
                         "N=14336; floor scale, RNE; Wgrad with deterministic Hadamard along T")
        self.workload = workload
        self.T, self.K = self.X.shape
        self.N = self.W.shape[0]
        self.seeds = {"X": wl.SR_SEED, "W": wl.SR_SEED + 1, "dY": wl.SR_SEED + 2}
        T, K, N = self.T, self.K, self.N
        u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
        self.buf = {
            "Xq": (u8(T, K // 2), u8(T, K // 32)), "Wq": (u8(N, K // 2), u8(N, K // 32)),
            "dYq": (u8(T, N // 2), u8(T, N // 32)), "Wt": (u8(K, N // 2), u8(K, N // 32)),
            "dYt": (u8(N, T // 2), u8(N, T // 32)), "Xt": (u8(K, T // 2), u8(K, T // 32)),
        }
        bf = torch.bfloat16
        self.Y = torch.empty((T, N), dtype=bf, device=dev)
        self.dX = torch.empty((T, K), dtype=bf, device=dev)
        self.dW = torch.empty((N, K), dtype=bf, device=dev)
        self.flops = {"fprop": 2.0 * T * N * K, "dgrad": 2.0 * T * K * N, "wgrad": 2.0 * N * K * T}

    def quant(self, name, src, axis, q, seed_key):
        had, mask, rule, rnd = q
        c, s = self.buf[name]
        self.mx.mx_quantize(src, axis=axis, scale_rule=rule, round=rnd, hadamard=had,
                            sign_mask=mask, seed=self.seeds[seed_key], codes=c, scales=s)

    # the step's launches in order: (name, kind, source or GEMM operands)
    QUANTS = (("Xq", "X", 1, "fprop_q"), ("Wq", "W", 1, "fprop_q"), ("dYq", "dY", 1, "dgrad_q"),
              ("Wt", "W", 0, "dgrad_q"), ("dYt", "dY", 0, "wgrad_q"), ("Xt", "X", 0, "wgrad_q"))
    GEMMS = (("fprop", "Xq", "Wq", "Y"), ("dgrad", "dYq", "Wt", "dX"), ("wgrad", "dYt", "Xt", "dW"))
    LAUNCHES = tuple(q[0] for q in QUANTS) + tuple(g[0] for g in GEMMS)

    def step(self, ev=None):
        """One pass of the path. ev: None, or len(LAUNCHES) + 1 events recorded on the current
        stream around the launches (event i before launch i, the last one after the step)."""
        mx = self.mx
        i = 0
        for name, key, axis, q in self.QUANTS:
            if ev is not None:
                ev[i].record()
            i += 1
            self.quant(name, getattr(self, key), axis, getattr(self, q), key)
        b = self.buf
        fns = {"fprop": mx.mx_gemm_fprop, "dgrad": mx.mx_gemm_dgrad, "wgrad": mx.mx_gemm_wgrad}
        for name, a, bb, o in self.GEMMS:
            if ev is not None:
                ev[i].record()
            i += 1
            fns[name](*b[a], 1, *b[bb], 1, alpha_exp=self.alpha[name], out=getattr(self, o))
        if ev is not None:
            ev[i].record()

    def quant_bytes(self, name):
        """Algorithmic bytes of one quantize launch: bf16 in, packed codes and scales out."""
        src = {"Xq": self.X, "Wq": self.W, "dYq": self.dY, "Wt": self.W, "dYt": self.dY,
               "Xt": self.X}[name]
        return src.numel() * QUANT_BYTES_PER_ELEM

    def launch_report(self, evs, prefix=""):
        """Per-launch times averaged over the timed steps' events, with GB/s (quantize) and
        TFLOP/s (GEMM) and their fractions of the MI355X peaks; plus all six quantize launches
        together (total bytes over total time)."""
        n = len(evs)
        ms = {name: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / n
              for i, name in enumerate(self.LAUNCHES)}
        res = {}
        qb = qt = 0.0
        for name, *_ in self.QUANTS:
            gbs = self.quant_bytes(name) / (ms[name] * 1e-3) / 1e9
            qb += self.quant_bytes(name)
            qt += ms[name]
            res[f"{prefix}quant_{name}_ms"] = round(ms[name], 4)
            res[f"{prefix}quant_{name}_gbs"] = round(gbs, 1)
            res[f"{prefix}quant_{name}_pct_of_hbm_peak"] = round(100.0 * gbs / PEAK_HBM_GBS, 2)
        for name, *_ in self.GEMMS:
            tf = self.flops[name] / (ms[name] * 1e-3) / 1e12
            res[f"{prefix}{name}_gemm_ms"] = round(ms[name], 4)
            res[f"{prefix}{name}_gemm_tflops"] = round(tf, 1)
            res[f"{prefix}{name}_pct_of_fp4_peak"] = round(100.0 * tf / PEAK_FP4_TFLOPS, 2)
        agg = qb / (qt * 1e-3) / 1e9
        res[f"{prefix}quant_all6_ms"] = round(qt, 4)
        res[f"{prefix}quant_all6_gbs"] = round(agg, 1)
        res[f"{prefix}quant_all6_pct_of_hbm_peak"] = round(100.0 * agg / PEAK_HBM_GBS, 2)
        return res, ms


def host_ahead(torch):
    """Queues a few milliseconds of idle GPU work (a spin kernel) ahead of launches timed with
    events, so that the host has queued them all before the GPU reaches them: kernels of 15-50 us
    are otherwise timed together with the host's per-launch Python work. Called outside the
    intervals the events measure."""
    torch.cuda._sleep(5_000_000)


def timed_steps(layer, torch, steps):
    """Runs `steps` steps with events around every launch; returns the events."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(layer.LAUNCHES) + 1)]
           for _ in range(steps)]
    for e in evs:
        layer.step(e)
    return evs


def llama8b_components(mx, wl, torch, steps: int = 5):
    """Outside the timed step: the Llama-3.1-8B up-projection step (T=8192, K=4096, N=14336;
    floor scale, RNE; Wgrad with deterministic Hadamard along T), every launch timed."""
    layer = Layer(mx, wl, "llama8b_up")
    layer.step()
    torch.cuda.synchronize()
    host_ahead(torch)
    evs = timed_steps(layer, torch, steps)
    torch.cuda.synchronize()
    res, _ = layer.launch_report(evs, prefix="llama8b_")
    res["llama8b_workload"] = layer.desc
    del layer
    torch.cuda.empty_cache()
    return res


def cpu_threads() -> int:
    """Host threads the oracle may use: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(layer, gemm_rows: int = 64, gemm_elements: int = 1024):
    """The CPU oracle as it stands, timed on this host beside the GPU step.

    Quantize: the threaded oracle over each of the step's six operand quantizations on the full
    tensors (every thread gets at least one 32-row piece), as elements/s and GB/s of algorithmic
    traffic (bf16 in, packed codes and scales out).
    GEMM: for each of the three products, the float64 oracle on `gemm_rows` random full output
    rows (every column) and separately on `gemm_elements` random single outputs. The full GEMM's
    time is extrapolated from the row sample: dequantization scales with the operand elements
    (M + N) * K, the float64 products with the output rows M.
    Returns the whole-step rate in TFLOP/s with the pieces it was built from."""
    import numpy as np
    import threadpoolctl
    from oracle import oracle as orc
    import workloads as wl
    threads = cpu_threads()
    L = layer
    rng = np.random.default_rng(2024)
    quant = {}
    total = 0.0
    host = {}
    specs = [("Xq", "X", 1, L.fprop_q), ("Wq", "W", 1, L.fprop_q), ("dYq", "dY", 1, L.dgrad_q),
             ("Wt", "W", 0, L.dgrad_q), ("dYt", "dY", 0, L.wgrad_q), ("Xt", "X", 0, L.wgrad_q)]
    for name, key, axis, (had, mask, rule, rnd) in specs:
        if key not in host:
            host[key] = wl.host_input(getattr(L, key))
        x = host[key]
        t0 = time.perf_counter()
        orc.quantize(x, axis=axis, scale_rule=rule, round_mode=rnd, hadamard=had,
                     sign_mask=mask, seed=L.seeds[key], nthreads=threads)
        dt = time.perf_counter() - t0
        total += dt
        n = x.size
        quant[name] = {"elements": n, "s": round(dt, 3), "elements_per_s": round(n / dt, 1),
                       "GB_per_s": round(n * (2 + 0.5 + 1 / 32) / dt / 1e9, 3)}
    host.clear()
    b = L.buf
    gemm = {}
    with threadpoolctl.threadpool_limits(limits=threads):
        blas = [d["num_threads"] for d in threadpoolctl.threadpool_info()
                if d.get("user_api") == "blas"]
        for name, (aq, as_), (bq, bs), M, N, K in [
                ("fprop", b["Xq"], b["Wq"], L.T, L.N, L.K),
                ("dgrad", b["dYq"], b["Wt"], L.T, L.K, L.N),
                ("wgrad", b["dYt"], b["Xt"], L.N, L.K, L.T)]:
            ha, hsa = aq.cpu().numpy(), as_.cpu().numpy()
            hb, hsb = bq.cpu().numpy(), bs.cpu().numpy()
            rows = np.sort(rng.choice(M, size=min(gemm_rows, M), replace=False))
            tm = {}
            orc.gemm(ha, hsa, 1, hb, hsb, 1, M, N, K, L.alpha[name], rows=rows, timings=tm)
            r = len(rows)
            deq_rate = (r + N) * K / tm["dequant_s"]
            mm_flops = 2.0 * 2 * r * N * K  # the signed and the absolute product
            full_s = (M + N) * K / deq_rate + tm["matmul_s"] * M / r
            em = rng.integers(0, M, gemm_elements)
            en = rng.integers(0, N, gemm_elements)
            t0 = time.perf_counter()
            for m, n in zip(em, en):
                orc.gemm(ha, hsa, 1, hb, hsb, 1, M, N, K, L.alpha[name], rows=[m], cols=[n])
            el_s = (time.perf_counter() - t0) / gemm_elements
            total += full_s
            gemm[name] = {
                "sample_rows": r, "dequant_s": round(tm["dequant_s"], 3),
                "dequant_elements_per_s": round(deq_rate, 1),
                "matmul_s": round(tm["matmul_s"], 3),
                "matmul_GFLOP_per_s": round(mm_flops / tm["matmul_s"] / 1e9, 2),
                "full_gemm_extrapolated_s": round(full_s, 2),
                "single_element_us": round(el_s * 1e6, 1),
            }
    flops = sum(L.flops.values())
    return {"value": round(flops / total / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"oracle quantize of all six operand quantizations on the full tensors "
                       f"({threads} threads); oracle float64 GEMM on {gemm_rows} random full "
                       f"output rows and {gemm_elements} random single outputs of each product, "
                       f"full GEMM time extrapolated by (M+N)*K for dequantization and by M for "
                       f"the products; whole step {total:.1f} s"),
            "blas_threads": blas[0] if blas else None,
            "quantize": quant, "gemm": gemm}


def load_traffic(launch_flops_key: str, workload: str):
    # the record holds the counters of the llama70b_down launches only
    if workload != "llama70b_down" or not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("gemm_sha") != sha(GEMM_SRC):
        return None  # counters were taken on an older kernel
    return rec.get(launch_flops_key)


def fused_epilogue(layer, torch, reps: int = 5):
    """Outside the timed step: Fprop with its output quantized in the GEMM epilogue (1x32 along N,
    the layer's quantization options) against Fprop to bf16 followed by the row quantizer."""
    mx, L = layer.mx, layer
    had, mask, rule, rnd = L.fprop_q
    b = L.buf
    yq = torch.empty((L.T, L.N // 2), dtype=torch.uint8, device="cuda")
    ys = torch.empty((L.T, L.N // 32), dtype=torch.uint8, device="cuda")

    def fused():
        mx.mx_gemm_fprop_quant(*b["Xq"], 1, *b["Wq"], 1, alpha_exp=L.alpha["fprop"],
                               scale_rule=rule, round=rnd, hadamard=had, sign_mask=mask,
                               seed=L.seeds["X"], codes=yq, scales=ys)

    def separate():
        mx.mx_gemm_fprop(*b["Xq"], 1, *b["Wq"], 1, alpha_exp=L.alpha["fprop"], out=L.Y)
        mx.mx_quantize(L.Y, axis=1, scale_rule=rule, round=rnd, hadamard=had, sign_mask=mask,
                       seed=L.seeds["X"], codes=yq, scales=ys)

    res = {}
    for name, fn in (("fprop_quant_fused_ms", fused), ("fprop_then_quant_ms", separate)):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / reps, 4)
    return res


def linear_layer(layer, torch, reps: int = 3):
    """Outside the timed step: forward + backward of the MXFP4 linear layer (autograd op, the
    layer's quantization options on all three GEMMs; and the 2-D tile recipe) against the same op
    with every GEMM in bf16."""
    from mxfp4_block_scaled_hadamard32_amd import linear
    L = layer

    def spec(q):
        had, mask, rule, rnd = q
        return linear.QuantSpec(scale_rule=rule, round=rnd, hadamard=had, sign_mask=mask)

    x = L.X.detach().requires_grad_(True)
    w = L.W.detach().requires_grad_(True)
    dy = L.dY
    res = {}
    for name, cfg in (
            ("mx_linear_fwd_bwd_ms", linear.MXLinearConfig(fprop_q=spec(L.fprop_q),
                                                            dgrad_q=spec(L.dgrad_q),
                                                            wgrad_q=spec(L.wgrad_q))),
            ("mx_linear_tiles32_fwd_bwd_ms",  # W and dY in 32x32 tiles, X 1x32, ceil, RNE
             linear.MXLinearConfig(fprop_q=linear.QuantSpec(scale_rule=1),
                                   dgrad_q=linear.QuantSpec(scale_rule=1),
                                   wgrad_q=linear.QuantSpec(scale_rule=1), w_block=32,
                                   dy_block=32)),
            ("bf16_linear_fwd_bwd_ms", linear.MXLinearConfig(fprop=False, dgrad=False,
                                                              wgrad=False))):
        def run():
            x.grad = w.grad = None
            linear.MXLinearFunction.apply(x, w, cfg).backward(dy)
        run()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            run()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / reps, 4)
    x.grad = w.grad = None
    return res


PEAK_FP8_TFLOPS = 5000.0     # MI355X dense MXFP8 matrix-core peak
FP8_QUANT_BYTES_PER_ELEM = 2 + 1 + 1 / 32  # bf16 in, one code byte, one scale byte per 32


def mxfp8_attention(mx, wl, torch, reps: int = 5):
    """Outside the timed step: the MXFP8 variant for the attention query projection of the 70B
    model, one GPU's share (X 16384x8192, Wq 8192x8192, dY 16384x8192, bf16): X and Wq in E4M3,
    dY in E5M2, ceil scale, nearest-even; the X-along-K quantization and the three GEMMs."""
    d = wl.llama70b_attn_q(device="cuda")
    X, W, dY = d["X"], d["W"], d["dY"]
    T, D = X.shape
    N = W.shape[0]
    q = mx.mx_quantize_mxfp8
    xq, xs = q(X, fmt=0, scale_rule=1)
    wq, ws = q(W, fmt=0, scale_rule=1)
    wtq, wts = q(W, fmt=0, axis=0, scale_rule=1)
    dyq, dys = q(dY, fmt=1, scale_rule=1)
    dytq, dyts = q(dY, fmt=1, axis=0, scale_rule=1)
    xtq, xts = q(X, fmt=0, axis=0, scale_rule=1)
    bf = torch.bfloat16
    y = torch.empty((T, N), dtype=bf, device="cuda")
    dx = torch.empty((T, D), dtype=bf, device="cuda")
    dw = torch.empty((N, D), dtype=bf, device="cuda")
    runs = [("quant_x_rows", lambda: q(X, fmt=0, scale_rule=1, codes=xq, scales=xs)),
            ("fprop", lambda: mx.mx_gemm_mxfp8(xq, xs, 0, wq, ws, 0, out=y)),
            ("dgrad", lambda: mx.mx_gemm_mxfp8(dyq, dys, 1, wtq, wts, 0, out=dx)),
            ("wgrad", lambda: mx.mx_gemm_mxfp8(dytq, dyts, 1, xtq, xts, 0, out=dw))]
    flops = 2.0 * T * D * N
    res = {"mxfp8_workload": "70B attention query projection, T=16384, D=8192, N=8192; "
                             "X, Wq E4M3, dY E5M2; ceil scale, RNE"}
    for name, fn in runs:
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        host_ahead(torch)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[f"mxfp8_{name}_ms"] = round(ms, 4)
        if name == "quant_x_rows":
            gbs = T * D * FP8_QUANT_BYTES_PER_ELEM / (ms * 1e-3) / 1e9
            res["mxfp8_quant_x_rows_gbs"] = round(gbs, 1)
            res["mxfp8_quant_x_rows_pct_of_hbm_peak"] = round(100.0 * gbs / PEAK_HBM_GBS, 2)
        else:
            tf = flops / (ms * 1e-3) / 1e12
            res[f"mxfp8_{name}_tflops"] = round(tf, 1)
            res[f"mxfp8_{name}_pct_of_fp8_peak"] = round(100.0 * tf / PEAK_FP8_TFLOPS, 2)
    return res


def quant_stream(mx, wl, torch, reps: int = 24, copies: int = 8):
    """Outside the timed step: the quantize-only stream workload exactly (A 8192x4096 bf16 ~ t(3)
    with 0.5% of channels x100; random-sign Hadamard32, ceil scale, SR with Philox key 1234),
    along rows, at 2.53125 algorithmic B/element. The launches rotate over `copies` copies of A
    (537 MB, twice the 256 MB Infinity Cache, so every launch streams its input from HBM) and are
    replayed from a captured HIP graph, so the event time holds no host gaps between launches."""
    A = wl.quant_stream(device="cuda")["A"]
    rows, cols = A.shape
    srcs = [A.clone() for _ in range(copies)]
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")

    def run(x):
        mx.mx_quantize(x, scale_rule=1, round=1, hadamard=1, sign_mask=wl.sign_mask(),
                       seed=wl.SR_SEED, codes=codes, scales=scales)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up off the capture
        for x in srcs:
            run(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            run(srcs[i % copies])
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del g, srcs
    gbs = rows * cols * QUANT_BYTES_PER_ELEM / (ms * 1e-3) / 1e9
    return {"quant_stream_8192x4096_ms": round(ms, 4), "quant_stream_8192x4096_gbs": round(gbs, 1),
            "quant_stream_8192x4096_pct_of_hbm_peak": round(100.0 * gbs / PEAK_HBM_GBS, 2)}


def mfma_ceiling(torch, workgroups: int = 2048, iters: int = 1000, reps: int = 3):
    """Measured ceiling of the block-scaled FP4 matrix instruction (libmx_probe.so, a measurement
    aid): one wave per SIMD, 16 independent 32x32x64 accumulator chains per wave, random FP4
    operand bits and scales near 1, no memory traffic. Returns the median TFLOP/s of `reps`
    timed launches after one warm-up launch."""
    import ctypes
    from mxfp4_block_scaled_hadamard32_amd import build as hip_build
    if not os.path.exists(hip_build.PROBE_LIB):
        raise SystemExit("libmx_probe.so is not built (run __graft_entry__.build())")
    P = ctypes.CDLL(hip_build.PROBE_LIB)
    P.mx_probe_mfma_fp4.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                    ctypes.c_void_p, ctypes.c_void_p]
    P.mx_probe_mfma_fp4.restype = ctypes.c_int32
    sink = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    rates = []
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = P.mx_probe_mfma_fp4(workgroups, iters, 0x9E3779B9 + r, sink.data_ptr(), stream)
        e1.record()
        torch.cuda.synchronize()
        if rc != 0:
            raise SystemExit(f"mx_probe_mfma_fp4 failed with HIP error {rc}")
        if r > 0:
            flops = workgroups * 4 * iters * 16 * 2.0 * 32 * 32 * 64
            rates.append(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return sorted(rates)[len(rates) // 2]


def power_phases(layer, torch, secs: float):
    """Board power, clock and hotspot temperature (amdsmi, read-only; sampled every 50 ms) while
    each of the Wgrad GEMM, the row quantizer of X, the column quantizer of X and the
    matrix-core probe runs back to back for `secs` seconds, after 1.5 s idle each. The first
    third of each phase's samples (the ramp) is left out of its averages."""
    import threading
    try:
        import amdsmi
    except ImportError as e:
        raise SystemExit(f"--power needs the amdsmi module: {e}")
    import ctypes
    from mxfp4_block_scaled_hadamard32_amd import build as hip_build
    amdsmi.amdsmi_init()
    h = amdsmi.amdsmi_get_processor_handles()[0]
    try:
        cap = amdsmi.amdsmi_get_power_cap_info(h)
    except Exception as e:  # not every driver reports it
        cap = {"error": str(e)}
    samples, phase, stop = [], ["idle"], [False]

    def sampler():
        while not stop[0]:
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                samples.append((phase[0], m.get("current_socket_power"), m.get("current_gfxclk"),
                                m.get("temperature_hotspot")))
            except Exception:
                pass
            time.sleep(0.05)

    P = ctypes.CDLL(hip_build.PROBE_LIB)
    P.mx_probe_mfma_fp4.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                    ctypes.c_void_p, ctypes.c_void_p]
    P.mx_probe_mfma_fp4.restype = ctypes.c_int32
    sink = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    b, mx = layer.buf, layer.mx

    def wgrad():
        mx.mx_gemm_wgrad(*b["dYt"], 1, *b["Xt"], 1, alpha_exp=layer.alpha["wgrad"], out=layer.dW)

    def probe():
        if P.mx_probe_mfma_fp4(2048, 1000, 0x9E3779B9, sink.data_ptr(), stream) != 0:
            raise SystemExit("mx_probe_mfma_fp4 failed")

    phases = [
        ("wgrad_gemm", wgrad, layer.flops["wgrad"] / 1e12, "TFLOP/s"),
        ("quant_Xq", lambda: layer.quant("Xq", layer.X, 1, layer.fprop_q, "X"),
         layer.quant_bytes("Xq") / 1e9, "GB/s"),
        ("quant_Xt", lambda: layer.quant("Xt", layer.X, 0, layer.wgrad_q, "X"),
         layer.quant_bytes("Xt") / 1e9, "GB/s"),
        ("mfma_probe", probe, 2048 * 4 * 1000 * 16 * 2.0 * 32 * 32 * 64 / 1e12, "TFLOP/s"),
    ]
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    res = {"power_cap": cap, "seconds_per_phase": secs}
    for name, fn, work, unit in phases:
        phase[0] = "idle"
        time.sleep(1.5)
        fn()
        torch.cuda.synchronize()
        phase[0] = name
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < secs:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()
            n += 4
        dt = time.perf_counter() - t0
        phase[0] = "idle"
        res[name] = {"launches": n, "us_per_launch": round(1e6 * dt / n, 1),
                     "rate": round(work * n / dt, 1), "unit": unit}
        print(f"bench: power phase {name} done ({n} launches)", file=sys.stderr, flush=True)
    time.sleep(0.5)
    stop[0] = True
    th.join()
    for name in ["idle"] + [ph[0] for ph in phases]:
        v = [x for x in samples if x[0] == name]
        tail = v if name == "idle" else v[len(v) // 3:]

        def avg(i):
            xs = [x[i] for x in tail if isinstance(x[i], (int, float)) and x[i] != 0xFFFF]
            return round(sum(xs) / len(xs), 1) if xs else None
        res.setdefault(name, {}).update({"samples": len(v), "socket_power_w": avg(1),
                                         "gfxclk_mhz": avg(2), "hotspot_c": avg(3)})
    amdsmi.amdsmi_shut_down()
    return res


def block_variants(mx, wl, torch, reps: int = 5):
    """Outside the timed step: the tile-size variants on the 2-D workload (W 14336x4096, X
    8192x4096, dY 8192x14336, bf16, ceil scale, RNE unless stated): 8x8, 32x32 and 64x64
    quantization with both code layouts, Fprop on W's 32x32 and 64x64 scales against 1x32, Dgrad
    and Wgrad consuming the transposed 32x32 tiles of W and of dY (SR) with no requantization,
    and the 1D scale-mismatch map of X with its summary (the share of elements whose two 1D
    scales differ, and the mean |difference|)."""
    d = wl.blocks_2d(device="cuda")
    X, W = d["X"], d["W"]
    N, K = W.shape
    T = X.shape[0]

    def timed(fn):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        host_ahead(torch)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res = {"blocks_workload": "2-D workload W 14336x4096 and X 8192x4096 bf16, ceil scale, RNE"}
    ops = {}
    for B in (8, 32, 64):
        ops[B] = mx.mx_quantize_2d_blocks(W, block=B, scale_rule=1)
        c, sc, ct, st = ops[B]
        ms = timed(lambda: mx.mx_quantize_2d_blocks(W, block=B, scale_rule=1, codes=c, scales=sc,
                                                    codes_t=ct, scales_t=st))
        sbytes = sum(t.numel() for t in (ops[B][1], ops[B][3]))
        gbs = (N * K * 3 + sbytes) / (ms * 1e-3) / 1e9  # bf16 in, both code layouts, scales
        res[f"quant_2d_{B}x{B}_ms"] = round(ms, 4)
        res[f"quant_2d_{B}x{B}_gbs"] = round(gbs, 1)
    xq, xs = mx.mx_quantize(X, scale_rule=1)
    w1q, w1s = mx.mx_quantize(W, scale_rule=1)
    y = torch.empty((T, N), dtype=torch.bfloat16, device="cuda")
    flops = 2.0 * T * N * K
    for name, (wq, ws, g) in (("1x32", (w1q, w1s, 1)), ("32x32", (ops[32][0], ops[32][1], 32)),
                              ("64x64", (ops[64][0], ops[64][1], 64))):
        ms = timed(lambda: mx.mx_gemm_fprop(xq, xs, 1, wq, ws, g, out=y))
        res[f"fprop_w_{name}_ms"] = round(ms, 4)
        res[f"fprop_w_{name}_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
    # Dgrad and Wgrad on the transposed 32x32 tiles without requantization: dY 8192x14336 in
    # 32x32 tiles with SR, W's transposed tile codes, X 1x32 along T
    dY = d["dY"]
    dc, ds, dct, dst = mx.mx_quantize_2d(dY, scale_rule=1, round=1, seed=wl.SR_SEED + 2)
    ms = timed(lambda: mx.mx_quantize_2d(dY, scale_rule=1, round=1, seed=wl.SR_SEED + 2,
                                         codes=dc, scales=ds, codes_t=dct, scales_t=dst))
    res["quant_2d_dY_sr_ms"] = round(ms, 4)
    res["quant_2d_dY_sr_gbs"] = round((T * N * 3 + ds.numel() + dst.numel()) / (ms * 1e-3) / 1e9, 1)
    xtq, xts = mx.mx_quantize(X, axis=0, scale_rule=1)
    dx = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    dw = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    _, _, wct, wst = ops[32]
    for name, fn in (("dgrad", lambda: mx.mx_gemm_dgrad(dc, ds, 32, wct, wst, 32, out=dx)),
                     ("wgrad", lambda: mx.mx_gemm_wgrad(dct, dst, 32, xtq, xts, 1, out=dw))):
        ms = timed(fn)
        tf = flops / (ms * 1e-3) / 1e12
        res[f"tiles32_{name}_ms"] = round(ms, 4)
        res[f"tiles32_{name}_tflops"] = round(tf, 1)
        res[f"tiles32_{name}_pct_of_fp4_peak"] = round(100.0 * tf / PEAK_FP4_TFLOPS, 2)
    del dc, ds, dct, dst, xtq, xts, dx, dw
    m = mx.mx_scale_mismatch_map(X)
    ms = timed(lambda: mx.mx_scale_mismatch_map(X, out=m))
    res["mismatch_map_ms"] = round(ms, 4)
    res["mismatch_map_gbs"] = round(T * K * 3 / (ms * 1e-3) / 1e9, 1)
    mf = m.float()
    res["mismatch_1d_share_nonzero"] = round(float((m != 0).float().mean()), 4)
    res["mismatch_1d_mean_abs"] = round(float(mf.abs().mean()), 4)
    return res


COPY_BYTES = 1 << 30  # the --copy-calibration copy reads and writes 1 GiB


def counter_values(path: str, counter: str):
    """Per-dispatch values of `counter` from a rocprofv3 counter_collection.csv (summed over the
    hardware instances of each dispatch), as {kernel name: [values in dispatch order]}."""
    import collections
    import csv
    per = collections.defaultdict(float)
    name_of = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        per[d] += float(r["Counter_Value"])
        name_of[d] = r["Kernel_Name"]
    out = collections.defaultdict(list)
    for d in sorted(per):
        out[name_of[d]].append(per[d])
    return out


# the counter passes run 1 warm-up + 2 timed steps, each launching Fprop, Dgrad, Wgrad in turn
TRAFFIC_STEPS = 3
TRAFFIC_ORDER = ("fprop", "dgrad", "wgrad")


def write_traffic(fetch_csv: str, write_csv: str, workload: str):
    """HBM bytes per launch of each GEMM from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each
    scaled by what the same counter reads for the plain 1 GiB copy of the calibration run. The
    GEMM runs on a resident grid (the same workgroup count for every shape), so the launches are
    told apart by their order in the step; the bf16 output bytes each launch writes confirm it."""
    if workload != "llama70b_down":
        raise SystemExit("traffic records are kept for the llama70b_down workload")
    T, K, N = 16384, 28672, 8192  # tokens, FFN (Fprop reduction), hidden
    fetch, write = counter_values(fetch_csv, "FETCH_SIZE"), counter_values(write_csv, "WRITE_SIZE")

    def copy_value(table):
        # the calibration copy is the largest device-to-device copy dispatch of the run
        vals = [v for name, vs in table.items() if "copyBuffer" in name for v in vs]
        if not vals:
            raise SystemExit("no copy kernel in the counter file (run with --copy-calibration)")
        return max(vals)

    ff = COPY_BYTES / (copy_value(fetch) * 1024.0)
    wf = COPY_BYTES / (copy_value(write) * 1024.0)

    def gemm_launches(table):
        # the MXFP4 GEMM with plain output: the ping-pong kernel that serves reductions of a
        # multiple of 1024 (all three of this workload; template arguments A and B formats 4,
        # QOUT false), else the streaming kernel with template arguments ..., QOUT false, A and
        # B formats 4 (not the quantizing epilogue or MXFP8); the step's launches come first
        vals = [vs for name, vs in table.items() if "gemm_mx_pp_kernel<4, 4, false>" in name]
        if not vals:
            vals = [vs for name, vs in table.items()
                    if re.search(r"gemm_mx\w*<[^>]*false, 4, 4>", name)]
        if len(vals) != 1 or len(vals[0]) < 3 * TRAFFIC_STEPS:
            raise SystemExit("expected one MXFP4 GEMM kernel with the step's launches first")
        per = {k: [] for k in TRAFFIC_ORDER}
        for i, v in enumerate(vals[0][:3 * TRAFFIC_STEPS]):
            per[TRAFFIC_ORDER[i % 3]].append(v)
        return per

    shapes = {"fprop": (T, N, K), "dgrad": (T, K, N), "wgrad": (N, K, T)}
    fetch_l, write_l = gemm_launches(fetch), gemm_launches(write)
    for name, (M, Nn, Kk) in shapes.items():
        out_bytes = 2 * M * Nn
        got = sum(write_l[name]) / len(write_l[name]) * 1024.0 * wf
        if abs(got - out_bytes) > 0.08 * out_bytes:  # beyond C: register spill traffic
            raise SystemExit(f"{name}: launch writes {got:.3e} B, expected its bf16 output {out_bytes:.3e} B")
    def command(counter, csv_path):  # the counter pass that wrote csv_path (its -d folder)
        return (f"rocprofv3 --pmc {counter} --output-format csv -d {os.path.dirname(csv_path)} "
                "-o run -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline "
                "--step-only --with-variants --copy-calibration")
    rec = {"gemm_sha": sha(GEMM_SRC), "fetch_factor": ff, "write_factor": wf,
           "command_fetch": command("FETCH_SIZE", fetch_csv),
           "command_write": command("WRITE_SIZE", write_csv)}
    for name, (M, Nn, Kk) in shapes.items():
        fv = sum(fetch_l[name]) / len(fetch_l[name])
        wv = sum(write_l[name]) / len(write_l[name])
        hbm = fv * 1024.0 * ff + wv * 1024.0 * wf
        alg = (M + Nn) * (Kk // 2 + Kk // 32) + 2 * M * Nn  # both operands with scales + bf16 C
        rec[f"{name}_hbm_bytes_per_launch"] = int(round(hbm))
        rec[f"{name}_algorithmic_bytes_per_launch"] = int(alg)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    args = parse()
    if args.write_traffic:
        write_traffic(*args.write_traffic, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py: the path runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding along tokens with a Wgrad all-reduce is a design, not built)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import mxfp4_block_scaled_hadamard32_amd as mx
    import workloads as wl
    mx.lib()
    torch.cuda.set_device(0)
    print(f"bench: generating {args.workload} inputs", file=sys.stderr, flush=True)
    layer = Layer(mx, wl, args.workload)
    torch.cuda.synchronize()
    if args.power:
        layer.step()
        torch.cuda.synchronize()
        rec = power_phases(layer, torch, args.power)
        rec["workload"] = args.workload
        print(json.dumps(rec), flush=True)
        return
    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        a.fill_(1.0)
        c = torch.empty_like(a)
        c.copy_(a)
        torch.cuda.synchronize()
        del a, c
    for _ in range(args.warmup):
        layer.step()
    torch.cuda.synchronize()
    print(f"bench: warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs = timed_steps(layer, torch, args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = 1e3 * elapsed / args.steps
    launches, ms = layer.launch_report(evs)
    wgrad_ms = ms["wgrad"]

    flops = sum(layer.flops.values())
    value = flops / (ms_step * 1e-3) / 1e12
    wgrad_tflops = layer.flops["wgrad"] / (wgrad_ms * 1e-3) / 1e12
    traffic = load_traffic("wgrad_hbm_bytes_per_launch", args.workload)
    ceiling = mfma_ceiling(torch)  # after the timed steps, outside the timed region

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (e2m1 x e2m1 with e8m0 block scales, fp32 accumulate; bf16 in/out)",
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": args.workload, "description": layer.desc, "T": layer.T,
                   "K": layer.K, "N": layer.N, "step": "6 quantizations + Fprop + Dgrad + Wgrad"},
        "components": {
            "wgrad_gemm_ms": round(wgrad_ms, 4),
            "wgrad_gemm_tflops": round(wgrad_tflops, 2),
            "wgrad_pct_of_fp4_peak": round(100.0 * wgrad_tflops / PEAK_FP4_TFLOPS, 2),
            "hadamard_quant_kernel": "all six mx_quantize launches of the step (rows and columns)",
            "hadamard_quant_ms": launches["quant_all6_ms"],
            "hadamard_quant_gbs": launches["quant_all6_gbs"],
            "hadamard_quant_pct_of_hbm_peak": launches["quant_all6_pct_of_hbm_peak"],
            **launches,
        },
        "roofline": {
            "kernel": "gemm_mx_pp_kernel<4, 4, false> (Wgrad launch)",
            "bound": "mfma",
            "achieved": round(wgrad_tflops, 2),
            "peak": PEAK_FP4_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(wgrad_tflops / PEAK_FP4_TFLOPS, 4),
            "traffic": traffic,
            # the same matrix instruction measured on this GPU with random operand bits and no
            # memory traffic (clock falls under that power draw): what the kernel could reach
            "measured_ceiling": round(ceiling, 1),
            "frac_of_measured_ceiling": round(wgrad_tflops / ceiling, 4),
        },
    }
    if not args.step_only:
        out["components"].update(fused_epilogue(layer, torch))
        out["components"].update(linear_layer(layer, torch))
    if not args.step_only or args.with_variants:
        out["components"].update(quant_stream(mx, wl, torch))
        out["components"].update(mxfp8_attention(mx, wl, torch))
        out["components"].update(block_variants(mx, wl, torch))
        if args.workload != "llama8b_up":
            out["components"].update(llama8b_components(mx, wl, torch))
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle beside the step", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(layer, args.cpu_gemm_rows, args.cpu_gemm_elements)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
