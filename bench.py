"""Throughput of the exact-attention hot path on one MI355X.

A step is one pass of the whole path -- fa_fwd then fa_bwd (per-row
preprocess, the key-stationary dK/dV pass, the query-stationary dQ pass) --
over the forward+backward workload
B=2, H=16, N=4096, d=128, causal, bf16 Q/K/V/dO ~ N(0,1), with inputs resident
in device memory before the timed region.  ``value`` is attention TFLOP/s of
the step: 3.5 * (4*B*H*N^2*d / 2) FLOP per step (forward counted as
4*B*H*N^2*d halved for causal, backward as 2.5x the forward).

Also reported on the same line:
  configs    every measured workload (1: float32 tiny check, 2: forward
             B1 H8 N4096 d128, 3: causal forward B4 H16 N8192 d64 with wide
             scores, 4: causal forward B1 H8 N32768 d128, 5: the step), each
             with its time, TFLOP/s, share of the bf16 peak, its roofline
             (counter traffic when current) and the oracle timed on a
             bounded sample of it (cpu_oracle)
  n_doubling the forward workload at N = 4096 and N = 8192: per-head HBM bytes
             from the committed counters (about 2x, not 4x: no N x N tensor
             reaches HBM)
  fwd        the forward workload (2) again, with its roofline
  decode     split-KV forward (fa_fwd_splitkv), one query row per head against
             32768 keys, B=1, H=32, d=dv=128, against the HBM roofline
  dropout    the step's forward and backward with dropout p = 0.1
             (fa_fwd_dropout + fa_bwd_dropout, mask regenerated from the seed)
  varlen     fwd+bwd over 8 packed causal sequences of mixed lengths (H=16,
             d=128; fa_fwd_varlen + fa_bwd_varlen) against the same batch
             padded to the longest sequence in the dense layout
  phases     forward and backward of the step timed separately
  kernels    the forward and the three backward phases, each timed alone
             through its C entry point (fa_fwd, fa_bwd_prep, fa_bwd_dkdv,
             fa_bwd_dq); fa_bwd itself runs the dQ pass with the preprocess
             fused in, then dK/dV (that dQ launch is in the kernel trace)
  roofline   the dominant kernel of the step against the bf16 matrix-core
             peak; traffic from committed rocprofv3 counters when they were
             taken on the current kernel sources
  environment  ROCm version, gfx target, torch version, and the shader clock
             sampled over an untimed run of the same steps just before the
             timed one
  cpu_baseline  the float64 oracle on a bounded sample of the step's workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2048 bf16 FMA/clk (4096 FLOP) x 2.4 GHz, dense
HBM_PEAK_GBS = 8000.0      # HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def committed_traffic(kernel_key):
    """HBM bytes per launch from profiles/traffic.json, if still current."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None, "no counter record"
    rec = json.load(open(path))
    entry = rec.get("kernels", {}).get(kernel_key)
    if entry is None:
        return None, "kernel not in counter record"
    from exact_io_aware_16_amd.counters import kernel_source_digest

    if rec.get("source_sha256") != kernel_source_digest():
        return None, "kernel sources changed since the counters were taken"
    return entry["hbm_bytes_per_launch"], "rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated"


def time_calls(fn, iters, stream):
    """Average ms per call of fn() over iters calls, bracketed by events on the launch stream."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(iters):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / iters


def steady(fn, seconds):
    """Untimed calls of fn() for about `seconds`, one at a time.  After host
    work (input generation) the GPU has idled and its clock has dropped; a
    few warmup calls are too short to bring it back, this is long enough."""
    import torch

    t0 = time.perf_counter()
    for _ in range(100000):
        fn()
        torch.cuda.synchronize()
        if time.perf_counter() - t0 > seconds:
            break


class ClockSampler:
    """Samples the shader clock (MHz) from the driver's DPM table in sysfs
    while it runs (the current level is the starred line of pp_dpm_sclk),
    for the card whose PCI address is torch's device 0."""

    def __init__(self, period_s=0.01):
        import threading

        self.path = self._sclk_path()
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _sclk_path():
        import glob

        try:
            import torch

            bus = torch.cuda.get_device_properties(0).pci_bus_id
        except Exception:
            bus = None
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        for c in cards:
            try:
                slot = [l for l in open(os.path.join(os.path.dirname(c), "uevent")) if l.startswith("PCI_SLOT_NAME=")]
                if bus is not None and slot and int(slot[0].strip().split(":")[-2], 16) == bus:
                    return c
            except (OSError, ValueError):
                continue
        return cards[0] if len(cards) == 1 else None

    def _read(self):
        for line in open(self.path):
            if line.rstrip().endswith("*"):
                mhz = line.split(":")[1].strip().rstrip("*").strip().lower().replace("mhz", "")
                return float(mhz)
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
                if v is not None and v > 200:  # deep-sleep entries are not a running clock
                    self.samples.append(v)
            except (OSError, ValueError):
                pass
            self._stop.wait(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return {"source": self.path or "no pp_dpm_sclk readable", "samples": 0}
        xs = sorted(self.samples)
        return {"source": self.path, "samples": len(xs), "min_mhz": xs[0], "median_mhz": xs[len(xs) // 2],
                "max_mhz": xs[-1]}


def environment(clock):
    import torch

    try:
        rocm = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        rocm = None
    p = torch.cuda.get_device_properties(0)
    return {"rocm": rocm, "gfx": p.gcnArchName, "device": p.name, "compute_units": p.multi_processor_count,
            "torch": torch.__version__, "sclk_during_untimed_steps": clock.summary()}


def cpu_oracle_forward(w, t, rows_per_head=None, budget_s=5.0):
    """The oracle's forward (untuned) on whole heads of a forward workload
    until ~budget_s of work; rows_per_head limits each head to a seeded
    sample of rows (the long workload).  GFLOP/s counts the sample's share
    of the workload's forward FLOP."""
    from threadpoolctl import threadpool_info

    import oracle
    from exact_io_aware_16_amd.inputs import sample_rows, to_f64

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = rows = 0
    t0 = time.perf_counter()
    for b, h in heads:
        r = None if rows_per_head is None else sample_rows(w.N, rows_per_head, 1000 * w.case + b * w.H + h)
        oracle.attention_forward(*(to_f64(t[n][b, h]) for n in ("q", "k", "v")), w.scale, w.causal, rows=r)
        done += 1
        rows += w.N if r is None else len(r)
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    # FLOP of the rows evaluated: the full-row FLOP per row scaled by the rows
    flop = w.fwd_flop() * rows / (w.B * w.H * w.N)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    what = "full rows" if rows_per_head is None else f"{rows_per_head} seeded rows per head"
    return {"seconds": round(el, 3), "gflops": round(flop / el / 1e9, 2), "cores": threads, "kind": "oracle",
            "sample": f"{done} of {len(heads)} heads, {what}, float64 forward"}


def cpu_baseline(w, t, budget_s=12.0):
    """The oracle (untuned) on whole heads of the workload until ~budget_s of work."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from exact_io_aware_16_amd.inputs import to_f64

    f64 = {n: to_f64(t[n]) for n in ("q", "k", "v", "do")}
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, t0 = 0, time.perf_counter()
    for b, h in heads:
        oracle.attention_forward(f64["q"][b, h], f64["k"][b, h], f64["v"][b, h], w.scale, w.causal)
        oracle.attention_backward(f64["q"][b, h], f64["k"][b, h], f64["v"][b, h], f64["do"][b, h], w.scale, w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    flop = 3.5 * w.fwd_flop() * done / len(heads)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {
        "value": flop / el / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} heads of the step's workload, full rows, float64 forward + backward "
                  f"({el:.1f} s); FLOP counted as for the GPU step",
        "seconds": el,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this attention path has no multi-GPU mode "
              "(heads and batch shard across GPUs with no exchange between them). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_io_aware_16_amd as fa
    from exact_io_aware_16_amd import inputs as I

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    # ------------------------------------------------------------ the step: fwd + bwd
    w = I.FWDBWD_4K_D128
    t = I.make_inputs(w)
    q, k, v, do = (t[n].to(dev) for n in ("q", "k", "v", "do"))
    B, H, N, d = q.shape
    o = torch.empty((B, H, N, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ws = torch.empty((fa.library().fa_bwd_workspace_bytes(B, H, N, d),), dtype=torch.uint8, device=dev)

    def fwd():
        fa.forward(q, k, v, causal=True, out=o, lse=lse)

    def bwd():
        fa.backward(q, k, v, o, lse, do, causal=True, workspace=ws)

    def step():
        fwd()
        bwd()

    # untimed: about a second of steps brings the GPU to its steady clock, so
    # that neither the parts nor the step below are timed during the ramp
    steady(step, 1.0)

    # the forward and each backward phase alone (workspace prepared once for
    # the two passes); fa_bwd runs dQ with the preprocess fused in, then dK/dV
    dq_o, dk_o, dv_o = (torch.empty_like(o) for _ in range(3))
    fa.backward_prep(o, lse, do, ws)
    torch.cuda.synchronize()
    F = w.fwd_flop()
    kernels = {
        # name: (call, counter key, algorithmic FLOP, executed FLOP)
        "fa_fwd": (fwd, "fwd_step", F, F),
        "fa_bwd_prep": (lambda: fa.backward_prep(o, lse, do, ws), "bwd_prep", 0.0, 0.0),
        "fa_bwd_dkdv": (lambda: fa.backward_dkdv(q, k, v, do, ws, causal=True, dk=dk_o, dv=dv_o),
                        "bwd_dkdv", 2.0 * F, 2.0 * F),
        "fa_bwd_dq": (lambda: fa.backward_dq(q, k, v, do, ws, causal=True, dq=dq_o),
                      "bwd_dq", 0.5 * F, 1.5 * F),
    }
    kern = {}
    for name, (fn, key, flop, xflop) in kernels.items():
        for _ in range(3):
            fn()
        ms_k = time_calls(fn, args.steps, stream)
        kern[name] = {"ms": round(ms_k, 4), "counter_key": key,
                      "algorithmic_tflops": round(flop / (ms_k * 1e-3) / 1e12, 2) if flop else None,
                      "executed_tflops": round(xflop / (ms_k * 1e-3) / 1e12, 2) if xflop else None}
    # the shader clock is sampled over an untimed run of the same steps just
    # before the timed one: reading it from sysfs while steps run has measured
    # 0.3-1% slower per step, and about 1.5 ms slower in total on the first
    # run after the sampler starts, so no read happens in the timed region
    with ClockSampler() as clock:
        for _ in range(args.warmup + args.steps):
            step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly --steps steps, synchronised on both sides
    t_start = time.perf_counter()
    ms_step = time_calls(step, args.steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_flop = 3.5 * w.fwd_flop()
    value = step_flop / (ms_step * 1e-3) / 1e12

    ms_fwd = time_calls(fwd, args.steps, stream)
    ms_bwd = time_calls(bwd, args.steps, stream)
    bwd_tflops = 2.5 * w.fwd_flop() / (ms_bwd * 1e-3) / 1e12

    dom = max(kern, key=lambda n: kern[n]["ms"])
    dom_flop = kernels[dom][2]
    dom_ach = dom_flop / (kern[dom]["ms"] * 1e-3) / 1e12
    traffic, traffic_src = committed_traffic(kern[dom]["counter_key"])

    # ------------------------------------------------------------ forward headline workload
    wf = I.FWD_4K_D128
    tf = I.make_inputs(wf)
    qf, kf, vf = (tf[n].to(dev) for n in ("q", "k", "v"))
    of = torch.empty(qf.shape, dtype=torch.float32, device=dev)
    lf = torch.empty(qf.shape[:3], dtype=torch.float32, device=dev)

    def fwd2():
        fa.forward(qf, kf, vf, causal=False, out=of, lse=lf)

    steady(fwd2, 0.5)
    for _ in range(args.warmup):
        fwd2()
    ms_f2 = time_calls(fwd2, args.steps, stream)
    f2 = wf.fwd_flop() / (ms_f2 * 1e-3) / 1e12
    f2_traffic, f2_src = committed_traffic("fwd_4k")

    # ------------------------------------------------------------ the other forward workloads
    def time_forward(wl, seconds=0.5):
        """Steady-state ms per forward call of workload wl (inputs resident)."""
        tw = I.make_inputs(wl)
        qw, kw, vw = (tw[n].to(dev) for n in ("q", "k", "v"))
        ow = torch.empty((wl.B, wl.H, wl.N, wl.d), dtype=torch.float32, device=dev)
        lw = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device=dev)

        def call():
            fa.forward(qw, kw, vw, causal=wl.causal, out=ow, lse=lw)

        steady(call, seconds)
        for _ in range(args.warmup):
            call()
        ms_w = time_calls(call, args.steps, stream)
        del qw, kw, vw, ow, lw
        return tw, ms_w

    def roofline(flop, ms_w, entry, kernel):
        tr, src = committed_traffic(entry)
        ach = flop / (ms_w * 1e-3) / 1e12
        return {"kernel": kernel, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": tr,
                "traffic_source": src, "algorithmic_flop_per_launch": flop}

    cfg = {}
    t1, ms1 = time_forward(I.TINY_F32)
    cfg["1"] = {"workload": I.TINY_F32.name, "ms": round(ms1, 4),
                "tflops": round(I.TINY_F32.fwd_flop() / (ms1 * 1e-3) / 1e12, 3),
                "bound": "latency (one workgroup per 64 rows; not a roofline case)", "dtype": "f32"}
    cfg["2"] = {"workload": wf.name, "ms": round(ms_f2, 4), "tflops": round(f2, 2),
                "pct_of_peak": round(100 * f2 / PEAK_BF16_TFLOPS, 2),
                "roofline": roofline(wf.fwd_flop(), ms_f2, "fwd_4k",
                                     "fwd_r64_kernel<non-causal, two key ranges per workgroup> (the launch this grid gets)")}
    for key, wl, entry, kname in (("3", I.CAUSAL_8K_D64_WIDE, "fwd_8k_d64_wide", "fwd_bf16_kernel<64, causal>"),
                                  ("4", I.CAUSAL_32K_D128, "fwd_32k", "fwd_r64_kernel<causal>")):
        tw, ms_w = time_forward(wl)
        tfw = wl.fwd_flop() / (ms_w * 1e-3) / 1e12
        cfg[key] = {"workload": wl.name, "ms": round(ms_w, 4), "tflops": round(tfw, 2),
                    "pct_of_peak": round(100 * tfw / PEAK_BF16_TFLOPS, 2),
                    "roofline": roofline(wl.fwd_flop(), ms_w, entry, kname)}
        cfg[key]["_inputs"] = tw
    cfg["5"] = {"workload": w.name, "step_ms": round(ms_step, 4), "step_tflops": round(value, 2),
                "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2), "fwd_ms": None, "bwd_ms": None}
    # the N-doubling check: the forward workload at twice the rows
    _, ms_8k = time_forward(I.FWD_8K_D128)
    dbl = {"workloads": [wf.name, I.FWD_8K_D128.name], "ms": [round(ms_f2, 4), round(ms_8k, 4)]}
    b4, src4 = committed_traffic("fwd_4k")
    b8, _ = committed_traffic("fwd_8k")
    if b4 is not None and b8 is not None:
        heads = wf.B * wf.H
        dbl.update({"hbm_bytes_per_head": [round(b4 / heads), round(b8 / heads)], "ratio": round(b8 / b4, 3),
                    "materialised_score_bytes_per_head": [wf.N ** 2 * 4, I.FWD_8K_D128.N ** 2 * 4],
                    "traffic_source": src4})
    else:
        dbl.update({"hbm_bytes_per_head": None, "ratio": None, "traffic_source": src4})

    # ------------------------------------------------------------ decode (split-KV across workgroups)
    dc = I.DECODE_32K
    td = I.make_general(dc["B"], dc["H"], dc["Nq"], dc["Nk"], dc["d"], dc["dv"], dc["seed"])
    qd, kd, vd = (td[n].to(dev) for n in ("q", "k", "v"))
    od = torch.empty((dc["B"], dc["H"], dc["Nq"], dc["dv"]), dtype=torch.float32, device=dev)
    ld = torch.empty((dc["B"], dc["H"], dc["Nq"]), dtype=torch.float32, device=dev)
    wsd = torch.empty((max(4, fa.library().fa_fwd_splitkv_workspace_bytes(
        dc["B"], dc["H"], dc["Nq"], dc["Nk"], dc["d"], dc["dv"], 0)),), dtype=torch.uint8, device=dev)

    def dec():
        fa.forward_splitkv(qd, kd, vd, workspace=wsd, out=od, lse=ld)

    steady(dec, 0.5)
    for _ in range(args.warmup):
        dec()
    ms_dec = time_calls(dec, args.steps, stream)
    bh = dc["B"] * dc["H"]
    dec_bytes = (bh * dc["Nq"] * dc["d"] * 2 + bh * dc["Nk"] * (dc["d"] + dc["dv"]) * 2
                 + bh * dc["Nq"] * (dc["dv"] + 1) * 4)
    dec_gbs = dec_bytes / (ms_dec * 1e-3) / 1e9
    # measured HBM bytes of the call: the key-range kernel and the merge
    t_dec, dec_src = committed_traffic("decode")
    t_mrg, _ = committed_traffic("decode_merge")
    dec_traffic = t_dec + t_mrg if t_dec is not None and t_mrg is not None else None

    # ------------------------------------------------------------ the step with dropout
    def step_drop():
        fa.forward_dropout(q, k, v, 0.1, 2024, 0, causal=True, out=o, lse=lse)
        fa.backward_dropout(q, k, v, o, lse, do, 0.1, 2024, 0, causal=True, workspace=ws)

    def fwd_drop():
        fa.forward_dropout(q, k, v, 0.1, 2024, 0, causal=True, out=o, lse=lse)

    steady(step_drop, 0.5)
    ms_drop = time_calls(step_drop, args.steps, stream)
    ms_drop_fwd = time_calls(fwd_drop, args.steps, stream)

    # ------------------------------------------------------------ packed variable-length batch
    lens = [4096, 3000, 2048, 1500, 1024, 700, 512, 300]
    Hv, dv_ = 16, 128
    total = sum(lens)
    gv = torch.Generator("cpu").manual_seed(7)
    qv, kv, vv, dov = (torch.randn((Hv, total, dv_), generator=gv).to(torch.bfloat16).to(dev) for _ in range(4))
    cu = torch.tensor([0] + list(__import__("itertools").accumulate(lens)), dtype=torch.int32, device=dev)
    ov = torch.empty((Hv, total, dv_), dtype=torch.float32, device=dev)
    lv = torch.empty((Hv, total), dtype=torch.float32, device=dev)
    wsv = torch.empty((fa.library().fa_bwd_workspace_bytes(1, Hv, total, dv_),), dtype=torch.uint8, device=dev)

    def step_var():
        fa.forward_varlen(qv, kv, vv, cu, max(lens), causal=True, out=ov, lse=lv)
        fa.backward_varlen(qv, kv, vv, ov, lv, dov, cu, max(lens), causal=True, workspace=wsv)

    Np = max(lens)  # the same batch padded to the longest sequence, dense layout
    qp, kp, vp, dop = (torch.zeros((len(lens), Hv, Np, dv_), dtype=torch.bfloat16, device=dev) for _ in range(4))
    op = torch.empty((len(lens), Hv, Np, dv_), dtype=torch.float32, device=dev)
    lp = torch.empty((len(lens), Hv, Np), dtype=torch.float32, device=dev)
    wsp = torch.empty((fa.library().fa_bwd_workspace_bytes(len(lens), Hv, Np, dv_),), dtype=torch.uint8, device=dev)

    def step_pad():
        fa.forward(qp, kp, vp, causal=True, out=op, lse=lp)
        fa.backward(qp, kp, vp, op, lp, dop, causal=True, workspace=wsp)

    steady(step_var, 0.5)
    ms_var = time_calls(step_var, args.steps, stream)
    steady(step_pad, 0.5)
    ms_pad = time_calls(step_pad, args.steps, stream)
    var_flop = 3.5 * sum(4.0 * Hv * L * L * dv_ / 2 for L in lens)

    res = {
        "metric": "attention TFLOP/s (fwd, fwd+bwd) bf16 at 1 MI355X; % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": w.causal,
            "step": "fa_fwd + fa_bwd",
            "flop_per_step": step_flop,
            "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
            "parallelism": "single GPU",
        },
        "phases": {
            "fwd_ms": round(ms_fwd, 4),
            "fwd_tflops": round(w.fwd_flop() / (ms_fwd * 1e-3) / 1e12, 2),
            "bwd_ms": round(ms_bwd, 4),
            "bwd_tflops": round(bwd_tflops, 2),
        },
        "kernels": kern,
        "roofline": {
            "kernel": f"{dom} ({kern[dom]['counter_key']}), timed alone with HIP events on its launch stream",
            "bound": "mfma",
            "achieved": round(dom_ach, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(dom_ach / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "traffic_source": traffic_src,
            "algorithmic_flop_per_launch": dom_flop,
        },
        "fwd": {
            "workload": wf.name,
            "ms": round(ms_f2, 4),
            "tflops": round(f2, 2),
            "roofline": {
                "kernel": "fwd_r64_kernel<non-causal, two key ranges per workgroup> (the launch this grid gets)",
                "bound": "mfma",
                "achieved": round(f2, 2),
                "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(f2 / PEAK_BF16_TFLOPS, 4),
                "traffic": f2_traffic,
                "traffic_source": f2_src,
                "algorithmic_flop_per_launch": wf.fwd_flop(),
            },
        },
        "decode": {
            "workload": dc["name"],
            "ms": round(ms_dec, 4),
            "roofline": {
                "kernel": "decode_kernel (key ranges across workgroups, vector ALUs) + splitkv_merge_kernel (the fa_fwd_splitkv call)",
                "bound": "hbm",
                "achieved": round(dec_gbs, 1),
                "peak": HBM_PEAK_GBS,
                "unit": "GB/s",
                "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                "traffic": dec_traffic,
                "traffic_source": dec_src,
                "algorithmic_bytes_per_call": dec_bytes,
            },
        },
        "dropout": {
            "workload": w.name + "_dropout0.1",
            "step_ms": round(ms_drop, 4),
            "step_tflops": round(step_flop / (ms_drop * 1e-3) / 1e12, 2),
            "fwd_ms": round(ms_drop_fwd, 4),
            "fwd_tflops": round(w.fwd_flop() / (ms_drop_fwd * 1e-3) / 1e12, 2),
            "flop_convention": "same FLOP as the step without dropout",
        },
        "varlen": {
            "workload": "varlen_bf16_causal_h16d128_lens" + "-".join(map(str, lens)),
            "step_ms": round(ms_var, 4),
            "step_tflops": round(var_flop / (ms_var * 1e-3) / 1e12, 2),
            "padded_dense_step_ms": round(ms_pad, 4),
            "speedup_over_padding": round(ms_pad / ms_var, 3),
            "flop_convention": "attention FLOP of the real (unpadded) sequences, 3.5x the causal forward",
        },
        "timed_wall_s": round(wall, 3),
    }
    cfg["5"]["fwd_ms"], cfg["5"]["bwd_ms"] = res["phases"]["fwd_ms"], res["phases"]["bwd_ms"]
    cfg["5"]["fwd_tflops"], cfg["5"]["bwd_tflops"] = res["phases"]["fwd_tflops"], res["phases"]["bwd_tflops"]
    cfg["5"]["roofline"] = res["roofline"]
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, t)
        cfg["1"]["cpu_oracle"] = cpu_oracle_forward(I.TINY_F32, t1, budget_s=1.0)
        cfg["2"]["cpu_oracle"] = cpu_oracle_forward(wf, tf, budget_s=4.0)
        cfg["3"]["cpu_oracle"] = cpu_oracle_forward(I.CAUSAL_8K_D64_WIDE, cfg["3"]["_inputs"], budget_s=4.0)
        cfg["4"]["cpu_oracle"] = cpu_oracle_forward(I.CAUSAL_32K_D128, cfg["4"]["_inputs"], rows_per_head=256,
                                                    budget_s=4.0)
        cb = res["cpu_baseline"]
        cfg["5"]["cpu_oracle"] = {"seconds": round(cb["seconds"], 3), "gflops": round(cb["value"] * 1e3, 2),
                                  "cores": cb["cores"], "kind": "oracle", "sample": cb["sample"]}
    for c in cfg.values():
        c.pop("_inputs", None)
    res["configs"] = cfg
    res["n_doubling"] = dbl
    res["environment"] = environment(clock)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
