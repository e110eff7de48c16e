"""Hardware-counter collection for the attention kernels (run under rocprofv3).

  python -m exact_io_aware_16_amd.counters run
      Launches every hot-path kernel a few times on the measured workloads,
      plus one plain device-to-device copy of a known size (the calibration
      for FETCH_SIZE / WRITE_SIZE).  Meant to be run as
      ``rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR -- python -m
      exact_io_aware_16_amd.counters run`` (one counter group per run).

  python -m exact_io_aware_16_amd.counters summarize --fetch DIR --write DIR
        [--sq DIR] [--stats DIR] [--out profiles]
      Reads the rocprofv3 CSV output, scales FETCH_SIZE and WRITE_SIZE by
      what they read for the copy, and writes profiles/traffic.json (HBM bytes
      per launch, keyed to a digest of the kernel sources) and a markdown
      summary.

The copy moves COPY_BYTES in and COPY_BYTES out; the calibration factor of a
counter is COPY_BYTES / (counter reading for the copy).
"""

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
COPY_BYTES = 512 << 20
REPEAT = 5
# the SQ counter group of the summary (eight SQ counters fit one pass)
SQ_COUNTERS = ("SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES "
               "SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAIT_ANY SQ_WAVE_CYCLES")


def kernel_source_digest():
    """sha256 over the HIP sources; counter figures are tied to it."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def kernel_key(name):
    """Short key for a (possibly mangled) kernel name, or None.  The dropout
    instantiations get their own keys ("_dropout")."""
    b = r"(\d|true|false)"
    m = re.search(r"fwd_bf16_kernel(?:ILi|<)(\d+)(?:ELi|, )(\d+)(?:ELb|, )" + b + r"(?:ELi|, )(\d)"
                  r"(?:(?:ELb|, )" + b + r")?", name)
    if m:
        d, dv, causal, split = m.group(1), m.group(2), m.group(3) in ("1", "true"), m.group(4)
        drop = m.group(5) in ("1", "true")
        return (f"fwd_d{d}" + (f"_dv{dv}" if dv != d else "") + ("_causal" if causal else "")
                + ("_split2" if split == "2" else "") + ("_dropout" if drop else ""))
    m = re.search(r"fwd_r64_kernel(?:ILb|<)" + b + r"(?:ELi|, )(\d)", name)
    if m:
        return "fwd_r64" + ("_causal" if m.group(1) in ("1", "true") else "") + ("_split2" if m.group(2) == "2" else "")
    m = re.search(r"decode_kernel(?:ILi|<)(\d+)(?:ELi|, )(\d)(?:ELb|, )" + b, name)
    if m:
        return f"decode_d{m.group(1)}_rows{m.group(2)}" + ("_causal" if m.group(3) in ("1", "true") else "")
    m = re.search(r"splitkv_merge_kernel(?:ILi|<)(\d+)", name)
    if m:
        return f"splitkv_merge_dv{m.group(1)}"
    for kern, short in (("bwd_dkdv_kernel", "bwd_dkdv"), ("bwd_dq_kernel", "bwd_dq")):
        m = re.search(kern + r"(?:ILi|<)(\d+)(?:ELb|, )" + b + r"(?:(?:ELb|, )" + b + r")?(?:(?:ELb|, )" + b + r")?",
                      name)
        if m:
            causal = m.group(2) in ("1", "true")
            drop = m.group(3) in ("1", "true")
            fused = m.group(4) in ("1", "true")  # the dQ pass with the preprocess fused in (fa_bwd)
            return (f"{short}{'_fused' if fused else ''}_d{m.group(1)}" + ("_causal" if causal else "")
                    + ("_dropout" if drop else ""))
    m = re.search(r"bwd_pre_kernel(?:ILi|<)(\d+)", name)
    if m:
        return f"bwd_pre_d{m.group(1)}"
    m = re.search(r"fwd_f32_kernel(?:ILi|<)(\d+)", name)
    if m:
        return f"fwd_f32_d{m.group(1)}"
    if "copy" in name.lower():
        return "copy"
    return None


def _counted_workloads():
    from exact_io_aware_16_amd import inputs as I

    return (I.FWD_4K_D128, I.FWD_8K_D128, I.CAUSAL_8K_D64_WIDE, I.CAUSAL_32K_D128, I.FWDBWD_4K_D128)


def run():
    import torch

    import exact_io_aware_16_amd as fa
    from exact_io_aware_16_amd import inputs as I

    dev = torch.device("cuda:0")
    # the forward workloads (4k, its 8k double, the wide-score d = 64 one, the
    # 32k one) and the forward+backward workload (every kernel of the step)
    for w in _counted_workloads():
        t = I.make_inputs(w)
        q, k, v = (t[n].to(dev) for n in ("q", "k", "v"))
        reps = REPEAT if w.N <= 8192 else 2
        for _ in range(reps):
            o, lse = fa.forward(q, k, v, causal=w.causal)
        if w.backward:
            do = t["do"].to(dev)
            # fa_bwd (dQ with the preprocess fused in, then dK/dV) and the
            # separate phases (preprocess, dK/dV, dQ)
            for _ in range(REPEAT):
                fa.backward(q, k, v, o, lse, do, causal=w.causal)
            for _ in range(REPEAT):
                ws = fa.backward_prep(o, lse, do, None)
                fa.backward_dkdv(q, k, v, do, ws, causal=w.causal)
                fa.backward_dq(q, k, v, do, ws, causal=w.causal)
        torch.cuda.synchronize()
        del q, k, v, o, lse
        print(f"ran {w.name}", flush=True)
    # the decode workload: one query row per head against 32768 keys
    dc = I.DECODE_32K
    td = I.make_general(dc["B"], dc["H"], dc["Nq"], dc["Nk"], dc["d"], dc["dv"], dc["seed"])
    qd, kd, vd = (td[n].to(dev) for n in ("q", "k", "v"))
    for _ in range(REPEAT):
        fa.forward_splitkv(qd, kd, vd)
    torch.cuda.synchronize()
    print(f"ran {dc['name']}", flush=True)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(REPEAT):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("ran copy", flush=True)


def _read_counter_csv(d):
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        rows += list(csv.DictReader(open(f)))
    return rows


def _per_kernel_mean(rows, counter):
    """Mean counter value per launch, keyed "kernel@workgroups": one kernel
    serves several workloads, and the workgroup count tells them apart."""
    acc = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = kernel_key(r.get("Kernel_Name", ""))
        if key is None:
            continue
        if key != "copy":
            key += "@" + str(int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
        acc.setdefault(key, []).append(float(r["Counter_Value"]))
    # the runtime's small host-to-device copies run the same copy kernel as
    # the calibration copy: calibrate on the large copy's dispatches only
    if "copy" in acc:
        top = max(acc["copy"])
        acc["copy"] = [v for v in acc["copy"] if v >= 0.9 * top]
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _read_stats(d):
    """Per-dispatch durations from the kernel trace, grouped by kernel key and
    workgroup count: one kernel serves several workloads of the bench (the
    step, the padded comparison batch, packed sequences), and only the launches
    of one grid describe one workload."""
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    acc = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = kernel_key(r.get("Kernel_Name", ""))
            if not key:
                continue
            wg = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            ns = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            a = acc.setdefault(f"{key}@{wg}", {"key": key, "workgroups": wg, "calls": 0, "sum_ns": 0.0,
                                                "min_ns": ns, "max_ns": ns})
            a["calls"] += 1
            a["sum_ns"] += ns
            a["min_ns"] = min(a["min_ns"], ns)
            a["max_ns"] = max(a["max_ns"], ns)
    for a in acc.values():
        a["avg_ns"] = a.pop("sum_ns") / a["calls"]
    return acc


def summarize(args):
    fetch = _per_kernel_mean(_read_counter_csv(args.fetch), "FETCH_SIZE")
    write = _per_kernel_mean(_read_counter_csv(args.write), "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("copy calibration kernel not found in counter output")
    f_fetch = COPY_BYTES / (fetch["copy"] * 1024.0)
    f_write = COPY_BYTES / (write["copy"] * 1024.0)
    kernels = {}
    for launch in sorted(set(fetch) & set(write)):
        if launch not in BY_LAUNCH:
            continue
        fb = fetch[launch] * 1024.0 * f_fetch
        wb = write[launch] * 1024.0 * f_write
        kernels[BY_LAUNCH[launch]] = {"launch": launch, "fetch_bytes": fb, "write_bytes": wb,
                                      "hbm_bytes_per_launch": fb + wb, "fetch_kib_raw": fetch[launch],
                                      "write_kib_raw": write[launch]}
    rec = {
        "source_sha256": kernel_source_digest(),
        "calibration": {"copy_bytes_each_way": COPY_BYTES, "fetch_kib_raw": fetch["copy"],
                        "write_kib_raw": write["copy"], "fetch_factor": f_fetch, "write_factor": f_write},
        "kernels": kernels,
    }
    sq = {}
    if args.sq:
        rows = _read_counter_csv(args.sq)
        names = sorted({r["Counter_Name"] for r in rows})
        for n in names:
            for k, v in _per_kernel_mean(rows, n).items():
                if k in BY_LAUNCH:
                    sq.setdefault(BY_LAUNCH[k], {})[n] = v
        rec["sq"] = sq
    if args.stats:
        rec["kernel_stats"] = _read_stats(args.stats)
    os.makedirs(args.out, exist_ok=True)
    json.dump(rec, open(os.path.join(args.out, "traffic.json"), "w"), indent=1, sort_keys=True)
    with open(os.path.join(args.out, "counters_attention_kernels.md"), "w") as f:
        f.write(markdown_counters(rec, args))
    if args.stats:
        with open(os.path.join(args.out, "kernel_trace_bench_workloads.md"), "w") as f:
            f.write(markdown_stats(rec["kernel_stats"], args))
    print(json.dumps(rec, indent=1, sort_keys=True))


def _fwd_bytes(BH, N, d):
    """Q, K, V read once (bf16), O and L written once (float32)."""
    return 3 * BH * N * d * 2 + BH * N * d * 4 + BH * N * 4


_F5 = 2.0 * 32 * 4096 ** 2 * 128  # forward FLOP of B=2 H=16 N=4096 d=128 causal (two products)
# Counted launches: entry -> (kernel key, workgroups of the launch, workload,
# algorithmic HBM bytes per launch, algorithmic FLOP, FLOP the kernel executes).
# Workgroups: 128 query (or key) rows per workgroup; the 4k forward's grid
# (256 of them) takes the 8-wave launch with two key ranges per workgroup;
# 16 rows per workgroup for the preprocess; 16 key ranges x 32 heads for decode.
COUNTED = {
    "fwd_4k": ("fwd_r64_split2", 8 * 32, "B=1 H=8 N=4096 d=128 non-causal",
               _fwd_bytes(8, 4096, 128), 4.0 * 8 * 4096 ** 2 * 128, 4.0 * 8 * 4096 ** 2 * 128),
    "fwd_8k": ("fwd_r64", 8 * 32, "B=1 H=8 N=8192 d=128 non-causal",
               _fwd_bytes(8, 8192, 128), 4.0 * 8 * 8192 ** 2 * 128, 4.0 * 8 * 8192 ** 2 * 128),
    "fwd_8k_d64_wide": ("fwd_d64_causal", 64 * 64, "B=4 H=16 N=8192 d=64 causal, qk std 3",
                        _fwd_bytes(64, 8192, 64), 2.0 * 64 * 8192 ** 2 * 64, 2.0 * 64 * 8192 ** 2 * 64),
    "fwd_32k": ("fwd_r64_causal", 8 * 128, "B=1 H=8 N=32768 d=128 causal",
                _fwd_bytes(8, 32768, 128), 2.0 * 8 * 32768 ** 2 * 128, 2.0 * 8 * 32768 ** 2 * 128),
    "fwd_step": ("fwd_r64_causal", 32 * 16, "B=2 H=16 N=4096 d=128 causal", _fwd_bytes(32, 4096, 128), _F5, _F5),
    # reads dO (bf16), O and L (float32); writes scale*D and L log2(e)
    "bwd_prep": ("bwd_pre_d128", 32 * 4096 // 16, "B=2 H=16 N=4096 d=128",
                 32 * 4096 * 128 * (2 + 4) + 32 * 4096 * 4 * 3, 0.0, 0.0),
    # reads Q, K, V, dO and the two workspace floats per row; writes dK, dV.
    # S, dP, dV, dK: four of the backward's five products
    "bwd_dkdv": ("bwd_dkdv_d128_causal", 32 * 32, "B=2 H=16 N=4096 d=128 causal",
                 4 * 32 * 4096 * 128 * 2 + 32 * 4096 * 8 + 2 * 32 * 4096 * 128 * 4, 2.0 * _F5, 2.0 * _F5),
    # reads Q, K, V, dO and the workspace; writes dQ.  dQ is the fifth product;
    # S and dP are computed a second time (1.5x the forward executed)
    "bwd_dq": ("bwd_dq_d128_causal", 32 * 32, "B=2 H=16 N=4096 d=128 causal",
               4 * 32 * 4096 * 128 * 2 + 32 * 4096 * 8 + 32 * 4096 * 128 * 4, 0.5 * _F5, 1.5 * _F5),
    # fa_bwd's dQ pass: as bwd_dq, plus O and L read to compute the two
    # workspace floats per row itself (written, not read)
    "bwd_dq_fused": ("bwd_dq_fused_d128_causal", 32 * 32, "B=2 H=16 N=4096 d=128 causal",
                     4 * 32 * 4096 * 128 * 2 + 32 * 4096 * 128 * 4 + 32 * 4096 * 4 + 32 * 4096 * 8
                     + 32 * 4096 * 128 * 4, 0.5 * _F5, 1.5 * _F5),
    # decode, 16 key ranges: reads Q, K, V once, writes 16 partial (O, L) per row
    "decode": ("decode_d128_rows1", 32 * 16, "decode B=1 H=32 Nq=1 Nk=32768 d=128",
               32 * 128 * 2 + 2 * 32 * 32768 * 128 * 2 + 16 * 32 * 129 * 4, 0.0, 0.0),
    # reads the 16 partials per row, writes O and L
    "decode_merge": ("splitkv_merge_dv128", 32, "decode B=1 H=32 Nq=1 Nk=32768 d=128",
                     16 * 32 * 129 * 4 + 32 * 129 * 4, 0.0, 0.0),
}
# the same table by "kernel@workgroups" (the key of the counter records)
BY_LAUNCH = {f"{v[0]}@{v[1]}": k for k, v in COUNTED.items()}


def markdown_counters(rec, args):
    cal = rec["calibration"]
    out = ["# Hardware counters of the attention kernels (MI355X)", "",
           "Collected with the committed driver `exact_io_aware_16_amd/counters.py`: a few launches of",
           "each kernel on every measured workload (the forward workloads at N = 4096 and its N = 8192",
           "double, d = 64 wide scores at N = 8192, N = 32768 causal; the forward+backward workload",
           "B=2,H=16,N=4096,d=128 causal; the decode call B=1,H=32, one query row, 32768 keys, d=128),",
           "plus a 512 MiB device copy for calibration, one counter group per run:", "", "```",
           "cd /tmp && export TMPDIR=/tmp PYTHONPATH=$REPO",
           "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o run -- python -u -m exact_io_aware_16_amd.counters run",
           "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o run -- python -u -m exact_io_aware_16_amd.counters run",
           f"rocprofv3 --pmc {SQ_COUNTERS} --output-format csv -d $OUT/pmc_sq -o run -- python -u -m exact_io_aware_16_amd.counters run",
           "python -m exact_io_aware_16_amd.counters summarize --fetch $OUT/pmc_fetch --write $OUT/pmc_write --sq $OUT/pmc_sq --stats $OUT/prof_stats",
           "```", "",
           f"Kernel-source digest: `{rec['source_sha256'][:16]}`.  Launches are told apart by kernel and",
           "workgroup count (one kernel serves several workloads).", "",
           "## HBM traffic per launch", "",
           f"Calibration: the 512 MiB copy reads FETCH_SIZE = {cal['fetch_kib_raw']:.0f} KiB and WRITE_SIZE = "
           f"{cal['write_kib_raw']:.0f} KiB, so the factors are {cal['fetch_factor']:.3f} (fetch) and "
           f"{cal['write_factor']:.3f} (write).", "",
           "| entry | kernel@workgroups | workload | fetch MiB | write MiB | HBM MiB | algorithmic MiB | ratio |",
           "|---|---|---|---|---|---|---|---|"]
    for k in COUNTED:
        v = rec["kernels"].get(k)
        if v is None:
            continue
        _, _, wl, alg, _, _ = COUNTED[k]
        out.append(f"| {k} | {v['launch']} | {wl} | {v['fetch_bytes'] / 2**20:.1f} | {v['write_bytes'] / 2**20:.1f} | "
                   f"{v['hbm_bytes_per_launch'] / 2**20:.1f} | {alg / 2**20:.1f} | "
                   f"{v['hbm_bytes_per_launch'] / alg:.2f} |")
    k4, k8 = rec["kernels"].get("fwd_4k"), rec["kernels"].get("fwd_8k")
    if k4 and k8:
        out += ["", f"N-doubling (8 heads both): {k4['hbm_bytes_per_launch'] / 8 / 2**20:.2f} MiB per head at N = 4096, "
                f"{k8['hbm_bytes_per_launch'] / 8 / 2**20:.2f} MiB per head at N = 8192: "
                f"{k8['hbm_bytes_per_launch'] / k4['hbm_bytes_per_launch']:.2f}x for twice the rows (4x would mean "
                "an N x N term reaches HBM)."]
    if rec.get("sq"):
        out += ["", "## SQ counters per launch (raw sums over the device)", ""]
        names = sorted({n for d in rec["sq"].values() for n in d})
        out.append("| entry | " + " | ".join(names) + " |")
        out.append("|---|" + "---|" * len(names))
        for k in COUNTED:
            d = rec["sq"].get(k)
            if d:
                out.append(f"| {k} | " + " | ".join(f"{d.get(n, 0):.0f}" for n in names) + " |")
        out += ["", "SQ_VALU_MFMA_BUSY_CYCLES counts 32 per 32x32x16 bf16 MFMA summed over all SIMDs;",
                "SQ_VALU_MFMA_COEXEC_CYCLES counts cycles where a vector instruction issued while the matrix",
                "core was busy; SQ_WAIT_ANY / SQ_WAVE_CYCLES (both in quad-cycles) is the share of wave time",
                "spent waiting on dependencies; SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE is the fraction of",
                "LDS cycles lost to conflicts."]
        out += markdown_shares(rec)
    out.append("")
    return "\n".join(out)


NOMINAL_CLOCK_HZ = 2.4e9
SIMDS = 1024  # 256 compute units x 4


def markdown_shares(rec):
    """Shares derived from the SQ sums and each launch's average duration in
    the kernel trace of the bench run."""
    stats = rec.get("kernel_stats") or {}
    rows = []
    for k in COUNTED:
        d, kern = rec["sq"].get(k), rec["kernels"].get(k)
        st = stats.get(kern["launch"]) if kern else None
        if not (d and st):
            continue
        busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        n_mfma = busy / 32.0
        simd_cycles = st["avg_ns"] * 1e-9 * NOMINAL_CLOCK_HZ * SIMDS
        pct = lambda a, b: f"{100.0 * a / b:.1f}%" if b else "—"
        rows.append(f"| {k} | {st['avg_ns'] / 1e3:.1f} | {pct(busy, simd_cycles) if busy else '—'} | "
                    f"{d.get('SQ_INSTS_VALU', 0.0) / n_mfma:.2f} | " if n_mfma else
                    f"| {k} | {st['avg_ns'] / 1e3:.1f} | — | — | ")
        rows[-1] += (f"{pct(d.get('SQ_VALU_MFMA_COEXEC_CYCLES', 0.0), busy) if busy else '—'} | "
                     f"{pct(d.get('SQ_WAIT_ANY', 0.0), d.get('SQ_WAVE_CYCLES', 0.0))} | "
                     f"{pct(d.get('SQ_LDS_BANK_CONFLICT', 0.0), d.get('SQ_LDS_IDX_ACTIVE', 0.0))} |")
    if not rows:
        return []
    return ["", "## Shares per launch", "",
            "From the sums above and the launch's average duration in the kernel trace of the bench run",
            "(`kernel_trace_bench_workloads.md`).  The matrix-core share divides the MFMA-busy cycles by",
            "1024 SIMDs at the nominal 2.4 GHz; under load the chip runs slower (2.05-2.2 GHz on these",
            "boxes), so the share at the real clock is that much higher.  Vector instructions are",
            "SQ_INSTS_VALU per 32x32x16 MFMA (32 busy cycles each); the count includes the MFMAs",
            "themselves (the 64-row forward's loop has 4.5 other vector instructions per MFMA).", "",
            "| entry | avg µs | matrix core busy (2.4 GHz) | vector instr. per MFMA | MFMA-busy cycles with a vector issue | "
            "wave cycles waiting | LDS cycles in bank conflicts |",
            "|---|---|---|---|---|---|---|"] + rows


def markdown_stats(stats, args):
    out = ["# Kernel trace of the bench command (MI355X)", "",
           "```",
           "cd /tmp && export TMPDIR=/tmp",
           "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/prof_stats -o run -- "
           "python -u $REPO/bench.py --no-cpu-baseline --steps 20 --warmup 5",
           "```", "",
           "The bench runs the fwd+bwd step (B=2,H=16,N=4096,d=128 causal) untimed for about a second,",
           "then each of its kernels alone on the same inputs, then the timed steps, then the forward",
           "workloads (B=1,H=8,N=4096,d=128; the float32 tiny check; B=4,H=16,N=8192,d=64 causal;",
           "B=1,H=8,N=32768,d=128 causal; B=1,H=8,N=8192,d=128), the decode workload (B=1, H=32, one",
           "query row, 32768 keys, d=128: decode_d128_rows1 on key ranges across workgroups, then",
           "splitkv_merge_dv128), and the dropout (p = 0.1) and packed-sequence steps, the latter beside",
           "the same batch padded to B=8.  Each workload runs about half a second untimed before it is",
           "timed.  One kernel serves several of these workloads, so launches are grouped by kernel and",
           "workgroup count, taken from the per-dispatch trace.  Algorithmic TFLOP/s counts the",
           "attention products the method needs (forward 2, backward 5); executed TFLOP/s counts what",
           "the kernel runs (the dQ kernel recomputes S and dP).  Both are given for the launch of the",
           "workload named beside them; rows without a workload are the packed batch, its padded copy,",
           "the dropout step and the float32 kernel.", "",
           "| kernel | workgroups | workload | calls | average us | min us | max us | algorithmic TFLOP/s | "
           "executed TFLOP/s |",
           "|---|---|---|---|---|---|---|---|---|"]
    for launch, v in sorted(stats.items(), key=lambda kv: (kv[1]["key"], kv[1]["workgroups"])):
        k = v["key"]
        entry = BY_LAUNCH.get(launch)
        _, _, wl, _, flop, xflop = COUNTED[entry] if entry else ("", 0, "", 0, 0, 0)
        tf = f"{flop / (v['avg_ns'] * 1e-9) / 1e12:.1f}" if flop else ""
        xtf = f"{xflop / (v['avg_ns'] * 1e-9) / 1e12:.1f}" if xflop else ""
        out.append(f"| {k} | {v['workgroups']} | {wl} | {v['calls']} | {v['avg_ns'] / 1e3:.1f} | "
                   f"{v['min_ns'] / 1e3:.1f} | {v['max_ns'] / 1e3:.1f} | {tf} | {xtf} |")
    out.append("")
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    sub.add_parser("run")
    s = sub.add_parser("summarize")
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--sq")
    s.add_argument("--stats")
    s.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    a = ap.parse_args(argv)
    if a.cmd == "run":
        run()
    else:
        summarize(a)


if __name__ == "__main__":
    main()
