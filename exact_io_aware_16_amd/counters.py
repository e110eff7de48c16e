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
    """Short key for a (possibly mangled) kernel name, or None."""
    m = re.search(r"fwd_bf16_kernel(?:ILi|<)(\d+)(?:ELb|, )(\d|true|false)", name)
    if m:
        causal = m.group(2) in ("1", "true")
        return f"fwd_d{m.group(1)}" + ("_causal" if causal else "")
    m = re.search(r"bwd_main_kernel(?:ILi|<)(\d+)(?:ELb|, )(\d|true|false)", name)
    if m:
        causal = m.group(2) in ("1", "true")
        return f"bwd_main_d{m.group(1)}" + ("_causal" if causal else "")
    m = re.search(r"bwd_pre_kernel(?:ILi|<)(\d+)", name)
    if m:
        return f"bwd_pre_d{m.group(1)}"
    m = re.search(r"fwd_f32_kernel(?:ILi|<)(\d+)", name)
    if m:
        return f"fwd_f32_d{m.group(1)}"
    if "copy" in name.lower() or "elementwise" in name.lower():
        return "copy"
    return None


def run():
    import torch

    import exact_io_aware_16_amd as fa
    from exact_io_aware_16_amd import inputs as I

    dev = torch.device("cuda:0")
    for w in (I.FWD_4K_D128, I.FWDBWD_4K_D128):
        t = I.make_inputs(w)
        q, k, v = (t[n].to(dev) for n in ("q", "k", "v"))
        for _ in range(REPEAT):
            o, lse = fa.forward(q, k, v, causal=w.causal)
        if w.backward:
            do = t["do"].to(dev)
            for _ in range(REPEAT):
                fa.backward(q, k, v, o, lse, do, causal=w.causal)
        torch.cuda.synchronize()
        print(f"ran {w.name}", flush=True)
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
    acc = {}
    for r in rows:
        if r.get("Counter_Name") != counter:
            continue
        key = kernel_key(r.get("Kernel_Name", ""))
        if key is None:
            continue
        acc.setdefault(key, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _read_stats(d):
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    out = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = kernel_key(r.get("Name", ""))
            if key:
                out[key] = {"calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                            "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"])}
    return out


def summarize(args):
    fetch = _per_kernel_mean(_read_counter_csv(args.fetch), "FETCH_SIZE")
    write = _per_kernel_mean(_read_counter_csv(args.write), "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise SystemExit("copy calibration kernel not found in counter output")
    f_fetch = COPY_BYTES / (fetch["copy"] * 1024.0)
    f_write = COPY_BYTES / (write["copy"] * 1024.0)
    kernels = {}
    for key in sorted(set(fetch) & set(write)):
        if key == "copy":
            continue
        fb = fetch[key] * 1024.0 * f_fetch
        wb = write[key] * 1024.0 * f_write
        kernels[key] = {"fetch_bytes": fb, "write_bytes": wb, "hbm_bytes_per_launch": fb + wb,
                        "fetch_kib_raw": fetch[key], "write_kib_raw": write[key]}
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
                sq.setdefault(k, {})[n] = v
        rec["sq"] = sq
    if args.stats:
        rec["kernel_stats"] = _read_stats(args.stats)
    os.makedirs(args.out, exist_ok=True)
    json.dump(rec, open(os.path.join(args.out, "traffic.json"), "w"), indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1, sort_keys=True))


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
