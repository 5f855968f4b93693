"""Summaries of rocprofv3 CSV output for the profiles/ directory.

    python -m block_sparse_attention_poem_amd.rocprof_summary kernels  <dir> <title> <command>
    python -m block_sparse_attention_poem_amd.rocprof_summary counters <dir> <title> <command>
    python -m block_sparse_attention_poem_amd.rocprof_summary traffic  <fetch_dir> <write_dir> <copy_fetch_dir>
                                                                       <copy_write_dir> <copy_bytes> <title> <out.json>
                                                                       <command>
    python -m block_sparse_attention_poem_amd.rocprof_summary selector <kernels_dir> <fetch_dir> <l2_dir>
                                                                       <copy_fetch_dir> <copy_bytes> <out.json> <command>

kernels:  per-kernel calls and average / min / max duration from --kernel-trace --stats.
counters: the last dispatch of each kernel from a --pmc run, one column per counter.
traffic:  bytes from beyond L2 per dispatch: FETCH_SIZE and WRITE_SIZE (KiB) scaled by
          what the same counters read for a plain device copy of known size.
selector: per selector sweep, the scaled FETCH bytes, the L2 hit rate and the average
          duration, keyed by a hash of the selector sources (the benchmark reports them
          only while the sources still match).
Markdown goes to stdout; JSON records to the named file.
"""
import csv
import glob
import hashlib
import json
import os
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))


def _files(d, suffix):
    out = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not out:
        raise SystemExit(f"no *{suffix} under {d}")
    return out


def kernel_stats(d):
    rows = []
    for f in _files(d, "kernel_stats.csv"):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    out = []
    for r in rows:
        out.append(dict(name=r["Name"], calls=int(r["Calls"]), avg_us=float(r["AverageNs"]) / 1e3,
                        min_us=float(r["MinNs"]) / 1e3, max_us=float(r["MaxNs"]) / 1e3,
                        share=float(r["Percentage"])))
    return sorted(out, key=lambda x: -x["share"])


def last_dispatch_counters(d):
    """{kernel: {counter: value}} from the last dispatch of each kernel (summed over the
    counter's instances); also {kernel: duration_ns} of that dispatch."""
    per = defaultdict(lambda: defaultdict(float))
    dur = {}
    last = {}
    for f in _files(d, "counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                disp = int(r["Dispatch_Id"])
                if disp > last.get(name, -1):
                    last[name] = disp
                    per[name] = defaultdict(float)
                if disp == last[name]:
                    per[name][r["Counter_Name"]] += float(r["Counter_Value"])
                    if "End_Timestamp" in r and r.get("Start_Timestamp"):
                        dur[name] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    return per, dur


def cmd_kernels(d, title, command):
    print(f"# rocprofv3 kernel trace: {title}\n\ncommand: {command}\n")
    print("kernel | calls | avg_us | min_us | max_us | share\n---|---|---|---|---|---")
    for k in kernel_stats(d):
        print(f"{k['name']} | {k['calls']} | {k['avg_us']:.1f} | {k['min_us']:.1f} | {k['max_us']:.1f} | "
              f"{k['share']:.2f}%")


SIMDS = 1024  # 256 CUs x 4 SIMDs
XCDS = 8      # GRBM_GUI_ACTIVE sums the XCDs' busy cycles


def derived(v, dur_ns):
    """From one dispatch's SQ/GRBM counters: elapsed cycles (GRBM_GUI_ACTIVE / 8), clock
    (elapsed cycles / the dispatch's own duration), MFMA FLOP (512 per MOPS unit), MFMA
    busy share (SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x elapsed cycles))."""
    out = {}
    el = v.get("GRBM_GUI_ACTIVE", 0.0) / XCDS
    if el > 0:
        out["elapsed cycles"] = f"{el:.4g}"
        if dur_ns > 0:
            out["clock GHz"] = f"{el / dur_ns:.2f}"
        if "SQ_VALU_MFMA_BUSY_CYCLES" in v:
            out["MFMA busy"] = f"{100.0 * v['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * el):.1f}%"
    mops = sum(x for c, x in v.items() if c.startswith("SQ_INSTS_VALU_MFMA_MOPS_"))
    if mops > 0:
        out["MFMA FLOP"] = f"{512.0 * mops:.4g}"
        if dur_ns > 0:
            out["MFMA TFLOP/s"] = f"{512.0 * mops / dur_ns / 1e3:.0f}"
    return out


def cmd_counters(d, title, command):
    per, dur = last_dispatch_counters(d)
    names = sorted({c for v in per.values() for c in v})
    der = {k: derived(v, dur.get(k, 0.0)) for k, v in per.items()}
    dnames = [n for n in ("MFMA FLOP", "MFMA TFLOP/s", "elapsed cycles", "MFMA busy", "clock GHz")
              if any(n in x for x in der.values())]
    print(f"# rocprofv3 counters: {title}\n\ncommand: {command}\n\nThe last dispatch of each kernel "
          f"(counters serialize the dispatches). Derived: elapsed cycles = GRBM_GUI_ACTIVE / {XCDS}; clock = "
          f"elapsed cycles / dispatch duration; MFMA FLOP = 512 x MOPS; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
          f"({SIMDS} SIMDs x elapsed cycles).\n")
    cols = ["dispatch_us"] + dnames + names
    print("kernel | " + " | ".join(cols) + "\n" + "---|" * (len(cols) + 1))
    for k, v in per.items():
        vals = [f"{dur.get(k, 0) / 1e3:.1f}"] + [der[k].get(n, "") for n in dnames] + [f"{v.get(c, 0):.4g}" for c in names]
        print(f"{k} | " + " | ".join(vals))


def _copy_factor(d, counter, nbytes):
    per, _ = last_dispatch_counters(d)
    vals = [v[counter] for v in per.values() if counter in v]
    kib = max(vals)
    return nbytes / (kib * 1024.0), kib


def cmd_traffic(fd, wd, cfd, cwd, copy_bytes, title, out_json, command):
    copy_bytes = int(copy_bytes)
    sf, fk = _copy_factor(cfd, "FETCH_SIZE", copy_bytes)
    sw, wk = _copy_factor(cwd, "WRITE_SIZE", copy_bytes)
    fe, _ = last_dispatch_counters(fd)
    wr, _ = last_dispatch_counters(wd)
    src = b"".join(open(os.path.join(PKG, "csrc", f), "rb").read()
                   for f in ("poem_device.hpp", "poem_internal.hpp", "attn_fwd.hip"))
    rec = {"title": title, "command": command, "scale_fetch": sf, "scale_write": sw, "copy_probe_bytes": copy_bytes,
           "attn_source_sha256": hashlib.sha256(src).hexdigest(), "kernels": {}}
    print(f"# HBM traffic per dispatch (beyond L2): {title}\n\ncommand: {command} (one counter per run)\n")
    print(f"calibration: a plain device copy of {copy_bytes} bytes reads FETCH_SIZE {fk:.6g} KiB and WRITE_SIZE "
          f"{wk:.6g} KiB -> fetch x{sf:.3f}, write x{sw:.3f}\n")
    print("kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read GB | scaled write GB\n---|---|---|---|---")
    for k in fe:
        f = fe[k].get("FETCH_SIZE", 0.0)
        w = wr.get(k, {}).get("WRITE_SIZE", 0.0)
        rec["kernels"][k] = {"fetch_kib": f, "write_kib": w, "read_bytes": f * 1024 * sf, "write_bytes": w * 1024 * sw}
        print(f"{k} | {f:.4g} | {w:.4g} | {f * 1024 * sf / 1e9:.2f} | {w * 1024 * sw / 1e9:.3f}")
    json.dump(rec, open(out_json, "w"), indent=1)


def cmd_selector(kd, fd, ld, cfd, copy_bytes, out_json, command):
    copy_bytes = int(copy_bytes)
    sf, _ = _copy_factor(cfd, "FETCH_SIZE", copy_bytes)
    ks = {k["name"]: k for k in kernel_stats(kd)}
    fe, _ = last_dispatch_counters(fd)
    l2, _ = last_dispatch_counters(ld)
    src = b"".join(open(os.path.join(PKG, "csrc", f), "rb").read()
                   for f in ("poem_device.hpp", "poem_internal.hpp", "selector.hip"))
    rec = {"command": command, "selector_source_sha256": hashlib.sha256(src).hexdigest(), "sweeps": {}}
    print(f"# selector sweeps: bytes from beyond L2 and L2 hit rate\n\ncommand: {command}\n")
    print("sweep | avg_us | read GB (scaled FETCH_SIZE) | GB/s | L2 hit rate\n---|---|---|---|---")
    for k, v in fe.items():
        if "sel_sweep_kernel" not in k:
            continue
        rb = v.get("FETCH_SIZE", 0.0) * 1024 * sf
        us = ks.get(k, {}).get("avg_us", float("nan"))
        c = l2.get(k, {})
        hit = [c[n] for n in c if "HIT" in n]
        miss = [c[n] for n in c if "MISS" in n]
        rate = sum(hit) / (sum(hit) + sum(miss)) if hit and miss and sum(hit) + sum(miss) > 0 else None
        rec["sweeps"][k] = {"read_bytes": rb, "avg_us": us, "read_gbs": rb / (us * 1e-6) / 1e9, "l2_hit_rate": rate}
        print(f"{k} | {us:.1f} | {rb / 1e9:.2f} | {rb / (us * 1e-6) / 1e9:.0f} | "
              f"{'%.3f' % rate if rate is not None else 'n/a'}")
    json.dump(rec, open(out_json, "w"), indent=1)


if __name__ == "__main__":
    cmd, rest = sys.argv[1], sys.argv[2:]
    {"kernels": cmd_kernels, "counters": cmd_counters, "traffic": cmd_traffic, "selector": cmd_selector}[cmd](*rest)
