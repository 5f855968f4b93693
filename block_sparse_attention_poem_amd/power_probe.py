"""Socket power and graphics clock while one kernel of the path runs back to back.

    python3 -m block_sparse_attention_poem_amd.power_probe [--workload 3] [--seconds 8]

Phases of a few seconds each: idle, the selector (poem_select), the sparse attention
(poem_sparse_prefill on the selector's lists) and the dense attention
(poem_dense_prefill), idle again. A thread samples `amd-smi metric -p -c --json` (a child
process, read-only telemetry) throughout; each phase reports the mean socket power and
the mean graphics clock over its samples (the first second and the last 0.3 s of a
phase are left out), with the launches it ran. Markdown goes to stdout.
"""
import argparse
import json
import statistics
import subprocess
import threading
import time


def _sample(stop, out):
    while not stop.is_set():
        t = time.time()
        try:
            r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True,
                               timeout=20)
            d = json.loads(r.stdout)["gpu_data"][0]
            power = float(d["power"]["socket_power"]["value"])
            clks = [v["clk"]["value"] for k, v in d["clock"].items()
                    if k.startswith("gfx_") and isinstance(v, dict) and isinstance(v.get("clk"), dict)
                    and isinstance(v["clk"].get("value"), (int, float))]
            out.append((t, power, statistics.mean(clks) if clks else float("nan")))
        except (OSError, ValueError, KeyError, IndexError, subprocess.SubprocessError):
            pass
        stop.wait(0.2)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--seconds", type=float, default=8.0)
    args = ap.parse_args()

    import numpy as np
    import torch
    from . import _lib as L, synth

    assert torch.cuda.is_available(), "the power probe needs a GPU"
    L.load()
    w = synth.WORKLOADS[args.workload]
    inp = synth.make(w)
    if inp.is_bf16:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = conv(inp.q), conv(inp.k), conv(inp.v)
    gp = L.Problem(list(w.seqlens_q), list(w.seqlens_k), w.num_heads_q, w.num_heads_kv, w.head_dim, w.block_size,
                   0.0, w.dtype)
    out_dtype = "bf16" if w.dtype == "bf16" else "fp32"
    ws = L.SelectWorkspace(gp, w.rows_per_tile)
    sws = L.SparseWorkspace(gp)

    def select():
        return L.select(gp, q, k, v, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, workspace=ws)

    sel = select()
    rp, bi = sel["row_ptr"], sel["block_idx"]
    out, lse = L.sparse_prefill(gp, q, k, v, rp, bi, out_dtype=out_dtype, workspace=sws)
    phases = [("idle", None), ("select", select),
              ("sparse", lambda: L.sparse_prefill(gp, q, k, v, rp, bi, out_dtype=out_dtype, out=out, lse=lse,
                                                  workspace=sws)),
              ("dense", lambda: L.dense_prefill(gp, q, k, v, out_dtype=out_dtype, out=out, lse=lse)),
              ("idle", None)]
    torch.cuda.synchronize()

    samples = []
    stop = threading.Event()
    th = threading.Thread(target=_sample, args=(stop, samples), daemon=True)
    th.start()
    spans = []
    for name, fn in phases:
        t0 = time.time()
        n = 0
        while time.time() - t0 < args.seconds:
            if fn is None:
                time.sleep(0.25)
                continue
            for _ in range(4):
                fn()
            torch.cuda.synchronize()
            n += 4
        spans.append((name, t0, time.time(), n))
    stop.set()
    th.join()

    print(f"# socket power and graphics clock per phase: {w.name}\n")
    print(f"command: python3 -m block_sparse_attention_poem_amd.power_probe --workload {args.workload} "
          f"--seconds {args.seconds:g}\n")
    print("telemetry: amd-smi metric -p -c --json every ~0.2 s (socket power; mean of the gfx_* clocks)\n")
    print("phase | launches | ms per launch | samples | socket power W (mean, min-max) | graphics clock MHz")
    print("---|---|---|---|---|---")
    for name, t0, t1, n in spans:
        v = [(p, c) for t, p, c in samples if t0 + 1.0 <= t <= t1 - 0.3]
        if not v:
            continue
        ps = [p for p, _ in v]
        ms = f"{1e3 * (t1 - t0) / n:.2f}" if n else "-"
        print(f"{name} | {n} | {ms} | {len(v)} | {statistics.mean(ps):.0f} ({min(ps):.0f}-{max(ps):.0f}) | "
              f"{statistics.mean(c for _, c in v):.0f}")


if __name__ == "__main__":
    main()
