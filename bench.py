#!/usr/bin/env python3
"""Benchmark of POEM-style output-relative block-sparse prefill on one MI355X.

One step = the whole hot path on resident inputs: poem_select (selector sweeps,
ranking/threshold, CSR) followed by poem_sparse_prefill over the retained blocks.
poem_dense_prefill (same kernel, full causal lists) is timed beside it for the
speedup. Prints one JSON line.

value  = 4 d P_R / (t_select + t_sparse): retained-block attention FLOPs per second
         of the whole step (P_R = causal (query, key) pairs inside retained blocks,
         summed over query heads).
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 (MFMA and vector)
PEAK_HBM_GBS = 8000.0
METRIC = "sparse prefill attn latency + eff. TFLOP/s at 128K; speedup vs own dense kernel"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def tile_table(gp):
    """Per global tile: (n_rows, diag) from the problem geometry."""
    rows, diags = [], []
    B = gp.block_size
    for nq, nk in zip(gp.seqlens_q, gp.seqlens_k):
        d0 = (nk - nq) // B
        for t in range(-(-nq // B)):
            rows.append(min(B, nq - t * B))
            diags.append(d0 + t)
    return np.array(rows, np.int64), np.array(diags, np.int64)


def pair_counts(gp, rp, bi):
    """(retained pairs, dense pairs) over all (head, tile) rows of the CSR."""
    B = gp.block_size
    n_rows, diags = tile_table(gp)
    T = len(n_rows)
    H = gp.num_heads_q
    counts = np.diff(rp).reshape(H, T)
    # does each row hold its diagonal block? rows are ascending, so the diagonal is last
    last = np.where(counts.ravel() > 0, bi[np.maximum(rp[1:] - 1, 0)], -1).reshape(H, T)
    has_diag = (last == diags[None, :]).astype(np.int64)
    full = counts - has_diag
    tri = n_rows * (n_rows + 1) // 2
    retained = int((full * (n_rows[None, :] * B) + has_diag * tri[None, :]).sum())
    dense = int(H * (diags * n_rows * B + tri).sum())
    return retained, dense


WORKLOAD_TAGS = {1: "single_head_2k_fp32", 2: "llama8b_32k", 3: "llama8b_128k", 4: "qwen14b_64k", 5: "chunked_varlen"}


def measured_traffic(workload_id):
    """HBM bytes per launch of the sparse attention kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (scaled by a plain copy's readings), or None when the
    record is missing or the kernel sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{WORKLOAD_TAGS.get(workload_id, '')}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = b"".join(open(os.path.join(ROOT, "block_sparse_attention_poem_amd", "csrc", f), "rb").read()
                   for f in ("poem_device.hpp", "poem_internal.hpp", "attn_fwd.hip"))
    if hashlib.sha256(src).hexdigest() != rec.get("attn_source_sha256"):
        return None
    ks = [v for name, v in rec["kernels"].items() if "attn_sparse_persistent_kernel<" in name]
    if len(ks) != 1:
        return None
    return ks[0]["read_bytes"] + ks[0]["write_bytes"]


def unique_bytes(gp, rp, bi, in_bytes, out_bytes):
    """Minimum HBM bytes of one sparse launch: Q read once, O written once, and every
    (KV head, sequence, block) that some row retains read once (K and V)."""
    n_rows, _ = tile_table(gp)
    T = len(n_rows)
    G = gp.num_heads_q // gp.num_heads_kv
    seq_of_tile = np.concatenate([np.full(-(-nq // gp.block_size), s, np.int64)
                                  for s, nq in enumerate(gp.seqlens_q)]) if T else np.zeros(0, np.int64)
    counts = np.diff(rp)
    r = np.repeat(np.arange(len(counts)), counts)
    g = (r // T) // G
    sq = seq_of_tile[r % T]
    key = (g * len(gp.seqlens_q) + sq) * (1 << 20) + bi[:len(r)].astype(np.int64)
    n_blocks = len(np.unique(key))
    kv = 2 * n_blocks * gp.block_size * gp.head_dim * in_bytes
    q_o = gp.total_q * gp.num_heads_q * gp.head_dim * (in_bytes + out_bytes)
    return int(kv + q_o)


def cpu_baseline(w, inp, gp, rp, bi, seconds, gpu_scores=None):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload: per
    sampled (head, tile), the selector and the sparse attention over its oracle-kept
    blocks. Reported in the step's unit (retained-block TFLOP/s).

    After the timed loop (outside it), the oracle's selections of the sampled pairs are
    compared with the GPU's CSR and scores (gpu_scores: {(h, gtile): scores}) under the
    parity gates: the returned dict's "parity_sample" holds the agreement rate."""
    from block_sparse_attention_poem_amd import synth
    from oracle import poem_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    op = O.Problem(tuple(w.seqlens_q), tuple(w.seqlens_k), w.num_heads_q, w.num_heads_kv, w.head_dim, w.block_size)
    tl = O.tiles(op)
    rng = np.random.default_rng(0)
    order = rng.permutation([(h, t.gtile) for h in range(w.num_heads_q) for t in tl] if len(tl) * w.num_heads_q < 4096
                            else [(int(h), int(g)) for h, g in zip(rng.integers(0, w.num_heads_q, 4096),
                                                                     rng.integers(0, len(tl), 4096))])
    q = inp.q
    k64 = synth.to_f64(inp.k)
    v64 = synth.to_f64(inp.v)
    B = w.block_size
    flops = 0.0
    done = 0
    sels = []
    t0 = time.perf_counter()
    for h, gt in order:
        h, gt = int(h), int(gt)
        t = tl[gt]
        # widen only this tile's queries (the oracle reads exact bf16 -> fp64 values)
        qt = np.zeros((t.q_row0 + t.n_rows, w.num_heads_q, w.head_dim))
        qt[t.q_row0:t.q_row0 + t.n_rows, h] = synth.to_f64(q[t.q_row0:t.q_row0 + t.n_rows, h])
        sel = O.select_tile(op, qt, k64, v64, h, t, float(inp.tau[h]), w.n_sink_blocks, w.n_local_blocks,
                            w.rows_per_tile)
        O.tile_attention(op, qt, k64, v64, h, t, sel.retained)
        kept = sel.retained
        full = len(kept) - (1 if t.diag in kept else 0)
        pairs = full * t.n_rows * B + (t.n_rows * (t.n_rows + 1) // 2 if t.diag in kept else 0)
        flops += 4.0 * w.head_dim * pairs
        done += 1
        sels.append(sel)
        if time.perf_counter() - t0 > seconds:
            break
    el = time.perf_counter() - t0
    res = {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{done} (head, tile) pairs drawn uniformly from the workload; per pair the fp64 selector "
                     f"(8 sampled rows) and the sparse attention over its kept blocks; {el:.1f} s",
           "seconds": el, "host_cpus": len(os.sched_getaffinity(0))}
    if gpu_scores is not None:
        res["parity_sample"] = parity_sample(sels, inp, gp, rp, bi, gpu_scores)
    return res


def parity_sample(sels, inp, gp, rp, bi, gpu_scores):
    """GPU selection against the oracle's on the pairs the CPU leg computed: candidate
    score error (1e-3 relative gate, floored at tau / n_vis, and unfloored), mandatory
    score error, mask agreement over candidate blocks, and mismatches outside the
    near-threshold exemption (which must be zero)."""
    from tests import helpers as TH
    T = sum(-(-nq // gp.block_size) for nq in gp.seqlens_q)
    n_c = n_m = 0
    bad = 0
    worst = worst_unf = worst_mand = 0.0
    detail = {}
    for sel in sels:
        h, gt = sel.h, sel.tile.gtile
        tau = float(inp.tau[h])
        n_vis = sel.tile.diag + 1
        se, sm, info = TH.score_errors(sel, gpu_scores[(h, gt)], tau)
        worst, worst_mand = max(worst, se), max(worst_mand, sm)
        worst_unf = max(worst_unf, info.get("unfloored", 0.0))
        kept = bi[rp[h * T + gt]:rp[h * T + gt + 1]].tolist()
        nc, nm, b = TH.mask_agreement(sel, kept, tau, tau / n_vis, detail=detail)
        n_c, n_m, bad = n_c + nc, n_m + nm, bad + len(b)
    return {"pairs": len(sels), "candidates": n_c, "agreement": (n_m / n_c) if n_c else 1.0,
            "non_exempt_mismatches": bad, "mismatches_score_only_exemption": detail.get("score_only_bad", 0),
            "worst_candidate_score_rel_err": worst, "worst_candidate_score_rel_err_unfloored": worst_unf,
            "worst_mandatory_score_rel_err": worst_mand, "score_gate": 1e-3}


def mfma_probe():
    """On-card bf16 MFMA rate (libpoem_probe.so): MFMA-only waves, two per SIMD, on
    constant few-bit operands and on random operands that change from one MFMA to the
    next (as a kernel streaming real K and V sees them)."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "block_sparse_attention_poem_amd", "libpoem_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.poem_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.poem_probe_mfma_bf16.restype = ctypes.c_double
    lib.poem_probe_mfma_bf16_random.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                                                ctypes.c_void_p]
    lib.poem_probe_mfma_bf16_random.restype = ctypes.c_double
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()

    def rate(launch):
        best = 0.0
        for i in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            flop = launch()
            e1.record(st)
            torch.cuda.synchronize()
            if flop < 0:
                return None
            if i > 0:  # the first launch warms the clock up
                best = max(best, flop / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        return best

    sp, sv = ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(st.cuda_stream)
    const = rate(lambda: lib.poem_probe_mfma_bf16(sp, blocks, 40000, sv))
    rand = rate(lambda: lib.poem_probe_mfma_bf16_random(sp, blocks, 20000, 12345, sv))
    del sink
    if const is None or rand is None:
        return None
    clock = lambda tf: tf * 1e12 / (cus * 4096) / 1e9
    return {"achieved_tflops": const, "quoted_peak_tflops": PEAK_BF16_TFLOPS, "frac_of_quoted": const / PEAK_BF16_TFLOPS,
            "implied_clock_ghz": clock(const), "compute_units": cus,
            "kernel": "v_mfma_f32_32x32x16_bf16 chains on registers, 2 waves per SIMD, no memory traffic",
            "random_operands": {"achieved_tflops": rand, "frac_of_quoted": rand / PEAK_BF16_TFLOPS,
                                "implied_clock_ghz": clock(rand),
                                "operands": "8 pairs per wave of random sign and mantissa, rotated every MFMA"}}


def selector_streaming(gp, w, t_sel_ms, workload_id):
    """K/V streaming of the selector's two sweeps: the unique K and V bytes each pass
    reads, their rate over the whole selector call, and per sweep the bytes fetched
    from beyond L2 and the L2 hit rate from the committed rocprofv3 counters (when the
    selector sources still match the ones profiled)."""
    import hashlib
    in_bytes = 2 if w.dtype == "bf16" else 4
    kv = 2 * gp.total_k * gp.num_heads_kv * gp.head_dim * in_bytes
    out = {"unique_kv_bytes_per_pass": kv, "passes": 2,
           "algorithmic_gbs_over_select_call": 2 * kv / (t_sel_ms * 1e-3) / 1e9}
    path = os.path.join(ROOT, "profiles", f"selector_{WORKLOAD_TAGS.get(workload_id, '')}.json")
    if os.path.exists(path):
        rec = json.load(open(path))
        src = b"".join(open(os.path.join(ROOT, "block_sparse_attention_poem_amd", "csrc", f), "rb").read()
                       for f in ("poem_device.hpp", "poem_internal.hpp", "selector.hip"))
        if hashlib.sha256(src).hexdigest() == rec.get("selector_source_sha256"):
            out["counters"] = rec["sweeps"]
    return out


def sampled_row_index(gp, S):
    """Packed query-row indices of every tile's sampled rows (even stride ending at the
    tile's last row) and the tile each belongs to."""
    rows, tiles = [], []
    B = gp.block_size
    g = 0
    q0 = 0
    for nq in gp.seqlens_q:
        for t in range(-(-nq // B)):
            n = min(B, nq - t * B)
            st = min(S, n)
            for j in range(st):
                rows.append(q0 + t * B + (-(-((j + 1) * n) // st)) - 1)
                tiles.append(g)
            g += 1
        q0 += nq
    return np.array(rows, np.int64), np.array(tiles, np.int64)


def _err_stats(e, si, tau):
    """Row errors e [rows, H]: mean, rms, p99 (on up to 4M rows), max, and the share of
    the selector's sampled rows si whose error is within their head's tau."""
    import torch
    f = e.flatten()
    sub = f[torch.randperm(f.numel(), device=f.device)[:1 << 22]]
    return {"mean": float(f.mean()), "rms": float(torch.sqrt((f * f).mean())),
            "p99": float(torch.quantile(sub, 0.99)), "max": float(f.max()),
            "sampled_rows_within_tau": float((e[si] <= tau[None, :]).float().mean())}


def _time_select_sparse(gp, L, w, q, k, v, ws, sws, taus, mode, steps, **kw):
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    r = None
    for i in range(steps):
        ev[i][0].record()
        r = L.select(gp, q, k, v, taus, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, workspace=ws, mode=mode,
                     **kw)
        ev[i][1].record()
        prefill = L.sparse_prefill_group if mode == "group" else L.sparse_prefill
        prefill(gp, q, k, v, r["row_ptr"], r["block_idx"], out_dtype="bf16", want_lse=False, workspace=sws)
        ev[i][2].record()
    torch.cuda.synchronize()
    t_sel = float(np.median([ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)]))
    t_sp = float(np.median([ev[i][1].elapsed_time(ev[i][2]) for i in range(steps)]))
    return r, t_sel, t_sp


def selector_legs(args, w, inp, gp, L, q, k, v, ws, sws, rp_poem, steps):
    """The other selectors beside POEM's per-head one, on the same inputs:
    - mass-only and practical POEM: latency at a fixed budget, then each at POEM's
      per-head keep counts (each head's budget bisected until its kept-block count
      matches POEM's), with the output errors against dense attention;
    - group-shared lists: latency at the same thresholds, keep fraction and errors.
    Errors are ||O_sparse - O_dense|| per query row with fp32 outputs."""
    import torch
    H = w.num_heads_q
    T = L.num_tiles(gp)
    cap = L.csr_capacity(gp)
    srow, _ = sampled_row_index(gp, w.rows_per_tile)
    si = torch.from_numpy(srow).cuda()
    tau = torch.tensor([float(x) for x in inp.tau], device="cuda")
    od, _ = L.dense_prefill(gp, q, k, v, out_dtype="fp32", want_lse=False)

    def errors(rr, group=False):
        prefill = L.sparse_prefill_group if group else L.sparse_prefill
        o, _ = prefill(gp, q, k, v, rr["row_ptr"], rr["block_idx"], out_dtype="fp32", want_lse=False, workspace=sws)
        e = torch.linalg.vector_norm(o - od, dim=-1)
        del o
        return e

    # POEM's CSR again (the same thresholds reproduce it exactly)
    rpo = L.select(gp, q, k, v, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, workspace=ws)
    assert torch.equal(rpo["row_ptr"], torch.from_numpy(rp_poem.astype(np.int32)).cuda())
    e_p = errors(rpo)
    out = {"err_poem": _err_stats(e_p, si, tau)}
    del e_p

    vis = np.diff(rp_poem).reshape(H, T).sum(1)  # POEM's kept blocks per head

    def matched(mode, **kw):
        """Per-head budgets bisected (in log10) until each head keeps as many blocks as
        POEM; returns the budgets and the selection at them."""
        lo, hi = np.full(H, -9.0), np.zeros(H)
        best = [None] * H
        for _ in range(24):
            mid = 0.5 * (lo + hi)
            rr = L.select(gp, q, k, v, list(10.0 ** mid), w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile,
                          workspace=ws, mode=mode, **kw)
            kept = np.diff(rr["row_ptr"].cpu().numpy().astype(np.int64)).reshape(H, T).sum(1)
            for h in range(H):
                gap = abs(int(kept[h]) - int(vis[h]))
                if best[h] is None or gap < best[h][0]:
                    best[h] = (gap, float(10.0 ** mid[h]))
            more = kept > vis  # keeps too much: raise the budget
            lo = np.where(more, mid, lo)
            hi = np.where(more, hi, mid)
        eps = [b[1] for b in best]
        return eps, L.select(gp, q, k, v, eps, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, workspace=ws,
                             mode=mode, **kw)

    res_m = {}
    if not args.no_mass:
        r, t_sel, t_sp = _time_select_sparse(gp, L, w, q, k, v, ws, sws, [args.mass_eps] * H, "mass", steps)
        res_m = {"eps": args.mass_eps, "select_ms": t_sel, "sparse_ms": t_sp,
                 "keep_fraction_blocks": int(r["row_ptr"][-1].item()) / cap}
        eps_m, rm = matched("mass")
        e_m = errors(rm)
        res_m["matched_keep"] = {
            "keep_fraction_blocks_poem": float(rp_poem[-1]) / cap,
            "keep_fraction_blocks_mass": float(rm["row_ptr"][-1].item()) / cap,
            "eps_per_head": [float("%.4g" % e) for e in eps_m],
            "err_poem": out["err_poem"], "err_mass": _err_stats(e_m, si, tau)}
        del e_m
        # matched guarantee: each head's budget bisected to the largest for which every
        # sampled row's output error stays within the head's tau (POEM's guarantee by
        # construction), then the blocks mass-only needs for it
        lo, hi = np.full(H, -9.0), np.zeros(H)
        for _ in range(16):
            mid = 0.5 * (lo + hi)
            rr = L.select(gp, q, k, v, list(10.0 ** mid), w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile,
                          workspace=ws, mode="mass")
            e = errors(rr)
            ok = (e[si] <= tau[None, :]).all(dim=0).cpu().numpy()
            del e
            lo = np.where(ok, mid, lo)
            hi = np.where(ok, hi, mid)
        rg = L.select(gp, q, k, v, list(10.0 ** lo), w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile,
                      workspace=ws, mode="mass")
        e_g = errors(rg)
        res_m["matched_guarantee"] = {
            "keep_fraction_blocks_poem": float(rp_poem[-1]) / cap,
            "keep_fraction_blocks_mass": float(rg["row_ptr"][-1].item()) / cap,
            "eps_per_head": [float("%.4g" % e) for e in 10.0 ** lo],
            "err_mass": _err_stats(e_g, si, tau),
            "note": "per head, the largest mass budget (bisected) whose sampled rows all stay within tau"}
        del e_g

    # practical POEM: latency at a fixed budget, then errors at POEM's per-head keep counts
    res_p = {}
    if not args.no_practical:
        pk = dict(weight=args.practical_weight, presel_fraction=args.practical_presel)
        r, t_sel, t_sp = _time_select_sparse(gp, L, w, q, k, v, ws, sws, [args.mass_eps] * H, "practical", steps,
                                             **pk)
        res_p = {"eps": args.mass_eps, "weight": pk["weight"], "presel_fraction": pk["presel_fraction"],
                 "select_ms": t_sel, "sparse_ms": t_sp, "keep_fraction_blocks": int(r["row_ptr"][-1].item()) / cap}
        eps_p, rpr = matched("practical", **pk)
        e_pr = errors(rpr)
        res_p["matched_keep"] = {"keep_fraction_blocks_poem": float(rp_poem[-1]) / cap,
                                 "keep_fraction_blocks_practical": float(rpr["row_ptr"][-1].item()) / cap,
                                 "err_poem": out["err_poem"], "err_practical": _err_stats(e_pr, si, tau)}
        del e_pr

    r, t_sel, t_sp = _time_select_sparse(gp, L, w, q, k, v, ws, sws, inp.tau, "group", steps)
    e_g = errors(r, group=True)
    # retained-pair rate of the two-heads-per-workgroup kernel on the shared lists
    p_g, _ = pair_counts(gp, r["row_ptr"].cpu().numpy().astype(np.int64), r["block_idx"].cpu().numpy())
    tf_g = 4.0 * w.head_dim * p_g / (t_sp * 1e-3) / 1e12
    res_g = {"select_ms": t_sel, "sparse_ms": t_sp, "keep_fraction_blocks": int(r["row_ptr"][-1].item()) / cap,
             "sparse_tflops": tf_g, "sparse_frac_of_bf16_peak": tf_g / 2500.0,
             "err_group": _err_stats(e_g, si, tau), "err_poem": out["err_poem"],
             "note": "same per-head thresholds as the headline step; one list per (KV head, tile) from the "
                     "group's 8 sampled rows, run by poem_sparse_prefill_group (G even: two heads per workgroup, each "
                     "K/V stage loaded once for both); sampled_rows_within_tau is taken "
                     "on the per-head selector's rows"}
    del od, e_g
    torch.cuda.empty_cache()
    return res_m, res_g, res_p


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, help="synthetic workload id (1..5); 3 is the 128K layer")
    ap.add_argument("--sink-offset", type=float, default=None, help="L_s - ln N (default 6)")
    ap.add_argument("--near-output", type=float, default=0.0,
                    help="fraction of clusters whose values equal the sink's (default 0: the workload as defined)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="skip the mass-only and group-shared selector legs")
    ap.add_argument("--no-probe", action="store_true", help="skip the on-card MFMA rate probe")
    ap.add_argument("--no-mass", action="store_true", help="skip the mass-only selector leg")
    ap.add_argument("--no-practical", action="store_true", help="skip the practical POEM leg")
    ap.add_argument("--mass-eps", type=float, default=0.002,
                    help="omitted-mass budget of the mass-only and practical legs")
    ap.add_argument("--practical-weight", type=float, default=0.5, help="deviation weight of the practical leg")
    ap.add_argument("--practical-presel", type=float, default=0.95, help="preselected mass share (practical leg)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run one device-to-device copy of this many MiB (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.copy_probe_mib > 0:
        import torch
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n}))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "libpoem runs on one GPU: the path would shard by KV head with no intra-op "
                                   "communication, but only the single-GPU kernels exist; run with --gpus 1"}))
        sys.exit(2)

    import torch
    from block_sparse_attention_poem_amd import _lib as L
    from block_sparse_attention_poem_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    L.load()
    w = synth.WORKLOADS[args.workload]
    if args.sink_offset is not None:
        w = w.with_(sink_offset=args.sink_offset)
    if args.near_output > 0:
        w = w.with_(near_output=args.near_output)
    log(f"[bench] generating workload {args.workload}: {w.name}")
    inp = synth.make(w)
    if inp.is_bf16:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = conv(inp.q), conv(inp.k), conv(inp.v)
    gp = L.Problem(list(w.seqlens_q), list(w.seqlens_k), w.num_heads_q, w.num_heads_kv, w.head_dim, w.block_size,
                   0.0, w.dtype)
    ws = L.SelectWorkspace(gp, w.rows_per_tile)
    sws = L.SparseWorkspace(gp)
    T = L.num_tiles(gp)
    cap = L.csr_capacity(gp)
    row_ptr = torch.empty(w.num_heads_q * T + 1, dtype=torch.int32, device="cuda")
    block_idx = torch.empty(cap, dtype=torch.int32, device="cuda")
    out_dtype = "bf16" if w.dtype == "bf16" else "fp32"
    out, lse = L._alloc_out(gp, out_dtype, True, q.device)
    stream = torch.cuda.current_stream()

    import ctypes
    lib = L.load()
    cp = gp.c()
    tau_arr = (ctypes.c_float * w.num_heads_q)(*[float(x) for x in inp.tau])
    odt = L.POEM_FP32 if out_dtype == "fp32" else L.POEM_BF16

    def select():
        L._check(lib.poem_select(ctypes.byref(cp), L._ptr(q), L._ptr(k), L._ptr(v), tau_arr, w.n_sink_blocks,
                                 w.n_local_blocks, w.rows_per_tile, L._ptr(row_ptr), L._ptr(block_idx), cap,
                                 None, None, None, ctypes.c_void_p(ws.ptr), ws.nbytes,
                                 ctypes.c_void_p(stream.cuda_stream)))

    def sparse():
        L._check(lib.poem_sparse_prefill(ctypes.byref(cp), L._ptr(q), L._ptr(k), L._ptr(v), L._ptr(row_ptr),
                                         L._ptr(block_idx), L._ptr(out), odt, L._ptr(lse),
                                         ctypes.c_void_p(sws.ptr), sws.nbytes, ctypes.c_void_p(stream.cuda_stream)))

    dws = L.DenseWorkspace()

    def dense():
        L._check(lib.poem_dense_prefill(ctypes.byref(cp), L._ptr(q), L._ptr(k), L._ptr(v), L._ptr(out), odt,
                                        L._ptr(lse), ctypes.c_void_p(dws.ptr), dws.nbytes,
                                        ctypes.c_void_p(stream.cuda_stream)))

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        select()
        sparse()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        select()
        ev[i][1].record(stream)
        sparse()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_sel = np.array([ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)])
    t_sp = np.array([ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)])

    rp = row_ptr.cpu().numpy().astype(np.int64)
    bi = block_idx.cpu().numpy()
    p_ret, p_dense = pair_counts(gp, rp, bi)
    kept_blocks = int(rp[-1])
    flop_ret = 4.0 * w.head_dim * p_ret
    flop_dense = 4.0 * w.head_dim * p_dense

    t_dense = None
    if not args.no_dense:
        log("[bench] dense baseline")
        for _ in range(max(1, args.warmup // 2)):
            dense()
        evd = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            evd[i][0].record(stream)
            dense()
            evd[i][1].record(stream)
        torch.cuda.synchronize()
        t_dense = np.array([evd[i][0].elapsed_time(evd[i][1]) for i in range(args.steps)])

    ms_step = wall * 1e3 / args.steps
    sel_ms, sp_ms = float(np.median(t_sel)), float(np.median(t_sp))
    value = flop_ret / ((sel_ms + sp_ms) * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    # dominant kernel of the step: the sparse attention kernel (one launch per step);
    # its achieved rate uses the average launch duration over the timed steps
    attn_tflops = flop_ret / (sp_ms * 1e-3) / 1e12
    attn_tflops_avg = flop_ret / (float(t_sp.mean()) * 1e-3) / 1e12
    roofline = {"kernel": "attn_sparse_persistent_kernel", "bound": "mfma", "achieved": attn_tflops_avg,
                "peak": peak,
                "unit": "TFLOP/s", "frac": attn_tflops_avg / peak, "avg_launch_ms": float(t_sp.mean()),
                "traffic": measured_traffic(args.workload),
                "algorithmic": f"4 d P_R = {flop_ret:.4e} FLOP per launch",
                "algorithmic_bytes": unique_bytes(gp, rp, bi, q.element_size(),
                                                  out.element_size())}
    res = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "heads_q": w.num_heads_q, "heads_kv": w.num_heads_kv,
                   "head_dim": w.head_dim, "seqlens_k": list(w.seqlens_k), "seqlens_q": list(w.seqlens_q),
                   "block": w.block_size, "rows_per_tile": w.rows_per_tile, "sink_offset": w.sink_offset,
                   "near_output": w.near_output,
                   "tau": list(w.tau), "mandatory": {"sink_blocks": w.n_sink_blocks,
                                                     "local_blocks": w.n_local_blocks}},
        "latency_ms": {"select": sel_ms, "sparse_attn": sp_ms, "select_plus_sparse": sel_ms + sp_ms,
                       "dense_attn": float(np.median(t_dense)) if t_dense is not None else None,
                       "select_min": float(t_sel.min()), "sparse_min": float(t_sp.min())},
        "speedup_vs_dense": (float(np.median(t_dense)) / (sel_ms + sp_ms)) if t_dense is not None else None,
        "speedup_attn_only": (float(np.median(t_dense)) / sp_ms) if t_dense is not None else None,
        "eff_tflops_sparse_kernel": attn_tflops,
        "dense_tflops": (flop_dense / (float(np.median(t_dense)) * 1e-3) / 1e12) if t_dense is not None else None,
        "keep_fraction_blocks": kept_blocks / cap,
        "keep_fraction_per_head": [round(float(x), 4) for x in
                                   (np.diff(rp).reshape(w.num_heads_q, T).sum(1) / (cap / w.num_heads_q))],
        "keep_fraction_pairs": p_ret / p_dense,
        "roofline": roofline,
    }
    res["selector_streaming"] = selector_streaming(gp, w, sel_ms, args.workload)
    res["memory"] = {"select_workspace_bytes": ws.nbytes, "sparse_workspace_bytes": sws.nbytes,
                     "dense_workspace_bytes": dws.nbytes,
                     "csr_bytes": 4 * (len(rp) + kept_blocks), "csr_capacity_bytes": 4 * (len(rp) + cap),
                     "context": "the POEM summary page reports about 2 MiB of peak memory overhead at 128K "
                                "(whole system, hardware not stated)"}
    if not args.no_probe:
        log("[bench] MFMA rate probe")
        res["mfma_probe"] = mfma_probe()
    if not args.no_legs and inp.is_bf16:
        log("[bench] mass-only and group-shared selector legs")
        res_m, res_g, res_p = selector_legs(args, w, inp, gp, L, q, k, v, ws, sws, rp, args.steps)
        if res_m:
            res["mass_only"] = res_m
        res["group_shared"] = res_g
        if res_p:
            res["practical"] = res_p
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline ({args.cpu_seconds:.0f} s)")
        # the GPU's scores for the parity sample (one more selection, outside the timed steps)
        rd = L.select(gp, q, k, v, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True,
                      workspace=ws)
        assert torch.equal(rd["row_ptr"], row_ptr)
        scores_dev = rd["tile_scores"]
        del rd
        torch.cuda.synchronize()

        class _Scores(dict):
            def __missing__(self, key):
                v_ = scores_dev[key[0], key[1]].cpu().numpy()
                self[key] = v_
                return v_
        res["cpu_baseline"] = cpu_baseline(w, inp, gp, rp, bi, args.cpu_seconds, gpu_scores=_Scores())
        if "parity_sample" in res["cpu_baseline"]:
            res["parity_sample"] = res["cpu_baseline"].pop("parity_sample")
        del scores_dev
    # release device memory and let queued work finish before printing, so the process
    # ends right after its one line
    del q, k, v, out, lse, row_ptr, block_idx, ws, sws, dws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
