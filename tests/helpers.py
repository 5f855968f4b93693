"""Shared helpers for the GPU parity tests: device upload, oracle comparisons."""
import math

import numpy as np

from block_sparse_attention_poem_amd import _lib as L
from block_sparse_attention_poem_amd import synth
from oracle import poem_oracle as O

# Gates (stated by the method's acceptance criteria; fp32 ones derived in the design doc)
SCORE_RTOL = 1e-3        # selector scores, relative, floored at tau / n_vis
MANDATORY_SCORE_RTOL = SCORE_RTOL  # mandatory blocks too (never ranked, but reported)
SCORE_RTOL_FP32 = 1e-4   # candidate scores with fp32 inputs (fp32 products and weights)


def score_rtol(dtype):
    """The candidate-score gate for an input dtype."""
    return SCORE_RTOL_FP32 if dtype == "fp32" else SCORE_RTOL
OUT_ATOL_BF16 = 1e-2     # max-abs output error, bf16 inputs, fp32 accumulation
OUT_ATOL_FP32 = 1e-4     # fp32 inputs
LSE_ATOL_BF16 = 1e-3
LSE_ATOL_FP32 = 1e-5
NEAR_REL = 1e-3          # "near the threshold" exemption


def device_inputs(inp):
    import torch
    if inp.is_bf16:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    else:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return conv(inp.q), conv(inp.k), conv(inp.v)


def problems(w):
    gp = L.Problem(list(w.seqlens_q), list(w.seqlens_k), w.num_heads_q, w.num_heads_kv, w.head_dim,
                   w.block_size, 0.0, w.dtype)
    op = O.Problem(tuple(w.seqlens_q), tuple(w.seqlens_k), w.num_heads_q, w.num_heads_kv, w.head_dim,
                   w.block_size)
    return gp, op


def f64(inp):
    return synth.to_f64(inp.q), synth.to_f64(inp.k), synth.to_f64(inp.v)


def csr_rows(row_ptr, block_idx):
    rp = row_ptr.cpu().numpy().astype(np.int64)
    bi = block_idx.cpu().numpy()
    return rp, bi


def retained(rp, bi, r):
    return bi[rp[r]:rp[r + 1]].tolist()


def mask_agreement(sel, gpu_retained, tau, floor, target=None, detail=None):
    """Compare one tile's GPU retained set with the oracle's selection.

    Returns (n_candidates, n_matching_decisions, non_exempt_mismatches). A mismatch on
    block b is exempt when b's oracle score is within NEAR_REL of the oracle score at
    the last discarded or first retained position of the oracle's discard order, or
    when the oracle bound B(j) is within NEAR_REL * tau of tau at b's own position j
    or the one before it (target: the curve value at the cut, tau unless given; the
    group selector's excess curve cuts at 0). detail (a dict) receives
    "score_only_bad": the mismatches the score rule alone leaves unexempted."""
    target = tau if target is None else target
    order = sel.order
    ks = sel.k_star
    pos = {b: j + 1 for j, b in enumerate(order)}  # 1-based position in the discard order
    keep_o = set(sel.retained)
    keep_g = set(gpu_retained)
    near_scores = []
    if ks >= 1:
        near_scores.append(sel.score[order[ks - 1]])
    if ks < len(order):
        near_scores.append(sel.score[order[ks]])
    bad = []
    score_only_bad = 0
    match = 0
    for b in order:
        if (b in keep_o) == (b in keep_g):
            match += 1
            continue
        s = sel.score[b]
        ex = any(abs(s - ns) <= NEAR_REL * max(ns, floor) for ns in near_scores)
        score_only_bad += 0 if any(abs(s - ns) <= NEAR_REL * ns for ns in near_scores) else 1
        j = pos[b]
        for jj in (j, j - 1):
            if 0 <= jj < len(sel.curve) and abs(sel.curve[jj] - target) <= NEAR_REL * tau:
                ex = True
        if not ex:
            bad.append(b)
    if detail is not None:
        detail["score_only_bad"] = detail.get("score_only_bad", 0) + score_only_bad
    return len(order), match, bad


def score_errors(sel, gpu_scores, tau):
    """|gpu - oracle| / max(oracle, tau / n_vis) over a tile's visible blocks.

    Returns (worst over candidate blocks, worst over mandatory blocks, detail of the
    worst candidate). Only candidate scores are ranked and summed into the bound. The
    detail also holds "unfloored": the worst |gpu - oracle| / oracle over candidates
    with a positive oracle score."""
    n = sel.tile.diag + 1
    floor = tau / n
    ref = sel.score
    g = np.asarray(gpu_scores[:n], dtype=np.float64)
    rel = np.abs(g - ref) / np.maximum(ref, floor)
    cand = np.asarray(sel.order, dtype=np.int64)
    mand = np.asarray(sel.mandatory, dtype=np.int64)
    wc = float(rel[cand].max()) if len(cand) else 0.0
    wm = float(rel[mand].max()) if len(mand) else 0.0
    b = int(cand[rel[cand].argmax()]) if len(cand) else -1
    info = dict(block=b, oracle=float(ref[b]), gpu=float(g[b]), mass=float(sel.mass[b]), floor=floor) if b >= 0 else {}
    pos = cand[ref[cand] > 0] if len(cand) else cand
    info["unfloored"] = float((np.abs(g[pos] - ref[pos]) / ref[pos]).max()) if len(pos) else 0.0
    return wc, wm, info


def row_errors(O_a, O_b):
    return np.linalg.norm(np.asarray(O_a, np.float64) - np.asarray(O_b, np.float64), axis=-1)


def lse_close(a, b, atol):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_inf = np.isneginf(a) & np.isneginf(b)
    with np.errstate(invalid="ignore"):
        close = np.abs(a - b) <= atol
    return bool(np.all(both_inf | close))


def stratified_tiles(op, heads, per_head, seed=0):
    """Per head: first and last tiles plus seeded random ones (global tile ids)."""
    tl = O.tiles(op)
    rng = np.random.default_rng(seed)
    out = []
    for h in heads:
        picks = {0, len(tl) - 1}
        if len(tl) > 2:
            picks |= set(rng.choice(len(tl), size=min(per_head, len(tl)), replace=False).tolist())
        out += [(h, int(g)) for g in sorted(picks)]
    return out


def tile_rows(op, gtile):
    t = O.tiles(op)[gtile]
    return t.q_row0, t.n_rows


def is_nan_free(x):
    return not np.isnan(np.asarray(x)).any()


__all__ = [n for n in dir() if not n.startswith("_")] + ["math"]
