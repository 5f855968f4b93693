"""GPU parity of libpoem (through its C ABI) against the fp64 oracle.

Small problems are compared element by element; the full-size workloads run in
the benchmark's launch configuration and are checked on stratified tiles the
oracle computes one by one.
"""
import math
import sys

import numpy as np
import pytest

from block_sparse_attention_poem_amd import _lib as L
from block_sparse_attention_poem_amd import synth
from oracle import poem_oracle as O

from . import helpers as H

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    yield
    torch.cuda.synchronize()


def _sync():
    import torch
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# the three-block toy through the C ABI
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("shift", [0.0, 10.0])
def test_toy_through_c_abi(shift):
    import torch
    q, k, v, meta = synth.toy_block_inputs(shift)
    p = L.Problem([meta["n_q"]], [meta["n_k"]], 1, 1, meta["d"], meta["block"], 1.0, "fp32")
    qd, kd, vd = (torch.from_numpy(x).cuda() for x in (q, k, v))
    say("toy shift", shift)
    dense, _ = L.dense_prefill(p, qd, kd, vd, out_dtype="fp32")
    for tau, drop in ((0.5, []), (0.7, [2]), (2.0, [1, 2])):
        r = L.select(p, qd, kd, vd, [tau], 1, 1, 8, diagnostics=True)
        sp, _ = L.sparse_prefill(p, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
        _sync()
        sc = r["tile_scores"][0, 0, :4].cpu().numpy()
        assert np.allclose(sc, [0, 0.5, 0.5, 0], atol=1e-6), sc
        rp, bi = H.csr_rows(r["row_ptr"], r["block_idx"])
        kept = H.retained(rp, bi, 0)
        assert kept == sorted(set(range(4)) - set(drop)), (tau, kept)
        err = (dense[:, 0, 0] - sp[:, 0, 0]).abs().max().item()
        expect = {0.5: 0.0, 0.7: 2 / 3, 2.0: 0.0}[tau]
        assert abs(err - expect) < 1e-5, (tau, err)
        assert np.allclose(dense[:, 0, 0].cpu().numpy(), 2.0 + shift, atol=1e-6)
        rb = r["row_bound"][0, 0].cpu().numpy()
        assert np.all(rb <= tau + 1e-6)


# ---------------------------------------------------------------------------
# dense and sparse attention on small problems, element by element
# ---------------------------------------------------------------------------

SMALL = [
    # (n_q, n_k, hq, hkv, d, B, dtype, seqs)
    (300, 428, 4, 2, 64, 64, "bf16", 1),
    (300, 300, 4, 1, 128, 128, "bf16", 1),
    (200, 456, 8, 2, 128, 128, "bf16", 1),
    (130, 258, 2, 2, 64, 128, "bf16", 1),
    (190, 318, 4, 4, 128, 64, "bf16", 1),
    (300, 428, 2, 1, 64, 64, "fp32", 1),
    (129, 385, 2, 1, 128, 128, "fp32", 1),
    (100, 356, 4, 2, 128, 128, "bf16", 3),
]


def _small(case, seed=0):
    n_q, n_k, hq, hkv, d, B, dt, seqs = case
    w = synth.small_workload(n_q=n_q, n_k=n_k, hq=hq, hkv=hkv, d=d, block=B, dtype=dt, seqs=seqs, seed=seed)
    if seqs > 1:  # varlen: different prefix lengths per sequence, same chunk size
        w = w.with_(seqlens_k=tuple(n_k + B * i for i in range(seqs)), seqlens_q=tuple(n_q - 17 * i for i in range(seqs)))
        w = w.with_(seqlens_k=tuple(nk - 17 * i for i, nk in enumerate(w.seqlens_k)))
    return w


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "q%d_k%d_h%d-%d_d%d_B%d_%s_s%d" % c)
def test_dense_matches_oracle(case):
    w = _small(case)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    say("dense", case)
    out, lse = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    _sync()
    out = out.cpu().numpy()
    lse = lse.cpu().numpy()
    q, k, v = H.f64(inp)
    ref = O.dense_prefill(op, q, k, v)
    atol = H.OUT_ATOL_FP32 if w.dtype == "fp32" else H.OUT_ATOL_BF16
    latol = H.LSE_ATOL_FP32 if w.dtype == "fp32" else H.LSE_ATOL_BF16
    worst = 0.0
    for (h, gt), (Or, lr) in ref.items():
        r0, n = H.tile_rows(op, gt)
        err = np.abs(out[r0:r0 + n, h, :] - Or).max()
        worst = max(worst, err)
        assert err <= atol, (h, gt, err)
        assert H.lse_close(lse[h, r0:r0 + n], lr, latol), (h, gt)
    say("  max abs err", worst)


def _random_csr(op, rng, p_keep=0.4, empty_rows=True):
    tl = O.tiles(op)
    rows = []
    for h in range(op.num_heads_q):
        for t in tl:
            ids = [b for b in range(t.diag + 1) if rng.uniform() < p_keep or b in (0, t.diag)]
            if empty_rows and rng.uniform() < 0.1:
                ids = []
            rows.append(ids)
    rp = np.zeros(len(rows) + 1, np.int64)
    rp[1:] = np.cumsum([len(r) for r in rows])
    bi = np.array([b for r in rows for b in r], np.int32)
    return rp, bi


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "q%d_k%d_h%d-%d_d%d_B%d_%s_s%d" % c)
def test_sparse_given_mask_matches_oracle(case):
    import torch
    w = _small(case, seed=1)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    rng = np.random.default_rng(7)
    rp, bi = _random_csr(op, rng)
    rpd = torch.from_numpy(rp.astype(np.int32)).cuda()
    bid = torch.from_numpy(np.concatenate([bi, np.zeros(1, np.int32)])).cuda()
    say("sparse given mask", case)
    out, lse = L.sparse_prefill(gp, qd, kd, vd, rpd, bid, out_dtype="fp32")
    out2, lse2 = L.sparse_prefill(gp, qd, kd, vd, rpd, bid, out_dtype="fp32", workspace=None)
    _sync()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    out = out.cpu().numpy()
    lse = lse.cpu().numpy()
    q, k, v = H.f64(inp)
    ref = O.sparse_prefill(op, q, k, v, rp, bi)
    atol = H.OUT_ATOL_FP32 if w.dtype == "fp32" else H.OUT_ATOL_BF16
    latol = H.LSE_ATOL_FP32 if w.dtype == "fp32" else H.LSE_ATOL_BF16
    for (h, gt), (Or, lr) in ref.items():
        r0, n = H.tile_rows(op, gt)
        err = np.abs(out[r0:r0 + n, h, :] - Or).max()
        assert err <= atol, (h, gt, err)
        assert H.lse_close(lse[h, r0:r0 + n], lr, latol), (h, gt)


@pytest.mark.parametrize("case", [SMALL[0], SMALL[2], SMALL[5]], ids=lambda c: "q%d_k%d_h%d-%d_d%d_B%d_%s_s%d" % c)
def test_sparse_full_list_is_bitwise_dense(case):
    import torch
    w = _small(case, seed=2)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    tl = O.tiles(op)
    rows = [list(range(t.diag + 1)) for h in range(op.num_heads_q) for t in tl]
    rp = np.zeros(len(rows) + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    bi = np.array([b for r in rows for b in r], np.int32)
    say("bitwise", case)
    for od in ("fp32", "bf16"):
        d_out, d_lse = L.dense_prefill(gp, qd, kd, vd, out_dtype=od)
        bits = (lambda x: x.view(torch.int16)) if od == "bf16" else (lambda x: x.view(torch.int32))
        # the dense kernel's fixed interleave (no workspace) against its tile queue
        i_out, i_lse = L.dense_prefill(gp, qd, kd, vd, out_dtype=od, workspace=None)
        _sync()
        assert torch.equal(bits(d_out), bits(i_out))
        assert torch.equal(d_lse, i_lse)
        for ws in ("auto", None):  # persistent queue and one-workgroup-per-row schedules
            s_out, s_lse = L.sparse_prefill(gp, qd, kd, vd, torch.from_numpy(rp).cuda(),
                                            torch.from_numpy(bi).cuda(), out_dtype=od, workspace=ws)
            _sync()
            assert torch.equal(bits(d_out), bits(s_out)), ws
            assert torch.equal(d_lse, s_lse), ws


def test_empty_and_out_of_range_rows():
    import torch
    w = _small(SMALL[0], seed=3)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    tl = O.tiles(op)
    rows = []
    for h in range(op.num_heads_q):
        for t in tl:
            rows.append([] if (h + t.gtile) % 2 == 0 else [0, t.diag + 1, t.diag + 5])
    rp = np.zeros(len(rows) + 1, np.int32)
    rp[1:] = np.cumsum([len(r) for r in rows])
    bi = np.array([b for r in rows for b in r], np.int32)
    say("empty rows")
    out, lse = L.sparse_prefill(gp, qd, kd, vd, torch.from_numpy(rp).cuda(), torch.from_numpy(bi).cuda(),
                                out_dtype="fp32")
    _sync()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    q, k, v = H.f64(inp)
    for h in range(op.num_heads_q):
        for t in tl:
            r0, n = t.q_row0, t.n_rows
            if (h + t.gtile) % 2 == 0:
                assert np.all(out[r0:r0 + n, h] == 0.0)
                assert np.all(np.isneginf(lse[h, r0:r0 + n]))
            else:  # ids above the diagonal are skipped: only block 0 is used
                Or, lr = O.tile_attention(op, q, k, v, h, t, [0])
                assert np.abs(out[r0:r0 + n, h] - Or).max() <= H.OUT_ATOL_BF16


def test_lazy_reference_recomputes_spiked_tiles():
    """Keys whose logit exceeds every logit of a tile's first stage by 60 and by 200 nats
    (weights of 2^86 and, past fp32's range, 2^288 against the first stage's reference)
    make the lazy reference reject the tile, which is then computed with the exact
    running max. Dense and sparse outputs and LSE against the oracle on every tile; both
    schedules bit-identical; the sparse kernel on full lists equal to dense bit for bit."""
    import dataclasses
    import torch
    w = synth.small_workload(n_q=300, n_k=428, hq=4, hkv=2, d=128, block=128, dtype="bf16", seed=21)
    inp = synth.make(w)
    q = synth.bf16_bits_to_f32(inp.q).copy()
    k = synth.bf16_bits_to_f32(inp.k).copy()
    d = w.head_dim
    q[:, :, d - 1] = 1.0
    k[:, :, d - 1] = 0.0
    k[300, 0, d - 1] = 60.0 * math.sqrt(d)   # KV head 0, key block 2
    k[400, 1, d - 1] = 200.0 * math.sqrt(d)  # KV head 1, key block 3
    inp = dataclasses.replace(inp, q=synth.round_to_bf16_bits(q), k=synth.round_to_bf16_bits(k))
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    tl = O.tiles(op)
    rows = [list(range(t.diag + 1)) if (h + t.gtile) % 2 == 0 else [0, t.diag] + ([2] if t.diag > 2 else [])
            for h in range(op.num_heads_q) for t in tl]
    rows = [sorted(set(r)) for r in rows]
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    bi = np.array([b for r in rows for b in r] + [0], np.int32)
    rpd, bid = torch.from_numpy(rp).cuda(), torch.from_numpy(bi).cuda()
    say("lazy reference: spiked keys")
    d_out, d_lse = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    d_out2, d_lse2 = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32", workspace=None)
    s_out, s_lse = L.sparse_prefill(gp, qd, kd, vd, rpd, bid, out_dtype="fp32")
    s_out2, s_lse2 = L.sparse_prefill(gp, qd, kd, vd, rpd, bid, out_dtype="fp32", workspace=None)
    full = [list(range(t.diag + 1)) for h in range(op.num_heads_q) for t in tl]
    frp = torch.tensor(np.concatenate([[0], np.cumsum([len(r) for r in full])]), dtype=torch.int32, device="cuda")
    fbi = torch.tensor([b for r in full for b in r], dtype=torch.int32, device="cuda")
    f_out, f_lse = L.sparse_prefill(gp, qd, kd, vd, frp, fbi, out_dtype="fp32")
    _sync()
    assert torch.equal(d_out, d_out2) and torch.equal(d_lse, d_lse2)
    assert torch.equal(s_out, s_out2) and torch.equal(s_lse, s_lse2)
    assert torch.equal(f_out, d_out) and torch.equal(f_lse, d_lse)
    qf, kf, vf = H.f64(inp)
    ref_d = O.dense_prefill(op, qf, kf, vf)
    ref_s = O.sparse_prefill(op, qf, kf, vf, rp.astype(np.int64), bi)
    do, so, dl, sl = d_out.cpu().numpy(), s_out.cpu().numpy(), d_lse.cpu().numpy(), s_lse.cpu().numpy()
    spiked = 0
    for (h, gt), (Or, lr) in ref_d.items():
        r0, n = H.tile_rows(op, gt)
        assert np.abs(do[r0:r0 + n, h] - Or).max() <= H.OUT_ATOL_BF16, (h, gt)
        assert H.lse_close(dl[h, r0:r0 + n], lr, H.LSE_ATOL_BF16), (h, gt)
        Os, ls = ref_s[(h, gt)]
        assert np.abs(so[r0:r0 + n, h] - Os).max() <= H.OUT_ATOL_BF16, (h, gt)
        assert H.lse_close(sl[h, r0:r0 + n], ls, H.LSE_ATOL_BF16), (h, gt)
        spiked += int(lr.max() > 50)
    assert spiked >= 4  # the spikes reach several tiles of both KV heads


def test_pair_kernel_redo_is_per_head():
    """Group-shared lists run two heads of a group per workgroup. A key whose logit
    exceeds every logit of the first stage by 60 nats for one head of each pair only
    (that head's queries carry the spike channel, the other's do not) makes that head
    alone recompute with the exact running max: the two-head kernel's output equals the
    one-head kernel's bit for bit, under both schedules, and the oracle's."""
    import dataclasses
    import torch
    w = synth.small_workload(n_q=300, n_k=428, hq=4, hkv=2, d=128, block=128, dtype="bf16", seed=23)
    inp = synth.make(w)
    q = synth.bf16_bits_to_f32(inp.q).copy()
    k = synth.bf16_bits_to_f32(inp.k).copy()
    d = w.head_dim
    q[:, :, d - 1] = 0.0
    q[:, 0, d - 1] = 1.0   # group 0: head 0 sees the spike, head 1 does not
    q[:, 3, d - 1] = 1.0   # group 1: head 3 sees it, head 2 does not
    k[:, :, d - 1] = 0.0
    k[300, 0, d - 1] = 60.0 * math.sqrt(d)
    k[400, 1, d - 1] = 60.0 * math.sqrt(d)
    inp = dataclasses.replace(inp, q=synth.round_to_bf16_bits(q), k=synth.round_to_bf16_bits(k))
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    tl = O.tiles(op)
    G = op.group
    first = {t.gtile: (list(range(t.diag + 1)) if t.gtile % 2 == 0 else sorted({0, 2, t.diag} & set(range(t.diag + 1))))
             for t in tl}
    rows = [first[t.gtile] for h in range(op.num_heads_q) for t in tl]
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    bi = np.array([b for r in rows for b in r] + [0], np.int32)
    rpd, bid = torch.from_numpy(rp).cuda(), torch.from_numpy(bi).cuda()
    say("two-head kernel: per-head lazy-reference decisions")
    g_out, g_lse = L.sparse_prefill_group(gp, qd, kd, vd, rpd, bid, out_dtype="fp32")
    g_out2, g_lse2 = L.sparse_prefill_group(gp, qd, kd, vd, rpd, bid, out_dtype="fp32", workspace=None)
    s_out, s_lse = L.sparse_prefill(gp, qd, kd, vd, rpd, bid, out_dtype="fp32")
    _sync()
    assert torch.equal(g_out, s_out) and torch.equal(g_lse, s_lse)
    assert torch.equal(g_out2, s_out) and torch.equal(g_lse2, s_lse)
    qf, kf, vf = H.f64(inp)
    ref = O.sparse_prefill(op, qf, kf, vf, rp.astype(np.int64), bi)
    go, gl = g_out.cpu().numpy(), g_lse.cpu().numpy()
    spiked = {h: 0 for h in range(op.num_heads_q)}
    for (h, gt), (Os, ls) in ref.items():
        r0, n = H.tile_rows(op, gt)
        assert np.abs(go[r0:r0 + n, h] - Os).max() <= H.OUT_ATOL_BF16, (h, gt)
        assert H.lse_close(gl[h, r0:r0 + n], ls, H.LSE_ATOL_BF16), (h, gt)
        spiked[h] += int(ls.max() > 50)
    assert spiked[0] >= 1 and spiked[3] >= 1 and spiked[1] == 0 and spiked[2] == 0, spiked


def test_bf16_output_is_rounded_fp32_output():
    import torch
    w = _small(SMALL[1], seed=4)
    inp = synth.make(w)
    gp, _ = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    say("bf16 output")
    o32, l32 = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    o16, l16 = L.dense_prefill(gp, qd, kd, vd, out_dtype="bf16")
    _sync()
    assert torch.equal(o32.to(torch.bfloat16).view(torch.int16), o16.view(torch.int16))
    assert torch.equal(l32, l16)


# ---------------------------------------------------------------------------
# selector on small problems
# ---------------------------------------------------------------------------

SEL = [
    # (n_q, n_k, hq, hkv, d, B, dtype, seqs), sink_offset, n_local
    ((300, 428, 4, 1, 64, 64, "bf16", 1), 6.0, 1),
    ((300, 428, 8, 2, 128, 128, "bf16", 1), 6.0, 1),
    ((257, 641, 10, 2, 128, 64, "bf16", 1), 5.0, 2),
    ((300, 428, 2, 1, 64, 64, "fp32", 1), 6.0, 1),
    ((100, 356, 4, 1, 128, 128, "bf16", 3), 6.0, 1),
    ((64, 4160, 2, 1, 64, 64, "bf16", 1), 7.0, 1),
    # more than 1024 visible blocks: the threshold reads the records from the workspace
    ((128, 66048, 2, 1, 64, 64, "bf16", 1), 6.0, 1),
]


def check_selection(w, inp, gp, op, r, which, q, k, v, gpu_dense=None, gpu_sparse=None, mode="poem", taus=None):
    """Scores, masks (with exemptions) and the bound theorem on the (h, gtile) pairs in which.

    mode "poem": the triangle bound at the cut is <= tau and bounds each sampled row's
    error. mode "mass" (taus: omitted-mass budgets): each sampled row's omitted mass
    on the GPU's mask is <= eps, matches the reported row value, and its error is at
    most 2 R delta (BFLA Appendix B.1)."""
    T = L.num_tiles(gp)
    taus = inp.tau if taus is None else taus
    rp, bi = H.csr_rows(r["row_ptr"], r["block_idx"])
    scores = r["tile_scores"].cpu().numpy()
    bounds = r["row_bound"].cpu().numpy()
    sels = O.select(op, q, k, v, taus, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, which=which, mode=mode)
    n_cand = n_match = 0
    worst_score = worst_unfloored = worst_mand = 0.0
    detail = {}
    for (h, gt), sel in sels.items():
        tau = float(taus[h])
        n_vis = sel.tile.diag + 1
        se, sm, info = H.score_errors(sel, scores[h, gt], tau)
        worst_score = max(worst_score, se)
        worst_unfloored = max(worst_unfloored, info.get("unfloored", 0.0))
        worst_mand = max(worst_mand, sm)
        assert se <= H.score_rtol(w.dtype), (h, gt, se, info)
        assert sm <= H.MANDATORY_SCORE_RTOL, (h, gt, sm)
        assert np.all(scores[h, gt, n_vis:] == -1.0)
        kept = H.retained(rp, bi, h * T + gt)
        assert kept == sorted(kept) and len(set(kept)) == len(kept)
        assert set(sel.mandatory) <= set(kept)
        nc, nm, bad = H.mask_agreement(sel, kept, tau, tau / n_vis, detail=detail)
        n_cand += nc
        n_match += nm
        assert not bad, (h, gt, bad)
        # the bound theorem for each sampled row, exact arithmetic on the GPU's mask
        t = sel.tile
        od, _ = O.tile_attention(op, q, k, v, h, t)
        osp, _ = O.tile_attention(op, q, k, v, h, t, kept)
        dropped = [b for b in range(t.diag + 1) if b not in set(kept)]
        for j, row in enumerate(sel.rows):
            err = float(np.linalg.norm(od[row] - osp[row]))
            b = float(bounds[h, gt, j])
            assert b <= tau * (1 + 1e-6), (h, gt, j, b, tau)
            if mode == "mass":
                delta = float(sel.m[j, dropped].sum())
                assert abs(b - delta) <= H.NEAR_REL * max(delta, tau / (t.diag + 1)), (h, gt, j, b, delta)
                R = float(np.linalg.norm(v[t.k_row0:t.k_row0 + t.pos0 + row + 1, h // op.group], axis=1).max())
                assert err <= 2 * R * delta * (1 + 1e-9) + 1e-12, (h, gt, j, err, delta, R)
                b = 2 * R * delta
            else:
                assert err <= b * (1 + 1e-3) + 1e-6, (h, gt, j, err, b)
            if gpu_dense is not None:
                ge = float(np.linalg.norm(gpu_dense[t.q_row0 + row, h].astype(np.float64) -
                                          gpu_sparse[t.q_row0 + row, h].astype(np.float64)))
                assert ge <= b * (1 + 1e-3) + 2e-4, (h, gt, j, ge, b)
        assert np.all(bounds[h, gt, len(sel.rows):] == -1.0)
    say("  worst candidate score error unfloored", worst_unfloored, "mandatory", worst_mand,
        "mismatches under the score-only exemption", detail.get("score_only_bad", 0))
    return n_cand, n_match, worst_score


@pytest.mark.parametrize("case,sink,n_local", SEL, ids=lambda x: str(x))
def test_selector_matches_oracle(case, sink, n_local):
    w = _small(case, seed=5).with_(sink_offset=sink, n_local_blocks=n_local)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    say("selector", case, sink, n_local)
    r = L.select(gp, qd, kd, vd, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True)
    d_out, _ = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    s_out, _ = L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
    _sync()
    q, k, v = H.f64(inp)
    which = [(h, t.gtile) for h in range(op.num_heads_q) for t in O.tiles(op)]
    nc, nm, ws = check_selection(w, inp, gp, op, r, which, q, k, v, d_out.cpu().numpy(), s_out.cpu().numpy())
    say("  candidates", nc, "agreement", nm / max(nc, 1), "worst score rel err", ws)


NEAR = [
    # case, share of clusters whose values equal the sink's
    ((300, 428, 8, 2, 128, 128, "bf16", 1), 0.5),
    ((256, 4096, 8, 2, 128, 128, "bf16", 1), 1.0),
    ((300, 428, 2, 1, 64, 64, "fp32", 1), 0.5),
]


@pytest.mark.parametrize("case,near", NEAR, ids=lambda x: str(x))
def test_selector_near_output_values(case, near):
    """The selector where blocks' values sit at the output (the regime the note's
    three-block example describes): U_b - L_b o then cancels for heavy blocks, and
    their small scores must still meet the gate; masks, bounds and errors as above."""
    w = _small(case, seed=13).with_(near_output=near)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    say("selector near-output", case, near)
    r = L.select(gp, qd, kd, vd, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True)
    d_out, _ = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    s_out, _ = L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
    _sync()
    q, k, v = H.f64(inp)
    which = [(h, t.gtile) for h in range(op.num_heads_q) for t in O.tiles(op)]
    if len(which) > 96:
        which = H.stratified_tiles(op, sorted({0, op.num_heads_q - 1}), per_head=24, seed=13)
    nc, nm, ws = check_selection(w, inp, gp, op, r, which, q, k, v, d_out.cpu().numpy(), s_out.cpu().numpy())
    say("  candidates", nc, "agreement", nm / max(nc, 1), "worst score rel err", ws)


def _scale_value_blocks(inp, w, lo, hi, seed, p_zero=0.0):
    """V with each (key block, KV head) multiplied by 2^k, k uniform on lo..hi: exact in
    bf16, and it spans far more than fp16's range, so the fp16 copy of V that the
    selector's passes read must take a scale per block. With p_zero, that share of the
    blocks (never block 0) is all zeros instead."""
    import dataclasses
    rng = np.random.default_rng(seed)
    v = synth.bf16_bits_to_f32(inp.v) if inp.is_bf16 else inp.v.astype(np.float32)
    B = w.block_size
    out = v.copy()
    k0 = 0
    for nk in w.seqlens_k:
        for b0 in range(0, nk, B):
            for g in range(w.num_heads_kv):
                f = np.float32(2.0 ** int(rng.integers(lo, hi + 1)))
                if b0 > 0 and rng.uniform() < p_zero:
                    f = np.float32(0.0)
                out[k0 + b0:k0 + min(b0 + B, nk), g] *= f
        k0 += nk
    out_v = synth.round_to_bf16_bits(out) if inp.is_bf16 else out
    if inp.is_bf16:
        assert np.array_equal(synth.bf16_bits_to_f32(out_v), out)  # the scaling is exact
    return dataclasses.replace(inp, v=out_v)


SCALES = [
    # case, block scale exponents lo..hi, share of all-zero blocks
    ((300, 428, 8, 2, 128, 128, "bf16", 1), 20, 20, 0.0),
    ((300, 428, 8, 2, 128, 128, "bf16", 1), -24, -24, 0.0),
    ((300, 428, 8, 2, 128, 128, "bf16", 1), -20, 20, 0.0),
    ((256, 4096, 8, 2, 128, 128, "bf16", 1), -20, 20, 0.0),
    ((257, 641, 10, 2, 128, 64, "bf16", 1), -12, 12, 0.0),
    ((256, 4096, 8, 2, 128, 128, "bf16", 1), -16, 16, 0.3),
]


@pytest.mark.parametrize("case,lo,hi,p_zero", SCALES, ids=lambda x: str(x))
def test_selector_value_scales(case, lo, hi, p_zero):
    """Scores and masks when V's blocks range from 2^-24 to 2^20 in scale, or are all
    zero (both passes' fp16 V carries one power-of-two scale per key block and KV head,
    and pass 1 moves its accumulator between the blocks' scales)."""
    w = _small(case, seed=11)
    inp = _scale_value_blocks(synth.make(w), w, lo, hi, seed=3, p_zero=p_zero)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    say("selector with V block scales 2^", lo, "..", hi)
    r = L.select(gp, qd, kd, vd, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True)
    _sync()
    q, k, v = H.f64(inp)
    which = [(h, t.gtile) for h in range(op.num_heads_q) for t in O.tiles(op)]
    nc, nm, ws = check_selection(w, inp, gp, op, r, which, q, k, v)
    say("  candidates", nc, "agreement", nm / max(nc, 1), "worst score rel err", ws)


MASS = [
    # case, sink_offset, n_local, eps (omitted-mass budget)
    ((300, 428, 4, 1, 64, 64, "bf16", 1), 6.0, 1, 0.002),
    ((300, 428, 8, 2, 128, 128, "bf16", 1), 6.0, 1, 0.004),
    ((257, 641, 10, 2, 128, 64, "bf16", 1), 5.0, 2, 0.02),
    ((300, 428, 2, 1, 64, 64, "fp32", 1), 6.0, 1, 0.002),
    ((100, 356, 4, 1, 128, 128, "bf16", 3), 6.0, 1, 0.003),
    ((64, 4160, 2, 1, 64, 64, "bf16", 1), 7.0, 1, 0.001),
    ((128, 66048, 2, 1, 64, 64, "bf16", 1), 6.0, 1, 0.002),  # > 1024 visible blocks
]


@pytest.mark.parametrize("case,sink,n_local,eps", MASS, ids=lambda x: str(x))
def test_mass_selector_matches_oracle(case, sink, n_local, eps):
    """poem_select_mass against the oracle's mass-only selector."""
    w = _small(case, seed=7).with_(sink_offset=sink, n_local_blocks=n_local)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    eps_h = [eps * (1 + 0.5 * (h % 3)) for h in range(w.num_heads_q)]
    say("mass selector", case, sink, n_local, eps)
    r = L.select(gp, qd, kd, vd, eps_h, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True,
                 mode="mass")
    d_out, _ = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    s_out, _ = L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
    _sync()
    q, k, v = H.f64(inp)
    which = [(h, t.gtile) for h in range(op.num_heads_q) for t in O.tiles(op)]
    # the ranking key the GPU reports is the tile mass, in both score outputs
    assert np.array_equal(r["tile_scores"].cpu().numpy(), r["tile_mass"].cpu().numpy())
    nc, nm, ws = check_selection(w, inp, gp, op, r, which, q, k, v, d_out.cpu().numpy(), s_out.cpu().numpy(),
                                 mode="mass", taus=eps_h)
    say("  candidates", nc, "agreement", nm / max(nc, 1), "worst mass rel err", ws)


@pytest.mark.parametrize("dt,d", [("fp32", 64), ("bf16", 128)])
def test_selector_unsplit_sweeps(dt, d):
    """64 one-tile sequences x 16 KV heads: 1024 tile groups, enough that no sweep is
    split into block chunks, so the single-chunk epilogues of pass 1 run (small problems
    otherwise always split). POEM and mass-only selectors against the oracle."""
    case = (64, 128, 16, 16, d, 64, dt, 1)
    w = _small(case, seed=11).with_(seqlens_q=tuple([64] * 64),
                                    seqlens_k=tuple(64 + 64 * (i % 4) for i in range(64)), sink_offset=6.0)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    q, k, v = H.f64(inp)
    which = [(h, t.gtile) for h in range(op.num_heads_q) for t in O.tiles(op)]
    d_out, _ = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    for mode, taus in (("poem", None), ("mass", [0.002 * (1 + 0.5 * (h % 3)) for h in range(w.num_heads_q)])):
        say("unsplit sweeps", dt, d, mode)
        r = L.select(gp, qd, kd, vd, inp.tau if taus is None else taus, w.n_sink_blocks, w.n_local_blocks,
                     w.rows_per_tile, diagnostics=True, mode=mode)
        s_out, _ = L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
        _sync()
        nc, nm, ws = check_selection(w, inp, gp, op, r, which, q, k, v, d_out.cpu().numpy(), s_out.cpu().numpy(),
                                     mode=mode, taus=taus)
        say("  candidates", nc, "agreement", nm / max(nc, 1), "worst score rel err", ws)


LIMITS = [
    # case, rows_per_tile: the C ABI's maxima
    ((64, 262144, 2, 1, 64, 64, "bf16", 1), 8),    # POEM_MAX_VISIBLE_BLOCKS: 4096 blocks of 64 keys
    ((64, 262144, 2, 1, 64, 64, "fp32", 1), 8),
    ((300, 428, 8, 2, 128, 128, "bf16", 1), 32),   # POEM_MAX_ROWS_PER_TILE with G = 4 (128 columns)
    ((100, 228, 128, 32, 64, 64, "bf16", 1), 8),   # POEM_MAX_HEADS_Q
]


@pytest.mark.parametrize("case,S", LIMITS, ids=lambda x: str(x))
def test_selector_at_limits(case, S):
    """The selector (and the attention on its lists) at the largest sizes the C ABI
    accepts: a tile seeing 4096 key blocks (pass 1 in eight chunks of 512, the threshold
    reading its records from the workspace), 32 sampled rows per tile, 128 query heads."""
    w = _small(case, seed=13).with_(sink_offset=7.0, rows_per_tile=S)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    say("selector at limits", case, S)
    r = L.select(gp, qd, kd, vd, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True)
    d_out, _ = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    s_out, _ = L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
    _sync()
    assert L.max_visible_blocks(gp) <= 4096
    q, k, v = H.f64(inp)
    which = [(h, t.gtile) for h in range(op.num_heads_q) for t in O.tiles(op)]
    nc, nm, ws = check_selection(w, inp, gp, op, r, which, q, k, v, d_out.cpu().numpy(), s_out.cpu().numpy())
    say("  candidates", nc, "agreement", nm / max(nc, 1), "worst score rel err", ws)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_selector_degenerate(dt):
    """A batch whose middle sequence has no queries, at tau = 0 (any discard has a
    positive bound, so every visible block is kept) and tau = 1e30 (every candidate is
    discarded, only the mandatory blocks stay): the kept sets equal the oracle's, the
    retained-block attention equals the oracle's on them, the empty sequence writes
    nothing and its tiles do not exist in the CSR."""
    import torch
    B, d = (128, 128) if dt == "bf16" else (64, 64)
    w = _small((100, 356, 4, 1, d, B, dt, 1), seed=17).with_(
        seqlens_q=(100, 0, 66), seqlens_k=(100 + 6 * B, B, 66 + 6 * B), sink_offset=6.0)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    q, k, v = H.f64(inp)
    T = L.num_tiles(gp)
    tl = O.tiles(op)
    assert T == len(tl) and all(t.seq != 1 for t in tl)
    which = [(h, t.gtile) for h in range(op.num_heads_q) for t in tl]
    for tau in (0.0, 1e30):
        taus = [tau] * w.num_heads_q
        say("degenerate", dt, "tau", tau)
        r = L.select(gp, qd, kd, vd, taus, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True)
        sentinel = 123.0
        out = torch.full((gp.total_q, gp.num_heads_q, d), sentinel, dtype=torch.float32, device="cuda")
        lse = torch.full((gp.num_heads_q, gp.total_q), sentinel, dtype=torch.float32, device="cuda")
        L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32", out=out, lse=lse)
        _sync()
        assert gp.total_q == 166
        rp, bi = H.csr_rows(r["row_ptr"], r["block_idx"])
        out = out.cpu().numpy()
        sels = O.select(op, q, k, v, taus, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, which=which)
        for (h, gt), sel in sels.items():
            kept = H.retained(rp, bi, h * T + gt)
            t = sel.tile
            want = list(range(t.diag + 1)) if tau == 0.0 else sorted(sel.mandatory)
            assert sel.retained == want, (tau, h, gt, sel.retained, want)
            assert kept == want, (tau, h, gt, kept, want)
            Or, _ = O.tile_attention(op, q, k, v, h, t, kept)
            atol = H.OUT_ATOL_FP32 if dt == "fp32" else H.OUT_ATOL_BF16
            assert np.abs(out[t.q_row0:t.q_row0 + t.n_rows, h] - Or).max() <= atol, (tau, h, gt)
        # every output row belongs to a tile of sequence 0 or 2 and was written
        assert not np.any(out == sentinel)


def check_group_selection(w, taus, gp, op, r, which_units, q, k, v, gpu_dense=None, gpu_sparse=None):
    """poem_select_group against the oracle's group selection on (KV head, gtile) units:
    group scores, the shared list under every head, masks with exemptions, and for
    every sampled row (of its own head) error <= bound <= that head's tau."""
    T = L.num_tiles(gp)
    G = op.group
    rp, bi = H.csr_rows(r["row_ptr"], r["block_idx"])
    scores = r["tile_scores"].cpu().numpy()
    bounds = r["row_bound"].cpu().numpy()
    which = [(g * G, gt) for (g, gt) in which_units]
    sels = O.select(op, q, k, v, taus, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, which=which,
                    mode="group")
    n_cand = n_match = 0
    worst = worst_unfloored = worst_mand = 0.0
    detail = {}
    for (h0, gt), sel in sels.items():
        t = sel.tile
        n_vis = t.diag + 1
        tmin = min(float(taus[h]) for h in range(h0, h0 + G))
        kept = H.retained(rp, bi, h0 * T + gt)
        for h in range(h0, h0 + G):  # one list, the same scores and bounds under every head
            assert H.retained(rp, bi, h * T + gt) == kept
            assert np.array_equal(scores[h, gt], scores[h0, gt])
            assert np.array_equal(bounds[h, gt], bounds[h0, gt])
        se, sm, info = H.score_errors(sel, scores[h0, gt], tmin)
        worst = max(worst, se)
        worst_unfloored = max(worst_unfloored, info.get("unfloored", 0.0))
        worst_mand = max(worst_mand, sm)
        assert se <= H.score_rtol(w.dtype), (h0, gt, se, info)
        assert sm <= H.MANDATORY_SCORE_RTOL, (h0, gt, sm)
        assert np.all(scores[h0, gt, n_vis:] == -1.0)
        assert kept == sorted(kept) and len(set(kept)) == len(kept)
        assert set(sel.mandatory) <= set(kept)
        nc, nm, bad = H.mask_agreement(sel, kept, tmin, tmin / n_vis, target=0.0, detail=detail)
        n_cand += nc
        n_match += nm
        assert not bad, (h0, gt, bad)
        for j, (row, hh) in enumerate(zip(sel.rows, sel.heads)):
            od, _ = O.tile_attention(op, q, k, v, hh, t)
            osp, _ = O.tile_attention(op, q, k, v, hh, t, kept)
            err = float(np.linalg.norm(od[row] - osp[row]))
            b = float(bounds[h0, gt, j])
            assert b <= float(taus[hh]) * (1 + 1e-6), (h0, gt, j, b, taus[hh])
            assert err <= b * (1 + 1e-3) + 1e-6, (h0, gt, j, err, b)
            if gpu_dense is not None:
                ge = float(np.linalg.norm(gpu_dense[t.q_row0 + row, hh].astype(np.float64) -
                                          gpu_sparse[t.q_row0 + row, hh].astype(np.float64)))
                assert ge <= b * (1 + 1e-3) + 2e-4, (h0, gt, j, ge, b)
        assert np.all(bounds[h0, gt, len(sel.rows):] == -1.0)
    say("  worst candidate score error unfloored", worst_unfloored, "mandatory", worst_mand,
        "mismatches under the score-only exemption", detail.get("score_only_bad", 0))
    return n_cand, n_match, worst


GROUP = [
    # case, sink_offset, n_local, rows_per_tile (per KV head and tile)
    ((300, 428, 4, 1, 64, 64, "bf16", 1), 6.0, 1, 8),
    ((300, 428, 8, 2, 128, 128, "bf16", 1), 6.0, 1, 8),
    ((257, 641, 10, 2, 128, 64, "bf16", 1), 5.0, 2, 8),
    ((300, 428, 4, 2, 64, 64, "fp32", 1), 6.0, 1, 4),
    ((100, 356, 4, 1, 128, 128, "bf16", 3), 6.0, 1, 5),
    ((64, 4160, 4, 1, 64, 64, "bf16", 1), 7.0, 1, 16),
]


@pytest.mark.parametrize("case,sink,n_local,S", GROUP, ids=lambda x: str(x))
def test_group_selector_matches_oracle(case, sink, n_local, S):
    w = _small(case, seed=9).with_(sink_offset=sink, n_local_blocks=n_local, rows_per_tile=S)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    say("group selector", case, sink, n_local, S)
    r = L.select(gp, qd, kd, vd, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True,
                 mode="group")
    d_out, _ = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    s_out, _ = L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
    _sync()
    q, k, v = H.f64(inp)
    units = [(g, t.gtile) for g in range(op.num_heads_kv) for t in O.tiles(op)]
    nc, nm, ws = check_group_selection(w, inp.tau, gp, op, r, units, q, k, v, d_out.cpu().numpy(),
                                       s_out.cpu().numpy())
    say("  candidates", nc, "agreement", nm / max(nc, 1), "worst score rel err", ws)
    check_group_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"])


def check_group_prefill(gp, qd, kd, vd, row_ptr, block_idx):
    """poem_sparse_prefill_group on a shared-list CSR equals poem_sparse_prefill bit for
    bit, and reads only each group's first-head rows: with the other heads' rows emptied
    the result is the same, under both schedules (count-ordered queue and static)."""
    import torch
    s_out, s_lse = L.sparse_prefill(gp, qd, kd, vd, row_ptr, block_idx, out_dtype="fp32")
    g_out, g_lse = L.sparse_prefill_group(gp, qd, kd, vd, row_ptr, block_idx, out_dtype="fp32")
    rp, bi = H.csr_rows(row_ptr, block_idx)
    T = L.num_tiles(gp)
    G = gp.num_heads_q // gp.num_heads_kv
    rows, ids = [0], []
    for r in range(gp.num_heads_q * T):
        if (r // T) % G == 0:
            ids.extend(bi[rp[r]:rp[r + 1]].tolist())
        rows.append(len(ids))
    rp1 = torch.tensor(rows, dtype=torch.int32, device=qd.device)
    bi1 = torch.tensor(ids + [0], dtype=torch.int32, device=qd.device)
    f_out, f_lse = L.sparse_prefill_group(gp, qd, kd, vd, rp1, bi1, out_dtype="fp32")
    h_out, h_lse = L.sparse_prefill_group(gp, qd, kd, vd, rp1, bi1, out_dtype="fp32", workspace=None)
    _sync()
    assert torch.equal(g_out, s_out) and torch.equal(g_lse, s_lse)
    assert torch.equal(f_out, s_out) and torch.equal(f_lse, s_lse)
    assert torch.equal(h_out, s_out) and torch.equal(h_lse, s_lse)


def check_practical(w, eps_h, wt, rho, gp, op, r, which, q, k, v):
    """poem_select_practical against the oracle: pooled masses (1e-3 gate), rerank keys
    where defined, the retained set with exemptions at the preselection boundary (mass
    order) and at the kept boundary (rerank order), and the per-row omitted masses of
    the GPU's mask."""
    T = L.num_tiles(gp)
    rp, bi = H.csr_rows(r["row_ptr"], r["block_idx"])
    keys = r["tile_scores"].cpu().numpy()
    mass = r["tile_mass"].cpu().numpy()
    bounds = r["row_bound"].cpu().numpy()
    sels = O.select(op, q, k, v, eps_h, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, which=which,
                    mode="practical", practical=dict(w=wt, rho=rho))
    n_cand = n_match = 0
    for (h, gt), sel in sels.items():
        t = sel.tile
        n_vis = t.diag + 1
        eps = float(eps_h[h])
        floor = max(eps, 1e-3) / n_vis
        mbar, Ibar = sel.mass, sel.I.mean(axis=0)
        g_m = mass[h, gt, :n_vis].astype(np.float64)
        assert np.all(np.abs(g_m - mbar) <= H.NEAR_REL * np.maximum(mbar, floor)), (h, gt)
        assert np.all(mass[h, gt, n_vis:] == -1.0) and np.all(keys[h, gt, n_vis:] == -1.0)
        cand = [b for b in range(n_vis) if b not in set(sel.mandatory)]
        ok = [b for b in cand if mbar[b] > floor and Ibar[b] > floor]
        g_k = keys[h, gt, :n_vis].astype(np.float64)
        assert np.all(np.abs(g_k[ok] - sel.score[ok]) <= 4e-3 * (1 + abs(wt))), (h, gt)
        pre, order, kept = O.practical_retain(mbar, Ibar, sel.mandatory, cand, eps, wt, rho)
        by_mass = sorted(cand, key=lambda b: (-float(mbar[b]), int(b)))
        cum_m = np.cumsum([mbar[b] for b in by_mass]) if by_mass else np.zeros(0)
        need = rho * (cum_m[-1] if len(cum_m) else 0.0)
        pos_m = {b: j for j, b in enumerate(by_mass)}
        pos_r = {b: j for j, b in enumerate(order)}
        before = {b: float(sum(mbar[x] for x in sel.mandatory) + sum(mbar[x] for x in order[:j]))
                  for j, b in enumerate(order)}
        target = (1 - eps) * float(mbar.sum())
        nb_m = [by_mass[j] for j in (len(pre) - 1, len(pre)) if 0 <= j < len(by_mass)]
        nb_r = [order[j] for j in (len(kept) - 1, len(kept)) if 0 <= j < len(order)]
        got = H.retained(rp, bi, h * T + gt)
        assert got == sorted(got) and set(sel.mandatory) <= set(got)
        for b in cand:
            n_cand += 1
            if (b in got) == (b in sel.retained):
                n_match += 1
                continue
            ex = any(abs(mbar[b] - mbar[x]) <= H.NEAR_REL * max(mbar[x], floor) for x in nb_m)
            j = pos_m[b]
            ex |= any(abs(cum_m[jj] - need) <= H.NEAR_REL * max(need, floor) for jj in (j - 1, j) if jj >= 0)
            if b in pos_r:
                ex |= any(abs(sel.score[b] - sel.score[x]) <= 4e-3 * (1 + abs(wt)) for x in nb_r)
                ex |= abs(before[b] - target) <= H.NEAR_REL * max(eps, floor)
            assert ex, (h, gt, b, b in got, b in sel.retained)
        dropped = [b for b in range(n_vis) if b not in set(got)]
        for j in range(len(sel.rows)):
            delta = float(sel.m[j, dropped].sum())
            assert abs(float(bounds[h, gt, j]) - delta) <= H.NEAR_REL * max(delta, floor), (h, gt, j)
        if [b for b in order if b not in set(got)]:
            assert float(sel.m[:, dropped].sum(axis=1).mean()) <= eps * (1 + H.NEAR_REL) + floor
    return n_cand, n_match


PRACTICAL = [
    # case, sink_offset, n_local, eps, weight, presel_fraction
    ((300, 428, 4, 1, 64, 64, "bf16", 1), 6.0, 1, 0.002, 0.5, 0.95),
    ((300, 428, 8, 2, 128, 128, "bf16", 1), 6.0, 1, 0.004, 1.0, 0.99),
    ((257, 641, 10, 2, 128, 64, "bf16", 1), 5.0, 2, 0.02, 0.0, 1.0),
    ((300, 428, 2, 1, 64, 64, "fp32", 1), 6.0, 1, 0.002, 2.0, 0.9),
    ((100, 356, 4, 1, 128, 128, "bf16", 3), 6.0, 1, 0.003, 0.5, 0.95),
    ((64, 4160, 2, 1, 64, 64, "bf16", 1), 7.0, 1, 0.001, 0.5, 0.95),
]


@pytest.mark.parametrize("case,sink,n_local,eps,wt,rho", PRACTICAL, ids=lambda x: str(x))
def test_practical_selector_matches_oracle(case, sink, n_local, eps, wt, rho):
    w = _small(case, seed=11).with_(sink_offset=sink, n_local_blocks=n_local)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    eps_h = [eps * (1 + 0.5 * (h % 3)) for h in range(w.num_heads_q)]
    say("practical selector", case, sink, n_local, eps, wt, rho)
    r = L.select(gp, qd, kd, vd, eps_h, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True,
                 mode="practical", weight=wt, presel_fraction=rho)
    _sync()
    q, k, v = H.f64(inp)
    which = [(h, t.gtile) for h in range(op.num_heads_q) for t in O.tiles(op)]
    nc, nm = check_practical(w, eps_h, wt, rho, gp, op, r, which, q, k, v)
    say("  candidates", nc, "agreement", nm / max(nc, 1))


# ---------------------------------------------------------------------------
# the workloads at full size
# ---------------------------------------------------------------------------


def test_workload1_full():
    """Single head, d=64, N=2048, fp32, B=64: every tile, every output."""
    w = synth.WORKLOADS[1]
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    say("workload 1 full")
    r = L.select(gp, qd, kd, vd, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True)
    d_out, d_lse = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    s_out, s_lse = L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
    _sync()
    q, k, v = H.f64(inp)
    which = [(0, t.gtile) for t in O.tiles(op)]
    nc, nm, ws = check_selection(w, inp, gp, op, r, which, q, k, v, d_out.cpu().numpy(), s_out.cpu().numpy())
    say("  candidates", nc, "agreement", nm / max(nc, 1), "worst score rel err", ws)
    rp, bi = H.csr_rows(r["row_ptr"], r["block_idx"])
    ref_d = O.dense_prefill(op, q, k, v)
    ref_s = O.sparse_prefill(op, q, k, v, rp, bi)
    do, so = d_out.cpu().numpy(), s_out.cpu().numpy()
    for key in ref_d:
        r0, n = H.tile_rows(op, key[1])
        assert np.abs(do[r0:r0 + n, 0] - ref_d[key][0]).max() <= H.OUT_ATOL_FP32
        assert np.abs(so[r0:r0 + n, 0] - ref_s[key][0]).max() <= H.OUT_ATOL_FP32


@pytest.mark.parametrize("wid", [2, 3, 4, 5])
def test_workload_full_size_sampled(wid):
    """Full-size run in the benchmark's configuration; oracle on stratified tiles."""
    import torch
    w = synth.WORKLOADS[wid]
    say("workload", wid, "generate")
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    say("workload", wid, "select + dense + sparse")
    r = L.select(gp, qd, kd, vd, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True)
    d_out, d_lse = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    s_out, s_lse = L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
    _sync()
    rp, bi = H.csr_rows(r["row_ptr"], r["block_idx"])
    keep = len(bi[:rp[-1]]) / L.csr_capacity(gp)
    say("  keep fraction", keep)
    q, k, v = H.f64(inp)
    heads = sorted({0, w.num_heads_q - 1, w.num_heads_q // 2 + 1})
    which = H.stratified_tiles(op, heads, per_head=3, seed=wid)
    if len(w.seqlens_q) > 1:  # chunked: every sequence's first and last tile, two heads
        tl = O.tiles(op)
        ends = sorted({i for s_ in range(len(w.seqlens_q)) for i in
                       (min(t.gtile for t in tl if t.seq == s_), max(t.gtile for t in tl if t.seq == s_))})
        which = sorted(set(which) | {(h, gt) for h in (0, w.num_heads_q - 1) for gt in ends})
    do, so = d_out.cpu().numpy(), s_out.cpu().numpy()
    del d_out, s_out
    torch.cuda.empty_cache()
    nc, nm, ws = check_selection(w, inp, gp, op, r, which, q, k, v, do, so)
    say("  sampled candidates", nc, "agreement", nm / max(nc, 1), "worst score rel err", ws)
    dl, sl = d_lse.cpu().numpy(), s_lse.cpu().numpy()
    T = L.num_tiles(gp)
    for (h, gt) in which:
        t = O.tiles(op)[gt]
        Od, ld = O.tile_attention(op, q, k, v, h, t)
        ids = H.retained(rp, bi, h * T + gt)
        Os, ls = O.tile_attention(op, q, k, v, h, t, ids)
        r0, n = t.q_row0, t.n_rows
        assert np.abs(do[r0:r0 + n, h] - Od).max() <= H.OUT_ATOL_BF16
        assert np.abs(so[r0:r0 + n, h] - Os).max() <= H.OUT_ATOL_BF16
        assert H.lse_close(dl[h, r0:r0 + n], ld, H.LSE_ATOL_BF16)
        assert H.lse_close(sl[h, r0:r0 + n], ls, H.LSE_ATOL_BF16)


def test_mass_full_size_sampled():
    """poem_select_mass at the 128K layer's full size; oracle on stratified tiles."""
    import torch
    w = synth.WORKLOADS[3]
    say("workload 3 mass-only: generate")
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    eps_h = [0.002] * w.num_heads_q
    say("workload 3 mass-only: select + sparse")
    r = L.select(gp, qd, kd, vd, eps_h, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True,
                 mode="mass")
    s_out, _ = L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
    _sync()
    rp, bi = H.csr_rows(r["row_ptr"], r["block_idx"])
    say("  keep fraction", len(bi[:rp[-1]]) / L.csr_capacity(gp))
    so = s_out.cpu().numpy()
    del s_out
    torch.cuda.empty_cache()
    q, k, v = H.f64(inp)
    which = H.stratified_tiles(op, [0, w.num_heads_q - 1], per_head=3, seed=33)
    nc, nm, ws = check_selection(w, inp, gp, op, r, which, q, k, v, mode="mass", taus=eps_h)
    say("  sampled candidates", nc, "agreement", nm / max(nc, 1), "worst mass rel err", ws)
    T = L.num_tiles(gp)
    for (h, gt) in which[:4]:
        t = O.tiles(op)[gt]
        Os, _ = O.tile_attention(op, q, k, v, h, t, H.retained(rp, bi, h * T + gt))
        assert np.abs(so[t.q_row0:t.q_row0 + t.n_rows, h] - Os).max() <= H.OUT_ATOL_BF16


def test_group_full_size_sampled():
    """poem_select_group at the 128K layer's full size; oracle on stratified units."""
    import torch
    w = synth.WORKLOADS[3]
    say("workload 3 group-shared: generate")
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    say("workload 3 group-shared: select + sparse")
    r = L.select(gp, qd, kd, vd, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True,
                 mode="group")
    s_out, _ = L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
    _sync()
    rp, bi = H.csr_rows(r["row_ptr"], r["block_idx"])
    say("  keep fraction", len(bi[:rp[-1]]) / L.csr_capacity(gp))
    so = s_out.cpu().numpy()
    del s_out
    torch.cuda.empty_cache()
    q, k, v = H.f64(inp)
    which = H.stratified_tiles(op, [0, w.num_heads_q - 1], per_head=3, seed=44)
    units = sorted({(h // op.group, gt) for (h, gt) in which})
    nc, nm, ws = check_group_selection(w, inp.tau, gp, op, r, units, q, k, v)
    say("  sampled candidates", nc, "agreement", nm / max(nc, 1), "worst score rel err", ws)
    T = L.num_tiles(gp)
    for (g, gt) in units[:3]:
        t = O.tiles(op)[gt]
        h = g * op.group + 1
        Os, _ = O.tile_attention(op, q, k, v, h, t, H.retained(rp, bi, h * T + gt))
        assert np.abs(so[t.q_row0:t.q_row0 + t.n_rows, h] - Os).max() <= H.OUT_ATOL_BF16


def test_practical_full_size_sampled():
    """poem_select_practical at the 128K layer's full size; oracle on stratified tiles."""
    w = synth.WORKLOADS[3]
    say("workload 3 practical: generate")
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    eps_h = [0.002] * w.num_heads_q
    say("workload 3 practical: select")
    r = L.select(gp, qd, kd, vd, eps_h, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True,
                 mode="practical", weight=0.5, presel_fraction=0.95)
    _sync()
    rp, bi = H.csr_rows(r["row_ptr"], r["block_idx"])
    say("  keep fraction", len(bi[:rp[-1]]) / L.csr_capacity(gp))
    q, k, v = H.f64(inp)
    which = H.stratified_tiles(op, [0, w.num_heads_q - 1], per_head=3, seed=55)
    nc, nm = check_practical(w, eps_h, 0.5, 0.95, gp, op, r, which, q, k, v)
    say("  sampled candidates", nc, "agreement", nm / max(nc, 1))


def test_workload3_every_tile_of_four_heads():
    """The 128K layer in the benchmark's configuration. The selector on every tile of
    query heads 0..3 (the KV head 0 group; 4 x 1,024 tiles): scores within 1e-3, masks
    with exemptions, per-row bounds within tau, and at every sampled row the error of
    the sparse output on the GPU's mask (fp64, and the GPU's own dense and sparse
    outputs) within its bound. Then the dense and sparse outputs and LSE on every row
    of 32 tiles of those heads, the three longest tiles of each head among them. The
    oracle runs in spawned worker processes on the group's sub-problem."""
    import torch
    from . import oracle_pool as P
    w = synth.WORKLOADS[3]
    say("workload 3 every tile of four heads: generate")
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    say("workload 3 every tile of four heads: select + dense + sparse")
    r = L.select(gp, qd, kd, vd, inp.tau, w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile, diagnostics=True)
    d_out, d_lse = L.dense_prefill(gp, qd, kd, vd, out_dtype="fp32")
    s_out, s_lse = L.sparse_prefill(gp, qd, kd, vd, r["row_ptr"], r["block_idx"], out_dtype="fp32")
    _sync()
    T = L.num_tiles(gp)
    G = op.group
    rp, bi = H.csr_rows(r["row_ptr"], r["block_idx"])
    tl = O.tiles(op)
    sub = O.Problem(tuple(w.seqlens_q), tuple(w.seqlens_k), G, 1, w.head_dim, w.block_size)
    q_sub = synth.to_f64(inp.q[:, 0:G])
    k_sub, v_sub = synth.to_f64(inp.k[:, 0:1]), synth.to_f64(inp.v[:, 0:1])
    jobs = [(h, gt, float(inp.tau[h]), w.n_sink_blocks, w.n_local_blocks, w.rows_per_tile,
             H.retained(rp, bi, h * T + gt)) for h in range(G) for gt in range(T)]
    rng = np.random.default_rng(31)
    out_tiles = []
    for h in range(G):
        picks = {0, T - 3, T - 2, T - 1} | set((1 + rng.choice(T - 4, size=4, replace=False)).tolist())
        out_tiles += [(h, int(gt)) for gt in sorted(picks)]
    say("  oracle on", len(jobs), "tiles and", len(out_tiles), "output tiles")
    with P.GroupPool(sub, q_sub, k_sub, v_sub) as pool:
        results = pool.select(jobs)
        attn = pool.attention([(h, gt, H.retained(rp, bi, h * T + gt)) for (h, gt) in out_tiles])
    scores = r["tile_scores"][:G].cpu().numpy()
    bounds = r["row_bound"][:G].cpu().numpy()
    # the sampled rows of every job, from the GPU's dense and sparse outputs
    rows = torch.tensor([tl[j[1]].q_row0 + r_ for j, (sel, _, _) in zip(jobs, results) for r_ in sel.rows],
                        device=d_out.device)
    heads = torch.tensor([j[0] for j, (sel, _, _) in zip(jobs, results) for _ in sel.rows], device=d_out.device)
    g_err = torch.linalg.vector_norm(d_out[rows, heads].double() - s_out[rows, heads].double(), dim=-1).cpu().numpy()
    n_cand = n_match = 0
    worst = worst_mand = worst_unf = 0.0
    detail = {}
    i = 0
    for (h, gt, tau, _, _, _, kept), (sel, err, delta) in zip(jobs, results):
        n_vis = tl[gt].diag + 1
        se, sm, info = H.score_errors(sel, scores[h, gt], tau)
        worst, worst_mand = max(worst, se), max(worst_mand, sm)
        worst_unf = max(worst_unf, info.get("unfloored", 0.0))
        assert se <= H.SCORE_RTOL, (h, gt, se, info)
        assert sm <= H.MANDATORY_SCORE_RTOL, (h, gt, sm)
        assert kept == sorted(kept) and set(sel.mandatory) <= set(kept)
        nc, nm, bad = H.mask_agreement(sel, kept, tau, tau / n_vis, detail=detail)
        n_cand, n_match = n_cand + nc, n_match + nm
        assert not bad, (h, gt, bad)
        for j in range(len(sel.rows)):
            b = float(bounds[h, gt, j])
            assert b <= tau * (1 + 1e-6), (h, gt, j, b)
            assert err[j] <= b * (1 + 1e-3) + 1e-6, (h, gt, j, err[j], b)
            assert g_err[i] <= b * (1 + 1e-3) + 2e-4, (h, gt, j, g_err[i], b)
            i += 1
        assert np.all(bounds[h, gt, len(sel.rows):] == -1.0)
    say("  heads 0..3, tiles", len(jobs), "candidates", n_cand, "agreement", n_match / max(n_cand, 1),
        "worst score", worst, "unfloored", worst_unf, "mandatory", worst_mand,
        "score-only mismatches", detail.get("score_only_bad", 0))
    worst_o = 0.0
    for (h, gt), ((Od, ld), (Os, ls)) in zip(out_tiles, attn):
        t = tl[gt]
        r0, n = t.q_row0, t.n_rows
        go_d = d_out[r0:r0 + n, h].cpu().numpy()
        go_s = s_out[r0:r0 + n, h].cpu().numpy()
        e = max(np.abs(go_d - Od).max(), np.abs(go_s - Os).max())
        worst_o = max(worst_o, e)
        assert e <= H.OUT_ATOL_BF16, (h, gt, e)
        assert H.lse_close(d_lse[h, r0:r0 + n].cpu().numpy(), ld, H.LSE_ATOL_BF16), (h, gt)
        assert H.lse_close(s_lse[h, r0:r0 + n].cpu().numpy(), ls, H.LSE_ATOL_BF16), (h, gt)
    say("  outputs on", len(out_tiles), "tiles: worst max-abs error", worst_o)
