"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each pin is independent of the oracle's own formulas: printed values of the
three-block example, closed forms, invariants, brute force on tiny inputs, and
textbook routines (scipy) for the softmax. A separate test plants plausible
mistakes in the oracle and checks that some pin fails for each of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from oracle import poem_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden", "toy_three_block.json")


def frac(s):
    return float(Fraction(s))


@pytest.fixture(scope="module")
def toy():
    with open(GOLD) as f:
        return json.load(f)


# --- printed values of the three-block example ------------------------------------


def pin_toy_pairs(toy):
    m = [frac(x) for x in toy["masses"]]
    v = [[frac(x)] for x in toy["values"]]
    assert abs(O.dense_output(m, v)[0] - frac(toy["dense_output"])) < 1e-12
    names = toy["blocks"]
    for key, exp in toy["removals"].items():
        D = [names.index(n) for n in key.split(",")]
        out = O.deleted_output(m, v, D)[0]
        assert abs(out - frac(exp["output"])) < 1e-12, key
        err = O.deletion_error(m, v, D)[0]
        assert abs(abs(err) - frac(exp["abs_error"])) < 1e-12, key
        assert abs((frac(toy["dense_output"]) - out) - err) < 1e-12, key
    I = O.proxy_scores(m, v)
    for got, exp in zip(I, toy["proxy_scores"]):
        assert abs(got - frac(exp)) < 1e-12
    assert abs(O.triangle_bound(m, v, [1, 2]) - frac(toy["triangle_bound"]["B,C"])) < 1e-12
    # one deleted block: the bound is tight, I_b / (1 - m_b) = |o - o_tilde| (POEM note, Eq. (4))
    for b in range(3):
        assert abs(O.triangle_bound(m, v, [b]) - abs(O.deletion_error(m, v, [b])[0])) < 1e-12


def pin_toy_shift(toy):
    m = [frac(x) for x in toy["masses"]]
    c = frac(toy["shift"]["c"])
    v = [[frac(x) + c] for x in toy["values"]]
    assert [x[0] for x in v] == [frac(x) for x in toy["shift"]["values"]]
    assert abs(O.dense_output(m, v)[0] - frac(toy["shift"]["dense_output"])) < 1e-12
    assert abs(O.deleted_output(m, v, [1])[0] - frac(toy["shift"]["remove_B_output"])) < 1e-12
    assert abs(abs(O.deletion_error(m, v, [1])[0]) - frac(toy["shift"]["abs_error"])) < 1e-12
    I0 = O.proxy_scores(m, [[frac(x)] for x in toy["values"]])
    assert np.allclose(O.proxy_scores(m, v), I0, atol=1e-12, rtol=0)


def pin_toy_from_logits(toy):
    """One token per block with logits (ln 2, 0, 0) realises the masses exactly."""
    K = np.array([[math.log(2.0)], [0.0], [0.0]])
    V = np.array([[frac(x)] for x in toy["values"]])
    q = np.array([[1.0]])
    o, lse = O.attention_rows(q, K, V, 1.0, [2])
    assert abs(o[0, 0] - frac(toy["dense_output"])) < 1e-12
    assert abs(lse[0] - math.log(4.0)) < 1e-12
    st = O.row_block_stats(q[0], K, V, 1.0, 2, 3, 1)
    assert np.allclose(st["m"], [frac(x) for x in toy["masses"]], atol=1e-12, rtol=0)
    assert np.allclose(st["I"], [frac(x) for x in toy["proxy_scores"]], atol=1e-12, rtol=0)
    # masked softmax without B reproduces the printed sparse output
    o2, _ = O.attention_rows(q, K, V, 1.0, [2], key_allowed=np.array([True, False, True]))
    assert abs(o2[0, 0] - frac(toy["removals"]["B"]["output"])) < 1e-12


def test_toy_pairs(toy):
    pin_toy_pairs(toy)


def test_toy_shift(toy):
    pin_toy_shift(toy)


def test_toy_from_logits(toy):
    pin_toy_from_logits(toy)


# --- identity, bound, closed forms on random tiny cases -----------------------------


def _random_cases(n_cases=10000, seed=0):
    rng = np.random.default_rng(seed)
    for _ in range(n_cases):
        nb = int(rng.integers(2, 9))
        d = int(rng.choice([1, 2, 3, 8]))
        m = rng.dirichlet(np.full(nb, 0.7))
        v = rng.standard_normal((nb, d)) * rng.choice([0.1, 1.0, 10.0]) + rng.standard_normal(d)
        kD = int(rng.integers(1, nb))
        D = sorted(rng.choice(nb, size=kD, replace=False).tolist())
        if m[D].sum() > 1 - 1e-6:
            continue
        yield m, v, D


def pin_identity_and_bound():
    for m, v, D in _random_cases():
        o = O.dense_output(m, v)
        o_t = O.deleted_output(m, v, D)
        err = O.deletion_error(m, v, D)
        scale = 1.0 + np.abs(v).max()
        assert np.abs((o - o_t) - err).max() <= 1e-12 * scale / (1 - m[D].sum())
        # rounding in o - o_tilde is amplified by 1 / (1 - delta), as in the check above
        assert np.linalg.norm(o - o_t) <= O.triangle_bound(m, v, D) * (1 + 1e-12) + 1e-12 * scale / (1 - m[D].sum())
        # derived equivalent: o - o_t = delta (vbar_D - o_t), vbar_D = sum_D m_b v_b / delta
        delta = m[D].sum()
        vbar = (m[D][:, None] * v[D]).sum(0) / delta
        assert np.abs((o - o_t) - delta * (vbar - o_t)).max() <= 1e-11 * scale / (1 - delta)


def test_identity_and_bound_random():
    pin_identity_and_bound()


def pin_singleton_closed_form():
    rng = np.random.default_rng(1)
    for _ in range(2000):
        nb = int(rng.integers(2, 7))
        d = int(rng.integers(1, 5))
        m = rng.dirichlet(np.ones(nb))
        v = rng.standard_normal((nb, d))
        b = int(rng.integers(nb))
        o = (m[:, None] * v).sum(0)
        closed = m[b] * np.linalg.norm(v[b] - o) / (1 - m[b])
        assert abs(np.linalg.norm(O.deletion_error(m, v, [b])) - closed) < 1e-12 * (1 + closed)
        assert abs(O.triangle_bound(m, v, [b]) - closed) < 1e-12 * (1 + closed)


def test_singleton_closed_form():
    pin_singleton_closed_form()


def test_cancelling_pairs():
    """Two discarded blocks with equal mass and deviations of opposite sign: exact error
    zero, bound positive (the note's closing experiment)."""
    rng = np.random.default_rng(2)
    for _ in range(500):
        d = int(rng.integers(1, 6))
        base = rng.standard_normal(d)
        dev = rng.standard_normal(d)
        a = rng.uniform(0.05, 0.3)
        rest = 1 - 2 * a
        m = np.array([rest, a, a])
        v = np.array([base, base + dev, base - dev])  # o = base
        err = O.deletion_error(m, v, [1, 2])
        assert np.abs(err).max() < 1e-12
        assert np.abs(O.deleted_output(m, v, [1, 2]) - base).max() < 1e-12
        assert O.triangle_bound(m, v, [1, 2]) > 0.1 * np.linalg.norm(dev) * a


def test_worst_case_two_r_delta():
    """BFLA Appendix B.1: with ||v_t|| <= R the error never exceeds 2 R delta, and
    opposite vectors on the retained and omitted sides attain it."""
    rng = np.random.default_rng(3)
    for _ in range(2000):
        n = int(rng.integers(2, 10))
        d = int(rng.integers(1, 5))
        R = rng.uniform(0.1, 10)
        p = rng.dirichlet(np.ones(n))
        V = rng.standard_normal((n, d))
        V *= (R * rng.uniform(0, 1, n) / np.linalg.norm(V, axis=1))[:, None]
        D = sorted(rng.choice(n, size=int(rng.integers(1, n)), replace=False).tolist())
        delta = p[D].sum()
        err = np.linalg.norm(O.deletion_error(p, V, D))
        assert err <= 2 * R * delta * (1 + 1e-12) + 1e-15
        e = np.zeros(d)
        e[0] = 1.0
        W = np.array([(-R if i in D else R) * e for i in range(n)])
        assert abs(np.linalg.norm(O.deletion_error(p, W, D)) - 2 * R * delta) < 1e-9 * R


# --- textbook softmax ---------------------------------------------------------------


def pin_attention_bruteforce():
    rng = np.random.default_rng(4)
    # pure-Python loops on tiny inputs
    for _ in range(20):
        n, d = int(rng.integers(1, 12)), int(rng.integers(1, 5))
        K = rng.standard_normal((n, d))
        V = rng.standard_normal((n, d))
        qs = rng.standard_normal((3, d))
        pos = [int(rng.integers(0, n)) for _ in range(3)]
        o, lse = O.attention_rows(qs, K, V, 0.7, pos)
        for i in range(3):
            w = [math.exp(0.7 * sum(qs[i][c] * K[j][c] for c in range(d))) for j in range(pos[i] + 1)]
            z = math.fsum(w)
            for c in range(d):
                assert abs(o[i][c] - math.fsum(w[j] * V[j][c] for j in range(len(w))) / z) < 1e-12
            assert abs(lse[i] - math.log(z)) < 1e-12
    # scipy logsumexp / softmax at moderate size
    n, d = 512, 16
    K = rng.standard_normal((n, d)) * 2
    V = rng.standard_normal((n, d))
    qs = rng.standard_normal((32, d))
    pos = rng.integers(0, n, 32)
    o, lse = O.attention_rows(qs, K, V, 0.5, pos)
    for i in range(32):
        s = 0.5 * K[:pos[i] + 1] @ qs[i]
        L = logsumexp(s)
        assert abs(lse[i] - L) < 1e-12 * (1 + abs(L))
        assert np.abs(o[i] - np.exp(s - L) @ V[:pos[i] + 1]).max() < 1e-12


def test_attention_bruteforce():
    pin_attention_bruteforce()


# --- geometry ----------------------------------------------------------------------


def test_sampled_rows():
    assert O.sampled_rows(128, 8) == [15, 31, 47, 63, 79, 95, 111, 127]
    assert O.sampled_rows(64, 8) == [7, 15, 23, 31, 39, 47, 55, 63]
    assert O.sampled_rows(5, 8) == [0, 1, 2, 3, 4]
    assert O.sampled_rows(100, 8) == [12, 24, 37, 49, 62, 74, 87, 99]
    assert O.sampled_rows(1, 8) == [0]


def test_mandatory_and_tiles():
    assert O.mandatory_blocks(10, 1, 1) == [0, 10]
    assert O.mandatory_blocks(10, 1, 2) == [0, 9, 10]
    assert O.mandatory_blocks(0, 1, 2) == [0]
    assert O.mandatory_blocks(1, 1, 2) == [0, 1]
    p = O.Problem((100, 64), (228, 64), 2, 1, 8, 64)
    tl = O.tiles(p)
    assert [(t.seq, t.t, t.q_row0, t.n_rows, t.pos0, t.diag, t.k_row0) for t in tl] == [
        (0, 0, 0, 64, 128, 2, 0), (0, 1, 64, 36, 192, 3, 0), (1, 0, 100, 64, 0, 0, 228)]
    assert O.csr_capacity(p) == 2 * (3 + 4 + 1)


# --- selector ----------------------------------------------------------------------


def _tiny_problem(seed, nq=200, nk=328, hq=2, hkv=1, d=8, B=64, sink=6.0):
    rng = np.random.default_rng(seed)
    p = O.Problem((nq,), (nk,), hq, hkv, d, B)
    q = rng.standard_normal((nq, hq, d)) * 1.5
    k = rng.standard_normal((nk, hkv, d)) * 1.5
    v = rng.standard_normal((nk, hkv, d)) + rng.standard_normal(d)
    k[0, :, :] = 0
    k[0, :, -1] = sink * math.sqrt(d)
    q[:, :, -1] = 1.0
    return p, q, k, v


def pin_row_stats_invariants():
    p, q, k, v = _tiny_problem(5)
    for t in O.tiles(p):
        for r in range(t.n_rows):
            st = O.row_block_stats(q[t.q_row0 + r, 0], k[:, 0], v[:, 0], p.scale, t.pos0 + r,
                                   t.diag + 1, p.block_size)
            assert abs(st["m"].sum() - 1) < 1e-12
            assert np.abs(st["u"].sum(0) - st["o"]).max() < 1e-12
            mask = st["m"] > 0
            vb = st["u"][mask] / st["m"][mask, None]
            assert np.allclose(st["I"][mask], st["m"][mask] * np.linalg.norm(vb - st["o"], axis=1),
                               rtol=1e-10, atol=1e-15)
            ref_o, ref_l = O.attention_rows(q[t.q_row0 + r:t.q_row0 + r + 1, 0], k[:, 0], v[:, 0],
                                            p.scale, [t.pos0 + r])
            assert np.abs(ref_o[0] - st["o"]).max() < 1e-12 and abs(ref_l[0] - st["lse"]) < 1e-12
            # brute force: per-block masses and sums from scipy's softmax, block by block
            pos = t.pos0 + r
            pr = softmax(p.scale * (k[:pos + 1, 0] @ q[t.q_row0 + r, 0]))
            for b in range(t.diag + 1):
                js = [j for j in range(b * p.block_size, min((b + 1) * p.block_size, pos + 1))]
                mb = math.fsum(pr[j] for j in js)
                assert abs(st["m"][b] - mb) < 1e-12
                ub = np.array([math.fsum(pr[j] * v[j, 0, c] for j in js) for c in range(p.head_dim)])
                assert np.abs(st["u"][b] - ub).max() < 1e-12
                assert abs(st["I"][b] - np.linalg.norm(ub - mb * ref_o[0])) < 1e-11


def test_row_stats_invariants():
    pin_row_stats_invariants()


def pin_threshold_bruteforce():
    """Brute force over every cut of the discard order, each bound computed from scratch,
    on <= 12 candidates; plus monotonicity of B(k)."""
    rng = np.random.default_rng(6)
    for _ in range(300):
        n = int(rng.integers(1, 13))
        S = int(rng.integers(1, 9))
        I = rng.uniform(0, 0.02, (S, n)) * (rng.uniform(0, 1, (S, n)) < 0.8)
        m = rng.dirichlet(np.ones(n + 2), size=S)[:, :n]
        score = I.mean(0)
        if rng.uniform() < 0.3:  # force ties
            score = np.round(score, 3)
        cand = list(range(n))
        order = O.discard_order(score, cand)
        # order: ascending score, larger id first on ties
        for a, b in zip(order, order[1:]):
            assert score[a] < score[b] or (score[a] == score[b] and a > b)
        tau = float(rng.uniform(0, 0.1))
        curve, per_row = O.bound_curve(I, m, order)
        assert all(curve[i] <= curve[i + 1] for i in range(len(curve) - 1))
        best = 0
        for kk in range(n + 1):
            D = order[:kk]
            bk = max((sum(I[i, b] for b in D) / (1 - sum(m[i, b] for b in D))) for i in range(S)) if D else 0.0
            assert abs(bk - curve[kk]) <= 1e-12 * (1 + bk)
            if all(max((sum(I[i, b] for b in order[:j]) / (1 - sum(m[i, b] for b in order[:j])))
                       for i in range(S)) <= tau for j in range(1, kk + 1)):
                best = kk
        assert O.cut(curve, tau) == best


def test_threshold_bruteforce():
    pin_threshold_bruteforce()


def pin_selection_theorem():
    """For each sampled row the measured sparse-vs-dense error is at most that row's
    bound at the cut, which is at most tau; the sparse output computed directly equals
    the one computed from dense quantities through the identity."""
    for seed in range(4):
        p, q, k, v = _tiny_problem(10 + seed)
        for tau in (0.005, 0.02, 0.08, 1.0):
            sel = O.select(p, q, k, v, [tau] * p.num_heads_q, 1, 1, 8)
            for (h, gt), s in sel.items():
                t = s.tile
                assert set(s.mandatory) <= set(s.retained)
                assert s.retained == sorted(s.retained)
                od, _ = O.tile_attention(p, q, k, v, h, t)
                os_, ls = O.tile_attention(p, q, k, v, h, t, s.retained)
                oi, li = O.tile_attention_via_identity(p, q, k, v, h, t, s.retained)
                assert np.abs(os_ - oi).max() < 1e-12 * (1 + np.abs(os_).max())
                assert np.abs(ls - li).max() < 1e-12 * (1 + np.abs(ls).max())
                for j, r in enumerate(s.rows):
                    err = np.linalg.norm(od[r] - os_[r])
                    assert err <= s.row_bound[j] * (1 + 1e-9) + 1e-15
                    assert s.row_bound[j] <= tau
                full, _ = O.tile_attention(p, q, k, v, h, t, list(range(t.diag + 1)))
                assert np.abs(full - od).max() == 0.0


def test_selection_theorem():
    pin_selection_theorem()


def test_nested_supports():
    """BFLA Appendix B.5: for fixed scores a larger budget gives nested supports and
    non-increasing omitted mass (here: a lower tau discards a prefix of the higher
    tau's discard list)."""
    p, q, k, v = _tiny_problem(20)
    taus = [1.0, 0.1, 0.05, 0.02, 0.01, 0.0]
    prev = None
    for tau in taus:
        sel = O.select(p, q, k, v, [tau] * 2, 1, 1, 8)
        if prev is not None:
            for key in sel:
                assert set(prev[key].retained) <= set(sel[key].retained)
                a = prev[key]
                om_prev = a.m[:, a.discarded].sum(1)
                om_now = sel[key].m[:, sel[key].discarded].sum(1)
                assert np.all(om_now <= om_prev + 1e-15)
        prev = sel


# --- mass-only selector ---------------------------------------------------------------


def pin_mass_cut():
    """Mass-only cut. One sampled row: keeping the discard order's longest acceptable
    prefix discards the largest number of blocks whose total mass fits the budget
    (brute force over every subset). Several rows: every prefix's largest per-row
    omitted mass recomputed from scratch."""
    import itertools
    rng = np.random.default_rng(31)
    for _ in range(300):
        n = int(rng.integers(1, 11))
        S = int(rng.integers(1, 5))
        m = rng.dirichlet(np.ones(n + 2), size=S)[:, :n]
        if rng.uniform() < 0.3:  # force ties
            m = np.round(m, 2)
        eps = float(rng.uniform(0, 0.3))
        mass = m.mean(0)
        order = O.discard_order(mass, list(range(n)))
        curve, _ = O.mass_curve(m, order)
        ks = O.cut(curve, eps)
        best = 0
        for kk in range(n + 1):
            if all(max(math.fsum(m[i, b] for b in order[:j]) for i in range(S)) <= eps for j in range(1, kk + 1)):
                best = kk
        assert ks == best
        if S == 1:
            most = max(len(D) for r in range(n + 1) for D in itertools.combinations(range(n), r)
                       if math.fsum(m[0, b] for b in D) <= eps)
            assert ks == most


def test_mass_cut():
    pin_mass_cut()


def pin_mass_selection():
    """Mass-only selection on tiny problems, checked with scipy's softmax: the discard
    order ascends in the tile mass (mean over sampled rows of the block masses), every
    sampled row keeps all but at most eps of its mass, and its error obeys the worst
    case 2 R delta of BFLA Appendix B.1 (R: the largest value norm the row sees)."""
    for seed in range(3):
        p, q, k, v = _tiny_problem(40 + seed)
        for eps in (0.0, 0.001, 0.01, 0.05, 0.5):
            sel = O.select(p, q, k, v, [eps] * p.num_heads_q, 1, 1, 8, mode="mass")
            for (h, gt), s in sel.items():
                t = s.tile
                assert set(s.mandatory) <= set(s.retained) and s.retained == sorted(s.retained)
                B = p.block_size
                bm = []
                for r in s.rows:
                    pos = t.pos0 + r
                    pr = softmax(p.scale * (k[:pos + 1, 0] @ q[t.q_row0 + r, h]))
                    bm.append([math.fsum(pr[b * B:min((b + 1) * B, pos + 1)]) for b in range(t.diag + 1)])
                bm = np.array(bm)
                tm = bm.mean(0)
                for a, b in zip(s.order, s.order[1:]):
                    assert tm[a] <= tm[b] + 1e-12
                od, _ = O.tile_attention(p, q, k, v, h, t)
                os_, _ = O.tile_attention(p, q, k, v, h, t, s.retained)
                drop = s.discarded
                for j, r in enumerate(s.rows):
                    delta = math.fsum(bm[j, b] for b in drop)
                    assert delta <= eps + 1e-12
                    R = np.linalg.norm(v[:t.pos0 + r + 1, 0], axis=1).max()
                    assert np.linalg.norm(od[r] - os_[r]) <= 2 * R * delta * (1 + 1e-9) + 1e-15


def test_mass_selection():
    pin_mass_selection()


def test_mass_nested_supports():
    """A smaller omitted-mass budget discards a subset (BFLA Appendix B.5)."""
    p, q, k, v = _tiny_problem(21)
    prev = None
    for eps in (0.9, 0.1, 0.02, 0.005, 0.0):
        sel = O.select(p, q, k, v, [eps] * 2, 1, 1, 8, mode="mass")
        if prev is not None:
            for key in sel:
                assert set(prev[key].retained) <= set(sel[key].retained)
        prev = sel


# --- group-shared selector -------------------------------------------------------------


def pin_group_cut():
    """Group cut: every prefix recomputed from scratch, each sampled row against its
    own head's threshold (rows of different heads carry different taus)."""
    rng = np.random.default_rng(41)
    for _ in range(300):
        n = int(rng.integers(1, 11))
        S = int(rng.integers(1, 9))
        I = rng.uniform(0, 0.02, (S, n)) * (rng.uniform(0, 1, (S, n)) < 0.8)
        m = rng.dirichlet(np.ones(n + 2), size=S)[:, :n]
        taus = rng.uniform(0, 0.1, S)
        order = O.discard_order(I.mean(0), list(range(n)))
        curve, _ = O.group_excess_curve(I, m, order, taus)
        best = 0
        for kk in range(n + 1):
            ok = True
            for j in range(1, kk + 1):
                D = order[:j]
                for i in range(S):
                    if math.fsum(I[i, b] for b in D) / (1 - math.fsum(m[i, b] for b in D)) > taus[i]:
                        ok = False
            if ok:
                best = kk
        assert O.cut(curve, 0.0) == best


def test_group_cut():
    pin_group_cut()


def pin_group_selection():
    """Group-shared lists on tiny GQA problems: row j of a tile comes from head
    g G + (j mod G); each sampled row's error (its own head's dense vs sparse output)
    is within its bound, which is within that head's tau; the list is shared."""
    cuts = []
    for seed in range(3):
        p, q, k, v = _tiny_problem(60 + seed, hq=4, hkv=2, sink=11.0)
        taus = [0.03, 1.0, 0.1, 3.0]
        sel = O.select(p, q, k, v, taus, 1, 1, 8, mode="group")
        for (h, gt), s in sel.items():
            g = h // p.group
            t = s.tile
            assert s.heads == [g * p.group + (j % p.group) for j in range(len(s.rows))]
            assert sel[(g * p.group, gt)].retained == s.retained
            assert set(s.mandatory) <= set(s.retained)
            cuts.append(s.k_star)
            for j, (r, hh) in enumerate(zip(s.rows, s.heads)):
                od, _ = O.tile_attention(p, q, k, v, hh, t)
                os_, _ = O.tile_attention(p, q, k, v, hh, t, s.retained)
                err = np.linalg.norm(od[r] - os_[r])
                b = s.per_row[s.k_star][j]
                assert b <= taus[hh] + 1e-15
                assert err <= b * (1 + 1e-9) + 1e-15
    assert max(cuts) > 0  # some tiles discard blocks


def test_group_selection():
    pin_group_selection()


def test_group_of_one_is_the_per_head_selector():
    """With one query head per KV head the group selector is the per-head selector."""
    p, q, k, v = _tiny_problem(70, hq=2, hkv=2)
    for tau in (0.005, 0.03, 0.2):
        a = O.select(p, q, k, v, [tau, tau * 2], 1, 1, 8)
        b = O.select(p, q, k, v, [tau, tau * 2], 1, 1, 8, mode="group")
        for key in a:
            assert a[key].retained == b[key].retained and a[key].k_star == b[key].k_star
            assert np.array_equal(a[key].score, b[key].score)


# --- practical POEM ---------------------------------------------------------------------


def _random_pooled(rng, n):
    mbar = rng.dirichlet(np.ones(n + 2))  # the last two entries play the mandatory blocks
    Ibar = mbar * rng.uniform(0.5, 20.0, n + 2) * (rng.uniform(0, 1, n + 2) < 0.9)
    if rng.uniform() < 0.3:
        mbar = np.round(mbar, 2)
        mbar = mbar / mbar.sum()
    return mbar, Ibar


def pin_practical_selection():
    """Practical POEM from pooled estimates, against brute force on <= 10 candidates:
    the preselection is the fewest candidates whose mass reaches rho of theirs (a
    largest-mass prefix); the rerank is non-increasing in log m + w log(I / m) with
    math.log; the kept prefix is the shortest one whose pooled mass, with the
    mandatory blocks, reaches (1 - eps) of the total; with w = 0 and rho = 1 the
    kept set is the fewest candidates that do so (subset brute force)."""
    import itertools
    rng = np.random.default_rng(51)
    for _ in range(300):
        n = int(rng.integers(1, 11))
        mbar, Ibar = _random_pooled(rng, n)
        mand = [n, n + 1]
        cand = list(range(n))
        eps = float(rng.uniform(0, 0.3))
        w = float(rng.choice([0.0, 0.5, 1.0, 2.0]))
        rho = float(rng.choice([1.0, 0.9, 0.6]))
        pre, order, kept = O.practical_retain(mbar, Ibar, mand, cand, eps, w, rho)
        tot_c = math.fsum(mbar[b] for b in cand)
        fewest = min(len(D) for r in range(n + 1) for D in itertools.combinations(cand, r)
                     if math.fsum(mbar[b] for b in D) >= rho * tot_c - 1e-15)
        assert len(pre) == fewest or tot_c == 0.0
        assert math.fsum(mbar[b] for b in pre) >= rho * tot_c - 1e-12
        assert sorted(order) == sorted(pre)

        def key(b):
            if mbar[b] <= 0 or (w != 0.0 and Ibar[b] <= 0):
                return -math.inf
            return math.log(mbar[b]) + (w * math.log(Ibar[b] / mbar[b]) if w != 0.0 else 0.0)
        for a, b in zip(order, order[1:]):
            assert key(a) > key(b) or (key(a) == key(b) and a < b)
        target = (1 - eps) * math.fsum(mbar)
        base = math.fsum(mbar[b] for b in mand)
        assert kept == order[:len(kept)]
        if len(kept) < len(order):
            assert base + math.fsum(mbar[b] for b in kept) >= target - 1e-12
        if kept:
            assert base + math.fsum(mbar[b] for b in kept[:-1]) < target + 1e-12
        if w == 0.0 and rho == 1.0:
            need = min((len(D) for r in range(n + 1) for D in itertools.combinations(cand, r)
                        if base + math.fsum(mbar[b] for b in D) >= target - 1e-15), default=n)
            assert len(kept) == need


def test_practical_selection():
    pin_practical_selection()


def test_practical_on_tiny_problems():
    """End to end on tiny problems: the mandatory blocks are kept, the list is
    ascending, and the pooled omitted mass is within eps whenever some preselected
    block was dropped."""
    p, q, k, v = _tiny_problem(82, sink=9.0)
    for eps in (0.001, 0.02, 0.2):
        sel = O.select(p, q, k, v, [eps] * 2, 1, 1, 8, mode="practical", practical=dict(w=0.5, rho=0.95))
        for (h, gt), s in sel.items():
            assert set(s.mandatory) <= set(s.retained) and s.retained == sorted(s.retained)
            dropped_pre = [b for b in s.order if b not in set(s.retained)]
            if dropped_pre:
                assert s.per_row[0].mean() <= eps + 1e-12


def test_gpu_toy_geometry_in_oracle():
    """The toy realised at block granularity (B = 64, d = 64, fp32, scale 1): blocks
    0, 1, 2, 3 with masses 1/2, 1/4, 1/4, ~0 and values 2, 0, 4, 0 along e_0; the
    mandatory set is {0, 3}, the candidates are B = block 1 and C = block 2."""
    q, k, v, p = toy_blocks(shift=0.0)
    for tau, drop in ((0.5, []), (0.7, [2]), (2.0, [1, 2])):
        sel = O.select(p, q, k, v, [tau], 1, 1, 8)[(0, 0)]
        assert np.allclose(sel.score, [0, 0.5, 0.5, 0], atol=1e-12)
        assert sorted(sel.discarded) == drop
        od, _ = O.tile_attention(p, q, k, v, 0, O.tiles(p)[0])
        os_, _ = O.tile_attention(p, q, k, v, 0, O.tiles(p)[0], sel.retained)
        err = np.abs(od[:, 0] - os_[:, 0]).max()
        assert abs(err - {0.5: 0.0, 0.7: 2 / 3, 2.0: 0.0}[tau]) < 1e-12
    q, k, v, p = toy_blocks(shift=10.0)
    sel = O.select(p, q, k, v, [0.7], 1, 1, 8)[(0, 0)]
    assert sorted(sel.discarded) == [2]
    od, _ = O.tile_attention(p, q, k, v, 0, O.tiles(p)[0])
    os_, _ = O.tile_attention(p, q, k, v, 0, O.tiles(p)[0], sel.retained)
    assert np.allclose(od[:, 0], 12.0, atol=1e-12)
    assert abs(np.abs(od[:, 0] - os_[:, 0]).max() - 2 / 3) < 1e-12


# --- whole-problem prefill and the CSR row walk ------------------------------------------
#
# Two sequences (the second is a chunk: queries at positions 8 .. 12 of 13 keys, BFLA
# Section 3.6), four query heads on two KV heads (head h reads KV head h // 2, BFLA
# Section 3.3), blocks of 4 keys, d = 3. The tile geometry and the CSR are written out
# by hand, and every output row is recomputed by pure-Python softmax over exactly the
# keys its tile may see (the retained-block output of the POEM note, Section 4.1).

# (global tile, first packed query row, rows, first position, diagonal block, first packed key row)
HAND_TILES = [(0, 0, 4, 0, 0, 0), (1, 4, 3, 4, 1, 0), (2, 7, 4, 8, 2, 7), (3, 11, 1, 12, 3, 7)]
# listed ids of each (query head, global tile); ids outside 0 .. diag take no part
HAND_ROWS = {
    (0, 0): [0], (0, 1): [1], (0, 2): [0, 2], (0, 3): [1, 3],
    (1, 0): [], (1, 1): [0, 1], (1, 2): [-3, 1, 2, 5], (1, 3): [0, 2],
    (2, 0): [0, 3], (2, 1): [0], (2, 2): [2], (2, 3): [3],
    (3, 0): [0], (3, 1): [1, 2], (3, 2): [0, 1, 2], (3, 3): [0, 1, 2, 3],
}


def _prefill_problem():
    rng = np.random.default_rng(61)
    p = O.Problem((7, 5), (7, 13), 4, 2, 3, 4, 0.6)
    q = rng.standard_normal((12, 4, 3)) * 1.5
    k = rng.standard_normal((20, 2, 3)) * 1.5
    v = rng.standard_normal((20, 2, 3))
    return p, q, k, v


def _brute_row(q, k, v, scale, qrow, h, g, k0, pos, blocks, B):
    """Softmax attention of packed query row qrow (head h) over the keys j <= pos of its
    sequence whose block j // B is in blocks; pure Python."""
    d = q.shape[2]
    s = [(scale * math.fsum(q[qrow, h, c] * k[k0 + j, g, c] for c in range(d)), j)
         for j in range(pos + 1) if j // B in blocks]
    if not s:
        return [0.0] * d, -math.inf
    mx = max(x for x, _ in s)
    e = [(math.exp(x - mx), j) for x, j in s]
    z = math.fsum(w for w, _ in e)
    return [math.fsum(w * v[k0 + j, g, c] for w, j in e) / z for c in range(d)], mx + math.log(z)


def _hand_csr(H, T):
    rows = [HAND_ROWS[(h, gt)] for h in range(H) for gt in range(T)]  # row h * T + gtile
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int64)
    return row_ptr, np.array([b for r in rows for b in r], np.int64)


def pin_prefill_walk():
    p, q, k, v = _prefill_problem()
    T = len(HAND_TILES)
    assert [(t.gtile, t.q_row0, t.n_rows, t.pos0, t.diag, t.k_row0) for t in O.tiles(p)] == HAND_TILES
    row_ptr, block_idx = _hand_csr(p.num_heads_q, T)
    sp = O.sparse_prefill(p, q, k, v, row_ptr, block_idx)
    de = O.dense_prefill(p, q, k, v)
    keys = [(h, gt) for h in range(p.num_heads_q) for gt in range(T)]
    assert sorted(sp) == keys and sorted(de) == keys
    for (gt, q0, n, pos0, diag, k0) in HAND_TILES:
        for h in range(p.num_heads_q):
            listed = {b for b in HAND_ROWS[(h, gt)] if 0 <= b <= diag}
            for (O_, L_), blocks in ((sp[(h, gt)], listed), (de[(h, gt)], set(range(diag + 1)))):
                assert O_.shape == (n, p.head_dim) and L_.shape == (n,)
                for i in range(n):
                    o, lse = _brute_row(q, k, v, p.scale, q0 + i, h, h // 2, k0, pos0 + i, blocks, p.block_size)
                    assert np.abs(O_[i] - np.array(o)).max() < 1e-12, (h, gt, i)
                    assert (L_[i] == lse == -math.inf) or abs(L_[i] - lse) < 1e-12, (h, gt, i)
    # a subset of the (head, tile) pairs gives the same rows
    sub = O.sparse_prefill(p, q, k, v, row_ptr, block_idx, which=[(3, 2), (1, 0)])
    assert sorted(sub) == [(1, 0), (3, 2)]
    assert np.array_equal(sub[(3, 2)][0], sp[(3, 2)][0])


def test_prefill_walk():
    pin_prefill_walk()


def pin_csr():
    """csr() lays the retained lists out in rows h * num_tiles + gtile, each ascending."""
    from types import SimpleNamespace
    p = O.Problem((7, 5), (7, 13), 2, 1, 3, 4)  # four tiles (HAND_TILES), two heads
    kept = {(0, 0): [0], (0, 1): [0, 1], (0, 2): [2], (0, 3): [0, 3],
            (1, 0): [0], (1, 1): [1], (1, 2): [0, 1, 2], (1, 3): [3]}
    rp, ids = O.csr(p, {key: SimpleNamespace(retained=r) for key, r in kept.items()})
    assert rp.tolist() == [0, 1, 3, 4, 6, 7, 8, 11, 12]
    assert ids.tolist() == [0, 0, 1, 2, 0, 3, 0, 1, 0, 1, 2, 3]
    assert O.csr_capacity(p) == 2 * (1 + 2 + 3 + 4)


def test_csr():
    pin_csr()


def pin_practical_tile():
    """select_tile_practical end to end: pooled masses and scores recomputed by brute
    force with scipy's softmax, the rerank key with math.log, the kept set equal to
    practical_retain on those values (itself pinned by subset brute force above), and
    the per-row omitted mass of the final discard set."""
    retain_ref = _orig_practical
    p, q, k, v = _tiny_problem(91, nq=256, nk=640, B=32, sink=8.0)  # 8 tiles, up to 20 visible blocks
    B = p.block_size
    for eps, w, rho in ((0.002, 0.5, 0.95), (0.05, 1.0, 0.9), (0.2, 0.0, 1.0), (0.01, 2.0, 0.99)):
        n_drop = 0
        sels = O.select(p, q, k, v, [eps, 2 * eps], 1, 1, 8, mode="practical", practical=dict(w=w, rho=rho))
        for (h, gt), s in sels.items():
            t = s.tile
            n_vis = t.diag + 1
            m_rows, I_rows = [], []
            for r in O.sampled_rows(t.n_rows, 8):
                pos = t.pos0 + r
                pr = softmax(p.scale * (k[:pos + 1, 0] @ q[t.q_row0 + r, h]))
                o = pr @ v[:pos + 1, 0]
                mb = np.array([pr[b * B:min((b + 1) * B, pos + 1)].sum() for b in range(n_vis)])
                ub = np.array([pr[b * B:min((b + 1) * B, pos + 1)] @ v[b * B:min((b + 1) * B, pos + 1), 0]
                               for b in range(n_vis)])
                m_rows.append(mb)
                I_rows.append(np.linalg.norm(ub - mb[:, None] * o[None, :], axis=1))
            m_rows, I_rows = np.array(m_rows), np.array(I_rows)
            mbar, Ibar = m_rows.mean(0), I_rows.mean(0)
            assert np.allclose(s.mass, mbar, rtol=1e-10, atol=1e-15)
            for b in range(n_vis):
                if mbar[b] > 0 and (w == 0.0 or Ibar[b] > 0):
                    want = math.log(mbar[b]) + (w * math.log(Ibar[b] / mbar[b]) if w != 0.0 else 0.0)
                    assert abs(s.score[b] - want) < 1e-9 * (1 + abs(want)), (h, gt, b)
            mand = O.mandatory_blocks(t.diag, 1, 1)
            cand = [b for b in range(n_vis) if b not in set(mand)]
            _, order, kept = retain_ref(mbar, Ibar, mand, cand, eps * (1 + h), w, rho)
            assert s.retained == sorted(set(mand) | set(kept)), (h, gt)
            assert s.order == order
            dropped = [b for b in range(n_vis) if b not in set(s.retained)]
            assert np.allclose(s.per_row[0], m_rows[:, dropped].sum(1), rtol=1e-10, atol=1e-15)
            assert s.k_star == len(dropped)
            n_drop += len(dropped)
        assert n_drop > 0


def test_practical_tile():
    pin_practical_tile()


def toy_blocks(shift=0.0):
    """Inputs of the block-level toy (shared with the GPU toy test)."""
    from block_sparse_attention_poem_amd.synth import toy_block_inputs
    q, k, v, meta = toy_block_inputs(shift)
    p = O.Problem((meta["n_q"],), (meta["n_k"],), 1, 1, meta["d"], meta["block"], 1.0)
    return q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), p


# --- planted mistakes: each must make some pin fail ----------------------------------


def _deleted_no_renorm(m, v, D):
    m = np.asarray(m, float)
    v = np.asarray(v, float).reshape(len(m), -1)
    keep = [b for b in range(len(m)) if b not in set(D)]
    return (m[keep][:, None] * v[keep]).sum(0)


def _identity_wrong_sign(m, v, D):
    m = np.asarray(m, float)
    v = np.asarray(v, float).reshape(len(m), -1)
    o = (m[:, None] * v).sum(0)
    D = list(D)
    return (m[D][:, None] * (v[D] + o)).sum(0) / (1 - m[D].sum())


def _bound_no_denominator(m, v, D):
    return O.proxy_scores(m, v)[list(D)].sum()


def _proxy_raw_value(m, v):
    m = np.asarray(m, float)
    v = np.asarray(v, float).reshape(len(m), -1)
    return m * np.linalg.norm(v, axis=1)


def _order_small_id_first(scores, cand):
    return sorted(cand, key=lambda b: (float(scores[b]), int(b)))


def _attention_off_by_one(qr, K, V, scale, positions, key_allowed=None):
    return _orig_attention(qr, K, V, scale, [p - 1 if p > 0 else p for p in positions], key_allowed)


_orig_attention = O.attention_rows


def _stats_transposed_mass(qr, K, V, scale, pos, n_vis, B):
    st = _orig_stats(qr, K, V, scale, pos, n_vis, B)
    st = dict(st)
    st["m"] = st["m"][::-1].copy()
    st["I"] = np.linalg.norm(st["u"] - st["m"][:, None] * st["o"][None, :], axis=1)
    return st


_orig_stats = O.row_block_stats


def _mass_curve_mean_rows(m_rows, order):
    m_rows = np.asarray(m_rows, dtype=np.float64)
    c = np.zeros(len(order) + 1)
    for kk in range(1, len(order) + 1):
        c[kk] = c[kk - 1] + m_rows[:, order[kk - 1]].mean()
    return c, np.repeat(c[:, None], m_rows.shape[0], axis=1)


def _mass_selector_ranks_by_proxy(p, q, k, v, h, tile, eps, n_sink, n_local, S):
    s = _orig_select_tile(p, q, k, v, h, tile, 1e9, n_sink, n_local, S)
    order = O.discard_order(s.score, [b for b in range(tile.diag + 1) if b not in set(s.mandatory)])
    curve, per_row = O.mass_curve(s.m, order)
    ks = O.cut(curve, eps)
    drop = set(order[:ks])
    return O.TileSelection(h, tile, s.rows, s.I, s.m, s.lse, s.o, s.mass, s.mass, s.mandatory, order, curve,
                           per_row, ks, [b for b in range(tile.diag + 1) if b not in drop])


_orig_select_tile = O.select_tile


def _group_curve_loosest_tau(I_rows, m_rows, order, row_tau):
    _, per_row = O.bound_curve(I_rows, m_rows, order)
    return per_row.max(axis=1) - max(row_tau), per_row


def _practical_rerank_ascending(mbar, Ibar, mandatory, candidates, eps, w, rho):
    pre, order, kept = _orig_practical(mbar, Ibar, mandatory, candidates, eps, w, rho)
    order = order[::-1]
    target = (1.0 - eps) * float(np.sum(mbar))
    acc = float(sum(mbar[b] for b in mandatory))
    kept = []
    for b in order:
        if acc >= target:
            break
        kept.append(b)
        acc += float(mbar[b])
    return pre, order, kept


_orig_practical = O.practical_retain


def _sparse_prefill_tile_major(p, q, k, v, row_ptr, block_idx, which=None):
    """CSR row read as gtile * H + h instead of h * num_tiles + gtile."""
    tl = O.tiles(p)
    if which is None:
        which = [(h, t.gtile) for h in range(p.num_heads_q) for t in tl]
    out = {}
    for (h, gt) in which:
        r = gt * p.num_heads_q + h
        ids = [int(b) for b in block_idx[row_ptr[r]:row_ptr[r + 1]] if 0 <= b <= tl[gt].diag]
        out[(h, gt)] = O.tile_attention(p, q, k, v, h, tl[gt], ids)
    return out


def _sparse_prefill_filter(lo_ok, hi_ok):
    def f(p, q, k, v, row_ptr, block_idx, which=None):
        tl = O.tiles(p)
        T = len(tl)
        if which is None:
            which = [(h, t.gtile) for h in range(p.num_heads_q) for t in tl]
        out = {}
        for (h, gt) in which:
            r = h * T + gt
            ids = [int(b) for b in block_idx[row_ptr[r]:row_ptr[r + 1]] if lo_ok(b) and hi_ok(b, tl[gt].diag)]
            out[(h, gt)] = O.tile_attention(p, q, k, v, h, tl[gt], ids)
        return out
    return f


_sparse_prefill_drops_diagonal = _sparse_prefill_filter(lambda b: b >= 0, lambda b, d: b < d)
_sparse_prefill_no_lower_bound = _sparse_prefill_filter(lambda b: True, lambda b, d: b <= d)


def _tile_attention_kv_modulo(p, q, k, v, h, tile, blocks=None):
    """KV head h % H_kv instead of h // G."""
    g = h % p.num_heads_kv
    Q = q[tile.q_row0:tile.q_row0 + tile.n_rows, h, :]
    K = k[tile.k_row0:tile.k_row0 + tile.n_k, g, :]
    V = v[tile.k_row0:tile.k_row0 + tile.n_k, g, :]
    allowed = None
    if blocks is not None:
        allowed = np.zeros(tile.n_k, dtype=bool)
        for b in blocks:
            allowed[b * p.block_size:(b + 1) * p.block_size] = True
    return O.attention_rows(Q, K, V, p.scale, [tile.pos0 + i for i in range(tile.n_rows)], allowed)


def _csr_tile_major(p, selections):
    tl = O.tiles(p)
    rp = [0]
    ids = []
    for t in tl:
        for h in range(p.num_heads_q):
            r = selections[(h, t.gtile)].retained
            ids.extend(r)
            rp.append(len(ids))
    return np.asarray(rp, np.int64), np.asarray(ids, np.int64)


def _practical_tile_swapped(p, q, k, v, h, tile, eps, n_sink, n_local, S, w=0.5, rho=0.95):
    """select_tile_practical with mbar and Ibar swapped in its call to practical_retain."""
    g = h // p.group
    K = k[tile.k_row0:tile.k_row0 + tile.n_k, g, :]
    V = v[tile.k_row0:tile.k_row0 + tile.n_k, g, :]
    n_vis = tile.diag + 1
    rows = O.sampled_rows(tile.n_rows, S)
    st = [O.row_block_stats(q[tile.q_row0 + r, h, :], K, V, p.scale, tile.pos0 + r, n_vis, p.block_size)
          for r in rows]
    I = np.stack([x["I"] for x in st])
    m = np.stack([x["m"] for x in st])
    Ibar, mbar = I.mean(axis=0), m.mean(axis=0)
    mand = O.mandatory_blocks(tile.diag, n_sink, n_local)
    cand = [b for b in range(n_vis) if b not in set(mand)]
    pre, order, kept = _orig_practical(Ibar, mbar, mand, cand, float(eps), float(w), float(rho))
    retained = sorted(set(mand) | set(kept))
    drop = [b for b in range(n_vis) if b not in set(retained)]
    omitted = m[:, drop].sum(axis=1) if drop else np.zeros(len(rows))
    return O.TileSelection(h, tile, rows, I, m, np.array([x["lse"] for x in st]),
                           np.stack([x["o"] for x in st]), O.practical_keys(mbar, Ibar, w), mbar, mand, order,
                           np.zeros(0), omitted[None, :], len(drop), retained)


@pytest.mark.parametrize("name,fn,pins", [
    ("practical_retain", _practical_rerank_ascending, ["practical"]),
    ("group_excess_curve", _group_curve_loosest_tau, ["group_cut", "group_selection"]),
    ("mass_curve", _mass_curve_mean_rows, ["mass_cut"]),
    ("select_tile_mass", _mass_selector_ranks_by_proxy, ["mass_selection"]),
    ("deleted_output", _deleted_no_renorm, ["toy_pairs"]),
    ("deletion_error", _identity_wrong_sign, ["toy_pairs", "identity"]),
    ("triangle_bound", _bound_no_denominator, ["toy_pairs", "singleton"]),
    ("proxy_scores", _proxy_raw_value, ["toy_pairs", "toy_shift"]),
    ("discard_order", _order_small_id_first, ["threshold"]),
    ("attention_rows", _attention_off_by_one, ["attention", "toy_logits"]),
    ("row_block_stats", _stats_transposed_mass, ["row_stats", "toy_logits"]),
    ("sparse_prefill", _sparse_prefill_tile_major, ["prefill"]),
    ("sparse_prefill", _sparse_prefill_drops_diagonal, ["prefill"]),
    ("sparse_prefill", _sparse_prefill_no_lower_bound, ["prefill"]),
    ("tile_attention", _tile_attention_kv_modulo, ["prefill"]),
    ("csr", _csr_tile_major, ["csr"]),
    ("select_tile_practical", _practical_tile_swapped, ["practical_tile"]),
])
def test_planted_mistakes_are_caught(monkeypatch, toy, name, fn, pins):
    runners = {
        "toy_pairs": lambda: pin_toy_pairs(toy),
        "toy_shift": lambda: pin_toy_shift(toy),
        "toy_logits": lambda: pin_toy_from_logits(toy),
        "identity": pin_identity_and_bound,
        "singleton": pin_singleton_closed_form,
        "threshold": pin_threshold_bruteforce,
        "attention": pin_attention_bruteforce,
        "row_stats": pin_row_stats_invariants,
        "mass_cut": pin_mass_cut,
        "mass_selection": pin_mass_selection,
        "group_cut": pin_group_cut,
        "practical": pin_practical_selection,
        "group_selection": pin_group_selection,
        "prefill": pin_prefill_walk,
        "csr": pin_csr,
        "practical_tile": pin_practical_tile,
    }
    monkeypatch.setattr(O, name, fn)
    for pin in pins:
        with pytest.raises(AssertionError):
            runners[pin]()


def test_oracle_pool_matches_direct_calls():
    """The spawned oracle workers the large GPU parity tests use give exactly what the
    oracle gives when called directly (selection, per-row errors on a given list, tile
    attention)."""
    from tests import oracle_pool as P
    p, q, k, v = _tiny_problem(7, nq=256, nk=640, hq=4, hkv=1, B=32, sink=6.0)
    tl = O.tiles(p)
    jobs = [(h, t.gtile, 0.05, 1, 1, 8, list(range(0, t.diag + 1, 2)) + [t.diag]) for h in (1, 3) for t in tl]
    with P.GroupPool(p, q, k, v, workers=2) as pool:
        res = pool.select(jobs)
        att = pool.attention([(1, 5, [0, 3, 5]), (2, 7, None)])
    for (h, gt, tau, ns, nl, S, kept), (sel, err, delta) in zip(jobs, res):
        ref = O.select_tile(p, q, k, v, h, tl[gt], tau, ns, nl, S)
        assert sel.retained == ref.retained and sel.order == ref.order and np.array_equal(sel.score, ref.score)
        assert np.array_equal(sel.curve, ref.curve)
        kept = sorted(set(kept))
        od, _ = O.tile_attention(p, q, k, v, h, tl[gt])
        os_, _ = O.tile_attention(p, q, k, v, h, tl[gt], kept)
        assert np.allclose(err, np.linalg.norm(od[ref.rows] - os_[ref.rows], axis=1), rtol=1e-12, atol=1e-15)
        dropped = [b for b in range(tl[gt].diag + 1) if b not in set(kept)]
        assert np.allclose(delta, ref.m[:, dropped].sum(axis=1), rtol=1e-12, atol=1e-15)
    (d, s_), = [att[0]]
    assert np.array_equal(d[0], O.tile_attention(p, q, k, v, 1, tl[5])[0])
    assert np.array_equal(s_[0], O.tile_attention(p, q, k, v, 1, tl[5], [0, 3, 5])[0])
