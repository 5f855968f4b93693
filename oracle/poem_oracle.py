"""Plain fp64 CPU oracle for output-relative (POEM-style) block-sparse causal prefill.

TEST INFRASTRUCTURE. Only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code, table or helper with
the HIP path and never calls it; it is slow on purpose and written so that each
step can be read against the pages.

Sources (cited by title and section):
  [note]  the reading note on POEM's attention deletion error (Wu et al.,
          "POEM: Output-Relative Block-Sparse Attention for Long-Context
          Prefilling", arXiv:2611.13578): block decomposition and deletion
          identity (its Section 4.1, Equation (3), Appendix A.2), the three-block
          toy, the shift check, the proxy score and triangle bound (Equation (4)),
          and practical POEM (Equation (6), Appendix B).
  [BFLA]  "BFLA: Block-Filtered Long-Context Attention Mechanism": GQA head
          grouping (Section 3.3), chunk positions (Section 3.6), mandatory sink /
          local blocks (Sections 4, 5.1), tie-breaking and ascending traversal
          (Appendix A, "Block ordering"), the 2R-delta worst case (Appendix B.1)
          and nested supports (Appendix B.5).

Readings where the pages are silent (each listed in the design doc):
  * One tile decision from several sampled rows: per-row m, u, o and I; the tile
    score is the mean of I over the sampled rows; the stopping rule applies the
    triangle bound per row and takes the maximum over rows.
  * Sampled rows: even stride ending at the tile's last row,
    r_j = ceil((j+1) n_t / S_t) - 1 with S_t = min(S, n_t).
  * A discard set is acceptable iff its bound is <= tau; 1 - delta <= 0 gives +inf.
  * Ties in the score: the smaller block id is retained first, so among equal
    scores the larger id is discarded first. Retained ids are reported ascending.
  * Chunk alignment: the queries of a chunk sit at N_k - N_q .. N_k - 1 and
    (N_k - N_q) is a multiple of the block size.
  * Mass-only baseline: rank by the tile mass; cut at the last prefix whose
    largest per-row omitted mass is <= eps (the per-head budget).
  * Practical POEM: pooled estimates mbar and Ibar / mbar, preselection of the
    shortest top-mass prefix covering rho of the candidates' mass, rerank by
    log mbar + w log(Ibar / mbar), keep in that order until the pooled retained
    mass reaches (1 - eps) of the total.
  * Group-shared lists: the S sampled rows of a (KV head, tile) are spread over
    its G query heads (row j from head g G + j mod G); every sampled row's bound
    must stay within its own head's tau.

Everything is float64; inputs are widened exactly from bf16 / fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# ---------------------------------------------------------------------------
# Block decomposition and the deletion identity for one query and one head
# ([note] Section 4.1, Equation (3)).  m: masses [n_blocks], v: block mean
# values [n_blocks, d], D: iterable of discarded block indices.
# ---------------------------------------------------------------------------


def dense_output(m, v):
    """o = sum_b m_b v_b."""
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64).reshape(len(m), -1)
    return (m[:, None] * v).sum(axis=0)


def deleted_output(m, v, D):
    """Output recomputed from the retained blocks only: (o - sum_D m_b v_b) / (1 - delta).

    Written from the definition (renormalise the retained part), not from the identity."""
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64).reshape(len(m), -1)
    keep = np.ones(len(m), dtype=bool)
    keep[list(D)] = False
    retained_mass = m[keep].sum()
    return (m[keep][:, None] * v[keep]).sum(axis=0) / retained_mass


def deletion_error(m, v, D):
    """The identity: o - o_tilde = sum_{b in D} m_b (v_b - o) / (1 - delta)."""
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64).reshape(len(m), -1)
    o = dense_output(m, v)
    D = list(D)
    delta = m[D].sum()
    return (m[D][:, None] * (v[D] - o)).sum(axis=0) / (1.0 - delta)


def proxy_scores(m, v):
    """I_b = m_b ||v_b - o|| ([note] Equation (4))."""
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64).reshape(len(m), -1)
    o = dense_output(m, v)
    return m * np.linalg.norm(v - o, axis=1)


def triangle_bound(m, v, D):
    """sum_{b in D} I_b / (1 - delta), the triangle-inequality bound on ||o - o_tilde||."""
    m = np.asarray(m, dtype=np.float64)
    D = list(D)
    delta = m[D].sum()
    if delta >= 1.0:
        return math.inf
    return proxy_scores(m, v)[D].sum() / (1.0 - delta)


# ---------------------------------------------------------------------------
# Problem geometry ([BFLA] Sections 3.3 and 3.6)
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class Problem:
    seqlens_q: tuple
    seqlens_k: tuple
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    block_size: int
    softmax_scale: float = 0.0  # <= 0 means 1/sqrt(head_dim)

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.num_heads_q // self.num_heads_kv


@dataclass(frozen=True)
class Tile:
    seq: int
    t: int  # tile index inside the chunk
    gtile: int  # global tile index over all sequences
    q_row0: int  # first packed query row
    n_rows: int
    pos0: int  # absolute position of the first row inside its sequence
    diag: int  # key block that holds the tile's rows
    k_row0: int  # first packed key row of the sequence
    n_k: int


def tiles(p: Problem):
    out = []
    qo = ko = g = 0
    B = p.block_size
    for s, (nq, nk) in enumerate(zip(p.seqlens_q, p.seqlens_k)):
        start = nk - nq
        for t in range(-(-nq // B)):
            n = min(B, nq - t * B)
            out.append(Tile(s, t, g, qo + t * B, n, start + t * B, (start + t * B) // B, ko, nk))
            g += 1
        qo += nq
        ko += nk
    return out


def sampled_rows(n_rows: int, S: int):
    """Local row indices sampled in a tile: r_j = ceil((j+1) n / S_t) - 1, S_t = min(S, n)."""
    St = min(S, n_rows)
    return [-(-((j + 1) * n_rows) // St) - 1 for j in range(St)]


def mandatory_blocks(diag: int, n_sink: int, n_local: int):
    """Sink blocks 0 .. n_sink-1 and local blocks diag-n_local+1 .. diag (the diagonal included)."""
    return sorted({b for b in range(min(n_sink, diag + 1))} |
                  {b for b in range(max(0, diag - n_local + 1), diag + 1)})


# ---------------------------------------------------------------------------
# Attention (textbook softmax, max subtracted)
# ---------------------------------------------------------------------------


def attention_rows(qr, K, V, scale, positions, key_allowed=None):
    """Causal softmax attention of query rows qr [n, d] against keys K, V [n_k, d].

    Row i sees keys j <= positions[i] (and, if given, key_allowed[j]).
    Returns O [n, d] and natural-log LSE [n]; a row that sees no key gets O = 0, LSE = -inf."""
    qr = np.asarray(qr, dtype=np.float64)
    n = qr.shape[0]
    pmax = int(max(positions)) + 1
    s = scale * (qr @ np.asarray(K[:pmax], dtype=np.float64).T)
    j = np.arange(pmax)
    ok = j[None, :] <= np.asarray(positions)[:, None]
    if key_allowed is not None:
        ok &= np.asarray(key_allowed[:pmax], dtype=bool)[None, :]
    s = np.where(ok, s, -np.inf)
    M = s.max(axis=1)
    O = np.zeros((n, qr.shape[1]))
    lse = np.full(n, -np.inf)
    live = np.isfinite(M)
    if live.any():
        e = np.exp(s[live] - M[live, None])
        Z = e.sum(axis=1)
        O[live] = (e @ np.asarray(V[:pmax], dtype=np.float64)) / Z[:, None]
        lse[live] = M[live] + np.log(Z)
    return O, lse


def _head_view(x, row0, n, head):
    return x[row0:row0 + n, head, :]


def tile_attention(p: Problem, q, k, v, h: int, tile: Tile, blocks=None):
    """O and LSE of one (query head, tile); blocks=None is dense, else only those key blocks."""
    g = h // p.group
    Q = _head_view(q, tile.q_row0, tile.n_rows, h)
    K = _head_view(k, tile.k_row0, tile.n_k, g)
    V = _head_view(v, tile.k_row0, tile.n_k, g)
    pos = [tile.pos0 + i for i in range(tile.n_rows)]
    allowed = None
    if blocks is not None:
        allowed = np.zeros(tile.n_k, dtype=bool)
        for b in blocks:
            allowed[b * p.block_size:(b + 1) * p.block_size] = True
    return attention_rows(Q, K, V, p.scale, pos, allowed)


# ---------------------------------------------------------------------------
# Per-row block statistics ([note] Section 4.1, Equation (4))
# ---------------------------------------------------------------------------


def row_block_stats(qr, K, V, scale, pos: int, n_vis: int, B: int):
    """For one query row at absolute position pos over visible blocks 0 .. n_vis-1:
    dense softmax probabilities p_j (j <= pos), the dense output o, and per block
    the mass m_b = sum_{j in b} p_j, the weighted sum u_b = sum_{j in b} p_j v_j
    (= m_b v_b) and the proxy I_b = ||u_b - m_b o|| (= m_b ||v_b - o||)."""
    qr = np.asarray(qr, dtype=np.float64)
    Kv = np.asarray(K[:pos + 1], dtype=np.float64)
    Vv = np.asarray(V[:pos + 1], dtype=np.float64)
    s = scale * (Kv @ qr)
    M = s.max()
    e = np.exp(s - M)
    Z = e.sum()
    pr = e / Z
    o = pr @ Vv
    m = np.zeros(n_vis)
    u = np.zeros((n_vis, Kv.shape[1]))
    for b in range(n_vis):
        lo, hi = b * B, min((b + 1) * B, pos + 1)
        if lo < hi:
            m[b] = pr[lo:hi].sum()
            u[b] = pr[lo:hi] @ Vv[lo:hi]
    I = np.linalg.norm(u - m[:, None] * o[None, :], axis=1)
    return dict(M=M, Z=Z, lse=M + math.log(Z), o=o, m=m, u=u, I=I)


# ---------------------------------------------------------------------------
# Ranking and threshold ([note] Equation (4); tie rule [BFLA] Appendix A)
# ---------------------------------------------------------------------------


def discard_order(scores, candidates):
    """Candidates ordered lowest score first; equal scores: larger id first.

    The reverse of this order retains the highest scores first and, among equal
    scores, the smaller id first."""
    return sorted(candidates, key=lambda b: (float(scores[b]), -int(b)))


def bound_curve(I_rows, m_rows, order):
    """B(k) for k = 0 .. len(order): max over sampled rows i of
    A_i(k) / (1 - Delta_i(k)), with A_i(k) = sum of I_i over the first k blocks of
    the discard order and Delta_i(k) the sum of m_i over them (+inf once
    1 - Delta_i <= 0). Also returns the per-row bounds [k, row]."""
    I_rows = np.asarray(I_rows, dtype=np.float64)
    m_rows = np.asarray(m_rows, dtype=np.float64)
    nrow = I_rows.shape[0]
    per_row = np.zeros((len(order) + 1, nrow))
    A = np.zeros(nrow)
    Dl = np.zeros(nrow)
    for k in range(1, len(order) + 1):
        b = order[k - 1]
        A = A + I_rows[:, b]
        Dl = Dl + m_rows[:, b]
        with np.errstate(divide="ignore"):
            per_row[k] = np.where(1.0 - Dl > 0.0, A / np.maximum(1.0 - Dl, 1e-300), np.inf)
    return per_row.max(axis=1), per_row


def cut(curve, tau: float) -> int:
    """k* = the largest k with B(k') <= tau for every k' <= k (B(0) = 0)."""
    k = 0
    while k + 1 < len(curve) and curve[k + 1] <= tau:
        k += 1
    return k


@dataclass
class TileSelection:
    h: int
    tile: Tile
    rows: list  # local sampled rows
    I: np.ndarray  # [S_t, n_vis]
    m: np.ndarray  # [S_t, n_vis]
    lse: np.ndarray  # [S_t]
    o: np.ndarray  # [S_t, d]
    score: np.ndarray  # [n_vis] mean of I over sampled rows
    mass: np.ndarray  # [n_vis] mean of m over sampled rows
    mandatory: list
    order: list  # discard order of the candidates
    curve: np.ndarray  # B(k), k = 0 .. |candidates|
    per_row: np.ndarray  # [|cand|+1, S_t]
    k_star: int
    retained: list  # ascending
    heads: list = None  # group selection: query head of each sampled row

    @property
    def discarded(self):
        return self.order[:self.k_star]

    @property
    def row_bound(self):
        return self.per_row[self.k_star]


def select_tile(p: Problem, q, k, v, h: int, tile: Tile, tau: float, n_sink: int,
                n_local: int, S: int) -> TileSelection:
    """The selector for one (query head, tile), step by step:
    sample rows; per row dense softmax, block masses m, block sums u, output o and
    proxies I; tile score = mean of I; mandatory set; discard order; bound curve;
    cut; retained set."""
    g = h // p.group
    K = _head_view(k, tile.k_row0, tile.n_k, g)
    V = _head_view(v, tile.k_row0, tile.n_k, g)
    n_vis = tile.diag + 1
    rows = sampled_rows(tile.n_rows, S)
    stats = [row_block_stats(q[tile.q_row0 + r, h, :], K, V, p.scale, tile.pos0 + r, n_vis, p.block_size)
             for r in rows]
    I = np.stack([st["I"] for st in stats])
    m = np.stack([st["m"] for st in stats])
    score = I.mean(axis=0)
    mass = m.mean(axis=0)
    mand = mandatory_blocks(tile.diag, n_sink, n_local)
    cand = [b for b in range(n_vis) if b not in set(mand)]
    order = discard_order(score, cand)
    curve, per_row = bound_curve(I, m, order)
    ks = cut(curve, float(tau))
    drop = set(order[:ks])
    retained = [b for b in range(n_vis) if b not in drop]
    return TileSelection(h, tile, rows, I, m, np.array([st["lse"] for st in stats]),
                         np.stack([st["o"] for st in stats]), score, mass, mand, order, curve,
                         per_row, ks, retained)


# ---------------------------------------------------------------------------
# Mass-only selector: the baseline the note measures POEM against (ranking by
# attention mass alone). Ranking key: the tile mass mean of m over the sampled
# rows. Stopping rule (a reading; the pages fix no mass threshold): a discard set
# is acceptable while every sampled row keeps all but at most eps of its dense
# mass, i.e. max_i Delta_i(k) <= eps. With values of norm <= R that caps each
# sampled row's error at 2 R eps ([BFLA] Appendix B.1, worst case 2 R delta).
# ---------------------------------------------------------------------------


def mass_curve(m_rows, order):
    """Delta(k) for k = 0 .. len(order): max over sampled rows of the summed mass
    of the first k blocks of the discard order; also the per-row values [k, row]."""
    m_rows = np.asarray(m_rows, dtype=np.float64)
    per_row = np.zeros((len(order) + 1, m_rows.shape[0]))
    for k in range(1, len(order) + 1):
        per_row[k] = per_row[k - 1] + m_rows[:, order[k - 1]]
    return per_row.max(axis=1), per_row


def select_tile_mass(p: Problem, q, k, v, h: int, tile: Tile, eps: float, n_sink: int,
                     n_local: int, S: int) -> TileSelection:
    """Mass-only selection for one (query head, tile): the same sampled rows and
    per-row block masses as select_tile, ranked by the tile mass (discard order:
    lowest mass first, larger id first among equal masses) and cut at the last
    prefix whose largest per-row omitted mass is <= eps. `score` holds the ranking
    key (the tile mass); I and o are reported as in select_tile."""
    g = h // p.group
    K = _head_view(k, tile.k_row0, tile.n_k, g)
    V = _head_view(v, tile.k_row0, tile.n_k, g)
    n_vis = tile.diag + 1
    rows = sampled_rows(tile.n_rows, S)
    stats = [row_block_stats(q[tile.q_row0 + r, h, :], K, V, p.scale, tile.pos0 + r, n_vis, p.block_size)
             for r in rows]
    I = np.stack([st["I"] for st in stats])
    m = np.stack([st["m"] for st in stats])
    mass = m.mean(axis=0)
    mand = mandatory_blocks(tile.diag, n_sink, n_local)
    cand = [b for b in range(n_vis) if b not in set(mand)]
    order = discard_order(mass, cand)
    curve, per_row = mass_curve(m, order)
    ks = cut(curve, float(eps))
    drop = set(order[:ks])
    retained = [b for b in range(n_vis) if b not in drop]
    return TileSelection(h, tile, rows, I, m, np.array([st["lse"] for st in stats]),
                         np.stack([st["o"] for st in stats]), mass, mass, mand, order, curve,
                         per_row, ks, retained)


# ---------------------------------------------------------------------------
# GQA-group-shared selection: one list per (KV head, tile) for the G query heads
# that share the KV head ([BFLA] Section 3.3 shares K/V across a head group).
# Reading: the S sampled rows of the tile (the positions of sampled_rows) are spread
# over the group: row j is taken from query head g G + (j mod G). The score of a
# block is the mean of I over those rows and the discard order is as in
# select_tile. A discard set is acceptable iff every sampled row's bound
# A_i / (1 - Delta_i) is <= the threshold of that row's head, so each sampled row
# keeps the triangle-bound guarantee of its own head.
# ---------------------------------------------------------------------------


def group_excess_curve(I_rows, m_rows, order, row_tau):
    """E(k) = max over sampled rows of (A_i(k) / (1 - Delta_i(k)) - tau_i) for
    k = 0 .. len(order): a prefix is acceptable iff E(k) <= 0. Also the per-row
    bounds [k, row]."""
    _, per_row = bound_curve(I_rows, m_rows, order)
    excess = per_row - np.asarray(row_tau, dtype=np.float64)[None, :]
    return excess.max(axis=1), per_row


def select_tile_group(p: Problem, q, k, v, g: int, tile: Tile, tau, n_sink: int, n_local: int,
                      S: int) -> TileSelection:
    """Group-shared selection for KV head g and one tile; tau: thresholds of all
    query heads. The returned selection (h = g G) holds the sampled rows, their
    heads, the group score and the shared retained list."""
    G = p.group
    K = _head_view(k, tile.k_row0, tile.n_k, g)
    V = _head_view(v, tile.k_row0, tile.n_k, g)
    n_vis = tile.diag + 1
    rows = sampled_rows(tile.n_rows, S)
    heads = [g * G + (j % G) for j in range(len(rows))]
    stats = [row_block_stats(q[tile.q_row0 + r, h, :], K, V, p.scale, tile.pos0 + r, n_vis, p.block_size)
             for r, h in zip(rows, heads)]
    I = np.stack([st["I"] for st in stats])
    m = np.stack([st["m"] for st in stats])
    score = I.mean(axis=0)
    mass = m.mean(axis=0)
    mand = mandatory_blocks(tile.diag, n_sink, n_local)
    cand = [b for b in range(n_vis) if b not in set(mand)]
    order = discard_order(score, cand)
    curve, per_row = group_excess_curve(I, m, order, [float(tau[h]) for h in heads])
    ks = cut(curve, 0.0)
    drop = set(order[:ks])
    retained = [b for b in range(n_vis) if b not in drop]
    return TileSelection(g * G, tile, rows, I, m, np.array([st["lse"] for st in stats]),
                         np.stack([st["o"] for st in stats]), score, mass, mand, order, curve,
                         per_row, ks, retained, heads)


# ---------------------------------------------------------------------------
# Practical POEM ([note] Equation (6) and its selection procedure, Appendix B):
# estimates of block mass and output deviation, a mass preselection, a rerank by
# log mass plus a weighted log deviation, and a retention threshold on pooled mass
# accumulated in the reranked order.
# Readings (the pages leave these open):
#   estimates   pooled over the sampled rows: mbar_b (mean mass) and the deviation
#               dhat_b = Ibar_b / mbar_b, the mass-weighted mean of ||v_ib - o_i||;
#   preselect   the shortest prefix of the candidates in (mbar descending, id
#               ascending) order whose mass reaches rho times the candidates' mass;
#   rerank      the preselected blocks by log mbar_b + w log dhat_b, descending (a
#               block with zero mass, or with zero deviation when w != 0, scores
#               -inf; with w = 0 the deviation term is absent), smaller id first
#               among equal scores;
#   threshold   blocks are kept in that order until the pooled retained mass
#               (mandatory blocks included) reaches (1 - eps) of the pooled total.
# w, rho and the per-head eps are parameters.
# ---------------------------------------------------------------------------


def practical_keys(mbar, Ibar, w: float):
    """Rerank score log mbar + w log(Ibar / mbar) per block: -inf for a block with no
    mass, or (when w != 0) with no deviation; with w = 0 the deviation term is absent."""
    mbar = np.asarray(mbar, dtype=np.float64)
    Ibar = np.asarray(Ibar, dtype=np.float64)
    out = np.full(len(mbar), -np.inf)
    okm = mbar > 0
    out[okm] = np.log(mbar[okm])
    if w != 0.0:
        okI = okm & (Ibar > 0)
        out[okm & ~okI] = -np.inf
        out[okI] += w * np.log(Ibar[okI] / mbar[okI])
    return out


def practical_retain(mbar, Ibar, mandatory, candidates, eps: float, w: float, rho: float):
    """The practical selection from pooled estimates. Returns (preselected, reranked
    order, kept candidates)."""
    mbar = np.asarray(mbar, dtype=np.float64)
    by_mass = sorted(candidates, key=lambda b: (-float(mbar[b]), int(b)))
    cum = np.cumsum([mbar[b] for b in by_mass]) if by_mass else np.zeros(0)
    need = rho * (cum[-1] if len(cum) else 0.0)
    n_pre = 0
    while n_pre < len(by_mass) and (n_pre == 0 or cum[n_pre - 1] < need):
        n_pre += 1
    if len(cum) and need <= 0.0:
        n_pre = 0
    pre = by_mass[:n_pre]
    key = practical_keys(mbar, Ibar, w)
    order = sorted(pre, key=lambda b: (-float(key[b]), int(b)))
    target = (1.0 - eps) * float(mbar.sum())
    acc = float(sum(mbar[b] for b in mandatory))
    kept = []
    for b in order:
        if acc >= target:
            break
        kept.append(b)
        acc += float(mbar[b])
    return pre, order, kept


def select_tile_practical(p: Problem, q, k, v, h: int, tile: Tile, eps: float, n_sink: int, n_local: int,
                          S: int, w: float = 0.5, rho: float = 0.95) -> TileSelection:
    """Practical POEM for one (query head, tile). `order` holds the reranked
    preselected blocks, `score` the rerank score, `per_row` the per-row omitted mass of
    the final discard set (one row), k_star the number of discarded candidates."""
    g = h // p.group
    K = _head_view(k, tile.k_row0, tile.n_k, g)
    V = _head_view(v, tile.k_row0, tile.n_k, g)
    n_vis = tile.diag + 1
    rows = sampled_rows(tile.n_rows, S)
    stats = [row_block_stats(q[tile.q_row0 + r, h, :], K, V, p.scale, tile.pos0 + r, n_vis, p.block_size)
             for r in rows]
    I = np.stack([st["I"] for st in stats])
    m = np.stack([st["m"] for st in stats])
    Ibar = I.mean(axis=0)
    mbar = m.mean(axis=0)
    mand = mandatory_blocks(tile.diag, n_sink, n_local)
    cand = [b for b in range(n_vis) if b not in set(mand)]
    pre, order, kept = practical_retain(mbar, Ibar, mand, cand, float(eps), float(w), float(rho))
    retained = sorted(set(mand) | set(kept))
    drop = [b for b in range(n_vis) if b not in set(retained)]
    omitted = m[:, drop].sum(axis=1) if drop else np.zeros(len(rows))
    return TileSelection(h, tile, rows, I, m, np.array([st["lse"] for st in stats]),
                         np.stack([st["o"] for st in stats]), practical_keys(mbar, Ibar, w), mbar, mand, order,
                         np.zeros(0), omitted[None, :], len(drop), retained)


def select(p: Problem, q, k, v, tau, n_sink: int, n_local: int, S: int, which=None, mode: str = "poem",
           practical=None):
    """Selections for every (head, tile), or for the (h, gtile) pairs in `which`.
    mode "poem" uses the output-relative selector (tau: error threshold per head),
    "mass" the mass-only one (tau: omitted-mass budget per head), "group" the
    group-shared output-relative selector (one list per KV head and tile),
    "practical" practical POEM (tau: pooled omitted-mass budget per head;
    practical = dict(w=..., rho=...)).

    Returns {(h, gtile): TileSelection}."""
    tl = tiles(p)
    if which is None:
        which = [(h, t.gtile) for h in range(p.num_heads_q) for t in tl]
    if mode == "group":
        # one selection per (KV head, tile), shared by the heads of the group
        shared = {}
        out = {}
        for (h, gt) in which:
            key = (h // p.group, gt)
            if key not in shared:
                shared[key] = select_tile_group(p, q, k, v, key[0], tl[gt], tau, n_sink, n_local, S)
            out[(h, gt)] = shared[key]
        return out
    if mode == "practical":
        return {(h, gt): select_tile_practical(p, q, k, v, h, tl[gt], float(tau[h]), n_sink, n_local, S,
                                               **(practical or {}))
                for (h, gt) in which}
    fn = {"poem": select_tile, "mass": select_tile_mass}[mode]
    return {(h, gt): fn(p, q, k, v, h, tl[gt], float(tau[h]), n_sink, n_local, S)
            for (h, gt) in which}


def csr(p: Problem, selections):
    """CSR over rows h * total_tiles + gtile from a complete selection dict."""
    tl = tiles(p)
    nrows = p.num_heads_q * len(tl)
    row_ptr = np.zeros(nrows + 1, dtype=np.int64)
    ids = []
    for h in range(p.num_heads_q):
        for t in tl:
            r = selections[(h, t.gtile)].retained
            row_ptr[h * len(tl) + t.gtile + 1] = len(r)
            ids.extend(r)
    return np.cumsum(row_ptr), np.asarray(ids, dtype=np.int64)


def csr_capacity(p: Problem) -> int:
    return p.num_heads_q * sum(t.diag + 1 for t in tiles(p))


# ---------------------------------------------------------------------------
# Sparse output from dense quantities, the second independent computation
# ([note] Section 4.1: o_tilde = (o - sum_D m_b v_b) / (1 - delta)).
# ---------------------------------------------------------------------------


def tile_attention_via_identity(p: Problem, q, k, v, h: int, tile: Tile, blocks):
    g = h // p.group
    K = _head_view(k, tile.k_row0, tile.n_k, g)
    V = _head_view(v, tile.k_row0, tile.n_k, g)
    keep = set(blocks)
    n_vis = tile.diag + 1
    O = np.zeros((tile.n_rows, p.head_dim))
    lse = np.full(tile.n_rows, -np.inf)
    for r in range(tile.n_rows):
        st = row_block_stats(q[tile.q_row0 + r, h, :], K, V, p.scale, tile.pos0 + r, n_vis, p.block_size)
        D = [b for b in range(n_vis) if b not in keep]
        delta = st["m"][D].sum()
        if delta >= 1.0 or not keep:
            continue
        O[r] = (st["o"] - st["u"][D].sum(axis=0)) / (1.0 - delta)
        lse[r] = st["lse"] + math.log1p(-delta)
    return O, lse


# ---------------------------------------------------------------------------
# Whole-problem prefill (for small problems and for sampled tiles)
# ---------------------------------------------------------------------------


def dense_prefill(p: Problem, q, k, v, which=None):
    """{(h, gtile): (O, LSE)} for dense causal attention."""
    tl = tiles(p)
    if which is None:
        which = [(h, t.gtile) for h in range(p.num_heads_q) for t in tl]
    return {(h, gt): tile_attention(p, q, k, v, h, tl[gt]) for (h, gt) in which}


def sparse_prefill(p: Problem, q, k, v, row_ptr, block_idx, which=None):
    """{(h, gtile): (O, LSE)} attending only to the CSR row's blocks. A retained set is
    a subset of the tile's visible blocks 0 .. diag ([note] Section 4.1), so ids
    outside that range take no part."""
    tl = tiles(p)
    T = len(tl)
    if which is None:
        which = [(h, t.gtile) for h in range(p.num_heads_q) for t in tl]
    out = {}
    for (h, gt) in which:
        r = h * T + gt
        ids = [int(b) for b in block_idx[row_ptr[r]:row_ptr[r + 1]] if 0 <= b <= tl[gt].diag]
        out[(h, gt)] = tile_attention(p, q, k, v, h, tl[gt], ids)
    return out
