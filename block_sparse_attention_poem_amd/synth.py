"""Seeded synthetic Q/K/V for output-relative block-sparse prefill.

This module only draws inputs. It holds none of the method's arithmetic, so the
fp64 oracle (under ``oracle/``) and the HIP path can both consume its tensors
without sharing any computation.

Recipe (the pages measure on real model Q/K/V over RULER and similar suites;
those are stood in for by a clustered generator at the models' attention
shapes):

* Every random stream is ``PCG64(SeedSequence([seed, workload_id, seq, tensor_id, head]))``.
* Per KV head g and sequence: ``n_centers`` unit centres (normalised N(0,1)^d),
  one value offset N(0,1)^d per centre, and a block -> centre assignment made of
  runs whose lengths are uniform on {1 .. run_max}, each run's centre uniform.
  K_j = 3 C[c(j)] + N(0,1)^d and V_j = U[c(j)] + N(0,1)^d.
* Per query head h: each query tile draws ``n_t`` centres of its KV head without
  replacement (n_t fixed, or uniform on a range per tile), every row picks one
  of them uniformly, and Q_i = 3 C[c] + N(0,1)^d.
* Sink: a reserved channel. Q_i[d-1] = 1 for every query, K_0 of every sequence
  is ``L_s * sqrt(d) * e_{d-1}`` (zero elsewhere), so with the default
  1/sqrt(d) softmax scale every query gives the sink the logit L_s.
  L_s = ln(N_k) + ``sink_offset`` (default 6).
* Near-output clusters (``near_output`` = p > 0, off by default): the value offset of
  the first round(p * n_centers) centres of each KV head is replaced by the sink key's
  value vector, so their blocks' values sit near the outputs the sink dominates (the
  situation of the POEM note's three-block example, where a heavy block whose value
  equals the output costs nothing to drop). Default inputs do not change.
* Per-head thresholds tau: a fixed value, or uniform on a range per query head.
* Values are drawn in fp32 and rounded once to bf16 (round to nearest even)
  for bf16 workloads.

Layout is packed THD: Q [sum N_q, H_q, d], K and V [sum N_k, H_kv, d], with
sequences concatenated; a chunk's queries sit at absolute positions
N_k - N_q .. N_k - 1 of its sequence.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# tensor ids of the random streams
_T_CENTERS, _T_VOFF, _T_RUNS, _T_KNOISE, _T_VNOISE, _T_QTILE, _T_QNOISE, _T_TAU = range(8)


@dataclass(frozen=True)
class Workload:
    """One synthetic attention layer."""

    name: str
    workload_id: int
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    block_size: int
    seqlens_k: tuple
    seqlens_q: tuple
    n_centers: int
    run_max: int
    centers_per_tile: tuple  # (lo, hi) inclusive
    tau: tuple  # ("fixed", value) or ("uniform", lo, hi)
    n_sink_blocks: int
    n_local_blocks: int  # counts the diagonal block
    dtype: str  # "bf16" or "fp32"
    rows_per_tile: int = 8
    sink_offset: float = 6.0
    seed: int = 0
    near_output: float = 0.0

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    1: Workload("single-head d64 N2048 fp32 B64", 1, 1, 1, 64, 64, (2048,), (2048,),
                16, 1, (2, 2), ("fixed", 0.05), 1, 1, "fp32"),
    2: Workload("llama3.1-8b-shaped 32q/8kv d128 N32768 bf16 B128", 2, 32, 8, 128, 128,
                (32768,), (32768,), 64, 8, (4, 4), ("uniform", 0.02, 0.08), 1, 1, "bf16"),
    3: Workload("llama3.1-8b-shaped 32q/8kv d128 N131072 bf16 B128", 3, 32, 8, 128, 128,
                (131072,), (131072,), 64, 8, (4, 4), ("uniform", 0.02, 0.08), 1, 1, "bf16"),
    4: Workload("qwen3-14b-shaped 40q/8kv d128 N65536 bf16 B128", 4, 40, 8, 128, 128,
                (65536,), (65536,), 128, 8, (2, 6), ("fixed", 0.05), 1, 2, "bf16"),
    5: Workload("chunked varlen 4 seqs (16K,40K,72K,128K) x 8192-query chunks, 32q/8kv d128 bf16 B128",
                5, 32, 8, 128, 128, (16384, 40960, 73728, 131072), (8192,) * 4,
                64, 8, (4, 4), ("uniform", 0.02, 0.08), 1, 1, "bf16"),
}


@dataclass
class Inputs:
    workload: Workload
    q: np.ndarray  # [sum N_q, H_q, d]; uint16 bf16 bit patterns or float32
    k: np.ndarray  # [sum N_k, H_kv, d]
    v: np.ndarray
    tau: np.ndarray  # float32 [H_q]
    seqlens_q: np.ndarray = field(default=None)
    seqlens_k: np.ndarray = field(default=None)

    @property
    def is_bf16(self) -> bool:
        return self.q.dtype == np.uint16


def _rng(*entropy) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(e) for e in entropy])))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact widening of generator output (bf16 bits or fp32) to float64."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def _unit_rows(rng, n, d):
    c = rng.standard_normal((n, d), dtype=np.float32).astype(np.float64)
    c /= np.linalg.norm(c, axis=1, keepdims=True)
    return c.astype(np.float32)


def _block_centers(rng, n_blocks, n_centers, run_max):
    out = np.empty(n_blocks, dtype=np.int64)
    pos = 0
    while pos < n_blocks:
        c = int(rng.integers(n_centers))
        run = int(rng.integers(1, run_max + 1))
        out[pos:pos + run] = c
        pos += run
    return out


def _seq_kv(w: Workload, s: int, g: int, n_k: int):
    d, B = w.head_dim, w.block_size
    wid = w.workload_id
    centers = _unit_rows(_rng(w.seed, wid, s, _T_CENTERS, g), w.n_centers, d)
    voff = _rng(w.seed, wid, s, _T_VOFF, g).standard_normal((w.n_centers, d), dtype=np.float32)
    n_blocks = -(-n_k // B)
    bc = _block_centers(_rng(w.seed, wid, s, _T_RUNS, g), n_blocks, w.n_centers, w.run_max)
    cj = np.repeat(bc, B)[:n_k]
    k = _rng(w.seed, wid, s, _T_KNOISE, g).standard_normal((n_k, d), dtype=np.float32)
    k += np.float32(3.0) * centers[cj]
    v = _rng(w.seed, wid, s, _T_VNOISE, g).standard_normal((n_k, d), dtype=np.float32)
    n_near = int(round(w.near_output * w.n_centers))
    if n_near > 0:  # value offsets of the first n_near centres <- the sink key's value
        sink_v = v[0] + voff[cj[0]]
        voff = voff.copy()
        voff[:n_near] = sink_v
        v[0] = sink_v - voff[cj[0]]  # the sink's own value is unchanged
    v += voff[cj]
    # sink key at token 0: logit L_s for every query under the 1/sqrt(d) scale
    ls = math.log(n_k) + w.sink_offset
    k[0, :] = 0.0
    k[0, d - 1] = np.float32(ls * math.sqrt(d))
    return centers, k, v


def _seq_q(w: Workload, s: int, h: int, n_q: int, centers: np.ndarray):
    d, B = w.head_dim, w.block_size
    wid = w.workload_id
    rq = _rng(w.seed, wid, s, _T_QTILE, h)
    n_tiles = -(-n_q // B)
    lo, hi = w.centers_per_tile
    ci = np.empty(n_q, dtype=np.int64)
    for t in range(n_tiles):
        nt = int(rq.integers(lo, hi + 1))
        chosen = rq.choice(w.n_centers, size=nt, replace=False)
        rows = min(B, n_q - t * B)
        ci[t * B:t * B + rows] = chosen[rq.integers(0, nt, size=rows)]
    q = _rng(w.seed, wid, s, _T_QNOISE, h).standard_normal((n_q, d), dtype=np.float32)
    q += np.float32(3.0) * centers[ci]
    q[:, d - 1] = 1.0
    return q


def make(w: Workload, threads: int = 8) -> Inputs:
    """Draw the workload's Q/K/V (THD layout) and per-head thresholds."""
    Hq, Hkv, d = w.num_heads_q, w.num_heads_kv, w.head_dim
    assert Hq % Hkv == 0
    G = Hq // Hkv
    sk, sq = list(w.seqlens_k), list(w.seqlens_q)
    tot_k, tot_q = sum(sk), sum(sq)
    bf16 = w.dtype == "bf16"
    et = np.uint16 if bf16 else np.float32
    q = np.empty((tot_q, Hq, d), dtype=et)
    k = np.empty((tot_k, Hkv, d), dtype=et)
    v = np.empty((tot_k, Hkv, d), dtype=et)
    conv = round_to_bf16_bits if bf16 else (lambda a: a)
    koff = np.concatenate([[0], np.cumsum(sk)]).astype(np.int64)
    qoff = np.concatenate([[0], np.cumsum(sq)]).astype(np.int64)

    def job(s, g):
        centers, kk, vv = _seq_kv(w, s, g, sk[s])
        k[koff[s]:koff[s + 1], g, :] = conv(kk)
        v[koff[s]:koff[s + 1], g, :] = conv(vv)
        for hg in range(G):
            h = g * G + hg
            q[qoff[s]:qoff[s + 1], h, :] = conv(_seq_q(w, s, h, sq[s], centers))

    jobs = [(s, g) for s in range(len(sk)) for g in range(Hkv)]
    if threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(lambda a: job(*a), jobs))
    else:
        for a in jobs:
            job(*a)

    rt = _rng(w.seed, w.workload_id, 0, _T_TAU, 0)
    if w.tau[0] == "fixed":
        tau = np.full(Hq, w.tau[1], dtype=np.float32)
    else:
        tau = rt.uniform(w.tau[1], w.tau[2], size=Hq).astype(np.float32)
    return Inputs(w, q, k, v, tau, np.asarray(sq, np.int32), np.asarray(sk, np.int32))


def small_workload(n_q=300, n_k=300, hq=4, hkv=2, d=64, block=64, dtype="bf16",
                   seqs=1, n_centers=8, run_max=3, cpt=(2, 3), tau=("uniform", 0.02, 0.08),
                   n_sink=1, n_local=1, rows=8, sink_offset=6.0, seed=0, wid=100):
    """A small workload for tests: one or several equal-shaped sequences."""
    return Workload(f"small q{n_q} k{n_k}", wid, hq, hkv, d, block, (n_k,) * seqs, (n_q,) * seqs,
                    n_centers, run_max, cpt, tau, n_sink, n_local, dtype, rows, sink_offset, seed)


def toy_block_inputs(shift: float = 0.0):
    """The three-block example of the POEM note (masses 1/2, 1/4, 1/4 with scalar values
    2, 0, 4) realised with 64-key blocks in fp32, d = 64, softmax scale 1.

    One sequence, N_k = 256, N_q = 64 (rows at positions 192 .. 255, all with q = e_0).
    Block 0 (A): 64 keys with logit 0, value 2. Blocks 1 (B) and 2 (C): 32 keys with
    logit 0 and 32 keys with logit -60, values 0 and 4. Block 3, the rows' own block:
    logit -60, value 0. ``shift`` is added to coordinate 0 of every value."""
    n_k, n_q, d, B = 256, 64, 64, 64
    q = np.zeros((n_q, 1, d), np.float32)
    q[:, 0, 0] = 1.0
    k = np.zeros((n_k, 1, d), np.float32)
    k[96:128, 0, 0] = -60.0
    k[160:192, 0, 0] = -60.0
    k[192:256, 0, 0] = -60.0
    v = np.zeros((n_k, 1, d), np.float32)
    v[0:64, 0, 0] = 2.0
    v[128:192, 0, 0] = 4.0
    v[:, 0, 0] += np.float32(shift)
    return q, k, v, dict(n_q=n_q, n_k=n_k, d=d, block=B)
