"""Host-side tests of libpoem's C ABI (no GPU needed).

The library must load without a GPU, export every symbol include/poem.h declares,
and reject every invalid argument with the documented status before anything is
enqueued (so these calls never touch the HIP runtime's device paths).
"""
import ctypes
import os
import re

import pytest

from block_sparse_attention_poem_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x100000)  # never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libpoem.so is not built; run python -m block_sparse_attention_poem_amd.build")
    return L.load()


def header_functions():
    src = open(os.path.join(ROOT, "include", "poem.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(poem_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert set(declared) == set(L.SYMBOLS), declared
    for name in declared:
        assert hasattr(lib, name), name
    assert "gfx950" in L.version()


def test_binding_constants_match_header():
    src = open(os.path.join(ROOT, "include", "poem.h")).read()
    m = re.search(r"#define\s+POEM_DENSE_WORKSPACE_BYTES\s+(\d+)", src)
    assert m and int(m.group(1)) == L.POEM_DENSE_WORKSPACE_BYTES


def prob(**kw):
    d = dict(seqlens_q=[300], seqlens_k=[428], num_heads_q=4, num_heads_kv=2, head_dim=64, block_size=64,
             softmax_scale=0.0, dtype="bf16")
    d.update(kw)
    return L.Problem(**d)


def test_geometry_queries(lib):
    p = prob()
    # tiles of 64 rows: 5 tiles, diagonals 2..6 -> visible 3..7
    assert L.num_tiles(p) == 5
    assert L.max_visible_blocks(p) == 7
    assert L.csr_capacity(p) == 4 * (3 + 4 + 5 + 6 + 7)
    p2 = prob(seqlens_q=[64, 0, 100], seqlens_k=[128, 64, 100])
    assert L.num_tiles(p2) == 1 + 0 + 2
    assert L.csr_capacity(p2) == 4 * (2 + 1 + 2)
    ws = L.select_workspace_bytes(p, 8)
    assert ws > 0 and ws % 256 == 0


def _sweep_chunks(seqs, hkv, TG, max_chunks):
    """The selector's chunking of a sweep: the largest power-of-two chunk of 1024 .. 1
    blocks giving at least 1024 non-empty workgroups, doubled while a tile group would
    need more than max_chunks chunks. seqs: [(diag0, n_tiles)]."""
    mx = max([1] + [d + n for d, n in seqs if n > 0])
    nonempty = lambda C: hkv * sum(-(-(d + min(t0 + TG, n)) // C) for d, n in seqs for t0 in range(0, n, TG))
    C = 1024
    while C > 1 and nonempty(C) < 1024:
        C //= 2
    while -(-mx // C) > max_chunks:
        C *= 2
    return C, -(-mx // C)


def _select_layout_bytes(p, S, group_mode):
    """Per (KV head, tile) records of 2 d + 4 floats per column; partial records of
    pass 1's later chunks (d + 4 floats); per visible (tile, block) I and m per column;
    per query head counts and slots; bf16: the fp16 copy of V and its block scales.
    Selector workgroups hold 8 waves of 32 columns for bf16, 4 for fp32."""
    a256 = lambda x: -(-x // 256) * 256
    B, d, hkv = p.block_size, p.head_dim, p.num_heads_kv
    G = p.num_heads_q // hkv
    seqs = [((nk - nq) // B, -(-nq // B)) for nq, nk in zip(p.seqlens_q, p.seqlens_k)]
    T = sum(n for _, n in seqs)
    vis = sum(sum(d0 + t + 1 for t in range(n)) for d0, n in seqs)
    cols = S if group_mode else G * S
    total = a256(4 * hkv * T * cols * (2 * d + 4))
    waves = 8 if p.dtype == "bf16" else 4
    TG = waves * (32 // S) if group_mode else max(1, 32 * waves // cols)
    _, nch = _sweep_chunks(seqs, hkv, TG, 8)
    total += a256(4 * hkv * T * cols * (nch - 1) * (d + 4))
    total += a256(4 * hkv * vis * cols * 2) + a256(4 * p.num_heads_q * T) + a256(4 * p.num_heads_q * vis)
    if p.dtype == "bf16":
        nk = sum(p.seqlens_k)
        kblocks = sum(-(-n // B) for n in p.seqlens_k)
        total += a256(2 * nk * hkv * d) + a256(4 * hkv * kblocks)
    return total


def test_select_workspace_layout():
    """The select workspace is the larger of the per-head and group-shared layouts, with
    pass 1's partial records when its tile groups are split into chunks; bf16 inputs add
    an fp16 copy of V and one fp32 scale per (key block, KV head)."""
    cases = (dict(), dict(seqlens_q=[64, 0, 100], seqlens_k=[128, 64, 100]),
             dict(seqlens_q=[100], seqlens_k=[4196], head_dim=128, block_size=128),
             dict(seqlens_q=[128], seqlens_k=[66048], head_dim=64, block_size=64),
             dict(seqlens_q=[8192] * 2, seqlens_k=[16384, 131072], num_heads_q=32, num_heads_kv=8, head_dim=128,
                  block_size=128))
    for kw in cases:
        for dt in ("bf16", "fp32"):
            p = prob(dtype=dt, **kw)
            want = max(_select_layout_bytes(p, 8, True), _select_layout_bytes(p, 8, False))
            assert L.select_workspace_bytes(p, 8) == want, (kw, dt)
    # the long-prefix case runs pass 1 in chunks: five of 256 blocks (1032 blocks, one group)
    assert _sweep_chunks([(1030, 2)], 1, 8, 8) == (256, 5)
    # a small problem goes down to one-block chunks for pass 2 (the single-head 2K
    # workload: 32 tiles of 64 rows, 16 tiles per fp32 workgroup), four-block chunks
    # for pass 1 (at most eight chunks per group)
    assert _sweep_chunks([(0, 32)], 1, 16, 4096) == (1, 32)
    assert _sweep_chunks([(0, 32)], 1, 16, 8) == (4, 8)


@pytest.mark.parametrize("kw,status", [
    (dict(seqlens_q=[300], seqlens_k=[429]), L.POEM_ERR_INVALID_ARG),   # N_k - N_q not a multiple of B
    (dict(seqlens_q=[300], seqlens_k=[200]), L.POEM_ERR_INVALID_ARG),   # N_k < N_q
    (dict(seqlens_q=[-1], seqlens_k=[64]), L.POEM_ERR_INVALID_ARG),
    (dict(num_heads_q=3, num_heads_kv=2), L.POEM_ERR_INVALID_ARG),
    (dict(num_heads_q=0), L.POEM_ERR_INVALID_ARG),
    (dict(head_dim=96), L.POEM_ERR_UNSUPPORTED),
    (dict(head_dim=0), L.POEM_ERR_INVALID_ARG),
    (dict(block_size=32), L.POEM_ERR_UNSUPPORTED),
    (dict(block_size=-64), L.POEM_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), L.POEM_ERR_INVALID_ARG),
    (dict(softmax_scale=float("inf")), L.POEM_ERR_INVALID_ARG),
    (dict(seqlens_q=[64] * 65, seqlens_k=[64] * 65), L.POEM_ERR_UNSUPPORTED),
    (dict(seqlens_q=[], seqlens_k=[]), L.POEM_ERR_INVALID_ARG),
])
def test_problem_validation(lib, kw, status):
    p = prob(**kw).c()
    assert lib.poem_num_tiles(ctypes.byref(p)) == status
    assert lib.poem_last_error().decode() != ""
    rc = lib.poem_dense_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, L.POEM_FP32, None, None, 0, None)
    assert rc == status


def test_bad_dtype_and_null_problem(lib):
    p = prob().c()
    p.in_dtype = 7
    assert lib.poem_num_tiles(ctypes.byref(p)) == L.POEM_ERR_INVALID_ARG
    assert lib.poem_num_tiles(None) == L.POEM_ERR_INVALID_ARG
    assert "NULL" in lib.poem_last_error().decode()


def _select(lib, p, **over):
    cp = p.c()
    H = p.num_heads_q
    args = dict(q=FAKE, k=FAKE, v=FAKE, tau=(ctypes.c_float * H)(*([0.05] * H)), sink=1, local=1, S=8,
                row_ptr=FAKE, block_idx=FAKE, cap=L.csr_capacity(p), ts=None, tm=None, rb=None,
                ws=ctypes.c_void_p(0x200000), ws_bytes=L.select_workspace_bytes(p, 8))
    args.update(over)
    fn = args.pop("fn", "poem_select")
    if fn == "poem_select_practical":
        return lib.poem_select_practical(ctypes.byref(cp), args["q"], args["k"], args["v"], args["tau"], args["sink"],
                                         args["local"], args["S"], args.get("weight", 0.5), args.get("presel", 0.95),
                                         args["row_ptr"], args["block_idx"], args["cap"], args["ts"], args["tm"],
                                         args["rb"], args["ws"], args["ws_bytes"], None)
    fn = getattr(lib, fn)
    return fn(ctypes.byref(cp), args["q"], args["k"], args["v"], args["tau"], args["sink"],
                           args["local"], args["S"], args["row_ptr"], args["block_idx"], args["cap"], args["ts"],
                           args["tm"], args["rb"], args["ws"], args["ws_bytes"], None)


def test_select_validation(lib):
    p = prob()
    H = p.num_heads_q
    cases = [
        (dict(q=None), L.POEM_ERR_INVALID_ARG),
        (dict(row_ptr=None), L.POEM_ERR_INVALID_ARG),
        (dict(tau=None), L.POEM_ERR_INVALID_ARG),
        (dict(tau=(ctypes.c_float * H)(0.05, -0.1, 0.05, 0.05)), L.POEM_ERR_INVALID_ARG),
        (dict(tau=(ctypes.c_float * H)(0.05, float("nan"), 0.05, 0.05)), L.POEM_ERR_INVALID_ARG),
        (dict(tau=(ctypes.c_float * H)(0.05, float("inf"), 0.05, 0.05)), L.POEM_ERR_INVALID_ARG),
        (dict(sink=-1), L.POEM_ERR_INVALID_ARG),
        (dict(local=0), L.POEM_ERR_INVALID_ARG),
        (dict(S=0), L.POEM_ERR_INVALID_ARG),
        (dict(S=33), L.POEM_ERR_UNSUPPORTED),
        (dict(cap=L.csr_capacity(p) - 1), L.POEM_ERR_CAPACITY),
        (dict(ws=None), L.POEM_ERR_WORKSPACE),
        (dict(ws_bytes=4096), L.POEM_ERR_WORKSPACE),
        (dict(ws=ctypes.c_void_p(0x200010)), L.POEM_ERR_WORKSPACE),
    ]
    for fn in ("poem_select", "poem_select_mass", "poem_select_group", "poem_select_practical"):
        for over, status in cases:
            assert _select(lib, p, fn=fn, **over) == status, (fn, over)
            assert lib.poem_last_error().decode() != ""
    for over in (dict(weight=float("nan")), dict(weight=float("inf")), dict(presel=0.0), dict(presel=1.5),
                 dict(presel=float("nan"))):
        assert _select(lib, p, fn="poem_select_practical", **over) == L.POEM_ERR_INVALID_ARG, over
    # per-head lists use the largest layout, which the reported size covers exactly
    assert _select(lib, p, ws_bytes=L.select_workspace_bytes(p, 8) - 1) == L.POEM_ERR_WORKSPACE


def test_select_limits(lib):
    # 16 query heads per KV head x 16 rows = 256 columns > 128
    p = prob(num_heads_q=16, num_heads_kv=1)
    assert L.select_workspace_bytes(p, 8) > 0
    cp = p.c()
    # per-head lists are not built for 256 columns; a group-shared list has S columns
    ws16 = lib.poem_select_workspace_bytes(ctypes.byref(cp), 16)
    assert ws16 > 0
    assert _select(lib, p, S=16, ws_bytes=ws16) == L.POEM_ERR_UNSUPPORTED
    assert _select(lib, p, S=16, ws_bytes=ws16 - 256, fn="poem_select_group") == L.POEM_ERR_WORKSPACE
    assert _select(lib, p, S=16, ws_bytes=ws16 - 256, fn="poem_select_mass") == L.POEM_ERR_UNSUPPORTED
    # more than POEM_MAX_VISIBLE_BLOCKS blocks visible to a tile
    big = prob(seqlens_q=[64], seqlens_k=[64 * 5000])
    assert _select(lib, big) == L.POEM_ERR_UNSUPPORTED
    heads = prob(num_heads_q=130, num_heads_kv=65)
    tau = (ctypes.c_float * 130)(*([0.05] * 130))
    assert _select(lib, heads, tau=tau) == L.POEM_ERR_UNSUPPORTED


def test_attention_validation(lib):
    cp = prob().c()
    assert lib.poem_dense_prefill(ctypes.byref(cp), None, FAKE, FAKE, FAKE, L.POEM_FP32, None, None, 0, None) == \
        L.POEM_ERR_INVALID_ARG
    assert lib.poem_dense_prefill(ctypes.byref(cp), FAKE, FAKE, FAKE, None, L.POEM_FP32, None, None, 0, None) == \
        L.POEM_ERR_INVALID_ARG
    assert lib.poem_dense_prefill(ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, 5, None, None, 0, None) == \
        L.POEM_ERR_INVALID_ARG
    assert lib.poem_sparse_prefill(ctypes.byref(cp), FAKE, FAKE, FAKE, None, FAKE, FAKE, L.POEM_FP32, None,
                                   None, 0, None) == L.POEM_ERR_INVALID_ARG
    assert lib.poem_sparse_prefill(ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, None, FAKE, L.POEM_FP32, None,
                                   None, 0, None) == L.POEM_ERR_INVALID_ARG
    need = L.sparse_workspace_bytes(prob())
    assert need == 256 + ((4 * 4 * 5 + 255) // 256) * 256
    ws = ctypes.c_void_p(0x300000)
    assert lib.poem_sparse_prefill(ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, L.POEM_FP32, None,
                                   ws, need - 1, None) == L.POEM_ERR_WORKSPACE
    assert lib.poem_sparse_prefill(ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, L.POEM_FP32, None,
                                   ctypes.c_void_p(0x300004), need, None) == L.POEM_ERR_WORKSPACE
    # the dense tile queue: POEM_DENSE_WORKSPACE_BYTES, 256-byte aligned
    assert L.POEM_DENSE_WORKSPACE_BYTES == 256
    assert lib.poem_dense_prefill(ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, L.POEM_FP32, None, ws,
                                  L.POEM_DENSE_WORKSPACE_BYTES - 1, None) == L.POEM_ERR_WORKSPACE
    assert lib.poem_dense_prefill(ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, L.POEM_FP32, None,
                                  ctypes.c_void_p(0x300004), L.POEM_DENSE_WORKSPACE_BYTES, None) == L.POEM_ERR_WORKSPACE


def test_error_is_thread_local(lib):
    import threading
    cp = prob(head_dim=96).c()
    assert lib.poem_num_tiles(ctypes.byref(cp)) == L.POEM_ERR_UNSUPPORTED
    seen = {}

    def other():
        seen["msg"] = lib.poem_last_error().decode()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert "head_dim" in lib.poem_last_error().decode()


def test_noalloc_validation(lib):
    """poem_sparse_prefill_noalloc rejects, before any HIP call, what poem_sparse_prefill
    rejects and more CSR rows than its scratch holds."""
    src = open(os.path.join(ROOT, "include", "poem.h")).read()
    max_rows = int(re.search(r"#define\s+POEM_NOALLOC_MAX_ROWS\s+(\d+)", src).group(1))
    f = lib.poem_sparse_prefill_noalloc
    cp = prob().c()
    assert f(ctypes.byref(cp), None, FAKE, FAKE, FAKE, FAKE, FAKE, L.POEM_FP32, None, None) == L.POEM_ERR_INVALID_ARG
    assert f(ctypes.byref(cp), FAKE, FAKE, FAKE, None, FAKE, FAKE, L.POEM_FP32, None, None) == L.POEM_ERR_INVALID_ARG
    assert f(ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, FAKE, None, L.POEM_FP32, None, None) == L.POEM_ERR_INVALID_ARG
    assert f(ctypes.byref(cp), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 9, None, None) == L.POEM_ERR_INVALID_ARG
    bad = prob(head_dim=96).c()
    assert f(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, L.POEM_FP32, None, None) == L.POEM_ERR_UNSUPPORTED
    # 128 heads x 64 sequences x 129 tiles of 64 rows = 1056768 rows > POEM_NOALLOC_MAX_ROWS
    n = 64 * 129
    big = prob(seqlens_q=[n] * 64, seqlens_k=[n] * 64, num_heads_q=128, num_heads_kv=8)
    assert L.num_tiles(big) * 128 > max_rows
    assert f(ctypes.byref(big.c()), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, L.POEM_FP32, None, None) == \
        L.POEM_ERR_UNSUPPORTED
    assert "POEM_NOALLOC_MAX_ROWS" in lib.poem_last_error().decode()
