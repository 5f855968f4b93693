"""ctypes binding of libpoem (argument marshalling only).

Every step of the hot path runs in the HIP library; this module only checks that
tensors match the declared problem, allocates outputs with torch (device memory
and the current stream are all torch provides), and forwards raw pointers. It
raises if the library is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# POEM_LIB selects another build of the same library (the host AddressSanitizer build)
LIB_PATH = os.environ.get("POEM_LIB") or os.path.join(_HERE, "libpoem.so")

POEM_OK, POEM_ERR_INVALID_ARG, POEM_ERR_UNSUPPORTED, POEM_ERR_WORKSPACE, POEM_ERR_CAPACITY, POEM_ERR_HIP = \
    0, -1, -2, -3, -4, -5
POEM_BF16, POEM_FP32 = 0, 1
POEM_DENSE_WORKSPACE_BYTES = 256  # include/poem.h
STATUS_NAMES = {0: "POEM_OK", -1: "POEM_ERR_INVALID_ARG", -2: "POEM_ERR_UNSUPPORTED", -3: "POEM_ERR_WORKSPACE",
                -4: "POEM_ERR_CAPACITY", -5: "POEM_ERR_HIP"}
SYMBOLS = ["poem_num_tiles", "poem_csr_capacity", "poem_max_visible_blocks", "poem_select_workspace_bytes",
           "poem_sparse_workspace_bytes", "poem_select", "poem_select_mass", "poem_select_group", "poem_select_practical",
           "poem_sparse_prefill", "poem_sparse_prefill_group", "poem_sparse_prefill_noalloc", "poem_dense_prefill",
           "poem_last_error", "poem_version"]


class PoemError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class CProblem(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32),
                ("seqlens_q_host", ctypes.POINTER(ctypes.c_int32)),
                ("seqlens_k_host", ctypes.POINTER(ctypes.c_int32)),
                ("num_heads_q", ctypes.c_int32),
                ("num_heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float),
                ("in_dtype", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpoem.so (built in-tree by block_sparse_attention_poem_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libpoem is not built ({path} missing): run python -m block_sparse_attention_poem_amd.build")
    # torch ships its own HIP runtime with the same soname as ROCm's. Importing torch
    # first makes libpoem bind to that runtime, so the process has one HIP runtime and
    # torch's stream handles are valid inside the library. Loaded the other way round,
    # two runtimes coexist and launches from the library find no device.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(CProblem)
    vp, i32, i64, f32p = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_float)
    for name in ("poem_num_tiles", "poem_csr_capacity", "poem_max_visible_blocks", "poem_sparse_workspace_bytes"):
        getattr(lib, name).argtypes = [P]
        getattr(lib, name).restype = i64
    lib.poem_select_workspace_bytes.argtypes = [P, i32]
    lib.poem_select_workspace_bytes.restype = i64
    lib.poem_select.argtypes = [P, vp, vp, vp, f32p, i32, i32, i32, vp, vp, i64, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.poem_select.restype = ctypes.c_int
    lib.poem_select_mass.argtypes = lib.poem_select.argtypes
    lib.poem_select_mass.restype = ctypes.c_int
    lib.poem_select_group.argtypes = lib.poem_select.argtypes
    lib.poem_select_group.restype = ctypes.c_int
    lib.poem_select_practical.argtypes = [P, vp, vp, vp, f32p, i32, i32, i32, ctypes.c_float, ctypes.c_float, vp,
                                          vp, i64, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.poem_select_practical.restype = ctypes.c_int
    lib.poem_sparse_prefill.argtypes = [P, vp, vp, vp, vp, vp, vp, i32, vp, vp, ctypes.c_size_t, vp]
    lib.poem_sparse_prefill.restype = ctypes.c_int
    lib.poem_sparse_prefill_group.argtypes = lib.poem_sparse_prefill.argtypes
    lib.poem_sparse_prefill_group.restype = ctypes.c_int
    lib.poem_sparse_prefill_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, i32, vp, vp]
    lib.poem_sparse_prefill_noalloc.restype = ctypes.c_int
    lib.poem_dense_prefill.argtypes = [P, vp, vp, vp, vp, i32, vp, vp, ctypes.c_size_t, vp]
    lib.poem_dense_prefill.restype = ctypes.c_int
    lib.poem_last_error.restype = ctypes.c_char_p
    lib.poem_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


@dataclass
class Problem:
    """One prefill call: packed THD tensors, queries at positions N_k - N_q .. N_k - 1."""

    seqlens_q: Sequence[int]
    seqlens_k: Sequence[int]
    num_heads_q: int
    num_heads_kv: int
    head_dim: int
    block_size: int
    softmax_scale: float = 0.0
    dtype: str = "bf16"  # "bf16" or "fp32"

    def c(self):
        n = len(self.seqlens_q)
        sq = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in self.seqlens_q])
        sk = (ctypes.c_int32 * max(n, 1))(*[int(x) for x in self.seqlens_k])
        cp = CProblem(n, ctypes.cast(sq, ctypes.POINTER(ctypes.c_int32)), ctypes.cast(sk, ctypes.POINTER(ctypes.c_int32)),
                      self.num_heads_q, self.num_heads_kv, self.head_dim, self.block_size, float(self.softmax_scale),
                      POEM_BF16 if self.dtype == "bf16" else POEM_FP32)
        cp._keep = (sq, sk)  # keep host arrays alive for the call
        return cp

    @property
    def total_q(self):
        return int(sum(self.seqlens_q))

    @property
    def total_k(self):
        return int(sum(self.seqlens_k))


def _check(status: int):
    if status != POEM_OK:
        raise PoemError(status, load().poem_last_error().decode())


def _i64(v: int) -> int:
    if v < 0:
        raise PoemError(int(v), load().poem_last_error().decode())
    return int(v)


def num_tiles(problem: Problem) -> int:
    return _i64(load().poem_num_tiles(ctypes.byref(problem.c())))


def csr_capacity(problem: Problem) -> int:
    return _i64(load().poem_csr_capacity(ctypes.byref(problem.c())))


def max_visible_blocks(problem: Problem) -> int:
    return _i64(load().poem_max_visible_blocks(ctypes.byref(problem.c())))


def sparse_workspace_bytes(problem: Problem) -> int:
    return _i64(load().poem_sparse_workspace_bytes(ctypes.byref(problem.c())))


def select_workspace_bytes(problem: Problem, rows_per_tile: int) -> int:
    return _i64(load().poem_select_workspace_bytes(ctypes.byref(problem.c()), int(rows_per_tile)))


def version() -> str:
    return load().poem_version().decode()


# ---------------------------------------------------------------------------
# torch-facing calls
# ---------------------------------------------------------------------------


def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _keep_for_stream(stream, *tensors):
    """Buffers allocated here on torch's current stream but used by a launch on another
    stream: record that stream, so the caching allocator does not hand their memory to
    a new allocation before that stream's work on them is done."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _check_qkv(problem: Problem, q, k, v):
    torch = _torch()
    want = torch.bfloat16 if problem.dtype == "bf16" else torch.float32
    for name, t, rows, heads in (("q", q, problem.total_q, problem.num_heads_q),
                                 ("k", k, problem.total_k, problem.num_heads_kv),
                                 ("v", v, problem.total_k, problem.num_heads_kv)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dtype != want:
            raise ValueError(f"{name} has dtype {t.dtype}, problem says {want}")
        if tuple(t.shape) != (rows, heads, problem.head_dim):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(rows, heads, problem.head_dim)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


class Workspace:
    """A reusable 256-byte-aligned device workspace of nbytes bytes."""

    def __init__(self, nbytes: int, device="cuda"):
        torch = _torch()
        self.nbytes = int(nbytes)
        self.buf = torch.empty(max(self.nbytes, 256) + 256, dtype=torch.uint8, device=device)
        base = self.buf.data_ptr()
        self.ptr = (base + 255) & ~255


class SelectWorkspace(Workspace):
    """Workspace for select() (poem_select_workspace_bytes)."""

    def __init__(self, problem: Problem, rows_per_tile: int, device="cuda"):
        super().__init__(select_workspace_bytes(problem, rows_per_tile), device)


class SparseWorkspace(Workspace):
    """Workspace for sparse_prefill()'s row schedule (poem_sparse_workspace_bytes)."""

    def __init__(self, problem: Problem, device="cuda"):
        super().__init__(sparse_workspace_bytes(problem), device)


class DenseWorkspace(Workspace):
    """Workspace for dense_prefill()'s tile queue (POEM_DENSE_WORKSPACE_BYTES)."""

    def __init__(self, device="cuda"):
        super().__init__(POEM_DENSE_WORKSPACE_BYTES, device)


def select(problem: Problem, q, k, v, tau, n_sink_blocks: int = 1, n_local_blocks: int = 1,
           rows_per_tile: int = 8, diagnostics: bool = False, workspace: Optional[SelectWorkspace] = None,
           stream=None, mode: str = "poem", weight: float = 0.5, presel_fraction: float = 0.95):
    """Run poem_select (mode "poem", tau: error threshold per head), poem_select_mass
    (mode "mass", tau: omitted-mass budget per head) or poem_select_group (mode "group":
    one list per KV head and tile; rows_per_tile counts the group's sampled rows) or
    poem_select_practical (mode "practical", tau: pooled omitted-mass budget per head,
    with weight and presel_fraction).
    Returns dict(row_ptr, block_idx[, tile_scores, tile_mass, row_bound])."""
    torch = _torch()
    _check_qkv(problem, q, k, v)
    lib = load()
    cp = problem.c()
    T = num_tiles(problem)
    cap = csr_capacity(problem)
    dev = q.device
    tau_arr = (ctypes.c_float * max(problem.num_heads_q, 1))(*[float(x) for x in tau])
    row_ptr = torch.empty(problem.num_heads_q * T + 1, dtype=torch.int32, device=dev)
    block_idx = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    out = dict(row_ptr=row_ptr, block_idx=block_idx)
    sc = ms = rb = None
    if diagnostics:
        mv = max(max_visible_blocks(problem), 1)
        sc = torch.empty((problem.num_heads_q, T, mv), dtype=torch.float32, device=dev)
        ms = torch.empty_like(sc)
        rb = torch.empty((problem.num_heads_q, T, rows_per_tile), dtype=torch.float32, device=dev)
        out.update(tile_scores=sc, tile_mass=ms, row_bound=rb)
    ws = workspace if workspace is not None else SelectWorkspace(problem, rows_per_tile, dev)
    _keep_for_stream(stream, row_ptr, block_idx, sc, ms, rb, ws.buf if workspace is None else None)
    tail = (_ptr(row_ptr), _ptr(block_idx), cap, _ptr(sc), _ptr(ms), _ptr(rb), ctypes.c_void_p(ws.ptr), ws.nbytes,
            _stream_ptr(stream))
    head = (ctypes.byref(cp), _ptr(q), _ptr(k), _ptr(v), tau_arr, int(n_sink_blocks), int(n_local_blocks),
            int(rows_per_tile))
    if mode == "practical":
        _check(lib.poem_select_practical(*head, float(weight), float(presel_fraction), *tail))
    else:
        fn = {"poem": lib.poem_select, "mass": lib.poem_select_mass, "group": lib.poem_select_group}[mode]
        _check(fn(*head, *tail))
    out["_workspace"] = ws
    return out


def _alloc_out(problem: Problem, out_dtype: str, want_lse: bool, device):
    torch = _torch()
    od = torch.float32 if out_dtype == "fp32" else torch.bfloat16
    out = torch.empty((problem.total_q, problem.num_heads_q, problem.head_dim), dtype=od, device=device)
    lse = torch.empty((problem.num_heads_q, problem.total_q), dtype=torch.float32, device=device) if want_lse else None
    return out, lse


def sparse_prefill(problem: Problem, q, k, v, row_ptr, block_idx, out_dtype: str = "bf16", want_lse: bool = True,
                   out=None, lse=None, workspace="auto", stream=None):
    """Run poem_sparse_prefill. Returns (out, lse).

    workspace: a SparseWorkspace, "auto" (allocate one: persistent, count-ordered
    schedule) or None (one workgroup per row)."""
    _check_qkv(problem, q, k, v)
    if out is None:
        out, lse = _alloc_out(problem, out_dtype, want_lse, q.device)
        _keep_for_stream(stream, out, lse)
    if isinstance(workspace, str):
        workspace = SparseWorkspace(problem, q.device)
        _keep_for_stream(stream, workspace.buf)
    wp = ctypes.c_void_p(workspace.ptr) if workspace is not None else ctypes.c_void_p(0)
    wb = workspace.nbytes if workspace is not None else 0
    _check(load().poem_sparse_prefill(ctypes.byref(problem.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                      _ptr(block_idx), _ptr(out), POEM_FP32 if out_dtype == "fp32" else POEM_BF16,
                                      _ptr(lse), wp, wb, _stream_ptr(stream)))
    return out, lse


def sparse_prefill_group(problem: Problem, q, k, v, row_ptr, block_idx, out_dtype: str = "bf16",
                         want_lse: bool = True, out=None, lse=None, workspace="auto", stream=None):
    """Run poem_sparse_prefill_group (lists shared by each GQA group, read from the
    group's first head). Returns (out, lse). workspace as for sparse_prefill."""
    _check_qkv(problem, q, k, v)
    if out is None:
        out, lse = _alloc_out(problem, out_dtype, want_lse, q.device)
        _keep_for_stream(stream, out, lse)
    if isinstance(workspace, str):
        workspace = SparseWorkspace(problem, q.device)
        _keep_for_stream(stream, workspace.buf)
    wp = ctypes.c_void_p(workspace.ptr) if workspace is not None else ctypes.c_void_p(0)
    wb = workspace.nbytes if workspace is not None else 0
    _check(load().poem_sparse_prefill_group(ctypes.byref(problem.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                            _ptr(block_idx), _ptr(out),
                                            POEM_FP32 if out_dtype == "fp32" else POEM_BF16, _ptr(lse), wp, wb,
                                            _stream_ptr(stream)))
    return out, lse


def sparse_prefill_noalloc(problem: Problem, q, k, v, row_ptr, block_idx, out, lse=None, out_dtype: str = "bf16",
                           stream=None):
    """Run poem_sparse_prefill_noalloc into caller-allocated out (and lse): the library
    allocates nothing and uses its own per-device scratch. Returns (out, lse)."""
    _check_qkv(problem, q, k, v)
    _check(load().poem_sparse_prefill_noalloc(ctypes.byref(problem.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                              _ptr(block_idx), _ptr(out),
                                              POEM_FP32 if out_dtype == "fp32" else POEM_BF16, _ptr(lse),
                                              _stream_ptr(stream)))
    return out, lse


def dense_prefill(problem: Problem, q, k, v, out_dtype: str = "bf16", want_lse: bool = True, out=None, lse=None,
                  workspace="auto", stream=None):
    """Run poem_dense_prefill. Returns (out, lse).

    workspace: a DenseWorkspace, "auto" (allocate one: tiles pulled from a queue) or
    None (the fixed interleave of the same order)."""
    _check_qkv(problem, q, k, v)
    if out is None:
        out, lse = _alloc_out(problem, out_dtype, want_lse, q.device)
        _keep_for_stream(stream, out, lse)
    if isinstance(workspace, str):
        workspace = DenseWorkspace(q.device)
        _keep_for_stream(stream, workspace.buf)
    wp = ctypes.c_void_p(workspace.ptr) if workspace is not None else ctypes.c_void_p(0)
    wb = workspace.nbytes if workspace is not None else 0
    _check(load().poem_dense_prefill(ctypes.byref(problem.c()), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                     POEM_FP32 if out_dtype == "fp32" else POEM_BF16, _ptr(lse), wp, wb,
                                     _stream_ptr(stream)))
    return out, lse


def flops_dense(problem: Problem) -> float:
    """4 d H_q x (causal (query, key) pairs): the dense attention's algorithmic FLOPs."""
    pairs = 0
    for nq, nk in zip(problem.seqlens_q, problem.seqlens_k):
        start = nk - nq
        pairs += nq * (start + 1) + nq * (nq - 1) // 2
    return 4.0 * problem.head_dim * problem.num_heads_q * pairs
