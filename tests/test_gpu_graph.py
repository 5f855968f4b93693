"""The hot path under HIP graph capture.

poem_select, poem_sparse_prefill and poem_dense_prefill (both with their
persistent queues) are recorded once into a torch.cuda.CUDAGraph (a HIP graph on
ROCm) and replayed. The library allocates nothing, clears nothing with memset and
never synchronises the host, so every launch records; the queues are reset by
kernels inside the graph. The kernels are deterministic (the persistent
schedule changes which workgroup runs a row, not the row's arithmetic), so each
replay must reproduce the eager results bit for bit. Eager work and host
synchronisations run between the replays, and the inputs are refreshed in place
before the last ones, which must then track the new inputs.
"""
import pytest

from block_sparse_attention_poem_amd import _lib as L
from block_sparse_attention_poem_amd import synth

from . import helpers as H

pytestmark = pytest.mark.gpu


def _run(gp, w, inp, q, k, v, ws, sws, dws, bufs):
    """The hot path into fixed buffers, on torch's current stream."""
    import ctypes
    import torch
    lib = L.load()
    cp = gp.c()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    tau = (ctypes.c_float * w.num_heads_q)(*[float(x) for x in inp.tau])
    cap = L.csr_capacity(gp)
    L._check(lib.poem_select(ctypes.byref(cp), L._ptr(q), L._ptr(k), L._ptr(v), tau, w.n_sink_blocks,
                             w.n_local_blocks, w.rows_per_tile, L._ptr(bufs["row_ptr"]),
                             L._ptr(bufs["block_idx"]), cap, None, None, None, ctypes.c_void_p(ws.ptr),
                             ws.nbytes, stream))
    L._check(lib.poem_sparse_prefill(ctypes.byref(cp), L._ptr(q), L._ptr(k), L._ptr(v), L._ptr(bufs["row_ptr"]),
                                     L._ptr(bufs["block_idx"]), L._ptr(bufs["sparse"]), L.POEM_FP32,
                                     L._ptr(bufs["sparse_lse"]), ctypes.c_void_p(sws.ptr), sws.nbytes, stream))
    L._check(lib.poem_dense_prefill(ctypes.byref(cp), L._ptr(q), L._ptr(k), L._ptr(v), L._ptr(bufs["dense"]),
                                    L.POEM_FP32, L._ptr(bufs["dense_lse"]), ctypes.c_void_p(dws.ptr), dws.nbytes,
                                    stream))


def _snapshot(bufs):
    """Everything the path writes: block_idx only up to the retained count (the rest
    of its capacity is never written)."""
    snap = {name: t.clone() for name, t in bufs.items()}
    snap["block_idx"] = snap["block_idx"][:int(snap["row_ptr"][-1])]
    return snap


def _same(a, b, what):
    for name in a:
        assert a[name].shape == b[name].shape, (what, name, tuple(a[name].shape), tuple(b[name].shape))
        assert bool((a[name] == b[name]).all()), (what, name)


def test_graph_replay_matches_eager():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    # two ragged sequences, several tiles each, GQA 4:1
    w = synth.small_workload(n_q=700, n_k=1212, hq=8, hkv=2, d=128, block=128, dtype="bf16", seqs=2,
                             sink_offset=6.0, seed=11)
    inp = synth.make(w)
    gp, _ = H.problems(w)
    q, k, v = H.device_inputs(inp)
    ws = L.SelectWorkspace(gp, w.rows_per_tile)
    sws = L.SparseWorkspace(gp)
    dws = L.DenseWorkspace()
    T = L.num_tiles(gp)
    dev = q.device
    bufs = dict(
        row_ptr=torch.zeros(w.num_heads_q * T + 1, dtype=torch.int32, device=dev),
        block_idx=torch.zeros(max(L.csr_capacity(gp), 1), dtype=torch.int32, device=dev),
        sparse=torch.zeros((gp.total_q, w.num_heads_q, w.head_dim), dtype=torch.float32, device=dev),
        sparse_lse=torch.zeros((w.num_heads_q, gp.total_q), dtype=torch.float32, device=dev),
        dense=torch.zeros((gp.total_q, w.num_heads_q, w.head_dim), dtype=torch.float32, device=dev),
        dense_lse=torch.zeros((w.num_heads_q, gp.total_q), dtype=torch.float32, device=dev),
    )
    print("graph case", w.seqlens_q, w.seqlens_k, w.num_heads_q, w.num_heads_kv, flush=True)

    # eager reference (run twice: the path is deterministic)
    _run(gp, w, inp, q, k, v, ws, sws, dws, bufs)
    torch.cuda.synchronize()
    eager = _snapshot(bufs)
    _run(gp, w, inp, q, k, v, ws, sws, dws, bufs)
    torch.cuda.synchronize()
    _same(eager, _snapshot(bufs), "eager repeat")
    nnz = int(eager["row_ptr"][-1])
    assert 0 < nnz < int(L.csr_capacity(gp)), "the case should drop some blocks and keep some"

    # capture on a side stream (torch's capture protocol), then replay on the default stream
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(gp, w, inp, q, k, v, ws, sws, dws, bufs)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    for t in bufs.values():
        t.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        _run(gp, w, inp, q, k, v, ws, sws, dws, bufs)
    torch.cuda.synchronize()

    scratch = torch.randn(1 << 20, device=dev)
    for rep in range(3):
        for t in bufs.values():  # stale results must not survive a replay
            t.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        _same(eager, _snapshot(bufs), f"replay {rep}")
        # eager work between replays
        scratch.mul_(1.0001).add_(0.5)
        float(scratch.sum())
        torch.cuda.synchronize()

    # new inputs, written in place: the replays follow them (eager run on the same data)
    inp2 = synth.make(w.with_(seed=12))
    q2, k2, v2 = H.device_inputs(inp2)
    q.copy_(q2)
    k.copy_(k2)
    v.copy_(v2)
    torch.cuda.synchronize()
    _run(gp, w, inp, q, k, v, ws, sws, dws, bufs)
    torch.cuda.synchronize()
    eager2 = _snapshot(bufs)
    assert not bool((eager2["dense"] == eager["dense"]).all()), "the refreshed inputs should change the output"
    for rep in range(2):
        for t in bufs.values():
            t.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        _same(eager2, _snapshot(bufs), f"replay on new inputs {rep}")
