"""poem_sparse_prefill_noalloc (no workspace, library-owned scratch) against
poem_sparse_prefill with a caller workspace, through the C ABI: bit-identical
outputs and LSE on two calls in a row, the second on a smaller problem (the scratch
keeps the first call's contents, which the second must not depend on)."""
import sys

import numpy as np
import pytest

from block_sparse_attention_poem_amd import _lib as L
from block_sparse_attention_poem_amd import synth

from . import helpers as H

pytestmark = pytest.mark.gpu


def _case(n_q, n_k, hq, hkv, d, B, dtype, seed):
    import torch
    w = synth.small_workload(n_q=n_q, n_k=n_k, hq=hq, hkv=hkv, d=d, block=B, dtype=dtype, seed=seed)
    inp = synth.make(w)
    gp, op = H.problems(w)
    qd, kd, vd = H.device_inputs(inp)
    rng = np.random.default_rng(seed)
    from oracle import poem_oracle as O  # geometry of the random CSR only
    rows = []
    for h in range(hq):
        for t in O.tiles(op):
            rows.append([b for b in range(t.diag + 1) if rng.uniform() < 0.5 or b in (0, t.diag)])
    rp = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    bi = np.array([b for r in rows for b in r] + [0], np.int32)
    return gp, qd, kd, vd, torch.from_numpy(rp).cuda(), torch.from_numpy(bi).cuda()


def test_noalloc_matches_workspace_entry_point():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()
    # second call smaller than the first: fewer heads and tiles, another dtype
    for case in [(1000, 1128, 8, 2, 128, 128, "bf16", 3), (300, 428, 4, 2, 64, 64, "bf16", 4),
                 (129, 385, 2, 1, 128, 128, "fp32", 5)]:
        print("noalloc", case, flush=True)
        sys.stdout.flush()
        gp, q, k, v, rp, bi = _case(*case)
        for od in ("fp32", "bf16"):
            ref_o, ref_l = L.sparse_prefill(gp, q, k, v, rp, bi, out_dtype=od)
            out, lse = L._alloc_out(gp, od, True, q.device)
            out.fill_(7.0)
            lse.fill_(7.0)
            L.sparse_prefill_noalloc(gp, q, k, v, rp, bi, out, lse, out_dtype=od)
            torch.cuda.synchronize()
            bits = (lambda x: x.view(torch.int16)) if od == "bf16" else (lambda x: x.view(torch.int32))
            assert torch.equal(bits(out), bits(ref_o)), (case, od)
            assert torch.equal(lse, ref_l), (case, od)
