"""The input generator's options (CPU)."""
import numpy as np

from block_sparse_attention_poem_amd import synth


def _small(**kw):
    return synth.small_workload(n_q=256, n_k=1024, hq=2, hkv=1, d=64, block=64, dtype="fp32", seed=3, **kw)


def test_near_output_off_leaves_inputs_unchanged():
    w = _small()
    a, b = synth.make(w), synth.make(w.with_(near_output=0.0))
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)


def test_near_output_values_sit_at_the_sink_value():
    """With every cluster near the output, each key block's mean value is the sink key's
    value up to the per-key noise averaged over the block (per-coordinate rms 1/8);
    without the option the block means sit far from it. Keys and the sink are untouched."""
    w = _small()
    base, near = synth.make(w), synth.make(w.with_(near_output=1.0))
    assert np.array_equal(base.k, near.k)
    vb, vn = synth.to_f64(base.v[:, 0]), synth.to_f64(near.v[:, 0])
    assert np.array_equal(vb[0], vn[0])
    sink = vn[0]
    means_n = vn[64:].reshape(-1, 64, 64).mean(axis=1)
    means_b = vb[64:].reshape(-1, 64, 64).mean(axis=1)
    rms = lambda m: np.sqrt(((m - sink) ** 2).mean(axis=1))
    assert rms(means_n).max() < 0.3
    assert rms(means_b).min() > 0.6
