"""The seeded input generator: shapes, determinism, per-head independence, planted outliers."""
import numpy as np

import workloads as W


def test_shapes_and_lengths():
    assert W.WORKLOADS["tiny"].L == 256
    assert W.WORKLOADS["480p"].L == 32760
    assert W.WORKLOADS["smalld"].L == 17776
    assert W.WORKLOADS["720p"].L == 75600
    assert W.WORKLOADS["480p"].Dp == 192 and W.WORKLOADS["720p"].Dp == 128
    for w in W.WORKLOADS.values():
        assert sum(w.split) == w.D


def test_deterministic_per_head():
    w = W.WORKLOADS["tiny"]
    a = W.head_inputs(w, 0, 1)
    b = W.head_inputs(w, 0, 1)
    full = W.full_inputs(w, threads=2)
    for t in "qkv":
        assert a[t].dtype == np.float16 and a[t].shape == (256, 128)
        assert np.array_equal(a[t], b[t])
        assert np.array_equal(full[t][0, 1], a[t])
    assert not np.array_equal(full["q"][0, 0], full["q"][0, 1])


def test_outlier_channels_shared_by_q_and_k():
    w = W.WORKLOADS["tiny"]
    x = W.head_inputs(w, 0, 0)
    amax = {t: np.abs(x[t].astype(np.float32)).max(axis=0) for t in "qkv"}
    big = {t: set(np.nonzero(amax[t] > 15)[0].tolist()) for t in "qkv"}
    assert len(big["q"]) == 12 and big["q"] == big["k"]
    assert len(big["v"]) == 12
    for lo, hi in ((0, 44), (44, 86), (86, 128)):
        assert sum(lo <= c < hi for c in big["q"]) == 4


def test_head_mask():
    m = W.head_fallback_mask(W.WORKLOADS["mixed"])
    assert m.dtype == np.uint8 and m.shape == (12,) and m.sum() == 3
    assert W.head_fallback_mask(W.WORKLOADS["720p"]) is None
