"""The seeded generators are deterministic and have the stated shapes and
distributions."""
import numpy as np

import synthetic


def test_determinism_and_shapes():
    a = synthetic.weights(2, 16, 256)
    b = synthetic.weights(2, 16, 256)
    assert a.dtype == np.float32 and a.shape == (16, 256) and np.array_equal(a, b)
    assert not np.array_equal(a, synthetic.weights(2, 16, 256, rep=1))
    x = synthetic.activations(2, 3, 128)
    assert x.dtype == np.uint16 and x.shape == (3, 128)


def test_distributions():
    w = synthetic.weights(2, 256, 1024)
    assert abs(w.std() - 0.02) < 5e-4 and abs(w.mean()) < 5e-4
    x = synthetic.activations(3, 64, 2048, outliers=0.01).view(np.int16)
    xf = (x.astype(np.int32) << 16).view(np.float32)
    frac = (np.abs(xf) > 8).mean()          # N(0,1) almost never exceeds 8; x20 outliers often do
    assert 0.005 < frac < 0.011


def test_router_skew():
    ids, _ = synthetic.router_topk(4, 1024, 256, 8, rep=0)
    counts = np.bincount(ids.ravel(), minlength=256)
    assert counts.max() > 0.9 * 1024                 # the most popular expert gets most tokens
    assert (counts > 0).sum() < 200


def test_random_std_format():
    c, s, z = synthetic.random_std_format("uint4_zp", 2, 32, 256)
    assert c.shape == (2, 32, 128) and s.shape == (2, 32, 2) and z.shape == (2, 32, 2)
    c, s, z = synthetic.random_std_format("mxfp4", 1, 16, 128)
    assert s.shape == (1, 16, 4) and z is None
