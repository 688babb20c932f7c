"""A hand-worked 4x4 example of the block, derived from the definition on paper.

The pages print no worked example of the spectral layer, so this one is derived by hand:

grid 4x4, modes (1, 2) per corner, one channel, batch 1.
x[p0, p1] = cos(pi p1 / 2): every row is [1, 0, -1, 0].
Its only retained non-zero coefficient is k = (0, 1):
    X_(0,1) = sum_p x e^{-i pi p1/2} = 4 * (1*1 + (-1)*(-1)) = 8.
With W[corner 0, 0, 0, 0, 1] = 2 + 1i, yhat_(0,1) = 16 + 8i and
    y_spec = (1/16) * 2 * Re((16 + 8i) e^{i pi p1/2}) = 2 cos(pi p1/2) - sin(pi p1/2)
           = [2, -1, -2, 1] on every row.
With Wb = [[0.5]] and bias 0.25: z = y_spec + 0.5 x + 0.25 = [2.75, -0.75, -2.25, 1.25].
"""
import math

import numpy as np

import oracle.fno_oracle as O


def test_hand_worked_4x4():
    grid, modes = (4, 4), (1, 2)
    p1 = np.arange(4)
    x = np.tile(np.cos(np.pi * p1 / 2.0), (4, 1)).reshape(1, 1, 4, 4)
    w = np.zeros((2, 1, 1, 1, 2), dtype=np.complex128)
    w[0, 0, 0, 0, 1] = 2 + 1j
    w[0, 0, 0, 0, 0] = 5.0          # multiplies X_(0,0) = 0
    w[1, 0, 0, 0, :] = [7.0, -3j]   # multiplies X_(-1, .) = 0
    out = O.block_fwd(x, w, np.array([[0.5]]), np.array([0.25]), modes)
    assert abs(out["xhat"][0, 0, 0, 1] - 8.0) < 1e-12
    assert np.max(np.abs(np.delete(out["xhat"].ravel(), 1))) < 1e-12
    np.testing.assert_allclose(out["y_spec"][0, 0], np.tile([2.0, -1.0, -2.0, 1.0], (4, 1)),
                               atol=1e-12)
    z = np.array([2.75, -0.75, -2.25, 1.25])
    np.testing.assert_allclose(out["z"][0, 0], np.tile(z, (4, 1)), atol=1e-12)
    want = [0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in z]
    np.testing.assert_allclose(out["y"][0, 0], np.tile(want, (4, 1)), atol=1e-12)
