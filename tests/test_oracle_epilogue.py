"""Pins for the fused-epilogue part of the CPU oracle (yalm post, GPU matmul
section: the residual add accumulated into the product's destination and the
gated product silu(w1 x) * w3 x): closed forms of silu and exact sums.  CPU only."""
import numpy as np

import oracle


def test_swiglu_closed_forms():
    """silu(g) = g * sigmoid(g): silu(0) = 0; silu(ln 3) = 0.75 ln 3 (sigmoid = 3/4);
    silu(-ln 3) = -0.25 ln 3; large |g|: silu -> g and -> 0; u scales linearly."""
    ln3 = np.log(3.0)
    G = np.array([0.0, ln3, -ln3, 40.0, -40.0, 1.0])
    U = np.array([5.0, 1.0, 2.0, 1.0, 1.0, -3.0])
    H = oracle.swiglu(G, U)
    assert H[0] == 0.0
    assert abs(H[1] - 0.75 * ln3) <= 1e-15
    assert abs(H[2] - 2.0 * (-0.25 * ln3)) <= 1e-15
    assert abs(H[3] - 40.0) <= 1e-12 and abs(H[4]) <= 1e-15
    sig1 = 1.0 / (1.0 + np.exp(-1.0))
    assert abs(H[5] - (-3.0) * sig1) <= 1e-15
    # odd/even structure: silu(g) - silu(-g) = g
    g = np.linspace(-8, 8, 33)
    assert np.allclose(oracle.swiglu(g, np.ones_like(g)) - oracle.swiglu(-g, np.ones_like(g)), g,
                       rtol=0, atol=1e-14)


def test_residual_add_exact():
    P = np.array([1.5, -2.25, 0.0, 1e10])
    R = np.array([0.5, 0.25, -3.0, 1.0], dtype=np.float32)
    assert list(oracle.residual_add(P, R)) == [2.0, -2.0, -3.0, 1e10 + 1.0]
