"""The matrix-core tiled int4-g64 layout, written out from its definition in
include/lin.h (lin_q4g64_tile) as a byte permutation in numpy.  Test code: it
moves bytes and computes no part of the product."""
import numpy as np


def tiled_sizes(N, K):
    n16, kb = -(-N // 16), -(-K // 128)
    return n16 * kb * 1024, n16 * kb * 64


def tile_codes(Wq, N, K):
    """Wt as uint8 [ceil(N/16) * ceil(K/128) * 1024] from plain Wq uint8 [N, K/2]."""
    n16, kb = -(-N // 16), -(-K // 128)
    # plain rows padded to 16 T rows and 64 * kb bytes with zeros
    P = np.zeros((n16 * 16, kb * 64), dtype=np.uint8)
    P[:N, :K // 2] = Wq
    out = np.zeros((n16, kb, 64, 4, 4), dtype=np.uint8)   # unit (T, j), lane l, dword t, byte b
    for l in range(64):
        rows = np.arange(n16) * 16 + (l % 16)
        for t in range(4):
            for b in range(4):
                cols = 64 * np.arange(kb) + 16 * t + 4 * (l // 16) + b
                out[:, :, l, t, b] = P[rows][:, cols]
    return out.reshape(-1)


def tile_scales(S_bits, N, K):
    """St as uint16 [ceil(K/128) * ceil(N/16) * 32] from plain S bits uint16 [N, K/64]."""
    n16, kb = -(-N // 16), -(-K // 128)
    G = K // 64
    P = np.zeros((n16 * 16, 2 * kb), dtype=np.uint16)
    P[:N, :G] = S_bits
    out = np.zeros((kb, n16, 16, 2), dtype=np.uint16)      # unit (j, T), row r, group h
    for h in range(2):
        out[:, :, :, h] = P[:, 2 * np.arange(kb) + h].T.reshape(kb, n16, 16)
    return out.reshape(-1)
