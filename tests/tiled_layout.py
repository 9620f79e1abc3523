"""The matrix-core tiled int4-g64 layout, written out from its definition in
include/lin.h (lin_q4g64_tile) in numpy.  Test code: it moves codes and
computes no part of the product."""
import numpy as np


def tiled_sizes(N, K):
    n16, kb = -(-N // 16), -(-K // 128)
    return n16 * kb * 1024, n16 * kb * 64


def _positions(N, K):
    """For every code slot of Wt, as arrays over (T, j, lane, dword t, pair i,
    half h): the plain row n, the k, and the bit position inside the dword."""
    n16, kb = -(-N // 16), -(-K // 128)
    T, j, l, t, i, h = np.meshgrid(np.arange(n16), np.arange(kb), np.arange(64), np.arange(4),
                                   np.arange(4), np.arange(2), indexing="ij")
    n = 16 * T + l % 16
    k = 128 * j + 32 * t + 8 * (l // 16) + 2 * i + h
    bit = 4 * i + 16 * h
    dword = ((T * kb + j) * 64 + l) * 4 + t
    return n, k, bit, dword


def codes_of(Wq):
    """4-bit codes [N, K] of a plain Wq [N, K/2] (low nibble = even k)."""
    return np.stack([Wq & 0xF, Wq >> 4], axis=-1).reshape(Wq.shape[0], -1).astype(np.uint32)


def tile_codes(Wq, N, K):
    """Wt as uint8 [ceil(N/16) * ceil(K/128) * 1024] from plain Wq uint8 [N, K/2]."""
    wt, _ = tiled_sizes(N, K)
    c = codes_of(Wq)
    n, k, bit, dword = _positions(N, K)
    valid = (n < N) & (k < K)
    out = np.zeros(wt // 4, dtype=np.uint32)
    np.bitwise_or.at(out, dword[valid], c[n[valid], k[valid]] << bit[valid].astype(np.uint32))
    return out.view(np.uint8)


def untile_codes(Wt, N, K):
    """Inverse of tile_codes: codes [N, K] read back from Wt."""
    n, k, bit, dword = _positions(N, K)
    valid = (n < N) & (k < K)
    w = np.asarray(Wt).view(np.uint32)
    out = np.full((N, K), 99, dtype=np.int64)
    out[n[valid], k[valid]] = (w[dword[valid]] >> bit[valid].astype(np.uint32)) & 0xF
    return out, w, dword[~valid], bit[~valid]


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
