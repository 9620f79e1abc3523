"""The numpy statement of the tiled int4-g64 layout (tests/tiled_layout.py)
checked on the CPU against properties its definition fixes: every plain byte
appears exactly once, padding is zero, and each 8-code slice a lane feeds one
matrix-core step lies inside one 64-k scale group."""
import numpy as np

from tiled_layout import tile_codes, tile_scales, tiled_sizes


def _unique_plain(N, K, seed):
    # bytes that identify their own position: a permutation check by value
    rng = np.random.default_rng(seed)
    idx = rng.permutation(N * (K // 2)).reshape(N, K // 2)
    return idx


def test_codes_are_a_permutation_with_zero_padding():
    for N, K in [(1, 64), (16, 128), (17, 192), (33, 640), (40, 256)]:
        ids = _unique_plain(N, K, N + K)
        # move positions instead of bytes: tile three byte-planes of the index
        planes = [((ids >> (8 * p)) & 0xFF).astype(np.uint8) for p in range(3)]
        tiled = [tile_codes(pl, N, K).astype(np.int64) for pl in planes]
        pos = tiled[0] | (tiled[1] << 8) | (tiled[2] << 16)
        wt, _ = tiled_sizes(N, K)
        assert pos.size == wt
        # every valid byte appears once; padding bytes (position 0 aside) read 0
        valid = np.zeros(wt, dtype=bool)
        n16, kb = -(-N // 16), -(-K // 128)
        T, j, l, t, b = np.unravel_index(np.arange(wt), (n16, kb, 64, 4, 4))
        row = 16 * T + l % 16
        col = 64 * j + 16 * t + 4 * (l // 16) + b
        valid = (row < N) & (col < K // 2)
        assert np.array_equal(np.sort(pos[valid]), np.arange(N * (K // 2)))
        assert np.all(pos[~valid] == 0)
        assert np.array_equal(pos[valid], ids[row[valid], col[valid]])


def test_each_matrix_core_step_stays_in_one_group():
    # k of lane l, dword t, code e of unit column j: 128 j + 32 t + 8 (l // 16) + e
    for j in range(3):
        for t in range(4):
            ks = [128 * j + 32 * t + 8 * (l // 16) + e for l in range(64) for e in range(8)]
            assert len({k // 64 for k in ks}) == 1
            assert sorted(set(ks)) == list(range(128 * j + 32 * t, 128 * j + 32 * t + 32))


def test_scales_units():
    N, K = 37, 448   # G = 7 (odd), 4 blocks of 128
    rng = np.random.default_rng(5)
    S = rng.integers(1, 0x7BFF, (N, K // 64)).astype(np.uint16)
    st = tile_scales(S, N, K)
    _, sb = tiled_sizes(N, K)
    assert st.size * 2 == sb
    n16, kb = -(-N // 16), -(-K // 128)
    for j in range(kb):
        for T in range(n16):
            unit = st[(j * n16 + T) * 32:(j * n16 + T + 1) * 32]
            for r in range(16):
                for h in range(2):
                    n, g = 16 * T + r, 2 * j + h
                    expect = S[n, g] if n < N and g < K // 64 else 0
                    assert unit[2 * r + h] == expect
