"""The numpy statement of the tiled int4-g64 layout (tests/tiled_layout.py)
checked on the CPU against properties its definition fixes: every code lands
in one slot and reads back, padding is zero, the nibble order unpacks into
natural k pairs, and each 8-code slice a lane feeds one matrix-core step lies
inside one 64-k scale group."""
import numpy as np

from tiled_layout import codes_of, tile_codes, tile_scales, tiled_sizes, untile_codes


def test_codes_round_trip_with_zero_padding():
    """Every code of Wq lands in exactly one slot and reads back unchanged;
    every slot past row N - 1 or k = K - 1 holds zero bits."""
    rng = np.random.default_rng(3)
    for N, K in [(1, 64), (16, 128), (17, 192), (33, 640), (40, 256)]:
        Wq = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
        Wt = tile_codes(Wq, N, K)
        assert Wt.size == tiled_sizes(N, K)[0]
        back, w, pad_dword, pad_bit = untile_codes(Wt, N, K)
        assert np.array_equal(back, codes_of(Wq))
        assert np.all(((w[pad_dword] >> pad_bit.astype(np.uint32)) & 0xF) == 0)


def test_nibble_order_gives_natural_pairs():
    """((w >> 4 i) & 0x000F000F) of a tiled dword holds the codes of k0 + 2 i
    (low half) and k0 + 2 i + 1 (high half)."""
    N, K = 16, 128
    Wq = np.zeros((N, K // 2), dtype=np.uint8)
    codes = (np.arange(K) % 16).astype(np.uint8)   # code of k is k mod 16 in row 0
    Wq[0] = codes[0::2] | (codes[1::2] << 4)
    w = tile_codes(Wq, N, K).view(np.uint32)
    for lane in (0, 16, 32, 48):
        for t in range(4):
            k0 = 32 * t + 8 * (lane // 16)
            d = int(w[lane * 4 + t])
            for i in range(4):
                v = (d >> (4 * i)) & 0x000F000F
                assert v & 0xF == (k0 + 2 * i) % 16
                assert v >> 16 == (k0 + 2 * i + 1) % 16


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
