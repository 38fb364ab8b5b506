"""The oracle's packer against hand-built words and its own inverse."""
import numpy as np
import pytest

import oracle


def _block_words(codes64, bits, n=1):
    c = np.zeros((n, 64), dtype=np.uint8)
    c[0] = codes64
    return oracle.pack_codes(c, bits)[: 2 * bits]


def test_int4_word_by_hand():
    codes = np.zeros(64, np.uint8)
    codes[:8] = [1, 2, 3, 4, 5, 6, 7, 8]
    w = _block_words(codes, 4)
    # even codes 1,3,5,7 in the low half (LSB first), odd 2,4,6,8 in the high half
    assert w[0] == 0x86427531
    assert np.all(w[1:] == 0)
    codes[56:64] = 15
    assert _block_words(codes, 4)[7] == 0xFFFFFFFF


def test_int2_word_by_hand():
    codes = np.zeros(64, np.uint8)
    codes[:16] = [1, 2, 3, 0, 1, 2, 3, 0, 3, 3, 3, 3, 0, 0, 0, 1]
    w = _block_words(codes, 2)
    even = [1, 3, 1, 3, 3, 3, 0, 0]
    odd = [2, 0, 2, 0, 3, 3, 0, 1]
    lo = sum(v << (2 * i) for i, v in enumerate(even))
    hi = sum(v << (2 * i) for i, v in enumerate(odd))
    assert w[0] == (hi << 16) | lo
    assert np.all(w[1:] == 0)


def test_int8_word_by_hand():
    codes = np.zeros(64, np.uint8)
    codes[4:8] = [0x11, 0x22, 0x33, 0x44]
    w = _block_words(codes, 8)
    assert w[1] == 0x44223311
    assert w[0] == 0 and np.all(w[2:] == 0)


def test_int3_words_by_hand():
    # code 0 = 7: low bits 0b11 at bits 0-1 of word 0, bit 2 at bit 2 of word 2
    codes = np.zeros(64, np.uint8)
    codes[0] = 7
    w = _block_words(codes, 3)
    assert list(w) == [0b11, 0, 1 << 2, 0, 0, 0]
    # code 9 (odd, pair 4): low bits at 16 + 2*4 = 24 of word 0; high bit at 2*0+3+16 = 19
    codes[:] = 0
    codes[9] = 4
    assert list(_block_words(codes, 3)) == [0, 0, 1 << 19, 0, 0, 0]
    # code 16 (second low word, pair 0 even): high bit at (2 + 8) = 10 of word 2
    codes[:] = 0
    codes[16] = 6
    assert list(_block_words(codes, 3)) == [0, 0b10, 1 << 10, 0, 0, 0]
    # code 31 (second low word, pair 7 odd): (2*3+3+16 + 8) % 32 = 1
    codes[:] = 0
    codes[31] = 5
    assert list(_block_words(codes, 3)) == [0, 1 << 30, 1 << 1, 0, 0, 0]
    # second run uses words 3..5
    codes[:] = 0
    codes[32] = 7
    assert list(_block_words(codes, 3)) == [0, 0, 0, 0b11, 0, 1 << 2]


def test_int3_high_word_positions_are_a_bijection():
    for run in range(2):
        pos = []
        for c, entries in enumerate(oracle.code_bit_map(3)):
            if c // 32 != run:
                continue
            for code_bit, w, p in entries:
                if code_bit == 2:
                    assert w == 3 * run + 2
                    pos.append(p)
        assert sorted(pos) == list(range(32))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
def test_every_bit_used_once(bits):
    seen = set()
    for entries in oracle.code_bit_map(bits):
        assert sorted(e[0] for e in entries) == list(range(bits))
        for _, w, p in entries:
            assert 0 <= w < 2 * bits and 0 <= p < 32
            assert (w, p) not in seen
            seen.add((w, p))
    assert len(seen) == 64 * bits


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n", [1, 63, 64, 65, 200])
def test_round_trip(bits, n):
    rng = np.random.default_rng(n * 7 + bits)
    k = 192
    codes = rng.integers(0, 1 << bits, size=(n, k)).astype(np.uint8)
    words = oracle.pack_codes(codes, bits)
    assert words.dtype == np.uint32
    assert words.size == oracle.packed_words(n, k, bits)
    assert np.array_equal(oracle.unpack_codes(words, n, k, bits), codes)


def test_tile_positions():
    n, k, bits = 130, 128, 4
    codes = np.zeros((n, k), np.uint8)
    codes[129, 64] = 9           # tile 2, row 1, block 1, code 0
    words = oracle.pack_codes(codes, bits)
    kb, wpb = k // 64, 2 * bits
    off = ((129 // 64) * kb + 1) * 64 * wpb + (129 % 64) * wpb
    assert words[off] == 9
    assert np.count_nonzero(words) == 1


def test_meta_tiling():
    n, g = 70, 3
    t = np.arange(n * g, dtype=np.uint16).reshape(n, g)
    flat = oracle.tile_meta(t)
    assert flat.size == 2 * 64 * g
    assert flat[(1 * g + 2) * 64 + 5] == t[69, 2]
    assert flat[(0 * g + 1) * 64 + 10] == t[10, 1]
    assert np.array_equal(oracle.untile_meta(flat, n, g), t)
    assert np.all(flat[(1 * g + 0) * 64 + 6:(1 * g + 1) * 64] == 0)


def test_split_plane_words_by_hand():
    """5-7 bits: bits 0..3 in words 0..7 as for 4 bits, the rest in words
    8.. as a 1-, 2- or 3-bit code."""
    codes = np.zeros(64, np.uint8)
    codes[:4] = [0x1F, 0x10, 0x0F, 0x11]
    w = _block_words(codes, 5)
    # low nibbles F, 0, F, 1 -> word 0: even codes (F, F) low half, odd (0, 1) high half
    assert w[0] == (0x10 << 16) | 0xFF
    assert np.all(w[1:8] == 0)
    # bit 4 of codes 0, 1, 3 (1-bit arrangement: even codes low half, odd high)
    assert w[8] == (1 << 0) | (1 << 16) | (1 << 17)
    assert w[9] == 0
    codes = np.zeros(64, np.uint8)
    codes[63] = 0x3F
    w = _block_words(codes, 6)
    assert w[7] == 0xF << 28                  # code 63: odd, i = 7 of word 7
    assert w[11] == 0x3 << 30                 # 2-bit word 3, i = 15: 16 + 2*7
    codes = np.zeros(64, np.uint8)
    codes[0] = 0x70                           # high bits 0b111 of code 0, 7 bits
    w = _block_words(codes, 7)
    assert np.all(w[:8] == 0)
    # 3-bit arrangement of run 0, code 0: low two bits at 0, 1 of word 8, bit 2
    # at position 2 of word 10
    assert w[8] == 0x3 and w[9] == 0 and w[10] == 1 << 2
    assert np.all(w[11:] == 0)


@pytest.mark.parametrize("bits", [5, 6, 7])
def test_split_plane_is_two_plain_layouts(bits):
    """The 5-7 bit block equals the 4-bit packing of the low nibbles followed
    by the (bits-4)-bit packing of the high bits (for 2 and 3 high bits)."""
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(130, 256)).astype(np.uint8)
    words = oracle.pack_codes(codes, bits).reshape(-1, 2 * bits)
    lo = oracle.pack_codes(codes & 15, 4).reshape(-1, 8)
    assert np.array_equal(words[:, :8], lo)
    if bits > 5:
        hi = oracle.pack_codes(codes >> 4, bits - 4).reshape(-1, 2 * (bits - 4))
        assert np.array_equal(words[:, 8:], hi)
