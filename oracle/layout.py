"""Oracle packer/unpacker for the tiled packed-code layout.

TEST INFRASTRUCTURE ONLY (see ``oracle/reference.py``).  Written from the
textual definition of the layout in ``include/qlin.h``, bit by bit, with no
shortcut; the HIP library's packer and unpackers share nothing with it.

The layout (restated here so this file stands on its own):

* Rows are taken in tiles of 64 (the last tile padded with rows whose codes
  are 0); K is cut into blocks of 64 codes.  The 64 codes of row n, block j
  occupy ``2*bits`` consecutive 32-bit words, and the blocks are stored
  tile-major, then block, then row within the tile:
  ``word offset = ((n // 64) * (K // 64) + j) * 64 * 2*bits + (n % 64) * 2*bits``.
* bits in {2, 4, 8}: word w of a block holds codes c = w*(32/bits) + i,
  i = 0 .. 32/bits - 1.  Even i go in the low 16 bits, odd i in the high 16
  bits, each half filled from its least significant bit in order of i, bits
  bits per code:  bit position = 16*(i % 2) + bits*(i // 2).
* bits = 3: the 64 codes form two runs of 32 (run r = c // 32), each using
  three words: words 3r and 3r+1 hold the low two bits of the run's codes
  0..15 and 16..31, arranged as for bits=2; word 3r+2 holds bit 2 of each of
  the run's 32 codes.  For run code c' (0..31): u = c' // 16, i = c' % 16,
  p = i // 2, e = i % 2; the bit sits at position
  (2p + 2 if p < 4 else 2(p - 4) + 3) + 16e, plus 8 modulo 32 when u = 1.
* bits in {5, 6, 7} ("split planes"): words 0..7 hold bits 0..3 of the 64
  codes, arranged as for bits=4; words 8 .. 2*bits-1 hold bits 4 .. bits-1 of
  the 64 codes as a (bits-4)-bit code, arranged as for 1, 2 or 3 bits.  The
  1-bit arrangement follows the rule for {2, 4, 8}: word w holds codes
  c = 32w + i at bit position 16*(i % 2) + (i // 2).

Scales and zero points use the same tiling: entry (n, g) of the [N, G]
table is stored at ``((n // 64) * G + g) * 64 + (n % 64)``; padding rows hold 0.
"""
from __future__ import annotations

import numpy as np

TILE_ROWS = 64
KBLOCK = 64


PACKED_BITS = (2, 3, 4, 5, 6, 7, 8)


def words_per_block(bits: int) -> int:
    if bits not in PACKED_BITS:
        raise ValueError(f"unsupported bits {bits}")
    return 2 * bits


def _plain_bits(bits: int, c: int, word0: int, code_bit0: int):
    """Entries of code c (0..63) in the arrangement for 1, 2, 3, 4 or 8 bits,
    its words counted from word0, its bits counted from code_bit0."""
    entries = []
    if bits in (1, 2, 4, 8):
        per_word = 32 // bits
        w, i = divmod(c, per_word)
        pos = 16 * (i % 2) + bits * (i // 2)
        for b in range(bits):
            entries.append((code_bit0 + b, word0 + w, pos + b))
    else:  # bits == 3
        run, cr = divmod(c, 32)
        u, i = divmod(cr, 16)
        low_word = word0 + 3 * run + u
        pos = 16 * (i % 2) + 2 * (i // 2)
        entries.append((code_bit0, low_word, pos))
        entries.append((code_bit0 + 1, low_word, pos + 1))
        p, e = divmod(i, 2)
        hb = (2 * p + 2) if p < 4 else (2 * (p - 4) + 3)
        hb += 16 * e
        if u == 1:
            hb = (hb + 8) % 32
        entries.append((code_bit0 + 2, word0 + 3 * run + 2, hb))
    return entries


def code_bit_map(bits: int):
    """For every code index c of a 64-code block, the list of
    ``(code_bit, word, bit_position)``: bit ``code_bit`` of code c is stored at
    ``bit_position`` of block word ``word``.  Direct transcription of the
    definition in the module docstring."""
    words_per_block(bits)
    table = []
    for c in range(KBLOCK):
        if bits <= 4 or bits == 8:
            table.append(_plain_bits(bits, c, 0, 0))
        else:  # split planes: low 4 bits, then the high bits - 4
            table.append(_plain_bits(4, c, 0, 0) + _plain_bits(bits - 4, c, 8, 4))
    return table


def n_tiles(n: int) -> int:
    return (n + TILE_ROWS - 1) // TILE_ROWS


def packed_words(n: int, k: int, bits: int) -> int:
    """Number of uint32 words the packed codes of an [n, k] matrix occupy."""
    return n_tiles(n) * TILE_ROWS * (k // KBLOCK) * words_per_block(bits)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """uint8 codes [N, K] -> flat uint32 array in the tiled layout."""
    codes = np.asarray(codes)
    n, k = codes.shape
    if k % KBLOCK:
        raise ValueError("K must be a multiple of 64")
    if codes.size and int(codes.max()) >= (1 << bits):
        raise ValueError("code out of range for the bit width")
    t, kb, wpb = n_tiles(n), k // KBLOCK, words_per_block(bits)
    padded = np.zeros((t * TILE_ROWS, k), dtype=np.uint32)
    padded[:n] = codes
    # [tile, row, block, code] -> [tile, block, row, code]
    blocks = padded.reshape(t, TILE_ROWS, kb, KBLOCK).transpose(0, 2, 1, 3)
    words = np.zeros((t, kb, TILE_ROWS, wpb), dtype=np.uint32)
    for c, entries in enumerate(code_bit_map(bits)):
        for code_bit, w, pos in entries:
            bit = (blocks[..., c] >> np.uint32(code_bit)) & np.uint32(1)
            words[..., w] |= bit << np.uint32(pos)
    return words.reshape(-1)


def unpack_codes(words: np.ndarray, n: int, k: int, bits: int) -> np.ndarray:
    """Inverse of :func:`pack_codes` (padding rows dropped)."""
    t, kb, wpb = n_tiles(n), k // KBLOCK, words_per_block(bits)
    w4 = np.asarray(words, dtype=np.uint32).reshape(t, kb, TILE_ROWS, wpb)
    blocks = np.zeros((t, kb, TILE_ROWS, KBLOCK), dtype=np.uint32)
    for c, entries in enumerate(code_bit_map(bits)):
        for code_bit, w, pos in entries:
            bit = (w4[..., w] >> np.uint32(pos)) & np.uint32(1)
            blocks[..., c] |= bit << np.uint32(code_bit)
    full = blocks.transpose(0, 2, 1, 3).reshape(t * TILE_ROWS, k)
    return full[:n].astype(np.uint8)


def tile_meta(table: np.ndarray) -> np.ndarray:
    """[N, G] per-group table -> flat array in the tiled order."""
    table = np.asarray(table)
    n, g = table.shape
    t = n_tiles(n)
    padded = np.zeros((t * TILE_ROWS, g), dtype=table.dtype)
    padded[:n] = table
    return padded.reshape(t, TILE_ROWS, g).transpose(0, 2, 1).reshape(-1).copy()


def untile_meta(flat: np.ndarray, n: int, g: int) -> np.ndarray:
    t = n_tiles(n)
    a = np.asarray(flat).reshape(t, g, TILE_ROWS).transpose(0, 2, 1)
    return a.reshape(t * TILE_ROWS, g)[:n].copy()
