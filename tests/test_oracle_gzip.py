"""Pins of the oracle's compression stage against the gzip format itself (RFC 1952).

The pages fix only "gzip level 1 per block" and |gzip(.)| as the compressed size
("Gzip-guided Sparse Attention", flowchart and 核心公式 first display).  The format
fixes the rest: a member is a 10-byte header (magic 1f 8b, CM = 8 deflate, XFL = 4
for the fastest level), the deflate body, and an 8-byte trailer (CRC-32, ISIZE).
"""
import binascii
import gzip
import struct

import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(1234)
BLOCKS = [bytes(16), b"a" * 16, b"abcd" * 4, bytes(64), b"abcd" * 16, b"abcd" * 32,
          RNG.integers(0, 256, 16, dtype=np.uint8).tobytes(),
          RNG.integers(0, 256, 64, dtype=np.uint8).tobytes(),
          RNG.integers(0, 256, 128, dtype=np.uint8).tobytes(),
          RNG.integers(0x20, 0x7F, 64, dtype=np.uint8).tobytes()]


@pytest.mark.parametrize("blk", BLOCKS)
def test_member_is_a_level1_gzip_member(blk):
    m = oracle.gzip_member(blk)
    assert m[:2] == b"\x1f\x8b"            # ID1 ID2
    assert m[2] == 8                        # CM = deflate
    assert m[3] == 0                        # FLG: no name/extra/comment => 10-byte header
    assert m[8] == 4                        # XFL = 4: compressor used its fastest level
    crc, isize = struct.unpack("<II", m[-8:])
    assert crc == binascii.crc32(blk) & 0xFFFFFFFF
    assert isize == len(blk)
    assert gzip.decompress(m) == blk
    assert oracle.gzip_length(blk) == len(m)


@pytest.mark.parametrize("blk", BLOCKS)
def test_length_matches_gzip_module_at_level1(blk):
    # Python's gzip module writes its own header around a raw level-1 deflate stream;
    # the member size must agree (header and trailer are 18 bytes in both).
    assert oracle.gzip_length(blk) == len(gzip.compress(blk, compresslevel=1, mtime=0))


@pytest.mark.parametrize("b", [16, 64, 128])
def test_stored_block_bound(b):
    # Deflate can always fall back to one stored block: 5 bytes of block header plus
    # the raw bytes; with the 18-byte wrapper that bounds a member at b + 23.
    rng = np.random.default_rng(b)
    for _ in range(200):
        blk = rng.integers(0, 256, b, dtype=np.uint8).tobytes()
        assert oracle.gzip_length(blk) <= b + 23
    # Uniform random bytes do not compress, so at b >= 64 the bound is met exactly.
    if b >= 64:
        blk = rng.integers(0, 256, b, dtype=np.uint8).tobytes()
        assert oracle.gzip_length(blk) == b + 23


def test_compressed_lengths_are_per_block():
    rng = np.random.default_rng(7)
    b, n = 64, 12
    x = rng.integers(0x20, 0x7F, (2, b * n), dtype=np.uint8)
    x[0, 3 * b:4 * b] = ord("z")           # one very compressible block
    c = oracle.compressed_lengths(x, b)
    assert c.shape == (2, n)
    for s in range(2):
        for i in range(n):
            assert c[s, i] == oracle.gzip_length(x[s, i * b:(i + 1) * b].tobytes())
    # Each block is compressed on its own: permuting blocks permutes c.
    perm = rng.permutation(n)
    xp = x.reshape(2, n, b)[:, perm].reshape(2, n * b)
    assert np.array_equal(oracle.compressed_lengths(xp, b), c[:, perm])
    # Changing block 5 leaves every other block's length unchanged.
    y = x.copy()
    y[1, 5 * b:6 * b] = 0
    cy = oracle.compressed_lengths(y, b)
    mask = np.ones_like(c, dtype=bool)
    mask[1, 5] = False
    assert np.array_equal(cy[mask], c[mask])
    assert c[0, 3] < c[0, 2]


def test_compressed_lengths_shape_errors():
    with pytest.raises(ValueError):
        oracle.compressed_lengths(np.zeros((1, 100), np.uint8), 64)
    with pytest.raises(ValueError):
        oracle.compressed_lengths(np.zeros(64, np.uint8), 64)
