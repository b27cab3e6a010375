"""Pins of the oracle's packed tile layout: hand-derived bytes, exhaustive
round trips, and the bit accounting the pages quote (gpt-diffusion STEPQuant
analysis, "Qué dice realmente el «6-bit»": 6 + 16/128 + 16/128 bits per value
for a 128x128 tile with one 16-bit scale per row and per column; 5.03x state
compression for the 6-bit nominal configuration)."""
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    for line in open(os.path.join(GOLD, "pack_bytes.txt")):
        if line.startswith("case"):
            lhs, rhs = line[4:].split("->")
            n, i, j0, *codes = [int(x) for x in lhs.split()]
            off, *bs = rhs.split()
            yield n, i, j0, codes, int(off), [int(b, 16) for b in bs]


@pytest.mark.parametrize("case", list(_cases()))
def test_golden_bytes(orc, case):
    n, i0, j, codes, off, expect = case
    Q = np.zeros((128, 128), np.int32)
    Q[i0:i0 + 4, j] = codes
    sig = np.full(128, 0x3F80, np.uint16)
    t = orc.pack(n, Q, sig, sig)
    np.testing.assert_array_equal(t[off:off + len(expect)], np.array(expect, np.uint8))


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("n", [4, 6, 8, 16])
def test_roundtrip_every_code(orc, n, dk, dv):
    rng = np.random.default_rng(n * dk + dv)
    if n == 16:
        Q = rng.integers(0, 1 << 16, (dk, dv))
        Q[(Q & 0x7C00) == 0x7C00] = 0x3C00     # no inf/nan encodings
    else:
        qmax = 2 ** (n - 1) - 1
        Q = rng.integers(-qmax, qmax + 1, (dk, dv))
        Q.reshape(-1)[: 2 * qmax + 1] = np.arange(-qmax, qmax + 1)
    Q = Q.astype(np.int32)
    sig = rng.integers(0, 1 << 16, dk).astype(np.uint16)
    c = rng.integers(0, 1 << 16, dv).astype(np.uint16)
    t = orc.pack(n, Q, sig, c)
    assert t.size == dk * dv * n // 8 + (0 if n == 16 else 2 * (dk + dv))
    Q2, s2, c2 = orc.unpack(n, dk, dv, t)
    np.testing.assert_array_equal(Q2, Q)
    if n != 16:
        np.testing.assert_array_equal(s2, sig)
        np.testing.assert_array_equal(c2, c)


@pytest.mark.parametrize("n", [4, 6, 8, 16])
def test_every_code_byte_belongs_to_one_element(orc, n):
    """Changing one element changes only its own n/2-byte slice of a lane row."""
    dk = dv = 128
    base = orc.pack(n, np.zeros((dk, dv), np.int32), np.zeros(dk, np.uint16), np.zeros(dv, np.uint16))
    seen = np.zeros(dk * dv * n // 8, np.int32)
    rng = np.random.default_rng(n)
    for _ in range(300):
        i, j = rng.integers(0, 128, 2)
        Q = np.zeros((dk, dv), np.int32)
        Q[i, j] = 1 if n != 16 else 0x3C00
        t = orc.pack(n, Q, np.zeros(dk, np.uint16), np.zeros(dv, np.uint16))
        diff = np.nonzero(t != base)[0]
        assert 1 <= diff.size <= 2
        assert diff.max() - diff.min() <= 2


def test_bit_accounting(orc):
    assert orc.tile_bytes(6, 128, 128) == 12800
    assert 8 * 12800 / (128 * 128) == 6.25            # 6 + 16/128 + 16/128
    assert orc.tile_bytes(4, 128, 128) == 8704
    assert orc.tile_bytes(8, 128, 128) == 16896
    assert orc.tile_bytes(16, 128, 128) == 32768
    for n in (4, 6, 8, 16):
        for d in ((64, 64), (128, 128), (64, 128), (128, 64)):
            assert orc.tile_stride(n, *d) % 256 == 0
    # the 6-bit nominal GDN mix {4:9, 6:16, 8:6, FP16:1} of 32 heads:
    slot = 9 * 8704 + 16 * 12800 + 6 * 16896 + 32768
    assert slot == 417280
    ratio = 32 * 128 * 128 * 4 / slot
    assert round(ratio, 2) == 5.03                      # the pages' 5.03x for Qwen
