"""Pins for the oracle's sub-byte weight packing (uint8 [N, K/2] compressed
storage of the BitBLAS guide, case 2; 2-bit BitNet weights of case 1)."""
import itertools
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_bytes.txt")


def _golden():
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        bits, vals, packed = (p.strip() for p in line.split("|"))
        out.append((int(bits), [int(v) for v in vals.split()],
                    [int(b, 16) for b in packed.split()]))
    return out


@pytest.mark.parametrize("case", _golden(), ids=lambda c: f"int{c[0]}-{c[1]}")
def test_hand_derived_bytes(oracle, case):
    bits, vals, packed = case
    v = np.array([vals], np.int8)
    p = oracle.pack_int4(v) if bits == 4 else oracle.pack_int2(v)
    assert list(p[0]) == packed
    back = oracle.unpack(p, len(vals), bits)
    assert list(back[0]) == vals


def test_int4_exhaustive_roundtrips(oracle):
    allbytes = np.arange(256, dtype=np.uint16).astype(np.uint8)[:, None]
    v = oracle.unpack_int4(allbytes, 2)
    assert v.min() == -8 and v.max() == 7
    assert np.array_equal(oracle.pack_int4(v), allbytes)
    pairs = np.array(list(itertools.product(range(-8, 8), repeat=2)), np.int8)
    assert np.array_equal(oracle.unpack_int4(oracle.pack_int4(pairs), 2), pairs)
    # low nibble is the even k, two's complement
    assert np.array_equal(v[:, 0], ((allbytes[:, 0].astype(np.int16) & 0xF) ^ 8) - 8)


def test_int2_exhaustive_roundtrips(oracle):
    allbytes = np.arange(256, dtype=np.uint16).astype(np.uint8)[:, None]
    v = oracle.unpack_int2(allbytes, 4)
    assert v.min() == -2 and v.max() == 1
    assert np.array_equal(oracle.pack_int2(v), allbytes)
    quads = np.array(list(itertools.product(range(-2, 2), repeat=4)), np.int8)
    assert np.array_equal(oracle.unpack_int2(oracle.pack_int2(quads), 4), quads)
    for j in range(4):
        assert np.array_equal(v[:, j], ((allbytes[:, 0] >> (2 * j)) & 3).astype(np.int8) - 2)


def test_multirow_layout(oracle):
    g = np.random.default_rng(3)
    v4 = g.integers(-8, 8, (5, 12), dtype=np.int8)
    p4 = oracle.pack_int4(v4)
    assert p4.shape == (5, 6)
    for n in range(5):
        for j in range(6):
            lo, hi = v4[n, 2 * j], v4[n, 2 * j + 1]
            assert p4[n, j] == ((int(lo) & 15) | ((int(hi) & 15) << 4))
    v2 = g.integers(-2, 2, (3, 16), dtype=np.int8)
    p2 = oracle.pack_int2(v2)
    assert p2.shape == (3, 4)
    for n in range(3):
        for b in range(4):
            assert p2[n, b] == sum((int(v2[n, 4 * b + j]) + 2) << (2 * j) for j in range(4))


def test_rejects_bad_input(oracle):
    with pytest.raises(oracle.OracleError):
        oracle.pack_int4(np.array([[8, 0]], np.int8))
    with pytest.raises(oracle.OracleError):
        oracle.pack_int4(np.array([[-9, 0]], np.int8))
    with pytest.raises(oracle.OracleError):
        oracle.pack_int4(np.zeros((1, 3), np.int8))
    with pytest.raises(oracle.OracleError):
        oracle.pack_int2(np.array([[2, 0, 0, 0]], np.int8))
    with pytest.raises(oracle.OracleError):
        oracle.pack_int2(np.zeros((1, 6), np.int8))
