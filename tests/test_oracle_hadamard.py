"""Pins for the oracle's randomized Hadamard transform.

The transform is fixed by the pages only as a randomized Hadamard rotation over
head_dim (FastKVComp Sec. 4.1; KVServe Sec. 5.1, Hadamard as a transformer
module).  These tests tie the oracle to the textbook Sylvester matrix, to
orthonormality, and to the published splitmix64 outputs that drive the signs.
"""
import os

import numpy as np
import pytest

import oracle_api as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


def sylvester(n: int) -> np.ndarray:
    """H[i, j] = (-1)^popcount(i & j), from the definition."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bits = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(bits % 2 == 0, 1, -1).astype(np.int64)


def test_splitmix64_published_outputs():
    import ctypes as C
    want = [int(x, 16) for x in _read_golden("splitmix64_seed0.txt")]
    st = C.c_uint64(0)
    got = [O.lib().kvco_splitmix64(C.byref(st)) for _ in range(3)]
    assert got == want


def test_signs_follow_top_bit_of_splitmix64():
    want = [int(x, 16) for x in _read_golden("splitmix64_seed0.txt")]
    d = O.signs(0, 3)
    assert list(d) == [-1 if (w >> 63) else 1 for w in want]
    d128 = O.signs(0x5EED0F4ADA4A4D, 128)
    assert set(np.unique(d128)) <= {-1, 1}
    assert 40 < int((d128 == -1).sum()) < 88
    assert np.array_equal(d128, O.signs(0x5EED0F4ADA4A4D, 128))
    assert not np.array_equal(d128, O.signs(1, 128))


def test_sylvester_definition_matches_textbook_order4():
    rows = np.array([[int(v) for v in r.split()] for r in _read_golden("hadamard4.txt")])
    assert np.array_equal(sylvester(4), rows)


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128, 256])
def test_hadamard_is_orthogonal_in_integers(n):
    H = sylvester(n)
    assert np.array_equal(H @ H.T, n * np.eye(n, dtype=np.int64))
    # the orthonormal version H/sqrt(n) satisfies H H^T = I
    Hn = H / np.sqrt(n)
    assert np.allclose(Hn @ Hn.T, np.eye(n), atol=1e-12)


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64, 128, 256])
def test_fwht_of_unit_vectors_gives_columns_exactly(n):
    H = sylvester(n)
    for j in range(n):
        e = np.zeros(n, np.float32)
        e[j] = 1.0
        assert np.array_equal(O.fwht(e), H[:, j].astype(np.float32))


def test_fwht_n2_brute_force():
    for a, b in [(1.5, -2.25), (3.0, 3.0), (1e-3, 7.0), (-0.0, 0.0)]:
        out = O.fwht(np.array([a, b], np.float32))
        assert out[0] == np.float32(a) + np.float32(b)
        assert out[1] == np.float32(a) - np.float32(b)


def test_fwht_matches_dense_fp64_product():
    rng = np.random.default_rng(5)
    H = sylvester(128).astype(np.float64)
    for _ in range(50):
        x = (rng.standard_normal(128) * rng.choice([1, 15], 128)).astype(np.float32)
        ref = H @ x.astype(np.float64)
        got = O.fwht(x).astype(np.float64)
        assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_parseval_and_round_trip():
    rng = np.random.default_rng(6)
    c = np.float32(O.lib().kvco_norm_const(128))
    assert c == np.float32(1.0 / np.sqrt(128.0))
    for _ in range(50):
        x = rng.standard_normal(128).astype(np.float32)
        y = O.fwht(x) * c
        assert abs(np.linalg.norm(y.astype(np.float64)) / np.linalg.norm(x.astype(np.float64)) - 1) < 2e-7 * 16
        back = O.fwht(y) * c
        assert np.max(np.abs(back - x)) <= 1e-6 * np.max(np.abs(x)) * 8


def test_unnormalized_transform_is_an_involution_up_to_n():
    rng = np.random.default_rng(7)
    x = rng.integers(-1000, 1000, 128).astype(np.float32)
    # integer inputs of this size stay exact in binary32
    assert np.array_equal(O.fwht(O.fwht(x)), 128 * x)
