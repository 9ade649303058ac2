"""Pins for the oracle's lossless components (FastKVComp Sec. 4.2: tuple
reordering, bit shuffling, zero elimination; pipeline TUPL8_1 -> BIT_8 ->
RZE_2).  Each component is checked against a numpy formulation of its
definition, and every component and pipeline must round-trip bit-exactly."""
import numpy as np
import pytest

import oracle_api as O

S = O.STAGE_IDS
LENGTHS = [0, 1, 2, 7, 8, 15, 16, 63, 64, 511, 512, 513, 1000, 4095, 4096, 4100]


def patterns(n, rng):
    yield "random", rng.integers(0, 256, n, dtype=np.uint8)
    yield "zeros", np.zeros(n, np.uint8)
    yield "ones", np.full(n, 0xFF, np.uint8)
    sp = np.zeros(n, np.uint8)
    if n:
        idx = rng.choice(n, max(1, n // 50), replace=False)
        sp[idx] = rng.integers(1, 256, idx.size)
    yield "sparse", sp
    yield "alternating", (np.arange(n) % 2 * 0xA5).astype(np.uint8)
    yield "nibbles", rng.integers(0, 16, n, dtype=np.uint8) * 17


def np_tupl(x, k):
    m = x.size // k
    head = x[:m * k].reshape(m, k).T.reshape(-1)
    return np.concatenate([head, x[m * k:]])


def np_diff(x, w):
    nw = x.size // w
    dt = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}[w]
    words = x[:nw * w].copy().view(dt)
    out = words.copy()
    if nw > 1:
        out[1:] = words[1:] - words[:-1]        # unsigned arithmetic wraps mod 2^(8w)
    return np.concatenate([out.view(np.uint8), x[nw * w:]])


def np_bit(x, w):
    B = 8 * w
    gb = w * B
    ng = x.size // gb
    out = x.copy()
    for g in range(ng):
        blk = x[g * gb:(g + 1) * gb]
        bits = np.unpackbits(blk, bitorder="little").reshape(B, B)   # row = word, col = bit
        out[g * gb:(g + 1) * gb] = np.packbits(bits.T.reshape(-1), bitorder="little")
    return out


def np_rze(x, w):
    nw = x.size // w
    words = x[:nw * w].reshape(nw, w)
    nz = words.any(axis=1)
    bitmap = np.packbits(nz.astype(np.uint8), bitorder="little") if nw else np.zeros(0, np.uint8)
    return np.concatenate([bitmap, words[nz].reshape(-1), x[nw * w:]])


REFS = {
    "TUPL2_1": lambda x: np_tupl(x, 2), "TUPL4_1": lambda x: np_tupl(x, 4), "TUPL8_1": lambda x: np_tupl(x, 8),
    "DIFF1": lambda x: np_diff(x, 1), "DIFF2": lambda x: np_diff(x, 2), "DIFF4": lambda x: np_diff(x, 4),
    "DIFF8": lambda x: np_diff(x, 8),
    "BIT_1": lambda x: np_bit(x, 1), "BIT_2": lambda x: np_bit(x, 2), "BIT_4": lambda x: np_bit(x, 4),
    "BIT_8": lambda x: np_bit(x, 8),
    "RZE_1": lambda x: np_rze(x, 1), "RZE_2": lambda x: np_rze(x, 2), "RZE_4": lambda x: np_rze(x, 4),
    "RZE_8": lambda x: np_rze(x, 8),
}


@pytest.mark.parametrize("stage", list(REFS))
def test_stage_matches_numpy_definition_and_round_trips(stage):
    rng = np.random.default_rng(hash(stage) & 0xFFFF)
    for n in LENGTHS:
        for name, x in patterns(n, rng):
            st, enc = O.stage_encode(S[stage], x)
            assert st == O.OK
            assert np.array_equal(enc, REFS[stage](x)), (stage, n, name)
            st, dec = O.stage_decode(S[stage], enc, n)
            assert st == O.OK and np.array_equal(dec, x), (stage, n, name)


@pytest.mark.parametrize("k", [2, 4, 8])
def test_tupl_is_a_permutation(k):
    x = np.arange(4099, dtype=np.int64)
    perm = np_tupl(x, k)
    assert np.array_equal(np.sort(perm), x)
    xb = (np.arange(4099) % 251).astype(np.uint8)
    st, enc = O.stage_encode(S["TUPL%d_1" % k], xb)
    assert np.array_equal(enc, xb[perm])


@pytest.mark.parametrize("w", [1, 2, 4, 8])
def test_bit_transpose_is_an_involution(w):
    rng = np.random.default_rng(w)
    x = rng.integers(0, 256, 8 * w * w * 3 + 5, dtype=np.uint8)
    _, once = O.stage_encode(S["BIT_%d" % w], x)
    _, twice = O.stage_encode(S["BIT_%d" % w], once)
    assert np.array_equal(twice, x)
    assert not np.array_equal(once, x)


PIPELINES = [("TUPL8_1", "BIT_8", "RZE_2"), ("TUPL8_1", "RZE_2"), ("DIFF1", "RZE_1"),
             ("TUPL4_1", "DIFF4", "BIT_4", "RZE_4"), ("BIT_1",), ("RZE_8",)]


@pytest.mark.parametrize("pipe", PIPELINES)
def test_chunk_pipeline_round_trip(pipe):
    rng = np.random.default_rng(len(pipe))
    ids = [S[s] for s in pipe]
    for n in LENGTHS + [65536]:
        for name, x in patterns(n, rng):
            st, enc, raw = O.chunk_encode(ids, x)
            assert st == O.OK
            assert enc.size <= n
            assert raw == (1 if enc.size == n else 0)
            if raw:
                assert np.array_equal(enc, x)
            st, dec = O.chunk_decode(ids, enc, raw, n)
            assert st == O.OK and np.array_equal(dec, x), (pipe, n, name)


def test_chunk_composition_equals_stage_composition():
    rng = np.random.default_rng(9)
    x = (rng.random(65536) < 0.05).astype(np.uint8) * rng.integers(0, 16, 65536).astype(np.uint8)
    y = x
    for s in ("TUPL8_1", "BIT_8", "RZE_2"):
        y = REFS[s](y)
    st, enc, raw = O.chunk_encode([S["TUPL8_1"], S["BIT_8"], S["RZE_2"]], x)
    assert raw == 0 and np.array_equal(enc, y)


def test_zero_chunk_is_exactly_a_zero_bitmap():
    x = np.zeros(65536, np.uint8)
    st, enc, raw = O.chunk_encode([S["TUPL8_1"], S["BIT_8"], S["RZE_2"]], x)
    assert st == O.OK and raw == 0 and enc.size == 4096 and not enc.any()


def test_chunk_without_zero_words_is_stored_raw():
    rng = np.random.default_rng(11)
    x = rng.integers(1, 256, 65536, dtype=np.uint8)
    st, enc, raw = O.chunk_encode([S["TUPL8_1"], S["RZE_2"]], x)
    assert st == O.OK and raw == 1 and np.array_equal(enc, x)


def test_rze_decode_rejects_inconsistent_input():
    x = np.zeros(64, np.uint8)
    x[5] = 3
    st, enc = O.stage_encode(S["RZE_2"], x)
    assert st == O.OK
    assert O.stage_decode(S["RZE_2"], enc[:-1], 64)[0] == O.CORRUPT        # truncated
    bad = enc.copy(); bad[0] |= 0x80                                          # extra flagged word
    assert O.stage_decode(S["RZE_2"], bad, 64)[0] == O.CORRUPT
    bad = np.concatenate([enc[:4], np.zeros(2, np.uint8)])                    # flagged word is zero
    assert O.stage_decode(S["RZE_2"], bad, 64)[0] == O.CORRUPT
    assert O.chunk_decode([S["RZE_2"]], enc, 1, 64)[0] == O.CORRUPT          # raw with wrong size
