"""Pins for the oracle's number-format conversions against numpy and torch
(independent library routines) and against exact rational arithmetic."""
import numpy as np
import pytest
import torch

import oracle_api as O
from exact import fr, rd16, ru16


def _edge_floats():
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, 1e10, -1e10,
            6.1035156e-05, 5.9604645e-08, 2.9802322e-08, 2.9802326e-08, 8.940697e-08,
            1e-30, -1e-30, 3.4e38, 1.0009765625, 1.00048828125, 1.00146484375, 2049.0, 2051.0]
    # exact midpoints between adjacent fp16 values (ties) across the range
    h = np.arange(0, 0x7bff, 97, dtype=np.uint16).view(np.float16).astype(np.float64)
    h2 = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    vals += list(((h + h2) / 2).astype(np.float32))
    vals += [-v for v in vals]
    return np.array(vals, dtype=np.float32)


def test_f16_to_f32_all_patterns_match_numpy():
    L = O.lib()
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float32)
    got = np.array([L.kvco_f16_to_f32(int(p)) for p in pats], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_rn_matches_numpy():
    L = O.lib()
    rng = np.random.default_rng(1)
    x = np.concatenate([
        _edge_floats(),
        rng.standard_normal(4000).astype(np.float32) * 10.0 ** rng.integers(-9, 6, 4000),
        rng.uniform(-70000, 70000, 2000).astype(np.float32),
    ]).astype(np.float32)
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([L.kvco_f32_to_f16_rn(float(v)) for v in x], dtype=np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_f32_to_f16_rn_every_pattern_and_midpoint_matches_numpy():
    """Round to nearest-even on the bit fields, against numpy's conversion at
    every fp16 value of both signs, at every exact midpoint between
    neighbours (ties) and one binary32 step either side of each, and one
    step either side of each value."""
    L = O.lib()
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)       # finite magnitudes
    lo = h.view(np.float16).astype(np.float64)
    hi = np.append(lo[1:], 65536.0)
    mid = ((lo + hi) / 2).astype(np.float32)                            # exact in binary32
    assert np.all(mid.astype(np.float64) == (lo + hi) / 2)
    f = lo.astype(np.float32)
    x = np.concatenate([f, mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf)),
                        np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(0)),
                        np.array([np.inf, 2.0 ** -25, 2.0 ** -26, 1e-45, 3.0 * 2.0 ** -26], np.float32)])
    x = np.concatenate([x, -x]).astype(np.float32)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    fn = L.kvco_f32_to_f16_rn
    got = np.fromiter((fn(float(v)) for v in x), dtype=np.uint16, count=x.size)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]
    nan = fn(float("nan"))
    assert (nan & 0x7C00) == 0x7C00 and (nan & 0x3FF) != 0


def test_f32_to_f16_directed_rounding_exact():
    L = O.lib()
    rng = np.random.default_rng(2)
    x = np.concatenate([
        _edge_floats()[np.abs(_edge_floats()) < 65000],
        rng.standard_normal(1500).astype(np.float32) * 10.0 ** rng.integers(-8, 4, 1500),
    ]).astype(np.float32)
    for v in x:
        d = np.uint16(L.kvco_f32_to_f16_rd(float(v))).view(np.float16)
        u = np.uint16(L.kvco_f32_to_f16_ru(float(v))).view(np.float16)
        assert d == rd16(fr(v)), (float(v), d)
        assert u == ru16(fr(v)), (float(v), u)


def test_f16_directed_rounding_overflow():
    L = O.lib()
    assert L.kvco_f32_to_f16_ru(65504.5) == 0x7C00          # above max finite -> +inf
    assert L.kvco_f32_to_f16_rd(65504.5) == 0x7BFF          # down -> max finite
    assert L.kvco_f32_to_f16_rd(-65504.5) == 0xFC00         # down -> -inf
    assert L.kvco_f32_to_f16_rd(-1e-10) == 0x8001           # below -0 -> -min subnormal
    assert L.kvco_f32_to_f16_ru(1e-10) == 0x0001


def test_bf16_round_trip_matches_torch():
    L = O.lib()
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(5000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 5000),
        # ties: lower 16 bits exactly 0x8000, both parities of the kept part
        (rng.integers(0, 2 ** 15, 500, dtype=np.uint32) << 17 | 0x8000).view(np.float32),
        ((rng.integers(0, 2 ** 15, 500, dtype=np.uint32) << 17 | 0x18000)).view(np.float32),
    ]).astype(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([L.kvco_f32_to_bf16_rn(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)
    back = np.array([L.kvco_bf16_to_f32(int(b)) for b in ref[:200]], dtype=np.float32)
    assert np.array_equal(back, torch.from_numpy(ref[:200].view(np.int16)).view(torch.bfloat16).float().numpy())
