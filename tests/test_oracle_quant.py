"""Pins for the oracle's min-max quantizer.

The pages keep KVServe's min-max rule (FastKVComp Sec. 4.1) and fix the
metadata cost through KIVI's ~5.33x ceiling at 2 bits (KVServe Sec. 7.3).
These tests re-derive every parameter with exact rationals, check coverage,
the code range, brute-force nearest-level optimality on single groups, the
reconstruction bound, and the closed-form compression ratio.
"""
import os
from fractions import Fraction as F

import numpy as np
import pytest

import kvc_workloads as W
import oracle_api as O
from exact import fr, rd16, rd32, rn32, ru16, ru32
from test_oracle_hadamard import sylvester

C128 = np.float32(1.0 / np.sqrt(128.0))


def f16(bits: int) -> np.float16:
    return np.uint16(bits).view(np.float16)


def expected_params(z: np.ndarray, bits: int, c: np.float32):
    """Parameters recomputed from their definition with exact rationals."""
    k = (1 << bits) - 1
    zmin, zmax = fr(np.min(z)), fr(np.max(z))
    lo = rd32(zmin * fr(c))
    hi = ru32(zmax * fr(c))
    m = rd16(fr(lo))
    rng = ru32(fr(hi) - fr(m))
    s32 = ru32(fr(rng) / k)
    s = ru16(fr(s32))
    return s, m


def expected_codes(z, bits, c, s, m, inv):
    out = []
    for v in z:
        t = rn32(fr(v) * fr(c) - fr(m))             # one rounding: fused multiply-add
        q = round(fr(t) * fr(inv))                  # exact product, ties to even
        out.append(q)
    return np.array(out)


def groups(rng, n_groups=40, size=32):
    out = []
    for i in range(n_groups):
        kind = i % 8
        if kind == 0:
            g = rng.standard_normal(size)
        elif kind == 1:
            g = rng.standard_normal(size) * 200 + 30
        elif kind == 2:
            g = 1000.0 + rng.standard_normal(size) * 1e-3       # tiny range, large offset
        elif kind == 3:
            g = rng.standard_normal(size) * 1e-6                 # fp16-subnormal parameters
        elif kind == 4:
            g = np.full(size, 0.75)                              # constant, fp16-exact
        elif kind == 5:
            g = np.full(size, 0.1)                               # constant, not fp16-exact
        elif kind == 6:
            g = rng.uniform(-1, 1, size) * 12
        else:
            g = np.round(rng.standard_normal(size) * 4) / 4      # many ties
        out.append(g.astype(np.float32))
    return out


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_params_match_exact_definition_and_cover(bits):
    rng = np.random.default_rng(10 + bits)
    k = (1 << bits) - 1
    for z in groups(rng):
        for c in (C128, np.float32(1.0)):
            st, s, m, inv = O.group_params(z, bits, float(c))
            assert st == O.OK
            es, em = expected_params(z, bits, c)
            assert f16(s) == es and f16(m) == em, (z[:3], bits)
            sf, mf = fr(f16(s)), fr(f16(m))
            # coverage of the exact normalized range [c*min z, c*max z]
            assert mf <= fr(np.min(z)) * fr(c)
            assert mf + k * sf >= fr(np.max(z)) * fr(c)
            assert inv == (0.0 if sf == 0 else float(np.float32(1.0) / np.float32(f16(s))))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_codes_exact_definition_range_and_reconstruction(bits):
    rng = np.random.default_rng(20 + bits)
    k = (1 << bits) - 1
    for z in groups(rng):
        st, s, m, inv = O.group_params(z, bits, float(C128))
        st2, q = O.quantize_group(z, bits, float(C128), s, m, inv)
        assert st2 == O.OK
        assert q.min() >= 0 and q.max() <= k
        assert np.array_equal(q, expected_codes(z, bits, C128, f16(s), f16(m), np.float32(inv)))
        sf, mf = fr(f16(s)), fr(f16(m))
        ymax = max(abs(fr(v) * fr(C128)) for v in z)
        ulp = fr(np.spacing(np.float32(float(ymax)))) * 2
        for v, code in zip(z, q):
            y = fr(v) * fr(C128)
            assert abs(y - (code * sf + mf)) <= sf / 2 + ulp


@pytest.mark.parametrize("bits", [2, 4])
def test_single_group_brute_force_nearest_level(bits):
    """Each code is the nearest of all 2^b levels (up to exact ties)."""
    rng = np.random.default_rng(30 + bits)
    k = (1 << bits) - 1
    for _ in range(30):
        z = (rng.standard_normal(32) * rng.uniform(0.1, 50)).astype(np.float32)
        st, s, m, inv = O.group_params(z, bits, float(C128))
        _, q = O.quantize_group(z, bits, float(C128), s, m, inv)
        sf, mf = fr(f16(s)), fr(f16(m))
        for v, code in zip(z, q):
            y = fr(v) * fr(C128)
            d = [abs(y - (lv * sf + mf)) for lv in range(k + 1)]
            assert d[code] <= min(d) + sf * F(1, 1 << 20)


def test_constant_group_and_extremes():
    # a constant group always gets one code for all its elements
    z = np.full(32, 0.75 / C128, np.float32)
    st, s, m, inv = O.group_params(z, 4, float(C128))
    _, q = O.quantize_group(z, 4, float(C128), s, m, inv)
    assert np.all(q == q[0])
    # an exactly representable constant: zero scale, all-zero codes, exact minimum
    z = np.full(32, 0.75, np.float32)
    st, s, m, inv = O.group_params(z, 4, 1.0)
    _, q = O.quantize_group(z, 4, 1.0, s, m, inv)
    assert s == 0 and inv == 0.0 and f16(m) == np.float16(0.75) and np.all(q == 0)
    rng = np.random.default_rng(40)
    for bits in (2, 4, 8):
        for _ in range(20):
            z = rng.standard_normal(32).astype(np.float32) * 3
            st, s, m, inv = O.group_params(z, bits, float(C128))
            _, q = O.quantize_group(z, bits, float(C128), s, m, inv)
            assert q[np.argmin(z)] == 0
            assert q[np.argmax(z)] == (1 << bits) - 1


def test_range_error_on_overflowing_parameters():
    z = np.array([0.0, 1e6], np.float32)
    st, s, m, inv = O.group_params(z, 4, 1.0)
    assert st == O.RANGE
    z = np.array([-1e6, 0.0], np.float32)
    st, s, m, inv = O.group_params(z, 4, 1.0)
    assert st == O.RANGE


def _cr_q(wl, which):
    cfg = O.cfg_from_workload(wl, layers=1)
    T = 4096
    L = O.lib()
    import ctypes as C
    raw = T * wl.heads * wl.head_dim * 2
    q = L.kvco_codes_bytes(C.byref(cfg), which, T) + L.kvco_params_bytes(C.byref(cfg), which, T)
    return raw / q


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_quantized_size_closed_form(name):
    """Codes + params: b/8 + 4/G bytes per 2-byte value -> CR_q = 16/(b + 32/G)."""
    wl = W.WORKLOADS[name]
    for which, pol in ((0, wl.k), (1, wl.v)):
        assert _cr_q(wl, which) == pytest.approx(16.0 / (pol.bits + 32.0 / pol.group), rel=1e-12)


def test_kivi_metadata_ceiling_pin():
    rows = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "kivi_ceiling.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, val = line.split()
                rows[key] = float(val)
    wl = W.WORKLOADS["c1_single_layer_512"].with_(
        k=W.TensorPolicy(int(rows["bits"]), "token", int(rows["group"])),
        v=W.TensorPolicy(int(rows["bits"]), "token", int(rows["group"])))
    assert round(_cr_q(wl, 0), 2) == rows["ratio"]


def test_tensor_round_trip_error_bound_per_token():
    """Orthonormality: per head vector, ||x - x_hat||_2 <= sqrt(D) * max_g s_g / 2
    (plus output rounding to fp16)."""
    wl = W.WORKLOADS["c1_single_layer_512"]
    k, v = W.dense_kv(wl, tokens=64)
    cfg = O.cfg_from_workload(wl)
    x = W.as_u16(k)
    st, codes, params = O.quantize_tensor(cfg, 0, x, 64)
    assert st == O.OK
    st, xh = O.dequantize_tensor(cfg, 0, codes, params, 64)
    assert st == O.OK
    xf = x.view(np.float16).astype(np.float64).reshape(-1, 128)
    xhf = xh.view(np.float16).astype(np.float64).reshape(-1, 128)
    p = params.view(np.uint16).reshape(-1, 128 // 32, 2)
    smax = p[:, :, 0].view(np.float16).astype(np.float64).max(axis=1)
    err = np.linalg.norm(xf - xhf, axis=1)
    bound = np.sqrt(128) * smax / 2 + np.sqrt(128) * np.abs(xf).max(axis=1) * 2 ** -11
    assert np.all(err <= bound)


def test_tensor_round_trip_error_bound_per_channel_ragged():
    wl = W.WORKLOADS["c3_llama70b_32k"]
    T = 150                      # 2 full groups of 64 + a partial group of 22
    k, v = W.dense_kv(wl, layers=2, tokens=T)
    cfg = O.cfg_from_workload(wl, layers=2)
    x = W.as_u16(k)
    st, codes, params = O.quantize_tensor(cfg, 0, x, T)
    assert st == O.OK
    assert codes.size == 2 * (2 * 8 * 128 * 32 + 8 * 128 * 11)
    st, xh = O.dequantize_tensor(cfg, 0, codes, params, T)
    assert st == O.OK
    import torch
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy().reshape(2, T, 8, 128)
    xhf = torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).double().numpy().reshape(2, T, 8, 128)
    # params [L][NG][H][D] -> per (l, token, h) the largest scale over channels
    p = params.view(np.uint16).reshape(2, 3, 8, 128, 2)
    s = p[..., 0].view(np.float16).astype(np.float64)
    smax = s.max(axis=3)                                 # [L, NG, H]
    smax_t = np.repeat(smax, 64, axis=1)[:, :T]          # [L, T, H]
    err = np.linalg.norm(xf - xhf, axis=3)
    bound = np.sqrt(128) * smax_t / 2 + np.sqrt(128) * np.abs(xf).max(axis=3) * 2 ** -8
    assert np.all(err <= bound)


def test_per_token_layout_against_direct_computation():
    """Codes and params land where the format says, checked by recomputing
    each group directly from a dense fp64-verified transform."""
    wl = W.WORKLOADS["c1_single_layer_512"]
    T = 5
    k, _ = W.dense_kv(wl, tokens=T)
    cfg = O.cfg_from_workload(wl)
    x = W.as_u16(k).reshape(T * 8, 128)
    st, codes, params = O.quantize_tensor(cfg, 0, x, T)
    d = O.signs(wl.sign_seed, 128).astype(np.float32)
    H = sylvester(128).astype(np.float64)
    for vec in range(T * 8):
        v = x[vec].view(np.float16).astype(np.float32) * d
        z = O.fwht(v)
        assert np.max(np.abs(z - H @ v.astype(np.float64))) < 1e-3
        for g in range(4):
            zg = z[g * 32:(g + 1) * 32]
            _, s, m, inv = O.group_params(zg, 4, float(C128))
            assert params.view(np.uint16)[(vec * 4 + g) * 2] == s
            assert params.view(np.uint16)[(vec * 4 + g) * 2 + 1] == m
            _, q = O.quantize_group(zg, 4, float(C128), s, m, inv)
            row = codes[vec * 64:(vec + 1) * 64]
            nib = np.stack([row & 15, row >> 4], axis=1).reshape(-1)
            assert np.array_equal(nib[g * 32:(g + 1) * 32], q)
