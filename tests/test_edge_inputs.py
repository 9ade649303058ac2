"""The GPU edge-case inputs (tests/test_gpu_edge.py) are what they claim to be,
checked on the CPU with the oracle and exact arithmetic: tie inputs make
exact code ties, tiny inputs give fp16-subnormal parameters, overflow inputs
parameters near the largest fp16, and the zero inputs -0 group minimums."""
import numpy as np
import pytest
from fractions import Fraction as F

import kvc_workloads as W
import oracle_api as O
from exact import rn32
import test_gpu_edge as E

D = 128
C = E.C128


def _z(wl, x):
    d = O.signs(wl.sign_seed, D).astype(np.float32)
    xv = E._to_dtype(x, wl.dtype).float().numpy().reshape(-1, D)
    return np.stack([O.fwht(r * d) for r in xv])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("pols", range(len(E.POLICIES)))
def test_tie_inputs_make_exact_ties(dtype, pols):
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(dtype=dtype, heads=2)
    T = 200
    for pol in E.POLICIES[pols]:
        x = E.build_ties(wl, pol, 1, T, np.random.default_rng(1))
        assert np.array_equal(E._to_dtype(x, dtype).double().numpy(), x)       # exactly representable
        z = _z(wl, x).reshape(T, 2, D)
        ties = 0
        if pol.axis == "token":
            groups = [z[t, h, g:g + pol.group] for t in range(0, T, 17) for h in range(2)
                      for g in range(0, D, pol.group)]
        else:
            groups = [z[g:g + pol.group, h, ch] for g in range(0, T, pol.group) for h in range(2)
                      for ch in range(0, D, 29)]
        for zg in groups:
            st, s, m, inv = O.group_params(zg, pol.bits, float(C))
            assert st == O.OK
            mf = F(float(np.uint16(m).view(np.float16)))
            for v in zg:
                t = rn32(F(float(v)) * F(float(C)) - mf)
                if (F(float(t)) * F(float(np.float32(inv)))).denominator == 2:
                    ties += 1
        assert ties >= len(groups), (pol, ties, len(groups))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_tiny_and_overflow_inputs_reach_the_parameter_corners(dtype):
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(dtype=dtype, heads=2)
    T = 64
    pol = W.TensorPolicy(4, "token", 32)
    z = _z(wl, E.build_tiny(wl, pol, 1, T, np.random.default_rng(2)))
    ss, mm = [], []
    for r in z:
        for g in range(0, D, 32):
            st, s, m, _ = O.group_params(r[g:g + 32], 4, float(C))
            assert st == O.OK
            ss.append(s); mm.append(m)
    ss = np.array(ss, np.uint16); mm = np.array(mm, np.uint16)
    assert np.all((ss & 0x7C00) == 0) and np.all((mm & 0x7C00) == 0)     # subnormal (or zero) fp16
    z = _z(wl, E.build_overflow(wl, pol, 1, T, np.random.default_rng(3)))
    big = 0
    for r in z:
        for g in range(0, D, 32):
            st, s, m, _ = O.group_params(r[g:g + 32], 4, float(C))
            assert st == O.OK
            big += abs(float(np.uint16(m).view(np.float16))) > 55000
    assert big >= len(z) // 4


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_zero_inputs_have_negative_zero_group_minimums(dtype):
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(dtype=dtype, heads=2)
    T = 64
    z = _z(wl, E.build_zeros(wl, W.TensorPolicy(4, "channel", 64), 1, T, np.random.default_rng(4)))
    negzero_min_tok = 0
    for r in z:
        for g in range(0, D, 32):
            zg = r[g:g + 32]
            if np.all(zg == 0) and np.any(np.signbit(zg)):
                negzero_min_tok += 1
    assert negzero_min_tok > 0
    zc = z.reshape(T, 2, D)
    negzero_min_ch = sum(1 for h in range(2) for ch in range(D)
                         if zc[:, h, ch].min() == 0 and np.any(np.signbit(zc[:, h, ch]) & (zc[:, h, ch] == 0)))
    assert negzero_min_ch > 0
