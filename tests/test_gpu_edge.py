"""GPU parity on the corners of the quantizer's arithmetic, for both dtypes and
both group axes: the HIP library (through its C ABI) against the oracle on
the same input bytes, stream bytes and reconstructions compared exactly.

FastKVComp ("Beyond Compression Ratio: High-Throughput KV Compression for
Disaggregated LLM Serving", Sec. 4.1) keeps the original min-max quantization
rule; these inputs exercise where that rule's fixed-point arithmetic has its
corners:
  tiny      head vectors of magnitude ~1e-6: fp16-subnormal scale and minimum;
  overflow  head vectors scaled so the largest |c z| is just under 65000:
            parameters next to the largest finite fp16;
  ties      transform outputs chosen exactly (small integers times 2^e, so the
            rotation is exact) such that every zero output sits exactly half way
            between two codes (q + 1/2 = t * inv in exact arithmetic);
  zeros     head vectors of +0 and -0 (group extremes -0), constant transform
            outputs, and per-channel groups whose minimum is -0;
  nonfinite one NaN or infinite input value: both sides report a range error.
"""
import numpy as np
import pytest
import torch
from fractions import Fraction as F

import kv_cache_compression_kvc_amd as K
import kvc_workloads as W
import oracle_api as O
from exact import rn32
from gpu_helpers import DEV, gpu_decode, gpu_encode, log, oracle_encode, to_u16
from test_oracle_hadamard import sylvester

pytestmark = pytest.mark.gpu

TP = W.TensorPolicy
D = 128
C128 = np.float32(1.0 / np.sqrt(128.0))
HS = sylvester(D).astype(np.float64)

# (zmin, zmax, e): groups of transform outputs {zmin, zmax, 0...} * 2^e whose
# zero elements are exact code ties at that width (found with the oracle's
# parameters and exact arithmetic, re-checked by _assert_tie below); e >= -17
# keeps the inputs exact multiples of 2^-24, representable in fp16
TIES = {2: [(-1, 1, -17)],
        4: [(-12, 8, -17), (-6, 4, -16), (-3, 2, -15), (-1, 0, -15), (-1, 9, -17), (-2, 0, -16)],
        8: [(-11, 5, -16), (-10, 0, -15), (-7, 2, -14), (-5, 0, -14), (-11, 9, -14), (-8, 2, -15)]}

POLICIES = [(TP(4, "channel", 64), TP(2, "token", 32)),
            (TP(2, "channel", 32), TP(8, "token", 16)),
            (TP(8, "channel", 64), TP(4, "token", 128))]


def _assert_tie(bits, zmin, zmax, e):
    z = np.array([zmin, 0, zmax], np.float32) * np.float32(2.0 ** e)
    st, s, m, inv = O.group_params(z, bits, float(C128))
    assert st == O.OK
    mf = F(float(np.uint16(m).view(np.float16)))
    t = rn32(F(0) * F(float(C128)) - mf)
    p = F(float(t)) * F(float(np.float32(inv)))
    assert p.denominator == 2, (bits, zmin, zmax, e, p)


def _to_dtype(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return t.to(torch.float16 if dtype == "f16" else torch.bfloat16)


def _signs(wl):
    return O.signs(wl.sign_seed, D).astype(np.float64)


def _from_z(z: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Inputs whose transform FWHT(d * x) is exactly z (z * H / 128 is exact for
    the small-integer z used here)."""
    return (z @ HS.T) / 128.0 * d


def build_tiny(wl, pol, L, T, rng):
    return rng.standard_normal((L, T, wl.heads, D)) * 2e-6


def build_overflow(wl, pol, L, T, rng):
    d = _signs(wl)
    x = rng.standard_normal((L, T, wl.heads, D))
    y = C128 * ((x * d) @ HS.T)
    # the largest |c z| of each head vector near 64000, its inputs under 60000
    x *= np.minimum(64000.0 / np.abs(y).max(axis=-1, keepdims=True),
                    60000.0 / np.abs(x).max(axis=-1, keepdims=True))
    x *= rng.uniform(0.95, 1.0, x.shape[:-1] + (1,))
    for _ in range(20):                      # after rounding to the dtype: every |c z| < 65000
        xr = _to_dtype(x, wl.dtype).double().numpy()
        y = np.abs(C128 * ((xr * d) @ HS.T)).max(axis=-1, keepdims=True)
        if y.max() < 65000.0:
            return x
        x = np.where(y >= 65000.0, x * 0.995, x)
    raise AssertionError("could not place the inputs under the limit")


def build_ties(wl, pol, L, T, rng):
    d = _signs(wl)
    combos = TIES[pol.bits]
    for c in combos:
        _assert_tie(pol.bits, *c)
    z = np.zeros((L, T, wl.heads, D))
    scale = np.zeros((L, T, wl.heads, 1))
    if pol.axis == "token":
        pick = rng.integers(0, len(combos), (L, T, wl.heads))
        for idx, (zmin, zmax, e) in enumerate(combos):
            sel = pick == idx
            for g0 in range(0, D, pol.group):
                off = rng.integers(0, pol.group - 1)
                z[..., g0 + off][sel] = zmin
                z[..., g0 + off + 1][sel] = zmax
            scale[sel] = 2.0 ** e
    else:
        # per (layer, token group, head): the group's first token is zmin in
        # every channel, its second zmax, the others zero
        G = pol.group
        for l in range(L):
            for g0 in range(0, T, G):
                for h in range(wl.heads):
                    zmin, zmax, e = combos[rng.integers(0, len(combos))]
                    z[l, g0, h] = zmin
                    if g0 + 1 < T:
                        z[l, g0 + 1, h] = zmax
                    scale[l, g0:g0 + G, h] = 2.0 ** e
    return _from_z(z, d) * scale


def build_zeros(wl, pol, L, T, rng):
    d = _signs(wl)
    x = np.zeros((L, T, wl.heads, D))
    kind = rng.integers(0, 5, (L, T, wl.heads))
    neg = rng.integers(0, 2, (L, T, wl.heads, D)).astype(bool)
    x = np.where((kind == 0)[..., None], -0.0, x)                             # all -0
    x = np.where(((kind == 1)[..., None]) & neg, -0.0, x)                      # mixed signed zeros
    a = rng.integers(1, 64, (L, T, wl.heads)) * 2.0 ** -6                      # constant outputs a * 1
    const = np.zeros_like(x)
    const[..., 0] = a * d[0]
    x = np.where((kind == 2)[..., None], const, x)
    # transform outputs of 1 or 2 (positive): per-channel groups whose other
    # tokens are signed zeros then have the minimum -0 or +0
    zpos = rng.integers(1, 3, (L, T, wl.heads, D)).astype(np.float64)
    x = np.where((kind >= 3)[..., None], _from_z(zpos, d) * 2.0 ** -4, x)
    return x


BUILDERS = {"tiny": build_tiny, "overflow": build_overflow, "ties": build_ties, "zeros": build_zeros}


@pytest.mark.parametrize("kind", list(BUILDERS))
@pytest.mark.parametrize("pols", range(len(POLICIES)))
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_quantizer_corners_match_oracle(kind, pols, dtype):
    kp, vp = POLICIES[pols]
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(dtype=dtype, k=kp, v=vp, chunk_bytes=8192,
                                              name=f"edge_{kind}_{dtype}")
    L, T = 2, 200
    rng = np.random.default_rng([pols, len(kind), len(dtype)])
    k = _to_dtype(BUILDERS[kind](wl, kp, L, T, rng), dtype)
    v = _to_dtype(BUILDERS[kind](wl, vp, L, T, rng), dtype)
    log(f"edge case {kind} {dtype} K {kp} V {vp}")
    st, ref = oracle_encode(wl, to_u16(k), to_u16(v), T, L)
    assert st == O.OK, st
    plan, got, ws = gpu_encode(wl, k.to(DEV), v.to(DEV), T, L)
    assert got.size == ref.size and np.array_equal(got, ref), "GPU stream differs from the oracle's"
    st, kd, vd = O.decode(ref, L * T * wl.heads * D)
    assert st == O.OK
    st, kg, vg = gpu_decode(plan, got, wl, T, L)
    assert st == K.OK, K.status_string(st)
    assert np.array_equal(to_u16(kg).reshape(-1), kd) and np.array_equal(to_u16(vg).reshape(-1), vd)


@pytest.mark.parametrize("bad", ["nan", "inf", "-inf", "over"])
@pytest.mark.parametrize("axis", ["token", "channel"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_nonfinite_and_overflowing_inputs_are_range_errors(bad, axis, dtype):
    """One NaN or infinite value in one channel of one token, or one head
    vector whose transform reaches c z ~ -67900: the GPU's encode status and
    the oracle's are both KVC_ERR_RANGE.  Under per-channel groups the other
    tokens of the group are finite, so the group extremes must see the value."""
    pol = TP(4, axis, 64 if axis == "channel" else 32)
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(dtype=dtype, k=pol, v=TP(2, "token", 32), chunk_bytes=8192,
                                              name=f"range_{bad}")
    L, T = 2, 192
    k, v = W.dense_kv(wl, layers=L, tokens=T, seed=5)
    if bad == "over":
        # x = -6000 d: the transform's first output is -128 * 6000 (c z = -67882,
        # below the most negative fp16), all the others 0; 6000 rounds to 6016
        # in bfloat16, still below
        k[1, 100, 3] = _to_dtype(-6000.0 * _signs(wl)[None], dtype)[0]
    else:
        k[1, 100, 3, 17] = float(bad)
    log(f"range case {bad} {axis} {dtype}")
    st, _ = oracle_encode(wl, to_u16(k), to_u16(v), T, L)
    assert st == O.RANGE
    plan = K.Plan(K.config_from_workload(wl, max_tokens=T, layers=L))
    ms, wsb = plan.sizes(T)
    out = torch.empty(ms, dtype=torch.uint8, device=DEV)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    with pytest.raises(K.KvcError) as e:
        plan.encode(k.to(DEV), v.to(DEV), T, out, ws)
    assert e.value.status == K.ERR_RANGE
    # the workspace status was cleared by the failing call's read-back: a
    # clean encode with the same buffers succeeds
    k2, v2 = W.dense_kv(wl, layers=L, tokens=T, seed=6)
    plan.encode(k2.to(DEV), v2.to(DEV), T, out, ws)
