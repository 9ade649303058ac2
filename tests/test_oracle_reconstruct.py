"""Pins for the oracle's reconstruction, its per-channel layout, and the
special values of the group extremes.

Reconstruction follows FastKVComp ("Beyond Compression Ratio: High-Throughput
KV Compression for Disaggregated LLM Serving", Sec. 4.1, "Fused
Reconstruction"): dequantization, inverse Hadamard transformation,
normalization and sign restoration, in that order.  The pin feeds codes and
parameters chosen so that the dequantized values and every partial sum of the
transform are exact in binary32; the only roundings left are the product with
c = fl32(1/sqrt(128)) and the final conversion to the 16-bit dtype.  The
expected output is then computed without the oracle: an integer Sylvester
matrix product, one binary64 product (exact: 24 x 20 bits), one rounding to
binary32 by numpy, the sign, and numpy's (fp16) or torch's (bf16) rounding.
Folding c into the parameters before the transform (another order) changes
the rounding of about one element in 2^13 (fp16) and is caught here.

The codes and parameters are packed by this file's own reading of the
stream layouts (per-token codes [L][T][H][D] packed along head_dim,
parameters [L][T][H][D/G]; per-channel codes [L][ceil(T/G)][H][D][ceil(Gg*b/8)]
packed along the group's tokens, parameters [L][ceil(T/G)][H][D]; each
parameter an fp16 (scale, minimum) pair), so the dequantizer's addressing is
pinned by the same comparison.
"""
import numpy as np
import pytest
import torch

import kvc_workloads as W
import oracle_api as O
from test_oracle_hadamard import sylvester

C128 = np.float32(1.0 / np.sqrt(128.0))
D = 128
TP = W.TensorPolicy


def pack_lsb(q: np.ndarray, bits: int) -> np.ndarray:
    """Codes (last axis) packed LSB-first, 8 / bits per byte; a partial last
    byte is zero-padded."""
    per = 8 // bits
    n = q.shape[-1]
    pad = (-n) % per
    qq = np.concatenate([q, np.zeros(q.shape[:-1] + (pad,), q.dtype)], axis=-1).astype(np.uint8)
    qq = qq.reshape(q.shape[:-1] + (-1, per))
    out = np.zeros(qq.shape[:-1], np.uint8)
    for k in range(per):
        out |= (qq[..., k] << (bits * k)).astype(np.uint8)
    return out


def dyadic_params(rng, shape, exp=-8):
    """fp16 (scale, minimum) with few significant bits: s = js 2^exp,
    m = -im 2^exp (js in [1, 255], im in [0, 1023])."""
    js = rng.integers(1, 256, shape)
    im = rng.integers(0, 1024, shape)
    s = (js * 2.0 ** exp).astype(np.float16)
    m = (-im * 2.0 ** exp).astype(np.float16)
    m[im == 0] = np.float16(0.0)                   # +0, not -0
    assert np.all(s.astype(np.float64) == js * 2.0 ** exp) and np.all(m.astype(np.float64) == -im * 2.0 ** exp)
    return js, im, s, m


def params_bytes(s: np.ndarray, m: np.ndarray) -> np.ndarray:
    pair = np.stack([s.view(np.uint16), m.view(np.uint16)], axis=-1)
    return np.ascontiguousarray(pair).reshape(-1).view(np.uint8)


def expected_reconstruction(w_int: np.ndarray, exp: int, dtype: str, signs: np.ndarray) -> np.ndarray:
    """w_int [..., D]: dequantized values / 2^exp (integers).  Returns 16-bit
    patterns of d * RN16(RN32(c * (H w)))."""
    Hs = sylvester(D).astype(np.int64)
    v = w_int.astype(np.int64) @ Hs.T                 # exact
    assert np.abs(v).max() < 2 ** 29
    y = (np.float64(C128) * v.astype(np.float64) * 2.0 ** exp).astype(np.float32)   # one rounding
    y = y * signs.astype(np.float32)                  # exact
    if dtype == "f16":
        return y.astype(np.float16).view(np.uint16)
    return torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("bits,group", [(4, 32), (2, 128), (8, 16)])
def test_per_token_reconstruction_order_exact(dtype, bits, group):
    wl = W.WORKLOADS["c1_single_layer_512"].with_(dtype=dtype, k=TP(bits, "token", group))
    L, T, H = 1, 512, 8
    rng = np.random.default_rng([bits, group, len(dtype)])
    q = rng.integers(0, 1 << bits, (L, T, H, D))
    js, im, s, m = dyadic_params(rng, (L, T, H, D // group))
    codes = pack_lsb(q, bits).reshape(-1)
    params = params_bytes(s, m)
    cfg = O.cfg_from_workload(wl)
    st, got = O.dequantize_tensor(cfg, 0, codes, params, T)
    assert st == O.OK
    jsx = np.repeat(js, group, axis=-1)
    imx = np.repeat(im, group, axis=-1)
    w_int = q * jsx - imx
    d = O.signs(wl.sign_seed, D)
    ref = expected_reconstruction(w_int.reshape(-1, D), -8, dtype, d)
    assert np.array_equal(got.reshape(-1, D), ref), int((got.reshape(-1, D) != ref).sum())


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("bits,group,T", [(4, 64, 150), (2, 64, 200), (8, 32, 70), (2, 32, 250)])
def test_per_channel_reconstruction_order_and_layout_exact(dtype, bits, group, T):
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(dtype=dtype, heads=2, k=TP(bits, "channel", group))
    L, H = 2, 2
    ng = -(-T // group)
    rng = np.random.default_rng([bits, group, T, len(dtype)])
    q = rng.integers(0, 1 << bits, (L, T, H, D))
    js, im, s, m = dyadic_params(rng, (L, ng, H, D))
    parts = []
    for l in range(L):
        for g in range(ng):
            t0, t1 = g * group, min(T, (g + 1) * group)
            col = np.transpose(q[l, t0:t1], (1, 2, 0))          # [H][D][tokens of the group]
            parts.append(pack_lsb(col, bits).reshape(-1))
    codes = np.concatenate(parts)
    params = params_bytes(s, m)
    cfg = O.cfg_from_workload(wl, layers=L)
    st, got = O.dequantize_tensor(cfg, 0, codes, params, T)
    assert st == O.OK
    gidx = np.arange(T) // group
    w_int = q * js[:, gidx] - im[:, gidx]
    d = O.signs(wl.sign_seed, D)
    ref = expected_reconstruction(w_int.reshape(-1, D), -8, dtype, d)
    assert np.array_equal(got.reshape(-1, D), ref), int((got.reshape(-1, D) != ref).sum())


def test_per_channel_layout_against_direct_computation():
    """Per-channel codes and parameters land where the format puts them: each
    (layer, group, head, channel) column is recomputed from transform outputs
    checked against the dense Sylvester product, and found at
    codes[layer base + g*H*D*colb(G) + (h*D + ch)*colb(Gg)] (packed along the
    group's tokens) and params[((l*NG + g)*H + h)*D + ch]; T = 150 leaves a
    last group of 22 tokens (11 code bytes per column at 4 bits)."""
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(heads=2, dtype="f16")
    L, T, H, G, bits = 2, 150, 2, 64, 4
    k, _ = W.dense_kv(wl, layers=L, tokens=T)
    x = W.as_u16(k)
    cfg = O.cfg_from_workload(wl, layers=L)
    st, codes, params = O.quantize_tensor(cfg, 0, x, T)
    assert st == O.OK
    ng = -(-T // G)
    colb = [-(-min(G, T - g * G) * bits // 8) for g in range(ng)]
    layer_bytes = H * D * sum(colb)
    assert codes.size == L * layer_bytes and params.size == L * ng * H * D * 4
    d = O.signs(wl.sign_seed, D).astype(np.float32)
    Hs = sylvester(D).astype(np.float64)
    xv = x.view(np.float16).astype(np.float32).reshape(L, T, H, D)
    z = np.empty((L, T, H, D), np.float32)
    for l in range(L):
        for t in range(T):
            for h in range(H):
                v = xv[l, t, h] * d
                z[l, t, h] = O.fwht(v)
                assert np.max(np.abs(z[l, t, h] - Hs @ v.astype(np.float64))) < 1e-3
    p16 = params.view(np.uint16)
    for l in range(L):
        for g in range(ng):
            t0, t1 = g * G, min(T, (g + 1) * G)
            base = l * layer_bytes + g * H * D * colb[0]
            for h in range(H):
                for ch in range(0, D, 7):                     # every 7th channel, both ends of a column
                    zg = z[l, t0:t1, h, ch]
                    _, s, m, inv = O.group_params(zg, bits, float(C128))
                    gi = ((l * ng + g) * H + h) * D + ch
                    assert p16[2 * gi] == s and p16[2 * gi + 1] == m, (l, g, h, ch)
                    _, q = O.quantize_group(zg, bits, float(C128), s, m, inv)
                    off = base + (h * D + ch) * colb[g]
                    col = codes[off:off + colb[g]]
                    nib = np.stack([col & 15, col >> 4], axis=1).reshape(-1)
                    assert np.array_equal(nib[:t1 - t0], q), (l, g, h, ch)
                    assert np.all(nib[t1 - t0:] == 0)          # padding nibble of an odd group


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_signed_zero_extremes_use_plus_zero(bits):
    """-0 and +0 are one real value; a group whose minimum is -0 gets the
    minimum +0 (0x0000), never -0 (0x8000), whatever the order of the
    elements; a group of zeros of both signs gets scale 0 and minimum +0."""
    for z in ([-0.0, 0.5, 1.0], [0.5, -0.0, 1.0, 0.0], [0.0, -0.0], [-0.0, -0.0, -0.0], [-0.0, 0.0, 3.0]):
        for c in (1.0, float(C128)):
            st, s, m, inv = O.group_params(np.array(z, np.float32), bits, c)
            assert st == O.OK
            assert m == 0x0000, (z, hex(m))
            if max(z) == 0.0:
                assert s == 0 and inv == 0.0
    # a negative maximum of -0 is the same range as +0
    st, s, m, _ = O.group_params(np.array([-1.0, -0.0], np.float32), bits, 1.0)
    st2, s2, m2, _ = O.group_params(np.array([-1.0, 0.0], np.float32), bits, 1.0)
    assert (st, s, m) == (st2, s2, m2) and m == 0xBC00          # -1.0


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_nonfinite_group_values_are_range_errors(bad):
    for pos in (0, 5, 31):
        z = np.linspace(-1, 1, 32).astype(np.float32)
        z[pos] = bad
        for bits in (2, 4, 8):
            assert O.group_params(z, bits, float(C128))[0] == O.RANGE, (bad, pos, bits)


@pytest.mark.parametrize("bad", [np.nan, np.inf])
@pytest.mark.parametrize("axis", ["token", "channel"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_nonfinite_input_is_a_range_error(bad, axis, dtype):
    """One non-finite input value anywhere (here one channel of one token)
    makes the tensor's encode report a range error, for both axes: under
    per-channel groups the other 63 tokens of the group are finite."""
    pol = TP(4, axis, 64 if axis == "channel" else 32)
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(dtype=dtype, heads=2, k=pol, v=pol)
    L, T = 1, 128
    k, v = W.dense_kv(wl, layers=L, tokens=T)
    k[0, 70, 1, 9] = bad
    cfg = O.cfg_from_workload(wl, layers=L)
    st, _, _ = O.quantize_tensor(cfg, 0, W.as_u16(k), T)
    assert st == O.RANGE
    st, _, _ = O.quantize_tensor(cfg, 1, W.as_u16(v), T)
    assert st == O.OK
    st, _ = O.encode(cfg, W.as_u16(k), W.as_u16(v), T)
    assert st == O.RANGE
