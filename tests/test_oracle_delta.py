"""Pins for the oracle's token delta (KVServe Sec. 5.1 lists Delta, from
CacheGen, among the pre-quantization transforms; the pages name it only).
The reading pinned here: runs of D tokens from token 0 in each (layer, head);
the run's first token is kept; the others become their difference from it,
rounded to the 16-bit type; decoding adds the anchor back.

The pins use values whose differences and sums the arithmetic fixes by hand
(integers and dyadic fractions, one round-to-nearest tie), round trips that
must be exact when every difference is representable, the stream header, and
the whole stream: constant runs decode to their anchor's value exactly, and a
delta stream's sections are those of a plain stream of the transformed
input."""
import struct

import numpy as np
import pytest

import kvc_workloads as W
import oracle_api as O

C1 = W.WORKLOADS["c1_single_layer_512"]


def tiny_cfg(dtype="f16", k_delta=0, v_delta=0, heads=1, head_dim=16):
    wl = C1.with_(heads=heads, head_dim=head_dim, dtype=dtype,
                  k=W.TensorPolicy(4, "token", 16, delta=k_delta),
                  v=W.TensorPolicy(2, "token", 16, delta=v_delta), chunk_bytes=4096)
    return wl, O.cfg_from_workload(wl, layers=1)


def f16_bits(a):
    return np.asarray(a, np.float16).view(np.uint16)


def test_differences_from_the_run_anchor_by_hand():
    # x_t[d] = t + d / 4 (exact in fp16); runs of 4: anchors 0 and 4, so token
    # t holds (t mod 4) in every channel, token 4 keeps its own values
    wl, cfg = tiny_cfg(k_delta=4)
    T = 6
    x = np.array([[t + d / 4 for d in range(16)] for t in range(T)], np.float32)
    st, y = O.delta_forward(cfg, 0, f16_bits(x), T)
    assert st == O.OK
    y = y.reshape(T, 16).view(np.float16).astype(np.float32)
    want = np.array([x[0], np.full(16, 1.0), np.full(16, 2.0), np.full(16, 3.0), x[4], np.full(16, 1.0)])
    assert np.array_equal(y, want)
    # runs of 2: every odd token holds 1
    wl, cfg = tiny_cfg(k_delta=2)
    st, y = O.delta_forward(cfg, 0, f16_bits(x), T)
    y = y.reshape(T, 16).view(np.float16).astype(np.float32)
    assert np.array_equal(y[1::2], np.ones((3, 16)))
    assert np.array_equal(y[0::2], x[0::2])


def test_difference_rounds_to_nearest_even_in_bf16():
    # 512 - 1 = 511 lies half-way between the bf16 neighbours 510 and 512;
    # ties go to the even significand, 512 (0x4400).  And 512 - 2.5 = 509.5
    # lies nearer 510 (0x43FF) than 508
    wl, cfg = tiny_cfg(dtype="bf16", v_delta=2)
    x = np.zeros((4, 16), np.float32)
    x[0], x[1], x[2], x[3] = 1.0, 512.0, 2.5, 512.0
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    st, y = O.delta_forward(cfg, 1, bits, 4)
    assert st == O.OK
    y = y.reshape(4, 16)
    assert (y[1] == 0x4400).all() and (y[3] == 0x43FF).all()
    assert (y[0] == bits[0]).all() and (y[2] == bits[2]).all()


def test_heads_and_layers_have_their_own_anchors():
    # [layers=2][tokens=4][heads=2][16]: value = 100 l + 10 h + t; with runs of
    # 4 every non-anchor entry is t, independent of layer and head
    wl = C1.with_(heads=2, head_dim=16, k=W.TensorPolicy(4, "token", 16, delta=4),
                  v=W.TensorPolicy(2, "token", 16), chunk_bytes=4096)
    cfg = O.cfg_from_workload(wl, layers=2)
    x = np.zeros((2, 4, 2, 16), np.float32)
    for l in range(2):
        for t in range(4):
            for h in range(2):
                x[l, t, h] = 100 * l + 10 * h + t
    st, y = O.delta_forward(cfg, 0, f16_bits(x), 4)
    y = y.reshape(2, 4, 2, 16).view(np.float16).astype(np.float32)
    for t in range(1, 4):
        assert (y[:, t] == t).all()
    assert np.array_equal(y[:, 0], x[:, 0])
    # V has no delta: unchanged
    st, yv = O.delta_forward(cfg, 1, f16_bits(x), 4)
    assert np.array_equal(yv, f16_bits(x).reshape(-1))


@pytest.mark.parametrize("run", [2, 8, 64])
def test_inverse_undoes_forward_when_the_arithmetic_is_exact(run):
    # small integers: every difference and sum is exact in fp16
    rng = np.random.default_rng(run)
    wl, cfg = tiny_cfg(k_delta=run, heads=3)
    T = 150
    x = rng.integers(-300, 300, size=(T, 3, 16)).astype(np.float32)
    bits = f16_bits(x).reshape(-1)
    st, y = O.delta_forward(cfg, 0, bits, T)
    assert st == O.OK
    assert not np.array_equal(y, bits)
    st, back = O.delta_inverse(cfg, 0, y, T)
    assert st == O.OK and np.array_equal(back, bits)


def test_run_length_validation():
    for bad in (1, 3, 6, 65536):
        wl, cfg = tiny_cfg(k_delta=bad)
        st, _ = O.delta_forward(cfg, 0, np.zeros(16, np.uint16), 1)
        assert st == O.INVALID_ARG
    wl, cfg = tiny_cfg(k_delta=32768)
    assert O.delta_forward(cfg, 0, np.zeros(16, np.uint16), 1)[0] == O.OK


def test_header_carries_the_run_lengths():
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(k=W.TensorPolicy(4, "channel", 64, delta=16),
                                              v=W.TensorPolicy(2, "token", 32, delta=256), chunk_bytes=8192)
    k, v = W.dense_kv(wl, layers=1, tokens=70)
    cfg = O.cfg_from_workload(wl, layers=1)
    st, stream = O.encode(cfg, W.as_u16(k), W.as_u16(v), 70)
    assert st == O.OK
    assert struct.unpack_from("<H", stream.tobytes(), 30)[0] == 16
    assert struct.unpack_from("<H", stream.tobytes(), 38)[0] == 256
    st, info, T = O.stream_info(stream)
    assert st == O.OK and info.k_delta == 16 and info.v_delta == 256 and T == 70


def test_constant_runs_decode_to_their_anchor_exactly():
    # every token of a run equal to its anchor: the non-anchor vectors become
    # zero, a zero per-token group reconstructs to zero, and adding the anchor
    # back gives the anchor's reconstruction exactly
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(k=W.TensorPolicy(4, "token", 32, delta=8),
                                              v=W.TensorPolicy(2, "token", 32, delta=16), chunk_bytes=8192)
    L, T = 2, 100
    k, v = W.dense_kv(wl, layers=L, tokens=T)
    ku, vu = W.as_u16(k).reshape(L, T, wl.heads, 128), W.as_u16(v).reshape(L, T, wl.heads, 128)
    for x, run in ((ku, 8), (vu, 16)):
        for t in range(T):
            x[:, t] = x[:, t - t % run]
    cfg = O.cfg_from_workload(wl, layers=L)
    st, stream = O.encode(cfg, ku.reshape(-1), vu.reshape(-1), T)
    assert st == O.OK
    st, kd, vd = O.decode(stream, L * T * wl.heads * 128)
    assert st == O.OK
    for d, run in ((kd.reshape(L, T, wl.heads, 128), 8), (vd.reshape(L, T, wl.heads, 128), 16)):
        for t in range(T):
            assert np.array_equal(d[:, t], d[:, t - t % run]), t


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_delta_stream_quantizes_the_transformed_input(dtype):
    # the transform comes before the quantizer and the lossless backend: a
    # delta stream's parameters and payload are those of a plain stream of the
    # transformed tensors, and its decode is the plain decode with the anchors
    # added back
    base = W.WORKLOADS["c3_llama70b_32k"].with_(dtype=dtype, chunk_bytes=8192)
    wl = base.with_(k=W.TensorPolicy(base.k.bits, base.k.axis, base.k.group, delta=32),
                    v=W.TensorPolicy(base.v.bits, base.v.axis, base.v.group, delta=4))
    L, T = 2, 90
    k, v = W.correlated_kv(wl, L, T, seed=5)
    ku, vu = W.as_u16(k).reshape(-1), W.as_u16(v).reshape(-1)
    cfg = O.cfg_from_workload(wl, layers=L)
    st, s_delta = O.encode(cfg, ku, vu, T)
    assert st == O.OK
    ky, vy = O.delta_forward(cfg, 0, ku, T)[1], O.delta_forward(cfg, 1, vu, T)[1]
    pcfg = O.cfg_from_workload(base, layers=L)
    st, s_plain = O.encode(pcfg, ky, vy, T)
    assert st == O.OK
    assert s_delta.size == s_plain.size
    assert np.array_equal(s_delta[64:], s_plain[64:])
    n = L * T * wl.heads * 128
    st, kd, vd = O.decode(s_delta, n)
    st2, kp, vp = O.decode(s_plain, n)
    assert st == O.OK and st2 == O.OK
    assert np.array_equal(kd, O.delta_inverse(cfg, 0, kp, T)[1])
    assert np.array_equal(vd, O.delta_inverse(cfg, 1, vp, T)[1])
