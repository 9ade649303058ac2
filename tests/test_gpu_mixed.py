"""Mixed precision per (layer, head) on the GPU (KVServe Sec. 5.1 mechanism):
the stream of a mixed plan equals the oracle's byte for byte and decodes to
exactly the oracle's reconstruction, for per-token and per-channel policies,
ragged token counts, every width including 16-bit passthrough, and
compressible inputs; a stream is rejected by a plan whose widths differ."""
import dataclasses

import numpy as np
import pytest
import torch

import kv_cache_compression_kvc_amd as K
import kvc_workloads as W
import oracle_api as O
from gpu_helpers import DEV, log, to_u16

pytestmark = pytest.mark.gpu


def run_mixed(wl, L, T, bits, values="dense", seed=0):
    if values == "zero_rich":
        k, v = W.zero_rich_kv(wl, L, T, seed=seed, zero_frac=0.5)
    else:
        k, v = W.dense_kv(wl, layers=L, tokens=T)
    ku, vu = W.as_u16(k), W.as_u16(v)
    log(f"{wl.name} L={L} T={T} widths K {np.bincount(bits[0].reshape(-1), minlength=17)[[2, 4, 8, 16]].tolist()} "
        f"V {np.bincount(bits[1].reshape(-1), minlength=17)[[2, 4, 8, 16]].tolist()} values {values}")
    st, ref = O.encode_mixed(O.cfg_from_workload(wl, layers=L), bits, ku, vu, T)
    assert st == O.OK
    plan = K.Plan(K.config_from_workload(wl, max_tokens=max(T, 1), layers=L), bits)
    ms, wsb = plan.sizes(T)
    assert ms == O.lib().kvco_max_stream_bytes_mixed(O.C.byref(O.cfg_from_workload(wl, layers=L)),
                                                      np.ascontiguousarray(bits).ctypes.data, T)
    kd, vd = k.to(DEV), v.to(DEV)
    out = torch.full((ms,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device=DEV)
    n = plan.encode(kd, vd, T, out, ws)
    got = out[:n].cpu().numpy()
    assert n == ref.size, (n, ref.size)
    assert np.array_equal(got, ref)
    st, kr, vr = O.decode(ref, L * T * wl.heads * wl.head_dim)
    assert st == O.OK
    ko = torch.full_like(kd, 7)
    vo = torch.full_like(vd, 7)
    plan.decode(out, n, T, ko, vo, ws)
    assert plan.query_status(ws) == K.OK
    assert np.array_equal(to_u16(ko).reshape(-1), kr)
    assert np.array_equal(to_u16(vo).reshape(-1), vr)
    return plan, out, n


def widths(rng, L, H, choices=(2, 4, 8, 16)):
    return rng.choice(choices, size=(2, L, H)).astype(np.uint8)


@pytest.mark.parametrize("name,L,T", [("c3_llama70b_32k", 2, 200), ("c3_llama70b_32k", 2, 256),
                                      ("c1_single_layer_512", 1, 77), ("c2_llama8b_4k", 3, 130),
                                      ("c5_llama70b_128k", 1, 321)])
def test_mixed_random_widths(name, L, T):
    wl = W.WORKLOADS[name]
    run_mixed(wl, L, T, widths(np.random.default_rng(L * 1000 + T), L, wl.heads))


def test_mixed_single_width_and_passthrough_only():
    wl = W.WORKLOADS["c3_llama70b_32k"]
    L, T = 2, 192
    run_mixed(wl, L, T, np.full((2, L, wl.heads), 16, np.uint8))
    run_mixed(wl, L, T, np.full((2, L, wl.heads), 8, np.uint8))


def test_mixed_head_pattern_compressible():
    """A MixHQ-like pattern: two heads of every layer at 8 bits, the rest at 2,
    on zero-rich values so chunks compress."""
    wl = W.WORKLOADS["c3_llama70b_32k"]
    L, T = 3, 1024
    bits = np.full((2, L, wl.heads), 2, np.uint8)
    bits[:, :, :2] = 8
    run_mixed(wl, L, T, bits, values="zero_rich", seed=9)


def test_mixed_stream_rejected_by_other_plan():
    wl = W.WORKLOADS["c1_single_layer_512"]
    L, T = 1, 96
    bits = widths(np.random.default_rng(4), L, wl.heads)
    plan, out, n = run_mixed(wl, L, T, bits)
    other = bits.copy()
    other[0, 0, 0] = 4 if bits[0, 0, 0] != 4 else 8
    cfg = K.config_from_workload(wl, max_tokens=T, layers=L)
    for p2 in (K.Plan(cfg, other), K.Plan(cfg)):
        _, wsb = p2.sizes(T)
        ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
        k = torch.zeros((L, T, wl.heads, wl.head_dim), dtype=wl.torch_dtype, device=DEV)
        v = torch.zeros_like(k)
        p2.decode(out, n, T, k, v, ws)
        assert p2.query_status(ws) in (K.ERR_PLAN_MISMATCH, K.ERR_CORRUPT_STREAM)
