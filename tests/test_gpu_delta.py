"""Token delta on the GPU (KVServe Sec. 5.1, the Delta transformer module):
dense streams with a delta run length on K, V or both equal the oracle's byte
for byte and decode to exactly the oracle's reconstruction, over both 16-bit
types, per-token and per-channel policies, run lengths from 2 to beyond the
token count, ragged token counts, compressible inputs and mixed-precision
plans; the paged calls refuse delta plans."""
import numpy as np
import pytest
import torch

import kv_cache_compression_kvc_amd as K
import kvc_workloads as W
import oracle_api as O
from gpu_helpers import (DEV, assert_encode_parity, chunk_kinds, compare_encode, gpu_decode, gpu_encode, log,
                         oracle_encode, to_u16)

pytestmark = pytest.mark.gpu

TP = W.TensorPolicy
C2 = W.WORKLOADS["c2_llama8b_4k"]
C3 = W.WORKLOADS["c3_llama70b_32k"]


def with_delta(wl, kd, vd, **kw):
    return wl.with_(k=TP(wl.k.bits, wl.k.axis, wl.k.group, delta=kd),
                    v=TP(wl.v.bits, wl.v.axis, wl.v.group, delta=vd), **kw)


def run_delta(wl, L, T, values="correlated", seed=1):
    log(f"delta case {wl.name} {wl.dtype} L={L} T={T} k={wl.k} v={wl.v} values={values}")
    if values == "zero_rich":
        k, v = W.zero_rich_kv(wl, L, T, seed=seed, zero_frac=0.5)
    else:
        k, v = W.correlated_kv(wl, L, T, seed=seed)
    ku, vu = to_u16(k), to_u16(v)
    st, ref = oracle_encode(wl, ku, vu, T, L)
    assert st == O.OK
    plan, got, ws = gpu_encode(wl, k.to(DEV), v.to(DEV), T, L)
    stats = compare_encode(got, ref, wl, L, T)
    stats["chunks_raw"], stats["chunks_compressed"] = chunk_kinds(ref, wl, L, T)
    log(f"  encode: {stats}")
    assert_encode_parity(stats)
    assert stats["identical"]
    n = L * T * wl.heads * wl.head_dim
    st, kd, vd = O.decode(ref, n)
    assert st == O.OK
    st, kg, vg = gpu_decode(plan, ref, wl, T, L)
    assert st == K.OK, K.status_string(st)
    assert np.array_equal(to_u16(kg).reshape(-1), kd)
    assert np.array_equal(to_u16(vg).reshape(-1), vd)
    return stats


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("kd,vd", [(16, 4), (0, 2), (64, 0), (32768, 32768)])
def test_delta_matches_oracle(dtype, kd, vd):
    run_delta(with_delta(C3, kd, vd, dtype=dtype, chunk_bytes=8192, name="delta"), 2, 300)


@pytest.mark.parametrize("T", [1, 33, 4096])
def test_delta_token_counts(T):
    run_delta(with_delta(C2, 8, 128, chunk_bytes=16384, name="delta_T"), 2, T)


def test_delta_compressible_input():
    s = run_delta(with_delta(C3, 32, 8, chunk_bytes=65536, name="delta_zero_rich"), 2, 1024, values="zero_rich")
    assert s["chunks_compressed"] > 0


def test_delta_empty_input():
    wl = with_delta(C3, 4, 4, name="delta_empty")
    plan = K.Plan(K.config_from_workload(wl, max_tokens=64, layers=2))
    ms, wsb = plan.sizes(0)
    out = torch.zeros(ms, dtype=torch.uint8, device=DEV)
    ws = torch.zeros(wsb, dtype=torch.uint8, device=DEV)
    k = torch.zeros((2, 0, wl.heads, 128), dtype=wl.torch_dtype, device=DEV)
    n = plan.encode(k, k, 0, out, ws)
    st, ref = oracle_encode(wl, np.zeros(0, np.uint16), np.zeros(0, np.uint16), 0, 2)
    assert st == O.OK and n == ref.size
    assert np.array_equal(out[:n].cpu().numpy(), ref)


def test_delta_mixed_precision():
    wl = with_delta(C3, 16, 16, chunk_bytes=8192, name="delta_mixed")
    L, T = 2, 200
    rng = np.random.default_rng(4)
    bits = rng.choice(np.array([2, 4, 8, 16], np.uint8), size=(2, L, wl.heads))
    k, v = W.correlated_kv(wl, L, T, seed=3)
    ku, vu = W.as_u16(k), W.as_u16(v)
    st, ref = O.encode_mixed(O.cfg_from_workload(wl, layers=L), bits, ku, vu, T)
    assert st == O.OK
    plan = K.Plan(K.config_from_workload(wl, max_tokens=T, layers=L), bits)
    ms, wsb = plan.sizes(T)
    out = torch.full((ms,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device=DEV)
    n = plan.encode(k.to(DEV), v.to(DEV), T, out, ws)
    assert n == ref.size and np.array_equal(out[:n].cpu().numpy(), ref)
    st, kd, vd = O.decode(ref, L * T * wl.heads * 128)
    assert st == O.OK
    st, kg, vg = gpu_decode(plan, ref, wl, T, L)
    assert st == K.OK, K.status_string(st)
    assert np.array_equal(to_u16(kg).reshape(-1), kd) and np.array_equal(to_u16(vg).reshape(-1), vd)


def test_stream_without_delta_is_a_plan_mismatch():
    wl = with_delta(C3, 0, 4, chunk_bytes=8192, name="delta_mismatch")
    L, T = 1, 64
    k, v = W.correlated_kv(wl, L, T, seed=2)
    plain = C3.with_(chunk_bytes=8192)
    st, ref = oracle_encode(plain, to_u16(k), to_u16(v), T, L)
    assert st == O.OK
    plan = K.Plan(K.config_from_workload(wl, max_tokens=T, layers=L))
    assert gpu_decode(plan, ref, wl, T, L)[0] == K.ERR_PLAN_MISMATCH


def test_paged_calls_refuse_delta_plans():
    wl = with_delta(W.WORKLOADS["c4_paged_llama8b"], 4, 0, layers=1)
    plan = K.Plan(K.config_from_workload(wl, max_tokens=64, layers=1))
    lens = np.array([16], np.int32)
    pool = torch.zeros((1, 1, wl.page_tokens, wl.heads, 128), dtype=wl.torch_dtype, device=DEV)
    bt = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    out = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    offs = torch.zeros(2, dtype=torch.int64, device=DEV)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    # refused on the host, before any kernel is launched
    with pytest.raises(K.KvcError) as e:
        plan.encode_paged(pool, pool, 1, bt, lens, out, offs, ws)
    assert e.value.status == K.ERR_UNSUPPORTED
    with pytest.raises(K.KvcError) as e:
        plan.decode_paged(out, 1 << 20, offs, lens, pool, pool, 1, bt, ws)
    assert e.value.status == K.ERR_UNSUPPORTED
