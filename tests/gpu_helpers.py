"""Helpers for the GPU parity tests: run the HIP library through its C ABI
and the oracle on the same input bytes, and compare the results by the
rules the task fixes (lossless bytes exact given equal codes; codes equal
except for at most 1e-5 of them, each off by one; reconstructed values within
1e-3 relative)."""
from __future__ import annotations

import struct
import sys

import numpy as np
import torch

import kv_cache_compression_kvc_amd as K
import kvc_workloads as W
import oracle_api as O

DEV = "cuda"


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def a16(x):
    return (x + 15) & ~15


def to_u16(t: torch.Tensor) -> np.ndarray:
    return W.as_u16(t.detach().cpu())


def gpu_encode(wl, k, v, T, layers, fill=0xA5):
    """Encode on the GPU; returns (plan, stream bytes as numpy, workspace)."""
    plan = K.Plan(K.config_from_workload(wl, max_tokens=max(T, 1), layers=layers))
    ms, wsb = plan.sizes(T)
    out = torch.full((ms,), fill, dtype=torch.uint8, device=DEV)     # garbage everywhere: padding must be written
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device=DEV)
    n = plan.encode(k, v, T, out, ws)
    torch.cuda.synchronize()
    return plan, out[:n].cpu().numpy(), ws


def gpu_decode(plan, stream_np: np.ndarray, wl, T, layers, ws=None):
    shape = (layers, T, wl.heads, wl.head_dim)
    s = torch.from_numpy(np.ascontiguousarray(stream_np)).to(DEV)
    if s.numel() == 0:
        s = torch.zeros(16, dtype=torch.uint8, device=DEV)
    k = torch.full(shape, 7, dtype=wl.torch_dtype, device=DEV)
    v = torch.full(shape, 7, dtype=wl.torch_dtype, device=DEV)
    if ws is None:
        _, wsb = plan.sizes(T)
        ws = torch.full((wsb,), 0x33, dtype=torch.uint8, device=DEV)
    plan.decode(s, stream_np.size, T, k, v, ws)
    torch.cuda.synchronize()
    ctl = ws[:32].cpu().numpy()
    st = plan.query_status(ws)
    if st != K.OK:
        log(f"  decode status {st}: control words {ctl.view(np.uint32)[:2].tolist()} "
            f"header-diag {ctl.view(np.uint64)[2]:#x}")
    torch.cuda.synchronize()
    return st, k, v


def oracle_encode(wl, k_u16, v_u16, T, layers):
    cfg = O.cfg_from_workload(wl, layers=layers)
    st, stream = O.encode(cfg, k_u16, v_u16, T)
    return st, stream


def split_stream(stream: np.ndarray, wl, L, T):
    """(codes[2], params[2]) of a stream, chunks decoded with the oracle."""
    cfg = O.cfg_from_workload(wl, layers=L)
    import ctypes as C
    codes_b = [O.lib().kvco_codes_bytes(C.byref(cfg), w, T) for w in range(2)]
    params_b = [O.lib().kvco_params_bytes(C.byref(cfg), w, T) for w in range(2)]
    cb = wl.chunk_bytes
    nch = [-(-c // cb) for c in codes_b]
    table = np.frombuffer(stream.tobytes(), np.uint32, sum(nch), 64)
    p0 = a16(64 + 4 * sum(nch))
    p1 = a16(p0 + params_b[0])
    pay = a16(p1 + params_b[1])
    stages = [O.STAGE_IDS[s] for s in wl.stages]
    codes = []
    pos, ci = pay, 0
    for w in range(2):
        out = np.zeros(codes_b[w], np.uint8)
        for i in range(nch[w]):
            n = min(cb, codes_b[w] - i * cb)
            e = int(table[ci])
            stored, raw = e & 0x7FFFFFFF, e >> 31
            st, dec = O.chunk_decode(stages, stream[pos:pos + stored], raw, n)
            assert st == O.OK, (w, i, st)
            out[i * cb:i * cb + n] = dec
            pos += a16(stored)
            ci += 1
        codes.append(out)
    params = [stream[p0:p0 + params_b[0]], stream[p1:p1 + params_b[1]]]
    return codes, params


def chunk_layout(stream: np.ndarray, wl, L, T):
    """Every chunk of a dense stream: (section, index, raw size, byte offset,
    stored size, raw flag)."""
    cfg = O.cfg_from_workload(wl, layers=L)
    import ctypes as C
    codes_b = [O.lib().kvco_codes_bytes(C.byref(cfg), w, T) for w in range(2)]
    params_b = [O.lib().kvco_params_bytes(C.byref(cfg), w, T) for w in range(2)]
    cb = wl.chunk_bytes
    nch = [-(-c // cb) for c in codes_b]
    table = np.frombuffer(stream.tobytes(), np.uint32, sum(nch), 64)
    pos = a16(a16(a16(64 + 4 * sum(nch)) + params_b[0]) + params_b[1])
    out, ci = [], 0
    for w in range(2):
        for i in range(nch[w]):
            e = int(table[ci])
            out.append((w, i, min(cb, codes_b[w] - i * cb), pos, e & 0x7FFFFFFF, e >> 31))
            pos += a16(e & 0x7FFFFFFF)
            ci += 1
    return out


def chunk_kinds(stream: np.ndarray, wl, L, T):
    """(raw, compressed) chunk counts of a stream, from its chunk table."""
    cfg = O.cfg_from_workload(wl, layers=L)
    import ctypes as C
    codes_b = [O.lib().kvco_codes_bytes(C.byref(cfg), w, T) for w in range(2)]
    nch = sum(-(-c // wl.chunk_bytes) for c in codes_b)
    table = np.frombuffer(stream.tobytes(), np.uint32, nch, 64)
    raw = int((table >> 31).sum())
    return raw, nch - raw


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    per = 8 // bits
    sh = np.arange(per, dtype=np.uint8) * bits
    return ((packed[:, None] >> sh[None, :]) & ((1 << bits) - 1)).reshape(-1)


def compare_encode(gpu: np.ndarray, ref: np.ndarray, wl, L, T):
    """Apply the parity rules; returns a dict of statistics."""
    stats = {"identical": bool(gpu.size == ref.size and np.array_equal(gpu, ref))}
    if stats["identical"]:
        stats.update(code_diffs=0, max_code_diff=0, param_diffs=0)
        return stats
    gc, gp = split_stream(gpu, wl, L, T)
    rc, rp = split_stream(ref, wl, L, T)
    nd, md, ncodes = 0, 0, 0
    for w, pol in enumerate((wl.k, wl.v)):
        a = unpack_codes(gc[w], pol.bits).astype(np.int16)
        b = unpack_codes(rc[w], pol.bits).astype(np.int16)
        d = np.abs(a - b)
        nd += int((d != 0).sum())
        md = max(md, int(d.max()) if d.size else 0)
        ncodes += a.size
    stats.update(code_diffs=nd, max_code_diff=md, ncodes=ncodes,
                 param_diffs=int(sum((gp[w] != rp[w]).sum() for w in range(2))))
    # with identical codes the lossless bytes must be identical too
    if nd == 0 and stats["param_diffs"] == 0:
        stats["lossless_mismatch"] = True
    return stats


def assert_encode_parity(stats):
    assert not stats.get("lossless_mismatch"), "codes equal but lossless bytes differ"
    if stats["identical"]:
        return
    # the fp16 (scale, minimum) words follow the same min / max rule on both
    # sides: they must be equal even where a code sits on a rounding tie
    assert stats["param_diffs"] == 0, stats
    assert stats["max_code_diff"] <= 1, stats
    assert stats["code_diffs"] <= 1e-5 * stats["ncodes"], stats


def assert_values_close(got_u16: np.ndarray, ref_u16: np.ndarray, dtype: str, D=128):
    """|a - b| <= 1e-3 * max(|b|, 1e-2 * rms(head vector)) elementwise."""
    if dtype == "f16":
        a = got_u16.view(np.float16).astype(np.float64)
        b = ref_u16.view(np.float16).astype(np.float64)
    else:
        a = torch.from_numpy(got_u16.view(np.int16)).view(torch.bfloat16).double().numpy()
        b = torch.from_numpy(ref_u16.view(np.int16)).view(torch.bfloat16).double().numpy()
    a = a.reshape(-1, D)
    b = b.reshape(-1, D)
    rms = np.sqrt((b * b).mean(axis=1, keepdims=True))
    tol = 1e-3 * np.maximum(np.abs(b), 1e-2 * rms)
    bad = np.abs(a - b) > tol
    assert not bad.any(), f"{int(bad.sum())} values outside tolerance, worst {np.abs(a - b)[bad].max()}"
    return float((got_u16 == ref_u16).mean())
