"""Parity at full workload sizes, in the launch configuration bench.py times.

The GPU encodes and decodes a whole workload; sampled layers (dense) or
requests (paged) are checked against the oracle, which encodes and decodes
just those samples: codes, parameters and chunk bytes of the GPU stream
must equal the oracle's for the sampled layer, and the reconstruction must
equal the oracle's bit for bit.  Inputs are generated on the GPU and the
sampled slices are copied to the host for the oracle.
"""
from __future__ import annotations

import ctypes as C
import gc
import time

import numpy as np
import pytest
import torch

import kv_cache_compression_kvc_amd as K
import kvc_workloads as W
import oracle_api as O
from gpu_helpers import DEV, log, split_stream, to_u16

pytestmark = pytest.mark.gpu


def a16(x):
    return (x + 15) & ~15


def free():
    gc.collect()
    torch.cuda.empty_cache()


def layer_slices(out: torch.Tensor, wl, L, T, layer, Tp):
    """(codes[2], params[2]) of the first Tp tokens of one layer of a dense GPU
    stream, chunks decoded with the oracle's chunk decoder.  Both code layouts
    and both parameter layouts keep a layer's tokens in order, so its first Tp
    tokens are a prefix of the layer's bytes equal to a (1 layer, Tp tokens)
    stream's sections."""
    cfg = O.cfg_from_workload(wl, layers=L)
    cfg1 = O.cfg_from_workload(wl, layers=1)
    lib = O.lib()
    cb = wl.chunk_bytes
    codes_b = [lib.kvco_codes_bytes(C.byref(cfg), w, T) for w in range(2)]
    params_b = [lib.kvco_params_bytes(C.byref(cfg), w, T) for w in range(2)]
    layer_codes = [lib.kvco_codes_bytes(C.byref(cfg1), w, T) for w in range(2)]
    layer_params = [lib.kvco_params_bytes(C.byref(cfg1), w, T) for w in range(2)]
    lcodes = [lib.kvco_codes_bytes(C.byref(cfg1), w, Tp) for w in range(2)]
    lparams = [lib.kvco_params_bytes(C.byref(cfg1), w, Tp) for w in range(2)]
    nch = [-(-c // cb) for c in codes_b]
    table = out[64:64 + 4 * sum(nch)].cpu().numpy().view(np.uint32)
    stored = (table & 0x7FFFFFFF).astype(np.int64)
    offs = np.concatenate([[0], np.cumsum((stored + 15) & ~15)])
    p0 = a16(64 + 4 * sum(nch))
    p1 = a16(p0 + params_b[0])
    pay = a16(p1 + params_b[1])
    stages = [O.STAGE_IDS[s] for s in wl.stages]
    codes, params = [], []
    for w in range(2):
        assert lcodes[w] % cb == 0 and layer_codes[w] % cb == 0
        first = layer * layer_codes[w] // cb
        g0 = (nch[0] if w else 0) + first
        g1 = g0 + lcodes[w] // cb
        span = out[pay + int(offs[g0]):pay + int(offs[g1])].cpu().numpy()      # one copy per section
        parts = []
        for gi in range(g0, g1):
            pos = int(offs[gi] - offs[g0])
            raw = bool(table[gi] >> 31)
            st, dec = O.chunk_decode(stages, span[pos:pos + int(stored[gi])], raw, cb)
            assert st == O.OK
            parts.append(dec)
        codes.append(np.concatenate(parts))
        base = (p0, p1)[w]
        params.append(out[base + layer * layer_params[w]:base + layer * layer_params[w] + lparams[w]].cpu().numpy())
    return codes, params


def check_dense_full(name, layers_to_check, Tp=None):
    wl = W.WORKLOADS[name]
    L, T = wl.layers, wl.tokens
    log(f"{name}: generating {L} x {T} x {wl.heads} x {wl.head_dim} {wl.dtype} on the GPU")
    k, v = W.dense_kv(wl, device=DEV)
    plan = K.Plan(K.config_from_workload(wl))
    ms, wsb = plan.sizes(T)
    out = torch.empty(ms, dtype=torch.uint8, device=DEV)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    n = plan.encode(k, v, T, out, ws)
    log(f"{name}: GPU stream {n} bytes")
    kd = torch.empty_like(k)
    vd = torch.empty_like(v)
    plan.decode(out, n, T, kd, vd, ws)
    assert plan.query_status(ws) == K.OK
    Tp = T if Tp is None else Tp
    for l in layers_to_check:
        t0 = time.time()
        log(f"{name}: layer {l}: oracle encode + decode of its first {Tp} tokens")
        ku, vu = to_u16(k[l:l + 1, :Tp]), to_u16(v[l:l + 1, :Tp])
        cfg1 = O.cfg_from_workload(wl, layers=1)
        st, ref = O.encode(cfg1, ku, vu, Tp)
        assert st == O.OK
        rc, rp = split_stream(ref, wl, 1, Tp)
        gc_, gp = layer_slices(out, wl, L, T, l, Tp)
        for w in range(2):
            assert np.array_equal(gc_[w], rc[w]), f"layer {l} section {w}: codes differ"
            assert np.array_equal(gp[w], rp[w]), f"layer {l} section {w}: parameters differ"
        st, kr, vr = O.decode(ref, Tp * wl.heads * wl.head_dim)
        assert st == O.OK
        assert np.array_equal(to_u16(kd[l:l + 1, :Tp]).reshape(-1), kr), f"layer {l}: K reconstruction differs"
        assert np.array_equal(to_u16(vd[l:l + 1, :Tp]).reshape(-1), vr), f"layer {l}: V reconstruction differs"
        log(f"{name}: layer {l} identical ({time.time() - t0:.1f} s)")
    del k, v, kd, vd, out, ws
    free()


def test_llama70b_32k_full_size_sampled_layers():
    check_dense_full("c3_llama70b_32k", [0, 79])


def test_llama70b_128k_full_size_sampled_layer():
    # one whole layer of 131072 tokens (both fp16 tensors, 268 MB of K+V)
    check_dense_full("c5_llama70b_128k", [37])


def stream_chunks(stream: np.ndarray, wl, L, T):
    """Per section: (table entries, byte offset of each chunk) of a dense stream."""
    cfg = O.cfg_from_workload(wl, layers=L)
    lib = O.lib()
    cb = wl.chunk_bytes
    codes_b = [lib.kvco_codes_bytes(C.byref(cfg), w, T) for w in range(2)]
    params_b = [lib.kvco_params_bytes(C.byref(cfg), w, T) for w in range(2)]
    nch = [-(-c // cb) for c in codes_b]
    table = np.frombuffer(stream[64:64 + 4 * sum(nch)].tobytes(), np.uint32)
    stored = (table & 0x7FFFFFFF).astype(np.int64)
    offs = np.concatenate([[0], np.cumsum((stored + 15) & ~15)])
    pay = a16(a16(a16(64 + 4 * sum(nch)) + params_b[0]) + params_b[1])
    return table, pay + offs, nch


def test_llama70b_32k_full_size_compressible_sampled_layers():
    # half of the 64-token blocks zero: nearly every one of the 30720 chunks
    # compresses, so the single-pass placement moves every chunk far below its
    # codes and the look-back scan chains 30 blocks; the sampled layers' chunk
    # table entries and stored chunk bytes must equal the oracle's
    wl = W.WORKLOADS["c3_llama70b_32k"]
    L, T = wl.layers, wl.tokens
    log(f"{wl.name}: generating zero-rich {L} x {T} x {wl.heads} x {wl.head_dim} on the GPU")
    k, v = W.zero_rich_kv(wl, L, T, seed=W.SEED_BASE + 7, device=DEV, zero_frac=0.5)
    plan = K.Plan(K.config_from_workload(wl))
    ms, wsb = plan.sizes(T)
    out = torch.empty(ms, dtype=torch.uint8, device=DEV)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    n = plan.encode(k, v, T, out, ws)
    log(f"{wl.name}: GPU stream {n} bytes (CR {wl.uncompressed_bytes() / n:.3f})")
    kd = torch.empty_like(k)
    vd = torch.empty_like(v)
    plan.decode(out, n, T, kd, vd, ws)
    assert plan.query_status(ws) == K.OK
    gtab, gpos, gnch = stream_chunks(out[:1 << 18].cpu().numpy(), wl, L, T)      # header + chunk table
    assert int(gpos[-1]) == n, "chunk offsets must end at the stream size"
    compressed = int(np.count_nonzero((gtab >> 31) == 0))
    log(f"{wl.name}: {compressed} of {len(gtab)} chunks compressed")
    assert compressed > len(gtab) // 2
    for l in (0, 41, 79):
        t0 = time.time()
        ku, vu = to_u16(k[l:l + 1]), to_u16(v[l:l + 1])
        st, ref = O.encode(O.cfg_from_workload(wl, layers=1), ku, vu, T)
        assert st == O.OK
        rtab, rpos, rnch = stream_chunks(ref, wl, 1, T)
        for w in range(2):
            g0 = (gnch[0] if w else 0) + l * rnch[w]
            r0 = rnch[0] if w else 0
            assert np.array_equal(gtab[g0:g0 + rnch[w]], rtab[r0:r0 + rnch[w]]), f"layer {l} section {w}: table"
            gb = out[int(gpos[g0]):int(gpos[g0 + rnch[w]])].cpu().numpy()
            rb = ref[int(rpos[r0]):int(rpos[r0 + rnch[w]])]
            assert np.array_equal(gb, rb), f"layer {l} section {w}: chunk bytes differ"
        st, kr, vr = O.decode(ref, T * wl.heads * wl.head_dim)
        assert st == O.OK
        assert np.array_equal(to_u16(kd[l:l + 1]).reshape(-1), kr), f"layer {l}: K reconstruction differs"
        assert np.array_equal(to_u16(vd[l:l + 1]).reshape(-1), vr), f"layer {l}: V reconstruction differs"
        log(f"{wl.name}: layer {l} identical ({time.time() - t0:.1f} s)")
    del k, v, kd, vd, out, ws
    free()


def test_paged_llama8b_full_size_every_request():
    """The whole paged batch (64 requests, 1024..16384 tokens, pages scattered
    over the pool) encoded and decoded in one call each.  Every request is
    checked on the GPU: its gathered pages encoded by a one-request dense call
    must give its stream byte for byte, and that stream's dense decode must
    equal what the paged decode scattered through the second page map.  The
    shortest, a median and the longest request are also compared with the
    oracle (stream bytes and reconstruction), in parallel host threads."""
    from concurrent.futures import ThreadPoolExecutor
    wl = W.WORKLOADS["c4_paged_llama8b"]
    batch = W.paged_layout(wl)
    R = len(batch.seq_lens)
    t0 = time.time()
    log(f"c4: {R} requests, {batch.num_blocks} pages, generating pools on the GPU")
    kp, vp = W.paged_pools(wl, batch, device=DEV)
    torch.cuda.synchronize()
    log(f"c4: pools ready ({time.time() - t0:.1f} s)")
    plan = K.Plan(K.config_from_workload(wl, max_tokens=0))
    ms, wsb = plan.sizes_paged(batch.seq_lens)
    out = torch.empty(ms, dtype=torch.uint8, device=DEV)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    offs = torch.zeros(R + 1, dtype=torch.int64, device=DEV)
    bt = torch.from_numpy(batch.block_table).to(DEV)
    n = plan.encode_paged(kp, vp, batch.num_blocks, bt, batch.seq_lens, out, offs, ws)
    log(f"c4: GPU streams {n} bytes ({time.time() - t0:.1f} s)")
    dst = W.paged_layout(wl, stream=1)
    kq = torch.zeros_like(kp)
    vq = torch.zeros_like(vp)
    btd = torch.from_numpy(dst.block_table).to(DEV)
    plan.decode_paged(out, n, offs, dst.seq_lens, kq, vq, dst.num_blocks, btd, ws)
    assert plan.query_status(ws) == K.OK
    offs_h = offs.cpu().numpy()
    assert int(offs_h[R]) == n
    P = wl.page_tokens

    def gather(pool, table, r, T):
        npg = (T + P - 1) // P
        blocks = table[r, :npg].long()
        return pool[:, blocks].reshape(wl.layers, npg * P, wl.heads, wl.head_dim)[:, :T].contiguous()

    order = np.argsort(batch.seq_lens, kind="stable")
    sample = [int(order[0]), int(order[R // 2]), int(order[-1])]
    inputs = {r: (to_u16(gather(kp, bt, r, int(batch.seq_lens[r]))),
                  to_u16(gather(vp, bt, r, int(batch.seq_lens[r])))) for r in sample}
    cfg = O.cfg_from_workload(wl)

    def oracle_job(r):
        T = int(batch.seq_lens[r])
        st, ref = O.encode(cfg, inputs[r][0], inputs[r][1], T)
        st2, kr, vr = O.decode(ref, wl.layers * T * wl.heads * wl.head_dim)
        return st, ref, st2, kr, vr

    pool = ThreadPoolExecutor(max_workers=len(sample))          # the oracle's ctypes calls release the GIL
    futs = {r: pool.submit(oracle_job, r) for r in sample}
    log(f"c4: oracle running on requests {sample} ({[int(batch.seq_lens[r]) for r in sample]} tokens)")

    for r in range(R):
        T = int(batch.seq_lens[r])
        kin, vin = gather(kp, bt, r, T), gather(vp, bt, r, T)
        p1 = K.Plan(K.config_from_workload(wl, max_tokens=T))
        ms1, ws1 = p1.sizes(T)
        o1 = torch.empty(ms1, dtype=torch.uint8, device=DEV)
        w1 = torch.empty(ws1, dtype=torch.uint8, device=DEV)
        n1 = p1.encode(kin, vin, T, o1, w1)
        assert n1 == int(offs_h[r + 1] - offs_h[r]), f"request {r}: stream size differs"
        assert torch.equal(o1[:n1], out[int(offs_h[r]):int(offs_h[r + 1])]), f"request {r}: stream differs"
        kd, vd = torch.empty_like(kin), torch.empty_like(vin)
        p1.decode(o1, n1, T, kd, vd, w1)
        assert p1.query_status(w1) == K.OK
        assert torch.equal(kd.view(torch.int16), gather(kq, btd, r, T).view(torch.int16)), f"request {r}: K pages"
        assert torch.equal(vd.view(torch.int16), gather(vq, btd, r, T).view(torch.int16)), f"request {r}: V pages"
        del kin, vin, kd, vd, o1, w1
    log(f"c4: all {R} requests equal their dense encodes and decodes ({time.time() - t0:.1f} s)")

    for r in sample:
        T = int(batch.seq_lens[r])
        st, ref, st2, kr, vr = futs[r].result()
        assert st == O.OK and st2 == O.OK
        got = out[int(offs_h[r]):int(offs_h[r + 1])].cpu().numpy()
        assert np.array_equal(got, ref), f"request {r}: stream differs from the oracle's"
        assert np.array_equal(to_u16(gather(kq, btd, r, T)).reshape(-1), kr), f"request {r}: K reconstruction"
        assert np.array_equal(to_u16(gather(vq, btd, r, T)).reshape(-1), vr), f"request {r}: V reconstruction"
        log(f"c4: request {r} ({T} tokens) identical to the oracle ({time.time() - t0:.1f} s)")
    pool.shutdown()
    del kp, vp, kq, vq, out, ws
    free()
