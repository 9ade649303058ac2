#!/usr/bin/env python3
"""Throughput of the KV-cache compression path on one MI355X.

A step is one pass of the whole path over one batch of synthetic KV:
fused transform + quantize (K and V), lossless encode, scan and placement,
then lossless decode and fused reconstruction of the produced stream.  The
headline workload is the Llama-3.1-70B-shaped cache at 32768 tokens (80
layers x 8 KV heads x 128, bf16, K int4 per-channel groups of 64 tokens, V
int2 per-token groups of 32, lossless TUPL8_1 -> BIT_8 -> RZE_2), with all
inputs resident in HBM before timing starts.

Prints one JSON line.  `value` is uncompressed K+V bytes per second of a
whole headline step (encode + decode).  `sub_results` carries the other
workloads measured the same way: the headline shape on zero-rich KV (the
lossless stage compresses), the 131072-token 70B shape as one call and as
a layer-by-layer pipeline on two streams, and the paged 64-request batch.
Per-kernel times come from HIP events the library records around each
launch on its stream, averaged over the timed steps.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E peak
METRIC = "KV encode / decode GB/s (uncompressed bytes) + % HBM peak, compression ratio"
TIMING_NOTE = ("per-kernel ms: HIP events recorded by the library around each launch on its stream, "
               "averaged over the timed steps")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def fused_bytes_per_elem(pol):
    # read 2 B, write bits/8 B of codes and 4 B of parameters per group
    return 2.0 + pol.bits / 8.0 + 4.0 / pol.group


def counted_traffic(kind: str):
    """HBM bytes per launch of a fused kernel as counted by rocprofv3
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's counts), taken from the
    committed profile summary of the headline workload; None when that
    summary was made from a different version of the kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "fused_codec_llama70b_32k_hbm_bytes.json")
    src = os.path.join(ROOT, "kv_cache_compression_kvc_amd", "csrc", "kvc_codec.hip")
    try:
        with open(path) as f:
            js = json.load(f)
        with open(src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    k = js.get("kernels", {}).get(kind)
    if js.get("codec_sha256") != sha or not k:
        return None
    return {"read_bytes": round(k["read_bytes"]), "write_bytes": round(k["write_bytes"]),
            "bytes": round(k["read_bytes"] + k["write_bytes"])}


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(wl, layers: int, threads: int):
    """The oracle as it stands on the first `layers` layers of the workload
    (same value model, generated on the host): once on one thread, then on
    `threads` threads, each encoding and decoding its own layers (the oracle's
    ctypes calls release the interpreter lock; its arithmetic is unchanged)."""
    from concurrent.futures import ThreadPoolExecutor
    import kvc_workloads as W
    import oracle_api as O
    k, v = W.dense_kv(wl, layers=layers, device="cpu")
    ku, vu = W.as_u16(k), W.as_u16(v)
    n_layer = wl.tokens * wl.heads * wl.head_dim
    U = wl.uncompressed_bytes() / wl.layers * layers
    cfg = O.cfg_from_workload(wl, layers=layers)
    t0 = time.perf_counter()
    st, s = O.encode(cfg, ku, vu, wl.tokens)
    t1 = time.perf_counter()
    st2, _, _ = O.decode(s, layers * n_layer)
    t2 = time.perf_counter()
    assert st == O.OK and st2 == O.OK
    one = {"value": round(U / (t2 - t0) / 1e9, 6), "unit": "GB/s", "cores": 1,
           "encode_GBps": round(U / (t1 - t0) / 1e9, 6), "decode_GBps": round(U / (t2 - t1) / 1e9, 6),
           "seconds": round(t2 - t0, 2)}
    cfg1 = O.cfg_from_workload(wl, layers=1)
    kl = ku.reshape(layers, -1)
    vl = vu.reshape(layers, -1)

    def layer_job(l):
        a = time.perf_counter()
        st_, s_ = O.encode(cfg1, kl[l], vl[l], wl.tokens)
        b = time.perf_counter()
        st2_, _, _ = O.decode(s_, n_layer)
        c = time.perf_counter()
        assert st_ == O.OK and st2_ == O.OK
        return b - a, c - b

    reps = max(1, (threads + layers - 1) // layers)       # at least one layer per thread
    jobs = [l for _ in range(reps) for l in range(layers)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        t0 = time.perf_counter()
        res = list(ex.map(layer_job, jobs))
        t1 = time.perf_counter()
    Ua = U * reps
    enc_cpu = sum(r[0] for r in res)
    dec_cpu = sum(r[1] for r in res)
    wall = t1 - t0
    return {"value": round(Ua / wall / 1e9, 6), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"layers 0..{layers - 1} of the workload ({U / 1e9:.3f} GB of K+V) x {reps}, encode + decode, "
                      f"one (layer, repeat) per task on {threads} threads",
            "encode_GBps": round(Ua / wall / 1e9 * (enc_cpu + dec_cpu) / enc_cpu, 6),
            "decode_GBps": round(Ua / wall / 1e9 * (enc_cpu + dec_cpu) / dec_cpu, 6),
            "seconds": round(wall, 2), "single_thread": one,
            "host_cpu": host_cpu(), "host_logical_cpus": os.cpu_count()}


def selection_cost(U: float, s_enc: float, s_dec: float, cr: float, requests: int = 20000) -> dict:
    """Host cost of the service-aware controller (KVServe Sec. 6.2) per request:
    one choose + observe on the library's selector, with this run's measured
    profile and two derived ones (quantization only at twice the ratio and
    half the speed, and the reverse) in one bucket, over a sweep of link
    speeds around the profile's break-even bandwidth."""
    import random
    import kv_cache_compression_kvc_amd as K
    profs = [(0, 0, cr, s_enc, s_dec), (1, 0, 2 * cr, s_enc / 2, s_dec / 2), (2, 0, max(1.01, cr / 2), 2 * s_enc, 2 * s_dec)]
    sel = K.Selector(profs, epsilon=0.1, seed=1)
    rng = random.Random(0)
    bstar = K.break_even_bandwidth(cr, s_enc, s_dec)
    ctxs = [(0, bstar * 10 ** rng.uniform(-2, 0.5), U, 0.05, 1e9) for _ in range(requests)]
    t0 = time.perf_counter()
    for c in ctxs:
        pid, pred = sel.choose(*c)
        sel.observe(*c, pid, pred * 1.05)
    dt = time.perf_counter() - t0
    env = sel.envelope(0)
    sel.close()
    return {"us_per_request": round(dt / requests * 1e6, 3), "requests": requests,
            "break_even_bandwidth_GBps": round(bstar / 1e9, 1),
            "envelope": [{"profile": i, "from_GBps": (None if x == 0.0 else round(1 / x / 1e9, 1))}
                         for i, x in zip(*env)],
            "note": "python ctypes calls included; profile -1 = raw transfer"}


def mixed_widths(pattern: str, wl):
    """[2][layers][heads] widths of a named mixed-precision pattern (None = uniform)."""
    if pattern == "none":
        return None
    import numpy as np
    hi = 8 if pattern == "mixhq" else 16
    b = np.full((2, wl.layers, wl.heads), 2, np.uint8)
    b[:, :, :2] = hi
    return b


def mixed_bytes(widths, pol, elems: int) -> float:
    """Algorithmic bytes of one tensor's fused encode (or decode) under a width
    map: 2 bytes read per element, and per element b/8 code bytes plus a
    4-byte parameter word per group (16-bit heads: 2 bytes written)."""
    import numpy as np
    w = np.asarray(widths).reshape(-1)
    per_head = elems / w.size
    total = 0.0
    for b in w:
        total += per_head * (2.0 + (2.0 if b == 16 else b / 8.0 + 4.0 / pol.group))
    return total


# Figures the pages report for their own implementation, with the hardware
# they name (other machines: context, not a target for this metric).
PAGES_FIGURES = {
    "fused_transform_quantize_speedup": {
        "value": "up to 5.9x", "over": "separate transform and quantize kernels",
        "hardware": "NVIDIA RTX 5090 (local setup) and RTX PRO 6000 / H100 (remote setup); the figure is not tied to one"},
    "lossless_backend_GBps": {"before": "< 90 (nvCOMP integration)", "after": "> 500 (searched LC pipeline)",
                              "hardware": "as above"},
    "complete_path_table1": {
        "RTX PRO 6000, fused + LC": {"compression_ratio": 6.276, "comp_GBps": 139.218, "decomp_GBps": 155.841},
        "H100, fused + LC": {"compression_ratio": 6.280, "comp_GBps": 91.606, "decomp_GBps": 103.104}},
}


def gbps(nbytes: float, ms: float) -> float:
    return nbytes / (ms * 1e-3) / 1e9 if ms > 0 else 0.0


def kern(ms: float, nbytes: float) -> dict:
    g = gbps(nbytes, ms)
    return {"ms": round(ms, 4), "algorithmic_bytes": round(nbytes), "GBps": round(g, 1),
            "frac": round(g / HBM_PEAK_GBPS, 4)}


def chunk_stats(out, wl, L: int, T: int, plan_layout) -> dict:
    """Per code section of a dense stream: chunks, compressed chunks, their
    raw and stored bytes, the raw chunks the placement moves, and the bytes
    the section occupies in the stream (from the chunk table)."""
    import numpy as np
    codes_b, nch = plan_layout
    table = out[64:64 + 4 * sum(nch)].cpu().numpy().view(np.uint32)
    cb = wl.chunk_bytes
    secs = []
    allraw_pos = 0
    pos = 0
    gi = 0
    for w in range(2):
        n = np.minimum(cb, codes_b[w] - np.arange(nch[w], dtype=np.int64) * cb)
        e = table[gi:gi + nch[w]]
        raw = (e >> 31).astype(bool)
        stored = (e & 0x7FFFFFFF).astype(np.int64)
        a16 = (stored + 15) & ~15
        start = pos + np.concatenate([[0], np.cumsum(a16)[:-1]])
        start_raw = allraw_pos + np.concatenate([[0], np.cumsum((n + 15) & ~15)[:-1]])
        moved = raw & (start != start_raw)
        secs.append({"chunks": int(nch[w]), "compressed": int((~raw).sum()),
                     "compressed_raw_bytes": int(n[~raw].sum()), "compressed_stored_bytes": int(stored[~raw].sum()),
                     "moved_raw_bytes": int(n[moved].sum()), "stored_bytes": int(stored.sum()),
                     "raw_bytes": int(n.sum()), "sizes": n, "stored": stored, "raw": raw})
        pos += int(a16.sum())
        allraw_pos += int(((n + 15) & ~15).sum())
        gi += nch[w]
    return {"sections": secs}


def layout_of(wl, L: int, T: int):
    """Code bytes and chunk counts of the two sections of a dense stream (the
    closed-form layout the format defines)."""
    out = []
    for pol in (wl.k, wl.v):
        H, D = wl.heads, wl.head_dim
        if pol.axis == "token":
            c = L * T * H * D * pol.bits // 8
        else:
            ng = -(-T // pol.group)
            glast = T - (ng - 1) * pol.group
            c = L * ((ng - 1) * H * D * (pol.group * pol.bits // 8) + H * D * (-(-glast * pol.bits // 8)))
        out.append(c)
    return out, [-(-c // wl.chunk_bytes) for c in out]


def timed(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def timed_steps(fn, steps, stream):
    """(ms per call over all `steps` calls, [ms of each call]): one event
    before the first call, one after each call, all on `stream`, so the total
    is the same bracket as timed()'s."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    each = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, each


def spread(each) -> dict:
    """min, median and max of per-step times (ms)."""
    xs = sorted(each)
    n = len(xs)
    med = xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])
    return {"min": round(xs[0], 4), "median": round(med, 4), "max": round(xs[-1], 4)}


def profiled(fn, steps, warmup, stream):
    """(ms per call of fn, {kernel kind: ms per launch}, [ms of each call])
    over `steps` timed calls."""
    import torch
    import kv_cache_compression_kvc_amd as K
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    K.profile_reset()
    K.profile_enable(True)
    ms, each = timed_steps(fn, steps, stream)
    K.profile_enable(False)
    prof = {name: K.profile_query(name) for name in K.KERNELS}
    return ms, {k: t / c for k, (t, c) in prof.items() if c}, each


class Dense:
    """One dense workload resident on the GPU: inputs, outputs, stream and
    workspace, and its plan."""

    def __init__(self, wl, values: str, zero_frac: float = 0.5, rho: float = 0.95, bits=None):
        import torch
        import kv_cache_compression_kvc_amd as K
        import kvc_workloads as W
        self.wl = wl
        L, T = wl.layers, wl.tokens
        self.L, self.T = L, T
        dev = torch.device("cuda:0")
        log(f"generating {wl.name} ({values}): {L} x {T} x {wl.heads} x {wl.head_dim} {wl.dtype}")
        if values == "gaussian":
            self.k, self.v = W.dense_kv(wl, device=dev)
        elif values == "correlated":
            self.k, self.v = W.correlated_kv(wl, L, T, W.SEED_BASE + 7, device=dev, rho=rho)
        else:
            self.k, self.v = W.zero_rich_kv(wl, L, T, seed=W.SEED_BASE + 7, device=dev, zero_frac=zero_frac)
        self.bits = bits
        self.plan = K.Plan(K.config_from_workload(wl), bits)
        self.ms, wsb = self.plan.sizes(T)
        self.out = torch.empty(self.ms, dtype=torch.uint8, device=dev)
        self.ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        self.kd = torch.empty_like(self.k)
        self.vd = torch.empty_like(self.v)
        self.U = wl.uncompressed_bytes()
        self.elems = L * T * wl.heads * wl.head_dim
        torch.cuda.synchronize()
        self.n = self.plan.encode(self.k, self.v, T, self.out, self.ws)          # synchronous: size and status
        self.plan.decode(self.out, self.n, T, self.kd, self.vd, self.ws)
        st = self.plan.query_status(self.ws)
        assert st == K.OK, K.status_string(st)
        log(f"stream {self.n} bytes, ratio {self.U / self.n:.4f}")

    def encode(self):
        self.plan.encode(self.k, self.v, self.T, self.out, self.ws, sync=False)

    def decode(self):
        self.plan.decode(self.out, self.ms, self.T, self.kd, self.vd, self.ws)

    def step(self):
        self.encode()
        self.decode()

    def fused_bytes(self):
        wl, bits, elems = self.wl, self.bits, self.elems
        per_k = elems * fused_bytes_per_elem(wl.k) if bits is None else mixed_bytes(bits[0], wl.k, elems)
        per_v = elems * fused_bytes_per_elem(wl.v) if bits is None else mixed_bytes(bits[1], wl.v, elems)
        return {"ENCODE_K": per_k, "ENCODE_V": per_v, "DECODE_K": per_k, "DECODE_V": per_v}

    def codes_params(self):
        wl, bits, elems = self.wl, self.bits, self.elems
        total = 0.0
        for w, pol in enumerate((wl.k, wl.v)):
            if bits is None:
                total += elems * (pol.bits / 8.0 + 4.0 / pol.group)
            else:
                total += mixed_bytes(bits[w], pol, elems) - 2.0 * elems
        return total

    def measure(self, steps, warmup):
        """Step, encode-only and decode-only times and per-kernel figures."""
        import torch
        s = torch.cuda.current_stream()
        step_ms, kms, each = profiled(self.step, steps, warmup, s)
        enc_ms = timed(self.encode, steps, 2, s)
        dec_ms = timed(self.decode, steps, 2, s)
        import kv_cache_compression_kvc_amd as K
        st = self.plan.query_status(self.ws)
        assert st == K.OK, K.status_string(st)
        U, n = self.U, self.n
        cp = self.codes_params()
        fb = self.fused_bytes()
        kernels = {}
        for k_, ms_ in kms.items():
            kernels[k_] = kern(ms_, fb[k_]) if k_ in fb else {"ms": round(ms_, 4)}
        for name, a_, b_ in (("ENCODE_K+V", "ENCODE_K", "ENCODE_V"), ("DECODE_K+V", "DECODE_K", "DECODE_V")):
            if a_ in kms and b_ in kms:
                kernels[name] = kern(kms[a_] + kms[b_], fb[a_] + fb[b_])
        s_enc, s_dec = gbps(U, enc_ms), gbps(U, dec_ms)
        s_p = s_enc * s_dec / (s_enc + s_dec)
        return {"uncompressed_bytes": U, "ms_per_step": round(step_ms, 4), "step_ms_spread": spread(each),
                "GBps": round(gbps(U, step_ms), 3),
                "encode_ms": round(enc_ms, 4), "encode_GBps": round(s_enc, 3),
                "encode_frac_hbm_peak": round(s_enc / HBM_PEAK_GBPS, 4),
                "decode_ms": round(dec_ms, 4), "decode_GBps": round(s_dec, 3),
                "decode_frac_hbm_peak": round(s_dec / HBM_PEAK_GBPS, 4),
                "compression_ratio": round(U / n, 4), "compression_ratio_quant": round(U / cp, 4),
                "compression_ratio_lossless": round(cp / n, 4), "stream_bytes": n,
                "harmonic_s_p_GBps": round(s_p, 3), "break_even_bandwidth_GBps": round((1 - n / U) * s_p, 3),
                "kernels": kernels}, kms

    def lossless_kernels(self, kms) -> dict:
        """Algorithmic bytes of the lossless kernels of a step, from the
        stream's chunk table: the placement reads each compressed chunk's codes
        and writes its stored bytes, and moves raw chunks whose offset changed;
        the lossless decode pass reads and expands the compressed chunks the
        reconstruct kernels do not decode themselves (2-bit per-token values of
        TUPL8_1 -> BIT_8 -> RZE_2 in whole 4 KiB blocks are decoded by the
        value reconstruct kernel), and the value reconstruct then reads the
        stored bytes of its section in place of the raw codes."""
        wl = self.wl
        cs = chunk_stats(self.out, wl, self.L, self.T, layout_of(wl, self.L, self.T))["sections"]
        place = sum(s["compressed_raw_bytes"] + s["compressed_stored_bytes"] + 2 * s["moved_raw_bytes"] for s in cs)
        std = tuple(wl.stages) == ("TUPL8_1", "BIT_8", "RZE_2")
        dec = 0
        mirror = [std and pol.axis == "token" and pol.bits == 2 and wl.chunk_bytes % 4096 == 0 for pol in (wl.k, wl.v)]
        for w, s in enumerate(cs):
            comp = ~s["raw"]
            if mirror[w]:
                comp = comp & (s["sizes"] % 4096 != 0)
            dec += int(s["sizes"][comp].sum()) + int(s["stored"][comp].sum())
        out = {"chunks": sum(s["chunks"] for s in cs), "compressed_chunks": sum(s["compressed"] for s in cs)}
        if "COMPACT" in kms:
            out["COMPACT (single-pass placement)"] = kern(kms["COMPACT"], place)
        if "LOSSLESS_DEC" in kms:
            out["LOSSLESS_DEC"] = kern(kms["LOSSLESS_DEC"], dec)
        if mirror[1] and "DECODE_V" in kms:
            pol = wl.v
            v_read = cs[1]["stored_bytes"] + self.elems * 4.0 / pol.group
            out["DECODE_V (reads stored chunks)"] = kern(kms["DECODE_V"], v_read + 2.0 * self.elems)
        return out

    def release(self):
        for a in ("k", "v", "kd", "vd", "out", "ws"):
            setattr(self, a, None)


def layer_pipeline(d: Dense, steps, warmup) -> dict:
    """One-layer calls: layer l is encoded on stream A into its own stream
    buffer; stream B waits for that encode's event and decodes it, so B's
    decode of layer l overlaps A's encode of layer l + 1."""
    import torch
    import kv_cache_compression_kvc_amd as K
    wl, L, T, U = d.wl, d.L, d.T, d.U
    s = torch.cuda.current_stream()
    p1 = K.Plan(K.config_from_workload(wl, layers=1))
    ms1, ws1 = p1.sizes(T)
    bufs = torch.empty((L, ms1), dtype=torch.uint8, device=d.k.device)
    wa = torch.empty(ws1, dtype=torch.uint8, device=d.k.device)
    wb = torch.empty(ws1, dtype=torch.uint8, device=d.k.device)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    evs = [torch.cuda.Event() for _ in range(L)]

    def pipe(do_enc=True, do_dec=True):
        base = torch.cuda.current_stream()             # the capturing stream under graph capture
        sa.wait_stream(base)
        sb.wait_stream(base)
        for l in range(L):
            if do_enc:
                p1.encode(d.k[l], d.v[l], T, bufs[l], wa, sync=False, stream=sa)
                evs[l].record(sa)
            if do_dec:
                if do_enc:
                    sb.wait_event(evs[l])
                p1.decode(bufs[l], ms1, T, d.kd[l], d.vd[l], wb, stream=sb)
        base.wait_stream(sa)
        base.wait_stream(sb)

    pipe_ms = timed(pipe, steps, warmup, s)
    enc1_ms = timed(lambda: pipe(True, False), steps, 2, s)
    dec1_ms = timed(lambda: pipe(False, True), steps, 2, s)
    assert p1.query_status(wa) == K.OK and p1.query_status(wb) == K.OK
    # host time to enqueue one pass (the calls return without waiting)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    pipe()
    host_ms = (time.perf_counter() - h0) * 1e3
    torch.cuda.synchronize()
    # the same pass captured once in a HIP graph (both streams and the events
    # between them) and replayed: a serving loop's form without the host's
    # per-call launch cost
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(s)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            pipe()
    s.wait_stream(side)
    torch.cuda.synchronize()
    graph_ms = timed(g.replay, steps, 2, s)
    assert p1.query_status(wa) == K.OK and p1.query_status(wb) == K.OK
    del g, bufs, wa, wb
    return {"ms_per_step": round(pipe_ms, 4), "GBps": round(gbps(U, pipe_ms), 3),
            "encode_ms": round(enc1_ms, 4), "encode_GBps": round(gbps(U, enc1_ms), 3),
            "decode_ms": round(dec1_ms, 4), "decode_GBps": round(gbps(U, dec1_ms), 3),
            "host_enqueue_ms": round(host_ms, 3),
            "graph_replay": {"ms_per_step": round(graph_ms, 4), "GBps": round(gbps(U, graph_ms), 3)},
            "calls": f"{L} one-layer encodes on one stream, {L} one-layer decodes on another, "
                     "each decode after its layer's encode (an event)"}


def paged(wl, steps, warmup) -> dict:
    """The paged batch: every request's pages gathered by the fused encoder
    into its own stream (one call), then decoded and scattered into a second
    pool through an independent page map (one call)."""
    import torch
    import kv_cache_compression_kvc_amd as K
    import kvc_workloads as W
    dev = torch.device("cuda:0")
    batch = W.paged_layout(wl)
    dst = W.paged_layout(wl, stream=1)
    R = len(batch.seq_lens)
    log(f"generating {wl.name}: {R} requests, {batch.num_blocks} pages of {wl.page_tokens} tokens")
    kp, vp = W.paged_pools(wl, batch, device=dev)
    kq, vq = torch.zeros_like(kp), torch.zeros_like(vp)
    plan = K.Plan(K.config_from_workload(wl, max_tokens=0))
    ms, wsb = plan.sizes_paged(batch.seq_lens)
    out = torch.empty(ms, dtype=torch.uint8, device=dev)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    offs = torch.zeros(R + 1, dtype=torch.int64, device=dev)
    bt = torch.from_numpy(batch.block_table).to(dev)
    btd = torch.from_numpy(dst.block_table).to(dev)
    n = plan.encode_paged(kp, vp, batch.num_blocks, bt, batch.seq_lens, out, offs, ws)
    toks = int(batch.seq_lens.sum())
    U = 2 * wl.layers * toks * wl.heads * wl.head_dim * 2
    elems = wl.layers * toks * wl.heads * wl.head_dim

    def enc():
        plan.encode_paged(kp, vp, batch.num_blocks, bt, batch.seq_lens, out, offs, ws, sync=False)

    def dec():
        plan.decode_paged(out, n, offs, dst.seq_lens, kq, vq, dst.num_blocks, btd, ws)

    s = torch.cuda.current_stream()
    enc_ms, ke, _ = profiled(enc, steps, warmup, s)
    dec_ms, kd, _ = profiled(dec, steps, warmup, s)
    st = plan.query_status(ws)
    assert st == K.OK, K.status_string(st)
    fb = {"ENCODE_K": elems * fused_bytes_per_elem(wl.k), "ENCODE_V": elems * fused_bytes_per_elem(wl.v),
          "DECODE_K": elems * fused_bytes_per_elem(wl.k), "DECODE_V": elems * fused_bytes_per_elem(wl.v)}
    kernels = {}
    for k_, ms_ in list(ke.items()) + list(kd.items()):
        kernels[k_] = kern(ms_, fb[k_]) if k_ in fb else {"ms": round(ms_, 4)}
    cp = elems * (wl.k.bits / 8 + 4 / wl.k.group + wl.v.bits / 8 + 4 / wl.v.group)
    res = {"requests": R, "tokens": toks, "pages": batch.num_blocks, "uncompressed_bytes": U,
           "encode_ms": round(enc_ms, 4), "encode_GBps": round(gbps(U, enc_ms), 3),
           "encode_frac_hbm_peak": round(gbps(U, enc_ms) / HBM_PEAK_GBPS, 4),
           "decode_ms": round(dec_ms, 4), "decode_GBps": round(gbps(U, dec_ms), 3),
           "decode_frac_hbm_peak": round(gbps(U, dec_ms) / HBM_PEAK_GBPS, 4),
           "compression_ratio": round(U / n, 4), "compression_ratio_quant": round(U / cp, 4),
           "compression_ratio_lossless": round(cp / n, 4), "stream_bytes": n, "kernels": kernels}
    del kp, vp, kq, vq, out, ws
    return res


def bandwidth_probes(total_bytes: int = 4 << 30, reps: int = 5) -> dict:
    """What HBM gives a kernel that only streams 16-byte lines with
    non-temporal stores: read-only, write-only, copy, and the read:write
    mixes of the fused encoders (about 4:1) and decoders (about 1:4).  Each
    mix is measured with default-policy loads from a capped, looping grid
    (how most fused kernels load) and with non-temporal loads from one
    short-lived wave per 256 items (the fastest pattern found); "best" is the
    faster of the two.  GB/s counts bytes read plus bytes written."""
    import torch
    import kv_cache_compression_kvc_amd as K
    dev = torch.device("cuda:0")
    a = torch.empty(total_bytes, dtype=torch.uint8, device=dev)
    b = torch.empty(total_bytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream()
    out = {}
    for r, w in ((1, 0), (0, 1), (1, 1), (4, 1), (1, 4)):
        items = total_bytes // (16 * max(r, w))
        row = {}
        for tag, flags in (("default", 0), ("nt_short", K.PROBE_NT_LOADS | K.PROBE_SHORT_WAVES)):
            fn = lambda: K.probe_bandwidth(a, b, items, r, w, sink, s, flags=flags)
            ms = timed(fn, reps, 2, s)
            row[tag] = round(items * 16 * (r + w) / (ms * 1e-3) / 1e9, 1)
        best = max(row.values())
        out[f"{r}:{w}"] = {"GBps": row["default"], "frac": round(row["default"] / HBM_PEAK_GBPS, 4),
                           "nt_short_GBps": row["nt_short"], "best_frac": round(best / HBM_PEAK_GBPS, 4)}
    del a, b, sink
    return out


SUB_RESULTS = ("llama70b_32k_zero_rich", "llama70b_128k", "llama8b_paged_64_requests")


def sub_result(name: str, ss: int, sw: int) -> dict:
    """One sub-result of the default run, measured in this process."""
    import kvc_workloads as W
    if name == "llama70b_32k_zero_rich":
        # the headline shape on zero-rich KV: the lossless stage compresses
        dz = Dense(W.WORKLOADS["c3_llama70b_32k"], "zero_rich", 0.5)
        r, kz = dz.measure(ss, sw)
        r["values"] = "half of the 64-token blocks of each (layer, head) zero"
        r["lossless_kernels"] = dz.lossless_kernels(kz)
        return r
    if name == "llama70b_128k":
        # the 131072-token 70B shape (fp16, int2 K and V): one call, then a layer pipeline
        d5 = Dense(W.WORKLOADS["c5_llama70b_128k"], "gaussian")
        r, _ = d5.measure(ss, sw)
        r["layer_pipeline"] = layer_pipeline(d5, max(2, ss // 2), 1)
        return r
    if name == "llama8b_paged_64_requests":
        return paged(W.WORKLOADS["c4_paged_llama8b"], max(2, ss // 2), 1)
    raise SystemExit(f"unknown sub-result {name}")


def free():
    import torch
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3_llama70b_32k")
    ap.add_argument("--cpu-layers", type=int, default=8, help="layers of the oracle's timed sample")
    ap.add_argument("--cpu-threads", type=int, default=0, help="threads of the oracle's all-cores run (0: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sub", action="store_true", help="measure the headline workload only")
    ap.add_argument("--sub-steps", type=int, default=0, help="timed steps of each sub-result (0: min(steps, 10))")
    ap.add_argument("--sub-in-process", action="store_true",
                    help="measure the sub-results in this process, one after another (for a single-process "
                         "profiler trace of the whole run)")
    ap.add_argument("--sub-only", choices=["llama70b_32k_zero_rich", "llama70b_128k", "llama8b_paged_64_requests"],
                    default=None, help="measure one sub-result and print it as one JSON line (the default run "
                                       "runs each sub-result this way, in a child process)")
    ap.add_argument("--values", choices=["gaussian", "zero_rich", "correlated"], default="gaussian",
                    help="value model: the workload's Gaussian KV (headline), KV whose 64-token blocks "
                         "are zero with probability --zero-frac, or KV correlated along tokens (AR(1), "
                         "--rho); the last two exercise compressing chunks")
    ap.add_argument("--zero-frac", type=float, default=0.5)
    ap.add_argument("--rho", type=float, default=0.95)
    ap.add_argument("--mixed", choices=["none", "mixhq", "mixhq16"], default="none",
                    help="mixed precision per (layer, head): mixhq = heads 0-1 of every layer at 8 bits and the "
                         "others at 2 bits (K and V); mixhq16 = heads 0-1 kept at 16 bits, the others at 2")
    ap.add_argument("--overlap", action="store_true",
                    help="also time the headline workload as a layer pipeline on two streams")
    ap.add_argument("--layers", type=int, default=0, help="override the layer count (e.g. 1: one layer per call)")
    ap.add_argument("--heads", type=int, default=0,
                    help="override kv_heads (e.g. 1: one tensor-parallel rank's share of the 70B shape at TP = 8)")
    ap.add_argument("--delta", default="0:0",
                    help="token-delta run lengths K:V before the transform (0 = none, the headline)")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30,
                    help="size of the plain device copy timed as the practical bandwidth reference")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the compression path runs on one device and has no "
              "multi-GPU mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import kvc_workloads as W

    if args.sub_only:
        # one sub-result, printed for the parent run to collect
        r = sub_result(args.sub_only, args.sub_steps or min(args.steps, 10), min(args.warmup, 3))
        log(f"{args.sub_only}: encode {r['encode_GBps']:.1f} GB/s, decode {r['decode_GBps']:.1f} GB/s, CR "
            f"{r['compression_ratio']:.3f}")
        print(json.dumps(r), flush=True)
        return

    # plain device copy of known size: practical bandwidth reference, and the
    # kernel whose counters scale the HBM byte counts of the profile runs
    ca = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda:0")
    cb = torch.empty_like(ca)
    cb.copy_(ca)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        cb.copy_(ca)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * args.copy_bytes * 5 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    log(f"device copy of {args.copy_bytes} bytes: {copy_gbps:.1f} GB/s (read + write)")
    del ca, cb
    probes = bandwidth_probes()
    log("bandwidth reference (reads:writes of 16-byte lines): " +
        ", ".join(f"{k_} {v_['GBps']:.0f} GB/s" for k_, v_ in probes.items()))

    wl = W.WORKLOADS[args.workload]
    dk, dv = (int(x) for x in args.delta.split(":"))
    if dk or dv:
        import dataclasses
        wl = wl.with_(k=dataclasses.replace(wl.k, delta=dk), v=dataclasses.replace(wl.v, delta=dv))
    if args.heads:
        wl = wl.with_(heads=args.heads)
    if args.layers:
        wl = wl.with_(layers=args.layers)
    bits = mixed_widths(args.mixed, wl)
    d = Dense(wl, args.values, args.zero_frac, args.rho, bits)
    L, T, U = d.L, d.T, d.U
    head, kms = d.measure(args.steps, args.warmup)
    s = torch.cuda.current_stream()
    log(f"step {head['ms_per_step']:.3f} ms; per-kernel ms/launch: " +
        ", ".join(f"{k_}={v_:.3f}" for k_, v_ in kms.items()))

    # the same step captured once in a HIP graph and replayed (a serving loop's
    # form: the dense calls enqueue kernels only)
    graph_ms = None
    if bits is None:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(s)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                d.step()
        s.wait_stream(side)
        torch.cuda.synchronize()
        graph_ms = timed(g.replay, args.steps, 2, s)
        import kv_cache_compression_kvc_amd as K
        st = d.plan.query_status(d.ws)
        assert st == K.OK, K.status_string(st)
        del g
        log(f"graph replay {graph_ms:.3f} ms per step")
    log(f"encode {head['encode_ms']:.3f} ms ({head['encode_GBps']:.1f} GB/s), "
        f"decode {head['decode_ms']:.3f} ms ({head['decode_GBps']:.1f} GB/s)")
    overlap = layer_pipeline(d, args.steps, args.warmup) if (args.overlap and bits is None) else None

    # roofline of the dominant fused kernel, algorithmic bytes per launch
    fb = d.fused_bytes()
    dom = max((k_ for k_ in fb if k_ in kms), key=lambda k_: kms[k_])
    achieved = gbps(fb[dom], kms[dom])
    headline = (args.workload == "c3_llama70b_32k" and args.values == "gaussian" and args.mixed == "none"
                and not (dk or dv) and not args.heads and not args.layers)
    result = {
        "metric": METRIC,
        "value": head["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "step_ms_spread": head["step_ms_spread"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": {"gaussian": "synthetic", "zero_rich": f"synthetic-zero-rich-{args.zero_frac}",
                 "correlated": f"synthetic-correlated-rho-{args.rho}"}[args.values],
        "config": {"workload": ("llama3.1-70b-kv-32k-tokens" if args.workload == "c3_llama70b_32k" else wl.name)
                   + (f"-{wl.heads}-heads" if args.heads else "") + (f"-{L}-layers" if args.layers else ""),
                   "layers": L, "tokens": T, "kv_heads": wl.heads,
                   "head_dim": wl.head_dim, "io_dtype": wl.dtype,
                   "k_policy": f"int{wl.k.bits} per-{wl.k.axis} g{wl.k.group} hadamard",
                   "v_policy": f"int{wl.v.bits} per-{wl.v.axis} g{wl.v.group} hadamard",
                   "lossless": ">".join(wl.stages), "chunk_bytes": wl.chunk_bytes, "mixed": args.mixed,
                   "token_delta": [dk, dv],
                   "uncompressed_bytes": U},
    }
    for key in ("encode_GBps", "decode_GBps", "encode_frac_hbm_peak", "decode_frac_hbm_peak", "compression_ratio",
                "compression_ratio_quant", "compression_ratio_lossless", "stream_bytes", "harmonic_s_p_GBps",
                "break_even_bandwidth_GBps"):
        result[key] = head[key]
    result["layer_pipeline"] = overlap
    result["kernel_ms_per_launch"] = {k_: round(v_, 4) for k_, v_ in kms.items()}
    result["fused_kernels"] = {k_: v_ for k_, v_ in head["kernels"].items() if "ENCODE" in k_ or "DECODE" in k_}
    result["device_copy_GBps"] = round(copy_gbps, 1)
    result["bandwidth_reference"] = probes
    result["graph_replay"] = (None if graph_ms is None else
                              {"ms_per_step": round(graph_ms, 4), "GBps": round(gbps(U, graph_ms), 3)})
    result["roofline"] = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                          "algorithmic_bytes": round(fb[dom]), "traffic": None, "timing": TIMING_NOTE}
    t = counted_traffic(dom) if headline else None
    if t is not None:
        result["roofline"]["traffic"] = t["bytes"]
        result["roofline"]["traffic_read_write"] = [t["read_bytes"], t["write_bytes"]]
    result["pages_figures"] = PAGES_FIGURES
    result["selection"] = selection_cost(U, U / (head["encode_ms"] * 1e-3), U / (head["decode_ms"] * 1e-3),
                                         U / d.n)
    d.release()
    del d
    free()

    if not args.no_sub and headline:
        # each sub-result in a child process of its own: device memory that a
        # previous workload of tens of GB allocated and freed slows the next
        # one's kernels (the paged batch by 9 % after the 128K workload)
        sub = {}
        ss = args.sub_steps or min(args.steps, 10)
        sw = min(args.warmup, 3)
        for name in SUB_RESULTS:
            if args.sub_in_process:
                sub[name] = sub_result(name, ss, sw)
                free()
                continue
            cmd = [sys.executable, "-u", os.path.abspath(__file__), "--sub-only", name,
                   "--sub-steps", str(ss), "--warmup", str(sw)]
            pr = subprocess.run(cmd, stdout=subprocess.PIPE, text=True)
            if pr.returncode != 0:
                raise SystemExit(f"sub-result {name} failed (exit status {pr.returncode})")
            sub[name] = json.loads(pr.stdout.strip().splitlines()[-1])
        result["sub_results"] = sub
        for name, r in sub.items():
            log(f"{name}: encode {r['encode_GBps']:.1f} GB/s, decode {r['decode_GBps']:.1f} GB/s, CR "
                f"{r['compression_ratio']:.3f}")
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or host_cores()
        log(f"timing the oracle on {args.cpu_layers} layers on the host (1 and {threads} threads)")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_layers, threads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
