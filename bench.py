#!/usr/bin/env python3
"""Throughput of the KV-cache compression path on one MI355X.

A step is one pass of the whole path over one batch of synthetic KV:
fused transform + quantize (K and V), lossless encode, scan, compaction,
then lossless decode and fused reconstruction of the produced stream.  The
default workload is the Llama-3.1-70B-shaped cache at 32768 tokens (80
layers x 8 KV heads x 128, bf16, K int4 per-channel groups of 64 tokens, V
int2 per-token groups of 32, lossless TUPL8_1 -> BIT_8 -> RZE_2), with all
inputs resident in HBM before timing starts.

Prints one JSON line.  `value` is uncompressed K+V bytes per second of a
whole step (encode + decode); encode and decode rates are reported too.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, os.path.join(ROOT, "tests")):
    if p not in sys.path:
        sys.path.insert(0, p)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E peak


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def fused_bytes_per_elem(pol):
    # read 2 B, write bits/8 B of codes and 4 B of parameters per group
    return 2.0 + pol.bits / 8.0 + 4.0 / pol.group


def counted_traffic(kind: str):
    """HBM bytes per launch of a fused kernel as counted by rocprofv3
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's counts), taken from the
    committed profile summary of this workload; None when that summary was
    made from a different version of the kernel source."""
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


def cpu_baseline(wl, layers: int):
    """The oracle as it stands, single-threaded, on the first `layers` layers
    of the workload (same value model, generated on the host)."""
    import kvc_workloads as W
    import oracle_api as O
    k, v = W.dense_kv(wl, layers=layers, device="cpu")
    ku, vu = W.as_u16(k), W.as_u16(v)
    cfg = O.cfg_from_workload(wl, layers=layers)
    t0 = time.perf_counter()
    st, s = O.encode(cfg, ku, vu, wl.tokens)
    t1 = time.perf_counter()
    st2, _, _ = O.decode(s, layers * wl.tokens * wl.heads * wl.head_dim)
    t2 = time.perf_counter()
    assert st == O.OK and st2 == O.OK
    U = wl.uncompressed_bytes() / wl.layers * layers
    return {"value": round(U / (t2 - t0) / 1e9, 6), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"layers 0..{layers - 1} of the workload ({U / 1e9:.3f} GB of K+V), encode + decode",
            "encode_GBps": round(U / (t1 - t0) / 1e9, 6), "decode_GBps": round(U / (t2 - t1) / 1e9, 6),
            "seconds": round(t2 - t0, 2), "host_cpu": host_cpu(), "host_logical_cpus": os.cpu_count()}


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


def host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3_llama70b_32k")
    ap.add_argument("--cpu-layers", type=int, default=8, help="layers of the oracle's timed sample (about 15 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
                    help="also time a layer pipeline: layer l encoded on one stream while the other stream "
                         "decodes layer l - 1 (one-layer calls, an event between them)")
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
    import kv_cache_compression_kvc_amd as K
    import kvc_workloads as W

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

    wl = W.WORKLOADS[args.workload]
    dk, dv = (int(x) for x in args.delta.split(":"))
    if dk or dv:
        import dataclasses
        wl = wl.with_(k=dataclasses.replace(wl.k, delta=dk), v=dataclasses.replace(wl.v, delta=dv))
    if args.heads:
        wl = wl.with_(heads=args.heads)
    if args.layers:
        wl = wl.with_(layers=args.layers)
    L, T = wl.layers, wl.tokens
    dev = torch.device("cuda:0")
    log(f"generating {wl.name}: {L} x {T} x {wl.heads} x {wl.head_dim} {wl.dtype} on {dev}")
    if args.values == "gaussian":
        k, v = W.dense_kv(wl, device=dev)
    elif args.values == "correlated":
        k, v = W.correlated_kv(wl, L, T, W.SEED_BASE + 7, device=dev, rho=args.rho)
    else:
        k, v = W.zero_rich_kv(wl, L, T, seed=W.SEED_BASE + 7, device=dev, zero_frac=args.zero_frac)
    bits = mixed_widths(args.mixed, wl)
    plan = K.Plan(K.config_from_workload(wl), bits)
    ms, wsb = plan.sizes(T)
    out = torch.empty(ms, dtype=torch.uint8, device=dev)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    kd = torch.empty_like(k)
    vd = torch.empty_like(v)
    U = wl.uncompressed_bytes()
    torch.cuda.synchronize()

    n = plan.encode(k, v, T, out, ws)                       # synchronous: size and status
    plan.decode(out, n, T, kd, vd, ws)
    st = plan.query_status(ws)
    assert st == K.OK, K.status_string(st)
    log(f"stream {n} bytes, ratio {U / n:.4f}")

    def step():
        plan.encode(k, v, T, out, ws, sync=False)
        plan.decode(out, ms, T, kd, vd, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    s = torch.cuda.current_stream()
    K.profile_reset()
    K.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(args.steps):
        step()
    e1.record(s)
    torch.cuda.synchronize()
    K.profile_enable(False)
    step_ms = e0.elapsed_time(e1) / args.steps
    prof = {name: K.profile_query(name) for name in K.KERNELS}
    log(f"step {step_ms:.3f} ms; per-kernel ms/launch: " +
        ", ".join(f"{k_}={t / max(c, 1):.3f}" for k_, (t, c) in prof.items() if c))

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        for _ in range(args.steps):
            fn()
        b.record(s)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    enc_ms = timed(lambda: plan.encode(k, v, T, out, ws, sync=False))
    dec_ms = timed(lambda: plan.decode(out, ms, T, kd, vd, ws))
    st = plan.query_status(ws)
    assert st == K.OK, K.status_string(st)

    # the same step captured once in a HIP graph and replayed (a serving loop's
    # form: the dense calls enqueue kernels only)
    graph_ms = None
    if bits is None:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(s)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                step()
        s.wait_stream(side)
        torch.cuda.synchronize()
        graph_ms = timed(g.replay)
        st = plan.query_status(ws)
        assert st == K.OK, K.status_string(st)
        log(f"graph replay {graph_ms:.3f} ms per step")
    log(f"encode {enc_ms:.3f} ms ({U / enc_ms / 1e6:.1f} GB/s), decode {dec_ms:.3f} ms ({U / dec_ms / 1e6:.1f} GB/s)")

    overlap = None
    if args.overlap and bits is None:
        # one-layer calls: layer l is encoded on stream A into its own stream
        # buffer; stream B waits for that encode's event and decodes it, so
        # B's decode of layer l overlaps A's encode of layer l + 1
        p1 = K.Plan(K.config_from_workload(wl, layers=1))
        ms1, ws1 = p1.sizes(T)
        bufs = torch.empty((L, ms1), dtype=torch.uint8, device=dev)
        wa = torch.empty(ws1, dtype=torch.uint8, device=dev)
        wb = torch.empty(ws1, dtype=torch.uint8, device=dev)
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        evs = [torch.cuda.Event() for _ in range(L)]

        def pipe(do_enc=True, do_dec=True):
            sa.wait_stream(s)
            sb.wait_stream(s)
            for l in range(L):
                if do_enc:
                    p1.encode(k[l], v[l], T, bufs[l], wa, sync=False, stream=sa)
                    evs[l].record(sa)
                if do_dec:
                    if do_enc:
                        sb.wait_event(evs[l])
                    p1.decode(bufs[l], ms1, T, kd[l], vd[l], wb, stream=sb)
            s.wait_stream(sa)
            s.wait_stream(sb)

        pipe_ms = timed(pipe)
        enc1_ms = timed(lambda: pipe(True, False))
        dec1_ms = timed(lambda: pipe(False, True))
        assert p1.query_status(wa) == K.OK and p1.query_status(wb) == K.OK
        overlap = {"ms_per_step": round(pipe_ms, 4), "GBps": round(U / pipe_ms / 1e6, 3),
                   "encode_ms": round(enc1_ms, 4), "encode_GBps": round(U / enc1_ms / 1e6, 3),
                   "decode_ms": round(dec1_ms, 4), "decode_GBps": round(U / dec1_ms / 1e6, 3),
                   "calls": f"{L} one-layer encodes on one stream, {L} one-layer decodes on another"}
        log(f"layer pipeline {pipe_ms:.3f} ms ({U / pipe_ms / 1e6:.1f} GB/s); one-layer calls alone: "
            f"encode {enc1_ms:.3f} ms, decode {dec1_ms:.3f} ms")

    # roofline of the dominant fused kernel, algorithmic bytes per launch
    elems = L * T * wl.heads * wl.head_dim
    per_k = elems * fused_bytes_per_elem(wl.k) if bits is None else mixed_bytes(bits[0], wl.k, elems)
    per_v = elems * fused_bytes_per_elem(wl.v) if bits is None else mixed_bytes(bits[1], wl.v, elems)
    cand = {"ENCODE_K": per_k, "ENCODE_V": per_v, "DECODE_K": per_k, "DECODE_V": per_v}
    avg = {k_: prof[k_][0] / max(prof[k_][1], 1) for k_ in cand}
    dom = max(avg, key=avg.get)
    achieved = cand[dom] / (avg[dom] * 1e-3) / 1e9
    import ctypes as C
    codes_params = 0
    # quantized bytes (codes + parameters) from the closed form
    for w, pol in enumerate((wl.k, wl.v)):
        if bits is None:
            codes_params += elems * (pol.bits / 8.0 + 4.0 / pol.group)
        else:
            codes_params += mixed_bytes(bits[w], pol, elems) - 2.0 * elems
    result = {
        "metric": "KV encode / decode GB/s (uncompressed bytes) + % HBM peak, compression ratio",
        "value": round(U / step_ms / 1e6, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
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
        "encode_GBps": round(U / enc_ms / 1e6, 3),
        "decode_GBps": round(U / dec_ms / 1e6, 3),
        "encode_frac_hbm_peak": round(U / enc_ms / 1e6 / HBM_PEAK_GBPS, 4),
        "decode_frac_hbm_peak": round(U / dec_ms / 1e6 / HBM_PEAK_GBPS, 4),
        "compression_ratio": round(U / n, 4),
        "layer_pipeline": overlap,
        "compression_ratio_quant": round(U / codes_params, 4),
        "compression_ratio_lossless": round(codes_params / n, 4),
        "stream_bytes": n,
        "kernel_ms_per_launch": {k_: round(t / max(c, 1), 4) for k_, (t, c) in prof.items() if c},
        "device_copy_GBps": round(copy_gbps, 1),
        "graph_replay": (None if graph_ms is None else
                         {"ms_per_step": round(graph_ms, 4), "GBps": round(U / graph_ms / 1e6, 3)}),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "algorithmic_bytes": round(cand[dom]), "traffic": None},
    }
    # each fused kernel, and the K and V kernels of one direction together
    fk = {}
    for k_ in cand:
        gbps = cand[k_] / (avg[k_] * 1e-3) / 1e9
        fk[k_] = {"ms": round(avg[k_], 4), "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    for name, a_, b_ in (("ENCODE", "ENCODE_K", "ENCODE_V"), ("DECODE", "DECODE_K", "DECODE_V")):
        ms_ = avg[a_] + avg[b_]
        gbps = (cand[a_] + cand[b_]) / (ms_ * 1e-3) / 1e9
        fk[name + "_K+V"] = {"ms": round(ms_, 4), "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    result["fused_kernels"] = fk
    result["pages_figures"] = PAGES_FIGURES
    result["selection"] = selection_cost(U, U / (enc_ms * 1e-3), U / (dec_ms * 1e-3), U / n)
    t = (counted_traffic(dom) if (args.workload == "c3_llama70b_32k" and args.values == "gaussian"
                                   and args.mixed == "none" and not (dk or dv) and not args.heads
                                   and not args.layers) else None)
    if t is not None:
        result["roofline"]["traffic"] = t["bytes"]
        result["roofline"]["traffic_read_write"] = [t["read_bytes"], t["write_bytes"]]
    s_enc, s_dec = U / enc_ms / 1e6, U / dec_ms / 1e6
    s_p = s_enc * s_dec / (s_enc + s_dec)
    result["harmonic_s_p_GBps"] = round(s_p, 3)
    result["break_even_bandwidth_GBps"] = round((1 - n / U) * s_p, 3)
    if not args.no_cpu_baseline:
        log(f"timing the oracle on {args.cpu_layers} layers on the host")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_layers)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
