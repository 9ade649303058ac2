"""Offline lossless-pipeline search on the GPU.

"Beyond Compression Ratio: High-Throughput KV Compression for Disaggregated
LLM Serving", Sec. 4.2: the lossless backend is searchable -- candidate
pipelines of LC-style stages are run on the GPU, their encode time, decode
time and compressed size measured, and the Pareto-optimal ones kept and
ranked for the deployment's bandwidth.  Here a candidate is a plan whose
lossless list is one or two transform stages (TUPL, DIFF, BIT) followed by a
zero-elimination stage (RZE), or no lossless stage at all, optionally
behind the token delta that KVServe Sec. 5.1 lists among its transformer
modules (run lengths for K and V); each is timed end to end (delta, fused
quantize + lossless + scan + placement, and the mirror) on the same K/V,
through the library, and its reconstruction error is recorded (the delta
changes what is quantized; the lossless stages do not).  Ranking uses KVServe's Eq. 5-6
("KVServe: Service-Aware KV Cache Compression for Communication-Efficient
Disaggregated LLM Serving", Sec. 6.1): the break-even bandwidth of each
profile and the lower envelope of the latency lines, via the library's
selector.

    python -m kv_cache_compression_kvc_amd.search --layers 8 --values correlated
"""
from __future__ import annotations

import argparse
import itertools
import json
import os
import sys
import time
from typing import Dict, List, Sequence

TRANSFORMS = ("TUPL2_1", "TUPL4_1", "TUPL8_1", "DIFF1", "DIFF2", "DIFF4", "DIFF8", "BIT_1", "BIT_2", "BIT_4",
              "BIT_8")
REDUCERS = ("RZE_1", "RZE_2", "RZE_4", "RZE_8")


def candidate_pipelines(max_stages: int = 3, include_none: bool = True) -> List[tuple]:
    """Lossless lists to try: () (no lossless stage), then every
    transforms + reducer chain with 2 .. max_stages stages."""
    out = [()] if include_none else []
    for n in range(1, max_stages):
        for ts in itertools.product(TRANSFORMS, repeat=n):
            for r in REDUCERS:
                out.append(tuple(ts) + (r,))
    return out


# what the search minimizes: stream size, encode and decode time, and the
# reconstruction error (which only the token delta changes)
SEARCH_KEYS = ("stream_bytes", "enc_ms", "dec_ms", "rel_err")


def pareto_front(points: Sequence[Dict], keys=("stream_bytes", "enc_ms", "dec_ms")) -> List[int]:
    """Indices of the points no other point dominates (lower or equal in every
    key, lower in one), minimizing all keys; sorted by the first key."""
    order = sorted(range(len(points)), key=lambda i: tuple(points[i][k] for k in keys))
    front: List[int] = []
    for i in order:
        p = points[i]
        dominated = False
        for j in front:
            q = points[j]
            if all(q[k] <= p[k] for k in keys) and any(q[k] < p[k] for k in keys):
                dominated = True
                break
        if not dominated:
            # a later point in this order cannot dominate an earlier kept one
            # unless they tie on the first key; drop kept points it dominates
            front = [j for j in front
                     if not (all(p[k] <= points[j][k] for k in keys) and any(p[k] < points[j][k] for k in keys))]
            front.append(i)
    return sorted(front, key=lambda i: tuple(points[i][k] for k in keys))


def profile_numbers(uncompressed: int, stream_bytes: int, enc_ms: float, dec_ms: float) -> Dict:
    import kv_cache_compression_kvc_amd as K
    s_enc = uncompressed / (enc_ms * 1e-3)
    s_dec = uncompressed / (dec_ms * 1e-3)
    cr = uncompressed / stream_bytes
    return {"cr": cr, "s_enc": s_enc, "s_dec": s_dec, "s_p": K.harmonic_throughput(s_enc, s_dec),
            "b_star": K.break_even_bandwidth(cr, s_enc, s_dec)}


def measure(wl, k, v, tokens: int, pipelines: Sequence[tuple], reps: int = 3, log=print,
            deltas: Sequence[tuple] = ((0, 0),)) -> List[Dict]:
    """Encode + decode k, v ([L, T, H, D] on the GPU) under each (token-delta
    run lengths (K, V), pipeline) pair; time both directions with HIP events
    over `reps` runs after one warm-up, and record the relative error
    ||x' - x|| / ||x|| of the reconstruction (K and V together)."""
    import torch
    import kv_cache_compression_kvc_amd as K
    L = k.shape[0]
    U = 2 * k.numel() * k.element_size()
    base = K.config_from_workload(wl, max_tokens=tokens, layers=L)
    dev = k.device
    kd, vd = torch.empty_like(k), torch.empty_like(v)
    res = []
    out = ws = None
    t_start = time.time()
    cands = [(d, p) for d in deltas for p in pipelines]
    norm = float(torch.sqrt(k.float().square().sum() + v.float().square().sum()))
    for n, (dl, pipe) in enumerate(cands):
        cfg = K.make_config(L, tokens, wl.heads, wl.head_dim, base.dtype,
                            (base.k.bits, base.k.axis, base.k.group, base.k.hadamard, dl[0]),
                            (base.v.bits, base.v.axis, base.v.group, base.v.hadamard, dl[1]),
                            base.sign_seed, list(pipe), base.chunk_bytes, 0)
        plan = K.Plan(cfg)
        ms, wsb = plan.sizes(tokens)
        if out is None or out.numel() < ms:
            out = torch.empty(ms, dtype=torch.uint8, device=dev)
        if ws is None or ws.numel() < wsb:
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        nbytes = plan.encode(k, v, tokens, out, ws)                      # warm-up, size scalar
        plan.decode(out, nbytes, tokens, kd, vd, ws)
        st = plan.query_status(ws)
        if st != K.OK:
            raise RuntimeError(f"pipeline {pipe}: {K.status_string(st)}")
        err = float(torch.sqrt((kd.float() - k.float()).square().sum() + (vd.float() - v.float()).square().sum()))
        s = torch.cuda.current_stream()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(s)
        for _ in range(reps):
            plan.encode(k, v, tokens, out, ws, sync=False)
        e[1].record(s)
        for _ in range(reps):
            plan.decode(out, nbytes, tokens, kd, vd, ws)
        e[2].record(s)
        torch.cuda.synchronize()
        enc_ms = e[0].elapsed_time(e[1]) / reps
        dec_ms = e[1].elapsed_time(e[2]) / reps
        name = ">".join(pipe) if pipe else "none"
        if dl != (0, 0):
            name = f"delta{dl[0]}/{dl[1]} " + name
        r = {"pipeline": name, "delta": list(dl), "stream_bytes": int(nbytes),
             "enc_ms": enc_ms, "dec_ms": dec_ms, "rel_err": err / norm if norm > 0 else 0.0}
        r.update(profile_numbers(U, nbytes, enc_ms, dec_ms))
        res.append(r)
        if (n + 1) % 25 == 0 or n + 1 == len(cands):
            log(f"  {n + 1}/{len(cands)} candidates ({time.time() - t_start:.0f} s)")
    return res


def rank(points: Sequence[Dict], front: Sequence[int], bandwidths_gbps: Sequence[float]) -> Dict:
    """The front's lower envelope (library selector, raw transfer included)
    and its choice at each bandwidth."""
    import kv_cache_compression_kvc_amd as K
    profs = [(i, 0, points[i]["cr"], points[i]["s_enc"], points[i]["s_dec"]) for i in front]
    sel = K.Selector(profs)
    ids, xs = sel.envelope(0)
    env = [{"pipeline": "raw transfer" if i == K.PROFILE_RAW else points[i]["pipeline"],
            "from_GBps": (None if x == 0.0 else 1.0 / x / 1e9)} for i, x in zip(ids, xs)]
    choice = {}
    for g in bandwidths_gbps:
        i = sel.model_choice(0, g * 1e9 / 8)
        choice[f"{g:g} Gbps"] = "raw transfer" if i == K.PROFILE_RAW else points[i]["pipeline"]
    sel.close()
    return {"envelope": env, "choice": choice}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="c3_llama70b_32k")
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--tokens", type=int, default=0, help="0 = the workload's")
    ap.add_argument("--values", choices=("gaussian", "correlated", "zero_rich"), default="correlated")
    ap.add_argument("--rho", type=float, default=0.95)
    ap.add_argument("--max-stages", type=int, default=3)
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--pipelines", default="", help="comma-separated lossless lists to time instead of all "
                    "candidates, stages joined by '>' (e.g. 'TUPL8_1>RZE_2,none')")
    ap.add_argument("--deltas", default="0:0", help="comma-separated token-delta run lengths K:V to combine "
                    "with every pipeline (0 = none; e.g. '0:0,16:16')")
    ap.add_argument("--json", default="")
    args = ap.parse_args(argv)
    import torch
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import kvc_workloads as W
    wl = W.WORKLOADS[args.workload]
    T = args.tokens or wl.tokens
    dev = torch.device("cuda:0")
    print(f"{args.workload}: {args.layers} layers x {T} tokens, values {args.values}", flush=True)
    if args.values == "correlated":
        k, v = W.correlated_kv(wl, args.layers, T, wl.seed, device=dev, rho=args.rho)
    elif args.values == "zero_rich":
        k, v = W.zero_rich_kv(wl, args.layers, T, wl.seed, device=dev, zero_frac=0.5)
    else:
        k, v = W.dense_kv(wl, layers=args.layers, tokens=T, device=dev)
    if args.pipelines:
        pipes = [() if x == "none" else tuple(x.split(">")) for x in args.pipelines.split(",")]
    else:
        pipes = candidate_pipelines(args.max_stages)
    deltas = [tuple(int(x) for x in d.split(":")) for d in args.deltas.split(",")]
    print(f"{len(pipes)} pipelines x {len(deltas)} delta settings", flush=True)
    pts = measure(wl, k, v, T, pipes, reps=args.reps, log=lambda m: print(m, flush=True), deltas=deltas)
    front = pareto_front(pts, SEARCH_KEYS)
    ranking = rank(pts, front, (10, 25, 50, 100, 200, 400, 800, 1600))
    for i in front:
        p = pts[i]
        print(f"{p['pipeline']:28s} cr {p['cr']:.4f} enc {p['enc_ms']:.3f} ms dec {p['dec_ms']:.3f} ms "
              f"s_p {p['s_p'] / 1e9:.0f} GB/s B* {p['b_star'] / 1e9:.0f} GB/s rel_err {p['rel_err']:.5f}")
    print(json.dumps(ranking), flush=True)
    if args.json:
        with open(args.json, "w") as f:
            json.dump({"workload": args.workload, "layers": args.layers, "tokens": T, "values": args.values,
                       "deltas": deltas,
                       "rho": args.rho if args.values == "correlated" else None, "reps": args.reps,
                       "points": pts, "front": front, "ranking": ranking}, f, indent=1)


if __name__ == "__main__":
    main()
