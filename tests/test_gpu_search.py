"""Pipeline search on the GPU: every searched pipeline's stream equals the
oracle's stream for the same K/V and pipeline (lossless coding is exact
given equal codes, so the sizes the search ranks are the oracle's sizes),
and the Pareto/envelope ranking runs on the measured profiles."""
import dataclasses
import random

import numpy as np
import pytest
import torch

import kv_cache_compression_kvc_amd as K
import kvc_workloads as W
import oracle_api as O
from gpu_helpers import DEV, log, to_u16
from kv_cache_compression_kvc_amd import search as S

pytestmark = pytest.mark.gpu


def test_searched_pipelines_match_oracle_streams():
    wl = W.WORKLOADS["c3_llama70b_32k"]
    L, T = 1, 1024
    k, v = W.correlated_kv(wl, L, T, wl.seed, device=DEV, rho=0.95)
    rng = random.Random(5)
    cands = S.candidate_pipelines(3)
    pipes = [(), ("TUPL8_1", "BIT_8", "RZE_2"), ("TUPL8_1", "RZE_2")] + rng.sample(cands[1:], 21)
    log(f"search over {len(pipes)} pipelines on 1 x {T} tokens")
    pts = S.measure(wl, k, v, T, pipes, reps=1, log=log)
    ku, vu = to_u16(k), to_u16(v)
    U = 2 * k.numel() * k.element_size()
    for pipe, p in zip(pipes, pts):
        wlp = dataclasses.replace(wl, stages=tuple(pipe))
        st, ref = O.encode(O.cfg_from_workload(wlp, layers=L), ku, vu, T)
        assert st == O.OK
        assert p["stream_bytes"] == len(ref), pipe
        assert p["cr"] == pytest.approx(U / len(ref), rel=1e-12)
        # the bytes themselves, through the library
        plan = K.Plan(K.config_from_workload(wlp, max_tokens=T, layers=L))
        ms, wsb = plan.sizes(T)
        out = torch.empty(ms, dtype=torch.uint8, device=DEV)
        ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
        n = plan.encode(k, v, T, out, ws)
        assert np.array_equal(out[:n].cpu().numpy(), ref), pipe
    front = S.pareto_front(pts, S.SEARCH_KEYS)
    assert front
    r = S.rank(pts, front, (10, 100, 1000))
    assert r["envelope"][0]["pipeline"] == "raw transfer"
    log(f"front {[pts[i]['pipeline'] for i in front]}; choices {r['choice']}")


def test_searched_delta_variants_match_oracle_streams():
    # the token delta as a further transformer variant: each (run lengths,
    # pipeline) candidate's stream is the oracle's, and its recorded error is
    # the reconstruction's
    wl = W.WORKLOADS["c3_llama70b_32k"]
    L, T = 1, 512
    k, v = W.correlated_kv(wl, L, T, wl.seed, device=DEV, rho=0.95)
    pipes = [("TUPL8_1", "BIT_8", "RZE_2"), ("DIFF1", "RZE_1")]
    deltas = [(0, 0), (16, 16), (4, 64)]
    pts = S.measure(wl, k, v, T, pipes, reps=1, log=log, deltas=deltas)
    assert len(pts) == len(pipes) * len(deltas)
    ku, vu = to_u16(k), to_u16(v)
    for p, (dl, pipe) in zip(pts, [(d, q) for d in deltas for q in pipes]):
        wlp = dataclasses.replace(wl, stages=tuple(pipe), k=dataclasses.replace(wl.k, delta=dl[0]),
                                  v=dataclasses.replace(wl.v, delta=dl[1]))
        st, ref = O.encode(O.cfg_from_workload(wlp, layers=L), ku, vu, T)
        assert st == O.OK
        assert p["stream_bytes"] == len(ref), (dl, pipe)
        st, kd, vd = O.decode(ref, L * T * wl.heads * wl.head_dim)
        assert st == O.OK
        to_f = lambda u: torch.from_numpy(np.ascontiguousarray(u).reshape(-1).view(np.int16)).view(wl.torch_dtype).double()
        num = float(((to_f(kd) - to_f(ku)) ** 2).sum() + ((to_f(vd) - to_f(vu)) ** 2).sum())
        den = float((to_f(ku) ** 2).sum() + (to_f(vu) ** 2).sum())
        assert p["rel_err"] == pytest.approx((num / den) ** 0.5, rel=1e-4), (dl, pipe)
    log("; ".join(f"{p['pipeline']}: cr {p['cr']:.3f} err {p['rel_err']:.5f}" for p in pts))
