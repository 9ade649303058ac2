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
    front = S.pareto_front(pts)
    assert front
    r = S.rank(pts, front, (10, 100, 1000))
    assert r["envelope"][0]["pipeline"] == "raw transfer"
    log(f"front {[pts[i]['pipeline'] for i in front]}; choices {r['choice']}")
