"""A dense encode + decode captured in a HIP graph (through torch's graph
capture on the current stream) and replayed: the library's dense calls
enqueue only kernels (no host synchronization, no memset or copy nodes), so a
serving loop can capture them.  Every replay must reproduce the eager
stream byte for byte and the eager reconstruction bit for bit; eager work
and synchronizations run between the replays.  Also: one plan used from two
streams at once, each with its own workspace."""
import pytest
import torch

import kvc_workloads as W
import kv_cache_compression_kvc_amd as K
from gpu_helpers import DEV, log

pytestmark = pytest.mark.gpu

C3 = W.WORKLOADS["c3_llama70b_32k"]


@pytest.mark.parametrize("stages", [("TUPL8_1", "BIT_8", "RZE_2"), ("TUPL8_1", "RZE_2"), ("DIFF1", "RZE_1")])
def test_encode_decode_replay_in_a_graph(stages):
    wl = C3.with_(stages=stages, chunk_bytes=65536, name="graph")
    L, T = 4, 1024
    k, v = W.zero_rich_kv(wl, L, T, seed=31, device=DEV, zero_frac=0.5)
    plan = K.Plan(K.config_from_workload(wl, max_tokens=T, layers=L))
    ms, wsb = plan.sizes(T)
    out = torch.empty(ms, dtype=torch.uint8, device=DEV)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    kd, vd = torch.empty_like(k), torch.empty_like(v)
    n = plan.encode(k, v, T, out, ws)
    plan.decode(out, n, T, kd, vd, ws)
    assert plan.query_status(ws) == K.OK
    ref, kref, vref = out[:n].clone(), kd.clone(), vd.clone()

    out2, ws2 = torch.zeros_like(out), torch.zeros_like(ws)
    kd2, vd2 = torch.zeros_like(kd), torch.zeros_like(vd)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            plan.encode(k, v, T, out2, ws2, sync=False)
            plan.decode(out2, ms, T, kd2, vd2, ws2)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: clear the outputs with fill kernels
        out2.zero_()
        kd2.zero_()
        vd2.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out2[:n], ref), f"replay {rep}: stream differs"
        assert torch.equal(kd2, kref) and torch.equal(vd2, vref), f"replay {rep}: reconstruction differs"
        assert plan.query_status(ws2) == K.OK
        log(f"replay {rep} identical ({n} stream bytes)")


def test_one_plan_on_two_streams_at_once():
    # a plan is immutable: calls on two streams with their own workspaces may
    # run at the same time (here one stream encodes layer l while the other
    # decodes layer l - 1, ordered only by events), and every stream and
    # reconstruction equals the one-stream result
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(chunk_bytes=65536)
    L, T = 6, 2048
    k, v = W.zero_rich_kv(wl, L, T, seed=31, device=DEV, zero_frac=0.5)
    plan = K.Plan(K.config_from_workload(wl, max_tokens=T, layers=1))
    ms, wsb = plan.sizes(T)
    ref_streams, ref_k, ref_v = [], [], []
    ws0 = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    for l in range(L):
        out = torch.empty(ms, dtype=torch.uint8, device=DEV)
        n = plan.encode(k[l], v[l], T, out, ws0)
        ref_streams.append(out[:n].clone())
        kd, vd = torch.empty_like(k[l]), torch.empty_like(v[l])
        plan.decode(out, n, T, kd, vd, ws0)
        ref_k.append(kd)
        ref_v.append(vd)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    wa = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    wb = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    bufs = torch.empty((L, ms), dtype=torch.uint8, device=DEV)
    kd, vd = torch.empty_like(k), torch.empty_like(v)
    evs = [torch.cuda.Event() for _ in range(L)]
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for l in range(L):
        plan.encode(k[l], v[l], T, bufs[l], wa, sync=False, stream=sa)
        evs[l].record(sa)
        sb.wait_event(evs[l])
        plan.decode(bufs[l], ms, T, kd[l], vd[l], wb, stream=sb)
    torch.cuda.synchronize()
    assert plan.query_status(wa) == K.OK and plan.query_status(wb) == K.OK
    for l in range(L):
        n = ref_streams[l].numel()
        assert torch.equal(bufs[l, :n], ref_streams[l]), l
        assert torch.equal(kd[l], ref_k[l]) and torch.equal(vd[l], ref_v[l]), l
