"""kvc_encode_noalloc (the encode that allocates nothing and uses the
library's fixed device scratch) against kvc_encode with a caller workspace:
identical streams, on two calls in a row through one plan, the second with
a smaller input, for Gaussian and zero-rich (compressing) inputs; the
oracle's stream for the smaller call; the synchronous and the asynchronous
form; and host-side rejection of calls too large for the scratch."""
import numpy as np
import pytest
import torch

import kv_cache_compression_kvc_amd as K
import kvc_workloads as W
import oracle_api as O
from gpu_helpers import DEV, log, to_u16

pytestmark = pytest.mark.gpu

C3 = W.WORKLOADS["c3_llama70b_32k"]


@pytest.mark.parametrize("values", ["gaussian", "zero_rich"])
def test_noalloc_encode_equals_workspace_encode(values):
    wl = C3.with_(chunk_bytes=65536, name="noalloc")
    L = 2
    plan = K.Plan(K.config_from_workload(wl, max_tokens=2048, layers=L))
    for T, seed in ((2048, 1), (700, 2)):                        # the second call is smaller
        log(f"noalloc {values} L={L} T={T}")
        if values == "gaussian":
            k, v = W.dense_kv(wl, layers=L, tokens=T, seed=seed, device=DEV)
        else:
            k, v = W.zero_rich_kv(wl, L, T, seed=seed, device=DEV, zero_frac=0.5)
        ms, wsb = plan.sizes(T)
        assert wsb <= K.NOALLOC_SCRATCH_BYTES
        ref = torch.full((ms,), 0xA5, dtype=torch.uint8, device=DEV)
        ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device=DEV)
        n_ref = plan.encode(k, v, T, ref, ws)
        out = torch.full((ms,), 0x3C, dtype=torch.uint8, device=DEV)
        n = plan.encode_noalloc(k, v, T, out)
        assert n == n_ref
        assert torch.equal(out[:n], ref[:n_ref])
        # asynchronous form: the size is the header's total
        out2 = torch.full((ms,), 0x11, dtype=torch.uint8, device=DEV)
        assert plan.encode_noalloc(k, v, T, out2, sync=False) is None
        torch.cuda.synchronize()
        total = int(np.frombuffer(out2[56:64].cpu().numpy().tobytes(), np.uint64)[0])
        assert total == n and torch.equal(out2[:n], ref[:n])
        if T == 700:
            st, oref = O.encode(O.cfg_from_workload(wl, layers=L), to_u16(k), to_u16(v), T)
            assert st == O.OK
            assert np.array_equal(out[:n].cpu().numpy(), oref)


def test_noalloc_rejects_calls_larger_than_its_scratch():
    wl = W.WORKLOADS["c5_llama70b_128k"]
    plan = K.Plan(K.config_from_workload(wl, layers=4))
    ms, wsb = plan.sizes(wl.tokens)
    assert wsb > K.NOALLOC_SCRATCH_BYTES
    dummy = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(K.KvcError) as e:
        plan.encode_noalloc(dummy, dummy, wl.tokens, dummy)
    assert e.value.status == K.ERR_BUFFER_TOO_SMALL
    mixed = K.Plan(K.config_from_workload(C3, max_tokens=64, layers=1), np.full((2, 1, 8), 4, np.uint8))
    with pytest.raises(K.KvcError) as e:
        mixed.encode_noalloc(dummy, dummy, 64, dummy)
    assert e.value.status == K.ERR_UNSUPPORTED
