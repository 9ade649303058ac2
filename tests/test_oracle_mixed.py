"""Oracle pins for mixed precision per (layer, head) (KVServe Sec. 5.1,
head- and layer-wise mixed precision).  Heads are quantized independently
(per-token groups lie inside one head vector, per-channel groups inside one
(layer, head, channel)), so a mixed stream must reconstruct every head
exactly as a uniform stream of that head's width does, and keep 16-bit heads
unchanged; with one width everywhere its sections must be the uniform
stream's sections regrouped by (layer, head)."""
import dataclasses

import numpy as np
import pytest

import kvc_workloads as W
import oracle_api as O


def a16(x):
    return (x + 15) & ~15


def sections(stream, cfg, L, H, T, bits=None):
    """(codes[2], params[2]) of an oracle stream, codes de-chunked."""
    stages = [cfg.stages[i] for i in range(4)]
    cb = cfg.chunk_bytes
    if bits is None:
        nbytes = [O.lib().kvco_codes_bytes(O.C.byref(cfg), w, T) for w in range(2)]
        pbytes = [O.lib().kvco_params_bytes(O.C.byref(cfg), w, T) for w in range(2)]
        table = 64
    else:
        nbytes, pbytes = [0, 0], [0, 0]
        for w in range(2):
            for b in bits[w].reshape(-1):
                if b == 16:
                    nbytes[w] += T * 128 * 2
                else:
                    c1 = slab_cfg(cfg, w, int(b))
                    nbytes[w] += O.lib().kvco_codes_bytes(O.C.byref(c1), w, T)
                    pbytes[w] += O.lib().kvco_params_bytes(O.C.byref(c1), w, T)
        table = a16(64 + 2 * L * H)
    nch = [-(-n // cb) for n in nbytes]
    ent = stream[table:table + 4 * sum(nch)].view(np.uint32)
    p0 = a16(table + 4 * sum(nch))
    p1 = a16(p0 + pbytes[0])
    pos = a16(p1 + pbytes[1])
    codes = []
    gi = 0
    for w in range(2):
        parts = []
        for i in range(nch[w]):
            n = min(cb, nbytes[w] - i * cb)
            stored, raw = int(ent[gi] & 0x7FFFFFFF), bool(ent[gi] >> 31)
            st, dec = O.chunk_decode(stages, stream[pos:pos + stored], raw, n)
            assert st == O.OK
            parts.append(dec)
            pos += a16(stored)
            gi += 1
        codes.append(np.concatenate(parts) if parts else np.zeros(0, np.uint8))
    params = [stream[p0:p0 + pbytes[0]], stream[p1:p1 + pbytes[1]]]
    return codes, params


def slab_cfg(cfg, w, b):
    c = O.Cfg()
    for f, _ in O.Cfg._fields_:
        setattr(c, f, getattr(cfg, f))
    c.layers, c.heads = 1, 1
    setattr(c, ("k" if w == 0 else "v") + "_bits", b)
    return c


@pytest.mark.parametrize("name,L,T", [("c3_llama70b_32k", 2, 200), ("c1_single_layer_512", 1, 77),
                                      ("c2_llama8b_4k", 2, 130)])
def test_mixed_heads_reconstruct_like_uniform_streams(name, L, T):
    wl = W.WORKLOADS[name]
    H = wl.heads
    k, v = W.dense_kv(wl, layers=L, tokens=T)
    ku, vu = W.as_u16(k), W.as_u16(v)
    rng = np.random.default_rng(3)
    bits = rng.choice([2, 4, 8, 16], size=(2, L, H)).astype(np.uint8)
    cfg = O.cfg_from_workload(wl, layers=L)
    st, s = O.encode_mixed(cfg, bits, ku, vu, T)
    assert st == O.OK
    assert s[7] == 1 and np.array_equal(s[64:64 + 2 * L * H].reshape(2, L, H), bits)
    n = L * T * H * 128
    st, km, vm = O.decode(s, n)
    assert st == O.OK
    got = [km.reshape(L, T, H, 128), vm.reshape(L, T, H, 128)]
    src = [ku.reshape(L, T, H, 128), vu.reshape(L, T, H, 128)]
    for b in (2, 4, 8):
        wlb = dataclasses.replace(wl, k=dataclasses.replace(wl.k, bits=b), v=dataclasses.replace(wl.v, bits=b))
        st, su = O.encode(O.cfg_from_workload(wlb, layers=L), ku, vu, T)
        assert st == O.OK
        st, ku_b, vu_b = O.decode(su, n)
        ref = [ku_b.reshape(L, T, H, 128), vu_b.reshape(L, T, H, 128)]
        for w in range(2):
            for l in range(L):
                for h in range(H):
                    if bits[w, l, h] == b:
                        assert np.array_equal(got[w][l, :, h], ref[w][l, :, h]), (w, l, h, b)
    for w in range(2):
        for l in range(L):
            for h in range(H):
                if bits[w, l, h] == 16:
                    assert np.array_equal(got[w][l, :, h], src[w][l, :, h])


@pytest.mark.parametrize("name,L,T", [("c3_llama70b_32k", 2, 192), ("c2_llama8b_4k", 1, 64)])
def test_single_width_mixed_stream_regroups_uniform_sections(name, L, T):
    wl = W.WORKLOADS[name]
    H = wl.heads
    k, v = W.dense_kv(wl, layers=L, tokens=T)
    ku, vu = W.as_u16(k), W.as_u16(v)
    cfg = O.cfg_from_workload(wl, layers=L)
    bits = np.stack([np.full((L, H), wl.k.bits), np.full((L, H), wl.v.bits)]).astype(np.uint8)
    st, sm = O.encode_mixed(cfg, bits, ku, vu, T)
    assert st == O.OK
    st, su = O.encode(cfg, ku, vu, T)
    assert st == O.OK
    cm, pm = sections(sm, cfg, L, H, T, bits)
    cu, pu = sections(su, cfg, L, H, T)
    for w, pol in enumerate((wl.k, wl.v)):
        if pol.axis == "token":
            ng = 128 // pol.group
            cu_r = cu[w].reshape(L, T, H, 128 * pol.bits // 8).transpose(0, 2, 1, 3)
            pu_r = pu[w].reshape(L, T, H, ng * 4).transpose(0, 2, 1, 3)
        else:
            assert T % pol.group == 0
            ng = T // pol.group
            cu_r = cu[w].reshape(L, ng, H, 128 * pol.group * pol.bits // 8).transpose(0, 2, 1, 3)
            pu_r = pu[w].reshape(L, ng, H, 128 * 4).transpose(0, 2, 1, 3)
        assert np.array_equal(cm[w], np.ascontiguousarray(cu_r).reshape(-1)), w
        assert np.array_equal(pm[w], np.ascontiguousarray(pu_r).reshape(-1)), w


def test_invalid_width_maps_are_rejected():
    wl = W.WORKLOADS["c1_single_layer_512"]
    k, v = W.dense_kv(wl, layers=1, tokens=32)
    cfg = O.cfg_from_workload(wl, layers=1)
    for bad in (0, 3, 6, 32):
        bits = np.full((2, 1, wl.heads), 4, np.uint8)
        bits[1, 0, 2] = bad
        st, _ = O.encode_mixed(cfg, bits, W.as_u16(k), W.as_u16(v), 32)
        assert st == O.INVALID_ARG
