"""Pins for the oracle's stream format: an independent Python reader checks the
header, the chunk table, the exclusive-scan chunk offsets (brute force), the
zero padding and the lossless round trip; corrupt streams must be rejected;
paged encoding must equal dense encoding of the gathered requests.

FastKVComp Sec. 4.2 keeps the compressed stream on the GPU and returns only
its size to the host; the layout itself is this project's format."""
import struct

import numpy as np
import pytest

import kvc_workloads as W
import oracle_api as O


def a16(x):
    return (x + 15) & ~15


def parse(stream: np.ndarray):
    b = stream.tobytes()
    (magic, ver, dtype, _r, L, T, H, D) = struct.unpack_from("<IHBBiiii", b, 0)
    kpol = struct.unpack_from("<BBBBHH", b, 24)
    vpol = struct.unpack_from("<BBBBHH", b, 32)
    seed, = struct.unpack_from("<Q", b, 40)
    stages = list(b[48:52])
    cb, total = struct.unpack_from("<IQ", b, 52)
    return dict(magic=magic, ver=ver, dtype=dtype, L=L, T=T, H=H, D=D, kpol=kpol, vpol=vpol,
                seed=seed, stages=stages, cb=cb, total=total)


def sections(wl, L, T):
    """codes / params sizes from the format definition"""
    out = []
    for pol in (wl.k, wl.v):
        if pol.axis == "token":
            codes = L * T * wl.heads * wl.head_dim * pol.bits // 8
            params = L * T * wl.heads * (wl.head_dim // pol.group) * 4
        else:
            ng = -(-T // pol.group)
            per_layer = 0
            for g in range(ng):
                gg = min(pol.group, T - g * pol.group)
                per_layer += wl.heads * wl.head_dim * (-(-gg * pol.bits // 8))
            codes = L * per_layer
            params = L * ng * wl.heads * wl.head_dim * 4
        out.append((codes, params))
    return out


def check_layout(stream, wl, L, T, codes_ref):
    h = parse(stream)
    assert h["magic"] == 0x3143564B and h["ver"] == 1
    assert (h["L"], h["T"], h["H"], h["D"]) == (L, T, wl.heads, wl.head_dim)
    assert h["total"] == stream.size
    secs = sections(wl, L, T)
    cb = wl.chunk_bytes
    nch = [-(-c // cb) for c, _ in secs]
    table = np.frombuffer(stream.tobytes(), np.uint32, sum(nch), 64)
    poff0 = a16(64 + 4 * sum(nch))
    poff1 = a16(poff0 + secs[0][1])
    pay = a16(poff1 + secs[1][1])
    # padding between the fixed sections is zero
    assert not stream[64 + 4 * sum(nch):poff0].any()
    assert not stream[poff0 + secs[0][1]:poff1].any()
    # offsets are the exclusive scan of the 16-byte aligned stored sizes
    sizes = (table & 0x7FFFFFFF).astype(np.int64)
    raw = (table >> 31).astype(bool)
    offs = [0]
    for s in sizes:
        offs.append(offs[-1] + a16(int(s)))
    assert pay + offs[-1] == stream.size
    # each chunk decodes to the reference codes
    ci = 0
    stages = [O.STAGE_IDS[s] for s in wl.stages]
    for w in range(2):
        for i in range(nch[w]):
            n = min(cb, secs[w][0] - i * cb)
            start = pay + offs[ci]
            data = stream[start:start + sizes[ci]]
            assert not stream[start + sizes[ci]:pay + offs[ci + 1]].any()     # zero pad
            st, dec = O.chunk_decode(stages, data, int(raw[ci]), n)
            assert st == O.OK
            assert np.array_equal(dec, codes_ref[w][i * cb:i * cb + n])
            ci += 1
    return h


@pytest.mark.parametrize("name,T,L", [("c1_single_layer_512", 512, 1), ("c1_single_layer_512", 37, 2),
                                      ("c3_llama70b_32k", 150, 2), ("c3_llama70b_32k", 1, 1),
                                      ("c2_llama8b_4k", 130, 2)])
def test_stream_layout_and_round_trip(name, T, L):
    wl = W.WORKLOADS[name].with_(chunk_bytes=8192)
    k, v = W.dense_kv(wl, layers=L, tokens=T)
    cfg = O.cfg_from_workload(wl, layers=L)
    ku, vu = W.as_u16(k), W.as_u16(v)
    st, stream = O.encode(cfg, ku, vu, T)
    assert st == O.OK
    assert stream.size <= O.max_stream_bytes(cfg, T)
    codes = [O.quantize_tensor(cfg, w, x, T)[1] for w, x in ((0, ku), (1, vu))]
    params = [O.quantize_tensor(cfg, w, x, T)[2] for w, x in ((0, ku), (1, vu))]
    check_layout(stream, wl, L, T, codes)
    secs = sections(wl, L, T)
    nch = sum(-(-c // wl.chunk_bytes) for c, _ in secs)
    p0 = a16(64 + 4 * nch)
    assert np.array_equal(stream[p0:p0 + secs[0][1]], params[0])
    p1 = a16(p0 + secs[0][1])
    assert np.array_equal(stream[p1:p1 + secs[1][1]], params[1])
    n = L * T * wl.heads * wl.head_dim
    st, kd, vd = O.decode(stream, n)
    assert st == O.OK
    assert np.array_equal(kd, O.dequantize_tensor(cfg, 0, codes[0], params[0], T)[1])
    assert np.array_equal(vd, O.dequantize_tensor(cfg, 1, codes[1], params[1], T)[1])


def test_empty_stream():
    wl = W.WORKLOADS["c1_single_layer_512"]
    cfg = O.cfg_from_workload(wl)
    z = np.zeros(0, np.uint16)
    st, stream = O.encode(cfg, z, z, 0)
    assert st == O.OK and stream.size == 64 and parse(stream)["total"] == 64
    st, kd, vd = O.decode(stream, 0)
    assert st == O.OK


def test_compressible_stream_uses_non_raw_chunks():
    wl = W.WORKLOADS["c3_llama70b_32k"].with_(chunk_bytes=8192)
    k, v = W.zero_rich_kv(wl, 2, 256, seed=3)
    cfg = O.cfg_from_workload(wl, layers=2)
    st, stream = O.encode(cfg, W.as_u16(k), W.as_u16(v), 256)
    assert st == O.OK
    h = parse(stream)
    codes = [O.quantize_tensor(cfg, w, W.as_u16(x), 256)[1] for w, x in ((0, k), (1, v))]
    check_layout(stream, wl, 2, 256, codes)
    secs = sections(wl, 2, 256)
    nch = sum(-(-c // 8192) for c, _ in secs)
    table = np.frombuffer(stream.tobytes(), np.uint32, nch, 64)
    assert (table >> 31 == 0).sum() > 0
    assert stream.size < O.max_stream_bytes(cfg, 256)


def test_corrupt_streams_are_rejected():
    wl = W.WORKLOADS["c1_single_layer_512"].with_(chunk_bytes=8192)
    k, v = W.zero_rich_kv(wl, 1, 128, seed=4)
    cfg = O.cfg_from_workload(wl)
    st, good = O.encode(cfg, W.as_u16(k), W.as_u16(v), 128)
    n = 128 * 8 * 128
    assert O.decode(good, n)[0] == O.OK
    bad = good.copy(); bad[0] ^= 1
    assert O.decode(bad, n)[0] == O.CORRUPT                     # magic
    assert O.decode(good[:good.size - 16], n)[0] == O.CORRUPT   # truncated
    assert O.decode(good[:40], n)[0] == O.CORRUPT               # shorter than a header
    rng = np.random.default_rng(5)
    nch = 2 * (-(-128 * 8 * 64 // 8192))
    for _ in range(40):
        bad = good.copy()
        pos = 64 + 4 * int(rng.integers(0, nch)) + int(rng.integers(0, 4))
        bad[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
        assert O.decode(bad, n)[0] in (O.CORRUPT,)               # chunk table damage is detected
    for _ in range(40):                                          # payload damage never crashes
        bad = good.copy()
        pos = int(rng.integers(64, good.size))
        bad[pos] ^= np.uint8(0xFF)
        assert O.decode(bad, n)[0] in (O.OK, O.CORRUPT)


def test_paged_equals_dense_per_request():
    wl = W.WORKLOADS["c4_paged_llama8b"].with_(layers=2, chunk_bytes=8192)
    batch = W.paged_layout(wl, requests=5, min_len=3, max_len=70)
    kp, vp = W.paged_pools(wl, batch)
    cfg = O.cfg_from_workload(wl)
    kpu, vpu = W.as_u16(kp), W.as_u16(vp)
    st, stream, offs = O.encode_paged(cfg, kpu, vpu, batch.num_blocks, wl.page_tokens,
                                      batch.block_table, batch.seq_lens)
    assert st == O.OK
    P = wl.page_tokens
    for r, T in enumerate(batch.seq_lens.tolist()):
        # independent gather of request r into a dense [L, T, H, D] array
        idx = np.array([batch.block_table[r, t // P] * P + t % P for t in range(T)], dtype=np.int64)
        kd = kpu.reshape(2, -1, 8, 128)[:, idx]
        vd = vpu.reshape(2, -1, 8, 128)[:, idx]
        st, ref = O.encode(cfg, kd, vd, T)
        assert st == O.OK
        assert np.array_equal(stream[offs[r]:offs[r + 1]], ref)
    # decode scatters into a second pool with an independent page map
    dst = W.paged_layout(wl, requests=5, min_len=3, max_len=70, stream=1)
    kq = np.zeros_like(kpu); vq = np.zeros_like(vpu)
    st = O.decode_paged(stream, offs, kq, vq, dst.num_blocks, P, dst.block_table, dst.seq_lens)
    assert st == O.OK
    for r, T in enumerate(batch.seq_lens.tolist()):
        idx = np.array([dst.block_table[r, t // P] * P + t % P for t in range(T)], dtype=np.int64)
        st, kd, vd = O.decode(stream[offs[r]:offs[r + 1]], 2 * T * 8 * 128)
        assert np.array_equal(kq.reshape(2, -1, 8, 128)[:, idx].reshape(-1), kd)
        assert np.array_equal(vq.reshape(2, -1, 8, 128)[:, idx].reshape(-1), vd)
