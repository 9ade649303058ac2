"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
identical seeded inputs.

Cases span several tiles and chunks with ragged tails, both dtypes, 2/4/8-bit
codes, per-token groups of 16..128 and per-channel groups of 32/64, partial
token groups, empty and one-token inputs, zero-rich inputs whose chunks
compress (both standard lossless pipelines and a generic DIFF pipeline), the
paged path, corrupt streams and out-of-range parameters.  Shapes follow the
workloads of kvc_workloads at reduced layer/token counts."""
import numpy as np
import pytest
import torch

import kvc_workloads as W
import oracle_api as O
from gpu_helpers import (DEV, assert_encode_parity, assert_values_close, chunk_kinds, chunk_layout, compare_encode, gpu_decode,
                         gpu_encode, log, oracle_encode, to_u16)
import kv_cache_compression_kvc_amd as K

pytestmark = pytest.mark.gpu

TP = W.TensorPolicy


def run_case(wl, L, T, seed=1, zero_rich=False, check_decode=True, zero_frac=0.9):
    log(f"case {wl.name} L={L} T={T} k={wl.k} v={wl.v} stages={wl.stages} cb={wl.chunk_bytes} zero_rich={zero_rich}")
    if zero_rich:
        k, v = W.zero_rich_kv(wl, L, T, seed=seed, zero_frac=zero_frac)
    else:
        k, v = W.dense_kv(wl, layers=L, tokens=T, seed=seed)
    ku, vu = to_u16(k), to_u16(v)
    st, ref = oracle_encode(wl, ku, vu, T, L)
    assert st == O.OK
    plan, got, ws = gpu_encode(wl, k.to(DEV), v.to(DEV), T, L)
    stats = compare_encode(got, ref, wl, L, T)
    stats["chunks_raw"], stats["chunks_compressed"] = chunk_kinds(ref, wl, L, T)
    log(f"  encode: {stats}")
    assert_encode_parity(stats)
    if check_decode:
        n = L * T * wl.heads * wl.head_dim
        st, kd, vd = O.decode(ref, n)
        assert st == O.OK
        # the GPU decoder on the oracle's stream: bit for bit
        st, kg, vg = gpu_decode(plan, ref, wl, T, L)
        assert st == K.OK, K.status_string(st)
        ek = assert_values_close(to_u16(kg).reshape(-1), kd, wl.dtype)
        ev = assert_values_close(to_u16(vg).reshape(-1), vd, wl.dtype)
        log(f"  decode exact fraction K {ek:.6f} V {ev:.6f}")
        assert ek == 1.0 and ev == 1.0
        # the GPU decoder on the GPU's own stream, against the oracle's
        # reconstruction (bit for bit when the streams are identical)
        if not stats["identical"]:
            st, kg, vg = gpu_decode(plan, got, wl, T, L)
            assert st == K.OK, K.status_string(st)
            ek = assert_values_close(to_u16(kg).reshape(-1), kd, wl.dtype)
            ev = assert_values_close(to_u16(vg).reshape(-1), vd, wl.dtype)
            log(f"  own-stream decode exact fraction K {ek:.6f} V {ev:.6f}")
    return stats


C1 = W.WORKLOADS["c1_single_layer_512"]
C2 = W.WORKLOADS["c2_llama8b_4k"]
C3 = W.WORKLOADS["c3_llama70b_32k"]
C5 = W.WORKLOADS["c5_llama70b_128k"]


def test_c1_full():
    s = run_case(C1, 1, 512)
    assert s["identical"]


def test_c2_shape_ragged_tokens():
    run_case(C2, 2, 600)


def test_c3_shape_bf16_mixed_precision():
    run_case(C3, 2, 640)


@pytest.mark.parametrize("T", [150, 37, 1, 64, 65])
def test_c3_partial_token_groups(T):
    run_case(C3.with_(chunk_bytes=8192), 2, T)


def test_c5_shape_int2():
    run_case(C5, 2, 384)


def test_empty_input():
    wl = C3
    plan, got, ws = gpu_encode(wl, torch.zeros(1, device=DEV, dtype=wl.torch_dtype),
                               torch.zeros(1, device=DEV, dtype=wl.torch_dtype), 0, 2)
    st, ref = oracle_encode(wl, np.zeros(0, np.uint16), np.zeros(0, np.uint16), 0, 2)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("bits,axis,group", [(8, "token", 32), (4, "token", 16), (2, "token", 64),
                                             (8, "channel", 64), (2, "channel", 32), (4, "channel", 32),
                                             (4, "token", 128), (8, "token", 128)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_policy_grid(bits, axis, group, dtype):
    wl = C1.with_(dtype=dtype, k=TP(bits, axis, group), v=TP(bits, "token", 32), chunk_bytes=8192,
                  name=f"grid_{bits}_{axis}_{group}_{dtype}")
    run_case(wl, 2, 200)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_channel_groups_of_32_with_a_long_tail(bits, dtype):
    # T = 250: the last 64-token tile holds one complete 32-token group and
    # one of 26 tokens (the tail tile's second half is partial)
    wl = C1.with_(dtype=dtype, k=TP(bits, "channel", 32), v=TP(bits, "token", 32), chunk_bytes=8192,
                  name=f"tail32_{bits}_{dtype}")
    s = run_case(wl, 2, 250)
    assert s["identical"]


@pytest.mark.parametrize("stages", [("TUPL8_1", "BIT_8", "RZE_2"), ("TUPL8_1", "RZE_2"),
                                    ("DIFF1", "RZE_1"), ("TUPL4_1", "DIFF4", "BIT_4", "RZE_4"), ()])
def test_zero_rich_inputs_compress(stages):
    wl = C3.with_(stages=stages, chunk_bytes=8192, name="zero_rich")
    s = run_case(wl, 2, 512, zero_rich=True)
    assert s["identical"]


@pytest.mark.parametrize("T", [4096, 4097])
def test_decode_front_at_the_small_call_limit(T):
    # one layer of 4-bit per-token keys and values in 4 KiB chunks: 2 ceil(T / 8)
    # chunks, 1024 at T = 4096 (a decode whose reset, table scan and
    # classification are one launch) and 1026 at T = 4097 (the multi-kernel
    # front); half-zero input, so that raw and compressed chunks are classified
    wl = C1.with_(chunk_bytes=4096, name="front_limit")
    s = run_case(wl, 1, T, zero_rich=True, zero_frac=0.5, seed=31)
    assert s["identical"]
    assert s["chunks_compressed"] >= 1 and s["chunks_raw"] >= 1, s


@pytest.mark.parametrize("stages", [("TUPL8_1", "BIT_8", "RZE_2"), ("TUPL8_1", "RZE_2")])
@pytest.mark.parametrize("T", [528, 516])
def test_word_parallel_lossless_full_chunks(stages, T):
    # 64 KiB chunks, half of the 64-token blocks zero: most chunks compress and
    # go through the word-parallel kernels; T = 528 leaves partial last chunks
    # whose size is a multiple of 4096 bytes, T = 516 one that is not
    wl = C3.with_(stages=stages, chunk_bytes=65536, name="word_parallel")
    s = run_case(wl, 2, T, zero_rich=True, zero_frac=0.5, seed=3)
    assert s["identical"]
    assert s["chunks_compressed"] >= 8, s


@pytest.mark.parametrize("stages", [("TUPL8_1", "BIT_8", "RZE_2"), ("TUPL8_1", "RZE_2")])
@pytest.mark.parametrize("k,v", [(TP(8, "channel", 64), TP(4, "token", 64)),
                                 (TP(4, "channel", 64), TP(8, "token", 16)),
                                 (TP(2, "channel", 64), TP(2, "token", 128))])
def test_fused_size_counts(stages, k, v):
    # the fused encoders count the non-zero RZE words of the chunks they write
    # (all code widths); compressed-chunk sizes must equal the oracle's
    wl = C3.with_(stages=stages, k=k, v=v, chunk_bytes=16384, name="fused_counts")
    s = run_case(wl, 2, 256, zero_rich=True, zero_frac=0.5, seed=11)
    assert s["identical"]
    assert s["chunks_compressed"] >= 4, s


@pytest.mark.parametrize("zero_frac,L,T", [(1.0, 8, 2048), (0.5, 8, 1024), (0.97, 4, 4096)])
def test_single_pass_placement(zero_frac, L, T):
    # a dense encode ends with one in-place pass over 64 KiB chunks: with
    # all-zero input every chunk shrinks to its bitmap and lands far below its
    # codes, so each write waits on announcements spanning many groups of 64
    # chunks; mixed inputs move raw chunks behind compressed ones
    wl = C3.with_(chunk_bytes=65536, name="placement")
    s = run_case(wl, L, T, zero_rich=True, zero_frac=zero_frac, seed=21)
    assert s["identical"]
    assert s["chunks_compressed"] >= 8, s


@pytest.mark.parametrize("stages", [("TUPL8_1", "BIT_8", "RZE_2"), ("TUPL8_1", "RZE_2")])
@pytest.mark.parametrize("cb", [4096, 12288, 45056])
def test_chunk_sizes_not_powers_of_two(stages, cb):
    # chunk sizes the placement, the scan and the decoders locate by division
    # (12288 and 45056 bytes) and the smallest one (4096), with ragged tails
    wl = C3.with_(stages=stages, chunk_bytes=cb, name="chunk_sizes")
    s = run_case(wl, 2, 448, zero_rich=True, zero_frac=0.5, seed=17)
    assert s["identical"]
    assert s["chunks_compressed"] >= 4, s


def test_range_error_is_reported():
    wl = C1
    k = torch.full((1, 64, 8, 128), 60000.0, dtype=torch.float16)
    v = torch.zeros_like(k)
    plan = K.Plan(K.config_from_workload(wl, max_tokens=64, layers=1))
    ms, wsb = plan.sizes(64)
    out = torch.empty(ms, dtype=torch.uint8, device=DEV)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    with pytest.raises(K.KvcError) as e:
        plan.encode(k.to(DEV), v.to(DEV), 64, out, ws)
    assert e.value.status == K.ERR_RANGE
    st, _ = oracle_encode(wl, to_u16(k), to_u16(v), 64, 1)
    assert st == O.RANGE


def test_corrupt_and_mismatched_streams_are_detected():
    wl = C3.with_(chunk_bytes=8192)
    L, T = 2, 256
    k, v = W.zero_rich_kv(wl, L, T, seed=5)
    st, ref = oracle_encode(wl, to_u16(k), to_u16(v), T, L)
    plan = K.Plan(K.config_from_workload(wl, max_tokens=T + 64, layers=L))
    st, _, _ = gpu_decode(plan, ref, wl, T, L)
    assert st == K.OK
    bad = ref.copy(); bad[0] ^= 1                                  # magic
    assert gpu_decode(plan, bad, wl, T, L)[0] == K.ERR_CORRUPT_STREAM
    bad = ref.copy(); bad[12] ^= 1                                 # token count
    assert gpu_decode(plan, bad, wl, T, L)[0] == K.ERR_PLAN_MISMATCH
    rng = np.random.default_rng(7)
    nch = 32 + 16                                                # K and V chunks of 8 KiB
    for _ in range(6):
        bad = ref.copy()
        pos = 64 + 4 * int(rng.integers(0, nch)) + int(rng.integers(0, 4))
        bad[pos] ^= np.uint8(1 << int(rng.integers(0, 8)))
        st = gpu_decode(plan, bad, wl, T, L)[0]
        assert st in (K.ERR_CORRUPT_STREAM,), st
    with pytest.raises(K.KvcError) as e:                          # truncated below the fixed sections
        gpu_decode(plan, ref[:100], wl, T, L)
    assert e.value.status == K.ERR_CORRUPT_STREAM


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("g", [16, 64, 128])
@pytest.mark.parametrize("cb", [8192, 65536])
def test_value_reconstruct_decodes_compressed_chunks(dtype, g, cb):
    # 2-bit per-token values with the standard pipeline: the reconstruct
    # kernel decodes their compressed chunks itself, for every group size
    # and both dtypes; T = 1000 leaves a last chunk whose size is not a
    # multiple of 4 KiB (decoded by the lossless pass instead)
    wl = C3.with_(dtype=dtype, v=TP(2, "token", g), chunk_bytes=cb, name="value_chunks")
    s = run_case(wl, 2, 1000, zero_rich=True, zero_frac=0.5, seed=23)
    assert s["identical"]
    assert s["chunks_compressed"] >= 2, s


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("cb,heads", [(8192, 8), (65536, 8), (8192, 2)])
def test_keys_with_raw_and_compressed_chunks(dtype, bits, cb, heads):
    # 2- or 4-bit keys in 64-token per-channel groups with the standard
    # pipeline: raw chunks are read in place by the reconstruct kernel,
    # compressed ones decoded by the lossless pass; zero-rich values give
    # both kinds in one call
    wl = C3.with_(dtype=dtype, heads=heads, k=TP(bits, "channel", 64), chunk_bytes=cb, name="key_chunks")
    s = run_case(wl, 2, 1024, zero_rich=True, zero_frac=0.5, seed=29)
    assert s["identical"]
    assert s["chunks_compressed"] >= 2 and s["chunks_raw"] >= 1, s


@pytest.mark.parametrize("section", [0, 1])
def test_zeroed_word_under_a_set_bitmap_bit_is_detected(section):
    # TUPL8_1 -> BIT_8 -> RZE_2 chunks whose bitmap still matches their size
    # but one of whose kept words was zeroed: keys go through the lossless
    # pass, 2-bit per-token values through the reconstruct kernel's own chunk
    # decoder; both must report the stream corrupt
    wl = C3.with_(chunk_bytes=8192, name="zeroed_word")
    L, T = 2, 512
    k, v = W.zero_rich_kv(wl, L, T, seed=9, zero_frac=0.5)
    st, ref = oracle_encode(wl, to_u16(k), to_u16(v), T, L)
    assert st == O.OK
    plan = K.Plan(K.config_from_workload(wl, max_tokens=T, layers=L))
    assert gpu_decode(plan, ref, wl, T, L)[0] == K.OK
    comp = [c for c in chunk_layout(ref, wl, L, T) if c[0] == section and not c[5] and c[4] > c[2] // 16]
    assert len(comp) >= 2, comp
    rng = np.random.default_rng(section)
    # random words, and the first and the last stored word of a chunk (the
    # last one shares its 16-byte line with bytes past the chunk's words)
    picks = [(c, None) for c in (comp[0], comp[-1], comp[int(rng.integers(0, len(comp)))])]
    picks += [(comp[0], "first"), (comp[0], "last"), (comp[-1], "last")]
    for (w, i, n, pos, stored, raw), which in picks:
        words = np.frombuffer(ref[pos + n // 16:pos + stored].tobytes(), np.uint16)
        assert (words != 0).all()
        bad = ref.copy()
        k = {None: int(rng.integers(0, words.size)), "first": 0, "last": words.size - 1}[which]
        at = pos + n // 16 + 2 * k
        bad[at:at + 2] = 0
        log(f"  section {w} chunk {i}: zeroed the word at byte {at - pos} of {stored}")
        assert gpu_decode(plan, bad, wl, T, L)[0] == K.ERR_CORRUPT_STREAM



def test_zeroed_last_word_before_a_line_end_is_detected():
    # 4-bit per-token keys in 4 KiB chunks: compressed chunks whose stored
    # words end inside a 16-byte line; zeroing the last word (the lossless
    # decode checks stored words per line, masking the bytes past them) or a
    # word of that line must still mark the stream corrupt
    wl = C1.with_(chunk_bytes=4096, name="partial_line")
    L, T = 1, 1024
    k, v = W.zero_rich_kv(wl, L, T, seed=31, zero_frac=0.5)
    st, ref = oracle_encode(wl, to_u16(k), to_u16(v), T, L)
    assert st == O.OK
    plan = K.Plan(K.config_from_workload(wl, max_tokens=T, layers=L))
    assert gpu_decode(plan, ref, wl, T, L)[0] == K.OK
    odd = [c for c in chunk_layout(ref, wl, L, T)
           if c[0] == 0 and not c[5] and c[4] > c[2] // 16 and (c[4] - c[2] // 16) % 16 != 0]
    assert len(odd) >= 2, odd
    for w, i, n, pos, stored, raw in odd[:3]:
        nw = (stored - n // 16) // 2
        for k_ in (nw - 1, (nw - 1) & ~7):                  # the last word, the first word of its line
            bad = ref.copy()
            at = pos + n // 16 + 2 * k_
            bad[at:at + 2] = 0
            log(f"  chunk {i}: zeroed word {k_} of {nw}")
            assert gpu_decode(plan, bad, wl, T, L)[0] == K.ERR_CORRUPT_STREAM

def test_paged_matches_oracle():
    wl = W.WORKLOADS["c4_paged_llama8b"].with_(layers=2, chunk_bytes=8192)
    batch = W.paged_layout(wl, requests=6, min_len=5, max_len=300)
    log(f"paged lens {batch.seq_lens.tolist()} blocks {batch.num_blocks}")
    kp, vp = W.paged_pools(wl, batch)
    cfg = O.cfg_from_workload(wl)
    st, ref, ref_offs = O.encode_paged(cfg, to_u16(kp), to_u16(vp), batch.num_blocks, wl.page_tokens,
                                       batch.block_table, batch.seq_lens)
    assert st == O.OK
    plan = K.Plan(K.config_from_workload(wl, max_tokens=0))
    ms, wsb = plan.sizes_paged(batch.seq_lens)
    out = torch.full((ms,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device=DEV)
    offs = torch.zeros(len(batch.seq_lens) + 1, dtype=torch.int64, device=DEV)
    bt = torch.from_numpy(batch.block_table).to(DEV)
    n = plan.encode_paged(kp.to(DEV), vp.to(DEV), batch.num_blocks, bt, batch.seq_lens, out, offs, ws)
    got = out[:n].cpu().numpy()
    assert np.array_equal(offs.cpu().numpy().astype(np.uint64), ref_offs)
    assert np.array_equal(got, ref)
    # decode into a second pool through an independent page map
    dst = W.paged_layout(wl, requests=6, min_len=5, max_len=300, stream=1)
    kq = torch.zeros_like(kp, device=DEV)
    vq = torch.zeros_like(vp, device=DEV)
    btd = torch.from_numpy(dst.block_table).to(DEV)
    s = torch.from_numpy(ref).to(DEV)
    plan.decode_paged(s, ref.size, offs, dst.seq_lens, kq, vq, dst.num_blocks, btd, ws)
    assert plan.query_status(ws) == K.OK
    kqo = np.zeros_like(to_u16(kp)); vqo = np.zeros_like(to_u16(vp))
    st = O.decode_paged(ref, ref_offs, kqo, vqo, dst.num_blocks, wl.page_tokens, dst.block_table, dst.seq_lens)
    assert st == O.OK
    assert np.array_equal(to_u16(kq), kqo) and np.array_equal(to_u16(vq), vqo)


def _paged_batch_with_lens(wl, lens, seed):
    """A PagedBatch of the given request lengths over a pool of exactly the
    pages they need, permuted by `seed`."""
    P = wl.page_tokens
    pages = (lens + P - 1) // P
    nb = int(pages.sum())
    maxb = max(1, int(pages.max()))
    perm = np.random.default_rng([seed, 13]).permutation(nb).astype(np.int32)
    bt = np.full((len(lens), maxb), -1, dtype=np.int32)
    pos = 0
    for r in range(len(lens)):
        bt[r, :pages[r]] = perm[pos:pos + pages[r]]
        pos += pages[r]
    return W.PagedBatch(seq_lens=lens.astype(np.int32), block_table=bt, num_blocks=nb, max_blocks=maxb)


def test_paged_many_requests_with_empty_ones():
    # 40 requests, six of them empty (first, last, two adjacent): empty
    # requests share their first tile with the next request, and the tile ->
    # request table of this call (about 9150 tiles per tensor) needs a shift of
    # 2, so the lookups go through table brackets of several requests; every
    # stream, offset and reconstructed value must equal the oracle's
    wl = W.WORKLOADS["c4_paged_llama8b"].with_(layers=2, chunk_bytes=8192)
    lens = W.paged_layout(wl, requests=40, min_len=1, max_len=900).seq_lens.copy()
    lens[[0, 7, 13, 14, 26, 39]] = 0
    batch = _paged_batch_with_lens(wl, lens, seed=5)
    log(f"paged lens {batch.seq_lens.tolist()} blocks {batch.num_blocks}")
    kp, vp = W.paged_pools(wl, batch)
    st, ref, ref_offs = O.encode_paged(O.cfg_from_workload(wl), to_u16(kp), to_u16(vp), batch.num_blocks,
                                       wl.page_tokens, batch.block_table, batch.seq_lens)
    assert st == O.OK
    plan = K.Plan(K.config_from_workload(wl, max_tokens=0))
    ms, wsb = plan.sizes_paged(batch.seq_lens)
    out = torch.full((ms,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device=DEV)
    offs = torch.zeros(len(lens) + 1, dtype=torch.int64, device=DEV)
    bt = torch.from_numpy(batch.block_table).to(DEV)
    n = plan.encode_paged(kp.to(DEV), vp.to(DEV), batch.num_blocks, bt, batch.seq_lens, out, offs, ws)
    assert np.array_equal(offs.cpu().numpy().astype(np.uint64), ref_offs)
    assert np.array_equal(out[:n].cpu().numpy(), ref)
    dst = _paged_batch_with_lens(wl, lens, seed=6)
    kq = torch.zeros_like(kp, device=DEV)
    vq = torch.zeros_like(vp, device=DEV)
    plan.decode_paged(torch.from_numpy(ref).to(DEV), ref.size, offs, dst.seq_lens, kq, vq, dst.num_blocks,
                      torch.from_numpy(dst.block_table).to(DEV), ws)
    assert plan.query_status(ws) == K.OK
    kqo = np.zeros_like(to_u16(kp)); vqo = np.zeros_like(to_u16(vp))
    st = O.decode_paged(ref, ref_offs, kqo, vqo, dst.num_blocks, wl.page_tokens, dst.block_table, dst.seq_lens)
    assert st == O.OK
    assert np.array_equal(to_u16(kq), kqo) and np.array_equal(to_u16(vq), vqo)


@pytest.mark.parametrize("kbits,vbits,stages,round_lens", [(4, 4, W.BYTE_SHUFFLE_RZE, 1),
                                                            (8, 2, W.BYTE_SHUFFLE_RZE, 1),
                                                            (4, 2, W.LLAMA_TUPL_BIT_RZE, 4),
                                                            (4, 2, W.LLAMA_TUPL_BIT_RZE, 1)])
def test_paged_mixed_raw_and_compressed_chunks(kbits, vbits, stages, round_lens):
    """Paged pools with half of the pages zero and 4 KiB chunks: compressed and
    raw chunks alternate, and the tiles (32 vectors, starting at layer
    boundaries that are not chunk-aligned) straddle pairs of chunks of every
    kind.  The encoders split a straddling tile's non-zero word count between
    its chunks; a reconstruct tile whose chunks are all raw reads the stream
    in place, the others read the codes area, which must then hold the raw
    neighbours of compressed chunks too.  With TUPL8_1 -> BIT_8 -> RZE_2 the
    encoders count only when every layer starts on a 1 KiB boundary (lengths
    rounded to multiples of 4 here); the ragged case takes the size pass."""
    TP = W.TensorPolicy
    wl = W.WORKLOADS["c4_paged_llama8b"].with_(layers=3, chunk_bytes=4096, k=TP(kbits, "token", 128),
                                                v=TP(vbits, "token", 32), stages=stages)
    batch = W.paged_layout(wl, requests=8, min_len=5, max_len=300)
    batch.seq_lens[:] = np.maximum(round_lens, batch.seq_lens // round_lens * round_lens)
    kp, vp = W.paged_pools(wl, batch)
    rng = np.random.default_rng(kbits)
    for pool in (kp, vp):
        zero = torch.from_numpy(rng.random(pool.shape[:2]) < 0.5)
        pool[zero] = 0
    log(f"paged mixed-chunk case K{kbits} V{vbits} {stages} lens {batch.seq_lens.tolist()}")
    cfg = O.cfg_from_workload(wl)
    st, ref, ref_offs = O.encode_paged(cfg, to_u16(kp), to_u16(vp), batch.num_blocks, wl.page_tokens,
                                       batch.block_table, batch.seq_lens)
    assert st == O.OK
    plan = K.Plan(K.config_from_workload(wl, max_tokens=0))
    ms, wsb = plan.sizes_paged(batch.seq_lens)
    out = torch.full((ms,), 0xA5, dtype=torch.uint8, device=DEV)
    ws = torch.full((wsb,), 0x5A, dtype=torch.uint8, device=DEV)
    offs = torch.zeros(len(batch.seq_lens) + 1, dtype=torch.int64, device=DEV)
    bt = torch.from_numpy(batch.block_table).to(DEV)
    n = plan.encode_paged(kp.to(DEV), vp.to(DEV), batch.num_blocks, bt, batch.seq_lens, out, offs, ws)
    assert np.array_equal(offs.cpu().numpy().astype(np.uint64), ref_offs)
    assert np.array_equal(out[:n].cpu().numpy(), ref)
    assert ref.size < ms, "no chunk compressed"
    dst = W.paged_layout(wl, requests=8, min_len=5, max_len=300, stream=1)
    dst.seq_lens[:] = batch.seq_lens
    kq = torch.zeros_like(kp, device=DEV)
    vq = torch.zeros_like(vp, device=DEV)
    s = torch.from_numpy(ref).to(DEV)
    ws.fill_(0x5A)
    plan.decode_paged(s, ref.size, offs, dst.seq_lens, kq, vq, dst.num_blocks,
                      torch.from_numpy(dst.block_table).to(DEV), ws)
    assert plan.query_status(ws) == K.OK
    kqo = np.zeros_like(to_u16(kp)); vqo = np.zeros_like(to_u16(vp))
    st = O.decode_paged(ref, ref_offs, kqo, vqo, dst.num_blocks, wl.page_tokens, dst.block_table, dst.seq_lens)
    assert st == O.OK
    assert np.array_equal(to_u16(kq), kqo) and np.array_equal(to_u16(vq), vqo)


def test_encode_is_deterministic_and_async_size_matches():
    wl = C3
    L, T = 2, 256
    k, v = W.dense_kv(wl, layers=L, tokens=T, seed=9)
    plan, a, ws = gpu_encode(wl, k.to(DEV), v.to(DEV), T, L)
    _, b, _ = gpu_encode(wl, k.to(DEV), v.to(DEV), T, L, fill=0x11)
    assert np.array_equal(a, b)
    ms, wsb = plan.sizes(T)
    out = torch.empty(ms, dtype=torch.uint8, device=DEV)
    plan.encode(k.to(DEV), v.to(DEV), T, out, ws, sync=False)
    torch.cuda.synchronize()
    total = int(np.frombuffer(out[56:64].cpu().numpy().tobytes(), np.uint64)[0])
    assert total == a.size and np.array_equal(out[:total].cpu().numpy(), a)


GUARD = 1 << 16


def _guarded(nbytes, fill=0x33):
    t = torch.full((nbytes + 2 * GUARD,), fill, dtype=torch.uint8, device=DEV)
    return t, t[GUARD:GUARD + nbytes]


def _canaries_intact(big, fill=0x33):
    a = big.cpu().numpy()
    return bool((a[:GUARD] == fill).all() and (a[-GUARD:] == fill).all())


@pytest.mark.parametrize("name,T", [("c3_llama70b_32k", 1), ("c3_llama70b_32k", 37), ("c2_llama8b_4k", 150),
                                    ("c5_llama70b_128k", 65), ("c1_single_layer_512", 3)])
def test_no_writes_outside_the_given_buffers(name, T):
    """Encode and decode touch only their own buffers (regression: tile counts
    that overran a ragged tail wrote past the output)."""
    wl = W.WORKLOADS[name].with_(chunk_bytes=8192)
    L = 2
    log(f"guard case {name} T={T}")
    k, v = W.dense_kv(wl, layers=L, tokens=T, seed=3)
    n_el = L * T * wl.heads * wl.head_dim
    plan = K.Plan(K.config_from_workload(wl, max_tokens=T, layers=L))
    ms, wsb = plan.sizes(T)
    kb, kin = _guarded(2 * n_el); vb, vin = _guarded(2 * n_el)
    kin.copy_(k.reshape(-1).view(torch.uint8).to(DEV)); vin.copy_(v.reshape(-1).view(torch.uint8).to(DEV))
    ob, out = _guarded(ms)
    wb, ws = _guarded(wsb)
    n = plan.encode(kin.view(wl.torch_dtype), vin.view(wl.torch_dtype), T, out, ws)
    for big in (kb, vb, ob, wb):
        assert _canaries_intact(big)
    kdb, kd = _guarded(2 * n_el); vdb, vd = _guarded(2 * n_el)
    wb2, ws2 = _guarded(wsb)
    plan.decode(out, n, T, kd.view(wl.torch_dtype), vd.view(wl.torch_dtype), ws2)
    assert plan.query_status(ws2) == K.OK
    for big in (ob, kdb, vdb, wb2):
        assert _canaries_intact(big)
    st, ref = oracle_encode(wl, to_u16(k), to_u16(v), T, L)
    assert np.array_equal(out[:n].cpu().numpy(), ref)
