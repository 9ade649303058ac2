"""ctypes access to the CPU oracle (oracle/liboracle.so).

Test infrastructure only: used by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  Builds the oracle with g++ if it is missing.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_PATH = os.path.join(ROOT, "oracle", "liboracle.so")

OK, INVALID_ARG, UNSUPPORTED, NO_MEMORY, BUFFER_TOO_SMALL, CORRUPT, PLAN_MISMATCH, RANGE = range(8)
INTERNAL = 99

STAGE_IDS = {name: i + 1 for i, name in enumerate(
    ("TUPL2_1", "TUPL4_1", "TUPL8_1", "DIFF1", "DIFF2", "DIFF4", "DIFF8",
     "BIT_1", "BIT_2", "BIT_4", "BIT_8", "RZE_1", "RZE_2", "RZE_4", "RZE_8"))}


class Cfg(C.Structure):
    _fields_ = [("layers", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32),
                ("dtype", C.c_int32),
                ("k_bits", C.c_int32), ("k_axis", C.c_int32), ("k_group", C.c_int32), ("k_hadamard", C.c_int32),
                ("v_bits", C.c_int32), ("v_axis", C.c_int32), ("v_group", C.c_int32), ("v_hadamard", C.c_int32),
                ("seed", C.c_uint64), ("stages", C.c_uint8 * 4), ("chunk_bytes", C.c_uint32),
                ("k_delta", C.c_int32), ("v_delta", C.c_int32)]


_lib = None


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIB_PATH):
        subprocess.check_call(["sh", os.path.join(ROOT, "oracle", "build_oracle.sh")])
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        sig = {
            "kvco_splitmix64": (C.c_uint64, [C.POINTER(C.c_uint64)]),
            "kvco_signs": (C.c_int, [C.c_uint64, C.c_int, P]),
            "kvco_norm_const": (C.c_float, [C.c_int]),
            "kvco_fwht": (C.c_int, [P, C.c_int]),
            "kvco_f16_to_f32": (C.c_float, [C.c_uint16]),
            "kvco_f32_to_f16_rn": (C.c_uint16, [C.c_float]),
            "kvco_f32_to_f16_rd": (C.c_uint16, [C.c_float]),
            "kvco_f32_to_f16_ru": (C.c_uint16, [C.c_float]),
            "kvco_bf16_to_f32": (C.c_float, [C.c_uint16]),
            "kvco_f32_to_bf16_rn": (C.c_uint16, [C.c_float]),
            "kvco_group_params": (C.c_int, [P, C.c_int, C.c_int, C.c_float, P, P, P]),
            "kvco_quantize_group": (C.c_int, [P, C.c_int, C.c_int, C.c_float, C.c_uint16, C.c_uint16, C.c_float, P]),
            "kvco_codes_bytes": (C.c_int64, [P, C.c_int, C.c_int]),
            "kvco_params_bytes": (C.c_int64, [P, C.c_int, C.c_int]),
            "kvco_quantize_tensor": (C.c_int, [P, C.c_int, P, C.c_int, P, P]),
            "kvco_dequantize_tensor": (C.c_int, [P, C.c_int, P, P, C.c_int, P]),
            "kvco_delta_forward": (C.c_int, [P, C.c_int, P, C.c_int, P]),
            "kvco_delta_inverse": (C.c_int, [P, C.c_int, P, C.c_int]),
            "kvco_stage_encode": (C.c_int, [C.c_int, P, C.c_size_t, P, C.c_size_t, P]),
            "kvco_stage_decode": (C.c_int, [C.c_int, P, C.c_size_t, P, C.c_size_t]),
            "kvco_chunk_encode": (C.c_int, [P, P, C.c_size_t, P, P, P]),
            "kvco_chunk_decode": (C.c_int, [P, P, C.c_size_t, C.c_int, P, C.c_size_t]),
            "kvco_max_stream_bytes": (C.c_int64, [P, C.c_int]),
            "kvco_encode": (C.c_int, [P, P, P, C.c_int, P, C.c_size_t, P]),
            "kvco_max_stream_bytes_mixed": (C.c_int64, [P, P, C.c_int]),
            "kvco_encode_mixed": (C.c_int, [P, P, P, P, C.c_int, P, C.c_size_t, P]),
            "kvco_stream_info": (C.c_int, [P, C.c_size_t, P, P]),
            "kvco_decode": (C.c_int, [P, C.c_size_t, P, P, C.c_size_t]),
            "kvco_encode_paged": (C.c_int, [P, P, P, C.c_int64, C.c_int, P, C.c_int, P, C.c_int,
                                            P, C.c_size_t, P, P]),
            "kvco_decode_paged": (C.c_int, [P, P, C.c_int, P, P, C.c_int64, C.c_int, P, C.c_int, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def cfg_from_workload(wl, layers=None) -> Cfg:
    c = Cfg()
    c.layers = wl.layers if layers is None else layers
    c.heads, c.head_dim = wl.heads, wl.head_dim
    c.dtype = 0 if wl.dtype == "f16" else 1
    for pre, pol in (("k", wl.k), ("v", wl.v)):
        setattr(c, pre + "_bits", pol.bits)
        setattr(c, pre + "_axis", 0 if pol.axis == "token" else 1)
        setattr(c, pre + "_group", pol.group)
        setattr(c, pre + "_hadamard", 1 if pol.hadamard else 0)
        setattr(c, pre + "_delta", pol.delta)
    c.seed = wl.sign_seed
    ids = [STAGE_IDS[s] for s in wl.stages] + [0] * (4 - len(wl.stages))
    for i in range(4):
        c.stages[i] = ids[i]
    c.chunk_bytes = wl.chunk_bytes
    return c


# ---------------------------------------------------------------- scalar helpers

def signs(seed: int, n: int) -> np.ndarray:
    out = np.zeros(n, dtype=np.int8)
    assert lib().kvco_signs(seed, n, _p(out)) == OK
    return out


def fwht(v: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(v, dtype=np.float32).copy()
    assert lib().kvco_fwht(_p(a), a.size) == OK
    return a


def group_params(z: np.ndarray, bits: int, c: float):
    z = np.ascontiguousarray(z, dtype=np.float32)
    s = np.zeros(1, np.uint16); m = np.zeros(1, np.uint16); inv = np.zeros(1, np.float32)
    st = lib().kvco_group_params(_p(z), z.size, bits, c, _p(s), _p(m), _p(inv))
    return st, int(s[0]), int(m[0]), float(inv[0])


def quantize_group(z: np.ndarray, bits: int, c: float, s: int, m: int, inv: float):
    z = np.ascontiguousarray(z, dtype=np.float32)
    q = np.zeros(z.size, np.uint8)
    st = lib().kvco_quantize_group(_p(z), z.size, bits, c, s, m, inv, _p(q))
    return st, q


# ---------------------------------------------------------------- tensors

def quantize_tensor(cfg: Cfg, which: int, x_u16: np.ndarray, tokens: int):
    L = lib()
    nc = L.kvco_codes_bytes(C.byref(cfg), which, tokens)
    npar = L.kvco_params_bytes(C.byref(cfg), which, tokens)
    codes = np.zeros(max(nc, 1), np.uint8)
    params = np.zeros(max(npar, 1), np.uint8)
    x = np.ascontiguousarray(x_u16, dtype=np.uint16)
    st = L.kvco_quantize_tensor(C.byref(cfg), which, _p(x), tokens, _p(codes), _p(params))
    return st, codes[:nc], params[:npar]


def dequantize_tensor(cfg: Cfg, which: int, codes: np.ndarray, params: np.ndarray, tokens: int):
    x = np.zeros(max(cfg.layers * tokens * cfg.heads * cfg.head_dim, 1), np.uint16)
    codes = np.ascontiguousarray(codes, np.uint8)
    params = np.ascontiguousarray(params, np.uint8)
    st = lib().kvco_dequantize_tensor(C.byref(cfg), which, _p(codes), _p(params), tokens, _p(x))
    return st, x[:cfg.layers * tokens * cfg.heads * cfg.head_dim]


def delta_forward(cfg: Cfg, which: int, x_u16: np.ndarray, tokens: int):
    x = np.ascontiguousarray(x_u16, dtype=np.uint16).reshape(-1)
    y = np.zeros(max(x.size, 1), np.uint16)
    st = lib().kvco_delta_forward(C.byref(cfg), which, _p(x), tokens, _p(y))
    return st, y[:x.size]


def delta_inverse(cfg: Cfg, which: int, y_u16: np.ndarray, tokens: int):
    x = np.array(y_u16, dtype=np.uint16).reshape(-1)
    st = lib().kvco_delta_inverse(C.byref(cfg), which, _p(x), tokens)
    return st, x


# ---------------------------------------------------------------- lossless

def stage_encode(stage: int, data: np.ndarray):
    data = np.ascontiguousarray(data, np.uint8)
    cap = data.size * 2 + 64
    out = np.zeros(cap, np.uint8)
    n = C.c_size_t(0)
    st = lib().kvco_stage_encode(stage, _p(data), data.size, _p(out), cap, C.byref(n))
    return st, out[:n.value]


def stage_decode(stage: int, data: np.ndarray, n: int):
    data = np.ascontiguousarray(data, np.uint8)
    out = np.zeros(max(n, 1), np.uint8)
    st = lib().kvco_stage_decode(stage, _p(data), data.size, _p(out), n)
    return st, out[:n]


def chunk_encode(stages, data: np.ndarray):
    st_arr = (C.c_uint8 * 4)(*(list(stages) + [0] * (4 - len(stages))))
    data = np.ascontiguousarray(data, np.uint8)
    out = np.zeros(max(data.size, 1), np.uint8)
    stored = C.c_size_t(0)
    raw = C.c_int(0)
    st = lib().kvco_chunk_encode(st_arr, _p(data), data.size, _p(out), C.byref(stored), C.byref(raw))
    return st, out[:stored.value], raw.value


def chunk_decode(stages, data: np.ndarray, raw: int, n: int):
    st_arr = (C.c_uint8 * 4)(*(list(stages) + [0] * (4 - len(stages))))
    data = np.ascontiguousarray(data, np.uint8)
    out = np.zeros(max(n, 1), np.uint8)
    st = lib().kvco_chunk_decode(st_arr, _p(data), data.size, raw, _p(out), n)
    return st, out[:n]


# ---------------------------------------------------------------- streams

def max_stream_bytes(cfg: Cfg, tokens: int) -> int:
    return lib().kvco_max_stream_bytes(C.byref(cfg), tokens)


def encode(cfg: Cfg, k_u16: np.ndarray, v_u16: np.ndarray, tokens: int):
    cap = max_stream_bytes(cfg, tokens)
    out = np.zeros(cap, np.uint8)
    nb = C.c_size_t(0)
    k = np.ascontiguousarray(k_u16, np.uint16)
    v = np.ascontiguousarray(v_u16, np.uint16)
    st = lib().kvco_encode(C.byref(cfg), _p(k), _p(v), tokens, _p(out), cap, C.byref(nb))
    return st, out[:nb.value]


def encode_mixed(cfg: Cfg, bits: np.ndarray, k_u16: np.ndarray, v_u16: np.ndarray, tokens: int):
    """bits: [2, layers, heads] of 2, 4, 8 or 16."""
    b = np.ascontiguousarray(bits, np.uint8)
    cap = lib().kvco_max_stream_bytes_mixed(C.byref(cfg), _p(b), tokens)
    if cap < 0:
        return INVALID_ARG, np.zeros(0, np.uint8)
    out = np.zeros(cap, np.uint8)
    nb = C.c_size_t(0)
    k = np.ascontiguousarray(k_u16, np.uint16)
    v = np.ascontiguousarray(v_u16, np.uint16)
    st = lib().kvco_encode_mixed(C.byref(cfg), _p(b), _p(k), _p(v), tokens, _p(out), cap, C.byref(nb))
    return st, out[:nb.value]


def stream_info(stream: np.ndarray):
    cfg = Cfg()
    t = C.c_int(0)
    s = np.ascontiguousarray(stream, np.uint8)
    st = lib().kvco_stream_info(_p(s), s.size, C.byref(cfg), C.byref(t))
    return st, cfg, t.value


def decode(stream: np.ndarray, elems: int):
    s = np.ascontiguousarray(stream, np.uint8)
    k = np.zeros(max(elems, 1), np.uint16)
    v = np.zeros(max(elems, 1), np.uint16)
    st = lib().kvco_decode(_p(s), s.size, _p(k), _p(v), elems)
    return st, k[:elems], v[:elems]


def encode_paged(cfg: Cfg, k_pool, v_pool, num_blocks, page_tokens, block_table, seq_lens):
    R = len(seq_lens)
    cap = sum(max_stream_bytes(cfg, int(t)) for t in seq_lens) + 16
    out = np.zeros(cap, np.uint8)
    offs = np.zeros(R + 1, np.uint64)
    nb = C.c_size_t(0)
    kp = np.ascontiguousarray(k_pool, np.uint16)
    vp = np.ascontiguousarray(v_pool, np.uint16)
    bt = np.ascontiguousarray(block_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    st = lib().kvco_encode_paged(C.byref(cfg), _p(kp), _p(vp), num_blocks, page_tokens, _p(bt),
                                 bt.shape[1], _p(sl), R, _p(out), cap, _p(offs), C.byref(nb))
    return st, out[:nb.value], offs


def decode_paged(stream, offs, k_pool, v_pool, num_blocks, page_tokens, block_table, seq_lens):
    s = np.ascontiguousarray(stream, np.uint8)
    bt = np.ascontiguousarray(block_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    st = lib().kvco_decode_paged(_p(s), _p(np.ascontiguousarray(offs, np.uint64)), len(seq_lens),
                                 _p(k_pool), _p(v_pool), num_blocks, page_tokens, _p(bt), bt.shape[1], _p(sl))
    return st
