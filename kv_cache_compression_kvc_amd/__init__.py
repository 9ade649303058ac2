"""Python binding of libkvc (the C ABI declared in include/kvc.h and
include/kvc_select.h).

Argument marshalling only: every step of the compression path runs in the
library's HIP kernels.  PyTorch supplies device memory and streams.  The
binding fails loudly if the built library is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvc.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_NO_MEMORY, ERR_BUFFER_TOO_SMALL, ERR_CORRUPT_STREAM, \
    ERR_PLAN_MISMATCH, ERR_RANGE, ERR_HIP = range(9)
F16, BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 128 << 20     # KVC_NOALLOC_SCRATCH_BYTES
PER_TOKEN, PER_CHANNEL = 0, 1
STAGES = {name: i + 1 for i, name in enumerate(
    ("TUPL2_1", "TUPL4_1", "TUPL8_1", "DIFF1", "DIFF2", "DIFF4", "DIFF8",
     "BIT_1", "BIT_2", "BIT_4", "BIT_8", "RZE_1", "RZE_2", "RZE_4", "RZE_8"))}
KERNELS = ("ENCODE_K", "ENCODE_V", "LOSSLESS_ENC", "SCAN", "COMPACT", "LOSSLESS_DEC",
           "DECODE_K", "DECODE_V", "AUX", "DELTA")


class TensorPolicy(C.Structure):
    _fields_ = [("bits", C.c_uint8), ("axis", C.c_uint8), ("hadamard", C.c_uint8), ("reserved0", C.c_uint8),
                ("group", C.c_uint16), ("delta", C.c_uint16)]


class Config(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("layers", C.c_int32), ("max_tokens", C.c_int32),
                ("kv_heads", C.c_int32), ("head_dim", C.c_int32), ("dtype", C.c_int32),
                ("k", TensorPolicy), ("v", TensorPolicy), ("sign_seed", C.c_uint64),
                ("lossless", C.c_uint8 * 4), ("chunk_bytes", C.c_uint32), ("page_tokens", C.c_int32)]


class Profile(C.Structure):
    _fields_ = [("id", C.c_int32), ("bucket", C.c_int32), ("cr", C.c_double), ("s_enc", C.c_double),
                ("s_dec", C.c_double)]


class SelectorConfig(C.Structure):
    _fields_ = [("struct_size", C.c_uint32), ("fallback_id", C.c_int32), ("alpha", C.c_double),
                ("epsilon", C.c_double), ("cooldown_k", C.c_int32), ("cooldown_m", C.c_int32),
                ("cooldown_len", C.c_int32), ("reserved", C.c_int32), ("seed", C.c_uint64)]


class RequestContext(C.Structure):
    _fields_ = [("bucket", C.c_int32), ("reserved", C.c_int32), ("bandwidth", C.c_double),
                ("volume", C.c_double), ("t_model", C.c_double), ("t_slo", C.c_double)]


PROFILE_RAW = -1


class KvcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({last_error()})")


_lib = None


def lib():
    """The loaded libkvc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with kv_cache_compression_kvc_amd/build.py")
        L = C.CDLL(LIB_PATH)
        P, I32, I64, SZ, U64P = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t, C.POINTER(C.c_uint64)
        sig = {
            "kvc_plan": [C.POINTER(Config), C.POINTER(C.c_void_p)],
            "kvc_plan_mixed": [C.POINTER(Config), P, C.POINTER(C.c_void_p)],
            "kvc_plan_destroy": [P],
            "kvc_plan_sizes": [P, I64, C.POINTER(SZ), C.POINTER(SZ)],
            "kvc_plan_sizes_paged": [P, P, I32, C.POINTER(SZ), C.POINTER(SZ)],
            "kvc_encode": [P, P, P, I32, P, SZ, P, SZ, C.POINTER(SZ), P],
            "kvc_encode_noalloc": [P, P, P, I32, P, SZ, C.POINTER(SZ), P],
            "kvc_decode": [P, P, SZ, I32, P, P, P, SZ, P],
            "kvc_encode_paged": [P, P, P, I64, P, I32, P, I32, P, SZ, P, P, SZ, C.POINTER(SZ), P],
            "kvc_decode_paged": [P, P, SZ, P, P, I32, P, P, I64, P, I32, P, SZ, P],
            "kvc_query_status": [P, P, P],
            "kvc_profile_enable": [C.c_int],
            "kvc_profile_reset": [],
            "kvc_profile_query": [C.c_int, C.POINTER(C.c_double), C.POINTER(C.c_int64)],
            "kvc_probe_bandwidth": [P, P, I64, C.c_int, C.c_int, C.c_int, P, P],
            "kvc_predicted_jct": [C.POINTER(Profile), C.POINTER(RequestContext), C.POINTER(C.c_double)],
            "kvc_selector_create": [C.POINTER(Profile), I32, C.POINTER(SelectorConfig), C.POINTER(C.c_void_p)],
            "kvc_selector_destroy": [P],
            "kvc_selector_envelope": [P, I32, I32, C.POINTER(I32), C.POINTER(C.c_double), C.POINTER(I32)],
            "kvc_selector_model_choice": [P, I32, C.c_double, C.POINTER(I32)],
            "kvc_selector_choose": [P, C.POINTER(RequestContext), C.POINTER(I32), C.POINTER(C.c_double)],
            "kvc_selector_observe": [P, C.POINTER(RequestContext), I32, C.c_double],
            "kvc_selector_state": [P, C.POINTER(RequestContext), I32, C.POINTER(C.c_double), C.POINTER(I64),
                                   C.POINTER(I32)],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = C.c_int
        L.kvc_status_string.argtypes = [C.c_int]
        L.kvc_status_string.restype = C.c_char_p
        L.kvc_last_error.argtypes = []
        L.kvc_last_error.restype = C.c_char_p
        for name in ("kvc_harmonic_throughput", "kvc_break_even_bandwidth"):
            f = getattr(L, name)
            f.argtypes = [C.c_double] * (2 if name == "kvc_harmonic_throughput" else 3)
            f.restype = C.c_double
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().kvc_status_string(s).decode()


def last_error() -> str:
    return lib().kvc_last_error().decode()


def _check(s: int, where: str):
    if s != OK:
        raise KvcError(s, where)


def make_config(layers: int, max_tokens: int, kv_heads: int, head_dim: int, dtype: int,
                k: Sequence[int], v: Sequence[int], sign_seed: int, lossless: Sequence[str],
                chunk_bytes: int = 65536, page_tokens: int = 0) -> Config:
    """k, v: (bits, axis, group, hadamard[, delta run length])."""
    c = Config()
    c.struct_size = C.sizeof(Config)
    c.layers, c.max_tokens, c.kv_heads, c.head_dim, c.dtype = layers, max_tokens, kv_heads, head_dim, dtype
    for dst, pol in ((c.k, k), (c.v, v)):
        dst.bits, dst.axis, dst.group, dst.hadamard = pol[0], pol[1], pol[2], pol[3]
        dst.delta = pol[4] if len(pol) > 4 else 0
    c.sign_seed = sign_seed
    ids = [STAGES[s] for s in lossless] + [0] * (4 - len(lossless))
    for i in range(4):
        c.lossless[i] = ids[i]
    c.chunk_bytes = chunk_bytes
    c.page_tokens = page_tokens
    return c


def config_from_workload(wl, max_tokens: Optional[int] = None, layers: Optional[int] = None) -> Config:
    """Config for an object with the fields of kvc_workloads.Workload."""
    pol = lambda p: (p.bits, PER_TOKEN if p.axis == "token" else PER_CHANNEL, p.group, 1 if p.hadamard else 0,
                     getattr(p, "delta", 0))
    return make_config(wl.layers if layers is None else layers,
                       wl.tokens if max_tokens is None else max_tokens,
                       wl.heads, wl.head_dim, F16 if wl.dtype == "f16" else BF16,
                       pol(wl.k), pol(wl.v), wl.sign_seed, wl.stages, wl.chunk_bytes, wl.page_tokens)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    return int(getattr(stream, "cuda_stream", stream))


class Plan:
    """An immutable plan (kvc_plan / kvc_plan_destroy)."""

    def __init__(self, cfg: Config, bits=None):
        """bits: optional [2][layers][kv_heads] widths (0 / 2 / 4 / 8 / 16) for a
        mixed-precision plan (kvc_plan_mixed)."""
        self.cfg = cfg
        h = C.c_void_p()
        if bits is None:
            _check(lib().kvc_plan(C.byref(cfg), C.byref(h)), "kvc_plan")
        else:
            import numpy as np
            b = np.ascontiguousarray(bits, dtype=np.uint8)
            _check(lib().kvc_plan_mixed(C.byref(cfg), b.ctypes.data, C.byref(h)), "kvc_plan_mixed")
        self.handle = h

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.kvc_plan_destroy(self.handle)
            self.handle = None

    def sizes(self, tokens: int):
        ms, ws = C.c_size_t(0), C.c_size_t(0)
        _check(lib().kvc_plan_sizes(self.handle, tokens, C.byref(ms), C.byref(ws)), "kvc_plan_sizes")
        return ms.value, ws.value

    def sizes_paged(self, seq_lens):
        import numpy as np
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        ms, ws = C.c_size_t(0), C.c_size_t(0)
        _check(lib().kvc_plan_sizes_paged(self.handle, sl.ctypes.data, len(sl), C.byref(ms), C.byref(ws)),
               "kvc_plan_sizes_paged")
        return ms.value, ws.value

    def encode(self, k, v, tokens: int, out, ws, sync: bool = True, stream=None) -> Optional[int]:
        nb = C.c_size_t(0)
        s = lib().kvc_encode(self.handle, _ptr(k), _ptr(v), tokens, _ptr(out), out.numel() * out.element_size(),
                             _ptr(ws), ws.numel() * ws.element_size(), C.byref(nb) if sync else None,
                             _stream(stream))
        _check(s, "kvc_encode")
        return nb.value if sync else None

    def encode_noalloc(self, k, v, tokens: int, out, sync: bool = True, stream=None) -> Optional[int]:
        """kvc_encode_noalloc: kvc_encode with the library's fixed device scratch
        (NOALLOC_SCRATCH_BYTES) as the workspace."""
        nb = C.c_size_t(0)
        s = lib().kvc_encode_noalloc(self.handle, _ptr(k), _ptr(v), tokens, _ptr(out),
                                     out.numel() * out.element_size(), C.byref(nb) if sync else None,
                                     _stream(stream))
        _check(s, "kvc_encode_noalloc")
        return nb.value if sync else None

    def decode(self, stream_buf, in_bytes: int, tokens: int, k, v, ws, stream=None):
        s = lib().kvc_decode(self.handle, _ptr(stream_buf), in_bytes, tokens, _ptr(k), _ptr(v), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream(stream))
        _check(s, "kvc_decode")

    def encode_paged(self, k_pool, v_pool, num_blocks: int, block_table, seq_lens, out, req_offsets, ws,
                     sync: bool = True, stream=None) -> Optional[int]:
        import numpy as np
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        nb = C.c_size_t(0)
        s = lib().kvc_encode_paged(self.handle, _ptr(k_pool), _ptr(v_pool), num_blocks, _ptr(block_table),
                                   block_table.shape[1], sl.ctypes.data, len(sl), _ptr(out),
                                   out.numel() * out.element_size(), _ptr(req_offsets), _ptr(ws),
                                   ws.numel() * ws.element_size(), C.byref(nb) if sync else None, _stream(stream))
        _check(s, "kvc_encode_paged")
        return nb.value if sync else None

    def decode_paged(self, stream_buf, in_bytes: int, req_offsets, seq_lens, k_pool, v_pool, num_blocks: int,
                     block_table, ws, stream=None):
        import numpy as np
        sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
        s = lib().kvc_decode_paged(self.handle, _ptr(stream_buf), in_bytes, _ptr(req_offsets), sl.ctypes.data,
                                   len(sl), _ptr(k_pool), _ptr(v_pool), num_blocks, _ptr(block_table),
                                   block_table.shape[1], _ptr(ws), ws.numel() * ws.element_size(), _stream(stream))
        _check(s, "kvc_decode_paged")

    def query_status(self, ws, stream=None) -> int:
        return lib().kvc_query_status(self.handle, _ptr(ws), _stream(stream))


def profile_enable(on: bool = True):
    _check(lib().kvc_profile_enable(1 if on else 0), "kvc_profile_enable")


def profile_reset():
    _check(lib().kvc_profile_reset(), "kvc_profile_reset")


def profile_query(kind) -> tuple:
    """(total milliseconds, launches) of one kernel kind since the last reset."""
    k = KERNELS.index(kind) if isinstance(kind, str) else int(kind)
    ms, n = C.c_double(0), C.c_int64(0)
    _check(lib().kvc_profile_query(k, C.byref(ms), C.byref(n)), "kvc_profile_query")
    return ms.value, n.value


PROBE_NT_LOADS, PROBE_SHORT_WAVES = 1, 2


def probe_bandwidth(src, dst, items: int, reads: int, writes: int, sink, stream=None, flags: int = 0):
    """Enqueue the bandwidth reference kernel (kvc_probe_bandwidth)."""
    _check(lib().kvc_probe_bandwidth(_ptr(src), _ptr(dst), items, reads, writes, flags, _ptr(sink),
                                     _stream(stream)), "kvc_probe_bandwidth")


# ---------------------------------------------------------------- selection
def harmonic_throughput(s_enc: float, s_dec: float) -> float:
    return lib().kvc_harmonic_throughput(s_enc, s_dec)


def break_even_bandwidth(cr: float, s_enc: float, s_dec: float) -> float:
    return lib().kvc_break_even_bandwidth(cr, s_enc, s_dec)


def _ctx(bucket: int, bandwidth: float, volume: float, t_model: float, t_slo: float) -> RequestContext:
    return RequestContext(bucket=bucket, bandwidth=bandwidth, volume=volume, t_model=t_model, t_slo=t_slo)


def predicted_jct(profile: Optional[tuple], bucket: int, bandwidth: float, volume: float, t_model: float,
                  t_slo: float = 0.0) -> float:
    """Eq. 1 prediction; profile = (id, bucket, cr, s_enc, s_dec) or None for raw transfer."""
    out = C.c_double()
    p = C.byref(Profile(*profile)) if profile is not None else None
    _check(lib().kvc_predicted_jct(p, C.byref(_ctx(bucket, bandwidth, volume, t_model, t_slo)), C.byref(out)),
           "kvc_predicted_jct")
    return out.value


class Selector:
    """Service-aware profile selector over measured profiles (host only)."""

    def __init__(self, profiles: Sequence[tuple], fallback_id: int = PROFILE_RAW, alpha: float = 0.2,
                 epsilon: float = 0.1, cooldown_k: int = 2, cooldown_m: int = 8, cooldown_len: int = 16,
                 seed: int = 0):
        arr = (Profile * max(len(profiles), 1))(*[Profile(*p) for p in profiles])
        cfg = SelectorConfig(struct_size=C.sizeof(SelectorConfig), fallback_id=fallback_id, alpha=alpha,
                             epsilon=epsilon, cooldown_k=cooldown_k, cooldown_m=cooldown_m,
                             cooldown_len=cooldown_len, seed=seed)
        h = C.c_void_p()
        _check(lib().kvc_selector_create(arr, len(profiles), C.byref(cfg), C.byref(h)), "kvc_selector_create")
        self._h = h

    def close(self):
        if self._h:
            lib().kvc_selector_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def envelope(self, bucket: int):
        n = C.c_int32()
        s = lib().kvc_selector_envelope(self._h, bucket, 0, None, None, C.byref(n))
        if s not in (OK, ERR_BUFFER_TOO_SMALL):
            _check(s, "kvc_selector_envelope")
        ids = (C.c_int32 * n.value)()
        xs = (C.c_double * n.value)()
        _check(lib().kvc_selector_envelope(self._h, bucket, n.value, ids, xs, C.byref(n)), "kvc_selector_envelope")
        return list(ids), list(xs)

    def model_choice(self, bucket: int, bandwidth: float) -> int:
        out = C.c_int32()
        _check(lib().kvc_selector_model_choice(self._h, bucket, bandwidth, C.byref(out)), "kvc_selector_model_choice")
        return out.value

    def choose(self, bucket: int, bandwidth: float, volume: float, t_model: float, t_slo: float):
        out, pred = C.c_int32(), C.c_double()
        _check(lib().kvc_selector_choose(self._h, C.byref(_ctx(bucket, bandwidth, volume, t_model, t_slo)),
                                         C.byref(out), C.byref(pred)), "kvc_selector_choose")
        return out.value, pred.value

    def observe(self, bucket: int, bandwidth: float, volume: float, t_model: float, t_slo: float, pid: int,
                observed: float):
        _check(lib().kvc_selector_observe(self._h, C.byref(_ctx(bucket, bandwidth, volume, t_model, t_slo)),
                                          pid, observed), "kvc_selector_observe")

    def state(self, bucket: int, bandwidth: float, pid: int):
        r, n, cl = C.c_double(), C.c_int64(), C.c_int32()
        _check(lib().kvc_selector_state(self._h, C.byref(_ctx(bucket, bandwidth, 0.0, 0.0, 0.0)), pid,
                                        C.byref(r), C.byref(n), C.byref(cl)), "kvc_selector_state")
        return r.value, n.value, cl.value
