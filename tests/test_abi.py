"""CPU checks of the C ABI: the library loads, exports every entry point
declared in include/kvc.h, validates arguments on the host, and computes the
same stream sizes as the oracle's independent layout code.  No GPU calls."""
import ctypes as C
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import kv_cache_compression_kvc_amd as K  # noqa: E402
import kvc_workloads as W  # noqa: E402
import oracle_api as O  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(K.LIB_PATH):
        subprocess.check_call([sys.executable, os.path.join(ROOT, "kv_cache_compression_kvc_amd", "build.py")])
    return K.lib()


def declared_functions():
    """Every function declared in include/*.h."""
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
            names.update(re.findall(r"\b(kvc_[a-z_]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kvc_plan", "kvc_plan_sizes", "kvc_encode", "kvc_decode", "kvc_encode_paged",
              "kvc_decode_paged", "kvc_plan_destroy", "kvc_status_string", "kvc_query_status",
              "kvc_last_error", "kvc_selector_create", "kvc_selector_choose", "kvc_selector_observe",
              "kvc_break_even_bandwidth"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.check_output(["nm", "-D", "--defined-only", K.LIB_PATH]).decode()
    exported = set(re.findall(r"\sT\s+(\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import importlib
    mod = importlib.import_module("kv_cache_compression_kvc_amd")
    monkeypatch.setattr(mod, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(mod, "_lib", None)
    with pytest.raises(ImportError):
        mod.lib()


def test_status_strings(lib):
    for s in range(9):
        assert K.status_string(s)


def good_cfg(**kw):
    wl = W.WORKLOADS["c3_llama70b_32k"]
    c = K.config_from_workload(wl, max_tokens=1024, layers=2)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_plan_accepts_the_workloads(lib):
    for name, wl in W.WORKLOADS.items():
        K.Plan(K.config_from_workload(wl, max_tokens=max(wl.tokens, 16)))


@pytest.mark.parametrize("field,value,status", [
    ("struct_size", 8, K.ERR_INVALID_ARG),
    ("layers", 0, K.ERR_INVALID_ARG),
    ("kv_heads", 0, K.ERR_INVALID_ARG),
    ("head_dim", 96, K.ERR_INVALID_ARG),
    ("head_dim", 64, K.ERR_UNSUPPORTED),
    ("dtype", 7, K.ERR_INVALID_ARG),
    ("chunk_bytes", 5000, K.ERR_INVALID_ARG),
    ("chunk_bytes", 1 << 17, K.ERR_INVALID_ARG),
    ("max_tokens", -1, K.ERR_INVALID_ARG),
])
def test_plan_rejects_bad_configs(lib, field, value, status):
    c = good_cfg(**{field: value})
    h = C.c_void_p()
    assert lib.kvc_plan(C.byref(c), C.byref(h)) == status
    assert K.last_error()


def test_plan_rejects_bad_policies(lib):
    for attr, val, st in (("bits", 3, K.ERR_INVALID_ARG), ("group", 48, K.ERR_INVALID_ARG),
                          ("axis", 2, K.ERR_INVALID_ARG), ("hadamard", 0, K.ERR_UNSUPPORTED)):
        c = good_cfg()
        setattr(c.k, attr, val)
        h = C.c_void_p()
        assert lib.kvc_plan(C.byref(c), C.byref(h)) == st, attr
    c = good_cfg()
    c.k.group = 128          # per-channel groups of 128 are valid but not on the GPU
    assert lib.kvc_plan(C.byref(c), C.byref(C.c_void_p())) == K.ERR_UNSUPPORTED
    c = good_cfg()
    c.lossless[0], c.lossless[1] = K.STAGES["RZE_2"], K.STAGES["BIT_8"]
    assert lib.kvc_plan(C.byref(c), C.byref(C.c_void_p())) == K.ERR_UNSUPPORTED
    c = good_cfg()
    c.lossless[0] = 99
    assert lib.kvc_plan(C.byref(c), C.byref(C.c_void_p())) == K.ERR_INVALID_ARG


@pytest.mark.parametrize("name", list(W.WORKLOADS))
@pytest.mark.parametrize("tokens", [0, 1, 37, 150, 4096])
def test_max_stream_bytes_matches_oracle_layout(lib, name, tokens):
    wl = W.WORKLOADS[name].with_(chunk_bytes=16384)
    p = K.Plan(K.config_from_workload(wl, max_tokens=4096, layers=3))
    ms, ws = p.sizes(tokens)
    assert ms == O.max_stream_bytes(O.cfg_from_workload(wl, layers=3), tokens)
    assert ws > 0 and ws % 256 == 0


def test_paged_sizes_are_sums_of_request_sizes(lib):
    wl = W.WORKLOADS["c4_paged_llama8b"].with_(layers=2)
    p = K.Plan(K.config_from_workload(wl, max_tokens=0))
    lens = [5, 16, 33, 1000]
    ms, ws = p.sizes_paged(lens)
    cfg = O.cfg_from_workload(wl)
    assert ms == sum(O.max_stream_bytes(cfg, t) for t in lens)


def test_host_argument_checks_need_no_gpu(lib):
    p = K.Plan(good_cfg())
    ms, wsb = p.sizes(64)
    # NULL output, unaligned workspace, too-small buffers and bad token counts
    # are rejected before anything touches a device
    assert lib.kvc_encode(p.handle, 16, 16, 64, None, ms, 256, wsb, None, None) == K.ERR_INVALID_ARG
    assert lib.kvc_encode(p.handle, 16, 16, 64, 16, ms, 257, wsb, None, None) == K.ERR_INVALID_ARG
    assert lib.kvc_encode(p.handle, 16, 16, 64, 16, ms - 1, 256, wsb, None, None) == K.ERR_BUFFER_TOO_SMALL
    assert lib.kvc_encode(p.handle, 16, 16, 64, 16, ms, 256, wsb - 256, None, None) == K.ERR_BUFFER_TOO_SMALL
    assert lib.kvc_encode(p.handle, 16, 16, 2048, 16, ms, 256, wsb, None, None) == K.ERR_INVALID_ARG
    assert lib.kvc_decode(p.handle, 16, 10, 64, 16, 16, 256, wsb, None) == K.ERR_CORRUPT_STREAM
    assert lib.kvc_encode_paged(p.handle, 16, 16, 4, 16, 1, None, 0, 16, 1, 16, 256, 1, None, None) \
        == K.ERR_INVALID_ARG   # plan built without page_tokens
    # the bandwidth probe: unknown flag bits, unsupported read:write pairs and
    # missing buffers are host errors
    assert lib.kvc_probe_bandwidth(16, 16, 1024, 1, 1, 4, 16, None) == K.ERR_INVALID_ARG
    assert lib.kvc_probe_bandwidth(16, 16, 1024, 3, 1, 0, 16, None) == K.ERR_UNSUPPORTED
    assert lib.kvc_probe_bandwidth(None, 16, 1024, 1, 1, K.PROBE_NT_LOADS, 16, None) == K.ERR_INVALID_ARG
    assert lib.kvc_probe_bandwidth(16, 16, -1, 1, 0, K.PROBE_SHORT_WAVES, 16, None) == K.ERR_INVALID_ARG
