"""Seeded synthetic KV-cache workloads.

This module only draws random numbers and shapes; it holds none of the
compression arithmetic.  It is the single piece shared by the tests, the CPU
oracle harness, the HIP library's tests and bench.py, so that both sides see
the same input bytes.

Shapes follow the model families the FastKVComp page evaluates ("Beyond
Compression Ratio: High-Throughput KV Compression for Disaggregated LLM
Serving", Sec. 5, Llama-3.1-8B) plus the Llama-3.1-70B shape (80 layers, 8 KV
heads, head_dim 128: 320 KiB of bf16 KV per token, as on the KVStream page's
model table).  The pages measure real KV from LongBench prompts; those are
not available here, so seeded Gaussian values with per-channel key outliers
stand in for them (the value model is stated per workload below).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import math

import numpy as np
import torch

SEED_BASE = 20261202

STAGE_NAMES = ("TUPL2_1", "TUPL4_1", "TUPL8_1", "DIFF1", "DIFF2", "DIFF4", "DIFF8",
               "BIT_1", "BIT_2", "BIT_4", "BIT_8", "RZE_1", "RZE_2", "RZE_4", "RZE_8")


@dataclasses.dataclass(frozen=True)
class TensorPolicy:
    bits: int
    axis: str          # "token" (groups along head_dim) or "channel" (groups along tokens)
    group: int
    hadamard: bool = True
    delta: int = 0     # token-delta run length (0 = none)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    layers: int
    tokens: int
    heads: int
    head_dim: int
    dtype: str                 # "f16" or "bf16"
    k: TensorPolicy
    v: TensorPolicy
    stages: Tuple[str, ...]
    chunk_bytes: int = 65536
    seed: int = SEED_BASE
    sign_seed: int = 0x5EED_0F_4ADA_4A4D
    value_model: str = "outliers2pct"   # see _fill_k / _fill_v
    # paged workloads
    requests: int = 0
    min_len: int = 0
    max_len: int = 0
    page_tokens: int = 0

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def uncompressed_bytes(self, tokens: Optional[int] = None) -> int:
        t = self.tokens if tokens is None else tokens
        return 2 * self.layers * t * self.heads * self.head_dim * 2


LLAMA_TUPL_BIT_RZE = ("TUPL8_1", "BIT_8", "RZE_2")
BYTE_SHUFFLE_RZE = ("TUPL8_1", "RZE_2")

WORKLOADS = {
    # Single layer, 512 tokens x 8 heads x 128, fp16; K and V ~ N(0,1) with 4
    # fixed K channels per head scaled by 15.  int4, groups of 32 along head_dim.
    "c1_single_layer_512": Workload(
        name="c1_single_layer_512", layers=1, tokens=512, heads=8, head_dim=128, dtype="f16",
        k=TensorPolicy(4, "token", 32), v=TensorPolicy(4, "token", 32),
        stages=LLAMA_TUPL_BIT_RZE, seed=SEED_BASE + 0, value_model="fixed4x15"),
    # Llama-3.1-8B-shaped: 32 layers x 4096 tokens x 8 x 128, fp16; int4, groups of 128.
    "c2_llama8b_4k": Workload(
        name="c2_llama8b_4k", layers=32, tokens=4096, heads=8, head_dim=128, dtype="f16",
        k=TensorPolicy(4, "token", 128), v=TensorPolicy(4, "token", 128),
        stages=BYTE_SHUFFLE_RZE, seed=SEED_BASE + 1),
    # Llama-3.1-70B-shaped: 80 layers x 32768 tokens x 8 x 128, bf16 (10.7 GB);
    # K int4 per-channel groups of 64 tokens, V int2 per-token groups of 32.
    "c3_llama70b_32k": Workload(
        name="c3_llama70b_32k", layers=80, tokens=32768, heads=8, head_dim=128, dtype="bf16",
        k=TensorPolicy(4, "channel", 64), v=TensorPolicy(2, "token", 32),
        stages=LLAMA_TUPL_BIT_RZE, seed=SEED_BASE + 2),
    # Paged batch: 64 requests, lengths uniform in [1024, 16384], Llama-3.1-8B shape,
    # fp16, 16-token pages scattered in a pool; int4 per-token groups of 128.
    "c4_paged_llama8b": Workload(
        name="c4_paged_llama8b", layers=32, tokens=0, heads=8, head_dim=128, dtype="f16",
        k=TensorPolicy(4, "token", 128), v=TensorPolicy(4, "token", 128),
        stages=BYTE_SHUFFLE_RZE, seed=SEED_BASE + 3,
        requests=64, min_len=1024, max_len=16384, page_tokens=16),
    # Long context: 80 layers x 131072 tokens x 8 x 128, fp16; int2 K per-channel
    # groups of 64, V per-token groups of 32.
    "c5_llama70b_128k": Workload(
        name="c5_llama70b_128k", layers=80, tokens=131072, heads=8, head_dim=128, dtype="f16",
        k=TensorPolicy(2, "channel", 64), v=TensorPolicy(2, "token", 32),
        stages=LLAMA_TUPL_BIT_RZE, seed=SEED_BASE + 4),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def _outlier_channels(wl: Workload, layer: int, gen_seed: int):
    """Per (layer, head): which K channels are outliers and their factors."""
    rng = np.random.default_rng([gen_seed, 7, layer])
    D, H = wl.head_dim, wl.heads
    if wl.value_model == "fixed4x15":
        # the same 4 channels of each head for every token and layer
        rng0 = np.random.default_rng([gen_seed, 7])
        chans = np.stack([rng0.permutation(D)[:4] for _ in range(H)])
        facs = np.full(chans.shape, 15.0)
        return chans, facs
    n = max(1, int(round(0.02 * D)))
    chans = np.stack([rng.permutation(D)[:n] for _ in range(H)])
    facs = rng.uniform(10.0, 20.0, size=chans.shape)
    return chans, facs


def _layer_values(wl: Workload, layer: int, tokens: int, which: str, seed: int, device) -> torch.Tensor:
    """fp32 values of one layer of K or V: [tokens, heads, head_dim]."""
    H, D = wl.heads, wl.head_dim
    g = _gen(seed * 1000003 + layer * 2 + (0 if which == "k" else 1), device)
    x = torch.randn((tokens, H, D), generator=g, device=device, dtype=torch.float32)
    if which == "k":
        chans, facs = _outlier_channels(wl, layer, seed)
        scale = torch.ones((H, D), dtype=torch.float32)
        for h in range(H):
            for c, f in zip(chans[h], facs[h]):
                scale[h, int(c)] = float(f)
        x = x * scale.to(device)
    elif wl.value_model != "fixed4x15":
        x = x * 0.5
    return x


def dense_kv(wl: Workload, layers: Optional[int] = None, tokens: Optional[int] = None,
             seed: Optional[int] = None, device="cpu", layer_offset: int = 0):
    """K and V as [layers, tokens, heads, head_dim] tensors of the workload dtype.

    Layer l of the result is layer (layer_offset + l) of the workload, so a
    sample of a large workload has exactly the bytes of the full one.
    """
    L = wl.layers if layers is None else layers
    T = wl.tokens if tokens is None else tokens
    s = wl.seed if seed is None else seed
    k = torch.empty((L, T, wl.heads, wl.head_dim), dtype=wl.torch_dtype, device=device)
    v = torch.empty_like(k)
    for l in range(L):
        k[l] = _layer_values(wl, layer_offset + l, T, "k", s, device).to(wl.torch_dtype)
        v[l] = _layer_values(wl, layer_offset + l, T, "v", s, device).to(wl.torch_dtype)
    return k, v


def as_u16(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a CPU fp16/bf16 tensor as a numpy uint16 array."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@dataclasses.dataclass
class PagedBatch:
    seq_lens: np.ndarray        # int32 [R]
    block_table: np.ndarray     # int32 [R, max_blocks]
    num_blocks: int
    max_blocks: int


def paged_layout(wl: Workload, requests: Optional[int] = None, min_len: Optional[int] = None,
                 max_len: Optional[int] = None, seed: Optional[int] = None,
                 stream: int = 0) -> PagedBatch:
    """Request lengths and a random page map over a pool of exactly the pages needed.

    stream selects an independent page permutation (0 for the source pool,
    1 for the destination pool of a decode)."""
    R = wl.requests if requests is None else requests
    lo = wl.min_len if min_len is None else min_len
    hi = wl.max_len if max_len is None else max_len
    s = wl.seed if seed is None else seed
    P = wl.page_tokens
    rng = np.random.default_rng([s, 11])
    lens = rng.integers(lo, hi + 1, size=R).astype(np.int32)
    pages = (lens + P - 1) // P
    nb = int(pages.sum())
    maxb = int(pages.max()) if R else 0
    perm = np.random.default_rng([s, 13, stream]).permutation(nb).astype(np.int32)
    bt = np.full((R, max(maxb, 1)), -1, dtype=np.int32)
    pos = 0
    for r in range(R):
        bt[r, :pages[r]] = perm[pos:pos + pages[r]]
        pos += pages[r]
    return PagedBatch(seq_lens=lens, block_table=bt, num_blocks=nb, max_blocks=max(maxb, 1))


def paged_pools(wl: Workload, batch: PagedBatch, seed: Optional[int] = None, device="cpu"):
    """K and V pools [layers, num_blocks, page_tokens, heads, head_dim] filled so
    that request r's token t holds the values a dense [layers, T_r, H, D]
    workload with seed (seed + 1 + r) would have."""
    s = wl.seed if seed is None else seed
    L, P = wl.layers, wl.page_tokens
    shape = (L, batch.num_blocks, P, wl.heads, wl.head_dim)
    kp = torch.zeros(shape, dtype=wl.torch_dtype, device=device)
    vp = torch.zeros(shape, dtype=wl.torch_dtype, device=device)
    bt = torch.as_tensor(batch.block_table, device=device).long()
    for r, T in enumerate(batch.seq_lens.tolist()):
        npg = (T + P - 1) // P
        blocks = bt[r, :npg]
        for l in range(L):
            for which, pool in (("k", kp), ("v", vp)):
                x = _layer_values(wl, l, npg * P, which, s + 1 + r, device).to(wl.torch_dtype)
                x[T:] = 0
                pool[l, blocks] = x.view(npg, P, wl.heads, wl.head_dim)
    return kp, vp


def correlated_kv(wl: Workload, layers: int, tokens: int, seed: int, device="cpu", rho=0.95):
    """K/V whose values follow a first-order autoregression along tokens
    (x_t = rho x_{t-1} + sqrt(1 - rho^2) e_t per layer, head and channel,
    unit variance), with the workload's K outlier channels scaled as in
    dense_kv.  A stand-in for the token locality of real KV caches (adjacent
    tokens carry similar values), which gives the lossless stage something to
    find; the values are synthetic, not taken from any model."""
    H, D = wl.heads, wl.head_dim
    out = []
    for which in ("k", "v"):
        t = torch.empty((layers, tokens, H, D), dtype=wl.torch_dtype, device=device)
        for l in range(layers):
            g = _gen(seed * 1000003 + l * 2 + (0 if which == "k" else 1), device)
            x = torch.randn((tokens, H, D), generator=g, device=device, dtype=torch.float32)
            x *= math.sqrt(1.0 - rho * rho)
            x[0] /= math.sqrt(1.0 - rho * rho)
            # y_t = sum_{s <= t} rho^(t - s) x_s by doubling: after the step
            # with shift d each y_t holds the terms s > t - 2d
            d, f = 1, rho
            while d < tokens:
                x[d:] = x[d:] + f * x[:-d].clone()
                d, f = 2 * d, f * f
            if which == "k":
                chans, facs = _outlier_channels(wl, l, seed)
                scale = torch.ones((H, D), dtype=torch.float32)
                for h in range(H):
                    for c, fc in zip(chans[h], facs[h]):
                        scale[h, int(c)] = float(fc)
                x = x * scale.to(device)
            t[l] = x.to(wl.torch_dtype)
        out.append(t)
    return out[0], out[1]


def zero_rich_kv(wl: Workload, layers: int, tokens: int, seed: int, device="cpu", zero_frac=0.9):
    """K/V in which whole blocks of 64 tokens of a head are exactly zero
    (probability zero_frac per block), so that quantized codes are zero-rich
    under both per-token and per-channel grouping and the lossless stage
    compresses; used to exercise non-raw chunks."""
    g = _gen(seed, device)
    shape = (layers, tokens, wl.heads, wl.head_dim)
    nb = (tokens + 63) // 64
    out = []
    for _ in range(2):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        keep = (torch.rand((layers, nb, wl.heads), generator=g, device=device) > zero_frac)
        keep = keep.repeat_interleave(64, dim=1)[:, :tokens]
        out.append((x * keep.unsqueeze(-1)).to(wl.torch_dtype))
    return out[0], out[1]
