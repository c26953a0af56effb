"""Seeded synthetic inputs for the compressed-attention path.

This module only draws random tensors and describes workload shapes.  It holds
none of the method's arithmetic (no pooling, rotation, scoring, selection or
attention) so that both the CPU oracle and the GPU path can be fed from it
without sharing any computation.

Workload shapes follow the DeepSeek-V4-Pro pages: 128 query heads of dim 512
on one shared KV head, a 64 x 128 lightning indexer keeping 1,024 entries, a
128-token sliding window, 8-token/stride-4 (CSA) and 128-token (HCA) pooling,
and RoPE base 160,000 on the last 64 dims (DeepSeek-V4-Pro page, "Raw config
fields" table; DeepSeek-V4-Pro vs Inkling, "Component by component" table,
attention rows).  The pages give no trained weights, so every tensor is drawn:
  kv, pooling logits z        ~ N(0, 1)
  q                           ~ N(0, 1/512)
  indexer q and keys          ~ N(0, 1/128)
  indexer head weights w      ~ U(0, 1)
  sink logits                 ~ N(0, 1)

Small inputs (the ones the oracle checks in full) are drawn on the host with
NumPy's PCG64 so they are identical on every machine.  Large caches for the
throughput workloads are drawn on the device with torch's generator; parity
checks at those sizes copy the device tensors back to the host for the oracle.

fp8 tensors are synthesized directly as OCP e4m3fn codes (the library cast of
a clamped Gaussian draw) plus positive per-block scales drawn around the value
that makes code x scale ~ N(0, sigma^2).  fp4 (MXFP4) caches are drawn the same
way: uniform E2M1 codes, two per byte, with power-of-two scales per 32 channels.
They are stand-ins for caches that an earlier step already stored; the path only
ever reads such bytes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

ROPE_THETA = 160000.0
FP8_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape of one decode/prefill step of one attention layer."""

    name: str
    mode: str                 # "csa" (pooled 8/4 + indexer + top-k) or "hca" (pooled 128/128, dense)
    B: int                    # sequences
    N: int                    # raw tokens per sequence, including the newest (query) token
    H: int                    # query heads
    topk: int = 1024
    Hi: int = 64              # indexer heads
    Di: int = 128             # indexer head dim
    D: int = 512              # shared KV / head dim
    R: int = 64               # rotated dims (the last R of D)
    W: int = 128              # sliding window (raw tokens)
    Tq: int = 1               # query tokens per sequence (decode 1, prefill chunk > 1)
    kv_dtype: str = "bf16"    # compressed KV cache storage: "bf16" | "fp8" | "fp4"
    kv_scale_block: int = 64  # channels per scale in the KV cache (fp8; fp4 caches use 32)
    idx_dtype: str = "bf16"   # indexer key storage: "bf16" | "fp8" (one scale per key)
    pos0: int = 1             # position of raw token 0
    compress_each_step: bool = True
    yarn_factor: float = 1.0  # rotary table: YaRN factor over yarn_base_len (1: plain table)
    yarn_base_len: int = 65536
    pool_window: int = 0      # compression geometry override (0: the mode's own)
    pool_stride: int = 0
    reuse: int = 0            # layers that reuse one computed layer's KV and selection (CSA2)

    @property
    def window(self) -> int:
        if self.pool_window:
            return self.pool_window
        return 8 if self.mode == "csa" else 128

    @property
    def stride(self) -> int:
        if self.pool_stride:
            return self.pool_stride
        return 4 if self.mode == "csa" else 128

    def n_entries(self, n_raw: Optional[int] = None) -> int:
        n = self.N if n_raw is None else n_raw
        if n < self.window:
            return 0
        return (n - self.window) // self.stride + 1

    @property
    def E(self) -> int:
        return self.n_entries()

    @property
    def q_pos(self) -> int:
        """Position of the newest token (the decode query)."""
        return self.pos0 + self.N - 1


# The five workloads: a tiny parity case and the four page-shaped throughput cases.  The
# page-shaped ones use the model's rotary table (YaRN factor 16 over 65,536 tokens: DeepSeek-V4-Pro
# vs Inkling, partial-RoPE row); the tiny case states plain partial RoPE with base 160,000.
WORKLOADS = {
    "tiny_csa_decode": Workload("tiny_csa_decode", "csa", B=1, N=4096, H=8, topk=256, Hi=8),
    "v4pro_csa_decode_65k": Workload("v4pro_csa_decode_65k", "csa", B=32, N=65536, H=128,
                                     idx_dtype="fp8", yarn_factor=16.0),
    "v4pro_hca_decode_1m": Workload("v4pro_hca_decode_1m", "hca", B=16, N=1048576, H=128, yarn_factor=16.0),
    "v4pro_csa_prefill_4k_on_131k": Workload("v4pro_csa_prefill_4k_on_131k", "csa", B=1,
                                             N=131072 + 4096, H=128, Tq=4096, yarn_factor=16.0),
    "v4flash_csa_decode_1m_fp8": Workload("v4flash_csa_decode_1m_fp8", "csa", B=4, N=1048576,
                                          H=64, kv_dtype="fp8", idx_dtype="fp8", yarn_factor=16.0),
    # multi-token decode: 4 query tokens per sequence (verifying draft tokens, as the MTP and
    # speculative-decoding components of the pages do) through the same step, causal within the 4
    "v4pro_csa_decode_65k_mtp4": Workload("v4pro_csa_decode_65k_mtp4", "csa", B=32, N=65536, H=128, Tq=4,
                                          idx_dtype="fp8", yarn_factor=16.0),
    # CSA2 (DeepSeek-V4.1-Flash vs Inkling, CSA2 encoder layers row): entries pool 2 raw tokens,
    # top-512; KV and selection computed in 3 of 18 layers and reused by the other 15 (5 per
    # computed layer).  The KV cache is FP4 (MXFP4, quantized after RoPE, the same page's
    # partial-RoPE row); indexer keys stay fp8.
    "v41flash_csa2_decode_1m_fp4": Workload("v41flash_csa2_decode_1m_fp4", "csa", B=4, N=1048576, H=64,
                                            topk=512, kv_dtype="fp4", kv_scale_block=32, idx_dtype="fp8",
                                            yarn_factor=16.0, pool_window=2, pool_stride=2, reuse=5),
}


class Draw:
    """Seeded draws; host draws come from NumPy PCG64, device draws from torch.

    Every tensor comes back as a torch tensor on `device`.  bf16 tensors are the
    round-to-nearest-even image of an fp32 draw; the bf16 tensor is the input.
    """

    def __init__(self, seed: int, device="cpu"):
        self.device = torch.device(device)
        self.seed = seed
        if self.device.type == "cpu":
            self.rng = np.random.Generator(np.random.PCG64(seed))
            self.gen = None
        else:
            self.rng = None
            self.gen = torch.Generator(device=self.device)
            self.gen.manual_seed(seed)

    def normal(self, shape, std=1.0, dtype=torch.bfloat16):
        if self.rng is not None:
            a = self.rng.standard_normal(size=shape, dtype=np.float32)
            t = torch.from_numpy(a)
            if std != 1.0:
                t = t * np.float32(std)
        else:
            t = torch.randn(shape, generator=self.gen, device=self.device, dtype=torch.float32)
            if std != 1.0:
                t = t * std
        return t.to(dtype)

    def uniform(self, shape, lo=0.0, hi=1.0):
        if self.rng is not None:
            a = self.rng.uniform(lo, hi, size=shape).astype(np.float32)
            return torch.from_numpy(a)
        t = torch.rand(shape, generator=self.gen, device=self.device, dtype=torch.float32)
        return t * (hi - lo) + lo

    def fp8_codes(self, shape, block, std=1.0):
        """Random fp8-e4m3fn codes and per-block scales whose product ~ N(0, std^2).

        Returns (codes uint8 [..., C], scales fp32 [..., C // block]).
        """
        c = shape[-1]
        assert c % block == 0
        g = self.normal(shape, std=FP8_MAX / 4.0, dtype=torch.float32)
        g = g.clamp_(-FP8_MAX, FP8_MAX)
        codes = g.to(torch.float8_e4m3fn).view(torch.uint8)
        sshape = tuple(shape[:-1]) + (c // block,)
        scales = self.uniform(sshape, 0.75, 1.25) * (4.0 * std / FP8_MAX)
        return codes, scales.to(torch.float32)

    def fp4_codes(self, shape, block=32):
        """Random MXFP4 rows: E2M1 codes uniform over all 16, packed two per byte (channel 2k in
        the low nibble of byte k), and power-of-two scales 2^e, e uniform in {-2, -1, 0}, per
        `block` channels, so code x scale has magnitude ~ 1.

        Returns (packed uint8 [..., C // 2], scales fp32 [..., C // block]).
        """
        c = shape[-1]
        assert c % block == 0 and c % 2 == 0
        codes = self.uniform(shape, 0.0, 16.0).floor_().clamp_(0, 15).to(torch.uint8)
        packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).contiguous()
        sshape = tuple(shape[:-1]) + (c // block,)
        e = self.uniform(sshape, -2.0, 1.0).floor_().clamp_(-2, 0)
        return packed, torch.exp2(e).to(torch.float32)

    def kv_rows(self, wl, shape):
        """Stored compressed-KV rows in the workload's format: (data, scales or None)."""
        if wl.kv_dtype == "fp8":
            return self.fp8_codes(shape, wl.kv_scale_block)
        if wl.kv_dtype == "fp4":
            return self.fp4_codes(shape, wl.kv_scale_block)
        return self.normal(shape), None


def seed_for(name: str) -> int:
    """Seed 1000 + index of the workload in WORKLOADS (insertion order)."""
    return 1000 + list(WORKLOADS).index(name) if name in WORKLOADS else 1999


def decode_inputs(wl: Workload, device="cpu", seed: Optional[int] = None, n_raw_tail=None):
    """All inputs of one decode step of `wl`, as torch tensors on `device`.

    Raw tokens: the last `n_raw_tail` raw tokens of each sequence (kv and pooling
    logits), or the whole stream when None.  The stored caches (compressed KV,
    indexer keys, rotated window) are drawn directly when the raw stream is
    partial; tests that run the full path from raw tokens pass n_raw_tail=None
    and build every cache through the path itself.
    Draw order: kv, z, q, q_idx, k_idx, w, sink, then the stored caches.
    """
    seed = seed_for(wl.name) if seed is None else seed
    d = Draw(seed, device)
    T = wl.N if n_raw_tail is None else n_raw_tail
    out = {}
    out["kv"] = d.normal((wl.B, T, wl.D))
    out["z"] = d.normal((wl.B, T, wl.D))
    out["q"] = d.normal((wl.B, wl.Tq, wl.H, wl.D), std=1.0 / math.sqrt(wl.D))
    if wl.mode == "csa":
        out["q_idx"] = d.normal((wl.B, wl.Tq, wl.Hi, wl.Di), std=1.0 / math.sqrt(wl.Di))
        E = wl.E
        if wl.idx_dtype == "fp8":
            codes, sc = d.fp8_codes((wl.B, E, wl.Di), wl.Di, std=1.0 / math.sqrt(wl.Di))
            out["k_idx"] = codes
            out["k_idx_scale"] = sc
        else:
            out["k_idx"] = d.normal((wl.B, E, wl.Di), std=1.0 / math.sqrt(wl.Di))
        out["w"] = d.uniform((wl.B, wl.Tq, wl.Hi))
    out["sink"] = d.normal((wl.H,), dtype=torch.float32)
    if n_raw_tail is not None:
        # Stored caches of the tokens before the tail: drawn, not computed.
        E = wl.E
        out["kv_cache"], sc = d.kv_rows(wl, (wl.B, E, wl.D))
        if sc is not None:
            out["kv_cache_scale"] = sc
        out["win_cache"] = d.normal((wl.B, wl.W, wl.D))
    return out


def step_tensors(wl: Workload, device="cpu", seed: Optional[int] = None):
    """Tensors of one timed step of `wl` (decode or prefill chunk), plain torch.

    The stored caches of everything before the step are drawn; the step's own
    raw tokens (the newest `window` tokens for decode, or the chunk plus the
    overlap for prefill) are drawn as raw kv / pooling logits, so the step runs
    the compressor, the raw-window write, the indexer, top-k and attention.
    Geometry (positions are pos0 + raw index; one cache row per entry):
      entries of the prefix:        E_pre = n_entries(N - Tq_new)
      entries after the step:       E     = n_entries(N)
      window cache rows:            the last W raw tokens before the step, then the step's tokens
    """
    seed = seed_for(wl.name) if seed is None else seed
    d = Draw(seed, device)
    B, D, Tq = wl.B, wl.D, wl.Tq
    new_tok = Tq                                   # raw tokens that arrive in this step
    E = wl.E
    E_pre = wl.n_entries(wl.N - new_tok)
    n_new_entries = E - E_pre
    # raw rows needed to compress the new entries (the first one overlaps the prefix)
    raw_first = E_pre * wl.stride                  # raw index of the first token of entry E_pre
    T_raw = wl.N - raw_first
    t = {}
    t["kv_raw"] = d.normal((B, T_raw, D))
    t["z_raw"] = d.normal((B, T_raw, D))
    t["q"] = d.normal((B, Tq, wl.H, D), std=1.0 / math.sqrt(D))
    if wl.mode == "csa":
        t["q_idx"] = d.normal((B, Tq, wl.Hi, wl.Di), std=1.0 / math.sqrt(wl.Di))
        if wl.idx_dtype == "fp8":
            t["k_idx"], t["k_idx_scale"] = d.fp8_codes((B, E, wl.Di), wl.Di, std=1.0 / math.sqrt(wl.Di))
        else:
            t["k_idx"] = d.normal((B, E, wl.Di), std=1.0 / math.sqrt(wl.Di))
        t["w"] = d.uniform((B, Tq, wl.Hi))
    t["sink"] = d.normal((wl.H,), dtype=torch.float32)
    t["kv_cache"], sc = d.kv_rows(wl, (B, E, D))
    if sc is not None:
        t["kv_cache_scale"] = sc
    win_cap = wl.W + new_tok
    t["win_cache"] = d.normal((B, win_cap, D))
    dev = t["q"].device
    t["kv_n_valid"] = torch.full((B,), E, dtype=torch.int32, device=dev)
    t["kv_pos0"] = torch.full((B,), wl.pos0, dtype=torch.int64, device=dev)
    # window cache row r holds raw position win_pos0 + r; the step writes rows W .. W+new_tok-1
    win_pos0 = wl.pos0 + wl.N - new_tok - wl.W
    t["win_n_valid"] = torch.full((B,), win_cap, dtype=torch.int32, device=dev)
    t["win_pos0"] = torch.full((B,), win_pos0, dtype=torch.int64, device=dev)
    q_pos = wl.pos0 + wl.N - new_tok + torch.arange(Tq, dtype=torch.int64, device=dev)
    t["q_pos"] = q_pos.unsqueeze(0).repeat(B, 1).contiguous()
    meta = dict(E=E, E_pre=E_pre, n_new_entries=n_new_entries, raw_first=raw_first, T_raw=T_raw,
                win_cap=win_cap, win_first_new=wl.W, new_tok=new_tok)
    return t, meta


def reuse_tensors(wl: Workload, device="cpu", seed: Optional[int] = None):
    """The new inputs of a layer that reuses another layer's KV and selection (CSA2 "Reuse"
    layers): its own queries q [B, Tq, H, D] ~ N(0, 1/D) and sink logits [H] ~ N(0, 1)."""
    seed = seed_for(wl.name) + 500009 if seed is None else seed
    d = Draw(seed, device)
    return {"q": d.normal((wl.B, wl.Tq, wl.H, wl.D), std=1.0 / math.sqrt(wl.D)),
            "sink": d.normal((wl.H,), dtype=torch.float32)}
