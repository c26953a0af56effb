"""Rotary frequency tables handed to the kernels (device fp64, one entry per rotated pair).

The compressed layers rotate the last 64 of 512 dims with base 160,000, and use YaRN with
factor 16 over a 65,536-token base to reach 1,048,576 positions (DeepSeek-V4-Pro vs Inkling,
Component-by-component table, partial-RoPE row; atlas Raw config fields compress_rope_theta,
max_position_embeddings).  The pages give no further YaRN parameters; the ramp and the
attention temperature follow the YaRN method as published (Peng et al., 2023: "NTK-by-parts"
interpolation with alpha = 1, beta = 32, and sqrt(1/t) = 0.1 ln(s) + 1).
"""
from __future__ import annotations

import math

import numpy as np
import torch


def rope_inv_freq(theta: float, rope_dim: int, device) -> torch.Tensor:
    """theta ** (-2i / rope_dim) for i < rope_dim / 2, fp64."""
    i = np.arange(rope_dim // 2, dtype=np.float64)
    return torch.from_numpy(np.power(theta, -2.0 * i / rope_dim)).to(device)


def yarn_inv_freq(theta: float, rope_dim: int, factor: float, base_len: int, device,
                  beta_fast: float = 32.0, beta_slow: float = 1.0) -> torch.Tensor:
    """YaRN ("NTK-by-parts") frequencies, fp64.

    Pair i with frequency f_i turns base_len * f_i / (2 pi) times over the base context.
    Pairs that turn more than beta_fast times keep f_i; pairs that turn fewer than
    beta_slow times are interpolated to f_i / factor; in between the two blend linearly in
    the number of turns.
    """
    i = np.arange(rope_dim // 2, dtype=np.float64)
    f = np.power(theta, -2.0 * i / rope_dim)
    turns = base_len * f / (2.0 * math.pi)
    keep = np.clip((turns - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    return torch.from_numpy(f * (keep + (1.0 - keep) / factor)).to(device)


def yarn_logit_scale(factor: float) -> float:
    """Multiplier of the attention logits under YaRN: 1/t = (0.1 ln(factor) + 1)^2 (1 for factor <= 1)."""
    if factor <= 1.0:
        return 1.0
    return (0.1 * math.log(factor) + 1.0) ** 2
