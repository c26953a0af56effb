"""One attention-layer step of the CSA/HCA path on the GPU, through the C ABI.

A step is what a layer does for one batch of new tokens:
  1. compress the entries the new tokens complete (csa_compress, pooled rows);
  2. write the new raw tokens, rotated, into the sliding-window cache
     (csa_compress with window = stride = 1);
  3. CSA only: score every visible entry with the lightning indexer and keep
     the top-k (csa_index_topk);
  4. attend (csa_attend over top-k + window, or hca_attend over every visible
     entry + window).
All buffers are allocated once, in __init__; run() only enqueues kernels.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from . import _lib as ops
from .rope import rope_inv_freq, yarn_inv_freq, yarn_logit_scale


class LayerStep:
    """Holds the caches and buffers of one layer for a workload and runs its step."""

    def __init__(self, wl, tensors: dict, meta: dict, out_dtype=torch.bfloat16, theta: float = 160000.0,
                 softmax_scale: Optional[float] = None):
        self.wl = wl
        self.t = tensors
        self.meta = meta
        dev = tensors["q"].device
        self.device = dev
        B = wl.B
        if wl.yarn_factor > 1.0:
            # the model's table: YaRN over the base context, with its attention temperature
            self.inv_freq = yarn_inv_freq(theta, wl.R, wl.yarn_factor, wl.yarn_base_len, dev)
            default_scale = yarn_logit_scale(wl.yarn_factor) / math.sqrt(wl.D)
        else:
            self.inv_freq = rope_inv_freq(theta, wl.R, dev)
            default_scale = 1.0 / math.sqrt(wl.D)
        self.scale = default_scale if softmax_scale is None else softmax_scale
        kv = tensors["kv_cache"]
        self.kv = ops.Cache(kv, tensors["kv_n_valid"], tensors["kv_pos0"], wl.window, wl.stride,
                            scales=tensors.get("kv_cache_scale"),
                            scale_block=wl.kv_scale_block if wl.kv_dtype != "bf16" else 0,
                            fmt=ops.CSA_FP4_E2M1 if wl.kv_dtype == "fp4" else None)
        self.win = ops.Cache(tensors["win_cache"], tensors["win_n_valid"], tensors["win_pos0"], 1, 1)
        if wl.mode == "csa":
            ks = tensors.get("k_idx_scale")
            self.keys = ops.Cache(tensors["k_idx"], tensors["kv_n_valid"], tensors["kv_pos0"], wl.window,
                                  wl.stride, scales=ks, scale_block=wl.Di if ks is not None else 0)
            self.idx = torch.empty((B, wl.Tq, wl.topk), dtype=torch.int32, device=dev)
            self.scores = torch.empty((B, wl.Tq, wl.E), dtype=torch.float32, device=dev)
            self.idx_ws = ops.workspace(ops.index_topk_workspace_bytes(B, wl.Tq, wl.Hi, wl.E, wl.topk), dev)
            ws = ops.csa_attend_workspace_bytes(B, wl.Tq, wl.H, wl.topk, wl.W)
        else:
            self.keys = None
            ws = ops.hca_attend_workspace_bytes(B, wl.Tq, wl.H, wl.E, wl.W)
        self.att_ws = ops.workspace(ws, dev)
        self.out = torch.empty((B, wl.Tq, wl.H, wl.D), dtype=out_dtype, device=dev)
        self.lse = torch.empty((B, wl.Tq, wl.H), dtype=torch.float32, device=dev)
        # raw tokens of this step: all rows for the compressor, the new tokens for the window
        self.kv_raw = tensors["kv_raw"]
        self.z_raw = tensors["z_raw"]
        self.new_raw = self.kv_raw[:, self.kv_raw.shape[1] - meta["new_tok"]:]

    def compress_calls(self):
        """The completed entries and the raw-window write of this step."""
        m = self.meta
        calls = []
        if m["n_new_entries"] > 0:
            calls.append((self.kv_raw, self.z_raw, self.kv, m["E_pre"], m["n_new_entries"], self.inv_freq, self.wl.R))
        calls.append((self.new_raw, None, self.win, m["win_first_new"], m["new_tok"], self.inv_freq, self.wl.R))
        return calls

    def compress(self, stream=None):
        """The step's compress calls, in one batched call."""
        ops.compress_batch(self.compress_calls(), stream)

    def index_compress(self, stream=None):
        """The compress calls and the indexer / top-k in one combined call (fewer launches)."""
        wl = self.wl
        ops.index_topk_compress(self.compress_calls(), self.t["q_idx"], self.t["w"], self.t["q_pos"], self.keys,
                                wl.topk, self.idx, scores_out=self.scores, workspace=self.idx_ws, stream=stream)

    def index(self, stream=None):
        wl = self.wl
        ops.index_topk(self.t["q_idx"], self.t["w"], self.t["q_pos"], self.keys, wl.topk, self.idx,
                       scores_out=self.scores, workspace=self.idx_ws, stream=stream)

    def attend(self, stream=None):
        wl = self.wl
        if wl.mode == "csa":
            ops.csa_attend(self.t["q"], self.t["q_pos"], self.kv, self.idx, self.win, wl.W, self.t["sink"],
                           self.inv_freq, wl.R, self.scale, self.out, self.lse, self.att_ws, stream)
        else:
            ops.hca_attend(self.t["q"], self.t["q_pos"], self.kv, self.win, wl.W, self.t["sink"], self.inv_freq,
                           wl.R, self.scale, self.out, self.lse, self.att_ws, stream)

    def run(self, stream=None, combined: bool = True):
        """The whole step.  A CSA step issues its compress calls with the indexer through the
        combined call unless `combined` is False (then as two calls)."""
        if self.wl.mode == "csa" and combined:
            self.index_compress(stream)
        else:
            self.compress(stream)
            if self.wl.mode == "csa":
                self.index(stream)
        self.attend(stream)


class ReuseStep:
    """A layer that reuses a computed layer's KV cache, window and top-k selection and brings
    only its own queries and sink (the CSA2 "Reuse" layers: KV and the top-512 selection are
    computed in 3 of 18 layers and reused by the rest; DeepSeek-V4.1-Flash vs Inkling, CSA2
    encoder layers row).  Its step is one csa_attend call."""

    def __init__(self, full: LayerStep, q: torch.Tensor, sink: torch.Tensor, out_dtype=torch.bfloat16):
        wl = full.wl
        assert wl.mode == "csa", "reuse applies to selected-entry (CSA) layers"
        self.full, self.wl, self.q, self.sink = full, wl, q, sink
        dev = q.device
        self.att_ws = ops.workspace(ops.csa_attend_workspace_bytes(wl.B, wl.Tq, wl.H, wl.topk, wl.W), dev)
        self.out = torch.empty((wl.B, wl.Tq, wl.H, wl.D), dtype=out_dtype, device=dev)
        self.lse = torch.empty((wl.B, wl.Tq, wl.H), dtype=torch.float32, device=dev)

    def run(self, stream=None):
        f, wl = self.full, self.wl
        ops.csa_attend(self.q, f.t["q_pos"], f.kv, f.idx, f.win, wl.W, self.sink, f.inv_freq, wl.R, f.scale,
                       self.out, self.lse, self.att_ws, stream)
