"""csa_attend_noalloc (the library's own scratch) against csa_attend (a caller workspace): the same
kernels on the same inputs, so outputs and lse must agree bit for bit.  Two calls in a row, the
second smaller, then a third on an fp8 cache: each call leaves the shared scratch holding its own
partials, which the next one must overwrite wherever it reads."""
import math

import numpy as np
import pytest
import torch

import csa_inputs as ci
from compressed_attention_long_amd import _lib as ops
from compressed_attention_long_amd.rope import rope_inv_freq

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(B, H, cap, topk, W, seed, fp8=False):
    d = ci.Draw(seed, "cpu")
    q = d.normal((B, 1, H, 512), std=2.0 / math.sqrt(512)).to(DEV)
    sink = d.normal((H,), dtype=torch.float32).to(DEV)
    nv = torch.tensor([cap - 37 * b for b in range(B)], dtype=torch.int32, device=DEV)
    p0 = torch.zeros(B, dtype=torch.int64, device=DEV)
    if fp8:
        codes, sc = d.fp8_codes((B, cap, 512), 64)
        kv = ops.Cache(codes.to(DEV), nv, p0, 8, 4, scales=sc.to(DEV), scale_block=64)
    else:
        kv = ops.Cache(d.normal((B, cap, 512)).to(DEV), nv, p0, 8, 4)
    qp = 4 * cap + 7
    win = ops.Cache(d.normal((B, W, 512)).to(DEV), torch.full((B,), W, dtype=torch.int32, device=DEV),
                    torch.full((B,), qp - W + 1, dtype=torch.int64, device=DEV), 1, 1)
    q_pos = torch.full((B, 1), qp, dtype=torch.int64, device=DEV)
    rng = np.random.default_rng(seed)
    idx = np.stack([np.sort(rng.choice(cap - 37 * b, topk, replace=False)) for b in range(B)]).astype(np.int32)
    return q, q_pos, kv, torch.from_numpy(idx.reshape(B, 1, topk)).to(DEV), win, sink


def _both(B, H, cap, topk, W, seed, fp8=False):
    q, q_pos, kv, idx, win, sink = _inputs(B, H, cap, topk, W, seed, fp8)
    fg = rope_inv_freq(160000.0, 64, DEV)
    scale = 1 / math.sqrt(512)
    need = ops.csa_attend_workspace_bytes(B, 1, H, topk, W)
    assert 0 < need <= ops.CSA_NOALLOC_SCRATCH_BYTES, need      # a split call that fits the scratch
    out_ref = torch.empty((B, 1, H, 512), dtype=torch.float32, device=DEV)
    lse_ref = torch.empty((B, 1, H), dtype=torch.float32, device=DEV)
    ops.csa_attend(q, q_pos, kv, idx, win, W, sink, fg, 64, scale, out_ref, lse_ref, ops.workspace(need, DEV))
    out = torch.full_like(out_ref, float("nan"))
    lse = torch.full_like(lse_ref, float("nan"))
    ops.csa_attend_noalloc(q, q_pos, kv, idx, win, W, sink, fg, 64, scale, out, lse)
    torch.cuda.synchronize()
    return out, lse, out_ref, lse_ref


def test_noalloc_equals_workspace_call_on_consecutive_calls():
    for what, args in [("first call, 8 rows", (8, 128, 4000, 1024, 128, 11)),
                       ("second call, 2 rows", (2, 128, 3000, 1024, 128, 12)),
                       ("third call, fp8 cache, 3 rows", (3, 64, 2500, 1024, 128, 13, True))]:
        print(f"[gpu case] no-alloc {what}", flush=True)
        out, lse, out_ref, lse_ref = _both(*args)
        assert torch.equal(out, out_ref), f"{what}: output differs from csa_attend's"
        assert torch.equal(lse, lse_ref), f"{what}: lse differs from csa_attend's"
        assert torch.isfinite(out).all()
