"""GPU parity of the grouped low-rank output projection (csa_out_proj) against the fp64 oracle.

Bar, derived from the kernel's arithmetic (the pages fix no tolerance for this step): bf16
factors and bf16 inputs multiply exactly in fp32; an fp32 input (an fp32 attention output, and
the fp32 codes z between the two products) enters as bf16 hi + lo parts, which leave at most
2^-17 of it out; sums are fp32 over K terms.  Hence, per code and per output,
    |z_gpu - z| <= (Kg u + 2^-17) sum_k |o_k| |wa_rk|                       (u = 2^-24)
    |y_gpu - y| <= sum_r |wb_jr| |z_gpu - z|_r + (G R u + 2^-17) sum_r |wb_jr| |z_r|
with a factor 2 of margin, plus half a bf16 spacing of y for bf16 output."""
import math

import numpy as np
import pytest
import torch

import csa_inputs as ci
from compressed_attention_long_amd import _lib as ops
from oracle import csa_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda"
U32 = 2.0 ** -24


def _draw(T, H, D, G, R, hidden, seed, o_dtype):
    d = ci.Draw(seed, "cpu")
    Kg = (H // G) * D
    o = d.normal((T, H, D), dtype=o_dtype)
    wa = d.normal((G, R, Kg), std=1.0 / math.sqrt(Kg))
    wb = d.normal((hidden, G * R), std=1.0 / math.sqrt(G * R))
    return o, wa, wb


def _bound(o, wa, wb, y_bf16):
    """Per-output bar of the module docstring (fp64 arrays of the inputs)."""
    T, H, D = o.shape
    G, R, Kg = wa.shape
    ao = np.abs(o).reshape(T, G, Kg)
    s1 = np.einsum("tgk,grk->tgr", ao, np.abs(wa)).reshape(T, G * R)       # sum |o| |wa| per code
    _, z = O.out_projection(o, wa, wb)
    dz = (Kg * U32 + 2.0 ** -17) * s1
    awb = np.abs(wb)
    tol = 2.0 * (dz @ awb.T + (G * R * U32 + 2.0 ** -17) * (np.abs(z.reshape(T, G * R)) @ awb.T))
    return tol


def _run(o, wa, wb, y_dtype):
    T = o.shape[0]
    G, R, _ = wa.shape
    hidden = wb.shape[0]
    y = torch.empty((T, hidden), dtype=y_dtype, device=DEV)
    ws = ops.workspace(ops.csa_out_proj_workspace_bytes(T, G, R, hidden), DEV)
    ops.csa_out_proj(o, wa, wb, y, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("T,H,D,G,R,hidden,o_dtype,y_dtype", [
    (1, 8, 64, 2, 64, 96, torch.bfloat16, torch.float32),      # one token
    (5, 8, 64, 2, 64, 96, torch.float32, torch.float32),       # fp32 attention output (hi + lo)
    (33, 8, 64, 4, 128, 64, torch.bfloat16, torch.float32),    # ragged over 32-row tiles, 4 groups
    (70, 16, 64, 2, 64, 160, torch.bfloat16, torch.bfloat16),  # three row tiles, bf16 output
    (3, 16, 128, 16, 64, 32, torch.float32, torch.bfloat16),   # one head per group
    (37, 8, 64, 2, 64, 256, torch.bfloat16, torch.bfloat16),  # hidden % 128 == 0: second product over 4 K ranges
    (2, 8, 64, 4, 64, 384, torch.float32, torch.float32),      # the same, fp32 in and out
])
def test_out_proj_parity(T, H, D, G, R, hidden, o_dtype, y_dtype):
    print(f"case T={T} H={H} D={D} G={G} R={R} hidden={hidden} o={o_dtype} y={y_dtype}", flush=True)
    o, wa, wb = _draw(T, H, D, G, R, hidden, 7 + T, o_dtype)
    y = _run(o.to(DEV), wa.to(DEV), wb.to(DEV), y_dtype)
    o64, wa64, wb64 = (x.double().numpy() for x in (o, wa, wb))
    y_ora, _ = O.out_projection(o64, wa64, wb64)
    tol = _bound(o64, wa64, wb64, y_dtype == torch.bfloat16)
    yg = y.double().cpu().numpy()
    if y_dtype == torch.bfloat16:
        tol = tol + 2.0 ** -9 * np.abs(y_ora) * (1 + 2.0 ** -7) + 1e-30
    err = np.abs(yg - y_ora)
    assert np.all(err <= tol), f"max err {err.max():.3e}, worst ratio {(err / tol).max():.3f}"
    # deterministic: a second call writes the same bytes
    y2 = _run(o.to(DEV), wa.to(DEV), wb.to(DEV), y_dtype)
    assert torch.equal(y, y2)


def test_out_proj_v4pro_decode_shape_sampled_rows():
    """The page config at the 65K decode batch (32 tokens x 128 heads x 512 -> 16 x 1,024 -> 7,168),
    in the bf16 attention output the decode step writes; rows 0, 17 and 31 against the oracle."""
    T, H, D, G, R, hidden = 32, 128, O.HEAD_DIM, O.O_GROUPS, O.O_LORA_RANK, O.HIDDEN
    print("case v4pro decode shape", flush=True)
    o, wa, wb = _draw(T, H, D, G, R, hidden, 2024, torch.bfloat16)
    y = _run(o.to(DEV), wa.to(DEV), wb.to(DEV), torch.float32)
    rows = [0, 17, 31]
    o64 = o[rows].double().numpy()
    wa64, wb64 = wa.double().numpy(), wb.double().numpy()
    y_ora, _ = O.out_projection(o64, wa64, wb64)
    tol = _bound(o64, wa64, wb64, False)
    err = np.abs(y.double().cpu().numpy()[rows] - y_ora)
    assert np.all(err <= tol), f"max err {err.max():.3e}, worst ratio {(err / tol).max():.3f}"
    # the rows are about unit scale, the errors far below the bar's fp32 terms
    assert err.max() < 1e-3 * np.abs(y_ora).max()
