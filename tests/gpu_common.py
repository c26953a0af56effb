"""Shared helpers of the GPU parity tests (not collected by pytest).

Parity bars (stated for the GPU path against the fp64 oracle):
  attention output   max |o_gpu - o_ora| <= 1e-2 * RMS(o_ora), fp32 output,
                     evaluated on the GPU's own top-k set and stored cache bytes
  indexer scores     |s_gpu - s_ora| <= 1e-3 * max(|s_ora|, 1e-3 * max_row |s_ora|)
  top-k sets         identical, except entries whose oracle score lies within
                     1e-3 relative of the k-th oracle score; and bit-identical to
                     the oracle's selection run on the GPU's own scores
  compressor         bf16 within one bf16 spacing of the fp64 value plus the fp32
                     error bound of the pooled sum (see pool_error_bound); fp8
                     codes within one code step, scales within 1e-6 relative;
                     fp4 (MXFP4) scales equal in >= 99% of blocks (else a factor
                     of 2 with the block maximum at a power of two), values within
                     one E2M1 grid step, codes equal in >= 99% of elements
  log-sum-exp        within 1e-4 absolute
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import csa_oracle as O

ATT_TOL = 1e-2
SCORE_TOL = 1e-3
TOPK_TIE = 1e-3
LSE_TOL = 1e-4


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def stored_rows(data: torch.Tensor, scales, block: int, kv_dtype: str = "") -> np.ndarray:
    """fp64 values of stored cache rows (bf16, fp8 codes times scales, or with kv_dtype "fp4"
    packed E2M1 codes times the 32-channel scales)."""
    if kv_dtype == "fp4":
        return O.mxfp4_block_dequantize(O.fp4_unpack(data.cpu().numpy()), scales.cpu().numpy(), block)
    if data.dtype == torch.uint8:
        return O.fp8_block_dequantize(data.cpu().numpy(), scales.cpu().numpy(), block)
    return np64(data)


def _e2m1_step(mag: np.ndarray) -> np.ndarray:
    """Spacing of the E2M1 grid at code magnitude `mag` (0.5 below 2, 1 below 4, else 2)."""
    return np.where(mag < 2.0, 0.5, np.where(mag < 4.0, 1.0, 2.0))


def check_fp4_rows(packed: np.ndarray, scales: np.ndarray, ref: np.ndarray, what: str = ""):
    """GPU MXFP4 rows (packed codes [n, C/2], scales [n, C/32]) against the oracle's
    quantization of the fp64 rows `ref` [n, C]."""
    codes_o, sc_o = O.mxfp4_block_quantize(ref)
    codes_g = O.fp4_unpack(packed)
    same_scale = scales == sc_o
    assert same_scale.mean() >= 0.99, f"{what}: only {same_scale.mean():.4f} of the block scales agree"
    if not same_scale.all():
        # a differing scale may only come from a block maximum at a power of two
        r = scales[~same_scale] / sc_o[~same_scale]
        assert np.all((r == 2.0) | (r == 0.5)), f"{what}: scales differ by more than a factor 2"
        amax = np.abs(ref.reshape(ref.shape[0], -1, 32)).max(-1)[~same_scale]
        near = np.abs(amax / np.exp2(np.round(np.log2(amax))) - 1.0)
        assert np.all(near < 1e-5), f"{what}: scales differ away from a power-of-two maximum"
    vg = O.fp4_e2m1_decode(codes_g) * np.repeat(scales, 32, axis=-1)
    vo = O.fp4_e2m1_decode(codes_o) * np.repeat(sc_o, 32, axis=-1)
    step = np.maximum(_e2m1_step(np.abs(O.fp4_e2m1_decode(codes_g))) * np.repeat(scales, 32, axis=-1),
                      _e2m1_step(np.abs(O.fp4_e2m1_decode(codes_o))) * np.repeat(sc_o, 32, axis=-1))
    assert np.all(np.abs(vg - vo) <= step), f"{what}: fp4 values more than one grid step apart"
    assert np.mean((codes_g == codes_o) | ((codes_g & 7) == 0) & ((codes_o & 7) == 0)) > 0.99, \
        f"{what}: fewer than 99% of the fp4 codes agree"


def check_attention(o_gpu: np.ndarray, o_ora: np.ndarray, what: str = ""):
    err = float(np.abs(o_gpu - o_ora).max())
    rms = float(np.sqrt((o_ora ** 2).mean()))
    assert err <= ATT_TOL * rms, f"{what}: max abs err {err:.3e} > {ATT_TOL} x RMS {rms:.3e}"
    return err / rms


def check_scores(s_gpu: np.ndarray, s_ora: np.ndarray, vis: np.ndarray, what: str = ""):
    sg, so = s_gpu[vis], s_ora[vis]
    assert np.all(np.isneginf(s_gpu[~vis])), f"{what}: invisible entries must score -inf"
    if so.size == 0:
        return 0.0
    floor = 1e-3 * np.abs(so).max()
    bound = SCORE_TOL * np.maximum(np.abs(so), floor)
    rel = np.abs(sg - so) / np.maximum(np.maximum(np.abs(so), floor), 1e-30)
    assert np.all(np.abs(sg - so) <= bound), f"{what}: worst relative score error {rel.max():.3e}"
    return float(rel.max())


def check_topk(idx_gpu: np.ndarray, s_gpu: np.ndarray, s_ora: np.ndarray, vis: np.ndarray, k: int,
               what: str = ""):
    """idx_gpu: one row of int32 indices (ascending, -1 padded)."""
    nvis = int(vis.sum())
    sel = idx_gpu[idx_gpu >= 0]
    assert np.all(idx_gpu[len(sel):] == -1), f"{what}: padding must follow the indices"
    assert len(sel) == min(k, nvis), f"{what}: {len(sel)} selected, expected {min(k, nvis)}"
    assert np.all(np.diff(sel) > 0), f"{what}: indices must be strictly ascending"
    assert np.all(vis[sel]), f"{what}: selected an invisible entry"
    # exact: the oracle's selection applied to the GPU's own scores
    exact = O.topk_select(s_gpu.astype(np.float64), vis, k)
    assert np.array_equal(sel, exact), f"{what}: selection differs from the oracle's on the same scores"
    # against the oracle's scores: differences only at near-ties of the k-th score
    ora = O.topk_select(s_ora, vis, k)
    diff = np.setxor1d(sel, ora)
    if diff.size and nvis > k:
        kth = np.sort(s_ora[vis])[::-1][k - 1]
        assert np.all(np.abs(s_ora[diff] - kth) <= TOPK_TIE * abs(kth)), \
            f"{what}: {diff.size} set differences outside the tie band"
    return int(diff.size)


def oracle_rows_csa(kv_rows: np.ndarray, idx_row: np.ndarray, win_rows: np.ndarray, win_pos: np.ndarray,
                    q_pos: int, W: int, n_valid: int):
    sel = idx_row[(idx_row >= 0) & (idx_row < n_valid)]
    wm = O.window_rows(win_pos, q_pos, W)
    return np.concatenate([kv_rows[sel], win_rows[wm]], 0)


def oracle_rows_hca(kv_rows: np.ndarray, ent_pos: np.ndarray, win_rows: np.ndarray, win_pos: np.ndarray,
                    q_pos: int, W: int):
    vis = O.visible_mask(ent_pos, q_pos)
    wm = O.window_rows(win_pos, q_pos, W)
    return np.concatenate([kv_rows[vis], win_rows[wm]], 0)


U32 = 2.0 ** -24


def pool_error_bound(kv: np.ndarray, z: np.ndarray, window: int, stride: int, rope_dim: int) -> np.ndarray:
    """Bound on |fp32 pooled-and-rotated entry - exact value|, per element.

    The kernel forms the softmax weights and the weighted mean in fp32.  Each of
    the `window` weights carries a relative error of a few units u = 2^-24 (the
    log2(e) scaling, the exp2 and the running rescales), and the sums add about one
    u per term, so the pooled value e = sum a_t kv_t / sum a_t is off by at most
    (window + 24) u M with M = sum a_t |kv_t| / sum a_t (the same pooling applied
    to |kv|).  A cancelling sum has a small e but not a small M, which is why a
    bound relative to e alone (one bf16 spacing) is not enough.  The rotation mixes
    the two channels of a pair, so rotated channels take M of both.
    """
    M = O.pool(np.abs(kv), z, window, stride)
    if rope_dim:
        D = M.shape[-1]
        pair = M[:, D - rope_dim:].reshape(M.shape[0], -1, 2).sum(-1)
        M = M.copy()
        M[:, D - rope_dim:] = np.repeat(pair, 2, axis=-1)
    return (window + 24) * U32 * M


def check_bf16_rows(got: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str = ""):
    spacing = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - 8)
    err = np.abs(got - ref)
    bad = err > spacing + bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - spacing - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} elements beyond bound; worst at {i}: got {got[i]!r} "
                             f"ref {ref[i]!r} spacing {spacing[i]:.3e} fp32 bound {bound[i]:.3e}")
    same = float(np.mean(got == O.bf16_round(ref)))
    assert same > 0.99, f"{what}: only {same:.4f} of the elements round identically"
