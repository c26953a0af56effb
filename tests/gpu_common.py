"""Shared helpers of the GPU parity tests (not collected by pytest).

Parity bars (stated for the GPU path against the fp64 oracle):
  attention output   max |o_gpu - o_ora| <= 1e-2 * RMS(o_ora), fp32 output,
                     evaluated on the GPU's own top-k set and stored cache bytes
  indexer scores     |s_gpu - s_ora| <= max(1e-3 |s_ora|, fp32 bound), the fp32 bound
                     being (128 + 64 + 4) 2^-24 * sum_h w_h sum_d |q_hd k_jd| (exact
                     bf16 products, fp32 sums over the key's 128 channels and the 64
                     heads, the key scale): it only matters for scores that cancel;
                     the fraction of scores within a strict 1e-3 is reported
  top-k sets         identical, except entries whose oracle score lies within
                     1e-3 relative of the k-th oracle score; and bit-identical to
                     the oracle's selection run on the GPU's own scores
  compressor         bf16 within one bf16 spacing of the fp64 value plus the fp32
                     error bound of the pooled sum (see pool_error_bound); fp8 and
                     fp4 (MXFP4) rows: scales equal to the oracle's up to that bound
                     (fp4: the power of two may differ only where the block maximum
                     lies within the bound of a power of two), and every code equal to
                     the rounding of the oracle's value under the row's own scale,
                     except where that value lies within the bound of a midpoint of
                     the format's grid (then either neighbour is a correct rounding)
  log-sum-exp        |lse_gpu - lse_ora| <= 1e-5 + 512 * 2^-24 * scale *
                     max_u sum_c |q'_c x_uc|: the logits are fp32 sums of 512
                     products (exact bf16 products; the rotated query's dims carried
                     to about 16 bits), so a logit is off by at most the textbook fp32
                     summation bound, and the log-sum-exp by at most the largest
                     logit error; 1e-5 covers exp2, the fp32 sums and the log
"""
from __future__ import annotations

import numpy as np
import torch

from oracle import csa_oracle as O

ATT_TOL = 1e-2
SCORE_TOL = 1e-3
TOPK_TIE = 1e-3
LSE_TOL = 1e-5            # absolute part of the lse bar (see lse_tolerance)
U32 = 2.0 ** -24


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


def _grid(kind: str) -> np.ndarray:
    """Positive magnitudes of a storage format, ascending: E2M1 (fp4) or E4M3FN (fp8, no NaN)."""
    if kind == "fp4":
        return O.fp4_e2m1_decode(np.arange(8))
    v = O.fp8_e4m3_decode(np.arange(0x7F))
    return np.sort(v)


def check_codes_against_grid(mag_g: np.ndarray, sign_g: np.ndarray, y: np.ndarray, tol: np.ndarray, kind: str,
                             what: str = ""):
    """Quantized magnitudes `mag_g` (with signs `sign_g`, +1 / -1) against exact scaled values `y`.

    Each magnitude must be the round-to-nearest-even of |y| on the format's grid (saturating),
    except where |y| lies within `tol` of a midpoint between two grid neighbours: there the
    kernel's fp32 value may fall on either side, and either neighbour is a correct rounding.
    A nonzero magnitude must carry the sign of y."""
    grid = _grid(kind)
    ay = np.abs(y)
    hi_i = np.clip(np.searchsorted(grid, ay, side="left"), 1, len(grid) - 1)
    lo, hi = grid[hi_i - 1], grid[hi_i]
    sat = ay >= grid[-1]
    mid = 0.5 * (lo + hi)
    exp = np.where(sat, grid[-1], np.where(ay < mid, lo, np.where(ay > mid, hi, np.nan)))
    # exact ties: round half to even (the even neighbour has the even code index)
    tie = np.isnan(exp)
    if tie.any():
        lo_even = (hi_i - 1) % 2 == 0
        exp = np.where(tie, np.where(lo_even, lo, hi), exp)
    ok = mag_g == exp
    near = (~sat) & (np.abs(ay - mid) <= tol) & ((mag_g == lo) | (mag_g == hi))
    near |= sat & (mag_g == grid[-1])
    bad = ~(ok | near)
    if bad.any():
        i = np.unravel_index(np.argmax(bad), bad.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} {kind} codes are not a rounding of the value; first at "
                             f"{i}: code magnitude {mag_g[i]!r}, scaled value {y[i]!r}, tolerance {tol[i]:.3e}")
    signed = mag_g > 0
    assert np.all(sign_g[signed] == np.sign(y[signed])), f"{what}: {kind} code with the wrong sign"
    return float(np.mean(ok))


def check_fp4_rows(packed: np.ndarray, scales: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str = ""):
    """GPU MXFP4 rows (packed codes [n, C/2], scales [n, C/32]) against the fp64 rows `ref` [n, C],
    whose fp32 computation the kernel carries out within `bound` [n, C] (pool_error_bound).

    Scales: the oracle's 2^(floor(log2 amax) - 2), except for blocks whose maximum lies within
    the bound of a power of two, where the neighbouring power is the other correct choice.
    Codes: the rounding of ref / scale (the row's own scale) on the E2M1 grid, up to the
    midpoint rule of check_codes_against_grid."""
    n, C = ref.shape
    codes_o, sc_o = O.mxfp4_block_quantize(ref)
    codes_g = O.fp4_unpack(packed)
    amax = np.abs(ref.reshape(n, -1, 32)).max(-1)
    bmax = bound.reshape(n, -1, 32).max(-1)
    diff = scales != sc_o
    if diff.any():
        r = scales[diff] / sc_o[diff]
        assert np.all((r == 2.0) | (r == 0.5)), f"{what}: scales differ by more than a factor 2"
        p2 = np.exp2(np.round(np.log2(amax[diff])))
        assert np.all(np.abs(amax[diff] - p2) <= bmax[diff] * (1 + 1e-6) + 1e-300), \
            f"{what}: scales differ where the block maximum is not within the fp32 bound of a power of two"
    s_full = np.repeat(scales.astype(np.float64), 32, axis=-1)
    y = ref / s_full
    mag = np.abs(O.fp4_e2m1_decode(codes_g))
    sign = np.where(codes_g & 8, -1.0, 1.0)
    return check_codes_against_grid(mag, sign, y, bound / s_full * (1 + 1e-6), "fp4", what)


def check_fp8_rows(codes_g: np.ndarray, scales: np.ndarray, ref: np.ndarray, bound: np.ndarray, block: int,
                   what: str = ""):
    """GPU fp8 rows (E4M3FN codes [n, C], fp32 scales [n, C/block]) against the fp64 rows `ref`,
    computed in fp32 by the kernel within `bound` [n, C].  Scales: fp32 amax / 448 of the oracle
    within the bound of the block maximum (divided by 448, plus fp32 rounding); codes: the
    rounding of ref / scale with the row's own scale, up to the midpoint rule."""
    n, C = ref.shape
    _, sc_o = O.fp8_block_quantize(ref, block)
    bmax = bound.reshape(n, -1, block).max(-1)
    tol_s = bmax / 448.0 + 2.0 * U32 * sc_o
    assert np.all(np.abs(scales.astype(np.float64) - sc_o) <= tol_s), f"{what}: fp8 scales off by more than the bound"
    s_full = np.repeat(scales.astype(np.float64), block, axis=-1)
    safe = np.where(s_full > 0, s_full, 1.0)
    y = np.where(s_full > 0, ref / safe, 0.0)
    mag = np.abs(O.fp8_e4m3_decode(codes_g))
    sign = np.where(codes_g & 0x80, -1.0, 1.0)
    # the kernel multiplies its fp32 value by the fp32 reciprocal of its scale: two more relative
    # roundings (of the reciprocal and of the product)
    tol = bound / safe * (1 + 1e-6) + 3.0 * U32 * np.abs(y)
    return check_codes_against_grid(mag, sign, y, tol, "fp8", what)


def check_attention(o_gpu: np.ndarray, o_ora: np.ndarray, what: str = ""):
    err = float(np.abs(o_gpu - o_ora).max())
    rms = float(np.sqrt((o_ora ** 2).mean()))
    assert err <= ATT_TOL * rms, f"{what}: max abs err {err:.3e} > {ATT_TOL} x RMS {rms:.3e}"
    return err / rms


def score_error_bound(q_idx: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """fp32 error bound of each entry's score: the bf16 products are exact, each head's dot
    product is an fp32 sum of Di terms, the weighted head sum one of Hi terms, then one
    multiplication by the key scale: (Di + Hi + 4) u * sum_h w_h sum_d |q_hd k_jd|."""
    q, k = np.abs(np.asarray(q_idx, np.float64)), np.abs(np.asarray(keys, np.float64))
    Hi, Di = q.shape
    return (Di + Hi + 4) * U32 * O.index_scores(q, np.abs(w), k)


def check_scores(s_gpu: np.ndarray, s_ora: np.ndarray, vis: np.ndarray, what: str = "", fp32_bound=None):
    """Visible scores within max(1e-3 |s_ora|, fp32_bound) (see score_error_bound); invisible
    entries -inf.  Returns (worst error relative to the allowed one, fraction of visible scores
    within a strict 1e-3 relative)."""
    sg, so = s_gpu[vis], s_ora[vis]
    assert np.all(np.isneginf(s_gpu[~vis])), f"{what}: invisible entries must score -inf"
    if so.size == 0:
        return 0.0, 1.0
    fb = np.zeros_like(so) if fp32_bound is None else np.asarray(fp32_bound)[vis]
    allowed = np.maximum(SCORE_TOL * np.abs(so), fb)
    err = np.abs(sg - so)
    worst = float(np.max(err / np.maximum(allowed, 1e-300)))
    assert np.all(err <= allowed), f"{what}: a score is off by {worst:.3f} x its allowed error"
    strict = float(np.mean(err <= SCORE_TOL * np.abs(so)))
    return worst, strict


def lse_tolerance(q: np.ndarray, q_pos: int, X: np.ndarray, scale: float, inv_freq: np.ndarray) -> np.ndarray:
    """Per-head lse bar: LSE_TOL + 512 u * scale * max_u sum_c |q'_c x_uc| (see the module docstring).

    With more than 64 rotated dims the rotated query channels below 448 are rounded to
    bf16 (unit roundoff 2^-8) before the product: those channels add 2^-8 |q'_c x_uc|."""
    qr = O.rope(q, q_pos, inv_freq)
    if X.shape[0] == 0:
        return np.full(q.shape[0], LSE_TOL)
    D = q.shape[-1]
    w = np.full(D, D * U32)
    w[D - 2 * len(inv_freq):D - 64] += 2.0 ** -8
    return LSE_TOL + abs(scale) * ((np.abs(qr) * w) @ np.abs(X).T).max(axis=1)


def check_lse(lse_gpu: np.ndarray, lse_ora: np.ndarray, tol: np.ndarray, what: str = ""):
    err = np.abs(np.asarray(lse_gpu, np.float64) - lse_ora)
    assert np.all(err <= tol), f"{what}: lse off by {err.max():.3e} (allowed {tol[np.argmax(err - tol)]:.3e})"
    return float(err.max())


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
