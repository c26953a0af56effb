"""Plain fp64 CPU oracle for Compressed Sparse Attention (CSA) and Heavily
Compressed Attention (HCA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or runs
this file: only the tests, the smoke check of the graft entry point and the
benchmark's CPU-baseline leg may use it.  It shares no code, table or helper
with the HIP kernels.

Every function follows a passage of the pages and writes out the plain
definition in fp64 (NumPy), with no blocking, fusion or reordering beyond what
the definition states.  Sources (page title, then section):

* "DeepSeek-V4-Pro vs Inkling", Component-by-component table, CSA row: each
  compressed entry pools 8 overlapping raw tokens at stride 4 with a softmax
  taken separately per channel; a lightning indexer with 64 heads of dim 128
  scores entries with ReLU dot products weighted per head and keeps 1,024;
  the 128 query heads attend to those entries plus the sliding-window tokens.
* same table, HCA row: one entry per 128 raw tokens; dense attention over all
  entries plus a 128-token window, one KV head shared by all query heads.
* same table, sink row: one learnable logit per head whose exponential joins
  the softmax denominator only (no value, no output gate), so a head's weights
  may total less than one.
* same table, partial-RoPE row: the last 64 of the 512 dims of queries and
  entries are rotated; because an entry is key and value at once, the same 64
  dims of each head's output are rotated back (inverse rotation) so that an
  entry contributes according to relative distance; base 160,000.
* "DeepSeek-V4.1-Flash vs Inkling", partial-RoPE row: the KV cache is
  quantized after RoPE (so stored caches hold rotated values).
* "DeepSeek-V4-Pro" (model atlas), Raw config fields: head_dim 512,
  qk_rope_head_dim 64, index_n_heads 64, index_head_dim 128, index_topk 1024,
  sliding_window 128, num_attention_heads 128, num_key_value_heads 1,
  compress_rope_theta 160000, compress_ratios 4 (CSA) and 128 (HCA); for the output side,
  o_groups 16, o_lora_rank 1024 and hidden_size 7168.

Readings where the pages are silent are listed beside the function that takes
them (pairing of rotated dims, position of an entry, window edge, tie order,
fp8 format).  Parity unpinned against the pages: the entry position (last raw
token), the adjacent pairing of rotated dims, the default softmax scale
1/sqrt(512), one indexer key per entry shared by all indexer heads, the window
edge (p - 128, p], and the YaRN ramp limits (1 and 32 turns) and temperature
(0.1 ln s + 1), which the pages leave to the published method, and the FP4 cache
format (OCP MXFP4: E2M1 elements, power-of-two scales per 32 channels).  The tests pin each of
these conventions as written,
but no value on the pages fixes them.  All floating point is fp64 except where a reading says that a
quantisation decision is taken in fp32 (the kernel's precision).
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 512
ROPE_DIM = 64
ROPE_THETA = 160000.0
SLIDING_WINDOW = 128
CSA_WINDOW, CSA_STRIDE = 8, 4
HCA_WINDOW, HCA_STRIDE = 128, 128
FP8_E4M3_MAX = 448.0


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_round(x):
    """Round fp64 values to the nearest bfloat16 (ties to even), as fp64.

    bfloat16 keeps 8 significant bits and fp32's exponent range; values below
    2**-126 use the fixed subnormal spacing 2**-133.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, ex = np.frexp(ax)                     # ax = m * 2**ex, m in [0.5, 1)
    ex = np.maximum(ex, -125)                # subnormal range: spacing stays 2**-133
    ulp = np.ldexp(1.0, ex - 8)
    r = np.rint(x / ulp) * ulp               # np.rint: round half to even
    return np.where(ax == 0, x, r)


def fp8_e4m3_decode(codes):
    """OCP FP8 E4M3FN code -> fp64 value (bias 7, no infinities, 0x7F/0xFF NaN)."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    sub = m * np.ldexp(1.0, -9)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, v)


def fp8_e4m3_encode(x):
    """fp64 -> OCP FP8 E4M3FN code, round to nearest even, saturating at +-448.

    Reading (fp8 format): the stored KV cache uses the OCP E4M3FN encoding with
    saturation; the pages name FP8 storage but not the rounding mode.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.minimum(np.abs(x), FP8_E4M3_MAX)
    _, ex = np.frexp(ax)
    e = np.maximum(ex - 1, -6)               # unbiased exponent; subnormals share -6
    ulp = np.ldexp(1.0, e - 3)
    r = np.minimum(np.rint(ax / ulp) * ulp, FP8_E4M3_MAX)
    # code from the rounded magnitude (rounding may carry into the next binade)
    _, ex2 = np.frexp(r)
    e2 = ex2 - 1
    is_norm = r >= np.ldexp(1.0, -6)
    E = np.where(is_norm, e2 + 7, 0)
    M = np.where(is_norm, np.rint((r / np.ldexp(1.0, np.where(is_norm, e2, 0)) - 1.0) * 8.0),
                 np.rint(r / np.ldexp(1.0, -9)))
    code = (E.astype(np.int64) << 3) | M.astype(np.int64)
    code = np.where(r == 0, 0, code)
    code = code | np.where(np.signbit(x) & (r != 0), 0x80, 0)
    return code.astype(np.uint8)


def fp8_block_quantize(x, block):
    """Quantize rows of `x` [..., C] to e4m3fn codes with one fp32 scale per block.

    Reading (fp8 format): scale = amax / 448 over the block, code = RNE(x / scale).
    The quantisation decision is taken in fp32, the kernels' precision: x is
    first rounded to fp32, amax and the division are fp32 operations.
    A block of zeros gets scale 0 and codes 0.
    """
    x32 = np.asarray(x, dtype=np.float32)
    C = x32.shape[-1]
    xb = x32.reshape(x32.shape[:-1] + (C // block, block))
    amax = np.abs(xb).max(axis=-1)
    scale = (amax / np.float32(FP8_E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (xb / safe[..., None]).astype(np.float32)
    codes = fp8_e4m3_encode(y.astype(np.float64))
    codes = np.where(scale[..., None] > 0, codes, 0).astype(np.uint8)
    return codes.reshape(x32.shape), scale


def fp8_block_dequantize(codes, scales, block):
    """codes [..., C] x scales [..., C/block] -> fp64 values (value times scale)."""
    v = fp8_e4m3_decode(codes)
    C = v.shape[-1]
    s = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=-1)
    assert s.shape[-1] == C
    return v * s


FP4_E2M1_MAX = 6.0
MX_BLOCK = 32


def fp4_e2m1_decode(codes):
    """OCP FP4 E2M1 code (low 4 bits) -> fp64 value: sign bit 3, exponent bits 2..1
    (bias 1), mantissa bit 0; exponent 0 holds 0 and the subnormal 0.5.  The magnitudes are
    0, 0.5, 1, 1.5, 2, 3, 4, 6."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    v = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.ldexp(1.0, e - 1))
    return sign * v


def fp4_e2m1_encode(x):
    """fp64 -> E2M1 code, round to nearest even, saturating at +-6.

    Reading (FP4 format): the pages name an FP4 KV cache quantized after RoPE
    ("DeepSeek-V4.1-Flash vs Inkling", partial-RoPE row) and MXFP4 in training; the
    element format taken is OCP E2M1 with round-to-nearest-even and saturation.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.minimum(np.abs(x), FP4_E2M1_MAX)
    ulp = np.where(ax < 2.0, 0.5, np.where(ax < 4.0, 1.0, 2.0))   # grid spacing of the binade
    r = np.minimum(np.rint(ax / ulp) * ulp, FP4_E2M1_MAX)           # rint: ties to even
    mags = fp4_e2m1_decode(np.arange(8))
    code = np.argmin(np.abs(r[..., None] - mags), axis=-1).astype(np.int64)   # r is on the grid
    code = code | np.where(np.signbit(x) & (r != 0), 8, 0)
    return code.astype(np.uint8)


def mxfp4_block_quantize(x, block=MX_BLOCK):
    """Quantize rows of `x` [..., C] to E2M1 codes with one power-of-two scale per block.

    Reading (FP4 format): OCP MXFP4 blocks of 32 channels; the block's scale is
    2^(floor(log2(amax)) - 2), which puts the largest magnitude in [4, 8) before rounding
    (values above 6 saturate); a block of zeros gets scale 1 and codes 0.  As for fp8, the
    decision is taken in fp32 (x rounded to fp32, amax and the scaling in fp32).  Returns the
    codes [..., C] (one per byte) and the fp32 scales [..., C / block].
    """
    x32 = np.asarray(x, dtype=np.float32)
    C = x32.shape[-1]
    xb = x32.reshape(x32.shape[:-1] + (C // block, block))
    amax = np.abs(xb).max(axis=-1)
    _, ex = np.frexp(amax.astype(np.float64))                      # amax = m * 2^ex, m in [0.5, 1)
    e = np.clip(ex - 1 - 2, -127, 127)
    scale = np.where(amax > 0, np.ldexp(np.float32(1.0), e), np.float32(1.0)).astype(np.float32)
    y = (xb / scale[..., None]).astype(np.float32)                 # exact: division by a power of two
    codes = fp4_e2m1_encode(y.astype(np.float64))
    return codes.reshape(x32.shape), scale


def mxfp4_block_dequantize(codes, scales, block=MX_BLOCK):
    """codes [..., C] (one E2M1 code per entry) x scales [..., C/block] -> fp64 values."""
    v = fp4_e2m1_decode(codes)
    s = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=-1)
    assert s.shape[-1] == v.shape[-1]
    return v * s


def fp4_pack(codes):
    """Two E2M1 codes per byte: channel 2k in the low nibble, 2k + 1 in the high nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def fp4_unpack(packed):
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


# --------------------------------------------------------------------------
# Partial RoPE
# --------------------------------------------------------------------------

def rope_inv_freq(theta=ROPE_THETA, rope_dim=ROPE_DIM):
    """Inverse frequencies theta**(-2i/rope_dim), i = 0 .. rope_dim/2 - 1 (fp64).

    Base 160,000 for the compressed layers (atlas page, Raw config fields,
    compress_rope_theta).  YaRN rescaling is not applied here: the kernels take
    the table from the caller.
    """
    i = np.arange(rope_dim // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / rope_dim)


def yarn_inv_freq(theta=ROPE_THETA, rope_dim=ROPE_DIM, factor=16.0, base_len=65536, alpha=1.0, beta=32.0):
    """YaRN frequencies for positions past the base context (fp64).

    The pages state YaRN with factor 16 over a 65,536-token base, base 160,000, up to
    1,048,576 positions ("DeepSeek-V4-Pro vs Inkling", Component-by-component table,
    partial-RoPE row).  Everything else is the YaRN method as published ("NTK-by-parts"):
    pair i has wavelength 2*pi/f_i and turns r_i = base_len / wavelength times over the
    base context; with ramp g = 0 below alpha turns, 1 above beta turns and linear in
    between, the new frequency is (1 - g) * f_i / factor + g * f_i.  Reading (parity
    unpinned): alpha = 1 and beta = 32, the values the method recommends; no page gives them.
    """
    out = np.empty(rope_dim // 2, dtype=np.float64)
    for i in range(rope_dim // 2):
        f = np.float64(theta) ** (-2.0 * i / rope_dim)
        wavelength = 2.0 * np.pi / f
        turns = base_len / wavelength
        if turns < alpha:
            g = 0.0
        elif turns > beta:
            g = 1.0
        else:
            g = (turns - alpha) / (beta - alpha)
        out[i] = (1.0 - g) * f / factor + g * f
    return out


def yarn_logit_scale(factor=16.0):
    """YaRN attention temperature as a multiplier of the logits: sqrt(1/t) = 0.1 ln(factor) + 1
    (the published method; parity unpinned: the pages give only the factor)."""
    if factor <= 1.0:
        return 1.0
    m = 0.1 * np.log(np.float64(factor)) + 1.0
    return float(m * m)


def rope(x, pos, inv_freq):
    """Rotate the last 2*len(inv_freq) dims of x at position(s) `pos`.

    Reading (pairing): dims (D-R+2i, D-R+2i+1) form the i-th pair, rotated by
    angle pos * inv_freq[i] (the complex-number view behind "rotate by -i" on
    the partial-RoPE row).  `pos` broadcasts against x.shape[:-1] and may be
    negative (the output's inverse rotation).
    """
    x = np.array(x, dtype=np.float64, copy=True)
    R = 2 * len(inv_freq)
    if R == 0:
        return x
    D = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * np.asarray(inv_freq, np.float64)
    c, s = np.cos(ang), np.sin(ang)
    a = x[..., D - R::2].copy()
    b = x[..., D - R + 1::2].copy()
    x[..., D - R::2] = a * c - b * s
    x[..., D - R + 1::2] = a * s + b * c
    return x


# --------------------------------------------------------------------------
# KV compression (CSA: window 8 / stride 4; HCA: window = stride = 128)
# --------------------------------------------------------------------------

def n_entries(n_raw, window, stride):
    """Number of complete windows of `window` raw tokens at step `stride`."""
    if n_raw < window:
        return 0
    return (n_raw - window) // stride + 1


def entry_positions(pos0, n, window, stride):
    """Position of entry j: that of the last raw token it pools.

    Reading (entry position): an entry is stamped with its last token's
    position, which is also when it becomes visible (a query sees an entry only
    once all of its tokens are at or before the query).
    """
    return np.int64(pos0) + np.arange(n, dtype=np.int64) * stride + (window - 1)


def pool(kv, z, window, stride):
    """Softmax pooling, per channel, of `window` consecutive raw rows at step `stride`.

    kv, z: [T, C].  Entry j, channel c:
        a_t = exp(z[stride*j + t, c]),  t = 0 .. window-1
        e[j, c] = sum_t a_t kv[stride*j + t, c] / sum_t a_t
    (max-subtracted for range; the value is the same).
    """
    kv = np.asarray(kv, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    T, C = kv.shape
    E = n_entries(T, window, stride)
    if E == 0:
        return np.zeros((0, C))
    zw = np.lib.stride_tricks.sliding_window_view(z, window, axis=0)[::stride][:E]    # [E, C, w]
    kw = np.lib.stride_tricks.sliding_window_view(kv, window, axis=0)[::stride][:E]
    m = zw.max(axis=-1, keepdims=True)
    a = np.exp(zw - m)
    return (a * kw).sum(axis=-1) / a.sum(axis=-1)


def compress(kv, z, window, stride, pos0, inv_freq):
    """Pool raw rows into entries and rotate each at its own position.

    Returns (entries [E, C] fp64, rotated; positions [E] int64).  With
    window = stride = 1 this is the raw-window write: each token rotated at its
    own position.
    """
    e = pool(kv, z, window, stride)
    p = entry_positions(pos0, e.shape[0], window, stride)
    return rope(e, p, inv_freq), p


# --------------------------------------------------------------------------
# Lightning indexer and top-k
# --------------------------------------------------------------------------

def index_scores(q_idx, w, keys):
    """s[j] = sum_h w[h] * max(0, q_idx[h] . keys[j]).

    q_idx [Hi, Di], w [Hi], keys [E, Di] (already dequantized).  Reading (key
    shape): one Di-dim key per compressed entry, shared by all indexer heads;
    no extra scale and no rotation inside the indexer.
    """
    q = np.asarray(q_idx, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    dots = k @ q.T                                    # [E, Hi]
    return np.maximum(dots, 0.0) @ w                  # [E]


def visible_mask(entry_pos, q_pos):
    """An entry is visible once its last token is at or before the query."""
    return np.asarray(entry_pos) <= q_pos


def topk_select(scores, visible, k):
    """Indices of the k visible entries with the largest score, ascending.

    Reading (ties): an exact tie goes to the smaller index.  All visible
    entries when at most k are visible.  The result is a set, returned sorted.
    """
    s = np.asarray(scores, dtype=np.float64)
    cand = np.nonzero(np.asarray(visible))[0]
    if cand.size <= k:
        return cand.astype(np.int64)
    order = np.lexsort((cand, -s[cand]))              # primary: -score, then index
    return np.sort(cand[order[:k]]).astype(np.int64)


def window_rows(row_pos, q_pos, W=SLIDING_WINDOW):
    """Raw tokens whose position lies in (q_pos - W, q_pos] (the query's own included)."""
    p = np.asarray(row_pos)
    return (p > q_pos - W) & (p <= q_pos)


# --------------------------------------------------------------------------
# Shared-KV attention with sink and output inverse rotation
# --------------------------------------------------------------------------

def attend(q, q_pos, X, sink, scale, inv_freq, return_weights=False):
    """Multi-query attention of H heads over rows X that are key and value at once.

    q [H, D] un-rotated, X [U, D] stored (already rotated) rows, sink [H].
      q'   = rope(q, q_pos)
      l_hu = scale * q'_h . X_u
      Z_h  = exp(sink_h) + sum_u exp(l_hu)
      o_h  = rope(sum_u exp(l_hu) / Z_h * X_u, -q_pos)
    Returns (o [H, D], lse [H] = log Z_h[, weights [H, U]]).
    """
    q = np.asarray(q, dtype=np.float64)
    X = np.asarray(X, dtype=np.float64)
    sink = np.asarray(sink, dtype=np.float64)
    qr = rope(q, q_pos, inv_freq)
    logits = scale * (qr @ X.T)                        # [H, U]
    if X.shape[0]:
        m = np.maximum(logits.max(axis=1), sink)
    else:
        m = sink.copy()
    e = np.exp(logits - m[:, None])
    es = np.exp(sink - m)
    Z = es + e.sum(axis=1)
    o = (e @ X) / Z[:, None]
    o = rope(o, -q_pos, inv_freq)
    lse = m + np.log(Z)
    if return_weights:
        return o, lse, e / Z[:, None]
    return o, lse


# --------------------------------------------------------------------------
# One decode / prefill step, composed from the functions above
# --------------------------------------------------------------------------

def csa_query(q, q_pos, q_idx, w, entries, entry_pos, keys, win, win_pos, sink, topk,
              scale, inv_freq, W=SLIDING_WINDOW):
    """CSA for one query token: index, select, then attend to top-k + window.

    Reading: the attended set is the plain union of the selected entries and
    the window rows (no de-duplication).
    Returns (o, lse, selected indices, scores, visible mask).
    """
    vis = visible_mask(entry_pos, q_pos)
    s = index_scores(q_idx, w, keys)
    sel = topk_select(s, vis, topk)
    wm = window_rows(win_pos, q_pos, W)
    X = np.concatenate([np.asarray(entries, np.float64)[sel], np.asarray(win, np.float64)[wm]], 0)
    o, lse = attend(q, q_pos, X, sink, scale, inv_freq)
    return o, lse, sel, s, vis


def hca_query(q, q_pos, entries, entry_pos, win, win_pos, sink, scale, inv_freq,
              W=SLIDING_WINDOW):
    """HCA for one query token: every visible entry plus the window."""
    vis = visible_mask(entry_pos, q_pos)
    wm = window_rows(win_pos, q_pos, W)
    X = np.concatenate([np.asarray(entries, np.float64)[vis], np.asarray(win, np.float64)[wm]], 0)
    return attend(q, q_pos, X, sink, scale, inv_freq)


# --------------------------------------------------------------------------
# Grouped low-rank output projection (after attention)
# --------------------------------------------------------------------------

O_GROUPS = 16
O_LORA_RANK = 1024
HIDDEN = 7168


def out_projection(o, wa, wb):
    """The attention output of a token, projected back to the hidden size through grouped low-rank
    factors ("DeepSeek-V4-Pro" model atlas, Raw config fields o_groups 16, o_lora_rank 1024,
    hidden_size 7168; the fields alone are given, the reading below is the plainest one they
    support): the heads' outputs (after the inverse rotation) are cut into G groups of H / G
    consecutive heads; group g's H/G * D values go through its own down factor
    wa[g] (R x (H/G) D) to R values; the G * R values, concatenated in group order, go through
    the up factor wb (hidden x G R).

    o: [T, H, D]; wa: [G, R, (H/G) D]; wb: [hidden, G R].  Returns (y [T, hidden], z [T, G, R])."""
    o = np.asarray(o, np.float64)
    wa = np.asarray(wa, np.float64)
    wb = np.asarray(wb, np.float64)
    T, H, D = o.shape
    G, R, Kg = wa.shape
    assert H % G == 0 and Kg == (H // G) * D and wb.shape[1] == G * R
    xg = o.reshape(T, G, Kg)                      # group g = heads g H/G .. (g + 1) H/G - 1
    z = np.einsum("tgk,grk->tgr", xg, wa)         # each group through its own down factor
    y = z.reshape(T, G * R) @ wb.T                # concatenated, through the up factor
    return y, z
