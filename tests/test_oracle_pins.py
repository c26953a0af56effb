"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: constants the
pages print, closed forms, invariants the pages state, library routines in a
special case, or the independent pure-Python brute force.  Chosen so that a
dropped term, a wrong sign or index, or a transposed operand fails one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import brute
from oracle import csa_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- constants

def test_oracle_constants_are_the_pages():
    g = json.load(open(os.path.join(GOLD, "page_config.json")))
    assert O.HEAD_DIM == g["head_dim"]["value"]
    assert O.ROPE_DIM == g["rope_dim"]["value"]
    assert O.ROPE_THETA == g["rope_theta"]["value"]
    assert O.SLIDING_WINDOW == g["sliding_window"]["value"]
    assert (O.CSA_WINDOW, O.CSA_STRIDE) == (g["csa_window"]["value"], g["csa_stride"]["value"])
    assert O.HCA_WINDOW == O.HCA_STRIDE == g["hca_window"]["value"]
    assert g["csa_layers"]["value"] + g["hca_layers"]["value"] == g["num_hidden_layers"]["value"]
    assert (O.O_GROUPS, O.O_LORA_RANK, O.HIDDEN) == (g["o_groups"]["value"], g["o_lora_rank"]["value"],
                                                     g["hidden_size"]["value"])


def test_entry_counts_golden():
    g = json.load(open(os.path.join(GOLD, "entry_counts.json")))
    for c in g["cases"]:
        w, s = {"csa": (8, 4), "csa2": (2, 2), "hca": (128, 128)}[c["mode"]]
        assert O.n_entries(c["n_raw"], w, s) == c["entries"], c
        # the vectorised pooling produces exactly that many rows on small streams
        if c["n_raw"] <= 4096:
            kv = np.zeros((c["n_raw"], 2))
            assert O.pool(kv, kv, w, s).shape[0] == c["entries"]


def test_entry_position_is_last_token():
    # An entry is visible exactly when all of its tokens are at or before the query.
    p = O.entry_positions(pos0=1, n=5, window=8, stride=4)
    assert list(p) == [8, 12, 16, 20, 24]
    assert list(O.visible_mask(p, 15)) == [True, True, False, False, False]
    assert list(O.entry_positions(pos0=0, n=2, window=128, stride=128)) == [127, 255]


# ---------------------------------------------------------------- pooling

def test_pool_equal_logits_is_window_mean_closed_form():
    T, C = 40, 3
    t = np.arange(T, dtype=np.float64)[:, None]
    c = np.arange(C, dtype=np.float64)[None, :]
    kv = t * (c + 1.0) + 0.25 * c            # row t, channel c
    z = np.full((T, C), 0.7)
    e = O.pool(kv, z, 8, 4)
    j = np.arange(e.shape[0], dtype=np.float64)[:, None]
    np.testing.assert_allclose(e, (4 * j + 3.5) * (c + 1.0) + 0.25 * c, rtol=0, atol=1e-12)
    # HCA geometry: entries cover disjoint 128-token blocks
    T = 300
    kv = np.arange(T, dtype=np.float64)[:, None] * np.ones((1, 2))
    e = O.pool(kv, np.zeros((T, 2)), 128, 128)
    np.testing.assert_allclose(e[:, 0], [63.5, 191.5], atol=1e-12)


def test_pool_dominant_logit_picks_that_token():
    r = rng(1)
    T, C = 24, 5
    kv = r.standard_normal((T, C))
    z = r.standard_normal((T, C))
    pick = r.integers(0, 8, size=C)
    E = O.n_entries(T, 8, 4)
    for j in range(E):
        zz = z.copy()
        for ch in range(C):
            zz[4 * j + pick[ch], ch] = 1e4
        e = O.pool(kv, zz, 8, 4)
        for ch in range(C):
            assert e[j, ch] == pytest.approx(kv[4 * j + pick[ch], ch], abs=1e-12)


def test_pool_softmax_is_per_channel():
    r = rng(2)
    kv = r.standard_normal((16, 4))
    z = r.standard_normal((16, 4))
    base = O.pool(kv, z, 8, 4)
    # a per-channel constant shift of the logits changes nothing
    np.testing.assert_allclose(O.pool(kv, z + np.array([3.0, -7.0, 0.5, 100.0]), 8, 4), base,
                               atol=1e-12)
    # changing one channel's logits leaves the other channels untouched
    z2 = z.copy()
    z2[:, 1] = r.standard_normal(16)
    e2 = O.pool(kv, z2, 8, 4)
    np.testing.assert_array_equal(e2[:, [0, 2, 3]], base[:, [0, 2, 3]])
    assert np.abs(e2[:, 1] - base[:, 1]).max() > 1e-3
    # window = stride = 1 is the identity
    np.testing.assert_allclose(O.pool(kv, z, 1, 1), kv, atol=0)


def test_pool_matches_torch_softmax():
    r = rng(3)
    kv = r.standard_normal((36, 6))
    z = r.standard_normal((36, 6))
    e = O.pool(kv, z, 8, 4)
    for j in range(e.shape[0]):
        zz = torch.from_numpy(z[4 * j:4 * j + 8])
        a = torch.softmax(zz, dim=0).numpy()
        np.testing.assert_allclose(e[j], (a * kv[4 * j:4 * j + 8]).sum(0), atol=1e-13)


# ---------------------------------------------------------------- RoPE

def test_inv_freq_closed_form():
    f = O.rope_inv_freq(160000.0, 64)
    assert f.shape == (32,)
    assert f[0] == 1.0
    assert f[31] == pytest.approx(160000.0 ** (-62 / 64), rel=1e-15)
    ratio = f[1:] / f[:-1]
    np.testing.assert_allclose(ratio, 160000.0 ** (-1 / 32), rtol=1e-14)


def test_rope_is_complex_rotation_of_last_pairs():
    r = rng(4)
    f = O.rope_inv_freq(160000.0, 64)
    x = r.standard_normal((3, 512))
    pos = np.array([0, 17, 1048575])
    y = O.rope(x, pos, f)
    np.testing.assert_array_equal(y[:, :448], x[:, :448])
    zc = (x[:, 448::2] + 1j * x[:, 449::2]) * np.exp(1j * pos[:, None] * f[None, :])
    np.testing.assert_allclose(y[:, 448::2], zc.real, atol=1e-12)
    np.testing.assert_allclose(y[:, 449::2], zc.imag, atol=1e-12)
    np.testing.assert_array_equal(y[0], x[0])                       # position 0
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_allclose(O.rope(y, -pos, f), x, atol=1e-12)   # inverse


def test_rope_dot_depends_on_distance_only():
    r = rng(5)
    f = O.rope_inv_freq(160000.0, 64)
    a = r.standard_normal(512)
    b = r.standard_normal(512)
    d1 = O.rope(a, 1000, f) @ O.rope(b, 900, f)
    d2 = O.rope(a, 5100, f) @ O.rope(b, 5000, f)
    d3 = O.rope(a, 1000, f) @ O.rope(b, 901, f)
    assert d1 == pytest.approx(d2, abs=1e-10)
    assert abs(d1 - d3) > 1e-6


# ---------------------------------------------------------------- indexer / top-k

def test_index_scores_special_cases():
    r = rng(6)
    K = r.standard_normal((50, 16))
    q = r.standard_normal((1, 16))
    s = O.index_scores(q, np.ones(1), K)
    np.testing.assert_allclose(s, np.maximum(np.dot(K, q[0]), 0), atol=1e-13)
    # all dot products negative -> zero score
    assert np.all(O.index_scores(-np.abs(q), np.ones(1), np.abs(K)) == 0)
    # several heads: weighted sum of the single-head scores, one key shared by all heads
    Q = r.standard_normal((4, 16))
    w = r.uniform(0, 1, 4)
    s4 = O.index_scores(Q, w, K)
    parts = sum(w[h] * O.index_scores(Q[h:h + 1], np.ones(1), K) for h in range(4))
    np.testing.assert_allclose(s4, parts, atol=1e-12)
    # the weight multiplies after the ReLU: a negative weight subtracts
    s_neg = O.index_scores(Q[:1], -np.ones(1), K)
    np.testing.assert_allclose(s_neg, -np.maximum(K @ Q[0], 0), atol=1e-13)


def test_topk_select_against_library_sorts():
    r = rng(7)
    s = r.standard_normal(300)
    vis = r.uniform(size=300) < 0.8
    k = 37
    sel = O.topk_select(s, vis, k)
    cand = np.nonzero(vis)[0]
    tv, ti = torch.topk(torch.from_numpy(s[cand]), k)
    assert set(sel.tolist()) == set(cand[ti.numpy()].tolist())
    order = np.argsort(-s[cand], kind="stable")[:k]
    assert set(sel.tolist()) == set(cand[order].tolist())
    # k at least the visible count -> every visible entry
    assert list(O.topk_select(s, vis, 1000)) == list(cand)
    # exact ties go to the smaller index
    t = np.array([1.0, 2.0, 2.0, 2.0, 0.5, 2.0])
    assert list(O.topk_select(t, np.ones(6, bool), 2)) == [1, 2]
    assert list(O.topk_select(t, np.array([1, 0, 1, 1, 1, 1], bool), 3)) == [2, 3, 5]


def test_window_edge():
    p = np.arange(1, 300)
    m = O.window_rows(p, 290, 128)
    assert p[m].min() == 163 and p[m].max() == 290 and m.sum() == 128
    m = O.window_rows(p, 50, 128)
    assert m.sum() == 50


# ---------------------------------------------------------------- attention

def _att_inputs(seed=8, H=4, U=30, D=64, sink_scale=1.0):
    r = rng(seed)
    return (r.standard_normal((H, D)), r.standard_normal((U, D)),
            sink_scale * r.standard_normal(H))


def test_attend_without_sink_is_sdpa():
    q, X, _ = _att_inputs()
    scale = 0.3
    o, lse = O.attend(q, 0, X, np.full(4, -np.inf), scale, np.zeros(0))
    ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None, :, None, :],
                                         torch.from_numpy(X)[None, None].expand(1, 4, -1, -1),
                                         torch.from_numpy(X)[None, None].expand(1, 4, -1, -1),
                                         scale=scale)[0, :, 0, :].numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)
    lse_ref = torch.logsumexp(torch.from_numpy(scale * q @ X.T), dim=1).numpy()
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_attend_sink_weights_sum_below_one():
    q, X, sink = _att_inputs(sink_scale=2.0)
    f = O.rope_inv_freq(160000.0, 16)
    o, lse, wts = O.attend(q, 77, X, sink, 0.2, f, return_weights=True)
    np.testing.assert_allclose(wts.sum(1), 1.0 - np.exp(sink - lse), atol=1e-13)
    assert np.all(wts.sum(1) < 1.0)
    # the sink carries no value: o equals the weighted rows, rotated back
    back = O.rope(wts @ X, -77, f)
    np.testing.assert_allclose(o, back, atol=1e-12)
    # an empty row set leaves only the sink
    o0, lse0 = O.attend(q, 5, X[:0], sink, 0.2, f)
    assert np.all(o0 == 0) and np.allclose(lse0, sink)


def test_attend_convexity_and_symmetries():
    q, X, sink = _att_inputs(seed=9, H=3, U=25, D=64)
    f = O.rope_inv_freq(160000.0, 16)
    o, lse = O.attend(q, 1234, X, sink, 1.0, f)
    # un-rotated dims are a sub-convex combination of the rows
    bound = np.abs(X[:, :48]).max(0)
    assert np.all(np.abs(o[:, :48]) <= bound + 1e-12)
    pairs = np.sqrt(X[:, 48::2] ** 2 + X[:, 49::2] ** 2).max(0)
    assert np.all(np.sqrt(o[:, 48::2] ** 2 + o[:, 49::2] ** 2) <= pairs + 1e-12)
    # row order does not matter
    perm = rng(10).permutation(25)
    o2, lse2 = O.attend(q, 1234, X[perm], sink, 1.0, f)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)
    # heads with the same query and sink give the same output
    qq = np.repeat(q[:1], 3, 0)
    o3, _ = O.attend(qq, 1234, X, np.repeat(sink[:1], 3), 1.0, f)
    np.testing.assert_allclose(o3[1], o3[0], atol=0)
    np.testing.assert_allclose(o3[2], o3[0], atol=0)


def _tiny_stream(seed, T, D=16, H=2, Hi=3, Di=8):
    r = rng(seed)
    return dict(kv=r.standard_normal((T, D)), z=r.standard_normal((T, D)),
                q=r.standard_normal((H, D)) / 2, q_idx=r.standard_normal((Hi, Di)),
                w=r.uniform(0, 1, Hi), keys=r.standard_normal((T, Di)),
                sink=r.standard_normal(H))


def _csa_from_stream(s, pos0, k, W, scale, f, q_pos=None, window=8, stride=4):
    T = s["kv"].shape[0]
    q_pos = pos0 + T - 1 if q_pos is None else q_pos
    ent, ep = O.compress(s["kv"], s["z"], window, stride, pos0, f)
    win, wp = O.compress(s["kv"], s["z"], 1, 1, pos0, f)
    E = ent.shape[0]
    return O.csa_query(s["q"], q_pos, s["q_idx"], s["w"], ent, ep, s["keys"][:E], win, wp,
                       s["sink"], k, scale, f, W)


def test_shift_of_all_positions_changes_nothing():
    s = _tiny_stream(11, 40)
    f = O.rope_inv_freq(160000.0, 4)
    o1, l1, sel1, *_ = _csa_from_stream(s, 1, 3, 6, 0.7, f)
    o2, l2, sel2, *_ = _csa_from_stream(s, 1 + 98765, 3, 6, 0.7, f)
    assert list(sel1) == list(sel2)
    np.testing.assert_allclose(o2, o1, atol=1e-10)
    np.testing.assert_allclose(l2, l1, atol=1e-12)


def test_topk_at_least_entries_is_dense_attention():
    s = _tiny_stream(12, 44)
    f = O.rope_inv_freq(160000.0, 4)
    T = 44
    o1, l1, sel, *_ = _csa_from_stream(s, 3, 1000, 6, 0.9, f)
    assert len(sel) == O.n_entries(T, 8, 4)
    ent, ep = O.compress(s["kv"], s["z"], 8, 4, 3, f)
    win, wp = O.compress(s["kv"], s["z"], 1, 1, 3, f)
    o2, l2 = O.hca_query(s["q"], 3 + T - 1, ent, ep, win, wp, s["sink"], 0.9, f, 6)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_prefill_visibility_excludes_incomplete_entries():
    s = _tiny_stream(13, 40)
    f = O.rope_inv_freq(160000.0, 4)
    # query at raw index 21 (position 22): entries ending at positions 8..20 are visible
    _, _, sel, sc, vis = _csa_from_stream(s, 1, 100, 6, 1.0, f, q_pos=22)
    assert list(np.nonzero(vis)[0]) == [0, 1, 2, 3]
    assert list(sel) == [0, 1, 2, 3]


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed,T,k,W,R,pos0", [(20, 16, 3, 4, 4, 1), (21, 37, 2, 5, 4, 0),
                                                 (22, 64, 5, 4, 4, 1000), (23, 8, 3, 4, 2, 7)])
def test_whole_csa_step_matches_brute_force(seed, T, k, W, R, pos0):
    s = _tiny_stream(seed, T, D=8, H=2)
    scale = 0.8
    f = O.rope_inv_freq(160000.0, R)
    fb = brute.inv_freq(160000.0, R)
    o, lse, sel, sc, vis = _csa_from_stream(s, pos0, k, W, scale, f)
    lst = lambda a: [list(map(float, r)) for r in a]
    ob, lb, selb, scb = brute.csa_step(lst(s["kv"]), lst(s["z"]), pos0, lst(s["q"]), pos0 + T - 1,
                                       lst(s["q_idx"]), list(s["w"]), lst(s["keys"]),
                                       list(s["sink"]), k, W, scale, fb)
    assert list(sel) == selb
    np.testing.assert_allclose(sc[:len(scb)], scb, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-12)


@pytest.mark.parametrize("seed,T,k,W", [(24, 16, 3, 4), (25, 33, 4, 5)])
def test_whole_csa2_step_matches_brute_force(seed, T, k, W):
    """CSA2 geometry: entries pool 2 raw tokens into 1 (window = stride = 2)."""
    s = _tiny_stream(seed, T, D=8, H=2)
    f = O.rope_inv_freq(160000.0, 4)
    o, lse, sel, sc, vis = _csa_from_stream(s, 3, k, W, 0.6, f, window=2, stride=2)
    lst = lambda a: [list(map(float, r)) for r in a]
    ob, lb, selb, scb = brute.csa_step(lst(s["kv"]), lst(s["z"]), 3, lst(s["q"]), 3 + T - 1,
                                       lst(s["q_idx"]), list(s["w"]), lst(s["keys"]),
                                       list(s["sink"]), k, W, 0.6, brute.inv_freq(160000.0, 4), 2, 2)
    assert list(sel) == selb
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-12)


@pytest.mark.parametrize("seed,T,window,W", [(30, 40, 8, 4), (31, 300, 128, 128)])
def test_whole_hca_step_matches_brute_force(seed, T, window, W):
    s = _tiny_stream(seed, T, D=8, H=2)
    f = O.rope_inv_freq(160000.0, 4)
    ent, ep = O.compress(s["kv"], s["z"], window, window, 5, f)
    win, wp = O.compress(s["kv"], s["z"], 1, 1, 5, f)
    o, lse = O.hca_query(s["q"], 5 + T - 1, ent, ep, win, wp, s["sink"], 0.5, f, W)
    lst = lambda a: [list(map(float, r)) for r in a]
    ob, lb = brute.hca_step(lst(s["kv"]), lst(s["z"]), 5, lst(s["q"]), 5 + T - 1, list(s["sink"]),
                            W, 0.5, brute.inv_freq(160000.0, 4), window, window)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lb, rtol=1e-12)


# ---------------------------------------------------------------- number formats

def test_fp8_decode_matches_library_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.fp8_e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(lib)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], lib[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def test_fp8_encode_matches_library_in_range_and_saturates():
    r = rng(14)
    x = np.concatenate([r.standard_normal(20000) * 50, r.standard_normal(5000) * 1e-2,
                        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10])])
    x = x[np.abs(x) <= 448].astype(np.float32)
    ours = O.fp8_e4m3_encode(x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # -0.0 encodes as +0 here; compare values for it
    np.testing.assert_array_equal(O.fp8_e4m3_decode(ours), O.fp8_e4m3_decode(lib))
    assert O.fp8_e4m3_encode(np.array([1e6]))[0] == 0x7E
    assert O.fp8_e4m3_encode(np.array([-500.0]))[0] == 0xFE
    codes, sc = O.fp8_block_quantize(r.standard_normal((3, 128)), 64)
    assert sc.dtype == np.float32 and sc.shape == (3, 2)
    assert np.all(np.abs(O.fp8_e4m3_decode(codes)).reshape(3, 2, 64).max(-1) == 448.0)


def test_fp8_block_dequantize_hand_values():
    """Codes and scales written out by hand, with every block a different scale, so that a
    block index taken modulo instead of divided (np.tile for np.repeat), a wrong block size or
    a transposed block layout moves a value."""
    one, neg_one, tiny, top = 0x38, 0xB8, 0x01, 0x7E        # 1.0, -1.0, 2^-9, 448 in E4M3FN
    pattern = np.array([one, neg_one, tiny, top], dtype=np.uint8)
    vals = np.array([1.0, -1.0, 2.0 ** -9, 448.0])
    codes = np.stack([np.full(256, one, dtype=np.uint8), np.tile(pattern, 64)])        # [2, 256]
    # block 64: four scales per row
    sc64 = np.array([[0.5, 2.0, 3.0, 0.25], [1.0, 4.0, 0.125, 10.0]], dtype=np.float32)
    want = np.empty((2, 256))
    want[0, 0:64], want[0, 64:128], want[0, 128:192], want[0, 192:256] = 0.5, 2.0, 3.0, 0.25
    for c in range(256):
        want[1, c] = vals[c % 4] * [1.0, 4.0, 0.125, 10.0][c // 64]
    got = O.fp8_block_dequantize(codes, sc64, 64)
    np.testing.assert_array_equal(got, want)
    # block 128: two scales per row (the indexer-key layout when C = 256)
    sc128 = np.array([[6.0, 0.75], [0.5, 8.0]], dtype=np.float32)
    want128 = np.empty((2, 256))
    want128[0, :128], want128[0, 128:] = 6.0, 0.75
    want128[1, :128] = np.tile(vals, 32) * 0.5
    want128[1, 128:] = np.tile(vals, 32) * 8.0
    np.testing.assert_array_equal(O.fp8_block_dequantize(codes, sc128, 128), want128)
    # leading batch dimensions broadcast row by row
    c3 = np.stack([codes, codes[::-1]])                        # [2, 2, 256]
    s3 = np.stack([sc64, sc64[::-1]])
    got3 = O.fp8_block_dequantize(c3, s3, 64)
    np.testing.assert_array_equal(got3[0], want)
    np.testing.assert_array_equal(got3[1], want[::-1])


def test_fp8_block_quantize_scales_and_codes():
    """Scales are fp32 amax / 448 per block and codes are the E4M3FN rounding of fp32 x / scale,
    checked against hand values and against torch's float8_e4m3fn conversion (a library routine),
    block by block, on rows whose blocks differ in magnitude by decades."""
    # hand values: block maxima that make the scale exact
    x = np.zeros((1, 256))
    x[0, 0:64] = np.linspace(-448.0, 100.0, 64)           # amax 448 -> scale 1, codes = E4M3(x)
    x[0, 64:128] = 0.0                                     # zero block -> scale 0, codes 0
    x[0, 128:192] = np.linspace(-3.0, 896.0, 64)           # amax 896 -> scale 2
    x[0, 192:256] = 1.0                                    # amax 1 -> scale fp32(1/448), codes 448
    codes, sc = O.fp8_block_quantize(x, 64)
    assert sc.dtype == np.float32 and sc.shape == (1, 4)
    assert sc[0, 0] == 1.0 and sc[0, 1] == 0.0 and sc[0, 2] == 2.0
    assert sc[0, 3] == np.float32(1.0) / np.float32(448.0)
    lib = lambda v: torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.fp8_e4m3_decode(codes[0, 0:64]), O.fp8_e4m3_decode(lib(x[0, 0:64])))
    assert np.all(codes[0, 64:128] == 0)
    np.testing.assert_array_equal(O.fp8_e4m3_decode(codes[0, 128:192]),
                                  O.fp8_e4m3_decode(lib(x[0, 128:192] / 2.0)))
    assert np.all(codes[0, 192:256] == 0x7E)
    # random rows: per-block magnitudes 1e-3 .. 1e3
    r = rng(16)
    y = r.standard_normal((5, 512)) * np.repeat(10.0 ** r.integers(-3, 4, size=(5, 8)), 64, axis=1)
    codes, sc = O.fp8_block_quantize(y, 64)
    y32 = torch.from_numpy(y.astype(np.float32)).view(5, 8, 64)
    sc_lib = (y32.abs().amax(-1) / torch.tensor(448.0, dtype=torch.float32)).numpy()
    np.testing.assert_array_equal(sc, sc_lib)
    code_lib = (y32 / torch.from_numpy(sc_lib)[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.fp8_e4m3_decode(codes.reshape(5, 8, 64)), O.fp8_e4m3_decode(code_lib))
    # the round trip is within half a code step of every value (the block's scale times 2^-4 of
    # the element's binade, or the subnormal spacing)
    back = O.fp8_block_dequantize(codes, sc, 64)
    step = np.repeat(sc.astype(np.float64), 64, axis=1) * np.ldexp(
        1.0, np.maximum(np.frexp(np.abs(y) / np.repeat(sc.astype(np.float64), 64, axis=1))[1] - 4, -9))
    assert np.all(np.abs(back - y) <= 0.5 * step * (1 + 1e-6))


def test_bf16_round_matches_library():
    r = rng(15)
    x = np.concatenate([r.standard_normal(20000).astype(np.float32),
                        (r.standard_normal(2000) * 1e-39).astype(np.float32)])
    ours = O.bf16_round(x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, lib)
    # exact ties go to the even neighbour
    assert O.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert O.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


# ---------------------------------------------------------------- YaRN table (partial-RoPE row: factor 16 over 65,536)

def test_yarn_factor_one_is_the_plain_table():
    # (1 - g) f + g f on the ramp pairs: equal to f up to one rounding
    np.testing.assert_allclose(O.yarn_inv_freq(160000.0, 64, factor=1.0, base_len=65536),
                               O.rope_inv_freq(160000.0, 64), rtol=4e-16, atol=0)


def test_yarn_regimes_follow_the_wavelengths():
    # a pair keeps its frequency when it turns more than 32 times over the base context and is
    # divided by the factor when it turns less than once; solving base_len * theta^(-2i/64) / (2 pi)
    # = turns for i gives the two index limits without the ramp formula
    theta, d, L, s = 160000.0, 64, 65536, 16.0
    f = O.rope_inv_freq(theta, d)
    y = O.yarn_inv_freq(theta, d, factor=s, base_len=L)
    i_keep = (d / 2) * math.log(L / (2 * math.pi * 32)) / math.log(theta)    # turns == 32
    i_interp = (d / 2) * math.log(L / (2 * math.pi)) / math.log(theta)       # turns == 1
    assert 10 < i_keep < i_interp < 31                                        # all three regimes occur
    for i in range(d // 2):
        if i < i_keep:
            assert y[i] == f[i]
        elif i > i_interp:
            assert y[i] == f[i] / s
        else:
            assert f[i] / s < y[i] < f[i]


def test_yarn_interpolated_pairs_map_the_longest_context_onto_the_base():
    # at the largest position (1,048,576 = 16 x 65,536) an interpolated pair turns exactly as far as
    # the plain table does at the end of the base context
    f = O.rope_inv_freq(160000.0, 64)
    y = O.yarn_inv_freq(160000.0, 64, factor=16.0, base_len=65536)
    slow = np.where(65536 * f / (2 * math.pi) < 1.0)[0]
    assert len(slow) > 0
    np.testing.assert_array_equal(1048576 * y[slow], 65536 * f[slow])


def test_yarn_table_is_monotone_and_between_the_limits():
    f = O.rope_inv_freq(160000.0, 64)
    y = O.yarn_inv_freq(160000.0, 64, factor=16.0, base_len=65536)
    assert np.all(np.diff(y) < 0)
    assert np.all(y <= f) and np.all(y >= f / 16.0)


def test_yarn_temperature_laws():
    # sqrt(scale) - 1 is proportional to ln(factor): no temperature at factor 1, and squaring the
    # factor doubles the excess
    assert O.yarn_logit_scale(1.0) == 1.0
    for s in (2.0, 4.0, 16.0):
        a = math.sqrt(O.yarn_logit_scale(s)) - 1.0
        b = math.sqrt(O.yarn_logit_scale(s * s)) - 1.0
        assert a > 0 and abs(b - 2 * a) < 1e-12
    assert O.yarn_logit_scale(16.0) > O.yarn_logit_scale(4.0)


# ---------------------------------------------------------------- FP4 (MXFP4) cache format

def test_fp4_decode_matches_the_format_table():
    g = json.load(open(os.path.join(GOLD, "fp4_e2m1.json")))
    v = O.fp4_e2m1_decode(np.arange(16))
    np.testing.assert_array_equal(v, np.array(g["values"]))
    assert np.all(np.signbit(v[8:])) and not np.any(np.signbit(v[:8]))


def test_fp4_encode_round_trip_ties_and_saturation():
    grid = O.fp4_e2m1_decode(np.arange(16))
    want = np.arange(16)
    want[8] = 0                                                            # -0 encodes as +0
    assert np.array_equal(O.fp4_e2m1_encode(grid), want)
    # midpoints between neighbours go to the neighbour with the even code
    mags = grid[:8]
    for a in range(7):
        mid = 0.5 * (mags[a] + mags[a + 1])
        want = a if a % 2 == 0 else a + 1
        assert O.fp4_e2m1_encode(mid) == want and O.fp4_e2m1_encode(-mid) == (want | 8 if want else 0)
    # nearest value off the midpoints, saturation past 6
    x = rng(5).uniform(-7, 7, 2000)
    got = O.fp4_e2m1_decode(O.fp4_e2m1_encode(x))
    best = grid[np.argmin(np.abs(x[:, None] - grid[None, :]), axis=1)]
    np.testing.assert_array_equal(np.abs(got), np.abs(best))
    assert O.fp4_e2m1_decode(O.fp4_e2m1_encode(100.0)) == 6.0 and O.fp4_e2m1_decode(O.fp4_e2m1_encode(-9.0)) == -6.0


def test_mxfp4_block_scales_are_powers_of_two_placing_amax_in_4_to_8():
    x = rng(6).normal(size=(7, 128)) * np.exp(rng(7).uniform(-8, 8, size=(7, 1)))
    x[3, 32:64] = 0.0
    codes, sc = O.mxfp4_block_quantize(x, 32)
    assert sc.shape == (7, 4) and sc.dtype == np.float32
    m, e = np.frexp(sc.astype(np.float64))
    assert np.all(m == 0.5)                                    # powers of two
    amax = np.abs(x.astype(np.float32).astype(np.float64)).reshape(7, 4, 32).max(-1)
    ratio = amax / sc
    nz = amax > 0
    assert np.all((ratio[nz] >= 4) & (ratio[nz] < 8))
    assert sc[3, 1] == 1.0 and np.all(codes[3, 32:64] == 0)   # a block of zeros
    # error: half a grid step where |x|/scale <= 6, the saturation gap above
    v = O.mxfp4_block_dequantize(codes, sc, 32)
    y = np.abs(x) / np.repeat(sc, 32, axis=-1)
    step = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
    bound = np.where(y <= 6, 0.5 * step, y - 6 + 1e-9) * np.repeat(sc, 32, axis=-1)
    assert np.all(np.abs(v - x) <= bound * (1 + 1e-6) + 1e-30)


def test_fp4_pack_order():
    c = np.array([[1, 2, 3, 4, 15, 0]], dtype=np.uint8)
    p = O.fp4_pack(c)
    assert list(p[0]) == [0x21, 0x43, 0x0F]
    assert np.array_equal(O.fp4_unpack(p), c)


# ---------------------------------------------------------------- grouped low-rank output projection

def _proj_case(T=3, H=8, D=6, G=4, R=5, hidden=7, seed=11):
    r = np.random.default_rng(seed)
    return r.normal(size=(T, H, D)), r.normal(size=(G, R, (H // G) * D)), r.normal(size=(hidden, G * R))


def test_out_projection_matches_brute_force_loops():
    o, wa, wb = _proj_case()
    y, _ = O.out_projection(o, wa, wb)
    yb = np.array(brute.out_projection(o.tolist(), wa.tolist(), wb.tolist()))
    assert np.allclose(y, yb, rtol=1e-12, atol=1e-12)


def test_out_projection_identity_down_factors_give_the_flat_output():
    # closed form: with wa[g] the identity (R = H/G * D) the rank-R codes are the group's own
    # values, head after head, and y is wb applied to the whole flattened output
    T, H, D, G = 2, 6, 4, 3
    o, _, _ = _proj_case(T, H, D, G, 8, 5)
    wa = np.stack([np.eye(8) for _ in range(G)])
    wb = np.random.default_rng(3).normal(size=(5, G * 8))
    y, z = O.out_projection(o, wa, wb)
    assert np.array_equal(z.reshape(T, H, D), o)
    assert np.allclose(y, o.reshape(T, H * D) @ wb.T, rtol=1e-13, atol=1e-13)


def test_out_projection_group_of_a_head_is_its_block_of_consecutive_heads():
    # zeroing the heads of group g changes only that group's codes, and y by exactly wb's block g
    o, wa, wb = _proj_case()
    G, R = wa.shape[:2]
    hg = o.shape[1] // G
    y, z = O.out_projection(o, wa, wb)
    for g in range(G):
        o2 = o.copy()
        o2[:, g * hg:(g + 1) * hg] = 0.0
        y2, z2 = O.out_projection(o2, wa, wb)
        keep = [x for x in range(G) if x != g]
        assert np.array_equal(z2[:, keep], z[:, keep])
        assert np.all(z2[:, g] == 0.0)
        assert np.allclose(y - y2, z[:, g] @ wb[:, g * R:(g + 1) * R].T, rtol=1e-12, atol=1e-12)


def test_out_projection_consistent_group_permutation_changes_nothing():
    o, wa, wb = _proj_case()
    G, R = wa.shape[:2]
    hg = o.shape[1] // G
    perm = np.array([2, 0, 3, 1])
    o2 = np.concatenate([o[:, p * hg:(p + 1) * hg] for p in perm], 1)
    wb2 = np.concatenate([wb[:, p * R:(p + 1) * R] for p in perm], 1)
    y, _ = O.out_projection(o, wa, wb)
    y2, _ = O.out_projection(o2, wa[perm], wb2)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-12)


def test_out_projection_one_group_is_two_matrix_products():
    # G = 1 reduces to the plain product wb (wa x), checked with torch's matmul in fp64
    o, _, _ = _proj_case(G=1)
    r = np.random.default_rng(5)
    wa = r.normal(size=(1, 5, o.shape[1] * o.shape[2]))
    wb = r.normal(size=(7, 5))
    y, _ = O.out_projection(o, wa, wb)
    x = torch.tensor(o.reshape(o.shape[0], -1))
    ref = torch.tensor(wb) @ (torch.tensor(wa[0]) @ x.T)
    assert np.allclose(y, ref.T.numpy(), rtol=1e-12, atol=1e-12)
