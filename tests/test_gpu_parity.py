"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Sizes span several tiles and ragged tails; edge cases: fewer visible entries
than k, a window cut by the start of the stream, heads fewer than one MFMA
block, split and unsplit attention, prefill rows with causal visibility, fp8
caches, tied scores, bf16 output and bitwise determinism.  Bars: tests/gpu_common.py.
"""
import math

import numpy as np
import pytest
import torch

import csa_inputs as ci
from compressed_attention_long_amd import _lib as ops
from compressed_attention_long_amd.rope import rope_inv_freq, yarn_inv_freq
from oracle import csa_oracle as O

from gpu_common import (ATT_TOL, LSE_TOL, check_attention, check_bf16_rows, check_fp4_rows, check_fp8_rows, check_lse, check_scores,
                        check_topk, lse_tolerance, np64, oracle_rows_csa, oracle_rows_hca, pool_error_bound,
                        score_error_bound, stored_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu case] {request.node.name}", flush=True)
    yield
    torch.cuda.synchronize()


def inv_freq_pair(R=64, yarn=False):
    """(table for the kernels, the oracle's own table): plain base 160,000, or YaRN 16 over 65,536."""
    if yarn:
        return yarn_inv_freq(160000.0, R, 16.0, 65536, DEV), O.yarn_inv_freq(160000.0, R, 16.0, 65536)
    return rope_inv_freq(160000.0, R, DEV), O.rope_inv_freq(160000.0, R)


# ---------------------------------------------------------------- compressor

@pytest.mark.parametrize("window,stride,dtype,B,n_new,first,R", [
    (8, 4, "bf16", 2, 1023, 0, 64),      # CSA, many rows (run mode), tiny-config length
    (8, 4, "bf16", 3, 37, 5, 64),        # ragged row count, offset first row
    (8, 4, "bf16", 1, 1, 9, 64),         # one decode-step entry
    (128, 128, "bf16", 2, 9, 1, 64),     # HCA geometry
    (1, 1, "bf16", 2, 200, 3, 64),       # raw-window write
    (8, 4, "fp8", 2, 333, 0, 64),        # fp8 cache, per-64 scales
    (128, 128, "fp8", 1, 5, 2, 64),
    (8, 4, "bf16", 1, 50, 0, 0),         # no rotation
    (8, 4, "bf16", 2, 77, 1, 128),       # wider rotations
    (128, 128, "fp8", 2, 5, 0, 512),
    (2, 2, "fp4", 2, 300, 2, 2),
    (8, 4, "bf16", 2, 37, 3, "yarn"),    # the model's table (YaRN 16 over 65,536), positions near 1M
    (128, 128, "fp8", 2, 5, 0, "yarn"),
    (1, 1, "bf16", 2, 60, 1, "yarn"),
    (2, 2, "bf16", 3, 700, 2, "yarn"),   # CSA2 geometry: 2 tokens per entry, no overlap
    (2, 2, "fp8", 2, 1, 5, "yarn"),      # CSA2 decode-step entry, fp8
    (8, 4, "fp4", 2, 333, 0, 64),        # MXFP4 cache (32-channel power-of-two scales), run mode
    (2, 2, "fp4", 3, 700, 2, "yarn"),    # CSA2 geometry, fp4 (the V4.1-Flash cache)
    (2, 2, "fp4", 2, 1, 5, "yarn"),      # CSA2 decode-step entry, fp4 (split layout)
    (128, 128, "fp4", 2, 5, 0, "yarn"),  # HCA geometry, fp4
])
def test_compress_parity(window, stride, dtype, B, n_new, first, R):
    yarn = R == "yarn"
    if yarn:
        R = 64
    d = ci.Draw(100 + n_new + window, "cpu")
    T = (n_new - 1) * stride + window + 3
    kv = d.normal((B, T, 512))
    z = d.normal((B, T, 512))
    cap = first + n_new + 2
    pos0_list = [1 + 977 * b for b in range(B)]
    pos0_list[-1] = 1048576 - (first + n_new) * stride - window      # large angles
    pos0 = torch.tensor(pos0_list, dtype=torch.int64)
    sb = 32 if dtype == "fp4" else 64
    if dtype == "bf16":
        data = torch.full((B, cap, 512), 12345, dtype=torch.int16).view(torch.bfloat16)
        scales = None
    else:
        data = torch.full((B, cap, 256 if dtype == "fp4" else 512), 0xAA, dtype=torch.uint8)
        scales = torch.full((B, cap, 512 // sb), -1.0, dtype=torch.float32)
    dg = data.to(DEV)
    sg = scales.to(DEV) if scales is not None else None
    cache = ops.Cache(dg, torch.full((B,), cap, dtype=torch.int32, device=DEV), pos0.to(DEV), window, stride,
                      scales=sg, scale_block=sb if dtype != "bf16" else 0,
                      fmt=ops.CSA_FP4_E2M1 if dtype == "fp4" else None)
    fg, fo = inv_freq_pair(R, yarn) if R else (None, np.zeros(0))
    ops.compress(kv.to(DEV), z.to(DEV) if window > 1 else None, cache, first, n_new, fg, R)
    torch.cuda.synchronize()
    out = dg.cpu()
    for b in range(B):
        ent, _ = O.compress(np64(kv[b]), np64(z[b]), window, stride, pos0_list[b] + first * stride, fo)
        ref = ent[:n_new]
        bound = pool_error_bound(np64(kv[b]), np64(z[b]), window, stride, R)[:n_new]
        if dtype == "bf16":
            got = np64(out[b, first:first + n_new])
            check_bf16_rows(got, ref, bound, f"b={b}")
            untouched = torch.cat([out[b, :first], out[b, first + n_new:]]).view(torch.int16)
            assert torch.all(untouched == 12345)
        elif dtype == "fp4":
            check_fp4_rows(out[b, first:first + n_new].numpy(), sg.cpu()[b, first:first + n_new].numpy(), ref,
                           bound, f"b={b}")
            assert torch.all(out[b, :first] == 0xAA) and torch.all(out[b, first + n_new:] == 0xAA)
            assert torch.all(sg.cpu()[b, :first] == -1.0) and torch.all(sg.cpu()[b, first + n_new:] == -1.0)
        else:
            check_fp8_rows(out[b, first:first + n_new].numpy(), sg.cpu()[b, first:first + n_new].numpy(), ref,
                           bound, sb, f"b={b}")
            assert torch.all(out[b, :first] == 0xAA) and torch.all(out[b, first + n_new:] == 0xAA)


@pytest.mark.parametrize("window,stride,dtype,B,n_ent,n_win", [
    (8, 4, "bf16", 32, 1, 1),         # CSA decode step: one entry and one window row, one launch
    (128, 128, "bf16", 16, 1, 1),     # HCA decode step
    (8, 4, "fp8", 4, 1, 4),           # fp8 entries, four window rows
    (8, 4, "bf16", 1, 1024, 4096),    # prefill chunk: too many rows for one launch (a launch per call)
])
def test_compress_batch_equals_separate_calls(window, stride, dtype, B, n_ent, n_win):
    """csa_compress_batch writes exactly what the same csa_compress calls write one by one."""
    d = ci.Draw(700 + n_ent + window, "cpu")
    T = (n_ent - 1) * stride + window
    kv = d.normal((B, T, 512)).to(DEV)
    z = d.normal((B, T, 512)).to(DEV)
    new = kv[:, T - n_win:]
    pos0 = torch.tensor([5 + 1000 * b for b in range(B)], dtype=torch.int64, device=DEV)
    first_e, first_w = 3, 128
    cap_e, cap_w = first_e + n_ent + 1, first_w + n_win

    def caches():
        if dtype == "bf16":
            e = ops.Cache(torch.zeros((B, cap_e, 512), dtype=torch.bfloat16, device=DEV),
                          torch.full((B,), cap_e, dtype=torch.int32, device=DEV), pos0, window, stride)
        else:
            e = ops.Cache(torch.zeros((B, cap_e, 512), dtype=torch.uint8, device=DEV),
                          torch.full((B,), cap_e, dtype=torch.int32, device=DEV), pos0, window, stride,
                          scales=torch.zeros((B, cap_e, 8), dtype=torch.float32, device=DEV), scale_block=64)
        w = ops.Cache(torch.zeros((B, cap_w, 512), dtype=torch.bfloat16, device=DEV),
                      torch.full((B,), cap_w, dtype=torch.int32, device=DEV), pos0 + 7, 1, 1)
        return e, w

    fg, _ = inv_freq_pair(64)
    e1, w1 = caches()
    ops.compress(kv, z, e1, first_e, n_ent, fg, 64)
    ops.compress(new, None, w1, first_w, n_win, fg, 64)
    e2, w2 = caches()
    ops.compress_batch([(kv, z, e2, first_e, n_ent, fg, 64), (new, None, w2, first_w, n_win, fg, 64)])
    torch.cuda.synchronize()
    assert torch.equal(e1.data, e2.data) and torch.equal(w1.data, w2.data)
    if dtype == "fp8":
        assert torch.equal(e1.scales, e2.scales)
    assert torch.count_nonzero(w2.data[:, first_w:].view(torch.int16)) > 0


# ---------------------------------------------------------------- indexer + top-k

def _keys_cache(B, cap, fp8, seed, n_valid, pos0, window=8, stride=4):
    d = ci.Draw(seed, "cpu")
    if fp8:
        codes, sc = d.fp8_codes((B, cap, 128), 128, std=1 / math.sqrt(128))
        c = ops.Cache(codes.to(DEV), torch.tensor(n_valid, dtype=torch.int32, device=DEV),
                      torch.tensor(pos0, dtype=torch.int64, device=DEV), window, stride,
                      scales=sc.to(DEV), scale_block=128)
        ref = O.fp8_block_dequantize(codes.numpy(), sc.numpy(), 128)
    else:
        k = d.normal((B, cap, 128), std=1 / math.sqrt(128))
        c = ops.Cache(k.to(DEV), torch.tensor(n_valid, dtype=torch.int32, device=DEV),
                      torch.tensor(pos0, dtype=torch.int64, device=DEV), window, stride)
        ref = np64(k)
    return c, ref


@pytest.mark.parametrize("B,Tq,Hi,cap,n_valid,fp8,topk,qpos_of", [
    (1, 1, 8, 1023, [1023], False, 256, "end"),               # tiny decode shape
    (3, 1, 64, 3010, [3000, 2500, 10], True, 1024, "end"),     # ragged caches, one row with < k visible
    (2, 5, 16, 700, [700, 650], False, 100, "causal"),         # prefill rows: causal visibility
    (1, 2, 48, 1500, [1500], True, 1, "end"),                  # k = 1, Hi not a multiple of 64
    (2, 1, 64, 20000, [20000, 19999], True, 1024, "end"),      # spans many blocks; two-stage top-k
    (2, 1, 64, 70000, [70000, 500], True, 1024, "end"),        # two-stage, 5 chunks; one row with < k visible
    (1, 1, 4, 300000, [300000], True, 1024, "end"),            # 19 chunks: an intermediate merge stage, then the final one
    (1, 1, 4, 100000, [99000], False, 4096, "end"),            # k = 4,096: merge groups of 4 chunks, two stages
    (2, 8, 16, 70000, [70000, 65000], False, 1024, "causal"),   # bf16 keys, 560-block scores grid (4-deep ring)
    (2, 37, 64, 3000, [3000, 2100], False, 256, "causal"),     # multi-row kernel: ragged row groups, causal
    (1, 16, 40, 1300, [1290], False, 64, "causal"),            # multi-row kernel, heads not a multiple of 16
    (1, 1, 64, 140000, [140000], True, 512, "end"),            # CSA2 selection: top-512 of a long row (chunked)
    (1, 128, 4, 40000, [40000], True, 256, "end"),             # 128 rows, one block each: 48 entries per lane
    (1, 128, 4, 34000, [33900], True, 1024, "causal"),         # 128 rows, one block each: 36 entries per lane
    (1, 128, 4, 60000, [59000], False, 512, "end"),            # 128 rows, one block each: 64 entries per lane
    # a sequence's 2 or 4 query rows in one scores block (one key pass per sequence)
    (3, 4, 64, 20000, [20000, 19990, 7], True, 1024, "end"),   # 4 rows per block, fp8, two-stage, < k visible
    (2, 4, 64, 5000, [5000, 4000], False, 512, "causal"),      # 4 rows per block, bf16, different counts per row
    (2, 2, 24, 3000, [3000, 2999], True, 300, "causal"),       # 2 rows per block, heads not a multiple of 16
    (4, 4, 40, 70000, [70000, 69000, 30000, 900], False, 1024, "end"),  # 4 rows per block, bf16, 276-block grid (4-deep ring), two-stage
])
def test_index_topk_parity(B, Tq, Hi, cap, n_valid, fp8, topk, qpos_of):
    d = ci.Draw(200 + cap, "cpu")
    q_idx = d.normal((B, Tq, Hi, 128), std=1 / math.sqrt(128))
    w = d.uniform((B, Tq, Hi))
    pos0 = [1, 40][:B] + [1] * max(0, B - 2)
    keys, kref = _keys_cache(B, cap, fp8, 300 + cap, n_valid, pos0)
    ent_pos = [O.entry_positions(pos0[b], cap, 8, 4) for b in range(B)]
    if qpos_of == "end":
        qp = np.array([[ent_pos[b][n_valid[b] - 1] + t for t in range(Tq)] for b in range(B)])
    else:
        qp = np.array([[ent_pos[b][0] + (t * (cap * 4)) // Tq for t in range(Tq)] for b in range(B)])
    q_pos = torch.tensor(qp, dtype=torch.int64, device=DEV)
    idx = torch.empty((B, Tq, topk), dtype=torch.int32, device=DEV)
    scores = torch.empty((B, Tq, cap), dtype=torch.float32, device=DEV)
    ws = ops.workspace(ops.index_topk_workspace_bytes(B, Tq, Hi, cap, topk), DEV)
    ops.index_topk(q_idx.to(DEV), w.to(DEV), q_pos, keys, topk, idx, scores_out=scores, workspace=ws)
    torch.cuda.synchronize()
    sg, ig = scores.cpu().numpy(), idx.cpu().numpy()
    for b in range(B):
        for t in range(Tq):
            vis = O.visible_mask(ent_pos[b], qp[b, t]) & (np.arange(cap) < n_valid[b])
            so = O.index_scores(np64(q_idx[b, t]), np64(w[b, t]), kref[b])
            check_scores(sg[b, t], so, vis, f"b={b} t={t}", score_error_bound(np64(q_idx[b, t]), np64(w[b, t]), kref[b]))
            check_topk(ig[b, t], sg[b, t], so, vis, topk, f"b={b} t={t}")
    # scores in the workspace instead of scores_out gives the same selection
    idx2 = torch.empty_like(idx)
    ops.index_topk(q_idx.to(DEV), w.to(DEV), q_pos, keys, topk, idx2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2)


@pytest.mark.parametrize("cap", [5000, 50000])
def test_topk_all_scores_tied(cap):
    # zero indexer queries: every visible score is 0, so the k smallest indices win (with
    # cap 50000 the selection runs in two stages and the tie spans its chunks)
    B, topk = 2, 777
    nv = [cap, cap - 1000]
    keys, _ = _keys_cache(B, cap, False, 11, nv, [1, 1])
    q_idx = torch.zeros((B, 1, 64, 128), dtype=torch.bfloat16, device=DEV)
    w = torch.ones((B, 1, 64), dtype=torch.float32, device=DEV)
    q_pos = torch.tensor([[1 + 4 * (nv[0] - 1) + 7], [1 + 4 * (nv[1] - 1) + 7]], dtype=torch.int64, device=DEV)
    idx = torch.empty((B, 1, topk), dtype=torch.int32, device=DEV)
    ops.index_topk(q_idx, w, q_pos, keys, topk, idx, workspace=ops.workspace(
        ops.index_topk_workspace_bytes(B, 1, 64, cap, topk), DEV))
    torch.cuda.synchronize()
    for b in range(B):
        assert idx[b, 0].cpu().tolist() == list(range(topk))


def test_topk_clustered_scores():
    # scores crowded into ~3000 ulps of one binade, with many exact duplicates:
    # score = 1 + lo with lo = bf16(m * 2^-23), m < 3000 (exact in fp32)
    cap, topk = 30000, 1024
    m = np.random.default_rng(5).integers(0, 3000, size=cap)
    kt = torch.zeros((1, cap, 128), dtype=torch.bfloat16)
    kt[0, :, 0] = 1.0
    kt[0, :, 1] = torch.from_numpy(m * 2.0 ** -23).to(torch.bfloat16)
    keys = ops.Cache(kt.to(DEV), torch.tensor([cap], dtype=torch.int32, device=DEV),
                     torch.tensor([1], dtype=torch.int64, device=DEV), 8, 4)
    q_idx = torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16)
    q_idx[..., 0] = 1.0
    q_idx[..., 1] = 1.0
    w = torch.ones((1, 1, 1), dtype=torch.float32, device=DEV)
    q_pos = torch.tensor([[1 + 4 * (cap - 1) + 7]], dtype=torch.int64, device=DEV)
    idx = torch.empty((1, 1, topk), dtype=torch.int32, device=DEV)
    scores = torch.empty((1, 1, cap), dtype=torch.float32, device=DEV)
    ops.index_topk(q_idx.to(DEV), w, q_pos, keys, topk, idx, scores_out=scores,
                   workspace=ops.workspace(ops.index_topk_workspace_bytes(1, 1, 1, cap, topk), DEV))
    torch.cuda.synchronize()
    sg = scores[0, 0].cpu().numpy()
    ref = 1.0 + np64(kt[0, :, 1])
    np.testing.assert_array_equal(sg.astype(np.float64), ref)
    assert 100 < len(np.unique(sg)) < cap // 5
    exact = O.topk_select(ref, np.ones(cap, bool), topk)
    assert np.array_equal(idx[0, 0].cpu().numpy(), exact)


# ---------------------------------------------------------------- attention

def _attend_case(mode, B, Tq, H, cap, n_valid, kv_fp8, topk, W, win_cap, scale, qmul, seed, out_dtype="fp32",
                 win_start=None, kv_gain=None, pos_base=1, yarn=False, R=64):
    d = ci.Draw(seed, "cpu")
    q = d.normal((B, Tq, H, 512), std=qmul / math.sqrt(512))
    sink = d.normal((H,), dtype=torch.float32)
    if kv_fp8 == "fp4":
        # MXFP4 entries: code x power-of-two scale is exact in bf16, so staging adds no rounding
        packed, sc = d.fp4_codes((B, cap, 512), 32)
        kv = ops.Cache(packed.to(DEV), torch.tensor(n_valid, dtype=torch.int32, device=DEV), None, 8, 4,
                       scales=sc.to(DEV), scale_block=32, fmt=ops.CSA_FP4_E2M1)
        kv_ref = O.mxfp4_block_dequantize(O.fp4_unpack(packed.numpy()), sc.numpy(), 32)
    elif kv_fp8:
        codes, sc = d.fp8_codes((B, cap, 512), 64)
        kv = ops.Cache(codes.to(DEV), torch.tensor(n_valid, dtype=torch.int32, device=DEV), None, 8, 4,
                       scales=sc.to(DEV), scale_block=64)
        kv_ref = O.fp8_block_dequantize(codes.numpy(), sc.numpy(), 64)
    else:
        kvt = d.normal((B, cap, 512))
        if kv_gain is not None:
            kvt = (kvt.float() * torch.as_tensor(kv_gain, dtype=torch.float32)[None, :, None]).to(torch.bfloat16)
        kv = ops.Cache(kvt.to(DEV), torch.tensor(n_valid, dtype=torch.int32, device=DEV), None, 8, 4)
        kv_ref = np64(kvt)
    if mode == "hca":
        kv.window, kv.stride = 128, 128
    kv_pos0 = [pos_base + 1000 * b for b in range(B)]
    kv.pos0 = torch.tensor(kv_pos0, dtype=torch.int64, device=DEV)
    ent_pos = [O.entry_positions(kv_pos0[b], cap, kv.window, kv.stride) for b in range(B)]
    # query positions: the newest token sits right after the last valid entry (prefill rows step back)
    qp = np.array([[ent_pos[b][max(n_valid[b], 1) - 1] + 1 - (Tq - 1 - t) * 3 for t in range(Tq)]
                   for b in range(B)])
    wt = d.normal((B, win_cap, 512))
    wpos0 = [int(qp[b, -1]) - win_cap + 1 if win_start is None else win_start for b in range(B)]
    win = ops.Cache(wt.to(DEV), torch.tensor([win_cap] * B, dtype=torch.int32, device=DEV),
                    torch.tensor(wpos0, dtype=torch.int64, device=DEV), 1, 1)
    q_pos = torch.tensor(qp, dtype=torch.int64, device=DEV)
    fg, fo = inv_freq_pair(R, yarn) if R else (None, np.zeros(0))
    odt = torch.float32 if out_dtype == "fp32" else torch.bfloat16
    out = torch.empty((B, Tq, H, 512), dtype=odt, device=DEV)
    lse = torch.empty((B, Tq, H), dtype=torch.float32, device=DEV)
    idx = None
    if mode == "csa":
        rng = np.random.default_rng(seed)
        idx_np = np.full((B, Tq, topk), -1, dtype=np.int32)
        for b in range(B):
            for t in range(Tq):
                nvis = int((ent_pos[b][:n_valid[b]] <= qp[b, t]).sum())
                take = min(topk, nvis)
                idx_np[b, t, :take] = np.sort(rng.choice(nvis, size=take, replace=False))
        idx = torch.from_numpy(idx_np).to(DEV)
        ws = ops.workspace(ops.csa_attend_workspace_bytes(B, Tq, H, topk, W), DEV)
        ops.csa_attend(q.to(DEV), q_pos, kv, idx, win, W, sink.to(DEV), fg, R, scale, out, lse, ws)
    else:
        ws = ops.workspace(ops.hca_attend_workspace_bytes(B, Tq, H, cap, W), DEV)
        ops.hca_attend(q.to(DEV), q_pos, kv, win, W, sink.to(DEV), fg, R, scale, out, lse, ws)
    torch.cuda.synchronize()
    og, lg = np64(out), lse.cpu().numpy()
    worst = 0.0
    win_ref = np64(wt)
    for b in range(B):
        wpos = wpos0[b] + np.arange(win_cap)
        for t in range(Tq):
            if mode == "csa":
                X = oracle_rows_csa(kv_ref[b], idx.cpu().numpy()[b, t], win_ref[b], wpos, qp[b, t], W, n_valid[b])
            else:
                X = oracle_rows_hca(kv_ref[b][:n_valid[b]], ent_pos[b][:n_valid[b]], win_ref[b], wpos,
                                    qp[b, t], W)
            o, l = O.attend(np64(q[b, t]), qp[b, t], X, np64(sink), scale, fo)
            if out_dtype == "fp32":
                worst = max(worst, check_attention(og[b, t], o, f"b={b} t={t}"))
            check_lse(lg[b, t], l, lse_tolerance(np64(q[b, t]), qp[b, t], X, scale, fo), f"b={b} t={t}")
    print(f"    worst output error = {worst / ATT_TOL:.3f} of the bar", flush=True)
    return out, lse, worst


@pytest.mark.parametrize("mode,B,Tq,H,cap,n_valid,fp8,topk,W,win_cap,scale,qmul", [
    ("csa", 1, 1, 8, 1023, [1023], False, 256, 128, 129, 1 / math.sqrt(512), 1.0),   # tiny decode shape
    ("csa", 2, 1, 128, 3000, [3000, 2000], False, 1024, 128, 129, 1 / math.sqrt(512), 1.0),  # splits
    ("csa", 2, 1, 128, 3000, [3000, 2000], False, 1024, 128, 129, 1.0, 8.0),           # peaked softmax
    ("csa", 2, 3, 64, 900, [900, 40], True, 300, 128, 140, 1 / math.sqrt(512), 1.0),   # fp8 KV, < k visible
    ("csa", 1, 1, 16, 500, [500], False, 0, 128, 129, 1 / math.sqrt(512), 1.0),        # window only
    ("csa", 4, 64, 64, 600, [600] * 4, False, 200, 128, 200, 0.1, 2.0),               # 256 rows: no split
    # 512 rows x 128 heads: the 4-wave block shape (two blocks per CU, no split)
    ("csa", 4, 128, 128, 600, [600, 599, 400, 300], False, 200, 128, 256, 0.1, 2.0),
    ("hca", 2, 256, 128, 300, [300, 250], False, 0, 128, 384, 1 / math.sqrt(512), 1.0),
    ("csa", 4, 1, 64, 6000, [6000, 5000, 512, 100], True, 512, 128, 129, 1 / math.sqrt(512), 4.0),  # CSA2: top-512, fp8
    ("hca", 2, 1, 128, 700, [700, 300], False, 0, 128, 129, 1 / math.sqrt(512), 1.0),
    ("hca", 1, 2, 128, 64, [64], True, 0, 128, 129, 1 / math.sqrt(512), 4.0),        # fp8, sharper q
    # fp8 rows at a peaked softmax (scale 1, q x 8): the kernel stages the exact codes and applies
    # the per-64-channel scales in fp32, so no rounding of code x scale enters the logits
    ("csa", 2, 1, 64, 3000, [3000, 2000], True, 1024, 128, 129, 1.0, 8.0),
    ("hca", 2, 1, 128, 700, [700, 300], True, 0, 128, 129, 1.0, 8.0),
    ("csa", 3, 2, 128, 2500, [2500, 2400, 60], True, 1024, 128, 129, 1.0, 4.0),     # fp8, 128 heads, < k visible
    ("hca", 3, 1, 24, 300, [300, 299, 1], False, 0, 0, 1, 1 / math.sqrt(512), 1.0),   # no window, H < 32
    ("csa", 4, 1, 64, 6000, [6000, 5000, 512, 100], "fp4", 512, 128, 129, 1 / math.sqrt(512), 4.0),  # CSA2, fp4
    ("csa", 2, 3, 64, 900, [900, 40], "fp4", 300, 128, 140, 1 / math.sqrt(512), 1.0),  # fp4, < k visible
    ("hca", 2, 1, 128, 700, [700, 300], "fp4", 0, 128, 129, 1 / math.sqrt(512), 1.0),  # fp4, dense, splits
    # enough rows for the 64-head block shape with 16 splits (the small cases above take the
    # 32-head shape, whose grid is the larger one for them)
    ("csa", 8, 1, 128, 3000, [3000, 2999, 2500, 2000, 1500, 1200, 1100, 1000], False, 1024, 128, 129,
     1 / math.sqrt(512), 2.0),
    ("hca", 8, 1, 128, 2000, [2000, 1999, 1500, 1000, 800, 700, 600, 500], False, 0, 128, 129,
     1 / math.sqrt(512), 2.0),
    # the largest top-k the indexer returns (4,096): bf16 with 256 heads; fp8 over several splits
    # whose staged index lists stay within the per-split limit
    ("csa", 1, 1, 256, 6000, [6000], False, 4096, 128, 129, 1 / math.sqrt(512), 1.0),
    ("csa", 2, 1, 64, 6000, [6000, 5000], True, 4096, 128, 129, 1 / math.sqrt(512), 4.0),
    ("hca", 1, 2, 1024, 300, [300], False, 0, 128, 129, 1 / math.sqrt(512), 1.0),       # the largest head count
    ("csa", 1, 1, 1000, 2000, [2000], "fp4", 1024, 128, 129, 1 / math.sqrt(512), 1.0),  # heads not a multiple of 64
])
def test_attend_parity(mode, B, Tq, H, cap, n_valid, fp8, topk, W, win_cap, scale, qmul):
    _attend_case(mode, B, Tq, H, cap, n_valid, fp8, topk, W, win_cap, scale, qmul, seed=400 + cap + H)


@pytest.mark.parametrize("mode", ["csa", "hca"])
def test_attend_scores_far_above_first_tile(mode):
    """Rows of the first tile score ~100 log2 units below later rows (small-norm rows first,
    then large-norm rows), so the first tile's maximum is no usable softmax reference and
    the kernel must fall back to the split's exact maximum."""
    cap = 3000
    gain = np.where(np.arange(cap) < 400, 0.01, 3.0)
    topk = 1024 if mode == "csa" else 0
    _attend_case(mode, 1, 1, 128, cap, [cap], False, topk, 128, 129, 1.0, 8.0, seed=31, kv_gain=gain)


@pytest.mark.parametrize("mode,cap,n_valid,topk", [
    ("csa", 3000, [3000, 2500], 1024),
    ("hca", 300, [300, 280], 0),
])
def test_attend_parity_yarn_near_1m(mode, cap, n_valid, topk):
    """The model's rotary table (YaRN 16 over 65,536) and temperature, with queries near position 1,048,576."""
    scale = O.yarn_logit_scale(16.0) / math.sqrt(512)
    pos_base = 1048576 - cap * (4 if mode == "csa" else 128) - 2000
    _attend_case(mode, 2, 1, 128, cap, n_valid, False, topk, 128, 129, scale, 1.0, seed=61, pos_base=pos_base,
                 yarn=True)


@pytest.mark.parametrize("mode,B,Tq,H,cap,n_valid,fp8,topk,R", [
    ("csa", 2, 1, 128, 3000, [3000, 2000], False, 1024, 0),     # no rotation: the query is used as stored
    ("csa", 2, 1, 128, 3000, [3000, 2000], True, 1024, 2),      # one rotated pair
    ("csa", 2, 1, 128, 3000, [3000, 2000], False, 1024, 128),   # rotated dims below 448 (bf16 query part)
    ("csa", 4, 64, 64, 600, [600] * 4, False, 200, 512),        # every dim rotated, multi-row block
    ("csa", 4, 128, 128, 600, [600, 599, 400, 300], True, 200, 96),
    ("hca", 2, 1, 128, 700, [700, 300], False, 0, 0),
    ("hca", 2, 256, 128, 300, [300, 250], "fp4", 0, 256),
])
def test_attend_parity_rope_widths(mode, B, Tq, H, cap, n_valid, fp8, topk, R):
    """Rotated widths other than the model's 64: none, one pair, and wider ones whose
    rotated channels reach below 448 (the query part there is carried in bf16)."""
    _attend_case(mode, B, Tq, H, cap, n_valid, fp8, topk, 128, 129 if Tq == 1 else 256, 1 / math.sqrt(512),
                 2.0, seed=800 + R + Tq, R=R)


@pytest.mark.parametrize("fp8,margin", [
    (False, 1.0),     # grouped kernel: bf16 weights in P V (measured near 0.9 of the bar here)
    (True, 0.5),      # wave-pair kernel: fp32 weights as bf16 hi + lo (near 0.001)
    ("fp4", 0.5),     # near 0.002
])
def test_attend_flat_softmax_margin(fp8, margin):
    """A flat softmax over a few hundred rows (q x 2 at the default scale, 512 query rows x 128
    heads): the output averages away while each weight's rounding error does not, so this is
    where the weights' precision shows.  The wave-pair kernel must keep well inside the bar."""
    _, _, worst = _attend_case("csa", 4, 128, 128, 600, [600, 599, 400, 300], fp8, 200, 128, 256,
                               1 / math.sqrt(512), 2.0, seed=992, R=64)
    assert worst <= margin * ATT_TOL, f"worst output error {worst / ATT_TOL:.3f} of the bar (allowed {margin})"


def test_attend_window_cut_by_stream_start():
    # the window cache starts 40 tokens before the query: only 41 window rows exist
    _attend_case("csa", 2, 1, 64, 200, [10, 10], False, 8, 128, 41, 1 / math.sqrt(512), 1.0, seed=9)


def test_attend_bf16_output_and_determinism():
    args = ("csa", 2, 1, 128, 2000, [2000, 1800], False, 1024, 128, 129, 1 / math.sqrt(512), 1.0)
    o32, l32, _ = _attend_case(*args, seed=77)
    o32b, l32b, _ = _attend_case(*args, seed=77)
    assert torch.equal(o32, o32b) and torch.equal(l32, l32b)        # bitwise deterministic
    o16, _, _ = _attend_case(*args, seed=77, out_dtype="bf16")
    ref = o32.double()
    spacing = torch.ldexp(torch.ones_like(ref), torch.frexp(ref.abs())[1] - 8)
    assert torch.all((o16.double() - ref).abs() <= spacing)


def test_attend_workspace_reused_across_calls():
    # One workspace serves split calls of 4, then 2, then 4 query rows (different splits, so
    # different partial layouts): each output must equal that of a fresh workspace bit for bit,
    # whatever the previous call left there.
    B, H, cap, topk, W = 4, 128, 4000, 1024, 128
    d = ci.Draw(5, "cpu")
    q = d.normal((B, 1, H, 512), std=1 / math.sqrt(512)).to(DEV)
    sink = d.normal((H,), dtype=torch.float32).to(DEV)
    kv = ops.Cache(d.normal((B, cap, 512)).to(DEV), torch.full((B,), cap, dtype=torch.int32, device=DEV),
                   torch.zeros(B, dtype=torch.int64, device=DEV), 8, 4)
    qp = 4 * cap + 7
    win = ops.Cache(d.normal((B, W, 512)).to(DEV), torch.full((B,), W, dtype=torch.int32, device=DEV),
                    torch.full((B,), qp - W + 1, dtype=torch.int64, device=DEV), 1, 1)
    q_pos = torch.full((B, 1), qp, dtype=torch.int64, device=DEV)
    rng = np.random.default_rng(5)
    idx = torch.from_numpy(np.stack([np.sort(rng.choice(cap, topk, replace=False)) for _ in range(B)])
                           .astype(np.int32).reshape(B, 1, topk)).to(DEV)
    fg, _ = inv_freq_pair(64)
    scale = 1 / math.sqrt(512)

    def sub(c, n):
        return ops.Cache(c.data[:n], c.n_valid[:n], c.pos0[:n], c.window, c.stride)

    def call(n, ws):
        out = torch.empty((n, 1, H, 512), dtype=torch.float32, device=DEV)
        lse = torch.empty((n, 1, H), dtype=torch.float32, device=DEV)
        ops.csa_attend(q[:n], q_pos[:n], sub(kv, n), idx[:n], sub(win, n), W, sink, fg, 64, scale, out, lse, ws)
        return out, lse

    need = ops.csa_attend_workspace_bytes(B, 1, H, topk, W)
    assert need > 0 and ops.csa_attend_workspace_bytes(2, 1, H, topk, W) <= need
    shared = ops.workspace(need, DEV)
    for n in (B, 2, B):
        got = call(n, shared)
        ref = call(n, ops.workspace(ops.csa_attend_workspace_bytes(n, 1, H, topk, W), DEV))
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), f"{n} rows"


@pytest.mark.parametrize("mode", ["csa", "hca"])
def test_attend_same_row_across_split_plans(mode):
    """One query row attended alone and as each row of a 32-row batch of its copies.  The plans
    differ: alone, the row set is cut into many short splits of 32-head blocks (36 for CSA);
    in the batch, into a few long splits of 64-head blocks (4).  Both match the oracle, they agree
    with each other to the same bar, and the batch's copies are equal bit for bit."""
    B, H, W = 32, 128, 128
    csa = mode == "csa"
    cap, topk = (4000, 1024) if csa else (1200, 0)
    window, stride = (8, 4) if csa else (128, 128)
    d = ci.Draw(17, "cpu")
    q1 = d.normal((1, 1, H, 512), std=2 / math.sqrt(512))
    sink = d.normal((H,), dtype=torch.float32)
    kv1 = d.normal((1, cap, 512))
    win1 = d.normal((1, W, 512))
    qp = (cap - 1) * stride + window           # every entry visible (pos0 0)
    idx1 = None
    if csa:
        rng = np.random.default_rng(17)
        idx1 = torch.from_numpy(np.sort(rng.choice(cap, topk, replace=False)).astype(np.int32).reshape(1, 1, topk))
    fg, fo = inv_freq_pair(64)
    scale = 1 / math.sqrt(512)

    def call(n):
        rep = lambda x: x.expand(n, *x.shape[1:]).contiguous().to(DEV)
        kv = ops.Cache(rep(kv1), torch.full((n,), cap, dtype=torch.int32, device=DEV),
                       torch.zeros(n, dtype=torch.int64, device=DEV), window, stride)
        win = ops.Cache(rep(win1), torch.full((n,), W, dtype=torch.int32, device=DEV),
                        torch.full((n,), qp - W + 1, dtype=torch.int64, device=DEV), 1, 1)
        q_pos = torch.full((n, 1), qp, dtype=torch.int64, device=DEV)
        out = torch.empty((n, 1, H, 512), dtype=torch.float32, device=DEV)
        lse = torch.empty((n, 1, H), dtype=torch.float32, device=DEV)
        if csa:
            ws = ops.workspace(ops.csa_attend_workspace_bytes(n, 1, H, topk, W), DEV)
            ops.csa_attend(rep(q1), q_pos, kv, rep(idx1), win, W, sink.to(DEV), fg, 64, scale, out, lse, ws)
        else:
            ws = ops.workspace(ops.hca_attend_workspace_bytes(n, 1, H, cap, W), DEV)
            ops.hca_attend(rep(q1), q_pos, kv, win, W, sink.to(DEV), fg, 64, scale, out, lse, ws)
        torch.cuda.synchronize()
        return np64(out), lse.cpu().numpy()

    print(f"case {mode} one row vs {B} copies", flush=True)
    o1, l1 = call(1)
    oB, lB = call(B)
    for b in range(1, B):
        assert np.array_equal(oB[b], oB[0]) and np.array_equal(lB[b], lB[0]), f"copy {b} differs"
    wpos = qp - W + 1 + np.arange(W)
    if csa:
        X = oracle_rows_csa(np64(kv1[0]), idx1.numpy()[0, 0], np64(win1[0]), wpos, qp, W, cap)
    else:
        ent_pos = O.entry_positions(0, cap, window, stride)
        X = oracle_rows_hca(np64(kv1[0]), ent_pos, np64(win1[0]), wpos, qp, W)
    o_ora, l_ora = O.attend(np64(q1[0, 0]), qp, X, np64(sink), scale, fo)
    check_attention(o1[0, 0], o_ora, "one row")
    check_attention(oB[0, 0], o_ora, "batch row")
    # the plans round different weights to bf16 (each split has its own reference maximum), so
    # the two outputs are held to the oracle's bar between them; lse uses the exact fp32 sums
    rms = float(np.sqrt((o_ora ** 2).mean()))
    diff = float(np.abs(o1 - oB[:1]).max())
    assert diff <= ATT_TOL * rms, f"plans differ by {diff / rms:.2e} x RMS"
    assert float(np.abs(l1 - lB[:1]).max()) <= LSE_TOL


# ---------------------------------------------------------------- tiny decode from raw tokens

def test_tiny_csa_decode_end_to_end():
    """The tiny decode workload (4,096 raw tokens, 8 heads, top-256) through the whole path."""
    wl = ci.WORKLOADS["tiny_csa_decode"]
    inp = ci.decode_inputs(wl, "cpu")
    N, B = wl.N, wl.B
    E = wl.E
    fg, fo = inv_freq_pair(wl.R)
    kv, z = inp["kv"].to(DEV), inp["z"].to(DEV)
    one = lambda v, dt: torch.tensor([v], dtype=dt, device=DEV)
    cache = ops.Cache(torch.empty((B, E, 512), dtype=torch.bfloat16, device=DEV), one(E, torch.int32),
                      one(wl.pos0, torch.int64), 8, 4)
    ops.compress(kv, z, cache, 0, E, fg, wl.R)
    win = ops.Cache(torch.empty((B, wl.W, 512), dtype=torch.bfloat16, device=DEV), one(wl.W, torch.int32),
                    one(wl.pos0 + N - wl.W, torch.int64), 1, 1)
    ops.compress(kv[:, N - wl.W:], None, win, 0, wl.W, fg, wl.R)
    keys = ops.Cache(inp["k_idx"].to(DEV), one(E, torch.int32), one(wl.pos0, torch.int64), 8, 4)
    q_pos = torch.tensor([[wl.q_pos]], dtype=torch.int64, device=DEV)
    assert wl.q_pos == 4096
    idx = torch.empty((B, 1, wl.topk), dtype=torch.int32, device=DEV)
    scores = torch.empty((B, 1, E), dtype=torch.float32, device=DEV)
    ops.index_topk(inp["q_idx"].to(DEV), inp["w"].to(DEV), q_pos, keys, wl.topk, idx, scores_out=scores)
    out = torch.empty((B, 1, wl.H, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, 1, wl.H), dtype=torch.float32, device=DEV)
    ws = ops.workspace(ops.csa_attend_workspace_bytes(B, 1, wl.H, wl.topk, wl.W), DEV)
    scale = 1 / math.sqrt(512)
    ops.csa_attend(inp["q"].to(DEV), q_pos, cache, idx, win, wl.W, inp["sink"].to(DEV), fg, wl.R, scale, out, lse, ws)
    torch.cuda.synchronize()

    # oracle, from the same raw tokens
    kv64, z64 = np64(inp["kv"][0]), np64(inp["z"][0])
    ent, ep = O.compress(kv64, z64, 8, 4, wl.pos0, fo)
    assert ent.shape[0] == 1023
    got = np64(cache.data[0])
    check_bf16_rows(got, ent, pool_error_bound(kv64, z64, 8, 4, wl.R), "tiny entries")
    raw, rp = O.compress(kv64, z64, 1, 1, wl.pos0, fo)
    check_bf16_rows(np64(win.data[0]), raw[N - wl.W:],
                    pool_error_bound(kv64, z64, 1, 1, wl.R)[N - wl.W:], "tiny window")
    keys64 = np64(inp["k_idx"][0])
    so = O.index_scores(np64(inp["q_idx"][0, 0]), np64(inp["w"][0, 0]), keys64)
    vis = O.visible_mask(ep, wl.q_pos)
    assert vis.all()
    sg = scores[0, 0].cpu().numpy()
    check_scores(sg, so, vis, "tiny", score_error_bound(np64(inp["q_idx"][0, 0]), np64(inp["w"][0, 0]), keys64))
    ig = idx[0, 0].cpu().numpy()
    ndiff = check_topk(ig, sg, so, vis, wl.topk, "tiny")
    # attention on the GPU's selection and stored bytes
    X = oracle_rows_csa(got, ig, np64(win.data[0]), rp[N - wl.W:], wl.q_pos, wl.W, E)
    o, l = O.attend(np64(inp["q"][0, 0]), wl.q_pos, X, np64(inp["sink"]), scale, fo)
    check_attention(np64(out[0, 0]), o, "tiny on GPU selection")
    check_lse(lse[0, 0].cpu().numpy(), l, lse_tolerance(np64(inp["q"][0, 0]), wl.q_pos, X, scale, fo), "tiny")
    # and the all-oracle path (fp64 entries, oracle selection) when the selections agree
    if ndiff == 0:
        o2, _, sel, _, _ = O.csa_query(np64(inp["q"][0, 0]), wl.q_pos, np64(inp["q_idx"][0, 0]),
                                       np64(inp["w"][0, 0]), ent, ep, keys64, raw, rp, np64(inp["sink"]),
                                       wl.topk, scale, fo, wl.W)
        check_attention(np64(out[0, 0]), o2, "tiny end to end")
