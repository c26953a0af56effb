"""GPU parity at the page-shaped workload sizes, in the launch configuration the
benchmark times (one LayerStep: compress, window write, indexer + top-k, attend).

The oracle recomputes query rows one by one (every row of the decode batches, sampled rows
of the prefill chunk and the multi-token decode) from the same device tensors
(the step's inputs and the cache bytes the step wrote); bars: tests/gpu_common.py.
"""
import numpy as np
import pytest
import torch

import csa_inputs as ci
from compressed_attention_long_amd.step import LayerStep
from oracle import csa_oracle as O

from gpu_common import (check_attention, check_bf16_rows, check_fp4_rows, check_fp8_rows, check_lse, check_scores,
                        check_topk, lse_tolerance, np64, oracle_rows_csa, oracle_rows_hca, pool_error_bound,
                        score_error_bound, stored_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def oracle_table(wl):
    """The oracle's own rotary table for the workload (YaRN for the page-shaped workloads)."""
    if wl.yarn_factor > 1.0:
        return O.yarn_inv_freq(160000.0, wl.R, wl.yarn_factor, wl.yarn_base_len)
    return O.rope_inv_freq(160000.0, wl.R)


def oracle_scale(wl):
    """The oracle's softmax scale: 1/sqrt(512), times the YaRN temperature for YaRN workloads."""
    return O.yarn_logit_scale(wl.yarn_factor) / np.sqrt(wl.D) if wl.yarn_factor > 1.0 else 1 / np.sqrt(wl.D)


def run_step(name):
    wl = ci.WORKLOADS[name]
    print(f"\n[gpu case] full-size step {name}", flush=True)
    t, meta = ci.step_tensors(wl, DEV)
    step = LayerStep(wl, t, meta, out_dtype=torch.float32)
    step.run()
    torch.cuda.synchronize()
    return wl, t, meta, step


def check_rows(wl, t, meta, step, samples):
    fo = oracle_table(wl)
    kv_block = wl.kv_scale_block
    ent_pos_all = O.entry_positions(wl.pos0, wl.E, wl.window, wl.stride)
    win_pos = int(t["win_pos0"][0]) + np.arange(meta["win_cap"])
    sink = np64(t["sink"])
    cached_b, keys, kv_rows = None, None, None
    for b, tq in samples:
        qp = int(t["q_pos"][b, tq])
        win_rows = np64(step.win.data[b])
        sc_b = step.kv.scales[b] if step.kv.scales is not None else None
        if b != cached_b:            # one sequence's stored rows, converted once for its query rows
            cached_b = b
            if wl.mode == "csa":
                ks = t.get("k_idx_scale")
                keys = stored_rows(t["k_idx"][b], ks[b] if ks is not None else None, wl.Di)
            else:
                kv_rows = stored_rows(step.kv.data[b], sc_b, kv_block, wl.kv_dtype)
        if wl.mode == "csa":
            qi, wi = np64(t["q_idx"][b, tq]), np64(t["w"][b, tq])
            so = O.index_scores(qi, wi, keys)
            vis = O.visible_mask(ent_pos_all, qp)
            sg = step.scores[b, tq].cpu().numpy()
            check_scores(sg, so, vis, f"{wl.name} b={b} t={tq}", score_error_bound(qi, wi, keys))
            ig = step.idx[b, tq].cpu().numpy()
            check_topk(ig, sg, so, vis, wl.topk, f"{wl.name} b={b} t={tq}")
            sel = torch.from_numpy(ig[ig >= 0].astype(np.int64)).to(DEV)
            kv_sel = stored_rows(step.kv.data[b][sel], sc_b[sel] if sc_b is not None else None, kv_block,
                                 wl.kv_dtype)
            X = oracle_rows_csa(kv_sel, np.arange(len(sel)), win_rows, win_pos, qp, wl.W, len(sel))
        else:
            X = oracle_rows_hca(kv_rows, ent_pos_all, win_rows, win_pos, qp, wl.W)
        q64 = np64(t["q"][b, tq])
        o, l = O.attend(q64, qp, X, sink, oracle_scale(wl), fo)
        check_attention(np64(step.out[b, tq]), o, f"{wl.name} b={b} t={tq}")
        check_lse(step.lse[b, tq].cpu().numpy(), l, lse_tolerance(q64, qp, X, oracle_scale(wl), fo),
                  f"{wl.name} b={b} t={tq}")


def check_new_entry(wl, t, meta, step, b):
    """The entries this step compressed, against the oracle on the same raw rows."""
    fo = oracle_table(wl)
    first = meta["E_pre"]
    n = meta["n_new_entries"]
    ent, _ = O.compress(np64(t["kv_raw"][b]), np64(t["z_raw"][b]), wl.window, wl.stride,
                        wl.pos0 + first * wl.stride, fo)
    bound = pool_error_bound(np64(t["kv_raw"][b]), np64(t["z_raw"][b]), wl.window, wl.stride, wl.R)[:n]
    what = f"{wl.name} new entries b={b}"
    if wl.kv_dtype == "fp4":
        check_fp4_rows(step.kv.data[b, first:first + n].cpu().numpy(),
                       step.kv.scales[b, first:first + n].cpu().numpy(), ent[:n], bound, what)
    elif wl.kv_dtype == "fp8":
        check_fp8_rows(step.kv.data[b, first:first + n].cpu().numpy(),
                       step.kv.scales[b, first:first + n].cpu().numpy(), ent[:n], bound, wl.kv_scale_block, what)
    else:
        check_bf16_rows(np64(step.kv.data[b, first:first + n]), ent[:n], bound, what)


def every_row(wl):
    return [(b, t) for b in range(wl.B) for t in range(wl.Tq)]


def test_v4pro_csa_decode_65k():
    """Every query row of the batch, and every sequence's new entry."""
    wl, t, meta, step = run_step("v4pro_csa_decode_65k")
    for b in range(wl.B):
        check_new_entry(wl, t, meta, step, b)
    check_rows(wl, t, meta, step, every_row(wl))


def test_v4pro_hca_decode_1m():
    wl, t, meta, step = run_step("v4pro_hca_decode_1m")
    for b in range(wl.B):
        check_new_entry(wl, t, meta, step, b)
    check_rows(wl, t, meta, step, every_row(wl))


def test_v4flash_csa_decode_1m_fp8():
    wl, t, meta, step = run_step("v4flash_csa_decode_1m_fp8")
    for b in range(wl.B):
        check_new_entry(wl, t, meta, step, b)
    check_rows(wl, t, meta, step, every_row(wl))


def test_v4flash_csa_decode_1m_fp8_peaked_queries():
    """The Flash fp8 decode with queries scaled by 4 (a sharper softmax over the fp8 cache; the
    scaling is exact in bf16): attention over the same selection and stored bytes."""
    wl, t, meta, step = run_step("v4flash_csa_decode_1m_fp8")
    t["q"].mul_(4.0)
    step.attend()
    torch.cuda.synchronize()
    check_rows(wl, t, meta, step, every_row(wl))


def test_v4pro_csa_prefill_4k_on_131k():
    wl, t, meta, step = run_step("v4pro_csa_prefill_4k_on_131k")
    check_new_entry(wl, t, meta, step, 0)
    check_rows(wl, t, meta, step, [(0, 0), (0, 1), (0, 2047), (0, 4095)])


def test_v4pro_csa_decode_65k_mtp4():
    """Four query tokens per sequence (draft verification): each sees entries and window rows
    up to its own position only."""
    wl, t, meta, step = run_step("v4pro_csa_decode_65k_mtp4")
    check_new_entry(wl, t, meta, step, 9)
    check_rows(wl, t, meta, step, [(0, 0), (0, 3), (21, 1), (31, 2)])


def test_v41flash_csa2_decode_1m_fp4_with_reuse():
    """CSA2 at 1M: entries pool 2 tokens, top-512 of 524,288, MXFP4 KV; then a reuse layer (its own
    queries and sink over the computed layer's KV and selection)."""
    from compressed_attention_long_amd.step import ReuseStep
    wl, t, meta, step = run_step("v41flash_csa2_decode_1m_fp4")
    check_rows(wl, t, meta, step, [(0, 0), (3, 0)])
    check_new_entry(wl, t, meta, step, 1)
    r = ci.reuse_tensors(wl, DEV)
    rs = ReuseStep(step, r["q"], r["sink"], out_dtype=torch.float32)
    rs.run()
    torch.cuda.synchronize()
    fo = oracle_table(wl)
    win_pos = int(t["win_pos0"][0]) + np.arange(meta["win_cap"])
    for b in (0, 2):
        qp = int(t["q_pos"][b, 0])
        ig = step.idx[b, 0].cpu().numpy()
        sel = torch.from_numpy(ig[ig >= 0].astype(np.int64)).to(DEV)
        kv_sel = stored_rows(step.kv.data[b][sel], step.kv.scales[b][sel], wl.kv_scale_block, wl.kv_dtype)
        X = oracle_rows_csa(kv_sel, np.arange(len(sel)), np64(step.win.data[b]), win_pos, qp, wl.W, len(sel))
        o, l = O.attend(np64(r["q"][b, 0]), qp, X, np64(r["sink"]), oracle_scale(wl), fo)
        check_attention(np64(rs.out[b, 0]), o, f"reuse layer b={b}")
        check_lse(rs.lse[b, 0].cpu().numpy(), l, lse_tolerance(np64(r["q"][b, 0]), qp, X, oracle_scale(wl), fo),
                  f"reuse layer b={b}")


@pytest.mark.parametrize("name", ["v4pro_csa_decode_65k", "v41flash_csa2_decode_1m_fp4", "v4pro_csa_decode_65k_mtp4",
                                  "v4pro_csa_prefill_4k_on_131k"])
def test_combined_compress_index_call_equals_separate_calls(name):
    """csa_index_topk_compress writes bit for bit what csa_compress_batch + csa_index_topk write:
    the compress blocks riding in the scores launch (decode), or the separate launches it falls
    back to (the prefill chunk: many-row compress and the many-query-row scores kernel)."""
    wl = ci.WORKLOADS[name]
    print(f"\n[gpu case] combined call {name}", flush=True)
    t, meta = ci.step_tensors(wl, DEV)
    step = LayerStep(wl, t, meta, out_dtype=torch.float32)
    e0, ne = meta["E_pre"], meta["n_new_entries"]
    w0, nw = meta["win_first_new"], meta["new_tok"]

    def clear():
        step.kv.data[:, e0:e0 + ne].zero_()
        if step.kv.scales is not None:
            step.kv.scales[:, e0:e0 + ne].zero_()
        step.win.data[:, w0:w0 + nw].zero_()
        step.idx.fill_(-7)
        step.scores.zero_()
        torch.cuda.synchronize()

    def state():
        s = [step.kv.data[:, e0:e0 + ne].clone(), step.win.data[:, w0:w0 + nw].clone(), step.idx.clone(),
             step.scores.clone()]
        if step.kv.scales is not None:
            s.append(step.kv.scales[:, e0:e0 + ne].clone())
        return s

    clear()
    step.compress()
    step.index()
    torch.cuda.synchronize()
    ref = state()
    clear()
    step.index_compress()
    torch.cuda.synchronize()
    got = state()
    for i, (x, y) in enumerate(zip(got, ref)):
        assert torch.equal(x, y), f"{name}: output {i} differs between the combined and the separate calls"
    assert torch.count_nonzero(ref[0]) > 0
