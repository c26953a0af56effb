"""A layer step captured in a HIP graph replays to the same bits as eager execution,
replay after replay, with eager work and synchronisations in between.  The reference is
the step with its compress and index calls issued separately; the graph and the later eager
runs take the default path (for CSA, the combined compress + index call).  Before every
replay the rows the compressor writes are cleared, so the replay must rewrite them."""
import pytest
import torch

import csa_inputs as ci
from compressed_attention_long_amd.step import LayerStep

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_csa_decode", "v4pro_hca_decode_1m"])
def test_graph_replay_matches_eager(name):
    print(f"\n[gpu case] graph replay {name}", flush=True)
    wl = ci.WORKLOADS[name]
    t, meta = ci.step_tensors(wl, "cuda", seed=31)
    step = LayerStep(wl, t, meta, out_dtype=torch.float32)
    step.run(combined=False)
    torch.cuda.synchronize()
    ref_out, ref_lse = step.out.clone(), step.lse.clone()
    ref_idx = step.idx.clone() if wl.mode == "csa" else None
    e0, ne = meta["E_pre"], meta["n_new_entries"]
    w0, nw = meta["win_first_new"], meta["new_tok"]
    ref_kv = step.kv.data[:, e0:e0 + ne].clone()
    ref_win = step.win.data[:, w0:w0 + nw].clone()
    assert ne > 0 and torch.count_nonzero(ref_kv) > 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    for rep in range(4):
        step.out.zero_()
        step.lse.zero_()
        step.kv.data[:, e0:e0 + ne].zero_()
        step.win.data[:, w0:w0 + nw].zero_()
        if ref_idx is not None:
            step.idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.kv.data[:, e0:e0 + ne], ref_kv), f"replay {rep}: new entries differ"
        assert torch.equal(step.win.data[:, w0:w0 + nw], ref_win), f"replay {rep}: window rows differ"
        assert torch.equal(step.out, ref_out), f"replay {rep}: output differs from eager"
        assert torch.equal(step.lse, ref_lse), f"replay {rep}: lse differs from eager"
        if ref_idx is not None:
            assert torch.equal(step.idx, ref_idx), f"replay {rep}: top-k differs from eager"
        step.run()                       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(step.out, ref_out)
