"""A layer step captured in a HIP graph replays to the same bits as eager execution,
replay after replay, with eager work and synchronisations in between."""
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
    step.run()
    torch.cuda.synchronize()
    ref_out, ref_lse = step.out.clone(), step.lse.clone()
    ref_idx = step.idx.clone() if wl.mode == "csa" else None
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
        if ref_idx is not None:
            step.idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, ref_out), f"replay {rep}: output differs from eager"
        assert torch.equal(step.lse, ref_lse), f"replay {rep}: lse differs from eager"
        if ref_idx is not None:
            assert torch.equal(step.idx, ref_idx), f"replay {rep}: top-k differs from eager"
        step.run()                       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(step.out, ref_out)
