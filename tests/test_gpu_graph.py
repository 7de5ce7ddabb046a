"""A captured step (pack + sparse up+down with the overflow path) replays to
the same bits as eager launches, replay after replay, with eager work and
synchronisations in between."""
import numpy as np
import pytest

import parity
from activation_sparse_feed_gate_amd import synth

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from activation_sparse_feed_gate_amd import tw

    w = synth.WORKLOADS["tiny"].with_(M=700, C=6, sigma_s=0.5, density=0.03)
    print(f"case {w}", flush=True)
    dev = parity.upload(synth.make_inputs(w))
    x, wg, wu, wd = dev["x"], dev["wg_t"], dev["wu_t"], dev["wd"]
    R_max = w.M
    bufs = tw.alloc_pack(w.M, w.N, w.T, w.C, R_max)
    ws = tw.workspace(w.M, w.K, w.N, w.T, w.C, R_max)
    y = torch.empty((w.M, w.K), dtype=torch.float32, device="cuda")

    def step():
        tw.tw_pack_gate(x, wg, w.T, w.C, bufs["tw_val"], bufs["tw_idx"], bufs["tw_cnt"],
                        bufs["ovf_rows"], bufs["ovf_count"], R_max, ws)
        tw.tw_sparse_ffn_fwd(x, wg, wu, wd, w.T, w.C, bufs["tw_val"], bufs["tw_idx"],
                             bufs["tw_cnt"], bufs["ovf_rows"], bufs["ovf_count"], R_max, y, ws)

    def snapshot():
        torch.cuda.synchronize()
        n = int(bufs["ovf_count"].cpu()[0])
        return (y.cpu().numpy().copy(), bufs["tw_cnt"].cpu().numpy().copy(),
                bufs["ovf_rows"].cpu().numpy()[:n].copy(), n)

    step()
    ref = snapshot()
    assert ref[3] > 0  # the overflow path is part of the captured work

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)

    for rep in range(4):
        y.fill_(float("nan"))
        bufs["tw_cnt"].fill_(-1)
        g.replay()
        got = snapshot()
        assert got[3] == ref[3], rep
        for a, b in zip(got[:3], ref[:3]):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), rep
        tw.ffn(x, wg, wu, wd)  # unrelated eager work between replays
        torch.cuda.synchronize()
