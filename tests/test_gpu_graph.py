"""A captured step (pack + sparse up+down with the overflow path) replays to
the same bits as eager launches, replay after replay, with eager work and
synchronisations in between."""
import numpy as np
import pytest

import parity
from activation_sparse_feed_gate_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kw", [
    dict(M=700, C=6, sigma_s=0.5, density=0.03),  # one workgroup per row
    # 2B block: 48 rows (each over several workgroups, partial rows summed by
    # a second kernel) and 8 rows (the gate's reduction split into K-slices)
    dict(M=48, K=2048, N=8192, T=256, C=8, density=0.01, sigma_s=0.5, seed=21),
    dict(M=8, K=2048, N=8192, T=256, C=8, density=0.01, sigma_s=0.5, seed=22),
])
def test_graph_replay_matches_eager(kw):
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from activation_sparse_feed_gate_amd import tw

    w = synth.WORKLOADS["tiny"].with_(**kw)
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


def test_hybrid_graph_replay_matches_eager():
    """The training forward over hybrid storage (gate + TwELL, TwELL ->
    hybrid, up, down) captured once replays to the eager bits."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from activation_sparse_feed_gate_amd import tw

    w = synth.WORKLOADS["tiny"].with_(M=700, C=6, sigma_s=0.5, density=0.03)
    print(f"case {w}", flush=True)
    dev = parity.upload(synth.make_inputs(w))
    x, wg, wu, wd = dev["x"], dev["wg_t"], dev["wu_t"], dev["wd"]
    P, R_max = 32, w.M // 2
    bufs = tw.alloc_pack(w.M, w.N, w.T, w.C, w.M)
    ws = tw.workspace(w.M, w.K, w.N, w.T, w.C, w.M)
    hy = tw.alloc_hybrid(w.M, w.N, P, R_max, keep=True)
    wsh = torch.empty((tw.tw_hybrid_down_workspace_bytes(R_max),), dtype=torch.uint8,
                      device="cuda")
    y = torch.empty((w.M, w.K), dtype=torch.float32, device="cuda")

    def step():
        tw.tw_pack_gate(x, wg, w.T, w.C, bufs["tw_val"], bufs["tw_idx"], bufs["tw_cnt"],
                        bufs["ovf_rows"], bufs["ovf_count"], w.M, ws)
        tw.tw_hybrid_pack(w.T, w.C, bufs["tw_val"], bufs["tw_idx"], bufs["tw_cnt"], P,
                          hy["hy_g"], hy["hy_idx"], hy["hy_cnt"], hy["route"], hy["bk_rows"],
                          hy["bk_count"], R_max)
        tw.tw_hybrid_up(x, wg, wu, P, hy["hy_g"], hy["hy_idx"], hy["hy_cnt"], hy["route"],
                        hy["bk_rows"], hy["bk_count"], R_max, hy["hy_u"], hy["hy_h"],
                        hy["bk_g"], hy["bk_u"], hy["bk_h"])
        tw.tw_hybrid_down(wd, w.M, P, hy["hy_h"], hy["hy_idx"], hy["hy_cnt"], hy["route"],
                          hy["bk_rows"], hy["bk_count"], R_max, hy["bk_h"], y, wsh)

    def snapshot():
        torch.cuda.synchronize()
        n = int(hy["bk_count"].cpu()[0])
        return (y.cpu().numpy().copy(), hy["route"].cpu().numpy().copy(),
                hy["bk_rows"].cpu().numpy()[:n].copy(), hy["bk_h"][:n].cpu().view(torch.int16)
                .numpy().copy(), n)

    step()
    ref = snapshot()
    assert 0 < ref[4] <= R_max  # the backup path is part of the captured work

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)

    for rep in range(4):
        y.fill_(float("nan"))
        hy["route"].fill_(7)
        hy["bk_h"].fill_(0)
        g.replay()
        got = snapshot()
        assert got[4] == ref[4], rep
        for a, b in zip(got[:4], ref[:4]):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), rep
        tw.ffn(x, wg, wu, wd)  # unrelated eager work between replays
        torch.cuda.synchronize()
