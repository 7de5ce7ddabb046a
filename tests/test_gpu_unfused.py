"""The unfused gate + pack path (tw_gate_dense, then tw_pack_dense) against
the fused tw_pack_gate and the CPU oracle.

The dense gate must be bitwise the fused kernel's own gate (the same
kernel and arithmetic), and its packing must be bit-exact both with the
fused packing and with the oracle packer applied to that gate.  The packed
form then drives the sparse path to the same y as the fused packing.
"""
import numpy as np
import pytest

import parity
from activation_sparse_feed_gate_amd import synth

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


@pytest.fixture(scope="module")
def tw():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from activation_sparse_feed_gate_amd import tw as mod

    return mod


def _host(p):
    import torch

    torch.cuda.synchronize()
    out = {k: p[k].cpu().numpy() for k in ("tw_val", "tw_idx", "tw_cnt", "ovf_rows")}
    out["ovf_count"] = int(p["ovf_count"].cpu()[0])
    if "z" in p:
        out["z"] = p["z"].cpu().numpy()
    return out


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict()),
    ("tiny", dict(C=4)),                                          # most rows overflow
    ("tiny", dict(M=300, K=384, N=1152, C=6, density=0.03, sigma_s=0.5)),  # half column block
    ("tiny", dict(M=513, K=512, N=2048, T=256, C=12, density=0.01, sigma_s=0.7, seed=3)),
    ("tiny", dict(M=1, K=128, N=128, C=3, density=0.1)),
    ("tiny", dict(density=1.0, C=128)),                           # every entry active
    # few rows: the gate's reduction split into K-slices over workgroups
    # (fused: partial tiles summed by a second pass; dense: summed in place)
    ("tiny", dict(M=8, K=1024, N=2048, T=256, C=8, density=0.01, sigma_s=0.5)),
    ("ffn-0.5b", dict()),                                         # the full 0.5B block
    ("ffn-2b", dict()),                                           # full 2B block, T = 256
    ("ffn-ovf", dict()),                                          # full overflow-stress block
])
def test_unfused_equals_fused(tw, name, kw):
    w = W[name].with_(**kw)
    print(f"case {w}", flush=True)
    d = synth.make_inputs(w)
    dev = parity.upload(d)
    R_max = w.M
    fused = _host(tw.pack_gate(dev["x"], dev["wg_t"], w.T, w.C, R_max, z_debug=True))
    unf = _host(tw.pack_unfused(dev["x"], dev["wg_t"], w.T, w.C, R_max))
    assert np.array_equal(unf["z"].view(np.uint32), fused["z"].view(np.uint32)), "gates differ"
    parity.check_packing_bitexact(unf, w.T, w.C, R_max)
    assert np.array_equal(unf["tw_cnt"], fused["tw_cnt"])
    used = np.arange(w.C)[None, None, :] < np.minimum(fused["tw_cnt"], w.C)[:, :, None]
    assert np.array_equal(np.where(used, unf["tw_idx"], -1), np.where(used, fused["tw_idx"], -1))
    assert np.array_equal(np.where(used, unf["tw_val"], 0).view(np.uint32),
                          np.where(used, fused["tw_val"], 0).view(np.uint32))
    assert unf["ovf_count"] == fused["ovf_count"]
    n = min(fused["ovf_count"], R_max)
    assert np.array_equal(unf["ovf_rows"][:n], fused["ovf_rows"][:n])


def test_unfused_drives_sparse_path(tw):
    """y from the unfused packing equals y from the fused packing bit for bit."""
    import torch

    w = W["tiny"].with_(M=700, C=6, density=0.03, sigma_s=0.5)
    print(f"case {w}", flush=True)
    dev = parity.upload(synth.make_inputs(w))
    args = (dev["x"], dev["wg_t"], dev["wu_t"], dev["wd"])
    y_f = tw.sparse_ffn(*args, tw.pack_gate(dev["x"], dev["wg_t"], w.T, w.C))
    y_u = tw.sparse_ffn(*args, tw.pack_unfused(dev["x"], dev["wg_t"], w.T, w.C))
    torch.cuda.synchronize()
    assert torch.equal(y_f.view(torch.int32), y_u.view(torch.int32))
