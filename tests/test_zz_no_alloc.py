"""tw_pack_gate_noalloc (the entry point that takes no workspace and works
on the library's static per-GPU scratch) against tw_pack_gate, through the
C ABI: the same counts, indices, values, overflow list and count, and the
same gate, bit for bit.  Calls run back to back, the second on a smaller
input, so the second finds the first one's contents in the scratch."""
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


def _pack(tw, dev, w, R_max, noalloc):
    import torch

    M, K = dev["x"].shape
    out = tw.alloc_pack(M, w.N, w.T, w.C, R_max)
    z = torch.empty((M, w.N), dtype=torch.float32, device="cuda")
    args = (dev["x"], dev["wg_t"], w.T, w.C, out["tw_val"], out["tw_idx"], out["tw_cnt"],
            out["ovf_rows"], out["ovf_count"], R_max)
    if noalloc:
        tw.tw_pack_gate_noalloc(*args, z_debug=z)
    else:
        ws = tw.workspace(M, K, w.N, w.T, w.C, R_max)
        tw.tw_pack_gate(*args, ws, z_debug=z)
    torch.cuda.synchronize()
    g = {k: out[k].cpu().numpy() for k in ("tw_val", "tw_idx", "tw_cnt", "ovf_rows")}
    g["ovf_count"] = int(out["ovf_count"].cpu()[0])
    g["z"] = z.cpu().numpy()
    return g


def _same(a, b, C, R_max):
    assert np.array_equal(a["z"].view(np.uint32), b["z"].view(np.uint32)), "gate differs"
    assert np.array_equal(a["tw_cnt"], b["tw_cnt"]), "counts differ"
    used = np.arange(C)[None, None, :] < np.minimum(a["tw_cnt"], C)[:, :, None]
    assert np.array_equal(np.where(used, a["tw_idx"], -1), np.where(used, b["tw_idx"], -1))
    assert np.array_equal(np.where(used, a["tw_val"], 0).view(np.uint32),
                          np.where(used, b["tw_val"], 0).view(np.uint32))
    assert a["ovf_count"] == b["ovf_count"]
    n = min(a["ovf_count"], R_max)
    assert np.array_equal(a["ovf_rows"][:n], b["ovf_rows"][:n])


# Each sequence: the workloads of consecutive calls, larger first.  M = 16
# and M = 1 at the 2B shape take the small-batch gate whose reduction is
# split over workgroups, so their partial gates live in the scratch too.
SEQUENCES = [
    [("ffn-0.5b", {}), ("ffn-2b", dict(M=16))],
    [("ffn-2b", dict(M=16)), ("ffn-2b", dict(M=1))],
    [("tiny", dict(M=700, C=6, density=0.03, sigma_s=0.5)), ("tiny", dict(M=300, C=6))],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "+".join(n for n, _ in s))
def test_noalloc_equals_pack_gate(tw, seq):
    for name, kw in seq:
        w = W[name].with_(**kw)
        R_max = max(w.M // 8, 1)
        print(f"case {w} R_max={R_max}", flush=True)
        dev = parity.upload(synth.make_inputs(w))
        got = _pack(tw, dev, w, R_max, noalloc=True)
        ref = _pack(tw, dev, w, R_max, noalloc=False)
        _same(got, ref, w.C, R_max)
        # the same call again right after: equal to itself, bit for bit
        again = _pack(tw, dev, w, R_max, noalloc=True)
        _same(again, got, w.C, R_max)
