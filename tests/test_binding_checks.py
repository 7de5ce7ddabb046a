"""The Python binding checks every tensor's shape, dtype and device before
it calls the library (the C ABI sees bare pointers and cannot): a buffer of
the wrong size would otherwise be read or written out of bounds on the
device.  CPU tensors stand in for device ones; each case is rejected by the
binding before any pointer reaches the library."""
import pytest
import torch

BF, F32, I32, U8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8


@pytest.fixture(scope="module")
def tw():
    from activation_sparse_feed_gate_amd import tw as mod

    return mod


def e(*shape, dtype=F32):
    return torch.empty(shape, dtype=dtype)


M, K, N, T, C, R = 64, 256, 1024, 128, 16, 8
NT = N // T


def pack_args(**over):
    a = dict(x=e(M, K, dtype=BF), wg_t=e(N, K, dtype=BF), T=T, C=C,
             tw_val=e(M, NT, C), tw_idx=e(M, NT, C, dtype=I32), tw_cnt=e(M, NT, dtype=I32),
             ovf_rows=e(R, dtype=I32), ovf_count=e(1, dtype=I32), R_max=R, ws=e(16, dtype=U8))
    a.update(over)
    return a


@pytest.mark.parametrize("over,what", [
    (dict(tw_val=e(M, NT, C + 1)), "tw_val"),        # a packing made for another C
    (dict(tw_idx=e(M, NT // 2, C, dtype=I32)), "tw_idx"),  # ... for T = 256
    (dict(tw_cnt=e(M - 1, NT, dtype=I32)), "tw_cnt"),
    (dict(ovf_rows=e(R - 1, dtype=I32)), "ovf_rows"),  # shorter than R_max
    (dict(ovf_count=e(0, dtype=I32)), "ovf_count"),
    (dict(ovf_rows=None), "ovf_rows is required"),    # the list needs both or neither
    (dict(ovf_count=None), "ovf_count is required"),
    (dict(wg_t=e(N, K + 128, dtype=BF)), "wg_t"),
    (dict(tw_val=e(M, NT, C, dtype=torch.float64)), "tw_val"),
    (dict(tw_idx=e(M, NT, C, dtype=torch.int64)), "tw_idx"),
    (dict(x=e(M, K, dtype=F32)), "x"),
    (dict(T=100), "multiple of the tile width"),
    (dict(z_debug=e(M, N - 1)), "z_debug"),
    (dict(tw_val=torch.empty((M, NT, C), device="meta")), "is on meta"),
])
def test_pack_gate_rejects(tw, over, what):
    with pytest.raises((ValueError, TypeError), match=what):
        tw.tw_pack_gate(**pack_args(**over))


def test_pack_gate_valid_shapes_reach_the_device_check(tw):
    # every shape right: the only complaint left is that these are host tensors
    with pytest.raises(ValueError, match="device tensors"):
        tw.tw_pack_gate(**pack_args())
    # without an overflow list (both None) likewise
    with pytest.raises(ValueError, match="device tensors"):
        tw.tw_pack_gate(**pack_args(ovf_rows=None, ovf_count=None))


def sparse_args(**over):
    a = dict(x=e(M, K, dtype=BF), wg_t=e(N, K, dtype=BF), wu_t=e(N, K, dtype=BF),
             wd=e(N, K, dtype=BF), T=T, C=C, tw_val=e(M, NT, C), tw_idx=e(M, NT, C, dtype=I32),
             tw_cnt=e(M, NT, dtype=I32), ovf_rows=e(R, dtype=I32), ovf_count=e(1, dtype=I32),
             R_max=R, y=e(M, K), ws=e(16, dtype=U8))
    a.update(over)
    return a


@pytest.mark.parametrize("over,what", [
    (dict(wu_t=e(N - 128, K, dtype=BF)), "wu_t"),
    (dict(wd=e(K, N, dtype=BF)), "wd"),                # W_d given untransposed
    (dict(y=e(M, K, dtype=BF)), "y"),
    (dict(y=e(M + 1, K)), "y"),
    (dict(tw_val=e(M, NT, 4)), "tw_val"),
    (dict(ovf_rows=e(2, 4, dtype=I32)), "ovf_rows"),
])
def test_sparse_ffn_rejects(tw, over, what):
    with pytest.raises((ValueError, TypeError), match=what):
        tw.tw_sparse_ffn_fwd(**sparse_args(**over))


def test_dense_and_unfused_reject(tw):
    x, w = e(M, K, dtype=BF), e(N, K, dtype=BF)
    with pytest.raises(ValueError, match="y"):
        tw.tw_ffn_fwd(x, w, w, w, e(M, N), e(16, dtype=U8))
    with pytest.raises(ValueError, match="wd"):
        tw.tw_ffn_fwd(x, w, w, e(N, K + 128, dtype=BF), e(M, K), e(16, dtype=U8))
    with pytest.raises(ValueError, match="z"):
        tw.tw_gate_dense(x, w, e(M, N + 128))
    with pytest.raises(ValueError, match="tw_cnt"):
        tw.tw_pack_dense(e(M, N), T, C, e(M, NT, C), e(M, NT, C, dtype=I32),
                         e(M, NT + 1, dtype=I32), e(R, dtype=I32), e(1, dtype=I32), R,
                         e(16, dtype=U8))


P = 32
R1 = R


def hybrid_bufs(**over):
    b = dict(hy_g=e(M, P), hy_idx=e(M, P, dtype=I32), hy_cnt=e(M, dtype=I32),
             route=e(M, dtype=U8), bk_rows=e(R, dtype=I32), bk_count=e(1, dtype=I32),
             hy_u=e(M, P), hy_h=e(M, P), bk_g=e(R1, N, dtype=BF), bk_u=e(R1, N, dtype=BF),
             bk_h=e(R1, N, dtype=BF))
    b.update(over)
    return b


@pytest.mark.parametrize("over,what", [
    (dict(hy_idx=e(M, P + 1, dtype=I32)), "hy_idx"),   # storage made for another P
    (dict(route=e(M, dtype=I32)), "route"),
    (dict(bk_h=e(R1 - 1, N, dtype=BF)), "bk_h"),       # fewer rows than the backup room
    (dict(bk_u=e(R1, N, dtype=F32)), "bk_u"),
    (dict(hy_cnt=e(M, 1, dtype=I32)), "hy_cnt"),
])
def test_hybrid_up_rejects(tw, over, what):
    b = hybrid_bufs(**over)
    with pytest.raises((ValueError, TypeError), match=what):
        tw.tw_hybrid_up(e(M, K, dtype=BF), e(N, K, dtype=BF), e(N, K, dtype=BF), P, b["hy_g"],
                        b["hy_idx"], b["hy_cnt"], b["route"], b["bk_rows"], b["bk_count"], R,
                        b["hy_u"], b["hy_h"], b["bk_g"], b["bk_u"], b["bk_h"])


def test_hybrid_pack_and_down_reject(tw):
    b = hybrid_bufs()
    with pytest.raises(ValueError, match="tw_val"):
        tw.tw_hybrid_pack(T, C, e(M, NT, C - 1), e(M, NT, C, dtype=I32), e(M, NT, dtype=I32), P,
                          b["hy_g"], b["hy_idx"], b["hy_cnt"], b["route"], b["bk_rows"],
                          b["bk_count"], R)
    with pytest.raises(ValueError, match="y"):
        tw.tw_hybrid_down(e(N, K, dtype=BF), M, P, b["hy_h"], b["hy_idx"], b["hy_cnt"],
                          b["route"], b["bk_rows"], b["bk_count"], R, b["bk_h"], e(M, K + 1),
                          e(16, dtype=U8))
    with pytest.raises(ValueError, match="hy_h"):
        tw.tw_hybrid_down(e(N, K, dtype=BF), M + 1, P, b["hy_h"], b["hy_idx"], b["hy_cnt"],
                          b["route"], b["bk_rows"], b["bk_count"], R, b["bk_h"], e(M + 1, K),
                          e(16, dtype=U8))


def test_hybrid_backward_rejects(tw):
    b = hybrid_bufs()
    du, dz = e(M, P), e(M, P)
    bdu, bdz = e(R1, N, dtype=BF), e(R1, N, dtype=BF)
    with pytest.raises(ValueError, match="hy_dz"):
        tw.tw_hybrid_bwd_dh(e(M, K, dtype=BF), e(N, K, dtype=BF), P, 0.0, b["hy_g"], b["hy_u"],
                            b["hy_idx"], b["hy_cnt"], b["route"], b["bk_rows"], b["bk_count"], R,
                            b["bk_g"], b["bk_u"], du, e(M, P - 1), bdu, bdz)
    with pytest.raises(TypeError, match="dx"):
        tw.tw_hybrid_bwd_dx(e(N, K, dtype=BF), e(N, K, dtype=BF), M, P, du, dz, b["hy_idx"],
                            b["hy_cnt"], b["route"], b["bk_rows"], b["bk_count"], R, bdu, bdz,
                            e(M, K, dtype=BF), e(16, dtype=U8))
    with pytest.raises(ValueError, match="dwu_t"):
        tw.tw_hybrid_bwd_dw(e(M, K, dtype=BF), e(M, K, dtype=BF), P, b["hy_h"], du, dz,
                            b["hy_idx"], b["hy_cnt"], b["route"], b["bk_rows"], b["bk_count"], R,
                            b["bk_h"], bdu, bdz, e(N, K), e(N, K - 128), e(N, K),
                            e(16, dtype=U8))
