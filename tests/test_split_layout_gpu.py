"""GPU parity of the pages' alternative layout: the interaction writing only
the (B, P) dots (dlrm_emb_interact_dots) and the first top-MLP layer reading
cat(dense, dots) through a split A (linear_bias_act_split).  Against the
oracle, and bit for bit against the concatenated layout where the GEMM's k
order is the same (n > 8)."""
import numpy as np
import pytest

import oracle
from conftest import gpu_available
from gpu_helpers import assert_close, dev, host, make_uniform_case
from dlrm_embedding_bag_amd import abi, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

SPLIT_SHAPES = [  # (M, N, K_lo, K_hi)
    (1000, 512, 64, 351),    # the full forward's first top layer (dense | dots)
    (77, 40, 16, 6),         # ragged, aligned halves
    (33, 24, 7, 13),         # K_lo % 4 != 0: element-wise halves
    (130, 5, 64, 351),       # N <= 8: the matrix-vector kernel
    (9, 3, 5, 2),            # tiny, N <= 8, unaligned
    (300, 256, 128, 300),    # two full slabs then a tail
    (2048, 512, 64, 351),    # 64 x 64 tiles with k split over two wave groups
    (16402, 64, 8, 5),       # K <= 16 split: two row batches per wave, ragged
    (50, 40, 5, 6),          # K <= 16: the register-weight kernel
    (50, 40, 9, 7),          # K = 16, one row per wave
    (21, 12, 13, 1),         # K = 14, ragged
    (60, 2, 300, 400),       # N <= 8 past the register-staged row length
]


@pytest.mark.parametrize("act", ["none", "relu", "sigmoid"])
@pytest.mark.parametrize("M,N,K_lo,K_hi", SPLIT_SHAPES)
def test_linear_split_vs_oracle_and_concat(M, N, K_lo, K_hi, act):
    rng = np.random.default_rng(M + N + K_lo)
    a_lo = rng.standard_normal((M, K_lo)).astype(np.float32)
    a_hi = rng.standard_normal((M, K_hi)).astype(np.float32)
    w = (rng.standard_normal((N, K_lo + K_hi)) / np.sqrt(K_lo + K_hi)).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    cat = np.concatenate([a_lo, a_hi], axis=1)
    want = oracle.linear(cat, w, b, act)
    got = host(abi.linear_bias_act_split(dev(a_lo), dev(a_hi), dev(w), dev(b), act))
    assert_close(got, want, f"split {M}x{N}x({K_lo}+{K_hi})")
    if N > 8:
        same = host(abi.linear_bias_act(dev(cat), dev(w), dev(b), act))
        assert np.array_equal(got, same), "same k order as the concatenated matrix"


def test_linear_split_strided_halves():
    """The halves as column views of wider buffers (the dense part of R and
    a strided dots buffer)."""
    import torch
    rng = np.random.default_rng(2)
    M, N, K_lo, K_hi = 200, 64, 64, 351
    lo_buf = dev(rng.standard_normal((M, 416)).astype(np.float32))
    hi_buf = dev(rng.standard_normal((M, 360)).astype(np.float32))
    a_lo, a_hi = lo_buf[:, :K_lo], hi_buf[:, 5:5 + K_hi]
    w = dev((rng.standard_normal((N, K_lo + K_hi)) * 0.05).astype(np.float32))
    got = host(abi.linear_bias_act_split(a_lo, a_hi, w, None, "relu"))
    want = oracle.linear(np.concatenate([host(a_lo), host(a_hi)], axis=1), host(w), None, "relu")
    assert_close(got, want, "strided split")


@pytest.mark.parametrize("B,K,D,L", [(37, 5, 64, 7), (130, 26, 64, 20), (9, 8, 12, 3),
                                     (5, 3, 7, 2), (64, 32, 128, 4)])
def test_dots_only_vs_oracle(B, K, D, L):
    import torch
    w = inputs.Workload("dots", batch=B, num_tables=K, rows=300, dim=D, bag=L, dist="zipf")
    tables, idx, dense = make_uniform_case(w, seed=B)
    want = oracle.interact(dense, oracle.emb_bag_sum(tables, idx, batch=B))
    td, xd = [dev(t) for t in tables], [dev(i) for i in idx]
    P = (K + 1) * K // 2
    got = host(abi.dlrm_emb_interact_dots(td, xd, dev(dense)))
    assert got.shape == (B, P)
    assert_close(got, want[:, D:], "dots only")
    full = host(abi.dlrm_emb_interact(td, xd, dev(dense)))
    assert np.array_equal(got, full[:, D:]), "same dots as the [dense | dots] layout"
    # a strided destination: untouched padding columns
    buf = torch.full((B, P + 3), -7.0, device="cuda")
    abi.dlrm_emb_interact_dots(td, xd, dev(dense), out=buf[:, 1:P + 1])
    hb = host(buf)
    assert np.array_equal(hb[:, 1:P + 1], got)
    assert np.all(hb[:, 0] == -7.0) and np.all(hb[:, P + 1:] == -7.0)


def test_pages_layout_forward_equals_dlrm_forward():
    """The forward composed in the pages' layout -- bottom MLP, the (B, P) dots,
    a split-A first top layer, the rest of the top MLP -- equals dlrm_forward
    (which writes R = [dense | dots]) bit for bit when dlrm_forward runs the
    head as its own launch and splits no layer's k, and within the float bar
    with its default composition."""
    w = inputs.Workload("fwd-split", batch=1000, num_tables=26, rows=20000, dim=64, bag=20,
                        dist="zipf", dense_in=13, bottom=(512, 256, 64), top=(512, 256, 1))
    tables = [dev(inputs.table_host(w, k)) for k in range(w.num_tables)]
    idx = [dev(inputs.indices(w, k)) for k in range(w.num_tables)]
    dense = dev(inputs.dense(w))
    bottom, top = inputs.dlrm_layers(w, bias_std=0.1)
    bl = [(dev(a), dev(b), act) for a, b, act in bottom]
    tl = [(dev(a), dev(b), act) for a, b, act in top]
    model = abi.DlrmModel(bl, tl, tables, options=("unfused_head", "unsplit_k"))
    want = host(abi.dlrm_forward(model, dense, idx))
    fused = host(abi.dlrm_forward(abi.DlrmModel(bl, tl, tables), dense, idx))
    x = dense
    for wt, b, act in bl:
        x = abi.linear_bias_act(x, wt, b, act)
    dots = abi.dlrm_emb_interact_dots(tables, idx, x)
    wt, b, act = tl[0]
    y = abi.linear_bias_act_split(x, dots, wt, b, act)
    for wt, b, act in tl[1:]:
        y = abi.linear_bias_act(y, wt, b, act)
    assert np.array_equal(host(y), want)
    assert_close(fused, want, "fused head vs the pages' layout")
