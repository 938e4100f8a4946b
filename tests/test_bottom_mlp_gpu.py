"""GPU parity of the fused bottom MLP (three linear + bias + activation
layers in one launch, the hidden activations kept on chip), taken by
mlp_forward for a three-layer stack with 4 <= K0 <= 15, N0 a multiple of 64,
N1 <= 256 and N2 <= 64 multiples of 16 at any row count, and by dlrm_forward
for such a stack at 7,137..8,192 rows.  Checked against the CPU oracle (layer by layer, fp64) on sampled rows
and against the layer-by-layer launches within the float bar, over ragged
row counts, odd K0, strided operands, missing biases and every activation."""
import numpy as np
import pytest

import oracle
from conftest import gpu_available
from gpu_helpers import assert_close, dev, host, make_uniform_case
from dlrm_embedding_bag_amd import abi, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _layers(rng, widths, acts, bias=True):
    out = []
    for i, act in enumerate(acts):
        k, n = widths[i], widths[i + 1]
        bound = np.sqrt(6.0 / (k + n))
        w = rng.uniform(-bound, bound, (n, k)).astype(np.float32)
        b = (rng.standard_normal(n) * 0.1).astype(np.float32) if bias else None
        out.append((w, b, act))
    return out


def _oracle_rows(a, layers, rows):
    x = a[rows]
    for w, b, act in layers:
        x = oracle.linear(x, w, b, act)
    return x


STACKS = [  # (M, widths, acts)
    (8192, (13, 512, 256, 64), ("relu", "relu", "relu")),
    (300, (13, 512, 256, 64), ("relu", "relu", "relu")),
    (1, (13, 512, 256, 64), ("relu", "none", "relu")),
    (7137, (13, 512, 256, 64), ("relu", "relu", "relu")),
    (9001, (7, 128, 64, 16), ("relu", "none", "sigmoid")),
    (8200, (15, 192, 256, 32), ("sigmoid", "relu", "none")),
    (16385, (4, 64 * 3, 16, 48), ("none", "relu", "relu")),
]


@pytest.mark.parametrize("M,widths,acts", STACKS)
def test_fused_bottom_mlp_vs_oracle(M, widths, acts):
    rng = np.random.default_rng(M + widths[0])
    a = rng.standard_normal((M, widths[0])).astype(np.float32)
    layers = _layers(rng, widths, acts)
    dl = [(dev(w), dev(b), act) for w, b, act in layers]
    got = host(abi.mlp_forward(dev(a), dl))
    rows = np.unique(np.concatenate([np.arange(0, min(40, M)), np.arange(max(0, M - 40), M),
                                     rng.choice(M, min(200, M), replace=False)]))
    assert_close(got[rows], _oracle_rows(a, layers, rows), f"fused bottom {widths}")
    x = dev(a)
    for w, b, act in dl:
        x = abi.linear_bias_act(x, w, b, act)
    assert_close(got, host(x), f"fused bottom vs layer launches {widths}")


def test_fused_bottom_mlp_strided_and_no_bias():
    import torch
    rng = np.random.default_rng(5)
    M = 8192
    abuf = dev(rng.standard_normal((M, 17)).astype(np.float32))
    a = abuf[:, :13]
    layers = _layers(rng, (13, 512, 256, 64), ("relu", "relu", "relu"), bias=False)
    cbuf = torch.full((M, 72), -3.0, device="cuda")
    c = cbuf[:, :64]
    abi.mlp_forward(a, [(dev(w), None, act) for w, b, act in layers], out=c)
    rows = np.arange(0, M, 41)
    assert_close(host(c)[rows], _oracle_rows(host(a), layers, rows), "strided, no bias")
    assert np.all(host(cbuf)[:, 64:] == -3.0), "columns beyond N2 must be untouched"
    # an output row stride that is no multiple of 4: the scalar store path
    cbuf2 = torch.full((M * 65 + 1,), -3.0, device="cuda")
    c2 = cbuf2[1:].view(M, 65)[:, :64]
    abi.mlp_forward(a, [(dev(w), None, act) for w, b, act in layers], out=c2)
    assert np.array_equal(host(c2), host(c))
    assert host(cbuf2)[0] == -3.0 and np.all(host(cbuf2)[1:].reshape(M, 65)[:, 64] == -3.0)


@pytest.mark.parametrize("B", [8192, 7137, 7136, 8193])
def test_forward_with_fused_bottom(B):
    """dlrm_forward takes the fused bottom MLP at 7,137..8,192 samples; the same
    forward with each bottom layer as its own launch agrees within the float
    bar, and both match the oracle on sampled rows."""
    w = inputs.Workload("fb", batch=B, num_tables=26, rows=2000, dim=64, bag=4, dist="zipf",
                        dense_in=13, bottom=(512, 256, 64), top=(512, 256, 1))
    tables, idx, dense = make_uniform_case(w, seed=B)
    bl, tl = inputs.dlrm_layers(w, B, bias_std=0.1)
    dt = [dev(t) for t in tables]
    b = [(dev(a), dev(x), act) for a, x, act in bl]
    t = [(dev(a), dev(x), act) for a, x, act in tl]
    d, xi = dev(dense), [dev(i) for i in idx]
    got = host(abi.dlrm_forward(abi.DlrmModel(b, t, dt), d, xi))
    ref = host(abi.dlrm_forward(abi.DlrmModel(b, t, dt, options=("unfused_bottom",)), d, xi))
    assert_close(got, ref, "fused bottom vs layer launches")
    samples = np.arange(0, B, 97)
    want, _, _ = oracle.forward(dense[samples], bl, tl, tables,
                                [np.concatenate([i[s * w.bag:(s + 1) * w.bag] for s in samples])
                                 for i in idx])
    assert_close(got[samples], want, "forward with fused bottom vs oracle")
