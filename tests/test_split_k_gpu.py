"""GPU parity of the forward's partial sums across workgroups.  At batches
whose GEMM tiles would leave compute units idle, dlrm_forward cuts a layer's
k over several workgroups that store partial sums, and the next layer reads
their sum (in partial order), adds the bias and applies the activation as
it loads its A operand; a three-layer bottom MLP runs as one launch cut by
its hidden layer's columns (16- or 64-column slices), storing partials of
its output that the interaction adds as it loads the dense feature.  Checked against the CPU
oracle on sampled rows and against the composition without partials
(DLRM_FORWARD_UNSPLIT_K) within the float bar, over batches from 1 to past
the range where partials are taken, hidden activations other than ReLU,
layers without bias, widths that are not multiples of the tiles, plans,
the entry point without allocation, and NaN guard bands around the
output."""
import numpy as np
import pytest

import oracle
from conftest import gpu_available
from gpu_helpers import assert_close, dev, host, make_uniform_case
from dlrm_embedding_bag_amd import abi, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

FULL = ((512, 256, 64), (512, 256, 1))  # the full-size MLPs (D = 64)


def _case(B, K, D, bottom, top, seed, acts=None, no_bias=()):
    w = inputs.Workload("split", batch=B, num_tables=K, rows=3000, dim=D, bag=4, dist="zipf",
                        dense_in=13, bottom=bottom, top=top)
    tables, idx, dense = make_uniform_case(w, seed)
    bl, tl = inputs.dlrm_layers(w, seed, bias_std=0.1)
    if acts:
        bl = [(a, b, acts.get(("b", i), act)) for i, (a, b, act) in enumerate(bl)]
        tl = [(a, b, acts.get(("t", i), act)) for i, (a, b, act) in enumerate(tl)]
    bl = [(a, None if ("b", i) in no_bias else b, act) for i, (a, b, act) in enumerate(bl)]
    tl = [(a, None if ("t", i) in no_bias else b, act) for i, (a, b, act) in enumerate(tl)]
    return w, tables, idx, dense, bl, tl


def _model(tables, bl, tl, options=()):
    dv = [dev(t) for t in tables]
    b = [(dev(a), None if x is None else dev(x), act) for a, x, act in bl]
    t = [(dev(a), None if x is None else dev(x), act) for a, x, act in tl]
    return abi.DlrmModel(b, t, dv, options=options)


def _oracle_rows(w, dense, bl, tl, tables, idx, samples):
    want, _, _ = oracle.forward(dense[samples], bl, tl, tables,
                                [np.concatenate([i[s * w.bag:(s + 1) * w.bag] for s in samples])
                                 for i in idx])
    return want


@pytest.mark.parametrize("B", [1, 5, 100, 256, 1000, 2048, 3001, 4096, 6000])
def test_split_forward_full_model(B):
    """The full-size MLPs over batches on both sides of the split range."""
    w, tables, idx, dense, bl, tl = _case(B, 26, 64, *FULL, seed=B)
    d, x = dev(dense), [dev(i) for i in idx]
    split = _model(tables, bl, tl)
    plain = _model(tables, bl, tl, options=("unsplit_k",))
    got = host(abi.dlrm_forward(split, d, x))
    ref = host(abi.dlrm_forward(plain, d, x))
    assert got.shape == (B, 1)
    assert_close(got, ref, "split vs unsplit")
    samples = np.unique(np.linspace(0, B - 1, min(B, 96)).astype(int))
    assert_close(got[samples], _oracle_rows(w, dense, bl, tl, tables, idx, samples),
                 "split forward vs oracle")


def test_split_path_taken_at_small_batch():
    """At 256 samples the composition stores partials: its workspace holds
    more than one activation buffer's worth per hidden layer."""
    w, tables, idx, dense, bl, tl = _case(256, 26, 64, *FULL, seed=1)
    split = _model(tables, bl, tl)
    plain = _model(tables, bl, tl, options=("unsplit_k",))
    assert split.workspace_bytes(256) > plain.workspace_bytes(256)
    # at 8192 samples the tiles fill the chip and nothing is split
    assert split.workspace_bytes(8192) == plain.workspace_bytes(8192)


# (B, D, bottom widths, top widths, activations, layers without bias)
SHAPES = [
    (256, 64, (512, 256, 64), (512, 256, 1), {("b", 1): "sigmoid", ("t", 0): "none"}, ()),
    (300, 64, (512, 256, 64), (512, 256, 1), {}, (("b", 1), ("t", 0), ("t", 1))),
    (777, 32, (256, 192, 32), (384, 200, 1), {("t", 1): "sigmoid"}, ()),
    (1500, 16, (128, 64, 16), (256, 128, 3), {("b", 0): "none"}, (("b", 0),)),
    (64, 64, (512, 256, 128, 64), (512, 256, 128, 1), {}, ()),
    (500, 48, (640, 48), (320, 160, 2), {("b", 0): "sigmoid"}, ()),
    (200, 32, (128, 64, 32), (96, 48, 1), {("b", 2): "sigmoid"}, ()),
    (3000, 32, (128, 64, 32), (512, 48, 1), {("b", 2): "sigmoid"}, ()),  # one 64-wide slice
    (250, 32, (128, 512, 32), (512, 48, 1), {}, (("b", 2),)),  # 32 narrow slices
]


@pytest.mark.parametrize("B,D,bottom,top,acts,no_bias", SHAPES)
def test_split_forward_shapes(B, D, bottom, top, acts, no_bias):
    """Hidden sigmoid / identity activations and missing biases (applied by
    the reader of the partials), widths off the tile multiples, four-layer
    and two-layer bottom MLPs (no fused bottom launch), heads of 1-3 outputs."""
    K = 8
    w, tables, idx, dense, bl, tl = _case(B, K, D, bottom, top, seed=B + D, acts=acts,
                                          no_bias=no_bias)
    d, x = dev(dense), [dev(i) for i in idx]
    got = host(abi.dlrm_forward(_model(tables, bl, tl), d, x))
    ref = host(abi.dlrm_forward(_model(tables, bl, tl, options=("unsplit_k",)), d, x))
    assert_close(got, ref, "split vs unsplit")
    samples = np.unique(np.linspace(0, B - 1, min(B, 64)).astype(int))
    assert_close(got[samples], _oracle_rows(w, dense, bl, tl, tables, idx, samples),
                 "split forward vs oracle")


# Bottom MLPs (N0, 256, 32) for every hidden width N0 the slice kernels take
# (64 .. 512): at 250 samples the launch uses 16-column slices (16 bands x 16
# slices), at 1000 samples 64-column ones (63 bands x 4 slices).  The wide top
# MLP keeps the model above the one-launch forward's weight limit.
@pytest.mark.parametrize("B", [250, 1000])
@pytest.mark.parametrize("N0", [64, 128, 192, 256, 320, 448, 512])
def test_slice_kernels_every_width(B, N0):
    """Each slice-count instantiation of both slice kernels against the
    composition without partials and against the oracle."""
    K, D = 8, 32
    w, tables, idx, dense, bl, tl = _case(B, K, D, (N0, 256, D), (512, 256, 1), seed=N0 + B)
    d, x = dev(dense), [dev(i) for i in idx]
    got = host(abi.dlrm_forward(_model(tables, bl, tl), d, x))
    ref = host(abi.dlrm_forward(_model(tables, bl, tl, options=("unsplit_k",)), d, x))
    assert_close(got, ref, "slices vs unsplit")
    samples = np.unique(np.linspace(0, B - 1, 48).astype(int))
    assert_close(got[samples], _oracle_rows(w, dense, bl, tl, tables, idx, samples),
                 "slices vs oracle")


def test_split_forward_plans_noalloc_and_guards():
    """Plans (recorded launches and graph) and dlrm_forward_noalloc give the
    split forward's bits on every replay; the output's neighbours stay
    untouched."""
    import torch
    B = 256
    w, tables, idx, dense, bl, tl = _case(B, 26, 64, *FULL, seed=7)
    model = _model(tables, bl, tl)
    d, x = dev(dense), [dev(i) for i in idx]
    guard = 64
    big = torch.full((B + 2 * guard, 1), float("nan"), device="cuda")
    out = big[guard:guard + B]
    abi.dlrm_forward(model, d, x, out=out)
    eager = host(out).copy()
    g = host(big)
    assert np.all(np.isnan(g[:guard])) and np.all(np.isnan(g[guard + B:])), "guard bands"
    for mode in ("direct", "graph"):
        plan = abi.DlrmPlan(model, d, x, mode=mode)
        try:
            for _ in range(3):
                assert np.array_equal(host(plan.run()), eager), mode
                torch.cuda.synchronize()
        finally:
            plan.close()
    out2 = torch.empty((B, 1), device="cuda")
    assert np.array_equal(host(abi.dlrm_forward_noalloc(model, d, x, out2)), eager)
