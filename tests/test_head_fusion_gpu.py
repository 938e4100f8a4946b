"""GPU parity of the fused sigmoid head: dlrm_forward folds a one-output last
top layer into the epilogue of the layer before it (that layer's
activations are never stored) when tiles that own whole rows give about
one 32-row band per CU; at other batches the head is a launch of its own,
reading the layer before's k partials.  Checked against the CPU oracle and
against the unfused composition (DLRM_FORWARD_UNFUSED_HEAD) within the
float bar, over batches that leave the last tile partly empty, penultimate
widths below or between tile widths, K not a multiple of 4, every head
activation, and repeated calls on one workspace, in plans and without
allocation."""
import numpy as np
import pytest

import oracle
from conftest import gpu_available
from gpu_helpers import assert_close, dev, host, make_uniform_case
from dlrm_embedding_bag_amd import abi, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _case(B, K, D, top, seed, bottom=(64,), head_act="sigmoid"):
    w = inputs.Workload("head", batch=B, num_tables=K, rows=500, dim=D, bag=5, dist="zipf",
                        dense_in=13, bottom=bottom + (D,), top=top)
    tables, idx, dense = make_uniform_case(w, seed)
    bl, tl = inputs.dlrm_layers(w, seed, bias_std=0.1)
    tl[-1] = (tl[-1][0], tl[-1][1], head_act)
    return w, tables, idx, dense, bl, tl


def _models(tables, bl, tl):
    """The model with the head folded and with it unfused, both layered (the
    smaller models here would otherwise run as one launch)."""
    dv = [dev(t) for t in tables]
    b = [(dev(a), dev(x), act) for a, x, act in bl]
    t = [(dev(a), dev(x), act) for a, x, act in tl]
    return (abi.DlrmModel(b, t, dv, options=("layered",)),
            abi.DlrmModel(b, t, dv, options=("layered", "unfused_head")))


# (B, K, D, top widths) -- the full-size top MLP 415-512-256-1 and narrower ones;
# the whole-row launch is taken at 7,137..8,192 samples, other batches check
# that the composition falls back to two launches
CASES = [(8192, 26, 64, (512, 256, 1)), (7201, 4, 16, (64, 7, 1)), (7137, 3, 16, (40, 24, 1)),
         (9000, 8, 64, (512, 200, 1)), (8192, 5, 12, (130, 1)), (16385, 2, 8, (256, 1)),
         (1, 26, 64, (512, 256, 1)), (1000, 26, 64, (512, 256, 1)), (7136, 3, 16, (40, 24, 1))]
# the head launched on its own after a penultimate layer whose k is split
# in 8 (256 samples), 4 (333) and 2 (1000 above, 1536) or not (2049, 4096,
# 16384), on 64 x 32, 64 x 64 and 128-row tiles (at 1536 the bottom MLP is
# one launch of 384 slice workgroups); a penultimate width that leaves the
# last column tile partly empty (202), one column tile (32), and the top
# MLP's first layer as the penultimate one (reading R at K = 92 and K = 74)
SMALL_CASES = [(256, 26, 64, (512, 256, 1)), (333, 26, 64, (512, 256, 1)),
               (1536, 26, 64, (512, 256, 1)),
               (2049, 26, 64, (512, 256, 1)), (4096, 26, 64, (512, 256, 1)),
               (16384, 26, 64, (512, 256, 1)), (300, 8, 64, (512, 202, 1)),
               (700, 8, 32, (96, 32, 1)), (2000, 7, 64, (512, 1)), (129, 4, 64, (256, 1))]


@pytest.mark.parametrize("B,K,D,top", CASES)
def test_fused_head_vs_oracle_and_unfused(B, K, D, top):
    w, tables, idx, dense, bl, tl = _case(B, K, D, top, seed=B + len(top))
    fused, unfused = _models(tables, bl, tl)
    d, x = dev(dense), [dev(i) for i in idx]
    got = host(abi.dlrm_forward(fused, d, x))
    ref = host(abi.dlrm_forward(unfused, d, x))
    assert got.shape == (B, 1)
    assert_close(got, ref, "fused head vs unfused")
    samples = np.unique(np.linspace(0, B - 1, min(B, 256)).astype(int))
    want, _, _ = oracle.forward(dense[samples], bl, tl, tables,
                                [np.concatenate([i[s * w.bag:(s + 1) * w.bag] for s in samples])
                                 for i in idx])
    assert_close(got[samples], want, "fused head vs oracle")


@pytest.mark.parametrize("B,K,D,top", SMALL_CASES)
def test_head_after_split_layers_vs_oracle(B, K, D, top):
    w, tables, idx, dense, bl, tl = _case(B, K, D, top, seed=B + 3 * len(top))
    fused, unfused = _models(tables, bl, tl)
    d, x = dev(dense), [dev(i) for i in idx]
    got = host(abi.dlrm_forward(fused, d, x))
    ref = host(abi.dlrm_forward(unfused, d, x))
    assert got.shape == (B, 1)
    assert_close(got, ref, "default vs unfused head")
    samples = np.unique(np.linspace(0, B - 1, min(B, 200)).astype(int))
    want, _, _ = oracle.forward(dense[samples], bl, tl, tables,
                                [np.concatenate([i[s * w.bag:(s + 1) * w.bag] for s in samples])
                                 for i in idx])
    assert_close(got[samples], want, "head after split layers vs oracle")


@pytest.mark.parametrize("B", [256, 1000, 2048])
def test_small_batch_forward_repeats_in_plans_and_noalloc(B):
    """The small-batch compositions (slice launch, k partials, the head on its
    own): eager calls on one workspace, both plan modes replayed several
    times and the no-alloc forward all give the first call's output bit for
    bit."""
    import torch
    w, tables, idx, dense, bl, tl = _case(B, 26, 64, (512, 256, 1), seed=B)
    fused, _ = _models(tables, bl, tl)
    d, x = dev(dense), [dev(i) for i in idx]
    out = torch.empty((B, 1), device="cuda")
    ws = torch.empty(fused.workspace_bytes(B), dtype=torch.uint8, device="cuda")
    first = host(abi.dlrm_forward(fused, d, x, out=out, workspace=ws))
    for _ in range(3):
        out.fill_(float("nan"))
        assert np.array_equal(host(abi.dlrm_forward(fused, d, x, out=out, workspace=ws)), first)
    for mode in ("direct", "graph"):
        plan = abi.DlrmPlan(fused, d, x, mode=mode)
        for _ in range(3):
            assert np.array_equal(host(plan.run()), first), mode
        plan.close()
    out2 = torch.empty((B, 1), device="cuda")
    assert np.array_equal(host(abi.dlrm_forward_noalloc(fused, d, x, out2)), first)


@pytest.mark.parametrize("head_act", ["none", "relu", "sigmoid"])
def test_fused_head_activations(head_act):
    w, tables, idx, dense, bl, tl = _case(7300, 6, 32, (96, 64, 1), seed=9, head_act=head_act)
    fused, unfused = _models(tables, bl, tl)
    d, x = dev(dense), [dev(i) for i in idx]
    got = host(abi.dlrm_forward(fused, d, x))
    samples = np.arange(0, 7300, 37)
    want, _, _ = oracle.forward(dense[samples], bl, tl, tables,
                                [np.concatenate([i[s * w.bag:(s + 1) * w.bag] for s in samples])
                                 for i in idx])
    assert_close(got[samples], want, f"head {head_act}")
    assert_close(got, host(abi.dlrm_forward(unfused, d, x)), f"head {head_act} vs unfused")


def test_fused_head_in_plans_and_noalloc():
    """The fused launch replays in both plan modes and runs in the no-alloc
    forward, equal to the eager forward bit for bit."""
    import torch
    w, tables, idx, dense, bl, tl = _case(8192, 26, 64, (512, 256, 1), seed=3)
    fused, _ = _models(tables, bl, tl)
    d, x = dev(dense), [dev(i) for i in idx]
    eager = host(abi.dlrm_forward(fused, d, x))
    for mode in ("direct", "graph"):
        plan = abi.DlrmPlan(fused, d, x, mode=mode)
        for _ in range(3):
            assert np.array_equal(host(plan.run()), eager), mode
        plan.close()
    out = torch.empty((8192, 1), device="cuda")
    assert np.array_equal(host(abi.dlrm_forward_noalloc(fused, d, x, out)), eager)


HEAD_SHAPES = [  # (M, N, K)
    (8192, 256, 512), (1, 256, 512), (33, 256, 512), (300, 200, 415), (65, 1, 7),
    (100, 64, 13), (4097, 7, 64), (31, 256, 1), (257, 130, 131)]


@pytest.mark.parametrize("M,N,K", HEAD_SHAPES)
def test_linear_bias_act_head_vs_oracle(M, N, K):
    import torch
    rng = np.random.default_rng(M + N + K)
    a = rng.standard_normal((M, K)).astype(np.float32)
    bound = np.sqrt(6.0 / (K + N))
    w = rng.uniform(-bound, bound, (N, K)).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    hw = rng.uniform(-0.3, 0.3, (1, N)).astype(np.float32)
    hb = np.array([0.05], np.float32)
    want = oracle.linear(oracle.linear(a, w, b, "relu"), hw, hb, "sigmoid")
    got = host(abi.linear_bias_act_head(dev(a), dev(w), dev(b), "relu", dev(hw.ravel()), dev(hb)))
    assert_close(got, want, f"head {M}x{N}x{K}")
    # no biases, strided output rows (every other float of a guarded buffer)
    buf = torch.full((2 * M + 2,), float("nan"), device="cuda")
    out = buf[1:2 * M + 1].view(M, 2)[:, :1]
    abi.linear_bias_act_head(dev(a), dev(w), None, "none", dev(hw.ravel()), None, "none", out=out)
    want = oracle.linear(oracle.linear(a, w, None, "none"), hw, None, "none")
    hb_ = host(buf)
    assert_close(hb_[1:2 * M + 1:2].reshape(M, 1), want, "head strided")
    assert np.isnan(hb_[0]) and np.isnan(hb_[-1]) and np.all(np.isnan(hb_[2:2 * M + 1:2]))


def test_linear_bias_act_head_rejects_wide_layers():
    import torch
    a = torch.zeros((4, 8), device="cuda")
    w = torch.zeros((257, 8), device="cuda")
    with pytest.raises(abi.DlrmError) as e:
        abi.linear_bias_act_head(a, w, None, "relu", torch.zeros(257, device="cuda"))
    assert e.value.name == "DLRM_ERR_UNSUPPORTED"
