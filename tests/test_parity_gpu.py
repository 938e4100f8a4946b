"""GPU parity: every C-ABI entry point against the CPU oracle on the same
seeded inputs.  Integer, index and layout facts are compared bit for bit
(dyadic inputs make every summation order exact); float results must satisfy
|gpu - oracle| <= 1e-5 + 1e-5 |oracle|."""
import numpy as np
import pytest

import oracle
from conftest import gpu_available
from gpu_helpers import assert_close, dev, host, make_uniform_case
from dlrm_embedding_bag_amd import abi, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def W(name="case", **kw):
    base = dict(batch=16, num_tables=2, rows=100, dim=16, bag=4, dist="uniform")
    base.update(kw)
    return inputs.Workload(name, **base)


# ------------------------------------------------------------ emb_bag_sum_multi --
def test_emb_bag_tiny_workload():
    """B=32, K=2 tables x 1000 rows x D=16, 4 indices per bag."""
    w = inputs.WORKLOADS["tiny"]
    tables, idx, _ = make_uniform_case(w)
    want = oracle.emb_bag_sum(tables, idx, batch=w.batch)
    td = [dev(t) for t in tables]
    xd = [dev(i) for i in idx]
    got = host(abi.emb_bag_sum_multi(td, xd, batch=w.batch))
    assert_close(got, want, "tiny")
    offs = [dev(inputs.offsets(w)) for _ in tables]
    got_off = host(abi.emb_bag_sum_multi(td, xd, offsets=offs))
    assert np.array_equal(got_off, got), "arange offsets must equal uniform stride bit for bit"


EMB_SHAPES = [  # (B, K, rows, D, L)
    (37, 5, 333, 64, 7),      # ragged batch, several waves
    (130, 3, 50, 16, 20),     # tail of the unrolled bag loop
    (5, 64, 10, 4, 1),        # maximum K, one-lane rows
    (9, 4, 30, 12, 3),        # D % 16 != 0, three lanes per row
    (11, 3, 40, 7, 5),        # D % 4 != 0: scalar path
    (6, 2, 20, 256, 9),       # one full wave per row
    (3, 2, 10, 1024, 3),      # four column chunks per lane
    (4, 3, 25, 132, 2),       # 33 lanes per row
    (2, 1, 5, 1, 8),          # D = 1
    (300, 8, 1000, 128, 40),  # D = 128, L = 40
]


@pytest.mark.parametrize("B,K,rows,D,L", EMB_SHAPES)
def test_emb_bag_dyadic_bit_exact(B, K, rows, D, L):
    w = W(batch=B, num_tables=K, rows=rows, dim=D, bag=L)
    tables, idx, _ = make_uniform_case(w, seed=B + K, dyadic=True)
    want = oracle.emb_bag_sum(tables, idx, batch=B)
    got = host(abi.emb_bag_sum_multi([dev(t) for t in tables], [dev(i) for i in idx],
                                     batch=B))
    assert np.array_equal(got, want)


def test_emb_bag_random_values_within_tolerance():
    w = W(batch=257, num_tables=6, rows=5000, dim=64, bag=20, dist="zipf")
    tables, idx, _ = make_uniform_case(w, seed=3)
    want = oracle.emb_bag_sum(tables, idx, batch=w.batch)
    got = host(abi.emb_bag_sum_multi([dev(t) for t in tables], [dev(i) for i in idx],
                                     batch=w.batch))
    assert_close(got, want, "zipf random")


def _csr_case(rng, B, rows, D, max_len):
    lens = rng.integers(0, max_len + 1, size=B)
    lens[0] = 0            # first bag empty
    lens[-1] = 0           # last bag empty
    if B > 3:
        lens[B // 2] = max_len + 9   # one long bag
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    n = int(lens.sum())
    idx = rng.integers(0, rows, size=n).astype(np.int32)
    table = (rng.integers(-128, 128, (rows, D)) / 256.0).astype(np.float32)
    return table, idx, offs


@pytest.mark.parametrize("D", [64, 16, 7])
def test_emb_bag_csr_offsets(D):
    rng = np.random.default_rng(D)
    B = 41
    cases = [_csr_case(rng, B, 70, D, 12) for _ in range(3)]
    tables = [c[0] for c in cases]
    idx = [c[1] for c in cases]
    offs = [c[2] for c in cases]
    want = oracle.emb_bag_sum(tables, idx, offs)
    got = host(abi.emb_bag_sum_multi([dev(t) for t in tables], [dev(i) for i in idx],
                                     offsets=[dev(o) for o in offs]))
    assert np.array_equal(got, want)
    assert np.all(got[0] == 0) and np.all(got[-1] == 0)


def test_emb_bag_empty_bags_uniform():
    """L = 0 (no indices at all): every bag pools to zero."""
    import torch
    t = dev(np.ones((4, 8), np.float32))
    x = torch.empty(0, dtype=torch.int32, device="cuda")
    got = host(abi.emb_bag_sum_multi([t, t], [x, x], batch=5))
    assert got.shape == (5, 2, 8) and np.all(got == 0)


def test_emb_bag_unaligned_output_takes_scalar_path():
    import torch
    w = W(batch=13, num_tables=3, rows=20, dim=8, bag=3)
    tables, idx, _ = make_uniform_case(w, seed=9, dyadic=True)
    want = oracle.emb_bag_sum(tables, idx, batch=w.batch)
    buf = torch.zeros(13 * 3 * 8 + 1, dtype=torch.float32, device="cuda")
    out = buf[1:].view(13, 3, 8)
    abi.emb_bag_sum_multi([dev(t) for t in tables], [dev(i) for i in idx], batch=13, out=out)
    assert np.array_equal(host(out), want)
    assert host(buf)[0] == 0.0


def test_emb_bag_zero_batch_is_noop():
    import torch
    t = dev(np.ones((4, 8), np.float32))
    x = torch.empty(0, dtype=torch.int32, device="cuda")
    got = abi.emb_bag_sum_multi([t], [x], batch=0)
    assert got.shape == (0, 1, 8)


# ------------------------------------------------------- dlrm_interact_lower_tri --
INTERACT_SHAPES = [  # (B, K, D)
    (7, 1, 4), (33, 26, 64), (64, 32, 64), (19, 8, 12), (5, 3, 7), (3, 64, 128),
    (130, 2, 16), (2, 26, 128), (1, 5, 1), (9, 64, 4),
    (13, 7, 64), (11, 9, 16), (6, 11, 32), (4, 14, 8), (40, 1, 64), (3, 2, 256),
]


@pytest.mark.parametrize("B,K,D", INTERACT_SHAPES)
def test_interact_dyadic_bit_exact(B, K, D):
    rng = np.random.default_rng(B * 100 + K)
    dense = inputs.dyadic(rng, (B, D))
    emb = inputs.dyadic(rng, (B, K, D))
    want = oracle.interact(dense, emb)
    got = host(abi.dlrm_interact_lower_tri(dev(dense), dev(emb)))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("B,K,D", [(33, 26, 64), (17, 32, 64), (8, 26, 128), (5, 3, 7)])
def test_interact_random_within_tolerance(B, K, D):
    rng = np.random.default_rng(K + D)
    dense = rng.standard_normal((B, D)).astype(np.float32)
    emb = (rng.standard_normal((B, K, D)) * 0.05).astype(np.float32)
    want = oracle.interact(dense, emb)
    got = host(abi.dlrm_interact_lower_tri(dev(dense), dev(emb)))
    assert np.array_equal(got[:, :D], dense), "dense columns are an exact copy"
    assert_close(got, want, "interact")


# -------------------------------------------------------------- dlrm_emb_interact --
@pytest.mark.parametrize("B,K,rows,D,L,dist", [
    (32, 2, 1000, 16, 4, "uniform"), (77, 26, 500, 64, 20, "zipf"),
    (40, 32, 300, 64, 20, "zipf"), (21, 26, 200, 128, 40, "zipf"),
    (10, 5, 50, 7, 3, "uniform"), (3, 64, 20, 32, 2, "uniform")])
def test_emb_interact_fused(B, K, rows, D, L, dist):
    import torch
    w = W(batch=B, num_tables=K, rows=rows, dim=D, bag=L, dist=dist)
    for dyadic in (True, False):
        tables, idx, dense = make_uniform_case(w, seed=L, dyadic=dyadic)
        E = oracle.emb_bag_sum(tables, idx, batch=B)
        want = oracle.interact(dense, E)
        td = [dev(t) for t in tables]
        xd = [dev(i) for i in idx]
        emb_out = torch.empty((B, K, D), dtype=torch.float32, device="cuda")
        got = host(abi.dlrm_emb_interact(td, xd, dev(dense), emb_out=emb_out))
        if dyadic:
            assert np.array_equal(got, want)
            assert np.array_equal(host(emb_out), E)
        else:
            assert_close(got, want, "fused")
            assert_close(host(emb_out), E, "fused emb_out")
        # the pooled copy is the unfused gather's result bit for bit
        assert np.array_equal(host(emb_out), host(abi.emb_bag_sum_multi(td, xd, batch=B)))


def test_emb_interact_csr_offsets():
    rng = np.random.default_rng(5)
    B, D = 29, 16
    cases = [_csr_case(rng, B, 40, D, 9) for _ in range(4)]
    tables = [c[0] for c in cases]
    idx = [c[1] for c in cases]
    offs = [c[2] for c in cases]
    dense = inputs.dyadic(rng, (B, D))
    want = oracle.interact(dense, oracle.emb_bag_sum(tables, idx, offs))
    got = host(abi.dlrm_emb_interact([dev(t) for t in tables], [dev(i) for i in idx],
                                     dev(dense), offsets=[dev(o) for o in offs]))
    assert np.array_equal(got, want)


# ----------------------------------------------------------------- linear_bias_act --
LINEAR_SHAPES = [  # (M, N, K)
    (300, 512, 13), (300, 256, 512), (300, 64, 256), (300, 512, 415), (300, 256, 512),
    (300, 1, 256), (37, 19, 13), (129, 130, 131), (64, 8, 5), (1, 1, 1), (5, 9, 3),
    (257, 128, 64), (70, 3, 40), (513, 72, 36),
    (33, 22, 16), (40, 2, 600), (2000, 516, 16), (77, 4, 512),
    # 64-row tiles with two wave groups splitting k (K >= 128): 64 x 64 and
    # 64 x 32 tiles, ragged M, N and K, K = 128 exactly (two half slabs)
    (2048, 512, 415), (2048, 256, 512), (2100, 520, 200), (600, 96, 128), (300, 70, 127),
    # K <= 16 with N % 4 == 0 (the register-weight kernel): partial column
    # groups, K = 1, a ragged last row batch
    (37, 12, 13), (130, 1024, 7), (5, 260, 1), (1, 256, 16), (9, 20, 4),
    # two row batches per wave (enough rows for 2048 waves), ragged last batch
    (8192, 512, 13), (8195, 260, 5),
]


@pytest.mark.parametrize("M,N,K", LINEAR_SHAPES)
@pytest.mark.parametrize("act", ["none", "relu", "sigmoid"])
def test_linear_parity(M, N, K, act):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a = rng.standard_normal((M, K)).astype(np.float32)
    bound = np.sqrt(6.0 / (K + N))
    w = rng.uniform(-bound, bound, (N, K)).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    want = oracle.linear(a, w, b, act)
    got = host(abi.linear_bias_act(dev(a), dev(w), dev(b), act))
    assert_close(got, want, f"linear {M}x{N}x{K} {act}")


# N = 1 (the sigmoid head's kernel): one wave per row up to 4,096 rows with
# 256-column chunks, four rows per wave above with 64-column chunks; K that
# fills 1, 2, 4 or 8 chunks exactly or leaves the last one ragged, K = 4 (one
# float4), K > 1024 (the wave-per-4-rows fallback), an unaligned row stride
# (the fallback too), ragged row counts on both sides of the switch.
HEAD_ROW_SHAPES = [  # (M, K, lda)
    (1, 4, 4), (17, 60, 60), (300, 256, 256), (301, 260, 260), (4096, 512, 512),
    (63, 516, 516), (5, 1024, 1024), (4097, 64, 64), (4100, 100, 100), (8195, 256, 256),
    (4101, 300, 300), (6000, 512, 512), (9000, 516, 516), (33, 1028, 1028),
    (4200, 1100, 1100), (50, 255, 255), (70, 256, 257),
]


@pytest.mark.parametrize("M,K,lda", HEAD_ROW_SHAPES)
def test_linear_one_output_column(M, K, lda):
    import torch
    rng = np.random.default_rng(M + 3 * K + lda)
    abuf = rng.standard_normal((M, lda)).astype(np.float32)
    a = abuf[:, :K]
    w = rng.uniform(-0.2, 0.2, (1, K)).astype(np.float32)
    b = np.array([0.1], np.float32)
    want = oracle.linear(np.ascontiguousarray(a), w, b, "sigmoid")
    out = torch.full((M + 2,), float("nan"), device="cuda")
    got = abi.linear_bias_act(dev(abuf)[:, :K], dev(w), dev(b), "sigmoid",
                              out=out[1:M + 1].view(M, 1))
    assert_close(host(got), want, f"one output column {M}x{K}")
    o = host(out)
    assert np.isnan(o[0]) and np.isnan(o[-1])
    # dyadic inputs: every order of the sum is exact, so the kernel's output
    # equals the oracle's bit for bit
    ad = inputs.dyadic(rng, (M, K), max_int=64)
    wd = inputs.dyadic(rng, (1, K), max_int=64)
    got = host(abi.linear_bias_act(dev(ad), dev(wd), None, "none"))
    assert np.array_equal(got, oracle.linear(ad, wd, None, "none"))


def test_linear_dyadic_bit_exact_and_no_bias():
    rng = np.random.default_rng(2)
    for M, N, K in ((300, 512, 13), (129, 130, 131), (300, 1, 256)):
        a = inputs.dyadic(rng, (M, K))
        w = inputs.dyadic(rng, (N, K))
        want = oracle.linear(a, w, None, "relu")
        got = host(abi.linear_bias_act(dev(a), dev(w), None, "relu"))
        assert np.array_equal(got, want), (M, N, K)


def test_linear_strided_operands():
    """lda > k and ldc > n, as dlrm_forward uses inside its workspace."""
    import torch
    rng = np.random.default_rng(4)
    M, N, K = 99, 70, 45
    abuf = dev(rng.standard_normal((M, 52)).astype(np.float32))
    a = abuf[:, :K]
    w = rng.standard_normal((N, K)).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    cbuf = torch.full((M, 76), -7.0, device="cuda")
    c = cbuf[:, :N]
    abi.linear_bias_act(a, dev(w), dev(b), "relu", out=c)
    want = oracle.linear(host(a), w, b, "relu")
    assert_close(host(c), want, "strided")
    assert np.all(host(cbuf)[:, N:] == -7.0), "columns beyond n must be untouched"


def test_linear_thin_k_strided_operands():
    """K <= 16 with lda > k (unaligned rows of A) and ldc > n."""
    import torch
    rng = np.random.default_rng(6)
    M, N, K = 99, 64, 13
    abuf = dev(rng.standard_normal((M, 17)).astype(np.float32))
    a = abuf[:, :K]
    w = rng.standard_normal((N, K)).astype(np.float32)
    b = rng.standard_normal(N).astype(np.float32)
    cbuf = torch.full((M, 72), -7.0, device="cuda")
    c = cbuf[:, :N]
    abi.linear_bias_act(a, dev(w), dev(b), "sigmoid", out=c)
    assert_close(host(c), oracle.linear(host(a), w, b, "sigmoid"), "thin strided")
    assert np.all(host(cbuf)[:, N:] == -7.0), "columns beyond n must be untouched"


# --------------------------------------------------------------------- mlp_forward --
MLP_STACKS = [  # (M, widths, acts)
    (300, (13, 512, 256, 64), ("relu", "relu", "relu")),
    (300, (415, 512, 256, 1), ("relu", "relu", "sigmoid")),
    (37, (64, 128), ("none",)),
    (65, (100, 256, 4), ("relu", "sigmoid")),
    (96, (32, 64, 128, 256, 512), ("relu", "none", "relu", "relu")),
    (1, (13, 512, 256, 64), ("relu", "relu", "relu")),
    (513, (7, 64, 8), ("relu", "none")),
]


@pytest.mark.parametrize("M,widths,acts", MLP_STACKS)
def test_mlp_forward_parity(M, widths, acts):
    rng = np.random.default_rng(M + len(widths))
    a = rng.standard_normal((M, widths[0])).astype(np.float32)
    layers = []
    for i, act in enumerate(acts):
        k, n = widths[i], widths[i + 1]
        bound = np.sqrt(6.0 / (k + n))
        layers.append((rng.uniform(-bound, bound, (n, k)).astype(np.float32),
                       (rng.standard_normal(n) * 0.1).astype(np.float32), act))
    want = a
    for w, b, act in layers:
        want = oracle.linear(want, w, b, act)
    got = host(abi.mlp_forward(dev(a), [(dev(w), dev(b), act) for w, b, act in layers]))
    assert_close(got, want, f"mlp {widths}")


def test_mlp_forward_strided_and_no_bias():
    import torch
    rng = np.random.default_rng(8)
    M = 77
    abuf = dev(rng.standard_normal((M, 420)).astype(np.float32))
    a = abuf[:, :415]
    ws = [rng.standard_normal((512, 415)).astype(np.float32) * 0.05,
          rng.standard_normal((256, 512)).astype(np.float32) * 0.05,
          rng.standard_normal((64, 256)).astype(np.float32) * 0.05]
    cbuf = torch.full((M, 72), -3.0, device="cuda")
    c = cbuf[:, :64]
    abi.mlp_forward(a, [(dev(ws[0]), None, "relu"), (dev(ws[1]), None, "relu"),
                        (dev(ws[2]), None, "none")], out=c)
    want = host(a)
    for w, act in zip(ws, ("relu", "relu", "none")):
        want = oracle.linear(want, w, None, act)
    assert_close(host(c), want, "strided chain")
    assert np.all(host(cbuf)[:, 64:] == -3.0)


# -------------------------------------------------------------------- dlrm_forward --
def _forward_case(w, seed, bias_std=0.1):
    import torch
    tables, idx, dense = make_uniform_case(w, seed)
    bottom, top = inputs.dlrm_layers(w, seed, bias_std=bias_std)
    model = abi.DlrmModel([(dev(a), dev(b), act) for a, b, act in bottom],
                          [(dev(a), dev(b), act) for a, b, act in top],
                          [dev(t) for t in tables])
    return tables, idx, dense, bottom, top, model


@pytest.mark.parametrize("B,K,D,L", [(64, 4, 16, 3), (131, 26, 64, 20), (20, 8, 32, 1)])
def test_forward_small(B, K, D, L):
    w = inputs.Workload("fwd", batch=B, num_tables=K, rows=400, dim=D, bag=L, dist="zipf",
                        dense_in=13, bottom=(48, D), top=(40, 24, 1))
    tables, idx, dense, bottom, top, model = _forward_case(w, seed=K)
    want, _, _ = oracle.forward(dense, bottom, top, tables, idx)
    got = host(abi.dlrm_forward(model, dev(dense), [dev(i) for i in idx]))
    assert_close(got, want, "forward")
    offs = [dev(inputs.offsets(w)) for _ in range(K)]
    got2 = host(abi.dlrm_forward(model, dev(dense), [dev(i) for i in idx], offsets=offs))
    assert np.array_equal(got, got2)


@pytest.mark.parametrize("B", [40, 700, 1100])
def test_emb_interact_workgroup_sizes_bit_exact(B):
    """K = 32, D = 64: the fused launch takes 512-thread workgroups at B = 40,
    256 at B = 700 and 128 at B = 1100 (workgroups grow while the grid leaves
    CUs idle); dyadic inputs make every summation order exact, so each size
    must give the oracle's bits, and the standalone gather + interaction the
    same."""
    w = W(batch=B, num_tables=32, rows=300, dim=64, bag=20, dist="zipf")
    tables, idx, dense = make_uniform_case(w, seed=B, dyadic=True)
    E = oracle.emb_bag_sum(tables, idx, batch=B)
    want = oracle.interact(dense, E)
    td = [dev(t) for t in tables]
    xd = [dev(i) for i in idx]
    got = host(abi.dlrm_emb_interact(td, xd, dev(dense)))
    assert np.array_equal(got, want)
    unfused = host(abi.dlrm_interact_lower_tri(dev(dense), abi.emb_bag_sum_multi(td, xd, batch=B)))
    assert np.array_equal(unfused, want)
