"""GPU parity cases at the edges of the entry points:

- every one of the 256 FP8 E4M3 codes decoded through the gather kernels
  (vector and scalar paths, the standalone gather and the fused pooled copy),
  bit for bit against the oracle's decode of the format definition (the two
  NaN codes must come out as NaN);
- one table (F = 2, a single dot) through the fused call and the dots-only
  call, bit for bit on dyadic inputs;
- guard bands: every output is written into the middle of a NaN-filled
  buffer (a band before and after it, and the padding columns of strided
  outputs), and the bands must come back untouched, so a stray store outside
  an output fails even where the sampled values are right.
"""
import numpy as np
import pytest

import oracle
from conftest import gpu_available
from gpu_helpers import assert_close, dev, host, make_uniform_case
from dlrm_embedding_bag_amd import abi, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]

GUARD = 64  # floats of guard band on each side (256 bytes keep 16-byte alignment)


def _guarded(shape, pad_cols=0):
    """A NaN-filled device buffer with an output view of `shape` inside it:
    GUARD floats before and after, and pad_cols extra columns per row (the
    view is then row-strided).  Returns (buffer, view)."""
    import torch
    rows = int(np.prod(shape[:-1])) if len(shape) > 1 else 1
    cols = shape[-1] + pad_cols
    buf = torch.full((2 * GUARD + rows * cols,), float("nan"), dtype=torch.float32,
                     device="cuda")
    body = buf[GUARD:GUARD + rows * cols].view(rows, cols)
    view = body[:, :shape[-1]]
    if pad_cols == 0:
        view = view.reshape(shape)
    return buf, view


def _assert_guards_untouched(buf, shape, pad_cols=0, what=""):
    b = host(buf)
    assert np.all(np.isnan(b[:GUARD])), f"{what}: guard band before the output was written"
    assert np.all(np.isnan(b[-GUARD:])), f"{what}: guard band after the output was written"
    if pad_cols:
        rows = int(np.prod(shape[:-1]))
        body = b[GUARD:-GUARD].reshape(rows, shape[-1] + pad_cols)
        assert np.all(np.isnan(body[:, shape[-1]:])), f"{what}: padding columns were written"


# ------------------------------------------------------------- FP8 decoding --
def _fp8_dev(codes):
    import torch
    return torch.from_numpy(codes).cuda().view(torch.float8_e4m3fn)


def _all_code_bags(D):
    """A 256-row table whose row r holds code r in every column, and bags of
    length 1 with bag b = row b: pooled row b is the decoded code b."""
    table = np.repeat(np.arange(256, dtype=np.uint8)[:, None], D, axis=1)
    idx = np.arange(256, dtype=np.int32)
    return table, idx


def _check_decoded(got, D, what):
    """Bag b pools code b alone: the oracle's pooled value (its decode of the
    format definition, added to a zero sum, so -0 pools to +0), bit for bit;
    the two NaN codes pool to NaN."""
    table, idx = _all_code_bags(D)
    want = oracle.emb_bag([table], [idx], batch=256, scales=[1.0]).reshape(256, D)
    exact = oracle.fp8_e4m3_to_f64(np.arange(256, dtype=np.uint8))
    nan = np.isnan(exact)
    assert nan.sum() == 2, "the format has two NaN codes (0x7f, 0xff)"
    assert np.all(np.isnan(want[nan]))
    assert np.array_equal(want[~nan], np.repeat(exact[~nan, None], D, axis=1).astype(np.float32))
    g = got.reshape(256, D)
    assert np.all(np.isnan(g[nan])), f"{what}: NaN codes must pool to NaN"
    assert np.array_equal(g[~nan].view(np.uint32), want[~nan].view(np.uint32)), what


# D = 16, 32: generic vector path (one or two 16-code chunks per row); 64, 256:
# shuffle groups of 4 and 16 lanes; 7, 3: scalar path
@pytest.mark.parametrize("D", [16, 32, 64, 256, 7, 3])
def test_fp8_every_code_through_the_gather(D):
    table, idx = _all_code_bags(D)
    t = _fp8_dev(table)
    buf, out = _guarded((256, 1, D))
    abi.emb_bag_pool([t], [dev(idx)], batch=256, out=out, scales=[1.0])
    _check_decoded(host(out), D, f"emb_bag_pool D={D}")
    _assert_guards_untouched(buf, (256, 1, D), what="emb_bag_pool fp8")
    # without a scale (the scale multiply skipped) the bits are the same
    got = host(abi.emb_bag_pool([t], [dev(idx)], batch=256))
    _check_decoded(got, D, f"emb_bag_pool D={D}, no scale")


@pytest.mark.parametrize("D", [16, 64, 7])
def test_fp8_every_code_through_the_fused_pooled_copy(D):
    """The fused kernel's pooled copy (emb_out) of the same bags: its gather
    decodes every code as the standalone one does."""
    import torch
    table, idx = _all_code_bags(D)
    t = _fp8_dev(table)
    # a zero dense row keeps every dot finite except those touching NaN
    dense = torch.zeros((256, D), dtype=torch.float32, device="cuda")
    emb_out = torch.empty((256, 1, D), dtype=torch.float32, device="cuda")
    abi.dlrm_emb_interact_pool([t], [dev(idx)], dense, emb_out=emb_out)
    _check_decoded(host(emb_out), D, f"fused emb_out D={D}")


# ----------------------------------------------------------------- K = 1 --
@pytest.mark.parametrize("B,D,L", [(37, 64, 7), (300, 16, 3), (5, 7, 2), (1024, 128, 20)])
def test_one_table_fused_and_dots_only(B, D, L):
    """F = 2: one dot per sample, dense . pooled, in every layout."""
    import torch
    w = inputs.Workload("k1", batch=B, num_tables=1, rows=200, dim=D, bag=L, dist="zipf")
    tables, idx, dense = make_uniform_case(w, seed=B + D, dyadic=True)
    E = oracle.emb_bag_sum(tables, idx, batch=B)
    want = oracle.interact(dense, E)
    assert want.shape == (B, D + 1)
    td, xd = [dev(t) for t in tables], [dev(i) for i in idx]
    emb_out = torch.empty((B, 1, D), dtype=torch.float32, device="cuda")
    got = host(abi.dlrm_emb_interact(td, xd, dev(dense), emb_out=emb_out))
    assert np.array_equal(got, want)
    assert np.array_equal(host(emb_out), E)
    dots = host(abi.dlrm_emb_interact_dots(td, xd, dev(dense)))
    assert dots.shape == (B, 1) and np.array_equal(dots, want[:, D:])
    pool = host(abi.dlrm_emb_interact_pool(td, xd, dev(dense)))
    assert np.array_equal(pool, want)
    # CSR offsets equal to the uniform bags give the same bits
    offs = [dev(inputs.offsets(w))]
    assert np.array_equal(host(abi.dlrm_emb_interact(td, xd, dev(dense), offsets=offs)), want)


# ------------------------------------------------------------ guard bands --
@pytest.mark.parametrize("B,K,rows,D,L", [(37, 5, 333, 64, 7), (11, 3, 40, 7, 5),
                                          (130, 26, 200, 128, 40), (3, 2, 10, 1024, 3)])
def test_guard_bands_gather(B, K, rows, D, L):
    w = inputs.Workload("g", batch=B, num_tables=K, rows=rows, dim=D, bag=L, dist="zipf")
    tables, idx, _ = make_uniform_case(w, seed=K, dyadic=True)
    want = oracle.emb_bag_sum(tables, idx, batch=B)
    td, xd = [dev(t) for t in tables], [dev(i) for i in idx]
    buf, out = _guarded((B, K, D))
    abi.emb_bag_sum_multi(td, xd, batch=B, out=out)
    assert np.array_equal(host(out), want)
    _assert_guards_untouched(buf, (B, K, D), what="emb_bag_sum_multi")
    buf, out = _guarded((B, K, D))
    abi.emb_bag_pool(td, xd, batch=B, out=out, pool="mean")
    assert_close(host(out), oracle.emb_bag(tables, idx, batch=B, pool="mean"), "mean")
    _assert_guards_untouched(buf, (B, K, D), what="emb_bag_pool mean")


@pytest.mark.parametrize("B,K,D", [(33, 26, 64), (5, 3, 7), (40, 1, 64), (2, 26, 128),
                                   (1100, 32, 64)])
def test_guard_bands_interaction(B, K, D):
    rng = np.random.default_rng(B + K + D)
    dense = inputs.dyadic(rng, (B, D))
    emb = inputs.dyadic(rng, (B, K, D))
    want = oracle.interact(dense, emb)
    P = (K + 1) * K // 2
    buf, out = _guarded((B, D + P))
    abi.dlrm_interact_lower_tri(dev(dense), dev(emb), out=out)
    assert np.array_equal(host(out), want)
    _assert_guards_untouched(buf, (B, D + P), what="dlrm_interact_lower_tri")


@pytest.mark.parametrize("B,K,rows,D,L", [(77, 26, 500, 64, 20), (10, 5, 50, 7, 3),
                                          (21, 26, 200, 128, 40), (2048, 8, 1000, 64, 20)])
def test_guard_bands_fused(B, K, rows, D, L):
    """The fused call's [dense | dots] output, its pooled copy, and the
    dots-only layout into a row-strided destination."""
    w = inputs.Workload("gf", batch=B, num_tables=K, rows=rows, dim=D, bag=L, dist="zipf")
    tables, idx, dense = make_uniform_case(w, seed=L, dyadic=True)
    E = oracle.emb_bag_sum(tables, idx, batch=B)
    want = oracle.interact(dense, E)
    td, xd = [dev(t) for t in tables], [dev(i) for i in idx]
    P = (K + 1) * K // 2
    obuf, out = _guarded((B, D + P))
    ebuf, emb_out = _guarded((B, K, D))
    abi.dlrm_emb_interact(td, xd, dev(dense), out=out, emb_out=emb_out)
    assert np.array_equal(host(out), want)
    assert np.array_equal(host(emb_out), E)
    _assert_guards_untouched(obuf, (B, D + P), what="fused out")
    _assert_guards_untouched(ebuf, (B, K, D), what="fused emb_out")
    dbuf, dots = _guarded((B, P), pad_cols=5)
    abi.dlrm_emb_interact_dots(td, xd, dev(dense), out=dots)
    assert np.array_equal(host(dots), want[:, D:])
    _assert_guards_untouched(dbuf, (B, P), pad_cols=5, what="dots only")


@pytest.mark.parametrize("M,N,K", [(300, 512, 13), (300, 256, 512), (300, 1, 256),
                                   (129, 130, 131), (2048, 512, 415), (8192, 64, 256)])
def test_guard_bands_linear(M, N, K):
    rng = np.random.default_rng(M + N + K)
    a = rng.standard_normal((M, K)).astype(np.float32)
    wt = (rng.standard_normal((N, K)) * 0.05).astype(np.float32)
    b = (rng.standard_normal(N) * 0.1).astype(np.float32)
    want = oracle.linear(a, wt, b, "relu")
    for pad in (0, 3):
        buf, out = _guarded((M, N), pad_cols=pad)
        abi.linear_bias_act(dev(a), dev(wt), dev(b), "relu", out=out)
        assert_close(host(out), want, f"linear {M}x{N}x{K}")
        _assert_guards_untouched(buf, (M, N), pad_cols=pad, what=f"linear pad {pad}")


@pytest.mark.parametrize("options", [(), ("layered",), ("unfused_head",)])
def test_guard_bands_forward(options):
    w = inputs.Workload("gfwd", batch=1000, num_tables=26, rows=3000, dim=64, bag=20,
                        dist="zipf", dense_in=13, bottom=(512, 256, 64), top=(512, 256, 1))
    tables, idx, dense = make_uniform_case(w, seed=7)
    bottom, top = inputs.dlrm_layers(w, 7, bias_std=0.1)
    model = abi.DlrmModel([(dev(a), dev(b), act) for a, b, act in bottom],
                          [(dev(a), dev(b), act) for a, b, act in top],
                          [dev(t) for t in tables], options=options)
    want, _, _ = oracle.forward(dense, bottom, top, tables, idx)
    buf, out = _guarded((w.batch, 1))
    abi.dlrm_forward(model, dev(dense), [dev(i) for i in idx], out=out)
    assert_close(host(out), want, f"forward {options}")
    _assert_guards_untouched(buf, (w.batch, 1), what=f"forward {options}")
