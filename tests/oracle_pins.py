"""Pins of the CPU oracle to facts other than itself.

Each pin takes the loaded oracle library (`lib`), so that the same pins run
against the real oracle and against copies with a planted mistake
(test_oracle_mutants.py): every planted mistake must make some pin fail.

What pins what:
  pair map     closed form == double-loop enumeration == numpy.tril_indices
  emb-bag      numpy/torch float64 library routines (count-matrix product,
               torch embedding_bag), L=1 row copy, k identical indices == k*row,
               linearity, arange offsets == uniform stride, hand-worked CSR case
  emb-bag fp8  the E4M3 format's fixed points (1, +-, smallest subnormal and
               normal, 448, NaN), torch's float8_e4m3fn on all 256 codes, torch
               float64 embedding_bag on decoded tables times per-table scales,
               exact power-of-two scaling
  emb-bag ext  torch's bfloat16->float32 conversion on all 65536 patterns, torch
               float64 embedding_bag (mean; sum with per-sample weights; bf16
               tables), unit weights == sum, mean of copies == row, hand-worked
               mean / weighted case with an empty bag
  interaction  numpy float64 X X^T + tril_indices, torch bmm, symmetry of the
               Gram matrix, F=2 single dot, hand-worked F=3 case, dense copy
  linear       numpy float64 A W^T + b on non-square shapes, identity and zero
               weights, sigmoid(0) = 1/2, hand-worked case
  forward      torch float64 nn.EmbeddingBag / bmm / tril_indices / nn.Linear
"""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- pair map --
def pin_pair_map(lib):
    # spot values from the strict-lower-triangle row-major order
    spots = {0: (1, 0), 1: (2, 0), 2: (2, 1), 3: (3, 0), 4: (3, 1), 5: (3, 2),
             6: (4, 0)}
    for p, ij in spots.items():
        assert oracle.pair_closed_form(p, lib=lib) == ij, (p, ij)
    # brute force: the closed form equals the double loop for every F <= 4096
    # (the lower triangle of a smaller F is a prefix of a larger one)
    F = 4096
    ei, ej = oracle.pair_enumerate(F, lib=lib)
    ci, cj = oracle.pair_closed_form_range(0, len(ei), lib=lib)
    assert np.array_equal(ei, ci) and np.array_equal(ej, cj)
    # library routine: numpy.tril_indices(F, -1) is the same order
    for f in (2, 3, 5, 33, 27, 257):
        ti, tj = np.tril_indices(f, -1)
        ei, ej = oracle.pair_enumerate(f, lib=lib)
        assert np.array_equal(ei, ti) and np.array_equal(ej, tj), f
    # far beyond float precision the corrections keep the row-start inequality
    for p in (2**31 - 1, 2**31, 3 * 2**40 + 12345, 2**52 + 7):
        i, j = oracle.pair_closed_form(p, lib=lib)
        assert i * (i - 1) // 2 <= p < i * (i + 1) // 2, p
        assert 0 <= j < i and i * (i - 1) // 2 + j == p


# ----------------------------------------------------------------- emb-bag --
def _count_matrix(idx, B, L, rows):
    c = np.zeros((B, rows), np.float64)
    for b in range(B):
        np.add.at(c[b], idx[b * L:(b + 1) * L], 1.0)
    return c


def pin_emb_bag(lib):
    rng = np.random.default_rng(11)
    B, D, L = 6, 5, 3
    rows = [7, 11, 4]
    tables = [rng.standard_normal((r, D)).astype(np.float32) for r in rows]
    idx = [rng.integers(0, r, B * L).astype(np.int32) for r in rows]
    out = oracle.emb_bag_sum(tables, idx, batch=B, lib=lib)
    assert out.shape == (B, len(rows), D)
    # a library matrix product over the bag count matrix gives the same sums
    for k, (t, i) in enumerate(zip(tables, idx)):
        ref = _count_matrix(i, B, L, t.shape[0]) @ t.astype(np.float64)
        np.testing.assert_allclose(out[:, k, :], ref, rtol=1e-6, atol=1e-7)
    # torch's own embedding_bag in float64 (library routine)
    import torch
    for k, (t, i) in enumerate(zip(tables, idx)):
        ref = torch.nn.functional.embedding_bag(
            torch.from_numpy(i.astype(np.int64)),
            torch.from_numpy(t.astype(np.float64)),
            torch.arange(0, B * L, L), mode="sum").numpy()
        np.testing.assert_allclose(out[:, k, :], ref, rtol=1e-6, atol=1e-7)
    # L = 1: a bit-exact row copy
    one = oracle.emb_bag_sum([tables[0]], [idx[0][:B]], batch=B, lib=lib)
    assert np.array_equal(one[:, 0, :], tables[0][idx[0][:B]])
    # a bag of k copies of row r equals float(k * double(row r)) exactly
    for kk in (1, 2, 3, 7, 20, 129):
        bag = np.full(kk, 3, np.int32)
        got = oracle.emb_bag_sum([tables[1]], [bag], batch=1, lib=lib)[0, 0]
        want = (kk * tables[1][3].astype(np.float64)).astype(np.float32)
        assert np.array_equal(got, want), kk
    # linearity: pool(2 W1 + W2) = 2 pool(W1) + pool(W2), exact on dyadic data
    w1 = (rng.integers(-128, 128, (9, D)) / 256.0).astype(np.float32)
    w2 = (rng.integers(-128, 128, (9, D)) / 256.0).astype(np.float32)
    i9 = rng.integers(0, 9, B * 4).astype(np.int32)
    lhs = oracle.emb_bag_sum([2 * w1 + w2], [i9], batch=B, lib=lib)
    rhs = 2 * oracle.emb_bag_sum([w1], [i9], batch=B, lib=lib) + \
        oracle.emb_bag_sum([w2], [i9], batch=B, lib=lib)
    assert np.array_equal(lhs, rhs)
    # arange offsets give exactly the uniform-stride result
    offs = [np.arange(0, B * L, L, dtype=np.int32) for _ in rows]
    assert np.array_equal(oracle.emb_bag_sum(tables, idx, offs, lib=lib), out)
    # hand-worked CSR case with an empty bag
    g = _golden("emb_bag_csr.json")
    got = oracle.emb_bag_sum([np.array(g["table"], np.float32)],
                             [np.array(g["indices"], np.int32)],
                             [np.array(g["offsets"], np.int32)], lib=lib)
    assert np.array_equal(got[:, 0, :], np.array(g["expected"], np.float32))


# ------------------------------------- emb-bag: mean, weights, bf16 tables --
def pin_emb_bag_ext(lib):
    import torch
    F = torch.nn.functional
    rng = np.random.default_rng(21)
    # bf16 -> f32 against torch's own conversion (every 16-bit pattern)
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_to_f32(bits, lib=lib)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(mine, ref, equal_nan=True)
    B, D, L = 6, 5, 3
    rows = [9, 13]
    tables = [rng.standard_normal((r, D)).astype(np.float32) for r in rows]
    idx = [rng.integers(0, r, B * L).astype(np.int32) for r in rows]
    offs = torch.arange(0, B * L, L)
    t64 = [torch.from_numpy(t.astype(np.float64)) for t in tables]
    i64 = [torch.from_numpy(i.astype(np.int64)) for i in idx]
    # f32 sum is exactly oracle_emb_bag_sum
    assert np.array_equal(oracle.emb_bag(tables, idx, batch=B, lib=lib),
                          oracle.emb_bag_sum(tables, idx, batch=B, lib=lib))
    # mean against torch float64
    got = oracle.emb_bag(tables, idx, batch=B, pool="mean", lib=lib)
    for k in range(2):
        want = F.embedding_bag(i64[k], t64[k], offs, mode="mean").numpy()
        np.testing.assert_allclose(got[:, k], want, rtol=1e-6, atol=1e-7)
    # per-sample weights against torch float64
    wts = [rng.standard_normal(B * L).astype(np.float32) for _ in rows]
    got = oracle.emb_bag(tables, idx, batch=B, weights=wts, lib=lib)
    for k in range(2):
        want = F.embedding_bag(i64[k], t64[k], offs, mode="sum",
                               per_sample_weights=torch.from_numpy(wts[k].astype(np.float64))
                               ).numpy()
        np.testing.assert_allclose(got[:, k], want, rtol=1e-6, atol=1e-6)
    # all-ones weights are the plain sum, bit for bit
    ones = [np.ones(B * L, np.float32) for _ in rows]
    assert np.array_equal(oracle.emb_bag(tables, idx, batch=B, weights=ones, lib=lib),
                          oracle.emb_bag_sum(tables, idx, batch=B, lib=lib))
    # the mean of k copies of one row is that row exactly
    for kk in (1, 3, 7):
        got = oracle.emb_bag([tables[0]], [np.full(kk, 2, np.int32)], batch=1, pool="mean",
                             lib=lib)
        assert np.array_equal(got[0, 0], tables[0][2]), kk
    # bf16 tables: pooled like their exact f32 values (torch conversion)
    tb = [(rng.integers(0, 1 << 16, (r, D)) & 0x7f7f).astype(np.uint16) for r in rows]
    tb32 = [torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).double() for t in tb]
    for pool in ("sum", "mean"):
        got = oracle.emb_bag(tb, idx, batch=B, pool=pool, lib=lib)
        for k in range(2):
            want = F.embedding_bag(i64[k], tb32[k], offs, mode=pool).numpy()
            np.testing.assert_allclose(got[:, k], want, rtol=1e-6, atol=1e-30)
    # weights with mean pooling are rejected (torch rejects them too)
    try:
        oracle.emb_bag(tables, idx, batch=B, weights=wts, pool="mean", lib=lib)
        raise AssertionError("weights with mean pooling must be rejected")
    except oracle.OracleError:
        pass
    # hand-worked CSR case with an empty bag
    g = _golden("emb_bag_mean_weights.json")
    t = [np.array(g["table"], np.float32)]
    i = [np.array(g["indices"], np.int32)]
    o = [np.array(g["offsets"], np.int32)]
    got = oracle.emb_bag(t, i, o, pool="mean", lib=lib)
    assert np.array_equal(got[:, 0], np.array(g["expected_mean"], np.float32))
    got = oracle.emb_bag(t, i, o, weights=[np.array(g["weights"], np.float32)], lib=lib)
    assert np.array_equal(got[:, 0], np.array(g["expected_weighted_sum"], np.float32))


# -------------------------------------------- emb-bag: fp8 tables, scales --
def pin_emb_bag_fp8(lib):
    import torch
    F = torch.nn.functional
    # the format's own fixed points: 1.0, the smallest subnormal, the smallest
    # normal, the largest finite value, signs, and the NaN code
    spots = {0x38: 1.0, 0xB8: -1.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0x7E: 448.0,
             0x3C: 1.5, 0x00: 0.0, 0x07: 7 * 2.0 ** -9}
    for c, v in spots.items():
        assert oracle.fp8_e4m3_to_f64(np.array([c], np.uint8), lib=lib)[0] == v, hex(c)
    assert np.isnan(oracle.fp8_e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8), lib=lib)).all()
    # every code against torch's float8_e4m3fn
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.fp8_e4m3_to_f64(codes, lib=lib)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(mine, ref, equal_nan=True)
    # pooled fp8 tables against torch float64 embedding_bag on the decoded values
    rng = np.random.default_rng(31)
    B, D, L = 6, 8, 3
    rows = [11, 9]
    finite = codes[(codes & 0x7F) != 0x7F]
    tables = [rng.choice(finite, size=(r, D)).astype(np.uint8) for r in rows]
    idx = [rng.integers(0, r, B * L).astype(np.int32) for r in rows]
    wts = [rng.standard_normal(B * L).astype(np.float32) for _ in rows]
    scales = np.array([0.25, 3.0], np.float32)
    offs = torch.arange(0, B * L, L)
    dec = [torch.from_numpy(oracle.fp8_e4m3_to_f64(t, lib=lib)) for t in tables]
    for pool, w in (("sum", None), ("mean", None), ("sum", wts)):
        got = oracle.emb_bag(tables, idx, batch=B, weights=w, pool=pool, scales=scales, lib=lib)
        for k in range(2):
            psw = torch.from_numpy(w[k].astype(np.float64)) if w is not None else None
            want = F.embedding_bag(torch.from_numpy(idx[k].astype(np.int64)), dec[k], offs,
                                   mode=pool, per_sample_weights=psw).numpy() * float(scales[k])
            np.testing.assert_allclose(got[:, k], want, rtol=1e-6, atol=1e-6)
    # a power-of-two scale multiplies the pooled value exactly
    plain = oracle.emb_bag(tables, idx, batch=B, lib=lib)
    scaled = oracle.emb_bag(tables, idx, batch=B, scales=np.array([0.5, 4.0], np.float32),
                            lib=lib)
    assert np.array_equal(scaled, plain * np.array([0.5, 4.0], np.float32)[None, :, None])


# ------------------------------------------------------------- interaction --
def pin_interact(lib):
    rng = np.random.default_rng(12)
    for B, K, D in ((3, 1, 4), (4, 4, 8), (2, 8, 3), (5, 32, 16)):
        dense = rng.standard_normal((B, D)).astype(np.float32)
        emb = rng.standard_normal((B, K, D)).astype(np.float32)
        out = oracle.interact(dense, emb, lib=lib)
        F = K + 1
        assert out.shape == (B, D + F * (F - 1) // 2)
        # dense columns are a bit-exact copy
        assert np.array_equal(out[:, :D], dense)
        # library routine: float64 Gram matrix then numpy.tril_indices
        X = np.concatenate([dense[:, None, :], emb], axis=1).astype(np.float64)
        Z = X @ X.transpose(0, 2, 1)
        li, lj = np.tril_indices(F, -1)
        np.testing.assert_allclose(out[:, D:], Z[:, li, lj], rtol=1e-6, atol=1e-6)
        # torch bmm on the stacked features, the pages' own formulation
        import torch
        T = torch.from_numpy(X)
        Zt = torch.bmm(T, T.transpose(1, 2).contiguous())
        ti, tj = torch.tril_indices(F, F, -1)
        np.testing.assert_allclose(out[:, D:], Zt[:, ti, tj].numpy(),
                                   rtol=1e-6, atol=1e-6)
    # F = 2: the single dot of dense and the one pooled vector
    d = rng.standard_normal((1, 6)).astype(np.float32)
    e = rng.standard_normal((1, 1, 6)).astype(np.float32)
    got = oracle.interact(d, e, lib=lib)
    assert got.shape == (1, 7)
    want = np.float32(np.dot(d[0].astype(np.float64), e[0, 0].astype(np.float64)))
    assert got[0, 6] == want
    # symmetric pair sums: swapping which pooled vector is which permutes the
    # dots accordingly (pair (2,1) is invariant, (1,0) and (2,0) swap)
    d = rng.standard_normal((1, 5)).astype(np.float32)
    e = rng.standard_normal((1, 2, 5)).astype(np.float32)
    a = oracle.interact(d, e, lib=lib)[0, 5:]
    b = oracle.interact(d, e[:, ::-1, :].copy(), lib=lib)[0, 5:]
    assert a[0] == b[1] and a[1] == b[0] and a[2] == b[2]
    # hand-worked F = 3 example
    g = _golden("interact_f3.json")
    got = oracle.interact(np.array(g["dense"], np.float32),
                          np.array(g["emb"], np.float32), lib=lib)
    assert np.array_equal(got, np.array(g["expected"], np.float32))


# ------------------------------------------------------------------ linear --
def pin_linear(lib):
    rng = np.random.default_rng(13)
    for M, N, K in ((7, 5, 3), (3, 9, 13), (16, 1, 33)):
        a = rng.standard_normal((M, K)).astype(np.float32)
        w = rng.standard_normal((N, K)).astype(np.float32)
        b = rng.standard_normal(N).astype(np.float32)
        ref = a.astype(np.float64) @ w.astype(np.float64).T + b
        np.testing.assert_allclose(oracle.linear(a, w, b, "none", lib=lib), ref,
                                   rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(oracle.linear(a, w, b, "relu", lib=lib),
                                   np.maximum(ref, 0), rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(oracle.linear(a, w, b, "sigmoid", lib=lib),
                                   1 / (1 + np.exp(-ref)), rtol=1e-6, atol=1e-7)
        # no bias is a zero bias
        np.testing.assert_allclose(oracle.linear(a, w, None, lib=lib),
                                   ref - b, rtol=1e-6, atol=1e-6)
    # identity weight passes the input through the activation
    x = rng.standard_normal((4, 6)).astype(np.float32)
    eye = np.eye(6, dtype=np.float32)
    assert np.array_equal(oracle.linear(x, eye, None, "none", lib=lib), x)
    assert np.array_equal(oracle.linear(x, eye, None, "relu", lib=lib),
                          np.where(x > 0, x, 0).astype(np.float32))
    # zero weight leaves act(bias); sigmoid(0) is exactly one half
    bias = np.array([0.0, -2.0, 3.0], np.float32)
    z = oracle.linear(x, np.zeros((3, 6), np.float32), bias, "none", lib=lib)
    assert np.array_equal(z, np.tile(bias, (4, 1)))
    s = oracle.linear(x, np.zeros((3, 6), np.float32), None, "sigmoid", lib=lib)
    assert np.all(s == np.float32(0.5))
    # saturation stays finite and ordered
    big = np.array([[100.0], [-100.0]], np.float32)
    s = oracle.linear(big, np.ones((1, 1), np.float32), None, "sigmoid", lib=lib)
    assert s[0, 0] == 1.0 and 0.0 <= s[1, 0] < 1e-40
    # hand-worked case
    g = _golden("linear_2x3.json")
    a = np.array(g["a"], np.float32)
    w = np.array(g["w"], np.float32)
    b = np.array(g["bias"], np.float32)
    assert np.array_equal(oracle.linear(a, w, b, "none", lib=lib),
                          np.array(g["expected_none"], np.float32))
    assert np.array_equal(oracle.linear(a, w, b, "relu", lib=lib),
                          np.array(g["expected_relu"], np.float32))


# ----------------------------------------------------------------- forward --
def torch_dlrm_reference(dense_in, bottom, top, tables, indices, batch, bag):
    """DLRMv1 as torch CPU float64 modules: one nn.EmbeddingBag(sum) per table,
    cat + bmm + tril_indices interaction, nn.Linear layers."""
    import torch
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    x = t(dense_in)
    for w, b, act in bottom:
        x = torch.nn.functional.linear(x, t(w), t(b))
        x = torch.relu(x) if act == "relu" else torch.sigmoid(x)
    ly = []
    for tab, idx in zip(tables, indices):
        eb = torch.nn.EmbeddingBag.from_pretrained(t(tab), mode="sum", freeze=True)
        ly.append(eb(torch.from_numpy(idx.astype(np.int64)),
                     torch.arange(0, batch * bag, bag)))
    T = torch.cat([x.unsqueeze(1)] + [e.unsqueeze(1) for e in ly], dim=1)
    Z = torch.bmm(T, T.transpose(1, 2).contiguous())
    F = T.shape[1]
    li, lj = torch.tril_indices(F, F, -1)
    R = torch.cat([x, Z[:, li, lj]], dim=1)
    y = R
    for w, b, act in top:
        y = torch.nn.functional.linear(y, t(w), t(b))
        y = torch.relu(y) if act == "relu" else torch.sigmoid(y)
    return y.numpy(), R.numpy()


def pin_forward(lib):
    from dlrm_embedding_bag_amd import inputs
    w = inputs.Workload("pin", batch=16, num_tables=4, rows=50, dim=8, bag=3,
                        dist="zipf", dense_in=5, bottom=(12, 8), top=(10, 1))
    tables = [inputs.table_host(w, k, 5) for k in range(w.num_tables)]
    idx = [inputs.indices(w, k, 5) for k in range(w.num_tables)]
    dense_in = inputs.dense(w, 5)
    bottom, top = inputs.dlrm_layers(w, 5, bias_std=0.1)
    out, R, E = oracle.forward(dense_in, bottom, top, tables, idx, lib=lib)
    ref_out, ref_R = torch_dlrm_reference(dense_in, bottom, top, tables, idx,
                                          w.batch, w.bag)
    assert out.shape == (16, 1) and R.shape == (16, 8 + 10)
    np.testing.assert_allclose(R, ref_R, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(out, ref_out, rtol=1e-5, atol=1e-6)
    # the composition equals its parts
    offs = [inputs.offsets(w) for _ in range(w.num_tables)]
    out2, R2, E2 = oracle.forward(dense_in, bottom, top, tables, idx, offs, lib=lib)
    assert np.array_equal(out, out2) and np.array_equal(R, R2) and np.array_equal(E, E2)
    assert np.array_equal(E, oracle.emb_bag_sum(tables, idx, batch=w.batch, lib=lib))


ALL_PINS = (pin_pair_map, pin_emb_bag, pin_emb_bag_ext, pin_emb_bag_fp8, pin_interact,
            pin_linear, pin_forward)
