"""GPU parity of the general EmbeddingBag forms (emb_bag_pool and
dlrm_emb_interact_pool): bfloat16 and FP8 E4M3 tables with per-table scales,
mean pooling, per-sample weights, CSR bags of any size, against the CPU oracle
on the same seeded inputs.

Sums and weighted sums of dyadic values are exact in any order, so they are
compared bit for bit (bfloat16 holds these dyadic values exactly, and the fp8
cases draw codes whose sums stay exact); mean
pooling divides once more and is held to |gpu - oracle| <= 1e-5 + 1e-5
|oracle|, as are the random-valued cases.  The small cases span several
workgroups, ragged batches and every row-chunk path (16-byte shuffle groups
of 4..64 lanes, the generic vector path, the scalar path)."""
import numpy as np
import pytest

import oracle
from conftest import gpu_available
from gpu_helpers import assert_close, dev, host, sample_rows, sampled_bags
from dlrm_embedding_bag_amd import abi, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _bf16_dev(bits):
    import torch
    return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)


def _fp8_dev(codes):
    import torch
    return torch.from_numpy(codes).cuda().view(torch.float8_e4m3fn)


# E4M3 codes with exponent field 4..11: values 2^-3 .. 30, multiples of 2^-6.
# With weights n/256 (|n| < 16) and up to ~60 terms every partial sum stays
# below 2^24 units of 2^-14, so sums and weighted sums are exact in float32.
_EXACT_FP8 = np.array([c for c in range(256) if 4 <= ((c >> 3) & 15) <= 11], np.uint8)


def _case(B, K, rows, D, L, dtype, csr, weighted, seed, dyadic=True):
    """Host tables (float32 or uint16 bf16 bits), indices, offsets, weights."""
    rng = np.random.default_rng(seed)
    m = inputs.dyadic_max_int(D, L)
    tables, idx, offs, wts = [], [], [], []
    for k in range(K):
        if dtype == "fp8":
            if dyadic:
                tables.append(rng.choice(_EXACT_FP8, size=(rows, D)))
            else:   # the workloads' tables: N(0, 0.01^2) encoded at scale 2^-8
                tables.append(inputs.fp8_codes(rng.standard_normal((rows, D)) * 0.01))
        else:
            if dyadic:
                t = inputs.dyadic(rng, (rows, D), max_int=m)
            else:
                t = (rng.standard_normal((rows, D)) * 0.1).astype(np.float32)
            tables.append(inputs.bf16_bits(t) if dtype == "bf16" else t)
        if csr:
            lens = rng.integers(0, 2 * L + 1, size=B)
            lens[0] = 0                       # an empty first bag
            if B > 2:
                lens[B // 2] = 3 * L + 5      # one long bag
            o = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
            n = int(lens.sum())
            offs.append(o)
        else:
            n = B * L
        idx.append(rng.integers(0, rows, size=n).astype(np.int32))
        if weighted:
            wts.append(inputs.dyadic(rng, n, max_int=16) if dyadic
                       else rng.random(n, dtype=np.float32))
    return tables, idx, (offs if csr else None), (wts if weighted else None)


def _dev_tables(tables):
    return [_bf16_dev(t) if t.dtype == np.uint16 else _fp8_dev(t) if t.dtype == np.uint8
            else dev(t) for t in tables]


def _scales(dtype, K):
    """Per-table scales for fp8 tables: powers of two, so scaling is exact."""
    return [2.0 ** (-(k % 5) - 4) for k in range(K)] if dtype == "fp8" else None


def _gpu_pool(tables, idx, offs, wts, pool, B, scales=None):
    return host(abi.emb_bag_pool(
        _dev_tables(tables), [dev(i) for i in idx],
        offsets=[dev(o) for o in offs] if offs is not None else None,
        weights=[dev(w) for w in wts] if wts is not None else None, pool=pool, batch=B,
        scales=scales))


POOL_SHAPES = [  # (B, K, rows, D, L)
    (37, 5, 333, 64, 7),      # bf16: 8 lanes per row; f32: 16
    (130, 3, 50, 16, 20),     # bf16: 2 chunks per row (generic vector path)
    (9, 4, 30, 8, 3),         # bf16: one chunk per row
    (11, 3, 40, 12, 5),       # bf16 scalar path (D % 8 != 0); f32 vector path
    (7, 2, 20, 7, 4),         # scalar path for both
    (6, 2, 20, 256, 9),       # bf16: 32 lanes; f32: a full wave
    (3, 2, 10, 1024, 3),      # bf16: 128 chunks, 64 lanes
    (4, 3, 25, 24, 2),        # bf16: 3 chunks per row
    (5, 64, 10, 32, 1),       # maximum K; fp8: 2 chunks per row
    (8, 3, 40, 48, 6),        # fp8: 3 chunks per row (generic vector path)
    (6, 2, 30, 128, 4),       # fp8: 8 lanes per row
]
FORMS = [  # (dtype, pool, weighted)
    ("f32", "sum", False), ("f32", "mean", False), ("f32", "sum", True),
    ("bf16", "sum", False), ("bf16", "mean", False), ("bf16", "sum", True),
    ("fp8", "sum", False), ("fp8", "mean", False), ("fp8", "sum", True),
]


@pytest.mark.parametrize("dtype,pool,weighted", FORMS)
@pytest.mark.parametrize("csr", [False, True])
@pytest.mark.parametrize("B,K,rows,D,L", POOL_SHAPES)
def test_pool_forms(B, K, rows, D, L, dtype, pool, weighted, csr):
    tables, idx, offs, wts = _case(B, K, rows, D, L, dtype, csr, weighted,
                                   seed=B * 31 + K + D)
    sc = _scales(dtype, K)
    want = oracle.emb_bag(tables, idx, offs, batch=B, weights=wts, pool=pool, scales=sc)
    got = _gpu_pool(tables, idx, offs, wts, pool, B, scales=sc)
    if pool == "sum":
        assert np.array_equal(got, want), "dyadic sums are exact in any order"
    else:
        assert_close(got, want, f"{dtype} mean")
    if csr:
        assert np.all(got[0] == 0), "the empty first bag pools to zero"


@pytest.mark.parametrize("dtype,pool,weighted", FORMS)
def test_pool_forms_random_values(dtype, pool, weighted):
    B, K, rows, D, L = 257, 6, 5000, 64, 20
    tables, idx, offs, wts = _case(B, K, rows, D, L, dtype, True, weighted, seed=5,
                                   dyadic=False)
    sc = [0.3 + 0.1 * k for k in range(K)]          # any per-table scale, any storage
    want = oracle.emb_bag(tables, idx, offs, batch=B, weights=wts, pool=pool, scales=sc)
    got = _gpu_pool(tables, idx, offs, wts, pool, B, scales=sc)
    assert_close(got, want, f"{dtype} {pool} weighted={weighted} scaled")


def test_f32_sum_form_is_emb_bag_sum_multi():
    """emb_bag_pool with float32 sum bags runs the same kernel as
    emb_bag_sum_multi: bit for bit equal on random values."""
    tables, idx, offs, _ = _case(100, 4, 900, 64, 11, "f32", False, False, 7, dyadic=False)
    td = [dev(t) for t in tables]
    xd = [dev(i) for i in idx]
    a = host(abi.emb_bag_pool(td, xd, batch=100))
    b = host(abi.emb_bag_sum_multi(td, xd, batch=100))
    assert np.array_equal(a, b)


def test_unit_weights_equal_sum_and_uniform_mean_is_scaled_sum():
    """Weights of one give the plain sum bit for bit (fma(1, v, a) = a + v);
    the mean of power-of-two bags is the sum times 1/L exactly."""
    import torch
    B, K, rows, D, L = 64, 3, 400, 64, 8
    tables, idx, _, _ = _case(B, K, rows, D, L, "bf16", False, False, 11, dyadic=False)
    td = _dev_tables(tables)
    xd = [dev(i) for i in idx]
    ones = [torch.ones(B * L, device="cuda") for _ in range(K)]
    s = host(abi.emb_bag_pool(td, xd, batch=B))
    assert np.array_equal(host(abi.emb_bag_pool(td, xd, weights=ones, batch=B)), s)
    m = host(abi.emb_bag_pool(td, xd, pool="mean", batch=B))
    assert np.array_equal(m, s / np.float32(L))


def test_mean_of_empty_csr_bags_is_zero():
    import torch
    t = dev(np.ones((4, 16), np.float32))
    x = torch.zeros(3, dtype=torch.int32, device="cuda")
    o = dev(np.array([0, 0, 3, 3], np.int32))          # bags: {}, {0,0,0}, {}, {}
    got = host(abi.emb_bag_pool([t], [x], offsets=[o], pool="mean"))
    assert np.array_equal(got[:, 0, 0], np.array([0, 1, 0, 0], np.float32))


def test_weights_with_mean_rejected():
    import torch
    t = dev(np.ones((4, 16), np.float32))
    x = torch.zeros(8, dtype=torch.int32, device="cuda")
    with pytest.raises(abi.DlrmError) as e:
        abi.emb_bag_pool([t], [x], weights=[torch.ones(8, device="cuda")], pool="mean",
                         batch=2)
    assert e.value.name == "DLRM_ERR_UNSUPPORTED"


FUSED_SHAPES = [  # (B, K, rows, D, L)
    (37, 5, 333, 64, 7), (19, 26, 100, 64, 4), (9, 8, 50, 12, 3), (5, 3, 40, 7, 2),
    (3, 4, 30, 128, 5), (66, 32, 200, 64, 20),
]


@pytest.mark.parametrize("dtype,pool,weighted", FORMS)
@pytest.mark.parametrize("B,K,rows,D,L", FUSED_SHAPES)
def test_fused_pool_forms(B, K, rows, D, L, dtype, pool, weighted):
    """dlrm_emb_interact_pool against oracle.interact(dense, oracle.emb_bag(...));
    the pooled copy in emb_out against oracle.emb_bag."""
    import torch
    tables, idx, offs, wts = _case(B, K, rows, D, L, dtype, True, weighted, seed=B + 7 * K,
                                   dyadic=False)
    dense = np.random.default_rng(B).standard_normal((B, D)).astype(np.float32)
    sc = [2.0 ** -6] * K if dtype == "fp8" else None
    E = oracle.emb_bag(tables, idx, offs, weights=wts, pool=pool, scales=sc)
    want = oracle.interact(dense, E)
    emb_out = torch.empty((B, K, D), device="cuda")
    got = host(abi.dlrm_emb_interact_pool(
        _dev_tables(tables), [dev(i) for i in idx], dev(dense),
        offsets=[dev(o) for o in offs], weights=[dev(w) for w in wts] if wts else None,
        pool=pool, emb_out=emb_out, scales=sc))
    assert_close(got, want, f"fused {dtype} {pool}")
    assert np.array_equal(got[:, :D], dense)
    assert_close(host(emb_out), E, "pooled copy")


LONG_SHAPES = [  # (B, K, rows, D, L) with L x D >= 4096 pooled elements per bag
    (37, 5, 333, 128, 40),    # f32: 32 lanes per row; bf16 16; fp8 8
    (9, 3, 100, 64, 70),      # 4480 elements, 64-wide rows
    (5, 2, 50, 256, 20),      # a full wave per f32 row
    (3, 26, 200, 128, 33),    # many tables, ragged workgroup tail
]


@pytest.mark.parametrize("dtype,pool,weighted", FORMS)
@pytest.mark.parametrize("B,K,rows,D,L", LONG_SHAPES)
def test_long_bags_two_launch_route(B, K, rows, D, L, dtype, pool, weighted):
    """Long bags with emb_out given run as two launches (the gather into
    emb_out, then the interaction reading it).  out must equal the one-launch
    result (emb_out NULL) bit for bit, for both the [dense, dots] and the
    dots-only layouts, and both must match the oracle."""
    import torch
    tables, idx, offs, wts = _case(B, K, rows, D, L, dtype, False, weighted, seed=B + 3 * K,
                                   dyadic=False)
    dense = np.random.default_rng(B + 1).standard_normal((B, D)).astype(np.float32)
    sc = [2.0 ** -6] * K if dtype == "fp8" else None
    td = _dev_tables(tables)
    xd = [dev(i) for i in idx]
    wd = [dev(w) for w in wts] if wts else None
    dd = dev(dense)
    E = oracle.emb_bag(tables, idx, None, batch=B, weights=wts, pool=pool, scales=sc)
    want = oracle.interact(dense, E)
    emb_out = torch.full((B, K, D), float("nan"), device="cuda")
    two = host(abi.dlrm_emb_interact_pool(td, xd, dd, weights=wd, pool=pool, emb_out=emb_out,
                                          scales=sc))
    one = host(abi.dlrm_emb_interact_pool(td, xd, dd, weights=wd, pool=pool, scales=sc))
    assert np.array_equal(two, one), "the two-launch route must match the fused launch"
    assert_close(two, want, f"two-launch {dtype} {pool}")
    assert_close(host(emb_out), E, "pooled copy")
    emb_out.fill_(float("nan"))
    d_two = host(abi.dlrm_emb_interact_dots(td, xd, dd, weights=wd, pool=pool, emb_out=emb_out,
                                            scales=sc))
    d_one = host(abi.dlrm_emb_interact_dots(td, xd, dd, weights=wd, pool=pool, scales=sc))
    assert np.array_equal(d_two, d_one)
    assert np.array_equal(d_two, two[:, D:])
    assert_close(host(emb_out), E, "pooled copy (dots layout)")


def test_long_csr_bags_two_launch_route():
    """CSR bags (sizes 0..2L, one empty, one long) whose mean is long enough
    for the two-launch route."""
    import torch
    B, K, rows, D, L = 41, 4, 300, 128, 60
    tables, idx, offs, wts = _case(B, K, rows, D, L, "f32", True, True, seed=99, dyadic=False)
    assert sum(i.shape[0] for i in idx) * D >= 4096 * B * K
    dense = np.random.default_rng(3).standard_normal((B, D)).astype(np.float32)
    args = ([dev(t) for t in tables], [dev(i) for i in idx], dev(dense))
    kw = dict(offsets=[dev(o) for o in offs], weights=[dev(w) for w in wts])
    emb_out = torch.empty((B, K, D), device="cuda")
    two = host(abi.dlrm_emb_interact_pool(*args, emb_out=emb_out, **kw))
    one = host(abi.dlrm_emb_interact_pool(*args, **kw))
    assert np.array_equal(two, one)
    E = oracle.emb_bag(tables, idx, offs, weights=wts)
    assert_close(two, oracle.interact(dense, E), "two-launch csr")
    assert_close(host(emb_out), E, "pooled copy")


# ------------------------------------------------------------- full size --
def _full_inputs(w):
    tables = [inputs.table_device_typed(w, k) for k in range(w.num_tables)]
    idx = [inputs.indices(w, k) for k in range(w.num_tables)]
    offs = ([inputs.csr_offsets(w, k) for k in range(w.num_tables)]
            if w.lengths != "fixed" else None)
    wts = ([inputs.sample_weights(w, k, idx[k].shape[0]) for k in range(w.num_tables)]
           if w.weighted else None)
    return tables, idx, offs, wts


@pytest.mark.parametrize("name", ["nc32-bf16", "nc32-fp8", "nc32-mean", "nc32-weighted",
                                  "nc32-csr"])
def test_full_size_variants_sampled(name):
    """The benchmark's fused launch of each variant workload on the full batch
    (B=2048, K=32 tables x 1,000,000 rows x D=64); sampled rows vs the oracle,
    the dense columns exact on every row."""
    import torch
    w = inputs.WORKLOADS[name]
    print(f"\n[{name}] {w.description}", flush=True)
    tables, idx, offs, wts = _full_inputs(w)
    dense = inputs.dense(w)
    out = torch.empty((w.batch, w.out_width), device="cuda")
    sc = [inputs.table_scale(w)] * w.num_tables if inputs.table_scale(w) else None
    abi.dlrm_emb_interact_pool(
        tables, [dev(i) for i in idx], dev(dense),
        offsets=[dev(o) for o in offs] if offs is not None else None,
        weights=[dev(x) for x in wts] if wts is not None else None, pool=w.pool, out=out,
        scales=sc)
    got = host(out)
    assert np.all(np.isfinite(got))
    assert np.array_equal(got[:, :w.dim], dense)
    samples = sample_rows(w.batch, 48, seed=len(name))
    st, si, so, sw = sampled_bags(tables, idx, samples, bag=w.bag, offsets_host=offs,
                                  weights_host=wts)
    want = oracle.interact(dense[samples],
                           oracle.emb_bag(st, si, so, weights=sw, pool=w.pool, scales=sc))
    assert_close(got[samples], want, f"{name} sampled")
    del tables, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
