"""GPU test of dlrm_forward_noalloc, the forward whose workspace is the
library's fixed per-GPU scratch array: called through the C ABI, its output
must equal dlrm_forward's (same kernels, same launch shapes, caller
workspace) on two calls in a row, the second with a smaller batch, and
stay within the float bar of the CPU oracle; a forward whose workspace would
exceed the array is refused before any work is enqueued.  Collected last, so
that it also runs after every other GPU test in the same process."""
import numpy as np
import pytest

import oracle
from conftest import gpu_available
from gpu_helpers import assert_close, dev, host, make_uniform_case
from dlrm_embedding_bag_amd import abi, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _model(w, seed, options=()):
    tables, _, _ = make_uniform_case(w, seed)
    bottom, top = inputs.dlrm_layers(w, seed, bias_std=0.1)
    model = abi.DlrmModel([(dev(a), dev(b), act) for a, b, act in bottom],
                          [(dev(a), dev(b), act) for a, b, act in top],
                          [dev(t) for t in tables], options=options)
    return model, tables, bottom, top


def _batch(w, batch, seed):
    import dataclasses
    wb = dataclasses.replace(w, batch=batch)
    idx = [inputs.indices(wb, k, seed) for k in range(w.num_tables)]
    return inputs.dense(wb, seed), idx


@pytest.mark.parametrize("options", [(), ("unfused_head",)])
def test_noalloc_forward_equals_workspace_forward_twice(options):
    import torch
    w = inputs.Workload("noalloc", batch=4096, num_tables=26, rows=20000, dim=64, bag=20,
                        dist="zipf", dense_in=13, bottom=(512, 256, 64), top=(512, 256, 1))
    model, tables, bottom, top = _model(w, seed=11, options=options)
    # the first call fills most of the scratch array, the second a smaller part
    for batch, seed in ((4096, 1), (1000, 2)):
        dense, idx = _batch(w, batch, seed)
        d, x = dev(dense), [dev(i) for i in idx]
        want = host(abi.dlrm_forward(model, d, x))
        out = torch.full((batch, 1), float("nan"), device="cuda")
        got = host(abi.dlrm_forward_noalloc(model, d, x, out))
        assert np.array_equal(got, want), f"batch {batch}"
        assert_close(got, want, f"noalloc vs dlrm_forward, batch {batch}")
    # the oracle on the last (smaller) batch
    ref, _, _ = oracle.forward(dense, bottom, top, tables, idx)
    assert_close(got, ref, "noalloc vs oracle")


def test_noalloc_small_model_and_csr_bags():
    """A small model (the one-launch forward, no scratch) and CSR bags."""
    import torch
    w = inputs.cell_workload(8, 300)
    model, tables, bottom, top = _model(w, seed=3)
    rng = np.random.default_rng(4)
    lens = rng.integers(0, 5, size=(w.num_tables, w.batch))
    offs = [np.concatenate([[0], np.cumsum(l)[:-1]]).astype(np.int32) for l in lens]
    idx = [rng.integers(0, w.rows, int(l.sum())).astype(np.int32) for l in lens]
    dense = inputs.dense(w, 4)
    d, x, o = dev(dense), [dev(i) for i in idx], [dev(v) for v in offs]
    out = torch.empty((w.batch, 1), device="cuda")
    got = host(abi.dlrm_forward_noalloc(model, d, x, out, offsets=o))
    assert np.array_equal(got, host(abi.dlrm_forward(model, d, x, offsets=o)))
    want, _, _ = oracle.forward(dense, bottom, top, tables, idx, offs)
    assert_close(got, want, "noalloc small model, CSR")


def test_noalloc_refuses_a_workspace_beyond_the_array():
    import torch
    w = inputs.Workload("noalloc-big", batch=16384, num_tables=26, rows=2000, dim=64, bag=1,
                        dist="uniform", dense_in=13, bottom=(512, 256, 64), top=(512, 256, 1))
    model, _, _, _ = _model(w, seed=5)
    assert model.workspace_bytes(16384) > abi.NOALLOC_SCRATCH_BYTES
    dense, idx = _batch(w, 16384, 5)
    out = torch.full((16384, 1), -1.0, device="cuda")
    with pytest.raises(abi.DlrmError) as e:
        abi.dlrm_forward_noalloc(model, dev(dense), [dev(i) for i in idx], out)
    assert e.value.name == "DLRM_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert np.all(host(out) == -1.0), "a refused call enqueues nothing"
    # the largest batch that fits still runs
    assert model.workspace_bytes(8192) <= abi.NOALLOC_SCRATCH_BYTES
