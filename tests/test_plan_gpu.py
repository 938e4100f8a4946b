"""GPU tests of plans (dlrm_plan_*): the forward recorded into a HIP graph
and replayed.  A replay runs the same kernels as dlrm_forward on the same
buffers, so every replay must equal the eager forward bit for bit; eager
work, other launches and synchronizations run between the replays, and new
inputs are written into the bound buffers between them."""
import numpy as np
import pytest

import oracle
from conftest import gpu_available
from gpu_helpers import assert_close, dev, host
from dlrm_embedding_bag_amd import abi, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _model(w, seed=0):
    tables = [inputs.table_host(w, k, seed) for k in range(w.num_tables)]
    bottom, top = inputs.dlrm_layers(w, seed, bias_std=0.1)
    model = abi.DlrmModel([(dev(a), dev(b), act) for a, b, act in bottom],
                          [(dev(a), dev(b), act) for a, b, act in top],
                          [dev(t) for t in tables])
    return model, tables, bottom, top


def _batch(w, seed):
    idx = [inputs.indices(w, k, seed) for k in range(w.num_tables)]
    return inputs.dense(w, seed), idx


CASES = [inputs.cell_workload(2, 2), inputs.cell_workload(32, 2048),
         inputs.cell_workload(8, 100),
         inputs.Workload("mid-fwd", batch=1000, num_tables=26, rows=5000, dim=64, bag=20,
                         dist="zipf", dense_in=13, bottom=(512, 256, 64), top=(512, 256, 1))]


@pytest.mark.parametrize("mode", ["direct", "graph"])
@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_plan_replays_equal_eager_forward(w, mode):
    import torch
    model, tables, bottom, top = _model(w)
    dense0, idx0 = _batch(w, 0)
    dense_buf = dev(dense0)
    idx_buf = [dev(i) for i in idx0]
    plan = abi.DlrmPlan(model, dense_buf, idx_buf, mode=mode)
    # the first replay against the oracle
    got = host(plan.run())
    want, _, _ = oracle.forward(dense0, bottom, top, tables, idx0)
    assert_close(got, want, f"{w.name} plan vs oracle")
    noise = torch.randn(1 << 20, device="cuda")
    for it in range(1, 5):
        dense, idx = _batch(w, it)
        dense_buf.copy_(dev(dense))                 # new batch into the bound buffers
        for b, i in zip(idx_buf, idx):
            b.copy_(dev(i))
        eager = host(abi.dlrm_forward(model, dev(dense), [dev(i) for i in idx]))
        (noise * 2).sum()                           # unrelated eager work in between
        torch.cuda.synchronize()
        got = host(plan.run())
        assert np.array_equal(got, eager), f"replay {it}"
    plan.close()


@pytest.mark.parametrize("mode", ["direct", "graph"])
@pytest.mark.parametrize("layered", [False, True])
def test_plan_on_a_side_stream_and_update(mode, layered, monkeypatch):
    """A plan replays on a caller stream; update() rebinds other buffers,
    including CSR offsets (another gather kernel: a graph is rebuilt)."""
    import torch
    if layered:
        monkeypatch.setenv("DLRM_FORWARD_LAYERED", "1")
    w = inputs.cell_workload(16, 300)
    model, tables, bottom, top = _model(w, seed=3)
    dense, idx = _batch(w, 1)
    plan = abi.DlrmPlan(model, dev(dense), [dev(i) for i in idx], mode=mode)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        out = plan.run(stream=side)
    side.synchronize()
    assert np.array_equal(host(out), host(abi.dlrm_forward(model, dev(dense),
                                                           [dev(i) for i in idx])))
    # rebind to other buffers, same shapes
    dense2, idx2 = _batch(w, 2)
    d2, i2 = dev(dense2), [dev(i) for i in idx2]
    plan.update(dense_in=d2, indices=i2)
    got = host(plan.run())
    assert np.array_equal(got, host(abi.dlrm_forward(model, d2, i2)))
    # CSR bags of any size: the gather switches to its CSR kernel
    rng = np.random.default_rng(5)
    lens = rng.integers(0, 5, size=(w.num_tables, w.batch))
    offs = [np.concatenate([[0], np.cumsum(l)[:-1]]).astype(np.int32) for l in lens]
    idx3 = [rng.integers(0, w.rows, int(l.sum())).astype(np.int32) for l in lens]
    i3, o3 = [dev(i) for i in idx3], [dev(o) for o in offs]
    plan.update(indices=i3, offsets=o3)
    for _ in range(3):
        got = host(plan.run())
        assert np.array_equal(got, host(abi.dlrm_forward(model, d2, i3, offsets=o3)))
    want, _, _ = oracle.forward(dense2, bottom, top, tables, idx3, offs)
    assert_close(got, want, "plan CSR vs oracle")
    plan.close()
    plan.close()                                    # closing twice is harmless


def test_plan_rejects_bad_arguments():
    import torch
    w = inputs.cell_workload(4, 8)
    model, _, _, _ = _model(w)
    dense, idx = _batch(w, 0)
    with pytest.raises(abi.DlrmError) as e:
        abi.DlrmPlan(model, dev(dense), [dev(i) for i in idx][:-1] + [dev(idx[-1][:-1])])
    assert e.value.name == "DLRM_ERR_SHAPE"
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    for mode in ("direct", "graph"):
        with pytest.raises(abi.DlrmError) as e:
            abi.DlrmPlan(model, dev(dense), [dev(i) for i in idx], workspace=small, mode=mode)
        assert e.value.name == "DLRM_ERR_WORKSPACE"
