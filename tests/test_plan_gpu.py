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


def _model(w, seed=0, options=()):
    tables = [inputs.table_host(w, k, seed) for k in range(w.num_tables)]
    bottom, top = inputs.dlrm_layers(w, seed, bias_std=0.1)
    model = abi.DlrmModel([(dev(a), dev(b), act) for a, b, act in bottom],
                          [(dev(a), dev(b), act) for a, b, act in top],
                          [dev(t) for t in tables], options=options)
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
def test_plan_on_a_side_stream_and_update(mode, layered):
    """A plan replays on a caller stream; update() rebinds other buffers,
    including CSR offsets (another gather kernel: a graph is rebuilt)."""
    import torch
    w = inputs.cell_workload(16, 300)
    model, tables, bottom, top = _model(w, seed=3, options=("layered",) if layered else ())
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
    # new indices alone keep the CSR offsets bound
    idx4 = [rng.integers(0, w.rows, int(l.sum())).astype(np.int32) for l in lens]
    i4 = [dev(i) for i in idx4]
    plan.update(indices=i4)
    got = host(plan.run())
    assert np.array_equal(got, host(abi.dlrm_forward(model, d2, i4, offsets=o3)))
    # offsets=None explicitly returns to uniform-stride bags
    plan.update(indices=i2, offsets=None)
    assert np.array_equal(host(plan.run()), host(abi.dlrm_forward(model, d2, i2)))
    plan.close()
    plan.close()                                    # closing twice is harmless


def test_plan_update_with_mismatched_bags_keeps_the_plan():
    """A rejected update (uniform indices whose count is no multiple of the
    batch) leaves the plan bound to its previous buffers."""
    w = inputs.cell_workload(4, 50)
    model, _, _, _ = _model(w, seed=1)
    dense, idx = _batch(w, 1)
    d, x = dev(dense), [dev(i) for i in idx]
    plan = abi.DlrmPlan(model, d, x)
    want = host(plan.run())
    with pytest.raises(abi.DlrmError) as e:
        plan.update(indices=[i[:-1] for i in x])
    assert e.value.name == "DLRM_ERR_SHAPE"
    assert np.array_equal(host(plan.run()), want)
    plan.close()


def test_forward_on_a_side_stream_allocates_there():
    """dlrm_forward with a caller stream and no workspace: its temporaries
    belong to that stream, and the result equals the current-stream call."""
    import torch
    w = inputs.Workload("side", batch=700, num_tables=8, rows=3000, dim=64, bag=6,
                        dist="zipf", dense_in=13, bottom=(512, 256, 64), top=(512, 256, 1))
    model, _, _, _ = _model(w, seed=2)
    dense, idx = _batch(w, 2)
    d, x = dev(dense), [dev(i) for i in idx]
    want = host(abi.dlrm_forward(model, d, x))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        outs.append(abi.dlrm_forward(model, d, x, stream=side))
        # other work on the current stream in between, allocating and freeing
        junk = torch.ones(1 << 22, device="cuda") * 3.0
        del junk
    side.synchronize()
    for o in outs:
        assert np.array_equal(host(o), want)


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
