"""GPU tests of the kernel timing hook (dlrm_set_kernel_timing_events): a
launch with timing on gives the same output bit for bit as one without, the
events hold a positive kernel time, and a graph-mode plan created while
timing is on still replays the eager forward."""
import numpy as np
import pytest

import oracle
from conftest import gpu_available
from gpu_helpers import assert_close, dev, host, make_uniform_case
from dlrm_embedding_bag_amd import abi, inputs

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")]


def _timer(n):
    import bench
    return bench.KernelTimer(n)


def test_timed_fused_launch_matches_untimed():
    import torch
    w = inputs.Workload("timing", batch=300, num_tables=8, rows=2000, dim=64, bag=20,
                        dist="zipf")
    tables, idx, dense = make_uniform_case(w)
    td, xd, dd = [dev(t) for t in tables], [dev(i) for i in idx], dev(dense)
    plain = host(abi.dlrm_emb_interact(td, xd, dd))
    timer = _timer(2)
    try:
        for i in range(2):
            timer.arm(i)
            got = abi.dlrm_emb_interact(td, xd, dd)
            timer.disarm()
            torch.cuda.synchronize()
            assert np.array_equal(host(got), plain)
            assert 0.0 < timer.elapsed_ms(i) < 100.0
    finally:
        timer.close()
    want = oracle.interact(dense, oracle.emb_bag_sum(tables, idx, batch=w.batch))
    assert_close(plain, want, "fused, timing on and off")


def test_graph_plan_created_with_timing_on():
    import torch
    w = inputs.Workload("timing-fwd", batch=256, num_tables=4, rows=1000, dim=16, bag=4,
                        dist="uniform", dense_in=13, bottom=(32, 16), top=(24, 1))
    tables = [inputs.table_host(w, k) for k in range(w.num_tables)]
    bottom, top = inputs.dlrm_layers(w, bias_std=0.1)
    model = abi.DlrmModel([(dev(a), dev(b), act) for a, b, act in bottom],
                          [(dev(a), dev(b), act) for a, b, act in top],
                          [dev(t) for t in tables])
    dense = dev(inputs.dense(w))
    idx = [dev(inputs.indices(w, k)) for k in range(w.num_tables)]
    eager = host(abi.dlrm_forward(model, dense, idx))
    out = torch.empty_like(torch.from_numpy(eager)).cuda()
    timer = _timer(1)
    try:
        timer.arm(0)
        plan = abi.DlrmPlan(model, dense, idx, out=out, mode="graph")
        timer.disarm()
        for _ in range(3):
            plan.run()
            torch.cuda.synchronize()
            assert np.array_equal(host(out), eager)
        plan.close()
    finally:
        timer.close()


def test_direct_plan_replay_records_the_last_kernel():
    import torch
    w = inputs.Workload("timing-plan", batch=512, num_tables=8, rows=2000, dim=64, bag=10,
                        dist="zipf", dense_in=13, bottom=(128, 64), top=(64, 1))
    tables = [inputs.table_host(w, k) for k in range(w.num_tables)]
    bottom, top = inputs.dlrm_layers(w, bias_std=0.1)
    model = abi.DlrmModel([(dev(a), dev(b), act) for a, b, act in bottom],
                          [(dev(a), dev(b), act) for a, b, act in top],
                          [dev(t) for t in tables])
    dense = dev(inputs.dense(w))
    idx = [dev(inputs.indices(w, k)) for k in range(w.num_tables)]
    eager = host(abi.dlrm_forward(model, dense, idx))
    out = torch.empty(eager.shape, dtype=torch.float32, device="cuda")
    plan = abi.DlrmPlan(model, dense, idx, out=out, mode="direct")
    timer = _timer(1)
    try:
        timer.arm(0)
        plan.run()
        timer.disarm()
        torch.cuda.synchronize()
        assert 0.0 < timer.elapsed_ms(0) < 100.0
        assert np.array_equal(host(out), eager)
    finally:
        timer.close()
        plan.close()


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (256 << 20) + 48])
def test_stream_read_runs_and_leaves_the_sink(nbytes):
    """The streaming-read probe reads a buffer (sizes below one workgroup's
    sweep, ragged tails, larger than the L2) and writes nothing: a zero
    buffer never hashes to the key, so the sink keeps its value."""
    import torch
    buf = torch.zeros(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.full((1,), 7.0, device="cuda")
    timer = _timer(1)
    try:
        timer.arm(0)
        abi.dlrm_stream_read(buf, sink)
        timer.disarm()
        torch.cuda.synchronize()
        assert timer.elapsed_ms(0) > 0.0
    finally:
        timer.close()
    assert host(sink)[0] == 7.0
