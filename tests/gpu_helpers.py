"""Host-side helpers for the GPU parity tests: moving seeded inputs to the
device and cutting sampled sub-problems out of full-size inputs for the
oracle.  No arithmetic of the method happens here."""
import numpy as np

from dlrm_embedding_bag_amd import inputs

RTOL = 1e-5
ATOL = 1e-5


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def assert_close(got, want, what=""):
    """The float bar: |got - want| <= 1e-5 + 1e-5 |want| element by element."""
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), what
    np.testing.assert_allclose(got, want, rtol=RTOL, atol=ATOL, err_msg=what)


def make_uniform_case(w, seed=0, dyadic=False):
    """Host tables, indices and dense input of workload `w` (small sizes)."""
    if dyadic:
        tables = [inputs.table_dyadic(w, k, seed) for k in range(w.num_tables)]
        dense = inputs.dense_dyadic(w, seed)
    else:
        tables = [inputs.table_host(w, k, seed) for k in range(w.num_tables)]
        dense = inputs.dense(w, seed)
    idx = [inputs.indices(w, k, seed) for k in range(w.num_tables)]
    return tables, idx, dense


def sampled_subproblem(tables_dev, idx_host, bag, samples):
    """Cut the bags of `samples` out of a full-size problem.

    Returns host (tables, indices) whose pooled sums for sample s equal the
    full problem's for samples[s]: each table keeps only the rows those bags
    touch, copied from the device, and the indices are renumbered into it.
    """
    import torch
    sub_tables, sub_idx = [], []
    for t_dev, idx in zip(tables_dev, idx_host):
        bags = np.concatenate([idx[s * bag:(s + 1) * bag] for s in samples])
        rows = np.unique(bags)
        sub = t_dev.index_select(0, torch.from_numpy(rows.astype(np.int64)).to(t_dev.device))
        sub_tables.append(host(sub))
        sub_idx.append(np.searchsorted(rows, bags).astype(np.int32))
    return sub_tables, sub_idx


def sample_rows(B, count, seed=0):
    """Sorted sample ids: first, last and a seeded spread in between."""
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(B, size=min(count, B), replace=False).tolist())
    picks.update({0, B - 1})
    return np.array(sorted(picks))
