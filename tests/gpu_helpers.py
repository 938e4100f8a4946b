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


def host_table(t):
    """Host copy of a device table: float32, uint16 bit patterns for bfloat16,
    uint8 codes for float8_e4m3fn."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return host(t)


def sampled_bags(tables_dev, idx_host, samples, bag=None, offsets_host=None,
                 weights_host=None):
    """Cut the bags of `samples` out of a full-size problem, CSR or uniform.

    Returns host (tables, indices, offsets, weights) of a problem with one
    sample per entry of `samples`, whose pooled bags equal the full
    problem's: each table keeps only the rows its sampled bags touch (copied
    from the device in its storage type), indices are renumbered into it and
    the sampled bags are laid out back to back with CSR offsets.  weights is
    None when weights_host is None.
    """
    import torch
    sub_tables, sub_idx, sub_offs, sub_w = [], [], [], []
    for k, (t_dev, idx) in enumerate(zip(tables_dev, idx_host)):
        n = idx.shape[0]
        if offsets_host is None:
            bounds = [(s * bag, (s + 1) * bag) for s in samples]
        else:
            o = offsets_host[k]
            bounds = [(int(o[s]), int(o[s + 1]) if s + 1 < len(o) else n) for s in samples]
        picks = np.concatenate([np.arange(a, b) for a, b in bounds]).astype(np.int64)
        lens = np.array([b - a for a, b in bounds], np.int64)
        bags = idx[picks]
        rows = np.unique(bags) if bags.size else np.zeros(1, np.int64)
        sub = t_dev.index_select(0, torch.from_numpy(rows.astype(np.int64)).to(t_dev.device))
        sub_tables.append(host_table(sub))
        sub_idx.append(np.searchsorted(rows, bags).astype(np.int32))
        sub_offs.append(np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32))
        if weights_host is not None:
            sub_w.append(weights_host[k][picks])
    return sub_tables, sub_idx, sub_offs, (sub_w if weights_host is not None else None)


def sample_rows(B, count, seed=0):
    """Sorted sample ids: first, last and a seeded spread in between."""
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(B, size=min(count, B), replace=False).tolist())
    picks.update({0, B - 1})
    return np.array(sorted(picks))
