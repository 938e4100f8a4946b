"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point the header declares, and rejects bad arguments before it
enqueues any work."""
import ctypes
import os
import re

import pytest

from conftest import ROOT
from dlrm_embedding_bag_amd import abi

HEADER = os.path.join(ROOT, "include", "dlrm_embedding_bag.h")
FAKE = 0x10000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(abi.LIB_PATH):
        from dlrm_embedding_bag_amd import build
        build.build()
    return abi.load()


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^DLRM_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, re.M)


def test_header_declares_the_binding_names():
    assert sorted(declared_functions()) == sorted(abi.EXPORTS)


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    assert lib.dlrm_abi_version() == 2
    for code, name in abi.STATUS_NAMES.items():
        assert lib.dlrm_status_string(code).decode().startswith(name)
    assert lib.dlrm_status_string(99) == b"unknown dlrm_status"


def test_stream_read_argument_errors(lib):
    f = lib.dlrm_stream_read
    assert f(FAKE, 0, FAKE, None) == 0                                   # nothing to read
    assert f(None, 64, FAKE, None) == 1                                  # buf NULL
    assert f(FAKE, 64, None, None) == 1                                  # sink NULL
    assert f(FAKE, 63, FAKE, None) == 2                                  # size % 16
    assert f(FAKE + 4, 64, FAKE, None) == 2                              # misaligned


def test_kernel_timing_events_need_both_or_neither(lib):
    f = lib.dlrm_set_kernel_timing_events
    assert f(FAKE, None) == 1                                         # DLRM_ERR_NULL
    assert f(None, FAKE) == 1
    assert f(None, None) == 0                                         # off


def _tables(K, rows=10):
    t = (ctypes.c_void_p * K)(*[FAKE] * K)
    r = (ctypes.c_int64 * K)(*[rows] * K)
    i = (ctypes.c_void_p * K)(*[FAKE] * K)
    return t, r, i


def _n(K, n):
    return (ctypes.c_int64 * K)(*[n] * K)


def test_emb_bag_argument_errors(lib):
    t, r, i = _tables(2)
    f = lib.emb_bag_sum_multi
    assert f(0, 4, 8, t, r, i, None, _n(2, 8), FAKE, None) == 2          # K < 1
    assert f(65, 4, 8, t, r, i, None, _n(2, 8), FAKE, None) == 2         # K > max
    assert f(2, -1, 8, t, r, i, None, _n(2, 8), FAKE, None) == 2         # B < 0
    assert f(2, 4, 0, t, r, i, None, _n(2, 8), FAKE, None) == 2          # D < 1
    assert f(2, 4, 1025, t, r, i, None, _n(2, 8), FAKE, None) == 2       # D > max
    assert f(2, 4, 8, None, r, i, None, _n(2, 8), FAKE, None) == 1       # tables NULL
    assert f(2, 4, 8, t, r, i, None, _n(2, 8), None, None) == 1          # out NULL
    assert f(2, 4, 8, t, r, i, None, _n(2, 7), FAKE, None) == 2          # n_idx % B
    t0, r0, i0 = _tables(2)
    t0[1] = None
    assert f(2, 4, 8, t0, r0, i0, None, _n(2, 8), FAKE, None) == 1       # tables[1] NULL
    r0 = (ctypes.c_int64 * 2)(10, 0)
    assert f(2, 4, 8, t, r0, i, None, _n(2, 8), FAKE, None) == 2         # rows < 1
    assert f(2, 4, 8, t, r, i, None, _n(2, 2**31), FAKE, None) == 2      # n_idx > INT32_MAX
    offs = (ctypes.c_void_p * 2)(FAKE, None)
    assert f(2, 4, 8, t, r, i, offs, _n(2, 7), FAKE, None) == 1          # offsets[1] NULL
    # B == 0 is a valid no-op that launches nothing
    assert f(2, 0, 8, t, r, i, None, _n(2, 0), FAKE, None) == 0


def test_interact_argument_errors(lib):
    f = lib.dlrm_interact_lower_tri
    assert f(4, 0, 8, FAKE, FAKE, FAKE, None) == 2
    assert f(4, 65, 8, FAKE, FAKE, FAKE, None) == 2
    assert f(4, 2, 0, FAKE, FAKE, FAKE, None) == 2
    assert f(4, 2, 8, None, FAKE, FAKE, None) == 1
    assert f(4, 2, 8, FAKE, FAKE, None, None) == 1
    # one sample's F x D tile beyond the LDS budget: 65 x 1024 floats
    assert f(4, 64, 1024, FAKE, FAKE, FAKE, None) == 3
    assert f(0, 2, 8, FAKE, FAKE, FAKE, None) == 0


def test_emb_interact_argument_errors(lib):
    t, r, i = _tables(3)
    f = lib.dlrm_emb_interact
    assert f(3, 4, 8, t, r, i, None, _n(3, 8), None, FAKE, None, None) == 1   # dense NULL
    assert f(3, 4, 8, t, r, i, None, _n(3, 8), FAKE, None, None, None) == 1   # out NULL
    assert f(3, 4, 8, t, r, i, None, _n(3, 9), FAKE, FAKE, None, None) == 2   # n_idx % B
    t64, r64, i64 = _tables(64)
    assert f(64, 4, 1024, t64, r64, i64, None, _n(64, 8), FAKE, FAKE, None, None) == 3


def _bags(K=2, B=4, D=8, dtype=0, pool=0, n=8, weights=False, offsets=False):
    t, r, i = _tables(K)
    keep = [t, r, i, _n(K, n)]
    w = (ctypes.c_void_p * K)(*[FAKE] * K) if weights else None
    o = (ctypes.c_void_p * K)(*[FAKE] * K) if offsets else None
    keep += [w, o]
    g = abi.Bags(K, B, D, dtype, pool, ctypes.cast(t, ctypes.POINTER(ctypes.c_void_p)), r,
                 ctypes.cast(i, ctypes.POINTER(ctypes.c_void_p)),
                 ctypes.cast(o, ctypes.POINTER(ctypes.c_void_p)) if o else None, keep[3],
                 ctypes.cast(w, ctypes.POINTER(ctypes.c_void_p)) if w else None)
    g._keep = keep
    return g


def test_emb_bag_pool_argument_errors(lib):
    f = lib.emb_bag_pool
    ok = _bags()
    assert f(None, FAKE, None) == 1                                     # bags NULL
    assert f(ctypes.byref(_bags(dtype=3)), FAKE, None) == 2             # unknown dtype
    assert f(ctypes.byref(_bags(pool=2)), FAKE, None) == 2              # unknown pool
    assert f(ctypes.byref(_bags(pool=1, weights=True)), FAKE, None) == 3  # mean + weights
    assert f(ctypes.byref(_bags(n=7)), FAKE, None) == 2                 # n_idx % B
    assert f(ctypes.byref(_bags(K=0)), FAKE, None) == 2                 # K < 1
    assert f(ctypes.byref(ok), None, None) == 1                         # out NULL
    g = _bags(weights=True)
    g.weights[1] = None
    assert f(ctypes.byref(g), FAKE, None) == 1                          # weights[1] NULL
    g = _bags(offsets=True, n=7)
    g.offsets[0] = None
    assert f(ctypes.byref(g), FAKE, None) == 1                          # offsets[0] NULL
    assert f(ctypes.byref(_bags(B=0, n=0, dtype=1, pool=1)), None, None) == 0  # B == 0
    fi = lib.dlrm_emb_interact_pool
    assert fi(None, FAKE, FAKE, None, None) == 1
    assert fi(ctypes.byref(ok), None, FAKE, None, None) == 1            # dense NULL
    assert fi(ctypes.byref(ok), FAKE, None, None, None) == 1            # out NULL
    assert fi(ctypes.byref(_bags(pool=1, weights=True)), FAKE, FAKE, None, None) == 3
    big = _bags(K=64, D=1024, dtype=1)
    assert fi(ctypes.byref(big), FAKE, FAKE, None, None) == 3           # tile beyond LDS
    assert fi(ctypes.byref(_bags(B=0, n=0)), None, None, None, None) == 0


def test_split_and_dots_argument_errors(lib):
    f = lib.linear_bias_act_split
    #        m  n  klo a_lo  lda klo hi  lda   w  bias act  c  ldc stream
    assert f(4, 0, 3, FAKE, 3, 5, FAKE, 5, FAKE, None, 0, FAKE, 2, None) == 2     # n < 1
    assert f(4, 2, 0, FAKE, 3, 5, FAKE, 5, FAKE, None, 0, FAKE, 2, None) == 2     # k_lo < 1
    assert f(4, 2, 3, FAKE, 3, 0, FAKE, 5, FAKE, None, 0, FAKE, 2, None) == 2     # k_hi < 1
    assert f(4, 2, 3, FAKE, 2, 5, FAKE, 5, FAKE, None, 0, FAKE, 2, None) == 2     # lda_lo < k_lo
    assert f(4, 2, 3, FAKE, 3, 5, FAKE, 4, FAKE, None, 0, FAKE, 2, None) == 2     # lda_hi < k_hi
    assert f(4, 2, 3, FAKE, 3, 5, FAKE, 5, FAKE, None, 3, FAKE, 2, None) == 2     # bad act
    assert f(4, 2, 3, None, 3, 5, FAKE, 5, FAKE, None, 0, FAKE, 2, None) == 1     # a_lo NULL
    assert f(4, 2, 3, FAKE, 3, 5, None, 5, FAKE, None, 0, FAKE, 2, None) == 1     # a_hi NULL
    assert f(0, 2, 3, None, 3, 5, None, 5, None, None, 0, None, 2, None) == 0     # m == 0
    g = lib.dlrm_emb_interact_dots
    ok = _bags(K=3)
    assert g(None, FAKE, FAKE, 6, None, None) == 1
    assert g(ctypes.byref(ok), FAKE, FAKE, 5, None, None) == 2          # ld_dots < P = 6
    assert g(ctypes.byref(ok), None, FAKE, 6, None, None) == 1          # dense NULL
    assert g(ctypes.byref(ok), FAKE, None, 6, None, None) == 1          # dots NULL
    assert g(ctypes.byref(_bags(K=3, B=0, n=0)), None, None, 6, None, None) == 0


def test_linear_argument_errors(lib):
    f = lib.linear_bias_act
    assert f(4, 0, 3, FAKE, 3, FAKE, None, 0, FAKE, 1, None) == 2     # n < 1
    assert f(4, 2, 0, FAKE, 3, FAKE, None, 0, FAKE, 2, None) == 2     # k < 1
    assert f(4, 2, 3, FAKE, 2, FAKE, None, 0, FAKE, 2, None) == 2     # lda < k
    assert f(4, 2, 3, FAKE, 3, FAKE, None, 0, FAKE, 1, None) == 2     # ldc < n
    assert f(4, 2, 3, FAKE, 3, FAKE, None, 3, FAKE, 2, None) == 2     # bad act
    assert f(4, 2, 3, None, 3, FAKE, None, 0, FAKE, 2, None) == 1     # a NULL
    assert f(4, 2, 3, FAKE, 3, None, None, 0, FAKE, 2, None) == 1     # w NULL
    assert f(4, 2, 3, FAKE, 3, FAKE, None, 0, None, 2, None) == 1     # c NULL
    assert f(0, 2, 3, FAKE, 3, FAKE, None, 0, FAKE, 2, None) == 0     # m == 0: no-op


def test_mlp_forward_argument_errors(lib):
    f = lib.mlp_forward
    def layers(spec):
        arr = (abi.Layer * len(spec))()
        for n, (i, o, act) in enumerate(spec):
            arr[n].in_features, arr[n].out_features, arr[n].weight, arr[n].act = i, o, FAKE, act
        return arr
    good = layers([(13, 512, 1), (512, 256, 1), (256, 64, 1)])
    assert f(8, 0, good, FAKE, 13, FAKE, 64, None) == 2                 # no layers
    assert f(8, 3, None, FAKE, 13, FAKE, 64, None) == 1                 # layers NULL
    assert f(8, 3, layers([(13, 512, 1), (500, 64, 1), (64, 64, 1)]), FAKE, 13, FAKE, 64,
             None) == 2                                                  # widths do not chain
    assert f(8, 3, good, FAKE, 12, FAKE, 64, None) == 2                 # lda < in
    assert f(8, 3, good, None, 13, FAKE, 64, None) == 1                 # a NULL
    assert f(8, 2, layers([(13, 96, 1), (96, 64, 1)]), FAKE, 13, FAKE, 64,
             None) == 3                                                  # width 96 unsupported
    assert f(8, 1, layers([(13, 1, 2)]), FAKE, 13, FAKE, 1, None) == 3  # head needs a layer first
    assert f(8, 5, layers([(64, 64, 1)] * 5), FAKE, 64, FAKE, 64, None) == 3   # > 4 layers
    assert f(0, 3, good, None, 13, None, 64, None) == 0                 # m == 0: no-op


def _model(bottom, top, K, D, options=0):
    bl = (abi.Layer * len(bottom))()
    for n, (i, o, act) in enumerate(bottom):
        bl[n].in_features, bl[n].out_features, bl[n].weight, bl[n].act = i, o, FAKE, act
    tl = (abi.Layer * len(top))()
    for n, (i, o, act) in enumerate(top):
        tl[n].in_features, tl[n].out_features, tl[n].weight, tl[n].act = i, o, FAKE, act
    t, r, _ = _tables(K)
    m = abi.Model(len(bottom), bl, len(top), tl, K, D, t, r, options)
    m._keep = (bl, tl, t, r)
    return m


def test_forward_workspace_and_errors(lib):
    K, D = 26, 64
    P = 27 * 26 // 2
    good = _model([(13, 512, 1), (512, 256, 1), (256, 64, 1)],
                  [(D + P, 512, 1), (512, 256, 1), (256, 1, 2)], K, D)
    B = 8192
    ws = lib.dlrm_forward_workspace_bytes(ctypes.byref(good), B)
    # at 8192 samples the bottom MLP is one launch and the head is folded into
    # top layer 1: R (B x 416 floats) + one buffer for top layer 0's output
    # (B x 512)
    assert ws == B * 416 * 4 + B * 512 * 4
    # layer by layer (no fused or slice launches, no k partials): R + two
    # ping-pong buffers (B x 512)
    layered = _model([(13, 512, 1), (512, 256, 1), (256, 64, 1)],
                     [(D + P, 512, 1), (512, 256, 1), (256, 1, 2)], K, D,
                     options=abi.forward_options(("unfused_head", "unfused_bottom",
                                                  "unsplit_k")))
    assert (lib.dlrm_forward_workspace_bytes(ctypes.byref(layered), B)
            == B * 416 * 4 + 2 * B * 512 * 4)
    odd = _model([(13, 96, 1), (96, 64, 1)], [(D + P, 96, 1), (96, 1, 2)], K, D)
    # other widths: R + the bottom MLP's hidden layer (B x 96); the head is
    # folded into top layer 0
    assert lib.dlrm_forward_workspace_bytes(ctypes.byref(odd), B) == B * 416 * 4 + B * 96 * 4
    bad_chain = _model([(13, 512, 1), (500, 64, 1)], [(D + P, 1, 2)], K, D)
    assert lib.dlrm_forward_workspace_bytes(ctypes.byref(bad_chain), B) == 0
    bad_dim = _model([(13, 32, 1)], [(D + P, 1, 2)], K, D)       # bottom out != D
    assert lib.dlrm_forward_workspace_bytes(ctypes.byref(bad_dim), B) == 0
    bad_top = _model([(13, 64, 1)], [(D + P + 1, 1, 2)], K, D)   # top in != D + P
    assert lib.dlrm_forward_workspace_bytes(ctypes.byref(bad_top), B) == 0
    f = lib.dlrm_forward
    idx = (ctypes.c_void_p * K)(*[FAKE] * K)
    n = _n(K, B * 20)
    assert f(ctypes.byref(bad_chain), B, FAKE, idx, None, n, FAKE, FAKE, ws, None) == 2
    assert f(ctypes.byref(good), B, FAKE, idx, None, n, FAKE, FAKE, ws - 1, None) == 4
    assert f(ctypes.byref(good), B, FAKE, idx, None, n, FAKE, FAKE + 16, ws, None) == 4
    assert f(ctypes.byref(good), B, FAKE, idx, None, n, FAKE, None, ws, None) == 1
    assert f(ctypes.byref(good), B, None, idx, None, n, FAKE, FAKE, ws, None) == 1
    assert f(None, B, FAKE, idx, None, n, FAKE, FAKE, ws, None) == 1
    assert f(ctypes.byref(good), 0, FAKE, idx, None, _n(K, 0), FAKE, FAKE, ws, None) == 0


def test_forward_options_are_validated(lib):
    """dlrm_model.options: the documented bits are accepted (they change the
    composition, and with it the workspace: with DLRM_FORWARD_UNSPLIT_K it
    holds no partial sums, so at 256 samples it is smaller), any other bit
    is DLRM_ERR_SHAPE."""
    K, D = 26, 64
    P = 27 * 26 // 2
    spec = ([(13, 512, 1), (512, 256, 1), (256, 64, 1)],
            [(D + P, 512, 1), (512, 256, 1), (256, 1, 2)])
    B = 256
    base = lib.dlrm_forward_workspace_bytes(ctypes.byref(_model(*spec, K, D)), B)
    assert base > 0
    every = 0
    for v in abi.FORWARD_OPTIONS.values():
        every |= v
    unsplit = abi.FORWARD_OPTIONS["unsplit_k"]
    plain = lib.dlrm_forward_workspace_bytes(ctypes.byref(_model(*spec, K, D, options=unsplit)),
                                             B)
    assert 0 < plain < base, "at 256 samples the default composition stores k partials"
    for bits in list(abi.FORWARD_OPTIONS.values()) + [every]:
        m = _model(*spec, K, D, options=bits)
        ws = lib.dlrm_forward_workspace_bytes(ctypes.byref(m), B)
        assert ws == plain if bits & unsplit else ws > 0, bits
    idx = (ctypes.c_void_p * K)(*[FAKE] * K)
    for bits in (every + 1, 1 << 31, 0xFFFFFFFF):
        m = _model(*spec, K, D, options=bits)
        assert lib.dlrm_forward_workspace_bytes(ctypes.byref(m), B) == 0
        assert lib.dlrm_forward(ctypes.byref(m), B, FAKE, idx, None, _n(K, B * 20), FAKE,
                                FAKE, base, None) == 2
    assert abi.forward_options(("layered", "unfused_head", "unfused_bottom")) == 7
    with pytest.raises(ValueError):
        abi.forward_options(("fast",))


def test_no_environment_switch_in_the_library():
    """The library's behaviour is set by its arguments only: no source reads
    the process environment."""
    csrc = os.path.join(ROOT, "dlrm_embedding_bag_amd", "csrc")
    for name in os.listdir(csrc):
        text = open(os.path.join(csrc, name)).read()
        assert "getenv" not in text and "environ" not in text, name


def test_linear_head_argument_errors(lib):
    f = lib.linear_bias_act_head
    assert f(8, 257, 512, FAKE, 512, FAKE, None, 1, FAKE, None, 2, FAKE, 1, None) == 3  # n > 256
    assert f(8, 0, 512, FAKE, 512, FAKE, None, 1, FAKE, None, 2, FAKE, 1, None) == 2    # n < 1
    assert f(8, 64, 512, FAKE, 500, FAKE, None, 1, FAKE, None, 2, FAKE, 1, None) == 2   # lda < k
    assert f(8, 64, 512, FAKE, 512, FAKE, None, 1, FAKE, None, 3, FAKE, 1, None) == 2   # head act
    assert f(8, 64, 512, FAKE, 512, FAKE, None, 1, FAKE, None, 2, FAKE, 0, None) == 2   # ldo < 1
    assert f(8, 64, 512, FAKE, 512, FAKE, None, 1, None, None, 2, FAKE, 1, None) == 1   # head_w
    assert f(8, 64, 512, None, 512, FAKE, None, 1, FAKE, None, 2, FAKE, 1, None) == 1   # a NULL
    assert f(0, 64, 512, None, 512, None, None, 1, None, None, 2, None, 1, None) == 0   # m == 0


def test_noalloc_forward_argument_errors(lib):
    """dlrm_forward_noalloc validates like dlrm_forward and refuses, before
    any HIP call, a forward whose workspace exceeds its fixed array."""
    K, D = 26, 64
    P = 27 * 26 // 2
    good = _model([(13, 512, 1), (512, 256, 1), (256, 64, 1)],
                  [(D + P, 512, 1), (512, 256, 1), (256, 1, 2)], K, D)
    f = lib.dlrm_forward_noalloc
    idx = (ctypes.c_void_p * K)(*[FAKE] * K)
    big = 16384
    assert lib.dlrm_forward_workspace_bytes(ctypes.byref(good), big) > abi.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(good), big, FAKE, idx, None, _n(K, big * 20), FAKE, None) == 4
    assert f(None, 64, FAKE, idx, None, _n(K, 64 * 20), FAKE, None) == 1
    bad_dim = _model([(13, 32, 1)], [(D + P, 1, 2)], K, D)
    assert f(ctypes.byref(bad_dim), 64, FAKE, idx, None, _n(K, 64 * 20), FAKE, None) == 2
    assert f(ctypes.byref(good), 64, FAKE, idx, None, _n(K, 64 * 20 + 1), FAKE, None) == 2
    assert f(ctypes.byref(good), 0, FAKE, idx, None, _n(K, 0), FAKE, None) == 0
    assert abi.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_plan_argument_errors(lib):
    """dlrm_plan_create validates like dlrm_forward before touching HIP."""
    K, D = 26, 64
    P = 27 * 26 // 2
    good = _model([(13, 512, 1), (512, 256, 1), (256, 64, 1)],
                  [(D + P, 512, 1), (512, 256, 1), (256, 1, 2)], K, D)
    bad_dim = _model([(13, 32, 1)], [(D + P, 1, 2)], K, D)
    B = 64
    ws = lib.dlrm_forward_workspace_bytes(ctypes.byref(good), B)
    idx = (ctypes.c_void_p * K)(*[FAKE] * K)
    n = _n(K, B * 20)
    f = lib.dlrm_plan_create
    h = ctypes.c_void_p(FAKE)
    for mode in (0, 1):
        assert f(ctypes.byref(good), B, FAKE, idx, None, n, FAKE, FAKE, ws, mode, None) == 1
        assert f(ctypes.byref(bad_dim), B, FAKE, idx, None, n, FAKE, FAKE, ws, mode,
                 ctypes.byref(h)) == 2
        assert h.value is None, "a failed create leaves NULL in *plan"
        assert f(ctypes.byref(good), B, FAKE, idx, None, n, FAKE, FAKE, ws - 1, mode,
                 ctypes.byref(h)) == 4
        assert f(ctypes.byref(good), B, None, idx, None, n, FAKE, FAKE, ws, mode,
                 ctypes.byref(h)) == 1
        assert f(ctypes.byref(good), B, FAKE, idx, None, _n(K, B * 20 + 1), FAKE, FAKE, ws,
                 mode, ctypes.byref(h)) == 2
        assert f(ctypes.byref(good), 0, FAKE, idx, None, _n(K, 0), FAKE, FAKE, ws, mode,
                 ctypes.byref(h)) == 2                                  # batch 0: no plan
    assert f(ctypes.byref(good), B, FAKE, idx, None, n, FAKE, FAKE, ws, 2,
             ctypes.byref(h)) == 2                                      # unknown mode
    assert lib.dlrm_plan_run(None, None) == 1
    assert lib.dlrm_plan_update(None, FAKE, idx, None, n, FAKE) == 1
    assert lib.dlrm_plan_destroy(None) == 0


def test_binding_refuses_cpu_tensors(lib):
    import torch
    t = torch.zeros(4, 2)
    with pytest.raises(ValueError, match="no CPU path"):
        abi.emb_bag_sum_multi([t], [torch.zeros(4, dtype=torch.int32)], batch=2)
    with pytest.raises(ValueError, match="no CPU path"):
        abi.dlrm_interact_lower_tri(torch.zeros(2, 2), torch.zeros(2, 1, 2))


def test_bottom_slice_partials_in_the_workspace(lib):
    """The small-batch bottom MLP runs as one slice launch whose partial sums
    of the dense feature sit in the workspace beside R: 16 of them (16-column
    slices) while the grid of 16-row bands x 16 slices is at most 512
    workgroups, 4 (64-column slices) up to 384 workgroups of those, none
    (layer launches) beyond.  A one-layer top MLP adds no buffers, so the
    workspace is R + the partials exactly."""
    K, D = 26, 64
    P = 27 * 26 // 2
    bottom = [(13, 512, 1), (512, 256, 1), (256, D, 1)]
    m = _model(bottom, [(D + P, 1, 2)], K, D)
    ldR = 416  # D + P rounded up to 4 floats

    def ws(B):
        return lib.dlrm_forward_workspace_bytes(ctypes.byref(m), B)

    def r_bytes(B):
        return (B * ldR * 4 + 255) // 256 * 256

    for B, parts in ((1, 16), (256, 16), (500, 16), (512, 16), (513, 4), (1024, 4),
                     (1536, 4)):
        assert ws(B) == r_bytes(B) + (parts * B * D * 4 + 255) // 256 * 256, B
    # past 1,536 samples the bottom MLP runs layer by layer: its buffers hold
    # B x 512 hidden activations (or their k partials), more than the slices
    for B in (1537, 2048):
        assert ws(B) >= r_bytes(B) + B * 512 * 4, B
