"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


def test_pair_map(lib):
    oracle_pins.pin_pair_map(lib)


def test_emb_bag(lib):
    oracle_pins.pin_emb_bag(lib)


def test_emb_bag_mean_weights_bf16(lib):
    oracle_pins.pin_emb_bag_ext(lib)


def test_emb_bag_fp8_and_scales(lib):
    oracle_pins.pin_emb_bag_fp8(lib)


def test_interact(lib):
    oracle_pins.pin_interact(lib)


def test_linear(lib):
    oracle_pins.pin_linear(lib)


def test_forward(lib):
    oracle_pins.pin_forward(lib)


def test_rejects_bad_arguments(lib):
    t = np.zeros((4, 2), np.float32)
    with pytest.raises(oracle.OracleError):       # index out of range
        oracle.emb_bag_sum([t], [np.array([0, 4], np.int32)], batch=1, lib=lib)
    with pytest.raises(oracle.OracleError):       # negative index
        oracle.emb_bag_sum([t], [np.array([-1, 0], np.int32)], batch=1, lib=lib)
    with pytest.raises(oracle.OracleError):       # n_idx not a multiple of B
        oracle.emb_bag_sum([t], [np.array([0, 1, 2], np.int32)], batch=2, lib=lib)
    with pytest.raises(oracle.OracleError):       # decreasing offsets
        oracle.emb_bag_sum([t], [np.array([0, 1, 2], np.int32)],
                           [np.array([2, 1], np.int32)], lib=lib)
