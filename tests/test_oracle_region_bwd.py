"""Pins of the oracle's backward (see tests/oracle_pins.py)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_finite_differences(norm):
    pins.check_backward_finite_differences(norm)


@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_torch_autograd(norm):
    pins.check_backward_matches_torch_autograd(norm)


@pytest.mark.parametrize("norm", ["layernorm", "rmsnorm"])
def test_scale_identities(norm):
    pins.check_backward_scale_identities(norm)


def test_dbeta_is_column_sum():
    pins.check_dbeta_is_column_sum()


@pytest.mark.parametrize("norm,ragged", [("layernorm", False), ("rmsnorm", False), ("layernorm", True)])
def test_dropout_backward_finite_differences(norm, ragged):
    pins.check_dropout_backward_finite_differences(norm, ragged)


def test_dropout_backward_special_cases():
    pins.check_dropout_backward_special_cases()


def test_accumulate_split_batches():
    pins.check_accumulate_split_batches()


def test_accumulate_identities():
    pins.check_accumulate_identities()
