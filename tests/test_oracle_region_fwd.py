"""Pins of the oracle's forward (see tests/oracle_pins.py for what each ties to)."""
import pytest

import oracle_pins as pins


def test_layernorm_special_case_is_torch_layer_norm():
    pins.check_layernorm_matches_torch()


def test_rmsnorm_special_case_is_torch_rms_norm():
    pins.check_rmsnorm_matches_torch()


def test_hand_case_h2():
    pins.check_hand_case_h2()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_unit_affine_invariant(dtype):
    pins.check_unit_affine_invariant(dtype=dtype)


@pytest.mark.parametrize("dtype,p", [("f32", 0.1), ("bf16", 0.1), ("f32", 0.0), ("bf16", 0.5)])
def test_z_within_exact_bound(dtype, p):
    pins.check_z_within_exact_bound(dtype=dtype, p=p)


def test_shard_invariance():
    pins.check_shard_invariance()


def test_ragged_token_index_hand_example():
    pins.check_ragged_token_index()


def test_ragged_masks_tile_global():
    pins.check_ragged_masks_tile_global()


def test_rows_subset_equals_full():
    pins.check_rows_subset()
