"""Sensitivity of the oracle's pins: plant one plausible mistake in a copy of
an oracle module (on the CPU, by a textual edit of its source) and require
that the pin meant to guard that step fails.  The real oracle is untouched."""
import importlib
import inspect
import sys
import types

import numpy as np
import pytest
import torch

import oracle_pins as pins


def mutated(modname: str, find: str, replace: str) -> types.ModuleType:
    mod = importlib.import_module(modname)
    src = inspect.getsource(mod)
    assert src.count(find) == 1, f"mutation anchor not unique/found: {find!r}"
    new = types.ModuleType(modname + "_planted")
    new.__package__ = mod.__package__
    new.__file__ = mod.__file__
    exec(compile(src.replace(find, replace), mod.__file__ + " (planted)", "exec"), new.__dict__)
    return new


REGION_MUTATIONS = [
    # (id, find, replace, check)
    ("drop_slab0", "for k in range(1, t):", "for k in range(2, t):",
     lambda R: pins.check_z_within_exact_bound(R=R)),
    ("bias_sign", "acc = (acc + bias32[None, :])", "acc = (acc - bias32[None, :])",
     lambda R: pins.check_z_within_exact_bound(R=R)),
    ("no_inverted_scale", "(acc * scale).astype", "(acc * np.float32(1.0)).astype",
     lambda R: pins.check_z_within_exact_bound(R=R)),
    ("keep_inverted", "return u >= thr", "return u < thr",
     lambda R: pins.check_z_within_exact_bound(R=R)),
    ("no_residual", "zf = (decode(residual[r], dtype) + d)", "zf = (0 * decode(residual[r], dtype) + d)",
     lambda R: pins.check_z_within_exact_bound(R=R)),
    ("round_each_add", "acc = (acc + decode(partials[k][r], dtype)).astype(acc_t)",
     "acc = decode(encode((acc + decode(partials[k][r], dtype)).astype(acc_t), dtype), dtype)",
     lambda R: pins.check_z_within_exact_bound(dtype="bf16", R=R)),
    ("unbiased_variance", "var = ((z64 - mu[..., None]) ** 2).mean(axis=-1)",
     "var = ((z64 - mu[..., None]) ** 2).sum(axis=-1) / (z64.shape[-1] - 1)",
     lambda R: pins.check_layernorm_matches_torch(R=R)),
    ("eps_outside_sqrt", "rs = 1.0 / np.sqrt(var + eps64)", "rs = 1.0 / (np.sqrt(var) + eps64)",
     lambda R: pins.check_hand_case_h2(R=R)),
    ("rms_subtracts_mean", "return None, rs, z64 * rs[..., None]",
     "return None, rs, (z64 - z64.mean(axis=-1, keepdims=True)) * rs[..., None]",
     lambda R: pins.check_rmsnorm_matches_torch(R=R)),
    ("rank_ignored", "return rank * np.int64(T) + i", "return i",
     lambda R: pins.check_shard_invariance(R=R)),
    ("ragged_start_not_scaled", "g[a:b] = t * a + rank * (b - a) + (i[a:b] - a)",
     "g[a:b] = a + rank * (b - a) + (i[a:b] - a)",
     lambda R: pins.check_ragged_token_index(R=R)),
    ("ragged_interleaved", "g[a:b] = t * a + rank * (b - a) + (i[a:b] - a)",
     "g[a:b] = t * a + t * (i[a:b] - a) + rank",
     lambda R: pins.check_ragged_masks_tile_global(R=R)),
    ("bwd_c2_sign", "d = rs[:, None] * (g - c1[:, None] - xhat * c2[:, None])",
     "d = rs[:, None] * (g - c1[:, None] + xhat * c2[:, None])",
     lambda R: pins.check_backward_finite_differences("layernorm", R=R)),
    ("bwd_c1_dropped", "d = rs[:, None] * (g - c1[:, None] - xhat * c2[:, None])",
     "d = rs[:, None] * (g - xhat * c2[:, None])",
     lambda R: pins.check_backward_scale_identities("layernorm", R=R)),
    ("bwd_c2_without_gamma", "c2 = (g * xhat).mean(axis=1)", "c2 = (dy64 * xhat).mean(axis=1)",
     lambda R: pins.check_backward_matches_torch_autograd("layernorm", R=R)),
    ("bwd_dgamma_uses_z", "dgamma += (dy64 * xhat).sum(axis=0)", "dgamma += (dy64 * z64).sum(axis=0)",
     lambda R: pins.check_backward_finite_differences("layernorm", R=R)),
    ("bwd_rms_no_projection", "d = rs[:, None] * (g - xhat * c2[:, None])", "d = rs[:, None] * g",
     lambda R: pins.check_backward_finite_differences("rmsnorm", R=R)),
    ("bwd_dres_ignored", "d = d + decode(dres_in[r], dtype).astype(np.float64)", "d = d",
     lambda R: pins.check_backward_matches_torch_autograd("rmsnorm", R=R)),
    ("dropout_bwd_no_scale", "dpartial = np.where(keep, dx * scale, 0.0)", "dpartial = np.where(keep, dx, 0.0)",
     lambda R: pins.check_dropout_backward_finite_differences(R=R)),
    ("dropout_bwd_mask_inverted", "dpartial = np.where(keep, dx * scale, 0.0)",
     "dpartial = np.where(~keep, dx * scale, 0.0)",
     lambda R: pins.check_dropout_backward_finite_differences(R=R)),
    ("dropout_bwd_rank_ignored", "keep = keep_mask(seed, p_drop, token_index(T, t, rank, cu_seqlens)[rows], h)",
     "keep = keep_mask(seed, p_drop, token_index(T, t, 0, cu_seqlens)[rows], h)",
     lambda R: pins.check_dropout_backward_finite_differences(R=R)),
    ("dropout_bwd_uniform_index", "keep = keep_mask(seed, p_drop, token_index(T, t, rank, cu_seqlens)[rows], h)",
     "keep = keep_mask(seed, p_drop, token_index(T, t, rank, None)[rows], h)",
     lambda R: pins.check_dropout_backward_finite_differences(ragged=True, R=R)),
    ("dropout_bwd_dbias_from_dx", "return dict(dpartial=dpartial, dbias=dpartial.sum(axis=0),",
     "return dict(dpartial=dpartial, dbias=dx.sum(axis=0),",
     lambda R: pins.check_dropout_backward_finite_differences(R=R)),
    ("accumulate_overwrites", "np.asarray(buf, dtype=np.float64) + np.asarray(add, dtype=np.float64)",
     "0.0 * np.asarray(buf, dtype=np.float64) + np.asarray(add, dtype=np.float64)",
     lambda R: pins.check_accumulate_split_batches(R=R)),
    ("accumulate_subtracts", "np.asarray(buf, dtype=np.float64) + np.asarray(add, dtype=np.float64)",
     "np.asarray(buf, dtype=np.float64) - np.asarray(add, dtype=np.float64)",
     lambda R: pins.check_accumulate_split_batches(R=R)),
    ("accumulate_rounds_to_bf16", "np.asarray(buf, dtype=np.float64) + np.asarray(add, dtype=np.float64)",
     "decode(encode((np.asarray(buf, dtype=np.float64) + np.asarray(add, dtype=np.float64)).astype(np.float32), "
     "'bf16'), 'bf16').astype(np.float64)",
     lambda R: pins.check_accumulate_split_batches(R=R)),
]


@pytest.mark.parametrize("name,find,replace,check", REGION_MUTATIONS, ids=[m[0] for m in REGION_MUTATIONS])
def test_region_mistake_is_caught(name, find, replace, check):
    R = mutated("oracle.region", find, replace)
    with pytest.raises(AssertionError):
        check(R)


def _bf16_matches_torch(B):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(50_000) * np.exp(rng.uniform(-20, 20, 50_000))).astype(np.float32)
    x[:4] = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 3.4e38], dtype=np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(B.f32_to_bf16(x), ref)


@pytest.mark.parametrize("find,replace", [
    ("pick_away = (rest > half) | ((rest == half) & ((toward_zero & np.uint32(1)) == 1))", "pick_away = rest > half"),
    ("pick_away = (rest > half) | ((rest == half) & ((toward_zero & np.uint32(1)) == 1))", "pick_away = rest >= half"),
    ("pick_away = (rest > half) | ((rest == half) & ((toward_zero & np.uint32(1)) == 1))", "pick_away = rest > rest"),
], ids=["ties_down", "ties_away", "truncate"])
def test_bf16_mistake_is_caught(find, replace):
    B = mutated("oracle.bf16", find, replace)
    with pytest.raises(AssertionError):
        _bf16_matches_torch(B)


def _philox64_matches_numpy(P):
    bg = np.random.Philox(counter=np.array([3, 4, 5, 6], dtype=np.uint64), key=np.array([1, 2], dtype=np.uint64))
    raw = bg.random_raw(4)
    assert list(P.philox_ref([4, 4, 5, 6], [1, 2], width=64)) == [int(x) for x in raw]


@pytest.mark.parametrize("find,replace", [
    ("c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0", "c0, c1, c2, c3 = hi0 ^ c1 ^ k0, lo0, hi1 ^ c3 ^ k1, lo1"),
    ("c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0", "c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k0, lo0"),
    ("k0 = (k0 + c[\"W0\"]) & mask", "k0 = (k0 + c[\"W1\"]) & mask"),
    ("for r in range(rounds):\n        if r:", "for r in range(rounds):\n        if True:"),
], ids=["swap_products", "wrong_key_word", "wrong_weyl", "bump_before_first_round"])
def test_philox_structure_mistake_is_caught(find, replace):
    P = mutated("oracle.philox", find, replace)
    with pytest.raises(AssertionError):
        _philox64_matches_numpy(P)


def test_real_oracle_passes_the_same_checks():
    import oracle.bf16 as B
    import oracle.philox as P
    _bf16_matches_torch(B)
    _philox64_matches_numpy(P)
