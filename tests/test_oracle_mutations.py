"""Planted mistakes in the oracle (CPU only) must each fail one of the pins.

Each case patches one oracle function with a plausible slip -- a dropped term,
a wrong sign, a wrong index, a transposed operand, another reading of s -- and
runs the pins that should catch it.
"""
import numpy as np
import pytest

import test_oracle_pins as pins
from oracle import decompose, forward

_orig_factored = forward.factored


def _no_scale(x, W0, s, U, V):
    return _orig_factored(x, W0, np.ones_like(np.asarray(s, float)), U, V)


def _no_delta(x, W0, s, U, V):
    return _orig_factored(x, W0, s, U[:, :0], V[:, :0])


def _minus_delta(x, W0, s, U, V):
    return 2 * _orig_factored(x, W0, s, U[:, :0], V[:, :0]) - _orig_factored(x, W0, s, U, V)


def _v_reversed(x, W0, s, U, V):
    return _orig_factored(x, W0, s, U, np.asarray(V)[::-1])


def _scale_columns(x, W0, s, U, V):
    # s applied along K instead of N (only meaningful when N == K)
    x = np.asarray(x, float)
    if len(s) == x.shape[1]:
        return _orig_factored(x * np.asarray(s)[None, :], W0, np.ones(len(s)), U, V)
    return _orig_factored(x, W0, s, U, V) * 1.001


FORWARD_PINS = [pins.test_identity_block_scales_input, pins.test_rank_one_delta_closed_form,
                pins.test_forward_brute_force_loops]


@pytest.mark.parametrize("mutant", [_no_scale, _no_delta, _minus_delta, _v_reversed, _scale_columns])
def test_forward_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(forward, "factored", mutant)
    caught = 0
    for pin in FORWARD_PINS:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"{mutant.__name__} passed every forward pin"


def _ratio_scale(W, W0):
    return np.linalg.norm(W, axis=1) / np.linalg.norm(W0, axis=1)


def _interleaved_band(layer, L, G):
    return layer % G


_orig_tf = decompose.truncated_factors


def _full_sigma_split(R, rank):
    U, V, S = _orig_tf(R, rank)
    r = U.shape[1]
    return U * np.sqrt(S[:r])[None, :], V, S


def _skip_first_triplet(R, rank):
    N, K = R.shape
    r = min(rank, N, K)
    P, S, Qt = np.linalg.svd(R, full_matrices=False)
    sel = slice(1, r + 1)
    return P[:, sel] * np.sqrt(S[sel]), Qt[sel].T * np.sqrt(S[sel]), S


@pytest.mark.parametrize("name,attr,mutant", [
    ("norm-ratio scale", "row_scale", _ratio_scale),
    ("interleaved bands", "band_of", _interleaved_band),
    ("sigma applied twice", "truncated_factors", _full_sigma_split),
    ("wrong singular index", "truncated_factors", _skip_first_triplet),
])
def test_decompose_mutants_are_caught(monkeypatch, name, attr, mutant):
    monkeypatch.setattr(decompose, attr, mutant)
    if attr == "band_of":
        # decompose_family and band_members look the function up at call time
        pass
    caught = 0
    for pin, args in [(pins.test_band_assignment, ()),
                      (pins.test_decomposition_brute_force, (4, 2, 6, 5, 2)),
                      (pins.test_eckart_young_tail_energy, (5,)),
                      (pins.test_full_rank_reconstructs, (2,))]:
        try:
            pin(*args)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"{name} passed every decomposition pin"


def _mean_shared_block(weights, scales, deltas, W0_prev):
    # ignores the scales: the plain mean of W_l - D_l
    return sum(np.asarray(W, np.float64) - D for W, D in zip(weights, deltas)) / len(weights)


def _sum_s_shared_block(weights, scales, deltas, W0_prev):
    # divides by sum s instead of sum s^2
    num = sum(np.asarray(s)[:, None] * (np.asarray(W, np.float64) - D) for W, s, D in zip(weights, scales, deltas))
    den = sum(np.asarray(s) for s in scales)
    return num / np.where(den == 0, 1.0, den)[:, None]


def _als_with(slip):
    """als_band with one slip in its per-layer steps."""
    def als(weights, rank, sweeps, store=True):
        W0, members = decompose.decompose_band(weights, rank, store)
        Ws = [np.asarray(W, np.float64) for W in weights]
        for _ in range(sweeps):
            deltas = [decompose.delta_product(m["U"], m["V"]) for m in members]
            W0 = decompose.shared_block_given(Ws, [m["s"] for m in members], deltas, W0)
            new = []
            for W, D in zip(Ws, deltas):
                s = decompose.row_scale(W if slip == "s ignores delta" else W - D, W0)
                R = decompose.residual(W, W0, s)
                if slip == "delta subtracted twice":
                    R = R - D
                U, V, S = decompose.truncated_factors(R, rank)
                new.append({"s": s, "U": U, "V": V, "sigma": S,
                            "err": decompose.rel_frobenius_error(W, W0, s, U, V)})
            members = new
        return W0, members
    return als


@pytest.mark.parametrize("name,attr,mutant", [
    ("W0 step ignores the scales", "shared_block_given", _mean_shared_block),
    ("W0 step divides by sum s", "shared_block_given", _sum_s_shared_block),
    ("s step ignores the delta", "als_band", _als_with("s ignores delta")),
    ("delta fitted to the residual less the old delta", "als_band", _als_with("delta subtracted twice")),
])
def test_als_mutants_are_caught(monkeypatch, name, attr, mutant):
    monkeypatch.setattr(decompose, attr, mutant)
    caught = 0
    for pin, args in [(pins.test_als_objective_never_increases, (3, 10, 7, 2)),
                      (pins.test_als_objective_never_increases, (5, 12, 12, 3)),
                      (pins.test_als_shared_block_is_least_squares, ()),
                      (pins.test_als_scale_step_is_stationary, ()),
                      (pins.test_als_single_layer_band_stays_exact, ())]:
        try:
            pin(*args)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"{name} passed every ALS pin"


_orig_activation = forward.activation


def _tanh_wrong_constant(name, x):
    x = np.asarray(x, np.float64)
    if name == "gelu_tanh":
        return 0.5 * x * (1.0 + np.tanh(np.sqrt(1.0 / np.pi) * (x + 0.044715 * x ** 3)))
    return _orig_activation(name, x)


def _silu_for_everything(name, x):
    return _orig_activation("silu", x)


def _gelu_exact_for_tanh(name, x):
    return _orig_activation("gelu" if name == "gelu_tanh" else name, x)


@pytest.mark.parametrize("mutant", [_tanh_wrong_constant, _silu_for_everything, _gelu_exact_for_tanh])
def test_activation_mutants_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(forward, "activation", mutant)
    caught = 0
    for pin, args in [(pins.test_activation_matches_library_routines, ("gelu_tanh",)),
                      (pins.test_activation_closed_forms, ()),
                      (pins.test_gate_up_act_brute_force, ())]:
        try:
            pin(*args)
        except AssertionError:
            caught += 1
    assert caught >= 1, f"{mutant.__name__} passed every activation pin"


# --------------------------------------------------------------------------
# call resolution (oracle.workload): band, shared-block group, tied child
# --------------------------------------------------------------------------
import test_oracle_resolution as res_pins  # noqa: E402
from oracle import workload as owl  # noqa: E402


def _interleaved(layer, L, G):
    return layer % G


def _per_type_mlp_key(band, ltype, fam):
    return (band, ltype, fam)


_orig_families_of = owl.OracleWorkload.families_of


def _drop_tied_v(self, layer, call):
    return [f for f in _orig_families_of(self, layer, call) if not self.tied(layer, f)]


def _untied(self, layer, fam):
    return False


@pytest.mark.parametrize("name,target,attr,mutant", [
    ("interleaved bands", owl, "band_of", _interleaved),
    ("MLP W0 per layer type", owl, "w0_key", _per_type_mlp_key),
    ("tied v dropped", owl.OracleWorkload, "families_of", _drop_tied_v),
    ("v evaluated from its own bundle on tied types", owl.OracleWorkload, "tied", _untied),
])
def test_resolution_mutants_are_caught(monkeypatch, name, target, attr, mutant):
    monkeypatch.setattr(target, attr, mutant)
    caught = 0
    for pin, args in [(res_pins.test_direct_workload_calls_match_hand_tables, ()),
                      (res_pins.test_direct_workload_shares_mlp_blocks_across_types, ()),
                      (res_pins.test_decomposed_blocks_are_group_means, ("gate",)),
                      (res_pins.test_decomposed_blocks_are_group_means, ("q",)),
                      (res_pins.test_band_table_is_contiguous, ())]:
        try:
            pin(*args)
        except (AssertionError, KeyError, ValueError):
            caught += 1
    assert caught >= 1, f"{name} passed every resolution pin"


# --------------------------------------------------------------------------
# MXFP4 quantizer
# --------------------------------------------------------------------------
from oracle import quant  # noqa: E402

_orig_mx_exponent = quant.mx_exponent
_orig_e2m1_encode = quant.e2m1_encode


def _ceil_exponent(amax):
    # scale from ceil(log2 amax) - 2: the block maximum lands in (2, 4]
    import math
    return 0 if amax == 0.0 else math.ceil(math.log2(amax)) - 2


def _ties_away(v):
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), 6.0)
    mags = np.abs(quant.E2M1[:8])
    d = np.abs(mags[None, :] - a.reshape(-1, 1))
    idx = np.array([np.flatnonzero(row == row.min())[-1] for row in d])   # the larger on a tie
    return (idx | np.where(np.signbit(v.reshape(-1)) & (idx != 0), 8, 0)).astype(np.uint8).reshape(v.shape)


def _exponent_off_by_one(amax):
    return _orig_mx_exponent(amax) + (1 if amax else 0)


@pytest.mark.parametrize("attr,mutant", [("mx_exponent", _ceil_exponent), ("e2m1_encode", _ties_away),
                                         ("mx_exponent", _exponent_off_by_one)])
def test_mxfp4_mutants_are_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(quant, attr, mutant)
    caught = 0
    for pin in (pins.test_e2m1_rounding_brute_force, pins.test_mx_block_exponent_rule, pins.test_mxfp4_error_bound):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1, f"{mutant.__name__} passed every MXFP4 pin"
