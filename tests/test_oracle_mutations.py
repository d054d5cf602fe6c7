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
