"""Planted mistakes in the oracle (CPU only) must each fail at least one pin.

Every mutation below is a plausible slip in writing the recurrence (a dropped
term, a wrong sign, a wrong index, a transposed operand); the test patches
it into oracle.recurrence for the duration of one check and runs the pins of
test_oracle_pins against it.
"""
import numpy as np
import pytest

from oracle import recurrence as R
from tests import test_oracle_pins as P


def _step_sign(S, g_t, beta_t, v_t, k_t):
    Sd = S * np.exp(g_t)[..., None, None]
    pred = np.einsum("...vk,...k->...v", Sd, k_t)
    delta = beta_t[..., None] * (v_t + pred)
    return Sd, delta, Sd + delta[..., :, None] * k_t[..., None, :]


def _step_undecayed_pred(S, g_t, beta_t, v_t, k_t):
    Sd = S * np.exp(g_t)[..., None, None]
    pred = np.einsum("...vk,...k->...v", S, k_t)
    delta = beta_t[..., None] * (v_t - pred)
    return Sd, delta, Sd + delta[..., :, None] * k_t[..., None, :]


def _step_decay_after_write(S, g_t, beta_t, v_t, k_t):
    pred = np.einsum("...vk,...k->...v", S, k_t)
    delta = beta_t[..., None] * (v_t - pred)
    S_new = (S + delta[..., :, None] * k_t[..., None, :]) * np.exp(g_t)[..., None, None]
    return S * np.exp(g_t)[..., None, None], delta, S_new


def _step_no_beta_on_pred(S, g_t, beta_t, v_t, k_t):
    Sd = S * np.exp(g_t)[..., None, None]
    pred = np.einsum("...vk,...k->...v", Sd, k_t)
    delta = beta_t[..., None] * v_t - pred
    return Sd, delta, Sd + delta[..., :, None] * k_t[..., None, :]


def _step_transposed_state(S, g_t, beta_t, v_t, k_t):
    Sd = S * np.exp(g_t)[..., None, None]
    pred = np.einsum("...kv,...k->...v", Sd, k_t) if Sd.shape[-1] == Sd.shape[-2] else \
        np.einsum("...vk,...k->...v", Sd, k_t)
    delta = beta_t[..., None] * (v_t - pred)
    return Sd, delta, Sd + delta[..., :, None] * k_t[..., None, :]


def _l2norm_no_eps(x):
    x = np.asarray(x, np.float64)
    n = np.sqrt((x * x).sum(-1, keepdims=True))
    return x / np.where(n == 0, 1, n)


def _head_map_modulo(H, HV):
    return np.arange(HV) % H


_paged = R.paged_forward


def _paged_ignores_fresh_flags(q, k, v, g, beta, cu, pool, idx, init=None, scale=None):
    return _paged(q, k, v, g, beta, cu, pool, idx, None, scale)


def _paged_drops_end_states(q, k, v, g, beta, cu, pool, idx, init=None, scale=None):
    o, _ = _paged(q, k, v, g, beta, cu, pool, idx, init, scale)
    return o, np.asarray(pool, np.float64).copy()


def _paged_writes_the_start_state(q, k, v, g, beta, cu, pool, idx, init=None, scale=None):
    o, new = _paged(q, k, v, g, beta, cu, pool, idx, init, scale)
    live = np.asarray(idx) > 0
    if init is not None:
        live &= np.asarray(init) != 0
    new[np.asarray(idx)[live]] = np.asarray(pool, np.float64)[np.asarray(idx)[live]]
    return o, new


_transition = R.transition


def _transition_reverse_order(q, k, v, g, beta, cu, scale=None):
    M, s = _transition(q, k, v, g, beta, cu, scale)
    return np.swapaxes(M, -1, -2), s


MUTATIONS = {
    "transition product transposed (reverse token order)": ("transition",
                                                            _transition_reverse_order),
    "paged: fresh sequences resume from their block": ("paged_forward", _paged_ignores_fresh_flags),
    "paged: end states not written back": ("paged_forward", _paged_drops_end_states),
    "paged: start state written back": ("paged_forward", _paged_writes_the_start_state),
    "delta sign": ("_step", _step_sign),
    "prediction from the undecayed state": ("_step", _step_undecayed_pred),
    "decay after the write": ("_step", _step_decay_after_write),
    "beta dropped on the prediction": ("_step", _step_no_beta_on_pred),
    "transposed state in the prediction": ("_step", _step_transposed_state),
    "eps dropped from the norm": ("l2norm", _l2norm_no_eps),
    "value head -> key head by modulo": ("_head_map", _head_map_modulo),
}

PINS = [
    lambda c: P.test_chunk_form_equals_recurrence(4),
    lambda c: P.test_orthogonal_keys_reduce_to_causal_linear_attention(),
    lambda c: P.test_brute_force_matrix_form_exact(),
    lambda c: P.test_beta_zero_is_pure_decay(),
    lambda c: P.test_scalar_case_is_an_exponential_moving_average(),
    lambda c: P.test_forget_all_decay(),
    lambda c: P.test_grouped_heads_equal_repeated_key_heads(),
    lambda c: P.test_decode_is_one_recurrence_step_with_the_fused_gates(),
    lambda c: P.test_paged_prefix_then_continuation_equals_one_pass(),
    lambda c: P.test_paged_fresh_resumed_and_null_sequences(),
    lambda c: P.test_transition_reproduces_the_end_state_of_any_start_state(),
]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_a_planted_mistake_fails_a_pin(name, monkeypatch, contract):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(R, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin(contract)
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed >= 1, f"no pin caught the mutation: {name}"


def test_the_pins_pass_without_a_mutation(contract):
    for pin in PINS:
        pin(contract)
