"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
in test_oracle_pins.py catch every one of them.

Each mutant replaces one oracle function with a copy that carries a single
mistake; the pins are then run against the mutated oracle and at least one
must fail.
"""
import numpy as np
import pytest

import oracle
import oracle.prism as op
from tests import test_oracle_pins as pins

PIN_TESTS = [
    (pins.test_anchor_is_numpy_convolve, {}),
    (pins.test_chain_iterated_equals_closed_form, {"L": 3}),
    (pins.test_chain_iterated_equals_closed_form, {"L": 5}),
    (pins.test_L1_reduces_to_gdn_delta_form, {}),
    (pins.test_delta_rule_writes_value_at_key_L1, {}),
    (pins.test_delta_rule_with_rank_terms, {}),
    (pins.test_beta0_is_causal_linear_attention, {"gated": False}),
    (pins.test_beta0_is_causal_linear_attention, {"gated": True}),
    (pins.test_brute_force_dense_sum, {"L": 1}),
    (pins.test_brute_force_dense_sum, {"L": 3}),
    (pins.test_tree_order_scan_matches, {}),
    (pins.test_write_has_rank_L, {"L": 4}),
    (pins.test_linear_in_v, {}),
]


def _anchor_reversed(v, w, t):
    acc = np.zeros(v.shape[:-2] + v.shape[-1:])
    for j in range(4):
        s = t - 3 + j
        if s >= 0:
            acc = acc + w[..., 3 - j, :] * v[..., s, :]
    return acc


def _anchor_skips_t(v, w, t):
    acc = np.zeros(v.shape[:-2] + v.shape[-1:])
    for j in range(4):
        s = t - 4 + j
        if s >= 0:
            acc = acc + w[..., j, :] * v[..., s, :]
    return acc


def _chain_alpha_off_by_one(r0, alpha_t, gamma_t, L):
    r = r0
    res, wr = [], []
    for l in range(1, L):
        r = r - alpha_t[..., l, None] * gamma_t[..., l - 1, :] * r
        res.append(r)
        wr.append(alpha_t[..., l, None] * r)
    return res, wr


def _chain_written_uses_prev_alpha(r0, alpha_t, gamma_t, L):
    r = r0
    res, wr = [], []
    for l in range(1, L):
        r = r - alpha_t[..., l - 1, None] * gamma_t[..., l - 1, :] * r
        res.append(r)
        wr.append(alpha_t[..., l - 1, None] * r)
    return res, wr


def _make_step(mistake):
    def step(S, q_t, k_t, v_t, g_t, beta_t, anchor_t, u_t, alpha_t, gamma_t, L):
        vals = [(1.0 if mistake == "no_beta_write" else beta_t[:, None]) * v_t]
        keys = [k_t]
        if L > 1:
            _, written = op.residual_chain(v_t - anchor_t, alpha_t, gamma_t, L)
            for l in range(1, L):
                vals.append(written[l - 1])
                keys.append(k_t if mistake == "k_for_u" else u_t[:, l - 1, :])
        B_t = np.matmul(np.stack(vals, axis=2), np.stack(keys, axis=1))
        Sk = np.matmul(S, k_t[:, :, None])[:, :, 0]
        sign = 1.0 if mistake == "erase_sign" else -1.0
        core = S + sign * beta_t[:, None, None] * Sk[:, :, None] * k_t[:, None, :]
        if mistake == "decay_write":
            S_new = g_t[:, None, None] * (core + B_t)
        else:
            S_new = g_t[:, None, None] * core + B_t
        if mistake == "read_before_write":
            o_t = np.matmul(S, q_t[:, :, None])[:, :, 0]
        elif mistake == "transposed_read":
            o_t = np.matmul(np.swapaxes(S_new, 1, 2), q_t[:, :, None])[:, :, 0]
        else:
            o_t = np.matmul(S_new, q_t[:, :, None])[:, :, 0]
        return S_new, o_t
    return step


MUTANTS = {
    "anchor_reversed_taps": ("shortconv_anchor", _anchor_reversed),
    "anchor_skips_token_t": ("shortconv_anchor", _anchor_skips_t),
    "chain_alpha_off_by_one": ("residual_chain", _chain_alpha_off_by_one),
    "written_value_prev_alpha": ("residual_chain", _chain_written_uses_prev_alpha),
    "erase_sign": ("token_step", _make_step("erase_sign")),
    "decay_applied_to_write": ("token_step", _make_step("decay_write")),
    "readout_before_write": ("token_step", _make_step("read_before_write")),
    "transposed_readout": ("token_step", _make_step("transposed_read")),
    "beta_dropped_from_write": ("token_step", _make_step("no_beta_write")),
    "k_used_for_u": ("token_step", _make_step("k_for_u")),
}


def test_unmutated_oracle_passes_every_pin():
    for fn, kw in PIN_TESTS:
        fn(**kw)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fake = MUTANTS[name]
    monkeypatch.setattr(op, attr, fake)
    monkeypatch.setattr(oracle, attr, fake)
    caught = []
    for fn, kw in PIN_TESTS:
        try:
            fn(**kw)
        except (AssertionError, ValueError):   # a shape error also exposes it
            caught.append(fn.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
