"""The oracle against its pins, and planted mistakes that the pins must catch."""
import math
import types

import numpy as np
import pytest

import oracle.mla_oracle as mo
from tests.oracle_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    fn, tol = PINS[name]
    err = fn(mo)
    assert err <= tol, f"{name}: {err}"


def _failing_pins(module):
    failed = []
    for name, (fn, tol) in PINS.items():
        try:
            with np.errstate(all="ignore"):
                err = fn(module)
            if not (err <= tol):
                failed.append(name)
        except Exception:
            failed.append(name)
    return failed


def _mutant(**repl):
    m = types.ModuleType("oracle_mutant")
    m.__dict__.update({k: v for k, v in mo.__dict__.items() if not k.startswith("__")})
    m.__dict__["__builtins__"] = mo.__dict__["__builtins__"]
    for k, v in repl.items():
        if callable(v) and not isinstance(v, type):
            v = types.FunctionType(v.__code__, m.__dict__, k, v.__defaults__, v.__closure__)
        m.__dict__[k] = v
    # re-home every oracle function so calls between them see the mutation
    for k, v in list(m.__dict__.items()):
        if isinstance(v, types.FunctionType) and v.__module__ == mo.__name__ and k not in repl:
            m.__dict__[k] = types.FunctionType(v.__code__, m.__dict__, k, v.__defaults__,
                                               v.__closure__)
    return m


def _kv_no_rope(rows, w_uk_h, w_uv_h, d_c):
    c = rows[:, :d_c]
    K = np.concatenate([c @ w_uk_h, 0.0 * rows[:, d_c:]], axis=1)
    return K, c @ w_uv_h


def _kv_swapped(rows, w_uk_h, w_uv_h, d_c):
    c = rows[:, :d_c]
    return np.concatenate([c @ w_uv_h, rows[:, d_c:]], axis=1), c @ w_uk_h


def _window_off_by_one(n_keys, S):
    j = np.arange(n_keys)[None, :]
    s = np.arange(S)[:, None]
    return j < (n_keys - S + s)


def _combine_no_max(outs, lses):
    w = np.exp(np.asarray(lses, np.float64) * 1.0)
    z = w.sum(axis=0)
    return (w[..., None] * outs).sum(axis=0) / z[..., None], np.log(z)


def _combine_unnormalised(outs, lses):
    lses = np.asarray(lses, np.float64)
    m = lses.max(axis=0)
    w = np.exp(lses - m)
    return (w[..., None] * outs).sum(axis=0), m + np.log(w.sum(axis=0))


def _vup_head0(x, w_uv):
    return np.stack([x[:, h, :] @ w_uv[0] for h in range(x.shape[1])], axis=1)


def _absorb_wrong_head(q_nope, w_uk):
    H = q_nope.shape[1]
    return np.stack([q_nope[:, h, :] @ w_uk[(h + 1) % H].T for h in range(H)], axis=1)


def _attend_log2(q, K, V, scale, visible=None):
    o, l = ORIG_ATTEND(q, K, V, scale, visible)
    return o, l / math.log(2.0)


def _attend_noscale(q, K, V, scale, visible=None):
    return ORIG_ATTEND(q, K, V, 1.0, visible)


ORIG_ATTEND = mo.attend

MUTANTS = {
    "dropped rope key": dict(materialize_kv=_kv_no_rope),
    "W_UK/W_UV swapped": dict(materialize_kv=_kv_swapped),
    "causal window off by one": dict(causal_window_visible=_window_off_by_one),
    "combine without max shift": dict(lse_combine=_combine_no_max),
    "combine not normalised": dict(lse_combine=_combine_unnormalised),
    "v_up uses head 0": dict(v_up=_vup_head0),
    "q_absorb wrong head": dict(q_absorb=_absorb_wrong_head),
    "lse in log2": dict(attend=_attend_log2),
    "scale dropped": dict(attend=_attend_noscale),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    repl = dict(MUTANTS[name])
    # wrappers around the original attend must stay bound to the original
    m = _mutant(**repl)
    failed = _failing_pins(m)
    assert failed, f"planted mistake '{name}' passed every pin"


def test_mutant_harness_is_clean():
    """An unmodified copy of the oracle passes every pin, so a failure above is
    caused by the planted mistake and not by the harness."""
    assert _failing_pins(_mutant()) == []
