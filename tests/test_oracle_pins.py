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
        except (NameError, AttributeError, TypeError):
            raise  # a broken harness or mutant, not a caught mistake
        except Exception:
            failed.append(name)
    return failed


def _mutant(**repl):
    m = types.ModuleType("oracle_mutant")
    m.__dict__.update({k: v for k, v in mo.__dict__.items() if not k.startswith("__")})
    m.__dict__["__builtins__"] = mo.__dict__["__builtins__"]
    # the unmodified functions that mutant wrappers delegate to
    m.__dict__.update(ORIG_ATTEND=mo.attend, ORIG_ROPE=mo.rope, ORIG_SLOT=mo.cache_slot, np=np,
                      math=math)
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


def _rope_sign(x, pos, theta=10000.0):
    return ORIG_ROPE(x, -np.asarray(pos), theta)


def _rope_half_split(x, pos, theta=10000.0):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.asarray(pos, np.float64)[..., None] * theta ** (-2.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def _rope_freq(x, pos, theta=10000.0):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.asarray(pos, np.float64)[..., None] * theta ** (-1.0 * i / d)
    c, s = np.cos(ang), np.sin(ang)
    y = np.empty_like(x)
    y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    y[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return y


def _slot_off_by_one(b, pos, block_table, block_size, seq_stride):
    return ORIG_SLOT(b, pos + 1, block_table, block_size, seq_stride)


ORIG_ROPE = mo.rope
ORIG_SLOT = mo.cache_slot

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
    "rope rotates the wrong way": dict(rope=_rope_sign),
    "rope pairs halves": dict(rope=_rope_half_split),
    "rope frequency exponent": dict(rope=_rope_freq),
    "cache append off by one": dict(cache_slot=_slot_off_by_one),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    repl = dict(MUTANTS[name])
    # wrappers delegate to the unmodified functions (ORIG_*), which stay
    # bound to the original oracle module
    m = _mutant(**repl)
    failed = _failing_pins(m)
    assert failed, f"planted mistake '{name}' passed every pin"


def test_mutant_harness_is_clean():
    """An unmodified copy of the oracle passes every pin, so a failure above is
    caused by the planted mistake and not by the harness."""
    assert _failing_pins(_mutant()) == []
