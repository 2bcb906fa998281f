"""The RWKV-4 WKV oracle against its pins (CPU only), and planted mistakes
in it that each fail at least one pin."""
import numpy as np
import pytest

from oracle import wkv4_oracle as O4
from tests import wkv4_pins as P4


@pytest.mark.parametrize("pin", P4.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


_ORIG = O4.wkv4_forward


MUTATIONS = {
    # (attribute, replacement)
    "decay_sign": ("wkv4_forward", lambda w, u, k, v, state0=None: _ORIG(-np.asarray(w, float), u, k, v, state0)),
    "no_bonus": ("wkv4_forward", lambda w, u, k, v, state0=None:
                 _ORIG(w, np.zeros_like(np.asarray(u, float)), k, v, state0)),
    "bonus_sign": ("wkv4_forward", lambda w, u, k, v, state0=None: _ORIG(w, -np.asarray(u, float), k, v, state0)),
    "lag_off_by_one": ("_past_weights", lambda t, w, ek:
                       np.exp(-(t - np.arange(t))[None, :, None] * w[None, None, :]) * ek[:, :t]),
    "past_without_key": ("_past_weights", lambda t, w, ek:
                         np.exp(-(t - 1 - np.arange(t))[None, :, None] * w[None, None, :]) * np.ones_like(ek[:, :t])),
    "state_decay_off_by_one": ("_state_decay", lambda n, w: np.exp(-max(n - 1, 0) * w)[None, :]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O4, attr, fn)
    failed = []
    for pin in P4.ALL_PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
