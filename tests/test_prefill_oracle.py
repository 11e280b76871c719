"""The paged-prefill oracle against its pins (CPU), and planted mistakes in
copies of it that the pins must catch."""

import numpy as np
import pytest

from oracle import prefill_oracle as P
from tests import prefill_pins as PP


@pytest.mark.parametrize("pin", [PP.pin_prefill_dense, PP.pin_prefill_causal_square,
                                 PP.pin_prefill_one_query_is_decode, PP.pin_prefill_zero_query,
                                 PP.pin_prefill_invariants])
def test_prefill_pin(pin):
    pin()


_orig_visible = P.visible_keys


def _visible_top_left(num_q, num_k, causal, wl, wr):
    p = np.arange(num_q)[:, None]
    t = np.arange(num_k)[None, :]
    vis = np.ones((num_q, num_k), dtype=bool)
    if causal:
        vis &= t <= p
    if wl >= 0:
        vis &= t >= p - wl
    if wr >= 0:
        vis &= t <= p + wr
    return vis


def _visible_window_off_by_one(num_q, num_k, causal, wl, wr):
    return _orig_visible(num_q, num_k, causal, wl + 1 if wl >= 0 else wl, wr)


def _visible_right_ignored(num_q, num_k, causal, wl, wr):
    return _orig_visible(num_q, num_k, causal, wl, -1)


def _visible_causal_strict(num_q, num_k, causal, wl, wr):
    vis = _orig_visible(num_q, num_k, causal, wl, wr)
    if causal:
        p = (num_k - num_q + np.arange(num_q))[:, None]
        vis &= np.arange(num_k)[None, :] < p
    return vis


_orig_sequence = P.prefill_sequence


def _sequence_gqa_modulo(q, k, v, scale, visible, soft_cap=0.0):
    hkv = k.shape[1]
    out = np.zeros(q.shape)
    for h in range(q.shape[1]):
        out[:, h:h + 1] = _orig_sequence(q[:, h:h + 1], k[:, h % hkv:h % hkv + 1],
                                         v[:, h % hkv:h % hkv + 1], scale, visible, soft_cap)
    return out


def _sequence_no_scale(q, k, v, scale, visible, soft_cap=0.0):
    return _orig_sequence(q, k, v, 1.0, visible, soft_cap)


def _sequence_cap_ignored(q, k, v, scale, visible, soft_cap=0.0):
    return _orig_sequence(q, k, v, scale, visible, 0.0)


def _sequence_masked_rows_mean(q, k, v, scale, visible, soft_cap=0.0):
    out = _orig_sequence(q, k, v, scale, visible, soft_cap)
    empty = ~visible.any(axis=1)
    out[empty] = v.mean(axis=0).mean(axis=0)
    return out


def _gather_slot_swapped(key_cache, value_cache, table_row, num_keys):
    bs = key_cache.shape[2]
    t = np.arange(num_keys)
    phys = np.asarray(table_row)[t // bs]
    slot = (bs - 1 - t % bs)
    return key_cache[phys, :, slot, :], value_cache[phys, :, slot, :]




MUTATIONS = {
    "causal_top_left": ("visible_keys", _visible_top_left),
    "window_left_off_by_one": ("visible_keys", _visible_window_off_by_one),
    "window_right_ignored": ("visible_keys", _visible_right_ignored),
    "causal_excludes_diagonal": ("visible_keys", _visible_causal_strict),
    "gqa_head_modulo": ("prefill_sequence", _sequence_gqa_modulo),
    "scale_dropped": ("prefill_sequence", _sequence_no_scale),
    "soft_cap_ignored": ("prefill_sequence", _sequence_cap_ignored),
    "masked_rows_not_zero": ("prefill_sequence", _sequence_masked_rows_mean),
    "slot_order_reversed": ("gather_sequence_nhd", _gather_slot_swapped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_prefill_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(P, attr, fn)
    with pytest.raises(AssertionError):
        PP.run_all_prefill_pins()
