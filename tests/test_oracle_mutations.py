"""Each plausible mistake planted in the oracle must fail at least one pin.

The mutations are applied on the CPU with ``monkeypatch`` to the oracle
module only; they show that the pins are strong enough to catch a dropped
term, a wrong sign or index, or a transposed operand.
"""

import math

import numpy as np
import pytest

from oracle import pa_oracle as O
from tests import oracle_pins as P


def _gather_k_transposed_x(key_cache, value_cache, row, seq_len, bs):
    # dim d = j * (D/x) + c instead of c * x + j
    nb, hkv, dx, _, x = key_cache.shape
    n = (seq_len + bs - 1) // bs
    phys = np.asarray(row[:n], dtype=np.int64)
    k = key_cache[phys].transpose(0, 3, 1, 4, 2).reshape(n * bs, hkv, dx * x)
    v = value_cache[phys].transpose(0, 3, 1, 2).reshape(n * bs, hkv, dx * x)
    return k[:seq_len], v[:seq_len]


def _gather_v_wrong_axes(key_cache, value_cache, row, seq_len, bs):
    # V read as [.., bs, D] instead of [.., D, bs]
    k, _ = O.__dict__["_orig_gather"](key_cache, value_cache, row, seq_len, bs)
    nb, hkv, d, _ = value_cache.shape
    n = (seq_len + bs - 1) // bs
    phys = np.asarray(row[:n], dtype=np.int64)
    v = value_cache[phys].reshape(n, hkv, bs, d).transpose(0, 2, 1, 3).reshape(n * bs, hkv, d)
    return k, v[:seq_len]


def _gather_slot_off_by_one(key_cache, value_cache, row, seq_len, bs):
    # token t read from slot (t + 1) of the gathered sequence (wrapping)
    k, v = O.__dict__["_orig_gather"](key_cache, value_cache, row, seq_len, bs)
    return np.roll(k, -1, axis=0), np.roll(v, -1, axis=0)


def _window(s, window_left):
    if window_left >= 0:
        s[:, :max(0, s.shape[1] - 1 - window_left)] = -np.inf
    return s


def _logits_gqa_modulo(q, k, scale, slopes, window_left=-1, soft_cap=0.0):
    nh = q.shape[0]
    hkv = k.shape[1]
    s = np.stack([(k[:, h % hkv, :] @ q[h]) * scale for h in range(nh)])
    if soft_cap > 0.0:
        s = soft_cap * np.tanh(s / soft_cap)
    if slopes is not None:
        s = s + np.asarray(slopes)[:, None] * np.arange(k.shape[0])[None, :]
    return _window(s, window_left)


def _logits_alibi_relative(q, k, scale, slopes, window_left=-1, soft_cap=0.0):
    s = O.__dict__["_orig_logits"](q, k, scale, None, window_left, soft_cap)
    if slopes is not None:
        L = k.shape[0]
        s = s + np.asarray(slopes)[:, None] * (np.arange(L) - (L - 1))[None, :]
    return s


def _logits_alibi_scaled(q, k, scale, slopes, window_left=-1, soft_cap=0.0):
    s = O.__dict__["_orig_logits"](q, k, 1.0, slopes, window_left, soft_cap)
    return s * scale


def _logits_no_scale(q, k, scale, slopes, window_left=-1, soft_cap=0.0):
    return O.__dict__["_orig_logits"](q, k, 1.0, slopes, window_left, soft_cap)


def _logits_alibi_sign(q, k, scale, slopes, window_left=-1, soft_cap=0.0):
    s = O.__dict__["_orig_logits"](q, k, scale, None, window_left, soft_cap)
    if slopes is not None:
        s = s - np.asarray(slopes)[:, None] * np.arange(k.shape[0])[None, :]
    return s


def _logits_window_off_by_one(q, k, scale, slopes, window_left=-1, soft_cap=0.0):
    # one key fewer: t >= L - W instead of t >= L - 1 - W
    s = O.__dict__["_orig_logits"](q, k, scale, slopes, -1, soft_cap)
    if window_left >= 0:
        s[:, :max(0, k.shape[0] - window_left)] = -np.inf
    return s


def _logits_window_from_start(q, k, scale, slopes, window_left=-1, soft_cap=0.0):
    # window anchored at the first key instead of the query position
    s = O.__dict__["_orig_logits"](q, k, scale, slopes, -1, soft_cap)
    if window_left >= 0:
        s[:, window_left + 1:] = -np.inf
    return s


def _logits_cap_after_alibi(q, k, scale, slopes, window_left=-1, soft_cap=0.0):
    s = O.__dict__["_orig_logits"](q, k, scale, slopes, -1, 0.0)
    if soft_cap > 0.0:
        s = soft_cap * np.tanh(s / soft_cap)
    return _window(s, window_left)


def _logits_cap_inside_unscaled(q, k, scale, slopes, window_left=-1, soft_cap=0.0):
    # c * tanh(s) instead of c * tanh(s / c)
    s = O.__dict__["_orig_logits"](q, k, scale, None, -1, 0.0)
    if soft_cap > 0.0:
        s = soft_cap * np.tanh(s)
    if slopes is not None:
        s = s + np.asarray(slopes)[:, None] * np.arange(k.shape[0])[None, :]
    return _window(s, window_left)


def _logits_cap_ignored(q, k, scale, slopes, window_left=-1, soft_cap=0.0):
    return O.__dict__["_orig_logits"](q, k, scale, slopes, window_left, 0.0)


def _logits_window_ignored(q, k, scale, slopes, window_left=-1, soft_cap=0.0):
    return O.__dict__["_orig_logits"](q, k, scale, slopes, -1, soft_cap)


def _partials_masked_partition_zero_max(s, v, max_p, ps=O.PARTITION_SIZE):
    # a partition with no visible key reported with max 0 / sum 1 (as if it held one token)
    ml, es, to = O.__dict__["_orig_partials"](s, v, max_p, ps)
    L = s.shape[1]
    n = O.num_partitions(L, ps)
    dead = np.isneginf(ml[:, :n]) & (es[:, :n] == 0)
    ml[:, :n] = np.where(dead, 0.0, ml[:, :n])
    es[:, :n] = np.where(dead, 1.0, es[:, :n])
    return ml, es, to


def _partials_unnormalised(s, v, max_p, ps=O.PARTITION_SIZE):
    ml, es, to = O.__dict__["_orig_partials"](s, v, max_p, ps)
    return ml, es, to * es[:, :, None]


def _partials_pad_zero(s, v, max_p, ps=O.PARTITION_SIZE):
    ml, es, to = O.__dict__["_orig_partials"](s, v, max_p, ps)
    ml = np.where(np.isneginf(ml), 0.0, ml)
    return ml, es, to


def _partials_last_token_dropped(s, v, max_p, ps=O.PARTITION_SIZE):
    return O.__dict__["_orig_partials"](s[:, :-1] if s.shape[1] > 1 else s,
                                        v[:-1] if v.shape[0] > 1 else v, max_p, ps)


def _merge_without_sums(ml, es, to, n):
    m = ml[:, :n]
    r = np.exp(m - m.max(axis=1)[:, None])
    w = r / r.sum(axis=1)[:, None]
    return np.einsum("hp,hpd->hd", w, to[:, :n, :])


def _merge_without_rescale(ml, es, to, n):
    r = es[:, :n]
    w = r / r.sum(axis=1)[:, None]
    return np.einsum("hp,hpd->hd", w, to[:, :n, :])


def _softmax_wrong_axis_max(s, v):
    w = np.exp(s - s.max(axis=0, keepdims=True))
    return O._weighted_values(w, v) / w.sum(axis=1)[:, None]


def _num_partitions_floor(L, ps=O.PARTITION_SIZE):
    return max(1, L // ps)


def _fp8_bias_8():
    t = O.fp8_e4m3fn_table()
    return t / 2.0


def _decode_bf16_low(raw, kind):
    if kind == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32)
        return bits.view(np.float32).astype(np.float64)
    return O.__dict__["_orig_decode"](raw, kind)


MUTATIONS = {
    "k_x_packing_transposed": ("gather_sequence", _gather_k_transposed_x),
    "v_axes_swapped": ("gather_sequence", _gather_v_wrong_axes),
    "token_slot_off_by_one": ("gather_sequence", _gather_slot_off_by_one),
    "gqa_head_modulo": ("sequence_logits", _logits_gqa_modulo),
    "alibi_relative_positions": ("sequence_logits", _logits_alibi_relative),
    "alibi_bias_scaled": ("sequence_logits", _logits_alibi_scaled),
    "scale_dropped": ("sequence_logits", _logits_no_scale),
    "alibi_sign_flipped": ("sequence_logits", _logits_alibi_sign),
    "partition_output_unnormalised": ("partition_partials", _partials_unnormalised),
    "padding_max_zero": ("partition_partials", _partials_pad_zero),
    "last_token_dropped": ("partition_partials", _partials_last_token_dropped),
    "merge_drops_exp_sums": ("merge_partials", _merge_without_sums),
    "merge_drops_rescale": ("merge_partials", _merge_without_rescale),
    "softmax_max_over_heads": ("softmax_output", _softmax_wrong_axis_max),
    "partition_count_floor": ("num_partitions", _num_partitions_floor),
    "bf16_decode_low_half": ("decode_storage", _decode_bf16_low),
    "window_off_by_one": ("sequence_logits", _logits_window_off_by_one),
    "window_from_first_key": ("sequence_logits", _logits_window_from_start),
    "window_ignored": ("sequence_logits", _logits_window_ignored),
    "soft_cap_after_alibi": ("sequence_logits", _logits_cap_after_alibi),
    "soft_cap_without_inner_division": ("sequence_logits", _logits_cap_inside_unscaled),
    "soft_cap_ignored": ("sequence_logits", _logits_cap_ignored),
    "masked_partition_not_padding": ("partition_partials", _partials_masked_partition_zero_max),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS) + ["fp8_exponent_bias_8"])
def test_mutation_is_caught(name, monkeypatch):
    monkeypatch.setitem(O.__dict__, "_orig_gather", O.gather_sequence)
    monkeypatch.setitem(O.__dict__, "_orig_logits", O.sequence_logits)
    monkeypatch.setitem(O.__dict__, "_orig_partials", O.partition_partials)
    monkeypatch.setitem(O.__dict__, "_orig_decode", O.decode_storage)
    if name == "fp8_exponent_bias_8":
        bad = _fp8_bias_8()
        monkeypatch.setattr(O, "_FP8_TABLE", bad)
        monkeypatch.setattr(O, "fp8_e4m3fn_table", lambda: bad.copy())
    else:
        attr, fn = MUTATIONS[name]
        monkeypatch.setattr(O, attr, fn)
    with pytest.raises(AssertionError):
        P.run_all_pins()


def test_unmutated_oracle_passes_all_pins():
    P.run_all_pins()
