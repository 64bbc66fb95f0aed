"""Planted mistakes in the oracle must be caught by its pins.

Each mutant replaces one piece of the fp64 oracle (on the CPU, through
monkeypatch) with a plausible error: a dropped term, a wrong sign, a wrong
index, a wrong base or bias.  The pins of ``test_oracle_pins`` then run
against the mutated oracle, and at least one of them has to fail.  This is
what makes the pins a check of the oracle rather than of themselves.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import test_oracle_pins as P
from oracle import mla_oracle as orc

_orig_attend = orc.attend
_orig_merge = orc.merge_segments


def _attend_without_rope(q, rows, scale, sink=None):
    return _orig_attend(np.concatenate([q[:, :512], np.zeros_like(q[:, 512:])], axis=1),
                        rows, scale, sink)


def _attend_base2_lse(q, rows, scale, sink=None):
    o, l = _orig_attend(q, rows, scale, sink)
    return o, l / math.log(2.0)


def _attend_sink_sign(q, rows, scale, sink=None):
    return _orig_attend(q, rows, scale, None if sink is None else -np.asarray(sink))


def _attend_value_offset(q, rows, scale, sink=None):
    # V taken from dims 64..575 instead of the first 512 (scores unchanged)
    M, n = q.shape[0], rows.shape[0]
    out = np.zeros((M, 512))
    lse = np.full(M, -np.inf)
    if n:
        s = scale * (q @ rows.T)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1)
        lse = m[:, 0] + np.log(z)
        out = (e @ rows[:, 64:576]) / z[:, None]
    if sink is not None:
        sink = np.broadcast_to(np.asarray(sink, dtype=np.float64), (M,))
        new = np.logaddexp(lse, sink)
        out = out * (np.where(np.isfinite(lse), np.exp(lse - new), 0.0) if n else np.zeros(M))[:, None]
        lse = new
    return out, lse


def _attend_no_scale(q, rows, scale, sink=None):
    return _orig_attend(q, rows, 1.0, sink)


def _row_index_swapped(bt_row, j, B):
    return int(bt_row[j % len(bt_row)]) * B + j // B if len(bt_row) else 0


def _visible_off_by_one(seq_len, qlen, i, causal):
    return seq_len if not causal else max(0, seq_len - qlen + i)


def _tps_floor(seq_len, S, tile):
    return max(1, seq_len // (S * tile))


def _partials_natural_exp(q, rows, scale, start, end, n_visible):
    M = q.shape[0]
    hi = min(end, n_visible)
    if hi <= start:
        return (np.zeros((M, 512)), np.full(M, -np.inf), np.zeros(M))
    seg = rows[start:hi]
    x = (scale * orc.LOG2E) * (q @ seg.T)
    m = x.max(axis=1)
    p = np.exp(x - m[:, None])
    return p @ seg[:, :512], m, p.sum(axis=1)


def _merge_unweighted_sum(so, sm, se, part_lens, tile, sinks=None):
    # the exp-sums are added without the 2^(m_s - M) rescale
    T, H, S, D = so.shape
    out = np.zeros((T, H, D))
    lse = np.full((T, H), -np.inf)
    for t in range(T):
        nv = len(orc.segment_bounds(int(part_lens[t]), S, tile))
        if nv == 0:
            continue
        m = sm[t, :, :nv]
        M = m.max(axis=1)
        w8 = np.where(np.isfinite(m), np.exp2(m - M[:, None]), 0.0)
        L = se[t, :, :nv].sum(axis=1)
        out[t] = np.einsum("hs,hsd->hd", w8, so[t, :, :nv]) / L[:, None]
        lse[t] = orc.LOGE2 * (M + np.log2(L))
    if sinks is not None:
        new = np.logaddexp(lse, np.asarray(sinks)[None])
        out = out * np.where(np.isfinite(lse), np.exp(lse - new), 0.0)[:, :, None]
        lse = new
    return out, lse


def _merge_sink_no_rescale(so, sm, se, part_lens, tile, sinks=None):
    o, l = _orig_merge(so, sm, se, part_lens, tile, None)
    if sinks is not None:
        l = np.logaddexp(l, np.asarray(sinks)[None])
    return o, l


_orig_combine = orc.combine_lse


def _combine_base2(shard_out, shard_lse, sinks=None):
    # shard weights as 2^(lse_w - lse) instead of e^(lse_w - lse)
    return _orig_combine(shard_out, np.asarray(shard_lse) / math.log(2.0), sinks)


def _combine_sink_per_shard(shard_out, shard_lse, sinks=None):
    if sinks is None:
        return _orig_combine(shard_out, shard_lse)
    outs, lses = [], []
    for w in range(np.asarray(shard_out).shape[0]):
        o, l = _orig_combine(shard_out[w:w + 1], shard_lse[w:w + 1], sinks)
        outs.append(o)
        lses.append(l)
    return _orig_combine(np.stack(outs), np.stack(lses))


def _e4m3_bias8():
    def v(c):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if e == 15 and m == 7:
            return math.nan
        return s * (m / 8.0) * 2.0 ** -7 if e == 0 else s * (1 + m / 8.0) * 2.0 ** (e - 8)
    return np.array([v(c) for c in range(256)])


def _bf16_shift15(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return b.view(np.float32).astype(np.float64)


MUTANTS = {
    "score drops the rope dims": ("attend", _attend_without_rope),
    "LSE left in base 2": ("attend", _attend_base2_lse),
    "sink with the wrong sign": ("attend", _attend_sink_sign),
    "value read at the wrong offset": ("attend", _attend_value_offset),
    "softmax scale dropped": ("attend", _attend_no_scale),
    "page index and offset swapped": ("cache_row_index", _row_index_swapped),
    "causal window one short": ("visible_len", _visible_off_by_one),
    "segment span rounded down": ("tiles_per_segment", _tps_floor),
    "partials in natural exp": ("segment_partials", _partials_natural_exp),
    "merge drops the exp-sum rescale": ("merge_segments", _merge_unweighted_sum),
    "merge leaves the output unscaled by the sink": ("merge_segments", _merge_sink_no_rescale),
    "e4m3 exponent bias 8": ("_E4M3_TABLE", _e4m3_bias8()),
    "bf16 widened by 15 bits": ("decode_bf16", _bf16_shift15),
    "tile rule without the 128 cap": ("tile_size_for_block", lambda b: orc.largest_pow2_divisor(b)),
    "shard combine weighs in base 2": ("combine_lse", _combine_base2),
    "shard combine adds the sink on every shard": ("combine_lse", _combine_sink_per_shard),
}

# Cheapest pins first; a mutant only has to trip one of them.
PINS = [
    ("tile rule", P.test_tile_rule_closed_form),
    ("segment bounds", P.test_segment_bounds_worked_examples),
    ("e4m3 table", P.test_e4m3_table_matches_torch_cast),
    ("e4m3 definition", P.test_e4m3_definition_points),
    ("bf16 decode", P.test_bf16_decode_matches_torch_cast),
    ("single key", P.test_single_key_closed_form),
    ("identical keys", P.test_identical_keys_closed_form),
    ("sink only", P.test_sink_only_row),
    ("zero query partials", P.test_zero_query_integer_partials),
    ("base-2 segment", P.test_single_key_segment_is_base2),
    ("rope shift", P.test_rope_shift_closed_form),
    ("partition invariance", lambda: P.test_partition_invariance(4)),
    ("sdpa", P.test_oracle_matches_torch_sdpa_identity_table),
    ("brute force bf16", lambda: P.test_oracle_matches_brute_force("bf16", False, False)),
    ("brute force causal sinks", lambda: P.test_oracle_matches_brute_force("bf16", True, True)),
    ("brute force fp8 causal", lambda: P.test_oracle_matches_brute_force("fp8_e4m3", True, False)),
    ("combine closed forms", P.test_combine_lse_closed_forms),
    ("dcp shards", lambda: P.test_dcp_shards_combine_to_the_direct_decode(2, True)),
]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant, monkeypatch):
    attr, repl = MUTANTS[mutant]
    monkeypatch.setattr(orc, attr, repl)
    caught = []
    for name, pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught.append(name)
            break
    assert caught, f"no pin caught the planted mistake: {mutant}"
