"""Planted mistakes in the oracle must be caught by the pins (CPU only).

Each mutant is a plausible slip -- a dropped rescale, a strict causal boundary,
a missing scale, swapped operands, a flipped sign -- applied to a copy of an
oracle function through monkeypatching. The test asserts that at least one of
the pinned facts no longer holds for the mutant, so the pins are strong enough
to expose it.
"""

import math

import numpy as np
import pytest

import oracle.direct as oa
import oracle.online_softmax as oo


def _pin_scalar(fold_only=False):
    q = np.ones((1, 1, 1, 1))
    k = [np.zeros((1, 1, 1, 1)), np.full((1, 1, 1, 1), 10.0)]
    v = [np.zeros((1, 1, 1, 1)), np.ones((1, 1, 1, 1))]
    exact = math.exp(10) / (1 + math.exp(10))
    ok = abs(oo.ring_attention_fold(q, k, v, kv_offsets=[0, 1], scale=1.0)[0].item() - exact) < 1e-15
    if not fold_only:
        ok &= abs(oa.attention(q, k, v, kv_offsets=[0, 1], scale=1.0)["out"].item() - exact) < 1e-15
    return ok


def _pin_single_key():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((1, 1, 1, 4)), rng.standard_normal((1, 1, 5, 4)), rng.standard_normal((1, 1, 5, 4))
    out = oa.attention(q, [k], [v], q_positions=[50], kv_offsets=[50], causal=True)["out"]
    fold = oo.ring_attention_fold(q, [k], [v], q_positions=[50], kv_offsets=[50], causal=True)[0]
    return np.array_equal(out[0, 0, 0], v[0, 0, 0]) and np.max(np.abs(fold[0, 0, 0] - v[0, 0, 0])) == 0


def _pin_brute():
    rng = np.random.default_rng(4)
    q, k, v = rng.standard_normal((1, 1, 3, 2)), rng.standard_normal((1, 1, 4, 2)), rng.standard_normal((1, 1, 4, 2))
    ref = np.zeros((3, 2))
    for i in range(3):
        s = [0.5 * float(q[0, 0, i] @ k[0, 0, j]) for j in range(4)]
        w = [math.exp(x - max(s)) for x in s]
        ref[i] = sum(w[j] * v[0, 0, j] for j in range(4)) / sum(w)
    a = oa.attention(q, [k[:, :, :1], k[:, :, 1:]], [v[:, :, :1], v[:, :, 1:]], scale=0.5)["out"][0, 0]
    f = oo.ring_attention_fold(q, [k[:, :, :1], k[:, :, 1:]], [v[:, :, :1], v[:, :, 1:]], scale=0.5)[0][0, 0]
    return np.max(np.abs(a - ref)) < 1e-13 and np.max(np.abs(f - ref)) < 1e-13


def _pin_mass():
    q = np.ones((1, 1, 1, 1))
    k = [np.zeros((1, 1, 1, 1)), np.zeros((1, 1, 3, 1))]
    v = [np.zeros((1, 1, 1, 1)), np.ones((1, 1, 3, 1))]
    return abs(oo.ring_attention_fold(q, k, v, scale=1.0)[0].item() - 0.75) < 1e-15


ALL_PINS = [_pin_scalar, _pin_single_key, _pin_brute, _pin_mass]


def test_unmutated_oracle_passes_every_pin():
    assert all(p() for p in ALL_PINS)


def _merge_no_rescale(acc, chunk):
    u_a, l_a, m_a = acc
    u_b, l_b, m_b = chunk
    return u_a + u_b, l_a + l_b, np.maximum(m_a, m_b)


def _merge_rescale_chunk_only(acc, chunk):
    u_a, l_a, m_a = acc
    u_b, l_b, m_b = chunk
    m = np.maximum(m_a, m_b)
    with np.errstate(invalid="ignore"):
        ab = np.where(np.isneginf(m), 0.0, np.exp(m_b - m))
    return u_a + ab[..., None] * u_b, l_a + ab * l_b, m


def _merge_drop_denominator(acc, chunk):
    u, l, m = oo.__dict__["_orig_merge"](acc, chunk)
    return u, np.ones_like(l), m


def _rows_strict_causal(q_h, k_h, v_h, qpos, kpos, causal, scale):
    return oa.__dict__["_orig_rows"](q_h, k_h, v_h, qpos - 1 if causal else qpos, kpos, causal, scale)


def _rows_no_scale(q_h, k_h, v_h, qpos, kpos, causal, scale):
    return oa.__dict__["_orig_rows"](q_h, k_h, v_h, qpos, kpos, causal, 1.0)


def _rows_swapped_kv(q_h, k_h, v_h, qpos, kpos, causal, scale):
    return oa.__dict__["_orig_rows"](q_h, v_h, k_h, qpos, kpos, causal, scale)


def _stats_flipped_sign(q, k, v, scale, allowed=None):
    u, l, m = oo.__dict__["_orig_stats"](q, k, v, scale, allowed)
    return u, l, -m


MUTANTS = {
    "merge_without_rescale": ("merge_chunk_stats", _merge_no_rescale),
    "merge_rescales_only_chunk": ("merge_chunk_stats", _merge_rescale_chunk_only),
    "merge_drops_denominator": ("merge_chunk_stats", _merge_drop_denominator),
    "causal_boundary_strict": ("_rows_of_head", _rows_strict_causal),
    "scores_not_scaled": ("_rows_of_head", _rows_no_scale),
    "key_value_swapped": ("_rows_of_head", _rows_swapped_kv),
    "max_sign_flipped": ("chunk_stats", _stats_flipped_sign),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    target, fn = MUTANTS[name]
    monkeypatch.setitem(oo.__dict__, "_orig_merge", oo.merge_chunk_stats)
    monkeypatch.setitem(oo.__dict__, "_orig_stats", oo.chunk_stats)
    monkeypatch.setitem(oa.__dict__, "_orig_rows", oa._rows_of_head)
    mod = oa if target == "_rows_of_head" else oo
    monkeypatch.setattr(mod, target, fn)
    assert not all(p() for p in ALL_PINS), f"no pin caught mutant {name}"
