"""Pin of ``oracle.attention_rows`` (CPU only).

``attention_rows`` evaluates the same definition as ``oracle.attention`` on a
chosen set of ``(batch, head, row)`` query rows, for shares too large to
evaluate whole (it is the reference of every full-size GPU parity check). Its
own work is bookkeeping: grouping rows by key/value head, mapping a query head
to its key/value head, picking each row's query vector and global position,
and blocking rows. Each case here compares it element by element with
``oracle.attention`` (itself pinned by ``test_oracle_pins.py``) on shares that
exercise one piece of that bookkeeping: GQA over two batch entries, a
contiguous causal share, a paired early/late ("zigzag") share, a striped
share, rows from every head in scrambled order, and row blocks small enough
that the blocking splits (exercise page
"systems-distributed-ring-attention-online-softmax", problem statement: the
result is ordinary attention over the concatenated chunks, row by row).

Planted mistakes in the bookkeeping (one-line edits of the oracle's source)
must each break the pin.
"""

import importlib.util
import inspect

import numpy as np
import pytest

import oracle.direct as od


def _share(kind, seed=0):
    """Small share of the given layout: q, key chunks, value chunks, query positions, chunk offsets, strides."""
    rng = np.random.default_rng([seed, 17])
    if kind == "gqa":
        B, Hq, Hkv, d = 2, 8, 2, 5
        lens, offs, strides = [7, 1, 12], [0, 7, 8], [1, 1, 1]
        qpos = np.arange(9)
    elif kind == "causal":
        B, Hq, Hkv, d = 1, 4, 4, 6
        lens, offs, strides = [10, 10, 10], [20, 0, 10], [1, 1, 1]  # ring order: own shard first
        qpos = 20 + np.arange(10)
    elif kind == "zigzag":
        B, Hq, Hkv, d = 1, 4, 2, 4
        C, P, r = 4, 4, 1
        lens, offs, strides = [], [], []
        for j in [(r - s) % P for s in range(P)]:
            lens += [C, C]
            offs += [j * C, (2 * P - 1 - j) * C]
            strides += [1, 1]
        qpos = np.concatenate([r * C + np.arange(C), (2 * P - 1 - r) * C + np.arange(C)])
    elif kind == "striped":
        B, Hq, Hkv, d = 1, 2, 1, 3
        P, r, L = 3, 1, 6
        lens = [L] * P
        offs = [(r - s) % P for s in range(P)]
        strides = [P] * P
        qpos = r + P * np.arange(L)
    else:
        raise ValueError(kind)
    Lq = len(qpos)
    q = rng.standard_normal((B, Hq, Lq, d)) * 1.5
    kc = [rng.standard_normal((B, Hkv, n, d)) for n in lens]
    vc = [rng.standard_normal((B, Hkv, n, d)) for n in lens]
    return q, kc, vc, qpos, offs, strides


def _all_rows_scrambled(q, seed):
    B, Hq, Lq, _ = q.shape
    rows = [(b, h, i) for b in range(B) for h in range(Hq) for i in range(Lq)]
    perm = np.random.default_rng([seed, 5]).permutation(len(rows))
    return [rows[j] for j in perm]


def _pin_error(rows_fn, kind, causal, max_block_elems):
    q, kc, vc, qpos, offs, strides = _share(kind)
    full = od.attention(q, kc, vc, qpos, offs, causal=causal, kv_strides=strides)
    rows = _all_rows_scrambled(q, hash(kind) % 1000)
    got = rows_fn(q, kc, vc, rows, qpos, offs, causal=causal, kv_strides=strides, max_block_elems=max_block_elems)
    idx = tuple(np.array(rows).T)
    err = 0.0
    for key in ("out", "m", "l", "lse"):
        ref = full[key][idx]
        g = got[key]
        same_inf = np.array_equal(np.isneginf(g), np.isneginf(ref))
        fin = np.isfinite(ref)
        err = max(err, np.abs(g[fin] - ref[fin]).max() if fin.any() else 0.0, 0.0 if same_inf else np.inf)
    return err


CASES = [("gqa", False), ("gqa", True), ("causal", True), ("zigzag", True), ("striped", True), ("striped", False)]


@pytest.mark.parametrize("kind,causal", CASES)
@pytest.mark.parametrize("block", [1 << 24, 40, 1])
def test_rows_equal_full_attention(kind, causal, block):
    """Every row of the share, in scrambled order and in row blocks of several sizes (``max_block_elems``
    1 makes every row its own block), equals the same row of ``oracle.attention`` to 1e-13."""
    assert _pin_error(od.attention_rows, kind, causal, block) <= 1e-13


def test_rows_subset_and_repeats():
    """A subset with repeated rows: each occurrence is the full definition's row."""
    q, kc, vc, qpos, offs, strides = _share("zigzag", seed=3)
    full = od.attention(q, kc, vc, qpos, offs, causal=True)
    rows = [(0, 3, 7), (0, 0, 0), (0, 3, 7), (0, 1, 4), (0, 2, 3)]
    got = od.attention_rows(q, kc, vc, rows, qpos, offs, causal=True, max_block_elems=50)
    for t, (b, h, i) in enumerate(rows):
        assert np.abs(got["out"][t] - full["out"][b, h, i]).max() <= 1e-13
        assert abs(got["lse"][t] - full["lse"][b, h, i]) <= 1e-13


def _mutated_rows(old, new):
    src = inspect.getsource(od)
    assert src.count(old) == 1, old
    spec = importlib.util.spec_from_loader("oracle._direct_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "oracle_direct_mutant", "exec"), mod.__dict__)
    return mod.attention_rows


MUTANTS = [
    ("kv head from h mod Hkv", "by_kv.setdefault((b, h // group), [])", "by_kv.setdefault((b, h % Hkv), [])"),
    ("query position of the block's first row", "qpos_all[rows[t][2]] for t in sel",
     "qpos_all[rows[sel[0]][2]] for t in sel"),
    ("query vector of the kv head", "q[rows[t][0], rows[t][1], rows[t][2]]",
     "q[rows[t][0], rows[t][1] // group, rows[t][2]]"),
    ("key positions without strides", "key_positions(lens, kv_offsets, kv_strides)", "key_positions(lens, kv_offsets)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_planted_mistake(name, old, new):
    fn = _mutated_rows(old, new)
    worst = max(_pin_error(fn, kind, causal, 40) for kind, causal in CASES)
    assert worst > 1e-6, name
