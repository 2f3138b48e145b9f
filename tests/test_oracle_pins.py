"""Pins that tie the fp64 oracle to the pages and to mathematics (CPU only).

Each test checks the oracle against something other than itself: the worked
example printed on the blog page, closed forms, brute force in plain Python on
tiny inputs, and a library routine for the special case it covers.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import attention, chunk_stats, merge_chunk_stats, ring_attention_fold
from oracle.direct import key_positions

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# P1: the worked scalar example ("Do not average independently normalized shard outputs")


def _scalar_fixture():
    with open(os.path.join(GOLDEN, "scalar_two_shards.json")) as f:
        g = json.load(f)
    q = np.array(g["q"], dtype=np.float64)[None, None]  # [1,1,1,1]
    sh = {s["name"]: s for s in g["shards"]}
    return g, q, sh


@pytest.mark.parametrize("order", [("A", "B"), ("B", "A")])
def test_scalar_example_direct_and_fold(order):
    g, q, sh = _scalar_fixture()
    ks = [np.array(sh[n]["k"])[None, None] for n in order]
    vs = [np.array(sh[n]["v"])[None, None] for n in order]
    offs = [sh[n]["global_offset"] for n in order]
    exact = math.exp(10.0) / (1.0 + math.exp(10.0))
    direct = attention(q, ks, vs, kv_offsets=offs, scale=g["scale"])["out"].item()
    fold = ring_attention_fold(q, ks, vs, kv_offsets=offs, scale=g["scale"])[0].item()
    for got in (direct, fold):
        assert abs(got - exact) < 1e-15
        assert round(got, g["printed_digits"]) == g["expected_printed"]
        assert abs(got - g["naive_average"]) > 0.4


def test_scalar_example_naive_average_is_what_the_page_rejects():
    g, q, sh = _scalar_fixture()
    # each shard normalised on its own, then averaged: the page's 0.5
    local = [attention(q, [np.array(sh[n]["k"])[None, None]], [np.array(sh[n]["v"])[None, None]],
                       scale=g["scale"])["out"].item() for n in ("A", "B")]
    assert np.mean(local) == g["naive_average"]


def test_scalar_example_merge_statistics():
    g, q, sh = _scalar_fixture()
    a = chunk_stats(q, np.array(sh["A"]["k"])[None, None], np.array(sh["A"]["v"])[None, None], 1.0)
    b = chunk_stats(q, np.array(sh["B"]["k"])[None, None], np.array(sh["B"]["v"])[None, None], 1.0)
    # each chunk alone: the max is its own score, the denominator is exp(0) = 1
    assert a[2].item() == 0.0 and b[2].item() == 10.0
    assert a[1].item() == 1.0 and b[1].item() == 1.0
    u, l, m = merge_chunk_stats(a, b)
    assert m.item() == 10.0
    assert abs(l.item() - (1.0 + math.exp(-10.0))) < 1e-15
    assert abs(u.item() - 1.0) < 1e-15


# ---------------------------------------------------------------------------
# P2: any split gives the same result (problem statement: "even chunks of size 1")


def _compositions(n):
    for mask in range(1 << (n - 1)):
        sizes, run = [], 1
        for i in range(n - 1):
            if mask >> i & 1:
                sizes.append(run)
                run = 1
            else:
                run += 1
        sizes.append(run)
        yield sizes


@pytest.mark.parametrize("causal", [False, True])
def test_every_split_of_ten_keys(causal):
    n, d, lq = 10, 3, 4
    q = _rand((1, 2, lq, d), 1)
    k = _rand((1, 1, n, d), 2) * 2.0
    v = _rand((1, 1, n, d), 3)
    qpos = np.array([0, 3, 6, 9])
    ref = attention(q, [k], [v], q_positions=qpos, kv_offsets=[0], causal=causal)["out"]
    count = 0
    for sizes in _compositions(n):
        cuts = np.cumsum([0] + sizes)
        kc = [k[:, :, a:b] for a, b in zip(cuts[:-1], cuts[1:])]
        vc = [v[:, :, a:b] for a, b in zip(cuts[:-1], cuts[1:])]
        offs = list(cuts[:-1])
        out = ring_attention_fold(q, kc, vc, q_positions=qpos, kv_offsets=offs, causal=causal)[0]
        assert np.max(np.abs(out - ref)) <= 1e-12
        direct = attention(q, kc, vc, q_positions=qpos, kv_offsets=offs, causal=causal)["out"]
        assert np.max(np.abs(direct - ref)) <= 1e-12
        count += 1
    assert count == 2 ** (n - 1)


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_config_many_splits(causal):
    from ring_attention_chunk_amd import workloads as wl

    w = wl.tiny(causal)
    q, k, v = wl.generate_numpy(w)
    qpos = wl.q_positions(w)
    ref = attention(q, [k], [v], q_positions=qpos, kv_offsets=[0], causal=causal)["out"]
    rng = np.random.default_rng(5)
    splits = [[1] * 32, [1, 3, 12, 16], [32]]
    for _ in range(1000):
        cuts = np.sort(rng.choice(np.arange(1, 32), size=rng.integers(1, 12), replace=False))
        splits.append(list(np.diff(np.concatenate([[0], cuts, [32]]))))
    for sizes in splits:
        cuts = np.cumsum([0] + list(sizes))
        kc = [k[:, :, a:b] for a, b in zip(cuts[:-1], cuts[1:])]
        vc = [v[:, :, a:b] for a, b in zip(cuts[:-1], cuts[1:])]
        out = ring_attention_fold(q, kc, vc, q_positions=qpos, kv_offsets=list(cuts[:-1]),
                                  causal=causal)[0]
        assert np.max(np.abs(out - ref)) <= 1e-12


def test_chunk_order_does_not_change_the_result():
    # the math is order-free: the ring can present shards in any order
    q = _rand((1, 1, 5, 4), 11)
    k = _rand((1, 1, 12, 4), 12) * 3
    v = _rand((1, 1, 12, 4), 13)
    parts = [(0, 5), (5, 9), (9, 12)]
    ref = attention(q, [k], [v])["out"]
    for perm in itertools.permutations(parts):
        kc = [k[:, :, a:b] for a, b in perm]
        vc = [v[:, :, a:b] for a, b in perm]
        assert np.max(np.abs(ring_attention_fold(q, kc, vc)[0] - ref)) <= 1e-12


# ---------------------------------------------------------------------------
# P3: causal masking by global positions ("Causal masks depend on global positions")


def test_future_keys_do_not_matter():
    q = _rand((1, 2, 6, 8), 21)
    k = _rand((1, 2, 20, 8), 22)
    v = _rand((1, 2, 20, 8), 23)
    qpos = np.array([0, 4, 7, 12, 15, 19])
    ref = attention(q, [k], [v], q_positions=qpos, kv_offsets=[0], causal=True)["out"]
    for i, p in enumerate(qpos):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, p + 1:] = 1e3 * _rand(k2[:, :, p + 1:].shape, 100 + i)
        v2[:, :, p + 1:] = -7.0
        out = attention(q, [k2], [v2], q_positions=qpos, kv_offsets=[0], causal=True)["out"]
        assert np.array_equal(out[:, :, i], ref[:, :, i])


def test_single_allowed_key_returns_its_value():
    q = _rand((1, 1, 1, 8), 31)
    k = _rand((1, 1, 9, 8), 32)
    v = _rand((1, 1, 9, 8), 33)
    # query at position 100, keys at 100..108: only the first key is allowed
    out = attention(q, [k[:, :, :4], k[:, :, 4:]], [v[:, :, :4], v[:, :, 4:]], q_positions=[100],
                    kv_offsets=[100, 104], causal=True)["out"]
    assert np.array_equal(out[0, 0, 0], v[0, 0, 0])
    fold = ring_attention_fold(q, [k[:, :, :4], k[:, :, 4:]], [v[:, :, :4], v[:, :, 4:]],
                               q_positions=[100], kv_offsets=[100, 104], causal=True)[0]
    assert np.max(np.abs(fold[0, 0, 0] - v[0, 0, 0])) == 0.0


def test_last_row_of_tiny_causal_sees_everything():
    from ring_attention_chunk_amd import workloads as wl

    w = wl.tiny(True)
    q, k, v = wl.generate_numpy(w)
    qpos = wl.q_positions(w)
    kc = [k[:, :, o:o + n] for o, n in w.chunks]
    vc = [v[:, :, o:o + n] for o, n in w.chunks]
    offs = [o for o, _ in w.chunks]
    c = attention(q, kc, vc, q_positions=qpos, kv_offsets=offs, causal=True)["out"]
    nc = attention(q, kc, vc, causal=False)["out"]
    assert qpos[-1] == 31
    assert np.array_equal(c[:, :, -1], nc[:, :, -1])
    assert np.max(np.abs(c[:, :, 0] - nc[:, :, 0])) > 1e-3  # row at 24 does not see keys 25..31


def test_causal_row_equals_direct_on_truncated_keys():
    q = _rand((1, 1, 7, 5), 41)
    k = _rand((1, 1, 30, 5), 42)
    v = _rand((1, 1, 30, 5), 43)
    # keys in a zigzag-like order: positions are not sorted in the list
    kpos = np.concatenate([np.arange(20, 30), np.arange(0, 10), np.arange(10, 20)])
    order = np.argsort(kpos)
    chunks = [(0, 10), (10, 20), (20, 30)]
    kc = [k[:, :, a:b] for a, b in chunks]
    vc = [v[:, :, a:b] for a, b in chunks]
    offs = [20, 0, 10]
    qpos = np.array([0, 5, 9, 10, 19, 25, 29])
    out = attention(q, kc, vc, q_positions=qpos, kv_offsets=offs, causal=True)["out"]
    assert np.array_equal(key_positions([10, 10, 10], offs), kpos)
    for i, p in enumerate(qpos):
        keep = np.nonzero(kpos <= p)[0]
        sub = attention(q[:, :, i:i + 1], [k[:, :, keep]], [v[:, :, keep]])["out"]
        assert np.max(np.abs(sub[0, 0, 0] - out[0, 0, i])) <= 1e-14


# ---------------------------------------------------------------------------
# P4: closed forms


def test_zero_query_gives_mean_of_allowed_values():
    v = _rand((1, 1, 11, 6), 51)
    k = _rand((1, 1, 11, 6), 52)
    q = np.zeros((1, 1, 3, 6))
    qpos = np.array([0, 4, 10])
    out = attention(q, [k], [v], q_positions=qpos, kv_offsets=[0], causal=True)["out"]
    for i, p in enumerate(qpos):
        assert np.max(np.abs(out[0, 0, i] - v[0, 0, :p + 1].mean(axis=0))) <= 1e-15


def test_mass_example_three_to_one():
    # shard A: one key with score 0 and value 0; shard B: three keys with score 0 and value 1.
    # Global softmax weighs the four keys equally: 3/4. Averaging shard outputs would give 1/2.
    q = np.ones((1, 1, 1, 1))
    ka, va = np.zeros((1, 1, 1, 1)), np.zeros((1, 1, 1, 1))
    kb, vb = np.zeros((1, 1, 3, 1)), np.ones((1, 1, 3, 1))
    assert attention(q, [ka, kb], [va, vb], scale=1.0)["out"].item() == 0.75
    assert abs(ring_attention_fold(q, [ka, kb], [va, vb], scale=1.0)[0].item() - 0.75) <= 1e-15


def test_huge_score_gap_does_not_overflow():
    q = np.ones((1, 1, 1, 1))
    k = [np.zeros((1, 1, 1, 1)), np.full((1, 1, 1, 1), 1000.0)]
    v = [np.full((1, 1, 1, 1), 3.0), np.full((1, 1, 1, 1), -2.0)]
    for fn in (lambda: attention(q, k, v, scale=1.0)["out"],
               lambda: ring_attention_fold(q, k, v, scale=1.0)[0]):
        got = fn()
        assert np.all(np.isfinite(got)) and got.item() == -2.0


def test_lse_of_equal_scores():
    # n keys with the same score s: lse = s + ln n exactly (up to rounding)
    n, s = 37, 1.25
    q = np.ones((1, 1, 1, 1))
    k = np.full((1, 1, n, 1), s)
    v = _rand((1, 1, n, 1), 61)
    r = attention(q, [k], [v], scale=1.0)
    assert abs(r["lse"].item() - (s + math.log(n))) <= 1e-14
    assert r["m"].item() == s and abs(r["l"].item() - n) <= 1e-12
    assert abs(r["out"].item() - v.mean()) <= 1e-15


def test_no_allowed_key_gives_zero_output():
    q = _rand((1, 1, 2, 4), 71)
    k = _rand((1, 1, 5, 4), 72)
    v = _rand((1, 1, 5, 4), 73)
    r = attention(q, [k], [v], q_positions=[3, 10], kv_offsets=[5], causal=True)
    assert np.all(r["out"][0, 0, 0] == 0.0) and np.isneginf(r["lse"][0, 0, 0])
    assert r["l"][0, 0, 0] == 0.0 and np.isneginf(r["m"][0, 0, 0])
    out, lse, (u, l, m) = ring_attention_fold(q, [k], [v], q_positions=[3, 10], kv_offsets=[5],
                                              causal=True)
    assert np.all(out[0, 0, 0] == 0.0) and np.isneginf(lse[0, 0, 0]) and np.isneginf(m[0, 0, 0])
    assert np.max(np.abs(out[0, 0, 1] - r["out"][0, 0, 1])) <= 1e-14


def test_empty_chunk_contributes_nothing():
    q = _rand((1, 1, 3, 4), 81)
    k = _rand((1, 1, 6, 4), 82)
    v = _rand((1, 1, 6, 4), 83)
    e = np.zeros((1, 1, 0, 4))
    ref = ring_attention_fold(q, [k], [v])[0]
    got = ring_attention_fold(q, [e, k[:, :, :2], e, k[:, :, 2:], e], [e, v[:, :, :2], e, v[:, :, 2:], e])[0]
    assert np.max(np.abs(got - ref)) <= 1e-15
    u, l, m = chunk_stats(q, e, e, 0.5)
    assert np.all(u == 0) and np.all(l == 0) and np.all(np.isneginf(m))


def test_merge_identity_and_symmetry():
    q = _rand((1, 1, 4, 3), 91)
    a = chunk_stats(q, _rand((1, 1, 5, 3), 92), _rand((1, 1, 5, 3), 93), 0.7)
    b = chunk_stats(q, _rand((1, 1, 2, 3), 94) * 4, _rand((1, 1, 2, 3), 95), 0.7)
    ident = (np.zeros_like(a[0]), np.zeros_like(a[1]), np.full_like(a[2], -np.inf))
    for x, y in zip(merge_chunk_stats(ident, a), a):
        assert np.array_equal(x, y)
    ab, ba = merge_chunk_stats(a, b), merge_chunk_stats(b, a)
    for x, y in zip(ab, ba):
        assert np.max(np.abs(x - y)) <= 1e-14
    both = merge_chunk_stats(ident, ident)
    assert np.all(both[0] == 0) and np.all(both[1] == 0) and np.all(np.isneginf(both[2]))


# ---------------------------------------------------------------------------
# brute force in plain Python, and a library special case


def _brute(q, k, v, qpos, kpos, causal, scale, group):
    B, Hq, Lq, d = q.shape
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            for i in range(Lq):
                scores = []
                for j in range(k.shape[2]):
                    if causal and kpos[j] > qpos[i]:
                        continue
                    s = 0.0
                    for t in range(d):
                        s += q[b, h, i, t] * k[b, h // group, j, t]
                    scores.append((scale * s, j))
                if not scores:
                    continue
                top = max(s for s, _ in scores)
                den = sum(math.exp(s - top) for s, _ in scores)
                for t in range(d):
                    out[b, h, i, t] = sum(math.exp(s - top) * v[b, h // group, j, t] for s, j in scores) / den
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_gqa(causal):
    B, Hq, Hkv, Lq, d = 2, 4, 2, 5, 3
    lens, offs = [3, 1, 4], [4, 0, 1]
    q = _rand((B, Hq, Lq, d), 101)
    kc = [_rand((B, Hkv, n, d), 110 + i) * 1.5 for i, n in enumerate(lens)]
    vc = [_rand((B, Hkv, n, d), 120 + i) for i, n in enumerate(lens)]
    qpos = np.array([0, 1, 2, 4, 7])
    kpos = key_positions(lens, offs)
    ref = _brute(q, np.concatenate(kc, 2), np.concatenate(vc, 2), qpos, kpos, causal, 0.6, Hq // Hkv)
    got = attention(q, kc, vc, q_positions=qpos, kv_offsets=offs, causal=causal, scale=0.6)["out"]
    fold = ring_attention_fold(q, kc, vc, q_positions=qpos, kv_offsets=offs, causal=causal, scale=0.6)[0]
    assert np.max(np.abs(got - ref)) <= 1e-13
    assert np.max(np.abs(fold - ref)) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_float64(causal):
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, Lq, n, d = 1, 4, 2, 9, 23, 16
    q = _rand((B, Hq, Lq, d), 131)
    k = _rand((B, Hkv, n, d), 132)
    v = _rand((B, Hkv, n, d), 133)
    qpos = np.arange(14, 23)  # the last 9 positions of a 23-token sequence
    got = attention(q, [k[:, :, :7], k[:, :, 7:]], [v[:, :, :7], v[:, :, 7:]], q_positions=qpos,
                    kv_offsets=[0, 7], causal=causal)["out"]
    tk = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=1))
    tv = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=1))
    mask = torch.from_numpy(np.arange(n)[None, :] <= qpos[:, None]) if causal else None
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), tk, tv, attn_mask=mask)
    assert np.max(np.abs(got - ref.numpy())) <= 1e-12


# ---------------------------------------------------------------------------
# striped shares (glossary "ring attention", paragraph Variants: striped attention): device r of P
# owns positions r, r+P, r+2P, ...; its result must be those rows of ordinary causal attention over
# the whole sequence in natural order


@pytest.mark.parametrize("P,r", [(4, 0), (4, 3), (3, 1)])
def test_striped_share_equals_rows_of_whole_sequence_causal_sdpa(P, r):
    torch = pytest.importorskip("torch")
    from ring_attention_chunk_amd import workloads as wl

    n, H, d = 24, 2, 8
    q_all = _rand((1, H, n, d), 141 + P)
    k_all = _rand((1, H, n, d), 151 + P) * 1.3
    v_all = _rand((1, H, n, d), 161 + P)
    # the whole sequence, unsharded, by the library routine with its built-in causal mask
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q_all), torch.from_numpy(k_all), torch.from_numpy(v_all), is_causal=True).numpy()
    L = n // P
    order = wl.ring_order(r, P)
    kc = [k_all[:, :, j::P] for j in order]
    vc = [v_all[:, :, j::P] for j in order]
    qpos = r + P * np.arange(L)
    got = attention(q_all[:, :, r::P], kc, vc, q_positions=qpos, kv_offsets=order, causal=True,
                    kv_strides=[P] * P)["out"]
    fold = ring_attention_fold(q_all[:, :, r::P], kc, vc, q_positions=qpos, kv_offsets=order, causal=True,
                               kv_strides=[P] * P)[0]
    assert np.max(np.abs(got - ref[:, :, r::P])) <= 1e-12
    assert np.max(np.abs(fold - ref[:, :, r::P])) <= 1e-12
    # the same keys read as contiguous runs would be a different (wrong) mask
    wrong = attention(q_all[:, :, r::P], kc, vc, q_positions=qpos, kv_offsets=order, causal=True)["out"]
    assert np.max(np.abs(wrong - ref[:, :, r::P])) > 1e-3


def test_strided_key_positions_closed_form():
    assert key_positions([3, 2], [5, 0], [4, 7]).tolist() == [5, 9, 13, 0, 7]
    from oracle import query_positions

    assert query_positions([(2, 3, 5), (1, 2)]).tolist() == [2, 7, 12, 1, 2]
