"""Bookkeeping of the synthetic shares (CPU only).

The pages give the layouts only in words (contiguous shards, paired early/late
chunks, the ring order of shards), so these tests pin the generators by
construction: positions cover the sequence once, the ring order is
``(rank - step) mod P``, pair counts match closed forms, and re-splits keep
every key's value and position.
"""

import numpy as np
import pytest

from ring_attention_chunk_amd import workloads as wl


def _kpos(w):
    return np.concatenate([np.arange(n) + o for o, n in w.chunks])


@pytest.mark.parametrize("i", [1, 2, 3, 4])
def test_keys_cover_the_sequence_once(i):
    w = wl.config(i)
    assert np.array_equal(np.sort(_kpos(w)), np.arange(w.seq_len))


def test_ring_orders():
    assert wl.ring_order(0, 8) == [0, 7, 6, 5, 4, 3, 2, 1]
    assert wl.ring_order(5, 8) == [5, 4, 3, 2, 1, 0, 7, 6]
    assert wl.ring_order(3, 16) == [3, 2, 1, 0] + list(range(15, 3, -1))
    c2 = wl.config(2)
    assert [o // 8192 for o, _ in c2.chunks] == wl.ring_order(5, 8)
    assert c2.q_segments == [(40960, 8192)]


def test_zigzag_pairing():
    w = wl.config(3)
    assert w.q_segments == [(3 * 4096, 4096), (28 * 4096, 4096)]
    ids = [o // 4096 for o, _ in w.chunks]
    assert len(ids) == 32
    for s, j in enumerate(wl.ring_order(3, 16)):
        assert ids[2 * s] == j and ids[2 * s + 1] == 31 - j


def test_pair_counts_match_closed_forms():
    assert wl.unmasked_pairs_per_head(wl.config(1)) == 4096 * 32768
    # contiguous causal: query at p sees p + 1 keys
    p = np.arange(40960, 49152)
    assert wl.unmasked_pairs_per_head(wl.config(2)) == int((p + 1).sum()) == 369102848
    # zigzag: both segments, each row sees position + 1 keys; total n(n+1)/2/P
    n, P = 131072, 16
    assert wl.unmasked_pairs_per_head(wl.config(3)) == n * (n + 1) // 2 // P == 536875008
    assert wl.unmasked_pairs_per_head(wl.config(4)) == 16384 * 1048576
    assert wl.counted_flops(wl.config(1)) == 4 * 64 * 8 * 4096 * 32768
    t = wl.tiny(True)
    assert wl.unmasked_pairs_per_head(t) == sum(range(25, 33)) == 228


def test_round_to_bf16_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e38], np.float32)
    r = wl.round_to_bf16(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: goes to the even mantissa, 1.0
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.0 + 2 ** -6) and r[3] == 1.0
    assert r[4] == -2.5
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    torch = pytest.importorskip("torch")
    y = np.random.default_rng(0).standard_normal(4096).astype(np.float32)
    assert np.array_equal(wl.round_to_bf16(y), torch.from_numpy(y).to(torch.bfloat16).float().numpy())


def test_resplit_keeps_keys_and_values():
    w = wl.custom("t", "f32", 1, 2, 1, 8, [(0, 5)], [(10, 7), (0, 10), (17, 3)], True, seed=3)
    r = wl.resplit(w, [1, 2, 9, 12, 19])
    assert np.array_equal(_kpos(w), _kpos(r))
    assert len(r.chunks) > len(w.chunks)
    q1, k1, v1 = wl.generate_numpy(w)
    q2, k2, v2 = wl.generate_numpy(r)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2) and np.array_equal(q1, q2)


def test_values_are_keyed_by_position():
    a = wl.custom("a", "bf16", 1, 1, 1, 4, [(0, 1)], [(0, 9000)], False, seed=9)
    b = wl.custom("b", "bf16", 1, 1, 1, 4, [(0, 1)], [(0, 5000)], False, seed=9)
    _, ka, _ = wl.generate_numpy(a)
    _, kb, _ = wl.generate_numpy(b)
    assert np.array_equal(ka[:, :, :5000], kb)


def test_q_scale_of_long_gqa():
    w = wl.config(4)
    assert w.q_std == 4.0 and w.q_heads == 8 and w.kv_heads == 1


def test_sample_rows_cover_the_strata():
    w = wl.config(3)
    rows = wl.sample_rows(w, 2048)
    r = {x[2] for x in rows}
    assert {0, 4095, 4096, 8191} <= r  # segment ends
    assert {31, 32, 127, 128, 255, 256, 8191 - 256, 8192 - 256} <= r  # wave and workgroup edges
    assert set(range(256)) <= r and set(range(8192 - 256, 8192)) <= r  # first and last workgroup
    qpos = wl.q_positions(w)
    band = {i for i in range(w.lq) if qpos[i] % 64 in (0, 1, 62, 63)}
    assert band <= r  # the diagonal band of the causal share
    assert len(rows) >= 2048 and len(set(rows)) == len(rows)
    assert all(0 <= b < w.batch and 0 <= h < w.q_heads and 0 <= i < w.lq for b, h, i in rows)
    assert len({h for _, h, _ in rows}) == w.q_heads  # every head appears


def test_striped_share_bookkeeping():
    w = wl.causal_striped()
    P, L = 8, 8192
    assert w.pos_stride == P and w.q_segments == [(5, L)]
    assert [o for o, _ in w.chunks] == wl.ring_order(5, P)
    kpos = wl.k_positions(w)
    assert np.array_equal(np.sort(kpos), np.arange(P * L))  # every position once
    assert np.array_equal(wl.q_positions(w), 5 + P * np.arange(L))
    # query i (position 5 + 8i) sees i+1 keys of each shard j <= 5 and i keys of shards 6, 7
    i = np.arange(L)
    assert wl.unmasked_pairs_per_head(w) == int(((5 + 1) * (i + 1) + 2 * i).sum())


def test_striped_generation_holds_each_shard_contiguously():
    w = wl.custom("s", "f32", 1, 1, 1, 4, [(1, 5)], [(j, 6) for j in wl.ring_order(1, 3)], True, pos_stride=3)
    q, k, v = wl.generate_numpy(w)
    tq, tk, tv, kc, vc = wl.generate_torch(w)
    for (o, n), c in zip(w.chunks, kc):
        assert np.array_equal(c.numpy(), k[:, :, o:o + 3 * (n - 1) + 1:3])
    # queries are the rows at positions 1, 4, 7, ... of the whole sequence's seeded values
    full_q = wl._normal_positions(w.seed, 0, (1, 1), 0, 18, 4)
    assert np.array_equal(q, full_q[:, :, 1:14:3])
    # a re-split keeps every key in place
    r = wl.resplit(w, [2, 9, 13])
    kc2, _ = wl.chunk_views(r, tk, tv)
    assert np.array_equal(np.concatenate([c.numpy() for c in kc2], 2), np.concatenate([c.numpy() for c in kc], 2))
    assert np.array_equal(wl.k_positions(r), wl.k_positions(w))
