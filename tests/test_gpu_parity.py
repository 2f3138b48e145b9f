"""Parity of the HIP path with the fp64 oracle (needs an MI355X).

Every call goes through the C ABI via the ctypes binding. Tolerances: fp32
inputs max abs error <= 1e-5; bf16 inputs (fp32 accumulation) max abs error
<= 2e-2 and mean abs error <= 2e-3, both against the oracle on the exact
(upcast) inputs. The full-size shares are checked in full (the d = 64 share)
or on at least 2048 stratified rows (segment ends, wave and workgroup edges,
whole first and last workgroups, the causal diagonal band, random rows), each
of which the oracle computes against every key.

The log-sum-exp bound of the bf16 path comes from its arithmetic: the
denominator l sums the fp32 probabilities, each within 2^-9 of its exact value
(the bf16 rounding that P.V sees is the coarsest step on the path; l itself
skips it), so the sum of these positive terms is within 2^-9 too, and the
running sum adds one fp32 tile sum per key tile (relative error <= 2^-24 per
addition, at most one per 64 keys). So |lse - lse_ref| = |ln(l / l_ref)| <=
2^-9 + ceil(Lk / 64) 2^-24, plus 1e-5 for the fp32 scores and exponentials.
"""

import math
import os
import zlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import ring_attention_chunk_amd as ra
from ring_attention_chunk_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
F32_TOL = 1e-5
BF16_MAX, BF16_MEAN = 2e-2, 2e-3


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np(t):
    return t.detach().cpu().double().numpy()


def _check(got, ref, dtype):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    if dtype == "f32":
        assert err.max() <= F32_TOL, err.max()
    else:
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    return err.max()


def lse_tol(dtype, n_keys):
    """Bound on |lse - lse_ref| (module docstring)."""
    if dtype == "f32":
        return F32_TOL
    return 2.0 ** -9 + math.ceil(max(n_keys, 1) / 64) * 2.0 ** -24 + 1e-5


def _check_lse(got, ref, dtype, n_keys):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    err = np.abs(got[fin] - ref[fin]).max() if fin.any() else 0.0
    print(f"  lse max err {err:.3e} (bound {lse_tol(dtype, n_keys):.3e})", flush=True)
    assert err <= lse_tol(dtype, n_keys)
    return err


def _workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _oracle_rows_parallel(q, kc, vc, rows, qpos, offs, causal, kv_strides, workers=None):
    """oracle.attention_rows on groups of rows in a thread pool (one BLAS thread each); rows of one key/value
    head stay together so that each call concatenates few heads' keys. Returns out [R, d] and lse [R]."""
    from threadpoolctl import threadpool_limits

    workers = workers or _workers()
    group = q.shape[1] // kc[0].shape[1]
    qn = q.float().cpu().double().numpy()
    kn = [c.float().cpu().double().numpy() for c in kc]
    vn = [c.float().cpu().double().numpy() for c in vc]
    order = sorted(range(len(rows)), key=lambda t: (rows[t][0], rows[t][1] // group, rows[t][1], rows[t][2]))
    parts = [order[i * len(order) // workers:(i + 1) * len(order) // workers] for i in range(workers)]
    parts = [p for p in parts if p]

    def run(part):
        return oracle.attention_rows(qn, kn, vn, [rows[t] for t in part], qpos, offs, causal=causal,
                                     kv_strides=kv_strides, max_block_elems=1 << 25)

    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(len(parts)) as ex:
        res = list(ex.map(run, parts))
    out = np.zeros((len(rows), q.shape[-1]))
    lse = np.zeros(len(rows))
    for part, r in zip(parts, res):
        out[part] = r["out"]
        lse[part] = r["lse"]
    return out, lse


def _run(w, **kw):
    q, k, v, kc, vc = wl.generate_torch(w, DEV)
    offs = w.kv_offsets
    out, lse = ra.ring_attention(q, kc, vc, w.q_runs, offs, causal=w.causal, return_lse=True,
                                 scale=w.softmax_scale, kv_position_strides=w.kv_strides, **kw)
    torch.cuda.synchronize()
    return q, kc, vc, offs, out, lse


def _oracle(w, q, kc, vc, offs):
    return oracle.attention(q.cpu(), [c.cpu() for c in kc], [c.cpu() for c in vc], wl.q_positions(w), offs,
                            causal=w.causal, scale=w.softmax_scale, kv_strides=w.kv_strides)


# ---------------------------------------------------------------------------
# the pages' scalar example and the tiny fp32 share


@pytest.mark.parametrize("order", [(0, 1), (1, 0)])
@pytest.mark.parametrize("causal", [False, True])
def test_scalar_two_shards(order, causal):
    _say(f"scalar order={order} causal={causal}")
    s = wl.scalar_case()
    q = torch.from_numpy(s["q"]).to(DEV)
    kc = [torch.from_numpy(s["k"][i]).to(DEV) for i in order]
    vc = [torch.from_numpy(s["v"][i]).to(DEV) for i in order]
    offs = [s["kv_offsets"][i] for i in order]
    out = ra.ring_attention(q, kc, vc, 1, offs, causal=causal, scale=1.0)
    torch.cuda.synchronize()
    exact = math.exp(10) / (1 + math.exp(10))
    assert abs(out.item() - exact) <= F32_TOL
    assert abs(out.item() - 0.5) > 0.4


@pytest.mark.parametrize("causal", [False, True])
def test_tiny_f32_every_listed_split_is_bit_identical(causal):
    w = wl.tiny(causal)
    _say(w.name)
    q, kc, vc, offs, out, lse = _run(w)
    ref = _oracle(w, q, kc, vc, offs)
    _check(_np(out), ref["out"], "f32")
    assert np.abs(_np(lse) - ref["lse"]).max() <= F32_TOL
    rng = np.random.default_rng(1)
    splits = [list(range(1, 32)), [], [16], [5, 6, 7, 30]]
    splits += [sorted(rng.choice(np.arange(1, 32), size=int(rng.integers(1, 10)), replace=False)) for _ in range(20)]
    for cuts in splits:
        r = wl.resplit(w, cuts)
        _, _, _, _, out2, lse2 = _run(r)
        assert torch.equal(out2, out), cuts
        assert torch.equal(lse2, lse), cuts


def test_tiny_chunk_stats_and_merge_f32():
    w = wl.tiny(False)
    _say("tiny stats+merge")
    q, k, v, kc, vc = wl.generate_torch(w, DEV)
    acc = None
    ref_acc = None
    for c in range(len(kc)):
        st = ra.attention_chunk_stats(q, kc[c], vc[c])
        torch.cuda.synchronize()
        r = oracle.chunk_stats(q.cpu(), kc[c].cpu(), vc[c].cpu(), 1 / math.sqrt(16))
        # statistics compared in normalised form and as log-sum-exp
        assert np.abs(_np(st[2]) - r[2]).max() <= F32_TOL
        assert np.abs(_np(st[0]) / _np(st[1])[..., None] - r[0] / r[1][..., None]).max() <= F32_TOL
        assert np.abs(np.log(_np(st[1])) + _np(st[2]) - (np.log(r[1]) + r[2])).max() <= F32_TOL
        acc = st if acc is None else ra.merge_chunk_stats(acc, st)
        ref_acc = r if ref_acc is None else oracle.merge_chunk_stats(ref_acc, r)
    torch.cuda.synchronize()
    out = _np(acc[0]) / _np(acc[1])[..., None]
    direct = oracle.attention(q.cpu(), [k.cpu()], [v.cpu()])
    _check(out, direct["out"], "f32")
    assert np.abs(_np(acc[2]) - ref_acc[2]).max() <= F32_TOL


# ---------------------------------------------------------------------------
# small bf16 / fp32 shares that span several tiles, with ragged tails


SMALL = [
    # name, dtype, B, Hq, Hkv, d, q_segments, chunks, causal
    ("bf16_d64_nc", "bf16", 2, 4, 2, 64, [(0, 300)], [(0, 100), (100, 37), (137, 250), (387, 1), (388, 130)], False),
    ("bf16_d128_causal", "bf16", 1, 3, 3, 128, [(200, 260)], [(0, 64), (64, 200), (264, 236)], True),
    ("bf16_d128_zigzag", "bf16", 1, 2, 1, 128, [(64, 64), (448, 64)],
     [(64 * j, 64) for j in (1, 6, 0, 7, 3, 4, 2, 5)], True),
    ("bf16_d40_causal_gqa", "bf16", 1, 4, 1, 40, [(90, 150)], [(0, 33), (33, 200)], True),
    ("bf16_d8_nc", "bf16", 1, 1, 1, 8, [(0, 129)], [(0, 65), (65, 1)], False),
    ("bf16_d100_nc", "bf16", 1, 2, 2, 100, [(0, 77)], [(0, 190)], False),
    ("f32_d64_causal", "f32", 1, 2, 2, 64, [(100, 140)], [(0, 120), (120, 120)], True),
    ("f32_d128_nc", "f32", 1, 2, 1, 128, [(0, 70)], [(0, 90), (90, 50)], False),
    ("f32_d3_nc", "f32", 1, 2, 2, 3, [(0, 33)], [(0, 5), (5, 60)], False),
    # few query tiles and many keys: the key tiles are cut into ranges merged afterwards
    ("bf16_d128_split_causal", "bf16", 1, 2, 1, 128, [(3000, 200)], [(0, 1000), (1000, 2999), (3999, 2001)], True),
    ("bf16_d64_split_nc", "bf16", 2, 2, 2, 64, [(0, 130)], [(0, 4097), (4097, 3000)], False),
    ("f32_d16_split_causal", "f32", 1, 1, 1, 16, [(2500, 40), (100, 40)], [(2000, 2100), (0, 2000)], True),
    # shapes of the 256-row workgroups and 128-key tiles of the ring kernel: a query share that
    # ends one row into a workgroup, chunks cut inside a tile, a GQA zigzag at d = 64
    ("bf16_d32_causal_ragged", "bf16", 1, 2, 2, 32, [(500, 600)], [(0, 700), (700, 77), (777, 400)], True),
    ("bf16_d64_zigzag_gqa", "bf16", 1, 4, 2, 64, [(128, 128), (896, 128)],
     [(128 * j, 128) for j in (1, 6, 0, 7, 3, 4, 2, 5)], True),
    ("bf16_d128_nc_257", "bf16", 1, 2, 2, 128, [(0, 257)], [(0, 300), (300, 211)], False),
    # striped shares (positions advance by P per row and per key): whole tiles per chunk (pipelined
    # kernel with a position step), then chunks cut inside tiles (general kernel), fp32, and a split
    ("bf16_d64_striped_p4", "bf16", 1, 4, 2, 64, [(3, 300)], [(j, 256) for j in wl.ring_order(3, 4)], True, 4),
    ("bf16_d128_striped_p3", "bf16", 1, 2, 2, 128, [(1, 200)], [(j, 192) for j in wl.ring_order(1, 3)], True, 3),
    ("bf16_d64_striped_ragged", "bf16", 1, 2, 2, 64, [(2, 260)], [(j, 300) for j in wl.ring_order(2, 4)], True, 4),
    ("f32_d16_striped", "f32", 1, 2, 1, 16, [(5, 90)], [(j, 100) for j in wl.ring_order(5, 8)], True, 8),
    ("bf16_d128_striped_split", "bf16", 1, 1, 1, 128, [(0, 150)], [(j, 2048) for j in wl.ring_order(0, 2)], True, 2),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_shares(case):
    name, dtype, B, Hq, Hkv, d, qs, ch, causal = case[:9]
    pstep = case[9] if len(case) > 9 else 1
    _say(name)
    w = wl.custom(name, dtype, B, Hq, Hkv, d, qs, ch, causal, seed=zlib.crc32(name.encode()) % 1000,
                  pos_stride=pstep)
    q, kc, vc, offs, out, lse = _run(w)
    ref = _oracle(w, q, kc, vc, offs)
    _check(_np(out), ref["out"], dtype)
    _check_lse(_np(lse), ref["lse"], dtype, w.lk)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("bf16", 24), ("f32", 32)])
def test_chunk_stats_small(dtype, d):
    _say(f"chunk_stats {dtype} d={d}")
    w = wl.custom("st", dtype, 2, 4, 2, d, [(0, 200)], [(0, 333)], False, seed=d)
    q, k, v, kc, vc = wl.generate_torch(w, DEV)
    u, l, m = ra.attention_chunk_stats(q, kc[0], vc[0])
    torch.cuda.synchronize()
    ru, rl, rm = oracle.chunk_stats(q.cpu(), np.repeat(kc[0].cpu().float().numpy(), 2, axis=1),
                                    np.repeat(vc[0].cpu().float().numpy(), 2, axis=1), 1 / math.sqrt(d))
    _check(_np(u) / _np(l)[..., None], ru / rl[..., None], dtype)
    assert np.abs(_np(m) - rm).max() <= (F32_TOL if dtype == "f32" else 1e-4) * max(1, np.abs(rm).max())
    _check_lse(np.log(_np(l)) + _np(m), np.log(rl) + rm, dtype, 333)


@pytest.mark.parametrize("d,nk", [(64, 100), (64, 129), (64, 640), (32, 127), (32, 300), (64, 4096 + 77)])
def test_chunk_stats_key_halves(d, nk):
    """At head_dim <= 64 a chunk-statistics workgroup walks the first and the second half of the key tiles in
    two halves and merges them: one tile (the second half empty), two, an odd count with a ragged end, and a
    long chunk; 600 query rows over 4 heads so that several workgroups and a partial one run."""
    _say(f"chunk_stats halves d={d} keys={nk}")
    w = wl.custom("sthalves", "bf16", 1, 4, 2, d, [(0, 600)], [(0, nk)], False, seed=d * 7 + nk)
    q, k, v, kc, vc = wl.generate_torch(w, DEV)
    u, l, m = ra.attention_chunk_stats(q, kc[0], vc[0], workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    ru, rl, rm = oracle.chunk_stats(q.cpu(), np.repeat(kc[0].cpu().float().numpy(), 2, axis=1),
                                    np.repeat(vc[0].cpu().float().numpy(), 2, axis=1), 1 / math.sqrt(d))
    _check(_np(u) / _np(l)[..., None], ru / rl[..., None], "bf16")
    assert np.abs(_np(m) - rm).max() <= 1e-4 * max(1, np.abs(rm).max())
    _check_lse(np.log(_np(l)) + _np(m), np.log(rl) + rm, "bf16", nk)


@pytest.mark.parametrize("dtype,d,nk", [("bf16", 64, 4096), ("bf16", 128, 4096), ("f32", 32, 2048)])
def test_chunk_stats_key_range_split(dtype, d, nk):
    """Few query rows against a long chunk: the keys are cut into ranges and the partial statistics
    merged; the result matches the oracle and, to rounding, the uncut call."""
    _say(f"chunk_stats split {dtype} d={d} keys={nk}")
    w = wl.custom("stsplit", dtype, 1, 2, 2, d, [(0, 256)], [(0, nk)], False, seed=d + nk)
    q, k, v, kc, vc = wl.generate_torch(w, DEV)
    assert ra.api.load_library().ra_chunk_stats_workspace_bytes(1, 2, d, 256, nk) > 0
    u, l, m = ra.attention_chunk_stats(q, kc[0], vc[0])
    u0, l0, m0 = ra.attention_chunk_stats(q, kc[0], vc[0], workspace=torch.empty(0, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    ru, rl, rm = oracle.chunk_stats(q.cpu(), kc[0].cpu(), vc[0].cpu(), 1 / math.sqrt(d))
    _check(_np(u) / _np(l)[..., None], ru / rl[..., None], dtype)
    _check_lse(np.log(_np(l)) + _np(m), np.log(rl) + rm, dtype, nk)
    assert np.abs(_np(m) - rm).max() <= (F32_TOL if dtype == "f32" else 1e-4) * max(1, np.abs(rm).max())
    # the same statistics as the uncut call, up to rounding
    assert torch.equal(m, m0)
    tol = F32_TOL if dtype == "f32" else BF16_MAX
    assert np.abs(_np(u) / _np(l)[..., None] - _np(u0) / _np(l0)[..., None]).max() <= tol


def test_merge_random_statistics():
    _say("merge random")
    g = torch.Generator().manual_seed(3)
    for d in (128, 64, 5, 1):
        rows = 1000
        a = (torch.randn(rows, d, generator=g), torch.rand(rows, generator=g) + 0.5, torch.randn(rows, generator=g) * 8)
        b = (torch.randn(rows, d, generator=g), torch.rand(rows, generator=g) + 0.5, torch.randn(rows, generator=g) * 8)
        # rows with nothing seen yet on one or both sides
        a[2][:10] = -math.inf
        a[1][:10] = 0
        a[0][:10] = 0
        b[2][5:15] = -math.inf
        b[1][5:15] = 0
        b[0][5:15] = 0
        ga = tuple(t.to(DEV) for t in a)
        gb = tuple(t.to(DEV) for t in b)
        u, l, m = ra.merge_chunk_stats(ga, gb)
        torch.cuda.synchronize()
        ru, rl, rm = oracle.merge_chunk_stats(tuple(t.double().numpy() for t in a), tuple(t.double().numpy() for t in b))
        assert np.array_equal(np.isneginf(_np(m)), np.isneginf(rm))
        fin = ~np.isneginf(rm)
        assert np.abs(_np(m)[fin] - rm[fin]).max() == 0.0
        assert np.abs(_np(l) - rl).max() <= 1e-5 * max(1.0, np.abs(rl).max())
        assert np.abs(_np(u) - ru).max() <= 1e-5 * max(1.0, np.abs(ru).max())
        # in place
        ua, la, ma = (t.clone() for t in ga)
        ra.merge_chunk_stats((ua, la, ma), gb, inplace=True)
        torch.cuda.synchronize()
        assert torch.equal(ua, u) and torch.equal(la, l) and torch.equal(ma, m)


def test_merge_of_permuted_accumulator():
    """A dense accumulator with a transposed u (and strided l, m): the functional merge works on row-major
    copies and matches the oracle; the in-place merge refuses it."""
    _say("merge permuted accumulator")
    g = torch.Generator().manual_seed(8)
    rows, d = 300, 64
    ua = torch.randn(d, rows, generator=g).t()
    la2 = torch.rand(rows, 2, generator=g) + 0.5
    ma2 = torch.randn(rows, 2, generator=g) * 4
    b = (torch.randn(rows, d, generator=g), torch.rand(rows, generator=g) + 0.5, torch.randn(rows, generator=g) * 4)
    acc = (ua.to(DEV), la2.to(DEV)[:, 0], ma2.to(DEV)[:, 1])
    assert not acc[0].is_contiguous() and not acc[1].is_contiguous()
    gb = tuple(t.to(DEV) for t in b)
    u, l, m = ra.merge_chunk_stats(acc, gb)
    torch.cuda.synchronize()
    ru, rl, rm = oracle.merge_chunk_stats((ua.double().numpy(), la2[:, 0].double().numpy(),
                                           ma2[:, 1].double().numpy()), tuple(t.double().numpy() for t in b))
    assert np.abs(_np(u) - ru).max() <= 1e-5 * max(1.0, np.abs(ru).max())
    assert np.abs(_np(l) - rl).max() <= 1e-5 * max(1.0, np.abs(rl).max())
    assert np.abs(_np(m) - rm).max() == 0.0
    with pytest.raises(ra.RingAttentionError):
        ra.merge_chunk_stats(acc, gb, inplace=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["one_tile", "separate_tiles"])
@pytest.mark.parametrize("order", ["ab", "ba"])
def test_score_gap_of_1000(dtype, layout, order):
    """Scores 0 and 1000 (the blog's overflow case, stated through the max subtraction of the exercise's
    hint 1): exp(-1000) underflows, so every query's output is exactly the value of the key with score 1000,
    with no inf or NaN, whichever chunk comes first and whether both keys share a key tile. Shard A holds
    keys of score 0 (one key, or 200 keys so that B lies in a later tile); shard B one key of score 1000."""
    _say(f"score gap {dtype} {layout} {order}")
    d, lq = 8, 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    na = 1 if layout == "one_tile" else 200
    g = torch.Generator().manual_seed(21)
    q = torch.zeros(1, 2, lq, d)
    q[..., 0] = 1.0
    ka = torch.zeros(1, 2, na, d)
    kb = torch.zeros(1, 2, 1, d)
    kb[..., 0] = 1000.0
    va = torch.randn(1, 2, na, d, generator=g)
    vb = torch.randn(1, 2, 1, d, generator=g)
    q, ka, kb, va, vb = (t.to(tdt) for t in (q, ka, kb, va, vb))
    kc, vc = ([ka, kb], [va, vb]) if order == "ab" else ([kb, ka], [vb, va])
    out, lse = ra.ring_attention(q.to(DEV), [t.to(DEV) for t in kc], [t.to(DEV) for t in vc], scale=1.0,
                                 return_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    want = vb.float()[:, :, 0:1, :].expand(1, 2, lq, d).to(DEV)
    if dtype == "bf16":
        # the weight of the score-1000 key is exp2 of the fma residual r of its scaled score against the
        # running max (|r| < 2^-13) and exp(-1000) is exactly 0; P.V takes that weight rounded to bf16,
        # exactly 1, while l sums it in fp32, so out = v_B 2^-r: within 2^-13 |v_B|
        assert ((out - want).abs() <= 2.0 ** -13 * want.abs() + 1e-30).all()
    else:
        # fp32 keeps that weight as 1 + O(2^-13 ln 2), so u / l is v_B to a few ulp, not bit for bit
        assert ((out - want).abs() <= 4 * 2.0 ** -24 * want.abs() + 1e-30).all()
    assert torch.allclose(lse, torch.full_like(lse, 1000.0), rtol=0, atol=1e-3)


def test_stats_merge_composition_matches_ring():
    _say("stats+merge vs ring")
    w = wl.custom("comp", "bf16", 1, 4, 4, 128, [(0, 256)], [(0, 300), (300, 200), (500, 12)], False, seed=5)
    q, kc, vc, offs, out, lse = _run(w)
    acc = None
    for k, v in zip(kc, vc):
        st = ra.attention_chunk_stats(q, k, v)
        acc = st if acc is None else ra.merge_chunk_stats(acc, st)
    torch.cuda.synchronize()
    comp = acc[0] / acc[1][..., None]
    ref = _oracle(w, q, kc, vc, offs)
    _check(_np(comp), ref["out"], "bf16")
    assert (comp - out).abs().max().item() <= 2e-2


# ---------------------------------------------------------------------------
# edge cases


def test_edges():
    _say("edges")
    q = torch.randn(1, 2, 5, 64, device=DEV).to(torch.bfloat16)
    e = torch.empty(1, 2, 0, 64, device=DEV, dtype=torch.bfloat16)
    out, lse = ra.ring_attention(q, [e, e], [e, e], 0, [0, 0], causal=False, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    out, lse = ra.ring_attention(q, [], [], 0, [], causal=False, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    # queries before every key: nothing is visible
    k = torch.randn(1, 2, 70, 64, device=DEV).to(torch.bfloat16)
    out, lse = ra.ring_attention(q, [k], [k], 0, [100], causal=True, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    # a query whose only visible key is its own position returns that key's value
    # (to fp32 rounding: l sums the fp32 weight exp2(residual) = 1 +- 2^-23, while
    # u uses the same weight rounded to bf16, exactly 1)
    out = ra.ring_attention(q[:, :, :1], [k], [k * 3], 100, [100], causal=True)
    torch.cuda.synchronize()
    assert torch.allclose(out[0, :, 0], (k * 3)[0, :, 0].float(), atol=1e-6, rtol=1e-6)
    # no queries
    z = ra.ring_attention(q[:, :, :0], [k], [k], 0, [0])
    assert z.shape == (1, 2, 0, 64)
    u, l, m = ra.attention_chunk_stats(q, e, e)
    torch.cuda.synchronize()
    assert torch.all(u == 0) and torch.all(l == 0) and torch.all(torch.isneginf(m))


def test_errors_raise():
    _say("errors")
    q = torch.randn(1, 3, 5, 64, device=DEV).to(torch.bfloat16)
    k = torch.randn(1, 2, 7, 64, device=DEV).to(torch.bfloat16)
    with pytest.raises(ra.RingAttentionError):
        ra.ring_attention(q, [k], [k])  # 3 query heads on 2 kv heads
    with pytest.raises(ra.RingAttentionError):
        ra.ring_attention(q, [k], [k.float()])
    big = torch.randn(1, 1, 4, 130, device=DEV).to(torch.bfloat16)
    with pytest.raises(ra.RingAttentionError):
        ra.ring_attention(big, [big], [big])
    with pytest.raises(ra.RingAttentionError):
        ra.ring_attention(q[:, :2], [k], [k], 0, [-5], causal=True)


def test_kernel_timer_records_one_pair_per_call():
    _say("kernel timer")
    w = wl.custom("timer", "bf16", 1, 2, 2, 64, [(0, 256)], [(0, 512)], False, seed=4)
    q, k, v, kc, vc = wl.generate_torch(w, DEV)
    ref = ra.ring_attention(q, kc, vc, 0, [0])
    torch.cuda.synchronize()
    ra.api.kernel_timer(True)
    for _ in range(3):
        out = ra.ring_attention(q, kc, vc, 0, [0])
    ra.attention_chunk_stats(q, kc[0], vc[0])
    total, n = ra.api.kernel_timer_read()
    ra.api.kernel_timer(False)
    assert n == 4 and total > 0.0
    # recording changes nothing in the results
    assert torch.equal(out, ref)
    ra.ring_attention(q, kc, vc, 0, [0])
    assert ra.api.kernel_timer_read() == (0.0, 0)


# ---------------------------------------------------------------------------
# determinism and causal isolation on the GPU


def test_causal_future_perturbation_is_bitwise_invisible():
    _say("causal perturbation")
    w = wl.custom("pert", "bf16", 1, 2, 2, 128, [(300, 200)], [(0, 256), (256, 256), (512, 256)], True, seed=9)
    q, k, v, kc, vc = wl.generate_torch(w, DEV)
    offs = [o for o, _ in w.chunks]
    out = ra.ring_attention(q, kc, vc, w.q_segments, offs, causal=True)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 420:] = torch.randn_like(k2[:, :, 420:].float()).to(torch.bfloat16) * 5
    v2[:, :, 420:] = 7
    kc2 = [k2[:, :, o:o + n] for o, n in w.chunks]
    vc2 = [v2[:, :, o:o + n] for o, n in w.chunks]
    out2 = ra.ring_attention(q, kc2, vc2, w.q_segments, offs, causal=True)
    torch.cuda.synchronize()
    # rows at positions < 420 see none of the changed keys
    assert torch.equal(out[:, :, :120], out2[:, :, :120])
    assert not torch.equal(out[:, :, 121:], out2[:, :, 121:])


# ---------------------------------------------------------------------------
# the four full-size shares, in the launch configuration the benchmark times

_CACHE = {}


def _full(i):
    if i not in _CACHE:
        _CACHE.clear()
        w = wl.config(i)
        _CACHE[i] = (w, wl.generate_torch(w, DEV))
    return _CACHE[i]


def _resplit_is_bit_identical(w, q, k, v, out, lse):
    """The same ordered keys cut into other chunks (inside key tiles, at shard ends, one key from a shard
    end): bit-identical output and lse."""
    shard = w.chunks[0][1]
    cuts = [1000, shard, shard + 1, 2 * shard - 1, 3 * shard + 77, w.lk // 2 + 1, w.lk - shard + 33]
    r = wl.resplit(w, cuts)
    kc2, vc2 = wl.chunk_views(r, k, v)
    out2, lse2 = ra.ring_attention(q, kc2, vc2, r.q_runs, r.kv_offsets, causal=w.causal, return_lse=True,
                                   kv_position_strides=r.kv_strides)
    torch.cuda.synchronize()
    print(f"  re-split into {len(r.chunks)} chunks (from {len(w.chunks)})", flush=True)
    assert len(r.chunks) > len(w.chunks)
    assert torch.equal(out, out2)
    assert torch.equal(lse, lse2)


@pytest.mark.timeout(600)
def test_full_size_d64_every_row():
    """The d = 64 share in the launch configuration the benchmark times (key range split in two and
    merged), every (head, row) against the oracle over all 32768 keys; then a re-split of its keys must
    give bit-identical results."""
    w, (q, k, v, kc, vc) = _full(1)
    _say(f"{w.name} every row")
    out, lse = ra.ring_attention(q, kc, vc, w.q_runs, w.kv_offsets, causal=w.causal, return_lse=True)
    torch.cuda.synchronize()
    from threadpoolctl import threadpool_limits

    qn = q.float().cpu().double().numpy()
    kn = [c.float().cpu().double().numpy() for c in kc]
    vn = [c.float().cpu().double().numpy() for c in vc]
    tasks = [(h, r0) for h in range(w.q_heads) for r0 in range(0, w.lq, 1024)]

    def run(t):
        h, r0 = t
        hk = h * w.kv_heads // w.q_heads
        return oracle.attention(qn[:, h:h + 1, r0:r0 + 1024], [c[:, hk:hk + 1] for c in kn],
                                [c[:, hk:hk + 1] for c in vn], scale=w.softmax_scale)

    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(_workers()) as ex:
        res = list(ex.map(run, tasks))
    ref_out = np.zeros(tuple(q.shape))
    ref_lse = np.zeros(tuple(q.shape[:3]))
    for (h, r0), r in zip(tasks, res):
        ref_out[:, h, r0:r0 + 1024] = r["out"][:, 0]
        ref_lse[:, h, r0:r0 + 1024] = r["lse"][:, 0]
    err = _check(_np(out), ref_out, "bf16")
    print(f"  out max err {err:.3e}, mean {np.abs(_np(out) - ref_out).mean():.3e}", flush=True)
    _check_lse(_np(lse), ref_lse, "bf16", w.lk)
    _resplit_is_bit_identical(w, q, k, v, out, lse)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("i", [2, 3, 4, 5])
def test_full_size_stratified_rows(i):
    """The causal, zigzag, long GQA and striped shares in the launch configuration the benchmark times, on
    at least 2048 stratified (head, row) pairs (workloads.sample_rows), each against every key; then a
    repeat run and a re-split of the keys must be bit-identical."""
    w, (q, k, v, kc, vc) = _full(i)
    rows = wl.sample_rows(w, 2048, seed=i)
    _say(f"{w.name} stratified {len(rows)} rows")
    offs = w.kv_offsets
    out, lse = ra.ring_attention(q, kc, vc, w.q_runs, offs, causal=w.causal, return_lse=True,
                                 kv_position_strides=w.kv_strides)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()
    ref_out, ref_lse = _oracle_rows_parallel(q, kc, vc, rows, wl.q_positions(w), offs, w.causal, w.kv_strides,
                                             workers=min(_workers(), 8))
    idx = tuple(np.array(rows).T)
    got = out.cpu().double().numpy()[idx]
    err = _check(got, ref_out, "bf16")
    print(f"  out max err {err:.3e}, mean {np.abs(got - ref_out).mean():.3e}", flush=True)
    _check_lse(lse.cpu().double().numpy()[idx], ref_lse, "bf16", w.lk)
    out2 = ra.ring_attention(q, kc, vc, w.q_runs, offs, causal=w.causal, kv_position_strides=w.kv_strides)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    _resplit_is_bit_identical(w, q, k, v, out, lse)
