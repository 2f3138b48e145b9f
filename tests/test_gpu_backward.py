"""Parity of the HIP backward pass with the fp64 gradient oracle (needs an MI355X).

Every call goes through the C ABI. The oracle differentiates ordinary
attention over the concatenated chunks from the exact (upcast) bf16 inputs
("Ring Attention: Distributed Reads with Online Softmax", section "Backward
must aggregate shared dependencies": check against a single-device reference,
gradients included).

Tolerance, from the arithmetic: the kernels round the probabilities p and
the score gradients ds to bf16 (relative error <= 2^-9) before the matrix
products that form dV, dK and dQ, and sum in fp32. Each output element is a
sum of terms whose bf16-rounded factors carry independent errors, so its
error is below 2^-9 times the sum of the terms' magnitudes and, in practice,
a small fraction of that. The tests bound the error by BWD_MAX times the largest
reference magnitude and BWD_MEAN times the mean reference magnitude of each gradient.
"""

import zlib

import numpy as np
import pytest
import torch

import oracle
import ring_attention_chunk_amd as ra
from ring_attention_chunk_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BWD_MAX, BWD_MEAN = 1e-2, 5e-3


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np(t):
    return t.detach().cpu().double().numpy()


CASES = [
    # name, B, Hq, Hkv, d, q_segments, chunks, causal, position step
    ("d64_nc_gqa", 2, 4, 2, 64, [(0, 200)], [(0, 100), (100, 37), (137, 150)], False, 1),
    ("d128_causal", 1, 3, 3, 128, [(200, 260)], [(0, 64), (64, 200), (264, 236)], True, 1),
    ("d32_zigzag_gqa", 1, 4, 1, 32, [(64, 64), (448, 64)], [(64 * j, 64) for j in (1, 6, 0, 7, 3, 4, 2, 5)],
     True, 1),
    ("d64_striped", 1, 2, 2, 64, [(3, 150)], [(j, 150) for j in wl.ring_order(3, 4)], True, 4),
    ("d128_nc_one_chunk", 1, 2, 1, 128, [(0, 129)], [(0, 257)], False, 1),
    ("d64_causal_rows_before_keys", 1, 2, 2, 64, [(0, 96)], [(50, 100)], True, 1),
    # head dims that are not a tile width: columns past head_dim are zero-padded in the kernels
    ("d40_causal_gqa", 1, 4, 2, 40, [(100, 150)], [(0, 90), (90, 170)], True, 1),
    ("d16_nc", 1, 2, 2, 16, [(0, 70)], [(0, 33), (33, 60)], False, 1),
    ("d96_causal", 1, 2, 2, 96, [(64, 130)], [(0, 100), (100, 94)], True, 1),
]


def _run_case(w):
    q, k, v, kc, vc = wl.generate_torch(w, DEV)
    g = torch.Generator().manual_seed(zlib.crc32(w.name.encode()))
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(DEV)
    out, lse = ra.ring_attention(q, kc, vc, w.q_runs, w.kv_offsets, causal=w.causal, return_lse=True,
                                 kv_position_strides=w.kv_strides)
    dq, dks, dvs = ra.ring_attention_backward(q, kc, vc, out, lse, dout, w.q_runs, w.kv_offsets, causal=w.causal,
                                              kv_position_strides=w.kv_strides)
    torch.cuda.synchronize()
    return q, kc, vc, dout, out, lse, dq, dks, dvs


def _compare(name, got, ref):
    err = np.abs(got - ref)
    scale_max = max(np.abs(ref).max(), 1e-30)
    scale_mean = max(np.abs(ref).mean(), 1e-30)
    print(f"  {name}: max err {err.max():.3e} (ref max {scale_max:.3e}), mean err {err.mean():.3e} "
          f"(ref mean {scale_mean:.3e})", flush=True)
    assert np.all(np.isfinite(got))
    assert err.max() <= BWD_MAX * scale_max, (name, err.max(), scale_max)
    assert err.mean() <= BWD_MEAN * scale_mean, (name, err.mean(), scale_mean)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_backward_small_shares(case):
    name, B, Hq, Hkv, d, qs, ch, causal, step = case
    _say(f"backward {name}")
    w = wl.custom(name, "bf16", B, Hq, Hkv, d, qs, ch, causal, seed=zlib.crc32(name.encode()) % 1000,
                  pos_stride=step)
    q, kc, vc, dout, out, lse, dq, dks, dvs = _run_case(w)
    ref = oracle.attention_backward(q.cpu(), [c.cpu() for c in kc], [c.cpu() for c in vc], dout.cpu(),
                                    wl.q_positions(w), w.kv_offsets, causal=causal, kv_strides=w.kv_strides)
    _compare("dq", _np(dq), ref["dq"])
    _compare("dk", np.concatenate([_np(t) for t in dks], axis=2), ref["dk"])
    _compare("dv", np.concatenate([_np(t) for t in dvs], axis=2), ref["dv"])
    # keys that no local query sees get exact zeros
    if causal:
        kpos = wl.k_positions(w)
        unseen = kpos > wl.q_positions(w).max()
        if unseen.any():
            assert torch.all(torch.cat(dks, 2)[:, :, torch.from_numpy(unseen)] == 0)


def test_backward_is_bit_reproducible_and_split_invariant_in_dq():
    w = wl.custom("bwd_rep", "bf16", 1, 2, 2, 64, [(100, 200)], [(0, 128), (128, 128), (256, 128)], True, seed=3)
    _say("backward repeat and re-split")
    q, kc, vc, dout, out, lse, dq, dks, dvs = _run_case(w)
    dq2, dks2, dvs2 = ra.ring_attention_backward(q, kc, vc, out, lse, dout, w.q_runs, w.kv_offsets, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2)
    assert all(torch.equal(a, b) for a, b in zip(dks, dks2))
    assert all(torch.equal(a, b) for a, b in zip(dvs, dvs2))
    # the same ordered keys cut elsewhere: identical per-key gradients (every key row is summed over the
    # same queries in the same order) and identical dq (key tiles depend only on the list order)
    r = wl.resplit(w, [50, 200, 300])
    _, k, v, _, _ = wl.generate_torch(w, DEV)
    kc2, vc2 = wl.chunk_views(r, k, v)
    dq3, dks3, dvs3 = ra.ring_attention_backward(q, kc2, vc2, out, lse, dout, r.q_runs, r.kv_offsets, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq3)
    assert torch.equal(torch.cat(dks, 2), torch.cat(dks3, 2))
    assert torch.equal(torch.cat(dvs, 2), torch.cat(dvs3, 2))


def test_backward_errors_raise():
    _say("backward errors")
    q = torch.randn(1, 2, 8, 36, device=DEV).to(torch.bfloat16)
    out = torch.zeros(1, 2, 8, 36, device=DEV)
    lse = torch.zeros(1, 2, 8, device=DEV)
    with pytest.raises(ra.RingAttentionError):  # head_dim 36 is not a multiple of 8
        ra.ring_attention_backward(q, [q], [q], out, lse, q)
    qf = torch.randn(1, 2, 8, 64, device=DEV)
    with pytest.raises(ra.RingAttentionError):  # fp32 inputs
        ra.ring_attention_backward(qf, [qf], [qf], qf, lse, qf)


def _backward_oracle_parallel(q, kc, vc, dout, qpos, offs, causal, parts):
    """oracle.attention_backward on groups of query rows in a thread pool (one BLAS thread each): dq of each
    row comes from its own group; dk and dv are the sums of the groups' contributions (the gradient of a
    key is the sum over the query rows that see it). ``parts`` is a list of (head, row start, row stop)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    qn = q.float().cpu().double().numpy()
    dn = dout.float().cpu().double().numpy()
    kn = [c.float().cpu().double().numpy() for c in kc]
    vn = [c.float().cpu().double().numpy() for c in vc]
    B, Hq, Lq, d = qn.shape
    Hkv = kn[0].shape[1]
    group = Hq // Hkv

    def run(part):
        h, r0, r1 = part
        hk = h // group
        return oracle.attention_backward(qn[:, h:h + 1, r0:r1], [c[:, hk:hk + 1] for c in kn],
                                         [c[:, hk:hk + 1] for c in vn], dn[:, h:h + 1, r0:r1],
                                         None if qpos is None else qpos[r0:r1], offs, causal=causal)

    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(min(len(parts), 16)) as ex:
        res = list(ex.map(run, parts))
    n = sum(c.shape[2] for c in kn)
    dq = np.zeros((B, Hq, Lq, d))
    dk = np.zeros((B, Hkv, n, d))
    dv = np.zeros((B, Hkv, n, d))
    for (h, r0, r1), r in zip(parts, res):
        dq[:, h, r0:r1] = r["dq"][:, 0]
        dk[:, h // group] += r["dk"][:, 0]
        dv[:, h // group] += r["dv"][:, 0]
    return dq, dk, dv


@pytest.mark.timeout(900)
@pytest.mark.parametrize("i", [1, 2, 3])
def test_backward_full_size(i):
    """A full-size share in the benchmark's launch configuration: head 0 in full against the oracle,
    and on every head the sums that hold at any size: the key gradients of a head sum to zero (each row
    of ds sums to zero) and its value gradients sum to the upstream gradients of the rows that see a key
    (each row's weights sum to one)."""
    w = wl.config(i)
    _say(f"backward full size {w.name}")
    q, k, v, kc, vc = wl.generate_torch(w, DEV)
    g = torch.Generator(device=DEV).manual_seed(7)
    dout = torch.randn(q.shape, device=DEV, generator=g).to(torch.bfloat16)
    out, lse = ra.ring_attention(q, kc, vc, w.q_runs, w.kv_offsets, causal=w.causal, return_lse=True)
    dq, dks, dvs = ra.ring_attention_backward(q, kc, vc, out, lse, dout, w.q_runs, w.kv_offsets, causal=w.causal)
    torch.cuda.synchronize()
    dk, dv = torch.cat(dks, 2), torch.cat(dvs, 2)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    group = w.q_heads // w.kv_heads
    seen = torch.isfinite(lse)  # rows that see at least one key
    do_seen = (dout.float() * seen[..., None]).reshape(w.batch, w.kv_heads, group, w.lq, w.head_dim)
    sum_do = do_seen.sum(dim=(2, 3))
    assert ((dv.sum(2) - sum_do).abs() <= 1e-2 * do_seen.abs().sum(dim=(2, 3))).all()
    assert (dk.sum(2).abs() <= 1e-2 * dk.abs().sum(2)).all()
    assert w.q_heads == w.kv_heads  # head 0's key gradients come from query head 0 alone
    step = 512
    parts = [(0, r0, min(w.lq, r0 + step)) for r0 in range(0, w.lq, step)]
    rdq, rdk, rdv = _backward_oracle_parallel(q[:, :1], [c[:, :1] for c in kc], [c[:, :1] for c in vc],
                                              dout[:, :1], wl.q_positions(w) if w.causal else None, w.kv_offsets,
                                              w.causal, parts)
    _compare("dq head 0", _np(dq[:, :1]), rdq)
    _compare("dk head 0", _np(dk[:, :1]), rdk)
    _compare("dv head 0", _np(dv[:, :1]), rdv)


@pytest.mark.timeout(900)
def test_backward_long_gqa_full_share_sampled_dq():
    """The long GQA share (8 query heads on one key/value head, 1,048,576 keys) at full size: on every head
    the sums that hold at any size, and dq of 16 stratified rows per head against the oracle (a row's dq
    depends on that row and every key only, so the oracle of those rows alone gives it exactly)."""
    w = wl.config(4)
    _say(f"backward full size {w.name}: sums and sampled dq")
    q, k, v, kc, vc = wl.generate_torch(w, DEV)
    g = torch.Generator(device=DEV).manual_seed(7)
    dout = torch.randn(q.shape, device=DEV, generator=g).to(torch.bfloat16)
    out, lse = ra.ring_attention(q, kc, vc, return_lse=True)
    dq, dks, dvs = ra.ring_attention_backward(q, kc, vc, out, lse, dout)
    torch.cuda.synchronize()
    dk, dv = torch.cat(dks, 2), torch.cat(dvs, 2)
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()
    sum_do = dout.float().sum(dim=(1, 2))  # [B, d]: every row sees every key
    assert ((dv.sum(2)[:, 0] - sum_do).abs() <= 1e-2 * dout.float().abs().sum(dim=(1, 2))).all()
    assert (dk.sum(2).abs() <= 1e-2 * dk.abs().sum(2)).all()
    rows = [0, 31, 32, 255, 256, 8191, 8192, 16383] + [int(x) for x in np.random.default_rng(44).choice(
        np.arange(1, 16383), 8, replace=False)]
    sel = torch.tensor(rows, device=DEV)
    parts = [(h, 0, len(rows)) for h in range(w.q_heads)]
    rdq, _, _ = _backward_oracle_parallel(q[:, :, sel], kc, vc, dout[:, :, sel], None, w.kv_offsets, False, parts)
    _compare("dq sampled rows", _np(dq[:, :, sel]), rdq)


@pytest.mark.timeout(900)
def test_backward_long_gqa_keys_in_full():
    """The long GQA share at its full key length (1,048,576 keys in 64 shards, the same key and value data)
    with the first 128 queries of each of the 8 query heads: every key's gradient sums the contributions of
    all 8 heads sharing its key/value head; dq, dk and dv are compared in full."""
    base = wl.config(4)
    w = wl.custom("long_gqa_q128_k1m", "bf16", 1, 8, 1, 128, [(0, 128)], base.chunks, False, seq_len=base.seq_len,
                  q_std=base.q_std, seed=base.seed)
    _say(f"backward {w.name}")
    q, kc, vc, dout, out, lse, dq, dks, dvs = _run_case(w)
    parts = [(h, 0, w.lq) for h in range(w.q_heads)]
    rdq, rdk, rdv = _backward_oracle_parallel(q, kc, vc, dout, None, w.kv_offsets, False, parts)
    _compare("dq", _np(dq), rdq)
    _compare("dk", np.concatenate([_np(t) for t in dks], axis=2), rdk)
    _compare("dv", np.concatenate([_np(t) for t in dvs], axis=2), rdv)


def test_backward_very_negative_scores_with_ragged_last_tile():
    """Every score near -160 (lse near -110) makes exp(-lse) overflow fp32. The last key tile (100
    keys: 28 of 128 missing in the last workgroup, 4 of 32 in the last tile) must still be masked so
    that its missing keys give 0, not 0 * inf = NaN, in dq. The scores are made negative by a large
    query against keys whose mean is -1 and whose spread is 1, so that the common part of the keys
    (which the exact dq cancels) is no larger than the rest."""
    _say("backward very negative scores")
    g = torch.Generator().manual_seed(12)
    d, Lq, Lk = 64, 64, 100
    q = (20.0 * torch.ones(1, 2, Lq, d) + 0.5 * torch.randn(1, 2, Lq, d, generator=g)).to(torch.bfloat16)
    k = (-1.0 + torch.randn(1, 2, Lk, d, generator=g)).to(torch.bfloat16)
    v = torch.randn(1, 2, Lk, d, generator=g).to(torch.bfloat16)
    dout = torch.randn(1, 2, Lq, d, generator=g).to(torch.bfloat16)
    qd, kd, vd, dd = (t.to(DEV) for t in (q, k, v, dout))
    out, lse = ra.ring_attention(qd, [kd], [vd], return_lse=True)
    dq, dks, dvs = ra.ring_attention_backward(qd, [kd], [vd], out, lse, dd)
    torch.cuda.synchronize()
    print(f"  lse max {lse.max().item():.1f}", flush=True)
    assert lse.max().item() < -88.0  # exp(-lse) is beyond fp32
    ref = oracle.attention_backward(q, [k], [v], dout)
    _compare("dq", _np(dq), ref["dq"])
    _compare("dk", _np(dks[0]), ref["dk"])
    _compare("dv", _np(dvs[0]), ref["dv"])
