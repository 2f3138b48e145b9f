"""Parity of the block-sparse ring call with the block-sparse oracle (needs an MI355X).

``ra_ring_attention_block_sparse`` restricts ring attention to the key blocks a
mask over global positions allows ("Ring Attention: Distributed Reads with
Online Softmax", section "What is preserved, what is distributed?": the method
composes with sparse patterns). Every call goes through the C ABI. The oracle
is ``oracle.attention_block_sparse`` on the exact (upcast) inputs; tolerances
are those of the dense call (bf16: max abs 2e-2, mean abs 2e-3, lse within the
bound derived in test_gpu_parity; fp32: 1e-5).

Cases cover both kernels: the pipelined bf16 kernel (each wave's 32 rows in one
query block, consecutive key positions, key blocks of at least one key tile)
and the general kernel (fp32, striped positions, key blocks shorter than a
tile, waves that straddle query blocks, head_dim not a multiple of 8).
"""

import math
import zlib

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


def _lse_tol(dtype, n_keys):
    if dtype == "f32":
        return F32_TOL
    return 2.0 ** -9 + math.ceil(max(n_keys, 1) / 64) * 2.0 ** -24 + 1e-5


def _mask(kind, nqb, nkb, seed, density=0.5, width=2):
    rng = np.random.default_rng([seed, 77])
    if kind == "random":
        m = rng.random((nqb, nkb)) < density
    elif kind == "window":  # a band of key blocks around each query block plus the first key block
        a = np.arange(nqb)[:, None]
        b = np.arange(nkb)[None, :]
        scale = nkb / max(nqb, 1)
        m = (np.abs(b - a * scale) <= width) | (b == 0)
    elif kind == "ones":
        m = np.ones((nqb, nkb), bool)
    else:
        raise ValueError(kind)
    return m.astype(np.uint8)


def _run(w, mask, bq, bk, **kw):
    q, k, v, kc, vc = wl.generate_torch(w, DEV)
    out, lse = ra.ring_attention_block_sparse(q, kc, vc, torch.from_numpy(mask).to(DEV), bq, bk, w.q_runs,
                                              w.kv_offsets, causal=w.causal, scale=w.softmax_scale, return_lse=True,
                                              kv_position_strides=w.kv_strides, **kw)
    torch.cuda.synchronize()
    return q, k, v, kc, vc, out, lse


def _oracle(w, q, kc, vc, mask, bq, bk):
    return oracle.attention_block_sparse(q.cpu(), [c.cpu() for c in kc], [c.cpu() for c in vc], mask, bq, bk,
                                         wl.q_positions(w), w.kv_offsets, causal=w.causal, scale=w.softmax_scale,
                                         kv_strides=w.kv_strides)


def _compare(w, out, lse, ref):
    got, want = _np(out), ref["out"]
    err = np.abs(got - want)
    assert np.all(np.isfinite(got))
    if w.dtype == "f32":
        assert err.max() <= F32_TOL, err.max()
    else:
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    gl = _np(lse)
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isfinite(gl), fin)
    lerr = np.abs(gl[fin] - ref["lse"][fin]).max() if fin.any() else 0.0
    print(f"  out max err {err.max():.3e} mean {err.mean():.3e}; lse max err {lerr:.3e}; rows with no key "
          f"{int((~fin).sum())}", flush=True)
    assert lerr <= _lse_tol(w.dtype, w.lk)
    # rows with no allowed key: exactly 0
    assert np.all(got[~fin] == 0.0)


def _chunks(order, size):
    return [(j * size, size) for j in order]


CASES = [
    # name, dtype, B, Hq, Hkv, d, q_segments, chunks, causal, pos_stride, mask kind, block_q, block_k
    ("pipe_causal_d128_random", "bf16", 1, 4, 2, 128, [(1536, 512)], _chunks([3, 2, 1, 0], 512), True, 1,
     "random", 256, 128),
    ("pipe_nc_d64_gqa_ragged", "bf16", 2, 4, 1, 64, [(0, 300)], [(0, 400), (400, 600)], False, 1, "random", 64, 128),
    ("pipe_zigzag_d128_window", "bf16", 1, 2, 2, 128, [(512, 256), (3328, 256)],
     [c for j in (1, 0, 3, 2) for c in ((512 * j, 512), ((7 - j) * 512, 512))], True, 1, "window", 256, 256),
    ("pipe_causal_d64_sparse", "bf16", 1, 2, 2, 64, [(1024, 1024)], _chunks([1, 0, 3, 2], 512), True, 1, "random",
     128, 512),
    ("gen_f32_d32_small_blocks", "f32", 1, 2, 1, 32, [(200, 120)], [(0, 150), (150, 170)], True, 1, "random", 16, 16),
    ("gen_bf16_striped", "bf16", 1, 2, 2, 64, [(1, 256)], [(j, 256) for j in wl.ring_order(1, 4)], True, 4,
     "random", 64, 64),
    ("gen_bf16_waves_straddle", "bf16", 1, 2, 2, 64, [(0, 200)], [(0, 700)], False, 1, "window", 16, 128),
    ("gen_bf16_d100", "bf16", 1, 2, 2, 100, [(0, 150)], [(0, 300), (300, 100)], False, 1, "random", 32, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_block_sparse_small(case):
    name, dtype, B, Hq, Hkv, d, qs, ch, causal, step, kind, bq, bk = case
    _say(name)
    w = wl.custom(name, dtype, B, Hq, Hkv, d, qs, ch, causal, seed=zlib.crc32(name.encode()) % 1000,
                  pos_stride=step)
    nqb = -(-w.seq_len // bq)
    nkb = -(-w.seq_len // bk)
    mask = _mask(kind, nqb, nkb, zlib.crc32(name.encode()))
    q, k, v, kc, vc, out, lse = _run(w, mask, bq, bk)
    ref = _oracle(w, q, kc, vc, mask, bq, bk)
    _compare(w, out, lse, ref)
    # a re-split of the same ordered keys (cuts inside tiles) gives bit-identical results
    cuts = [7, w.lk // 3, w.lk // 2 + 5]
    r = wl.resplit(w, cuts)
    kc2, vc2 = wl.chunk_views(r, k, v)
    out2, lse2 = ra.ring_attention_block_sparse(q, kc2, vc2, torch.from_numpy(mask).to(DEV), bq, bk, r.q_runs,
                                                r.kv_offsets, causal=w.causal, scale=w.softmax_scale,
                                                return_lse=True, kv_position_strides=r.kv_strides)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("i", [0, 1, 2])
def test_all_ones_mask_is_the_dense_call_bit_for_bit(i):
    """With every block allowed the sparse call visits the dense call's tiles in the same order with the same
    arithmetic: bit-identical output and lse."""
    name, dtype, B, Hq, Hkv, d, qs, ch, causal, step, _, bq, bk = CASES[i]
    _say(f"all ones {name}")
    w = wl.custom(name, dtype, B, Hq, Hkv, d, qs, ch, causal, seed=3, pos_stride=step)
    mask = _mask("ones", -(-w.seq_len // bq), -(-w.seq_len // bk), 0)
    q, k, v, kc, vc, out, lse = _run(w, mask, bq, bk)
    dense, dlse = ra.ring_attention(q, kc, vc, w.q_runs, w.kv_offsets, causal=w.causal, return_lse=True,
                                    kv_position_strides=w.kv_strides)
    torch.cuda.synchronize()
    assert torch.equal(out, dense) and torch.equal(lse, dlse)


def test_block_sparse_rows_without_keys_and_empty_mask():
    """Query blocks whose mask row is empty get out = 0 and lse = -inf; an all-zero mask gives that for
    every row."""
    _say("empty rows")
    w = wl.custom("sp_empty", "bf16", 1, 2, 2, 64, [(0, 256)], [(0, 512)], False, seed=4)
    mask = np.ones((4, 4), np.uint8)
    mask[1] = 0
    q, k, v, kc, vc, out, lse = _run(w, mask, 64, 128)
    assert torch.all(out[:, :, 64:128] == 0) and torch.all(torch.isneginf(lse[:, :, 64:128]))
    assert torch.isfinite(lse[:, :, :64]).all() and torch.isfinite(lse[:, :, 128:]).all()
    out0, lse0 = ra.ring_attention_block_sparse(q, kc, vc, torch.zeros(4, 4, dtype=torch.uint8, device=DEV), 64, 128,
                                                return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out0 == 0) and torch.all(torch.isneginf(lse0))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("kind", ["window", "random"])
def test_block_sparse_medium_share_in_full(kind):
    """A causal share of 8 heads, d = 128, 2048 queries at 6144..8191 against 8192 keys in 4 shards in ring
    order, under a block mask of 256-position blocks (a band of key blocks plus the first key block, or
    random blocks at density 0.4): every row against the oracle."""
    _say(f"medium {kind}")
    w = wl.custom(f"sp_medium_{kind}", "bf16", 1, 8, 8, 128, [(6144, 2048)], _chunks([3, 2, 1, 0], 2048), True,
                  seed=31)
    mask = _mask(kind, 32, 32, 9, density=0.4, width=3)
    q, k, v, kc, vc, out, lse = _run(w, mask, 256, 256)
    from concurrent.futures import ThreadPoolExecutor

    qn, kn, vn = q.cpu(), [c.cpu() for c in kc], [c.cpu() for c in vc]

    def head(h):
        return oracle.attention_block_sparse(qn[:, h:h + 1], [c[:, h:h + 1] for c in kn], [c[:, h:h + 1] for c in vn],
                                             mask, 256, 256, wl.q_positions(w), w.kv_offsets, causal=True)

    with ThreadPoolExecutor(8) as ex:
        parts = list(ex.map(head, range(8)))
    ref = {key: np.concatenate([p_[key] for p_ in parts], axis=1) for key in ("out", "lse")}
    _compare(w, out, lse, ref)
