"""Pins of the block-sparse oracle (CPU only).

``oracle.block_sparse.attention_block_sparse`` is ordinary attention restricted
to the keys a block mask over global positions allows ("Ring Attention:
Distributed Reads with Online Softmax", section "What is preserved, what is
distributed?": the method composes with sparse patterns; section "Causal masks
depend on global positions": masks follow global positions). Each pin ties it
to something other than itself:

* an all-ones mask is dense attention (``oracle.attention``, pinned elsewhere);
* a block-lower-triangular mask with the causal flag is causal attention, since
  every causally visible key lies in a visible block;
* a mask that allows a set of key blocks is dense attention over just those
  keys (a sliding window of blocks, a single block, an empty row);
* torch's scaled_dot_product_attention in float64 with the boolean mask of a
  block pattern written as a comparison of block numbers;
* brute force in plain Python on tiny inputs;
* any re-split of the chunk list, and the fold of per-chunk masked statistics
  merged by the rescale rule, give the same result.

Planted mistakes (one-line source edits) must each break a pin.
"""

import importlib.util
import inspect
import math

import numpy as np
import pytest

import oracle
import oracle.block_sparse as obs
from oracle.direct import key_positions


def _share(seed, causal_layout="contig", B=1, Hq=4, Hkv=2, d=5, n=48, lq=12):
    """Query positions and a chunk list (offsets, lengths) over positions 0..n-1, plus random data."""
    rng = np.random.default_rng([seed, 3])
    if causal_layout == "contig":
        qpos = np.arange(n - lq, n)
        offs, lens = [32, 16, 0], [16, 16, 16]
    else:  # paired early/late query runs, chunks out of position order and cut unevenly
        qpos = np.concatenate([np.arange(4, 4 + lq // 2), np.arange(n - lq // 2, n)])
        offs, lens = [40, 8, 0, 27, 20], [8, 19, 8, 13, 7]
    q = rng.standard_normal((B, Hq, lq, d)) * 1.3
    kc = [rng.standard_normal((B, Hkv, ln, d)) for ln in lens]
    vc = [rng.standard_normal((B, Hkv, ln, d)) for ln in lens]
    return q, kc, vc, qpos, offs


def _err(a, b):
    fin = np.isfinite(b["lse"])
    e = max(np.abs(a["out"] - b["out"]).max(), np.abs(a["lse"][fin] - b["lse"][fin]).max() if fin.any() else 0.0)
    return e if np.array_equal(np.isneginf(a["lse"]), np.isneginf(b["lse"])) else np.inf


def _pin_all_ones(f):
    worst = 0.0
    for layout in ("contig", "zigzag"):
        q, kc, vc, qpos, offs = _share(1, layout)
        for causal in (False, True):
            mask = np.ones((3, 12), dtype=np.uint8)
            got = f(q, kc, vc, mask, 16, 4, qpos, offs, causal=causal)
            ref = oracle.attention(q, kc, vc, qpos, offs, causal=causal)
            worst = max(worst, _err(got, ref))
    return worst


def _pin_block_causal(f):
    worst = 0.0
    for layout in ("contig", "zigzag"):
        q, kc, vc, qpos, offs = _share(2, layout)
        B = 8
        mask = np.tril(np.ones((6, 6), dtype=np.uint8))
        got = f(q, kc, vc, mask, B, B, qpos, offs, causal=True)
        ref = oracle.attention(q, kc, vc, qpos, offs, causal=True)
        worst = max(worst, _err(got, ref))
    return worst


def _dense_over_key_subset(q, kc, vc, offs, keep_pos):
    """oracle.attention over only the keys whose positions are in keep_pos (as one-key chunks, in list
    order); rows see all of them (no mask)."""
    kpos = key_positions([c.shape[2] for c in kc], offs)
    k = np.concatenate(kc, axis=2)
    v = np.concatenate(vc, axis=2)
    idx = [j for j in range(len(kpos)) if kpos[j] in keep_pos]
    return oracle.attention(q, [k[:, :, idx]], [v[:, :, idx]])


def _pin_key_block_subsets(f):
    """Per query block, a window of key blocks (and one query block whose row of the mask is empty): every
    query row equals dense attention over exactly the keys of its allowed blocks."""
    worst = 0.0
    q, kc, vc, qpos, offs = _share(3, "zigzag", lq=12)
    bq, bk = 4, 8
    nqb, nkb = 12, 6
    mask = np.zeros((nqb, nkb), dtype=np.uint8)
    for a in range(nqb):
        mask[a, max(0, a // 2 - 1):a // 2 + 1] = 1  # a window of two key blocks
    mask[qpos[0] // bq] = 0  # an empty row
    mask[qpos[-1] // bq] = 0
    mask[qpos[-1] // bq, 3] = 1  # a single key block
    got = f(q, kc, vc, mask, bq, bk, qpos, offs)
    for i, p in enumerate(qpos):
        allowed_blocks = np.nonzero(mask[p // bq])[0]
        keep = {int(x) for b in allowed_blocks for x in range(b * bk, (b + 1) * bk)}
        if not keep:
            worst = max(worst, np.abs(got["out"][:, :, i]).max(), 0.0 if np.isneginf(got["lse"][:, :, i]).all()
                        else np.inf)
            continue
        ref = _dense_over_key_subset(q[:, :, i:i + 1], kc, vc, offs, keep)
        worst = max(worst, np.abs(got["out"][:, :, i:i + 1] - ref["out"]).max(),
                    np.abs(got["lse"][:, :, i:i + 1] - ref["lse"]).max())
    return worst


def _pin_torch_sdpa(f):
    torch = pytest.importorskip("torch")
    q, kc, vc, qpos, offs = _share(4, "zigzag", Hq=2, Hkv=2)
    bq, bk = 8, 4
    rng = np.random.default_rng(9)
    mask = (rng.random((6, 12)) < 0.5).astype(np.uint8)
    mask[:, 0] = 1  # every row sees something
    got = f(q, kc, vc, mask, bq, bk, qpos, offs)
    kpos = key_positions([c.shape[2] for c in kc], offs)
    qb = torch.tensor(qpos // bq)[:, None]
    kb = torch.tensor(kpos // bk)[None, :]
    tm = torch.tensor(mask, dtype=torch.bool)[qb.expand(-1, len(kpos)), kb.expand(len(qpos), -1)]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q), torch.tensor(np.concatenate(kc, axis=2)), torch.tensor(np.concatenate(vc, axis=2)),
        attn_mask=tm).numpy()
    return np.abs(got["out"] - ref).max()


def _pin_brute_force(f):
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 3, 2))
    kc = [rng.standard_normal((1, 1, 2, 2)), rng.standard_normal((1, 1, 3, 2))]
    vc = [rng.standard_normal((1, 1, 2, 2)), rng.standard_normal((1, 1, 3, 2))]
    offs = [3, 0]
    qpos = [1, 3, 4]
    kpos = [3, 4, 0, 1, 2]
    mask = [[1, 0, 1], [0, 1, 1], [1, 1, 0]]  # block size 2 for both
    worst = 0.0
    for causal in (False, True):
        got = f(q, kc, vc, np.array(mask, dtype=np.uint8), 2, 2, qpos, offs, causal=causal)
        K = [list(x) for x in np.concatenate(kc, axis=2)[0, 0]]
        V = [list(x) for x in np.concatenate(vc, axis=2)[0, 0]]
        for i in range(3):
            ok = [j for j in range(5) if mask[qpos[i] // 2][kpos[j] // 2] and (not causal or kpos[j] <= qpos[i])]
            if not ok:
                worst = max(worst, np.abs(got["out"][0, 0, i]).max())
                continue
            s = {j: sum(a * b for a, b in zip(q[0, 0, i], K[j])) / math.sqrt(2) for j in ok}
            mx = max(s.values())
            w = {j: math.exp(s[j] - mx) for j in ok}
            tot = sum(w.values())
            ref = [sum(w[j] * V[j][c] for j in ok) / tot for c in range(2)]
            worst = max(worst, np.abs(got["out"][0, 0, i] - ref).max(),
                        abs(got["lse"][0, 0, i] - (mx + math.log(tot))))
    return worst


def _resplit(kc, vc, offs, cuts):
    """The same ordered keys cut at the given indices of the concatenation; every key keeps its position."""
    out_k, out_v, out_o = [], [], []
    start = 0
    for k, v, o in zip(kc, vc, offs):
        n = k.shape[2]
        inner = [c - start for c in cuts if start < c < start + n]
        edges = [0] + inner + [n]
        for a, b in zip(edges[:-1], edges[1:]):
            out_k.append(k[:, :, a:b])
            out_v.append(v[:, :, a:b])
            out_o.append(o + a)
        start += n
    return out_k, out_v, out_o


def _pin_split_invariance(f):
    """Re-splits of the key list (including chunks of one key), and the fold of masked per-chunk statistics
    merged by the rescale rule, agree with the whole list."""
    q, kc, vc, qpos, offs = _share(6, "zigzag")
    rng = np.random.default_rng(6)
    mask = (rng.random((6, 6)) < 0.6).astype(np.uint8)
    bq = bk = 8
    n = sum(c.shape[2] for c in kc)
    worst = 0.0
    for causal in (False, True):
        ref = f(q, kc, vc, mask, bq, bk, qpos, offs, causal=causal)
        for cuts in ([1], [5, 6, 7], list(range(1, n)), [20, 33]):
            kc2, vc2, offs2 = _resplit(kc, vc, offs, cuts)
            worst = max(worst, _err(f(q, kc2, vc2, mask, bq, bk, qpos, offs2, causal=causal), ref))
        # the fold: statistics of each chunk under its part of the expanded mask, merged in list order
        Hq, Hkv = q.shape[1], kc[0].shape[1]
        acc = (np.zeros(q.shape), np.zeros(q.shape[:3]), np.full(q.shape[:3], -np.inf))
        for c in range(len(kc)):
            kp = key_positions([kc[c].shape[2]], [offs[c]])
            allowed = obs.expand_block_mask(mask, bq, bk, qpos, kp)
            if causal:
                allowed = allowed & (kp[None, :] <= qpos[:, None])
            st = oracle.chunk_stats(q, np.repeat(kc[c], Hq // Hkv, axis=1), np.repeat(vc[c], Hq // Hkv, axis=1),
                                    1 / math.sqrt(q.shape[-1]), allowed[None, None])
            acc = oracle.merge_chunk_stats(acc, st)
        out, lse = oracle.normalize(acc)
        worst = max(worst, _err({"out": out, "lse": lse}, ref))
    return worst


PINS = [_pin_all_ones, _pin_block_causal, _pin_key_block_subsets, _pin_torch_sdpa, _pin_brute_force,
        _pin_split_invariance]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    assert pin(obs.attention_block_sparse) <= 1e-12


def _mutated(old, new):
    src = inspect.getsource(obs)
    assert src.count(old) == 1, old
    spec = importlib.util.spec_from_loader("oracle._block_sparse_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "oracle_block_sparse_mutant", "exec"), mod.__dict__)
    return mod.attention_block_sparse


MUTANTS = [
    ("mask read transposed", "return bm[qb[:, None], kb[None, :]]", "return bm.T[qb[:, None] % bm.shape[1], "
                                                                   "kb[None, :] % bm.shape[0]]"),
    ("block sizes swapped", "expand_block_mask(block_mask, block_q, block_k, qpos, kpos)",
     "expand_block_mask(block_mask, block_k, block_q, qpos, kpos)"),
    ("query block off by one position", "qb = np.asarray(q_positions, dtype=np.int64) // int(block_q)",
     "qb = (np.asarray(q_positions, dtype=np.int64) + 1) // int(block_q)"),
    ("local key index instead of position", "kpos = key_positions([c.shape[2] for c in key_chunks], kv_offsets, "
     "kv_strides)", "kpos = np.arange(sum(c.shape[2] for c in key_chunks))"),
    ("block mask dropped under causal", "allowed = allowed & (kpos[None, :] <= qpos[:, None])",
     "allowed = kpos[None, :] <= qpos[:, None]"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new):
    f = _mutated(old, new)
    worst = 0.0
    for pin in PINS:
        try:
            worst = max(worst, pin(f))
        except (IndexError, ValueError):
            worst = np.inf
    assert worst > 1e-6, name
