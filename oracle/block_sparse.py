"""Test infrastructure: attention under a block-sparse mask in fp64 -- the oracle for the sparse ring call.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may use this module. The product path never imports it.

What it follows
---------------
* "Ring Attention: Distributed Reads with Online Softmax", section "What is
  preserved, what is distributed?": the method composes with tiled kernels
  and sparse patterns. The pages name no pattern; the reading here is a
  block-sparse mask over global positions: positions fall into query blocks of
  ``block_q`` and key blocks of ``block_k`` positions, and a boolean matrix
  ``block_mask[a, b]`` says whether a query in block ``a`` may see a key in
  block ``b``.
* Section "Causal masks depend on global positions": like the causal mask, the
  block mask is a function of global positions, never of local indices, so
  it means the same on every device and for every split into chunks. With
  ``causal`` the two masks combine: a key is allowed when the block mask
  allows it and its position is not after the query's.
* Exercise page "systems-distributed-ring-attention-online-softmax", problem
  statement: the ring result is ordinary attention over the concatenated
  keys; here it is ordinary attention restricted to the allowed keys.

So this oracle expands the block mask to the full boolean matrix
``allowed[i, j] = block_mask[qpos_i // block_q, kpos_j // block_k]`` (and
``kpos_j <= qpos_i`` when causal), and evaluates masked softmax attention with
the row maximum subtracted. A row with no allowed key gives output 0,
``l = 0`` and ``m = lse = -inf``. All arithmetic is numpy float64.
"""

from __future__ import annotations

import numpy as np

from .direct import _f64, key_positions


def expand_block_mask(block_mask, block_q, block_k, q_positions, k_positions) -> np.ndarray:
    """Boolean [Lq, Lk] matrix: query at position p sees key at position k iff
    ``block_mask[p // block_q, k // block_k]``."""
    bm = np.asarray(block_mask).astype(bool)
    qb = np.asarray(q_positions, dtype=np.int64) // int(block_q)
    kb = np.asarray(k_positions, dtype=np.int64) // int(block_k)
    return bm[qb[:, None], kb[None, :]]


def attention_block_sparse(q, key_chunks, value_chunks, block_mask, block_q, block_k, q_positions, kv_offsets,
                           causal=False, scale=None, kv_strides=None):
    """Attention of every query row over the allowed keys of the concatenated chunks.

    q [B, Hq, Lq, d]; chunks [B, Hkv, len, d]; query head ``h`` reads key/value
    head ``h // (Hq // Hkv)``. ``q_positions`` [Lq] and ``kv_offsets`` (with
    ``kv_strides``, default 1) give global positions; ``block_mask`` is
    [ceil(n / block_q), ceil(n / block_k)] for positions below ``n``. Returns a
    dict with ``out`` [B, Hq, Lq, d], ``m``, ``l`` and ``lse`` [B, Hq, Lq].
    """
    q = _f64(q)
    B, Hq, Lq, d = q.shape
    k = np.concatenate([_f64(c) for c in key_chunks], axis=2) if key_chunks else np.zeros((B, 1, 0, d))
    v = np.concatenate([_f64(c) for c in value_chunks], axis=2) if value_chunks else np.zeros((B, 1, 0, d))
    group = Hq // k.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qpos = np.asarray(q_positions, dtype=np.int64)
    kpos = key_positions([c.shape[2] for c in key_chunks], kv_offsets, kv_strides)
    allowed = expand_block_mask(block_mask, block_q, block_k, qpos, kpos)
    if causal:
        allowed = allowed & (kpos[None, :] <= qpos[:, None])
    out = np.zeros((B, Hq, Lq, d))
    m = np.full((B, Hq, Lq), -np.inf)
    l = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            s = scale * (q[b, h] @ k[b, h // group].T)
            s = np.where(allowed, s, -np.inf)
            if s.shape[1] == 0:
                continue
            mh = s.max(axis=1)
            seen = ~np.isneginf(mh)
            w = np.exp(s - np.where(seen, mh, 0.0)[:, None])
            lh = w.sum(axis=1)
            out[b, h] = np.where(seen[:, None], (w @ v[b, h // group]) / np.where(seen, lh, 1.0)[:, None], 0.0)
            m[b, h], l[b, h] = mh, lh
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return {"out": out, "m": m, "l": l, "lse": lse}
