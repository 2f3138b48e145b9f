"""Test infrastructure: ordinary softmax attention in fp64 -- the oracle for ring attention.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may use this module. The product path never imports it.

What it follows
---------------
* Exercise page "systems-distributed-ring-attention-online-softmax", problem
  statement: ``ring_attention`` must give exactly the result of ordinary
  attention over the full concatenated key/value sequence, for any split of
  that sequence into chunks. So this oracle *is* ordinary attention over the
  concatenation; it never splits, tiles or merges anything.
* Same page, hint 1: attention is scaled dot-product attention made stable by
  subtracting the row maximum before exponentiating. The scale defaults to
  ``1/sqrt(d)``.
* "Ring Attention: Distributed Reads with Online Softmax", section "Causal
  masks depend on global positions": the causal mask compares *global*
  positions, never local indices. A key is allowed for a query when its global
  position is not after the query's (a key at the same position is allowed).
* Glossary entry "ring attention", paragraph "Online softmax": the combination
  is a log-sum-exp; ``lse = m + ln(l)`` is returned alongside the output.

Rows with no allowed key produce output 0, ``l = 0``, ``m = lse = -inf``.

Layouts: ``q`` is ``[B, Hq, Lq, d]``; each key/value chunk is ``[B, Hkv, len, d]``;
query head ``h`` reads key/value head ``h // (Hq // Hkv)``. All arithmetic is
numpy float64 on the inputs' exact values (bf16 inputs are upcast exactly).
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    """Exact upcast to float64 (numpy array, or torch CPU tensor of any float dtype)."""
    if hasattr(x, "detach"):  # a torch tensor: go through float32, which holds bf16 exactly
        import torch

        x = x.detach().to("cpu")
        if x.dtype != torch.float64:
            x = x.to(torch.float32)
        x = x.numpy()
    return np.asarray(x, dtype=np.float64)


def key_positions(chunk_lengths, kv_offsets, kv_strides=None) -> np.ndarray:
    """Global position of every key of the concatenation, in list order.

    Key ``j`` of a chunk sits at ``offset + stride * j`` (section "Causal masks
    depend on global positions": shard metadata carries the global positions).
    The stride is 1 for a contiguous shard; a striped shard (glossary "ring
    attention", paragraph Variants: striped attention) holds every ``P``-th
    token, stride ``P``.
    """
    if kv_strides is None:
        kv_strides = [1] * len(chunk_lengths)
    parts = [int(o) + int(s) * np.arange(int(n), dtype=np.int64)
             for n, o, s in zip(chunk_lengths, kv_offsets, kv_strides)]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def query_positions(q_segments) -> np.ndarray:
    """Global position of every local query row.

    ``q_segments`` is a list of ``(global_offset, length)`` runs in row order
    (one run for a contiguous share, two for a paired early/late share), or
    ``(global_offset, length, stride)`` runs whose positions advance by
    ``stride`` per row (a striped share).
    """
    parts = [int(g[0]) + (int(g[2]) if len(g) > 2 else 1) * np.arange(int(g[1]), dtype=np.int64)
             for g in q_segments]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def _concat(chunks) -> np.ndarray:
    return np.concatenate([_f64(c) for c in chunks], axis=2)


def _rows_of_head(q_h, k_h, v_h, qpos, kpos, causal, scale):
    """Direct softmax attention for a block of query rows of one head.

    q_h [r, d], k_h [n, d], v_h [n, d], qpos [r], kpos [n]. Returns out [r, d],
    m [r], l [r] with m and l in natural-log score units.
    """
    s = scale * (q_h @ k_h.T)  # [r, n] scores
    if causal:
        allowed = kpos[None, :] <= qpos[:, None]
        s = np.where(allowed, s, -np.inf)
    n = s.shape[1]
    if n == 0:
        r = q_h.shape[0]
        return np.zeros((r, v_h.shape[1])), np.full(r, -np.inf), np.zeros(r)
    m = s.max(axis=1)  # row max over allowed keys (-inf when none)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(s - m_safe[:, None])  # exp(-inf) = 0 for masked keys
    l = w.sum(axis=1)
    num = w @ v_h
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(l[:, None] > 0, num / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return out, m, l


def attention(q, key_chunks, value_chunks, q_positions=None, kv_offsets=None, causal=False,
              scale=None, max_block_elems=1 << 24, kv_strides=None):
    """Ordinary attention of every query row against the concatenated chunks.

    Returns a dict with ``out`` [B, Hq, Lq, d], ``m``, ``l``, ``lse`` [B, Hq, Lq]
    (fp64). ``q_positions`` [Lq] and ``kv_offsets`` (one per chunk) are global
    positions; they are required when ``causal`` is true. ``kv_strides`` (one
    per chunk, default 1) is each chunk's position step.
    """
    q = _f64(q)
    B, Hq, Lq, d = q.shape
    k = _concat(key_chunks) if key_chunks else np.zeros((B, 1, 0, d))
    v = _concat(value_chunks) if value_chunks else np.zeros((B, 1, 0, d))
    Hkv = k.shape[1]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if causal:
        qpos = np.asarray(q_positions, dtype=np.int64)
        kpos = key_positions([c.shape[2] for c in key_chunks], kv_offsets, kv_strides)
    else:
        qpos = np.zeros(Lq, dtype=np.int64)
        kpos = np.zeros(k.shape[2], dtype=np.int64)
    n = k.shape[2]
    rb = max(1, min(Lq, max_block_elems // max(n, 1))) if Lq else 1
    out = np.zeros((B, Hq, Lq, d))
    m = np.full((B, Hq, Lq), -np.inf)
    l = np.zeros((B, Hq, Lq))
    for b in range(B):
        for h in range(Hq):
            kh, vh = k[b, h // group], v[b, h // group]
            for r0 in range(0, Lq, rb):
                r1 = min(Lq, r0 + rb)
                o_, m_, l_ = _rows_of_head(q[b, h, r0:r1], kh, vh, qpos[r0:r1], kpos, causal, scale)
                out[b, h, r0:r1], m[b, h, r0:r1], l[b, h, r0:r1] = o_, m_, l_
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return {"out": out, "m": m, "l": l, "lse": lse}


def attention_rows(q, key_chunks, value_chunks, rows, q_positions=None, kv_offsets=None,
                   causal=False, scale=None, max_block_elems=1 << 24, kv_strides=None):
    """The same definition evaluated only on selected ``(b, h, i)`` query rows.

    Used where the full output is too large for the CPU (long key sequences):
    each selected row is computed exactly as :func:`attention` would, against
    every key of the concatenation. Returns arrays ordered like ``rows``:
    ``out`` [R, d], ``m``, ``l``, ``lse`` [R].
    """
    q = _f64(q) if not isinstance(q, np.ndarray) else q.astype(np.float64, copy=False)
    B, Hq, Lq, d = q.shape
    Hkv = key_chunks[0].shape[1]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lens = [c.shape[2] for c in key_chunks]
    kpos = key_positions(lens, kv_offsets, kv_strides) if causal else np.zeros(sum(lens), dtype=np.int64)
    qpos_all = np.asarray(q_positions, dtype=np.int64) if causal else np.zeros(Lq, dtype=np.int64)
    rows = [tuple(int(x) for x in r) for r in rows]
    R = len(rows)
    out = np.zeros((R, d))
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    by_kv = {}
    for idx, (b, h, i) in enumerate(rows):
        by_kv.setdefault((b, h // group), []).append(idx)
    n = sum(lens)
    rb = max(1, max_block_elems // max(n, 1))
    for (b, hk), idxs in by_kv.items():
        kh = np.concatenate([_f64(c[b, hk]) for c in key_chunks], axis=0)
        vh = np.concatenate([_f64(c[b, hk]) for c in value_chunks], axis=0)
        for j0 in range(0, len(idxs), rb):
            sel = idxs[j0:j0 + rb]
            qs = np.stack([q[rows[t][0], rows[t][1], rows[t][2]] for t in sel])
            qp = np.array([qpos_all[rows[t][2]] for t in sel], dtype=np.int64)
            o_, m_, l_ = _rows_of_head(qs, kh, vh, qp, kpos, causal, scale)
            out[sel], m[sel], l[sel] = o_, m_, l_
    with np.errstate(divide="ignore"):
        lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return {"out": out, "m": m, "l": l, "lse": lse}
