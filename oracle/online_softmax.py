"""Test infrastructure: the exercise's three functions, written out in fp64.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may use this module. The product path never imports it.

This is the reference for the standalone ``attention_chunk_stats`` and
``merge_chunk_stats`` calls. It follows the exercise page
"systems-distributed-ring-attention-online-softmax":

* problem statement -- ``attention_chunk_stats(query, key_chunk, value_chunk)``
  returns ``(chunk_output, chunk_sum, chunk_max)``: the un-normalised weighted
  value sum ``u``, the un-normalised softmax denominator ``l`` and the row-wise
  maximum score ``m``, computed as if the chunk were the only one;
* hint 1 -- the statistics are the stabilised softmax with the row max
  subtracted, with numerator and denominator kept apart;
* hint 2 -- the merge multiplies each side by ``exp(own_max - new_max)`` with
  ``new_max = max(acc_max, chunk_max)`` before adding; statistics relative to
  different maxima are never added directly ("Ring Attention: Distributed Reads
  with Online Softmax", section "Do not average independently normalized shard
  outputs", says the same);
* ``ring_attention`` folds the chunks one at a time into a running summary and
  divides ``u / l`` once at the end (blog post, section "A simple forward
  schedule").

Readings where the pages are silent: the running summary starts at the merge
identity ``(u, l, m) = (0, 0, -inf)``; a chunk with no allowed key for a row has
statistics ``(0, 0, -inf)`` for that row; merging two ``-inf`` maxima keeps the
identity (both correction factors are taken as 0); a row whose final ``l`` is 0
normalises to 0. Scores are in natural-log units, ``s = scale * <q, k>``.
"""

from __future__ import annotations

import numpy as np

from .direct import _f64, key_positions


def chunk_stats(q, k, v, scale, allowed=None):
    """``attention_chunk_stats`` for one chunk: returns ``(u, l, m)``.

    q [..., Lq, d], k and v [..., Lc, d] with matching leading dims. ``allowed``
    is an optional boolean [..., Lq, Lc] mask (the page's function has none; the
    ring fold uses it for the causal case).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = scale * np.matmul(q, np.swapaxes(k, -1, -2))
    if allowed is not None:
        s = np.where(allowed, s, -np.inf)
    if s.shape[-1] == 0:
        lead = s.shape[:-1]
        return np.zeros(lead + (v.shape[-1],)), np.zeros(lead), np.full(lead, -np.inf)
    m = s.max(axis=-1)
    m_safe = np.where(np.isneginf(m), 0.0, m)
    w = np.exp(s - m_safe[..., None])
    l = w.sum(axis=-1)
    u = np.matmul(w, v)
    return u, l, m


def merge_chunk_stats(acc, chunk):
    """Rescale both summaries onto the shared new max, then add.

    ``acc`` and ``chunk`` are ``(u, l, m)`` triples; returns the merged triple.
    """
    u_a, l_a, m_a = (np.asarray(x, dtype=np.float64) for x in acc)
    u_b, l_b, m_b = (np.asarray(x, dtype=np.float64) for x in chunk)
    m = np.maximum(m_a, m_b)
    none = np.isneginf(m)
    with np.errstate(invalid="ignore"):
        alpha_a = np.where(none, 0.0, np.exp(m_a - np.where(none, 0.0, m)))
        alpha_b = np.where(none, 0.0, np.exp(m_b - np.where(none, 0.0, m)))
    l = alpha_a * l_a + alpha_b * l_b
    u = alpha_a[..., None] * u_a + alpha_b[..., None] * u_b
    return u, l, m


def normalize(acc):
    """Final ``u / l`` (0 for a row with ``l = 0``) and ``lse = m + ln l``."""
    u, l, m = acc
    pos = l > 0
    out = np.where(pos[..., None], u / np.where(pos, l, 1.0)[..., None], 0.0)
    with np.errstate(divide="ignore"):
        lse = np.where(pos, m + np.log(np.where(pos, l, 1.0)), -np.inf)
    return out, lse


def ring_attention_fold(q, key_chunks, value_chunks, q_positions=None, kv_offsets=None,
                        causal=False, scale=None, kv_strides=None):
    """Fold the chunks in list order from the identity, then normalise once.

    q [B, Hq, Lq, d]; chunks [B, Hkv, len, d]. ``kv_strides`` (one per chunk,
    default 1) is each chunk's position step. Returns ``(out, lse, (u, l, m))``.
    """
    q = _f64(q)
    B, Hq, Lq, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    acc = (np.zeros((B, Hq, Lq, d)), np.zeros((B, Hq, Lq)), np.full((B, Hq, Lq), -np.inf))
    qpos = np.asarray(q_positions, dtype=np.int64) if causal else None
    for c, (kc, vc) in enumerate(zip(key_chunks, value_chunks)):
        kc, vc = _f64(kc), _f64(vc)
        group = Hq // kc.shape[1]
        kc = np.repeat(kc, group, axis=1)
        vc = np.repeat(vc, group, axis=1)
        allowed = None
        if causal:
            kpos = key_positions([kc.shape[2]], [kv_offsets[c]], None if kv_strides is None else [kv_strides[c]])
            allowed = (kpos[None, :] <= qpos[:, None])[None, None]
        acc = merge_chunk_stats(acc, chunk_stats(q, kc, vc, scale, allowed))
    out, lse = normalize(acc)
    return out, lse, acc
