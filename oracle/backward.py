"""Test infrastructure: gradients of ring attention in fp64 -- the oracle for the backward pass.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may use this module. The product path never imports it.

What it follows
---------------
* "Ring Attention: Distributed Reads with Online Softmax", section "Backward
  must aggregate shared dependencies": a local query contributes gradients to
  the keys and values of every shard it attends to; those contributions are
  summed per key/value owner, with the same score scaling and mask as the
  forward pass, and the distributed result must match a single-device
  reference including gradients.
* The forward pass equals ordinary softmax attention over the concatenated
  chunks (exercise page, problem statement), so its gradients are the
  gradients of that ordinary attention. This module writes them out from the
  chain rule for one query row ``i`` with allowed key set ``A_i``:

    p_ij  = exp(s_ij - lse_i),  s_ij = scale * <q_i, k_j>      (j in A_i)
    dV_j += p_ij * dO_i
    dp_ij = <dO_i, v_j>
    ds_ij = p_ij * (dp_ij - sum_t p_it dp_it)                 (softmax Jacobian)
    dQ_i  = scale * sum_j ds_ij k_j
    dK_j += scale * ds_ij q_i

  ``sum_t p_it dp_it`` equals ``<dO_i, out_i>``. Rows with no allowed key
  contribute nothing. Query head ``h`` uses key/value head ``h // (Hq/Hkv)``,
  so the key/value gradients of a head sum over the query heads of its group.

All arithmetic is numpy float64 on the inputs' exact values. Nothing is
tiled, split or merged: every row sees the whole concatenated key list.
"""

from __future__ import annotations

import numpy as np

from .direct import _f64, key_positions


def attention_backward(q, key_chunks, value_chunks, dout, q_positions=None, kv_offsets=None, causal=False,
                       scale=None, kv_strides=None, max_block_elems=1 << 24):
    """Gradients of ``out = attention(q, chunks)`` against ``dout``.

    q, dout [B, Hq, Lq, d]; chunks [B, Hkv, len, d]. Returns a dict with
    ``dq`` [B, Hq, Lq, d] and ``dk``, ``dv`` [B, Hkv, Lk, d] over the
    concatenated key list (chunk ``c`` is the slice of its keys), plus the
    forward ``out`` and ``lse`` it recomputed. Query rows are taken a block at
    a time (at most ``max_block_elems`` scores) only to bound memory; the key
    gradients add the blocks' contributions.
    """
    q = _f64(q)
    do = _f64(dout)
    B, Hq, Lq, d = q.shape
    k = np.concatenate([_f64(c) for c in key_chunks], axis=2) if key_chunks else np.zeros((B, 1, 0, d))
    v = np.concatenate([_f64(c) for c in value_chunks], axis=2) if value_chunks else np.zeros((B, 1, 0, d))
    Hkv, n = k.shape[1], k.shape[2]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    qpos = np.asarray(q_positions, dtype=np.int64) if causal else None
    kpos = key_positions([c.shape[2] for c in key_chunks], kv_offsets, kv_strides) if causal else None
    dq = np.zeros_like(q)
    dk = np.zeros((B, Hkv, n, d))
    dv = np.zeros((B, Hkv, n, d))
    out = np.zeros((B, Hq, Lq, d))
    lse = np.full((B, Hq, Lq), -np.inf)
    rb = max(1, min(Lq, max_block_elems // max(n, 1))) if Lq else 1
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            for r0 in range(0, Lq, rb):
                r1 = min(Lq, r0 + rb)
                s = scale * (q[b, h, r0:r1] @ k[b, hk].T)
                if causal:
                    s = np.where(kpos[None, :] <= qpos[r0:r1, None], s, -np.inf)
                m = s.max(axis=1) if n else np.full(r1 - r0, -np.inf)
                seen = ~np.isneginf(m)
                w = np.exp(s - np.where(seen, m, 0.0)[:, None])
                l = w.sum(axis=1)
                p = np.where(seen[:, None], w / np.where(seen, l, 1.0)[:, None], 0.0)
                out[b, h, r0:r1] = p @ v[b, hk]
                lse[b, h, r0:r1] = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
                g = do[b, h, r0:r1]
                dp = g @ v[b, hk].T
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dq[b, h, r0:r1] = scale * (ds @ k[b, hk])
                dk[b, hk] += scale * (ds.T @ q[b, h, r0:r1])
                dv[b, hk] += p.T @ g
    return {"dq": dq, "dk": dk, "dv": dv, "out": out, "lse": lse}
