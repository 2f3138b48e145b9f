"""Seeded synthetic workloads for ring attention on one device's share.

This module only builds inputs: random values, bf16 rounding of those inputs,
and the position / ring-order bookkeeping of a share. It holds none of the
method's arithmetic, so both the HIP path and the fp64 oracle consume what it
produces without sharing any code with each other.

Positions follow "Ring Attention: Distributed Reads with Online Softmax":
a sequence of ``n`` tokens is cut into ``P`` shards (section "Partition the
sequence across devices"); the device at ring index ``r`` meets, at step
``s``, the shard of device ``(r - s) mod P`` (it receives from its
predecessor), so the chunk list below is in that ring order. Section "Causal
masks depend on global positions" gives the two causal layouts used here:
contiguous shards and paired early/late chunks ("zigzag": with ``2P`` chunks,
device ``r`` owns chunks ``r`` and ``2P-1-r``). The glossary entry "ring
attention" (paragraph Variants) adds striped attention, read here as the
round-robin layout: device ``r`` owns positions ``r, r+P, r+2P, ...``, so a
shard is a run of positions with step ``P`` (``pos_stride``) and its keys lie
contiguous in that device's memory.

Values: q, k, v are standard normal fp32, drawn per block of global positions
from ``numpy.random.default_rng([seed, tensor, block])`` so that any re-split of
the same positions sees identical values; bf16 workloads round them to bf16
(round to nearest even) before either side sees them.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

POS_BLOCK = 4096  # positions per seeded block


@dataclasses.dataclass
class Workload:
    """One device's share: local queries and the K/V chunks it meets, in ring order."""

    name: str
    dtype: str  # "f32" or "bf16"
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    q_segments: List[Tuple[int, int]]  # (global_offset, length) per run of local query rows
    chunks: List[Tuple[int, int]]  # (global_offset, length) per K/V chunk, list order = ring order
    causal: bool
    seq_len: int  # n: positions 0..n-1 hold keys
    q_std: float = 1.0
    seed: int = 0
    scale: Optional[float] = None  # None means 1/sqrt(head_dim)
    pos_stride: int = 1  # position step inside every query run and chunk (P for a striped share)

    @property
    def lq(self) -> int:
        return sum(n for _, n in self.q_segments)

    @property
    def lk(self) -> int:
        return sum(n for _, n in self.chunks)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / float(np.sqrt(self.head_dim))

    @property
    def kv_offsets(self) -> List[int]:
        return [o for o, _ in self.chunks]

    @property
    def kv_strides(self) -> List[int]:
        return [self.pos_stride] * len(self.chunks)

    @property
    def q_runs(self) -> List[Tuple[int, int, int]]:
        """Query runs as ``(global_offset, length, position step)``."""
        return [(o, n, self.pos_stride) for o, n in self.q_segments]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even); result stays fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) & np.uint32(0xFFFF0000)).view(np.float32)


def ring_order(rank: int, world: int) -> List[int]:
    """Shard seen at each ring step by device ``rank``: ``(rank - step) mod world``."""
    return [(rank - s) % world for s in range(world)]


# ---------------------------------------------------------------------------
# the five workloads


def scalar_case() -> dict:
    """Two single-key shards: A has score 0 and value 0, B has score 10 and value 1.

    From section "Do not average independently normalized shard outputs": with
    d = 1, scale 1 and q = 1 the scores are the keys themselves.
    """
    return {
        "q": np.ones((1, 1, 1, 1), np.float32),
        "k": [np.zeros((1, 1, 1, 1), np.float32), np.full((1, 1, 1, 1), 10.0, np.float32)],
        "v": [np.zeros((1, 1, 1, 1), np.float32), np.ones((1, 1, 1, 1), np.float32)],
        "kv_offsets": [0, 1],
        "q_positions": [1],
        "scale": 1.0,
    }


def tiny(causal: bool = False) -> Workload:
    """fp32, 1 head, d=16, 8 queries, 32 keys in chunks [1, 3, 12, 16]; causal queries at 24..31."""
    return Workload("tiny_f32" + ("_causal" if causal else ""), "f32", 1, 1, 1, 16,
                    [(24, 8)], [(0, 1), (1, 3), (4, 12), (16, 16)], causal, 32, seed=100)


def noncausal_d64() -> Workload:
    """bf16, 8 heads, d=64, 4096 local queries (device 0 of 8) vs 8 shards of 4096."""
    P, L = 8, 4096
    return Workload("noncausal_h8_d64_q4k_k32k", "bf16", 1, 8, 8, 64, [(0, L)],
                    [(j * L, L) for j in ring_order(0, P)], False, P * L, seed=101)


def causal_contiguous() -> Workload:
    """bf16, 32 heads, d=128, device 5 of 8, n=65536: 8192 queries at 40960..49151."""
    P, L, r = 8, 8192, 5
    return Workload("causal_contig_r5of8_h32_d128_n64k", "bf16", 1, 32, 32, 128, [(r * L, L)],
                    [(j * L, L) for j in ring_order(r, P)], True, P * L, seed=102)


def causal_zigzag() -> Workload:
    """bf16, 32 heads, d=128, device 3 of 16, n=131072 in 32 chunks of 4096.

    The local share is chunks 3 and 28; shard ``j`` is chunks ``j`` and ``31-j``,
    passed as two chunk descriptors each.
    """
    P, C, r = 16, 4096, 3
    chunks = []
    for j in ring_order(r, P):
        chunks += [(j * C, C), ((2 * P - 1 - j) * C, C)]
    return Workload("causal_zigzag_r3of16_h32_d128_n128k", "bf16", 1, 32, 32, 128,
                    [(r * C, C), ((2 * P - 1 - r) * C, C)], chunks, True, 2 * P * C, seed=103)


def long_gqa() -> Workload:
    """bf16 GQA, 8 query heads on 1 KV head, d=128, 16384 queries vs 64 shards of 16384."""
    P, L = 64, 16384
    return Workload("long_gqa_hq8_hkv1_d128_q16k_k1m", "bf16", 1, 8, 1, 128, [(0, L)],
                    [(j * L, L) for j in ring_order(0, P)], False, P * L, q_std=4.0, seed=104)


def causal_striped(P: int = 8, r: int = 5, n: int = 65536, heads: int = 32, d: int = 128) -> Workload:
    """bf16 striped causal share: device r of P holds positions r, r+P, ...; shard j holds j, j+P, ...

    At the defaults it is the contiguous causal share's shape (32 heads, d=128,
    n=65536, device 5 of 8) in the striped layout, where every shard is about
    half visible instead of whole shards being visible or hidden.
    """
    L = n // P
    return Workload(f"causal_striped_r{r}of{P}_h{heads}_d{d}_n{n // 1024}k", "bf16", 1, heads, heads, d,
                    [(r, L)], [(j, L) for j in ring_order(r, P)], True, n, seed=105, pos_stride=P)


CONFIGS = {0: tiny, 1: noncausal_d64, 2: causal_contiguous, 3: causal_zigzag, 4: long_gqa, 5: causal_striped}


def config(i: int, **kw) -> Workload:
    return CONFIGS[i](**kw)


def custom(name, dtype, batch, q_heads, kv_heads, head_dim, q_segments, chunks, causal,
           seq_len=None, q_std=1.0, seed=7, scale=None, pos_stride=1) -> Workload:
    if seq_len is None:
        ends = [o + pos_stride * (n - 1) + 1 for o, n in list(chunks) + list(q_segments) if n > 0]
        seq_len = max(ends + [0])
    return Workload(name, dtype, batch, q_heads, kv_heads, head_dim, list(q_segments), list(chunks),
                    causal, seq_len, q_std, seed, scale, pos_stride)


def resplit(w: Workload, cuts: Sequence[int]) -> Workload:
    """The same ordered key sequence cut into chunks at other places.

    ``cuts`` are indices into the concatenated key list. Adjacent chunks whose
    positions continue each other are first joined; the joined runs are then cut
    at ``cuts``. Every key keeps its place and its global position, so the data
    and the exact result are unchanged.
    """
    st = w.pos_stride
    runs = []
    for o, n in w.chunks:
        if n == 0:
            continue
        if runs and runs[-1][0] + st * runs[-1][1] == o:
            runs[-1] = (runs[-1][0], runs[-1][1] + n)
        else:
            runs.append((o, n))
    bounds = sorted(set(int(c) for c in cuts if 0 < int(c) < w.lk))
    out, s0 = [], 0
    for o, n in runs:
        inner = [c - s0 for c in bounds if s0 < c < s0 + n]
        edges = [0] + inner + [n]
        out += [(o + st * a, b - a) for a, b in zip(edges[:-1], edges[1:])]
        s0 += n
    return dataclasses.replace(w, chunks=out, name=w.name + "_resplit")


# ---------------------------------------------------------------------------
# value generation


def _normal_positions(seed: int, tensor: int, lead: Tuple[int, ...], start: int, stop: int,
                      d: int) -> np.ndarray:
    """Standard normals for positions [start, stop), seeded per block of POS_BLOCK positions."""
    out = np.empty(lead + (max(stop - start, 0), d), dtype=np.float32)
    if stop <= start:
        return out
    for blk in range(start // POS_BLOCK, (stop - 1) // POS_BLOCK + 1):
        g = np.random.default_rng([seed, tensor, blk])
        vals = g.standard_normal(lead + (POS_BLOCK, d), dtype=np.float32)
        lo, hi = max(start, blk * POS_BLOCK), min(stop, (blk + 1) * POS_BLOCK)
        out[..., lo - start:hi - start, :] = vals[..., lo - blk * POS_BLOCK:hi - blk * POS_BLOCK, :]
    return out


def generate_numpy(w: Workload):
    """Host inputs: q [B,Hq,Lq,d] and full k, v [B,Hkv,n,d] over global positions (fp32 arrays).

    bf16 workloads hold bf16-representable values. Chunk ``c`` of the ring list
    is ``k[:, :, o:o+len]`` with ``(o, len) = w.chunks[c]``.
    """
    B, Hq, Hkv, d = w.batch, w.q_heads, w.kv_heads, w.head_dim
    st = w.pos_stride
    q = np.concatenate([_normal_positions(w.seed, 0, (B, Hq), o, o + st * (n - 1) + 1, d)[..., ::st, :]
                        for o, n in w.q_segments if n > 0],
                       axis=2) if any(n > 0 for _, n in w.q_segments) else np.zeros((B, Hq, 0, d), np.float32)
    if w.q_std != 1.0:
        q = q * np.float32(w.q_std)
    k = _normal_positions(w.seed, 1, (B, Hkv), 0, w.seq_len, d)
    v = _normal_positions(w.seed, 2, (B, Hkv), 0, w.seq_len, d)
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return q, k, v


def generate_torch(w: Workload, device="cpu"):
    """The same inputs as torch tensors (bf16 or fp32) on ``device``.

    Returns ``(q, k_full, v_full, key_chunks, value_chunks)``; the chunk lists
    are views into ``k_full``/``v_full`` in ring order, so no data is copied.
    With contiguous positions ``k_full`` is in global-position order. A striped
    share (``pos_stride`` P) keeps each chunk's keys contiguous, as the device
    owning that shard holds them: ``k_full`` is then the chunks' keys one
    after another in list order.
    """
    import torch

    q, k, v = generate_numpy(w)
    st = w.pos_stride
    if st != 1:
        k = np.concatenate([k[:, :, o:o + st * (n - 1) + 1:st] for o, n in w.chunks if n > 0], axis=2)
        v = np.concatenate([v[:, :, o:o + st * (n - 1) + 1:st] for o, n in w.chunks if n > 0], axis=2)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    tq = torch.from_numpy(q).to(device=device).to(tdt)
    tk = torch.from_numpy(np.ascontiguousarray(k)).to(device=device).to(tdt)
    tv = torch.from_numpy(np.ascontiguousarray(v)).to(device=device).to(tdt)
    kc, vc = chunk_views(w, tk, tv)
    return tq, tk, tv, kc, vc


def chunk_views(w: Workload, k_full, v_full):
    """Views of ``w``'s chunks in buffers laid out as :func:`generate_torch` lays them out.

    Also valid for any :func:`resplit` of the workload the buffers were made
    for: contiguous shares are indexed by position, striped ones by the key's
    place in the concatenated list (which a re-split keeps).
    """
    if w.pos_stride == 1:
        return [k_full[:, :, o:o + n] for o, n in w.chunks], [v_full[:, :, o:o + n] for o, n in w.chunks]
    starts = np.cumsum([0] + [n for _, n in w.chunks])
    return ([k_full[:, :, int(a):int(a) + n] for a, (_, n) in zip(starts, w.chunks)],
            [v_full[:, :, int(a):int(a) + n] for a, (_, n) in zip(starts, w.chunks)])


# ---------------------------------------------------------------------------
# bookkeeping used by the benchmark and by sampled checks


def q_positions(w: Workload) -> np.ndarray:
    parts = [o + w.pos_stride * np.arange(n, dtype=np.int64) for o, n in w.q_segments]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def k_positions(w: Workload) -> np.ndarray:
    """Global position of every key, in list (ring) order."""
    parts = [o + w.pos_stride * np.arange(n, dtype=np.int64) for o, n in w.chunks]
    return np.concatenate(parts) if parts else np.zeros(0, np.int64)


def unmasked_pairs_per_head(w: Workload) -> int:
    """Number of (query, key) pairs the mask allows, per query head and batch entry."""
    if not w.causal:
        return w.lq * w.lk
    kpos = np.sort(k_positions(w))
    return int(np.searchsorted(kpos, q_positions(w), side="right").sum())


def counted_flops(w: Workload) -> int:
    """4 * d flops per allowed (query, key) pair per query head: two matmuls of 2*d each."""
    return 4 * w.head_dim * w.q_heads * w.batch * unmasked_pairs_per_head(w)


def sample_rows(w: Workload, count: int, seed: int = 0, wg_rows: int = 256, tile: int = 64
                ) -> List[Tuple[int, int, int]]:
    """Stratified ``(b, h, row)`` sample of at least ``count`` rows (fewer only if the share has fewer).

    Strata, each row with a seeded random batch entry and head:
      * the first and last row of every query segment;
      * the rows on both sides of every wave (32 rows), half-workgroup (128) and workgroup (256) edge of
        the first and last workgroup, and of every workgroup edge in between;
      * every row of the first and of the last workgroup of query rows;
      * causal shares: the diagonal band, rows whose global position is within 2 of a multiple of ``tile``
        (the mask boundary then falls at the edge of a key tile);
      * seeded random rows up to ``count``.
    Duplicates are dropped, so every pair appears once.
    """
    g = np.random.default_rng([seed, 991])
    lq = w.lq
    special = []
    starts = np.cumsum([0] + [n for _, n in w.q_segments])
    for s0, s1 in zip(starts[:-1], starts[1:]):
        if s1 > s0:
            special += [int(s0), int(s1) - 1]
    for base in sorted({0, max(0, (lq - 1) // wg_rows * wg_rows)}):
        for e in (32, 64, 96, 128, 160, 192, 224, 256):
            special += [base + e - 1, base + e]
    for t in range(wg_rows, lq, wg_rows):
        special += [t - 1, t]
    last_wg = max(0, (lq - 1) // wg_rows * wg_rows)
    special += list(range(0, min(wg_rows, lq))) + list(range(last_wg, lq))
    if w.causal:
        qpos = q_positions(w)
        band = np.nonzero(np.isin(qpos % tile, [0, 1, tile - 2, tile - 1]))[0]
        special += [int(x) for x in band]
    seen = set()
    picks = []

    def add(r):
        key = (int(g.integers(w.batch)), int(g.integers(w.q_heads)), int(r))
        if 0 <= r < lq and key not in seen:
            seen.add(key)
            picks.append(key)

    for r in special:
        add(r)
    tries = 0
    while len(picks) < count and tries < 50 * count:
        add(int(g.integers(lq)))
        tries += 1
    return picks
