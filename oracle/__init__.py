"""Test infrastructure: the plain fp64 CPU oracle for blockwise ring attention.

Nothing in the product path may import this package. Only the test suite,
the smoke check in ``__graft_entry__`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code with the HIP library: no kernels, no
headers, no helpers, no table generators.

Two independent statements of what the method computes live here:

* :mod:`oracle.direct` -- the plain definition. The ring method must give
  the same result as ordinary softmax attention over the whole concatenated
  key/value sequence, for any split into chunks (exercise page
  "systems-distributed-ring-attention-online-softmax", problem statement), so
  the oracle for ``ring_attention`` is that ordinary attention, with the
  causal mask taken from global positions ("Ring Attention: Distributed Reads
  with Online Softmax", section "Causal masks depend on global positions").
* :mod:`oracle.backward` -- the gradients of that ordinary attention (dQ,
  and dK, dV summed per key over every query that sees it), written out from
  the chain rule ("Ring Attention: Distributed Reads with Online Softmax",
  section "Backward must aggregate shared dependencies"). It is pinned by
  central finite differences of :mod:`oracle.direct` and by torch autograd.
* :mod:`oracle.block_sparse` -- ordinary attention restricted to the keys a
  block mask over global positions allows ("Ring Attention: Distributed Reads
  with Online Softmax", section "What is preserved, what is distributed?": the
  method composes with sparse patterns), optionally combined with the causal
  mask. It expands the block mask to the full boolean matrix and evaluates
  masked softmax attention; pinned by ``tests/test_oracle_block_sparse.py``.
* :mod:`oracle.online_softmax` -- the exercise's three functions written out
  in fp64 (chunk statistics, the rescale-to-shared-max merge, and the fold
  over chunks followed by one normalisation). It is the reference for the
  standalone ``attention_chunk_stats`` and ``merge_chunk_stats`` calls and is
  itself pinned against :mod:`oracle.direct` by split-invariance tests.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against the pages' worked example, closed forms, brute force on tiny inputs
and a library special case. ``attention_rows`` (the same definition on
selected rows, the reference of the full-size GPU checks) is pinned row for
row against ``attention`` on GQA, causal, paired early/late and striped
shares, with planted bookkeeping mistakes that the pin must catch
(``tests/test_oracle_rows.py``). No function is "parity unpinned".
"""

from .backward import attention_backward
from .block_sparse import attention_block_sparse, expand_block_mask
from .direct import attention, attention_rows, key_positions, query_positions
from .online_softmax import chunk_stats, merge_chunk_stats, ring_attention_fold, normalize

__all__ = [
    "attention",
    "attention_backward",
    "attention_block_sparse",
    "expand_block_mask",
    "attention_rows",
    "key_positions",
    "query_positions",
    "chunk_stats",
    "merge_chunk_stats",
    "ring_attention_fold",
    "normalize",
]
