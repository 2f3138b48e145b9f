"""The allocation-free ring call against the workspace ring call (needs an MI355X).

``ra_ring_attention_noalloc`` keeps its descriptor tables and key-range
partials in the library's static per-GPU array instead of a caller
workspace; it runs the same kernels with the same key-range cut, so its
output and lse must be bit-identical to ``ra_ring_attention``'s (stricter
than the oracle tolerances the kernels are held to). Calls in a row with
different shares check that nothing left in the shared array by one call
leaks into the next. Every call goes through the C ABI.
"""

import pytest
import torch

import ring_attention_chunk_amd as ra
from ring_attention_chunk_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _both(w, q, kc, vc):
    ref_out, ref_lse = ra.ring_attention(q, kc, vc, w.q_runs, w.kv_offsets, causal=w.causal, return_lse=True,
                                         kv_position_strides=w.kv_strides)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    got = ra.api.ring_attention_noalloc(q, kc, vc, w.q_runs, w.kv_offsets, causal=w.causal,
                                        kv_position_strides=w.kv_strides, out=out, lse=lse)
    torch.cuda.synchronize()
    assert got[0] is out and got[1] is lse
    return ref_out, ref_lse, out, lse


def test_noalloc_matches_the_workspace_call_on_calls_in_a_row():
    # 1: the d = 64 share: 8 heads x 4096 queries x 32768 keys, key range cut in two, so the partials
    #    (about 17 MB) live in the static array next to the tables
    big = wl.config(1)
    # 2: a smaller causal GQA share with a ragged tail and chunks cut inside tiles (other tables, no cut)
    small = wl.custom("noalloc_small", "bf16", 1, 4, 2, 128, [(300, 200)], [(0, 70), (70, 250), (320, 180)],
                      True, seed=12)
    # 3: a short share against many keys: cut into more ranges than the first
    cut = wl.custom("noalloc_cut", "bf16", 1, 2, 1, 64, [(0, 256)], [(0, 5000), (5000, 3192)], False, seed=13)
    for w in (big, small, cut, big):
        _say(f"noalloc {w.name}")
        q, k, v, kc, vc = wl.generate_torch(w, DEV)
        ref_out, ref_lse, out, lse = _both(w, q, kc, vc)
        assert torch.equal(out, ref_out)
        assert torch.equal(lse, ref_lse)


def test_noalloc_refuses_beyond_its_scratch():
    _say("noalloc refusal")
    q = torch.zeros(1, 8, 2048, 128, device=DEV, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 1 << 20, 128, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(ra.RingAttentionError, match="static scratch"):
        ra.api.ring_attention_noalloc(q, [k], [k])
