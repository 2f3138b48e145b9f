"""Pins of the fp64 gradient oracle (CPU only).

The gradients written out from the chain rule in ``oracle.backward`` are
checked against things that do not share its formulas: central finite
differences of the forward oracle, torch autograd through SDPA in float64,
and closed forms ("Ring Attention: Distributed Reads with Online Softmax",
section "Backward must aggregate shared dependencies": check the distributed
operation against a single-device reference, gradients included).
"""

import importlib.util
import inspect

import numpy as np
import pytest

import oracle.backward as ob
from oracle import attention, attention_backward


def _rand(shape, seed, s=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * s


def _loss(q, kc, vc, do, qpos, offs, causal, scale, strides=None):
    out = attention(q, kc, vc, q_positions=qpos, kv_offsets=offs, causal=causal, scale=scale,
                    kv_strides=strides)["out"]
    return float((out * do).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_finite_differences(causal):
    B, Hq, Hkv, Lq, d = 1, 2, 1, 4, 3
    lens, offs = [3, 2], [2, 0]  # list order is not position order
    q = _rand((B, Hq, Lq, d), 1)
    k = _rand((B, Hkv, sum(lens), d), 2, 1.5)
    v = _rand((B, Hkv, sum(lens), d), 3)
    do = _rand((B, Hq, Lq, d), 4)
    qpos = np.array([0, 1, 3, 4])
    scale = 0.7
    cut = lens[0]

    def chunks(kk, vv):
        return [kk[:, :, :cut], kk[:, :, cut:]], [vv[:, :, :cut], vv[:, :, cut:]]

    kc, vc = chunks(k, v)
    g = attention_backward(q, kc, vc, do, qpos, offs, causal=causal, scale=scale)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            key = name[1]
            args_p[key], args_m[key] = xp, xm
            kp, vp = chunks(args_p["k"], args_p["v"])
            km, vm = chunks(args_m["k"], args_m["v"])
            num[idx] = (_loss(args_p["q"], kp, vp, do, qpos, offs, causal, scale)
                        - _loss(args_m["q"], km, vm, do, qpos, offs, causal, scale)) / (2 * eps)
        assert np.max(np.abs(num - g[name])) <= 1e-7, name


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_torch_autograd_float64(causal):
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, Lq, n, d = 2, 4, 2, 6, 11, 8
    q = _rand((B, Hq, Lq, d), 11)
    k = _rand((B, Hkv, n, d), 12)
    v = _rand((B, Hkv, n, d), 13)
    do = _rand((B, Hq, Lq, d), 14)
    qpos = np.arange(5, 11)
    g = attention_backward(q, [k[:, :, :4], k[:, :, 4:]], [v[:, :, :4], v[:, :, 4:]], do, qpos, [0, 4],
                           causal=causal)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    mask = torch.from_numpy(np.arange(n)[None, :] <= qpos[:, None]) if causal else None
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk.repeat_interleave(Hq // Hkv, 1),
                                                           tv.repeat_interleave(Hq // Hkv, 1), attn_mask=mask)
    out.backward(torch.from_numpy(do))
    assert np.max(np.abs(g["out"] - out.detach().numpy())) <= 1e-12
    assert np.max(np.abs(g["dq"] - tq.grad.numpy())) <= 1e-12
    assert np.max(np.abs(g["dk"] - tk.grad.numpy())) <= 1e-12
    assert np.max(np.abs(g["dv"] - tv.grad.numpy())) <= 1e-12


def test_striped_gradients_match_whole_sequence_autograd():
    torch = pytest.importorskip("torch")
    P, r, n, H, d = 4, 2, 16, 1, 4
    q = _rand((1, H, n, d), 21)
    k = _rand((1, H, n, d), 22)
    v = _rand((1, H, n, d), 23)
    do = _rand((1, H, n, d), 24)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    # only device r's query rows carry a gradient: the share's own contribution
    mask_rows = np.zeros((1, H, n, d))
    mask_rows[:, :, r::P] = 1
    out.backward(torch.from_numpy(do * mask_rows))
    order = [(r - s) % P for s in range(P)]
    g = attention_backward(q[:, :, r::P], [k[:, :, j::P] for j in order], [v[:, :, j::P] for j in order],
                           do[:, :, r::P], r + P * np.arange(n // P), order, causal=True, kv_strides=[P] * P)
    assert np.max(np.abs(g["dq"] - tq.grad.numpy()[:, :, r::P])) <= 1e-12
    # dk of the concatenated list, shard j's keys are positions j, j+P, ...
    dk_ref = np.concatenate([tk.grad.numpy()[:, :, j::P] for j in order], axis=2)
    dv_ref = np.concatenate([tv.grad.numpy()[:, :, j::P] for j in order], axis=2)
    assert np.max(np.abs(g["dk"] - dk_ref)) <= 1e-12
    assert np.max(np.abs(g["dv"] - dv_ref)) <= 1e-12


def test_closed_forms():
    d = 5
    q = _rand((1, 1, 3, d), 31)
    k = _rand((1, 1, 6, d), 32)
    v = _rand((1, 1, 6, d), 33)
    do = _rand((1, 1, 3, d), 34)
    # zero upstream gradient: zero gradients
    g = attention_backward(q, [k], [v], np.zeros_like(do))
    assert all(np.all(g[x] == 0) for x in ("dq", "dk", "dv"))
    # a row whose only visible key is j: its weight is exactly 1, so it moves only dv_j (by dO)
    g = attention_backward(q[:, :, :1], [k], [v], do[:, :, :1], [0], [0], causal=True)
    assert np.max(np.abs(g["dq"])) == 0.0
    assert np.max(np.abs(g["dk"])) == 0.0
    assert np.max(np.abs(g["dv"][0, 0, 0] - do[0, 0, 0])) <= 1e-15
    assert np.all(g["dv"][0, 0, 1:] == 0)
    # a row with no visible key contributes nothing
    g = attention_backward(q[:, :, :1], [k], [v], do[:, :, :1], [0], [10], causal=True)
    assert all(np.all(g[x] == 0) for x in ("dq", "dk", "dv"))
    # dv sums the softmax weights times dO: its column sums equal sum_i dO_i (weights sum to 1)
    g = attention_backward(q, [k], [v], do)
    assert np.max(np.abs(g["dv"].sum(axis=2) - do.sum(axis=2))) <= 1e-12
    # shifting every key by the same vector c adds scale*<q, c> to a row's scores: softmax and dq do
    # not change, and sum_j dk_j = scale * sum_i (sum_j ds_ij) q_i = 0 since each row of ds sums to 0
    assert np.max(np.abs(g["dk"].sum(axis=2))) <= 1e-12


# ---------------------------------------------------------------------------
# planted mistakes: each plausible slip in the gradient oracle's source must break the finite-difference
# pin (GQA with two query heads on one key/value head, causal, chunks out of position order)

MUTANTS = [
    ("no softmax-Jacobian correction", "(dp - (p * dp).sum(axis=1, keepdims=True))", "dp"),
    ("dq without the scale", "dq[b, h, r0:r1] = scale * (ds @ k[b, hk])", "dq[b, h, r0:r1] = ds @ k[b, hk]"),
    ("dk from p instead of ds", "scale * (ds.T @ q[b, h, r0:r1])", "scale * (p.T @ q[b, h, r0:r1])"),
    ("dv from q instead of dout", "dv[b, hk] += p.T @ g", "dv[b, hk] += p.T @ q[b, h, r0:r1]"),
    ("strict causal boundary", "kpos[None, :] <= qpos[r0:r1, None]", "kpos[None, :] < qpos[r0:r1, None]"),
    ("GQA group overwrites dk", "dk[b, hk] += scale", "dk[b, hk] = scale"),
    ("dp against k instead of v", "dp = g @ v[b, hk].T", "dp = g @ k[b, hk].T"),
]


def _fd_error(fn):
    B, Hq, Hkv, Lq, d = 1, 2, 1, 4, 3
    lens, offs = [3, 2], [2, 0]
    q = _rand((B, Hq, Lq, d), 1)
    k = _rand((B, Hkv, sum(lens), d), 2, 1.5)
    v = _rand((B, Hkv, sum(lens), d), 3)
    do = _rand((B, Hq, Lq, d), 4)
    qpos = np.array([0, 1, 3, 4])
    cut = lens[0]

    def chunks(kk, vv):
        return [kk[:, :, :cut], kk[:, :, cut:]], [vv[:, :, :cut], vv[:, :, cut:]]

    kc, vc = chunks(k, v)
    g = fn(q, kc, vc, do, qpos, offs, causal=True, scale=0.7)
    worst, eps = 0.0, 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        for idx in np.ndindex(x.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = dict(args), dict(args)
            ap[name[1]], am[name[1]] = xp, xm
            lp = _loss(ap["q"], *chunks(ap["k"], ap["v"]), do, qpos, offs, True, 0.7)
            lm = _loss(am["q"], *chunks(am["k"], am["v"]), do, qpos, offs, True, 0.7)
            worst = max(worst, abs((lp - lm) / (2 * eps) - g[name][idx]))
    return worst


def _mutated(old, new):
    src = inspect.getsource(ob)
    assert src.count(old) == 1, old
    spec = importlib.util.spec_from_loader("oracle._backward_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "oracle_backward_mutant", "exec"), mod.__dict__)
    return mod.attention_backward


def test_finite_difference_pin_accepts_the_oracle():
    assert _fd_error(ob.attention_backward) <= 1e-7


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_finite_difference_pin_catches_planted_mistake(name, old, new):
    assert _fd_error(_mutated(old, new)) > 1e-4, name
