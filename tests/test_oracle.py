"""Pins of the fp64 CPU oracle to things other than itself (CPU only).

Each test ties an oracle function to the mathematics: central finite
differences of the forward loss, brute-force scalar loops, closed forms,
invariants of the softmax gradient, an independent library routine (torch's
attention and autograd in float64), and hand-derived worked examples stored
under tests/golden/.  A planted-mistake test at the end checks that the pins
catch the plausible slips (dropped term, wrong sign, transposed operand).
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))


def rand(rng, *shape):
    return rng.standard_normal(shape)


# --------------------------------------------------------------------------
# forward: brute force, library routine, worked examples
# --------------------------------------------------------------------------

def brute_head_forward(q, k, v, scale, causal):
    """Scalar loops with math.exp: the definition, no vectorisation."""
    sq, sk, d = len(q), len(k), len(q[0])
    o, lse = [], []
    for i in range(sq):
        vis = [j for j in range(sk) if (not causal) or j <= i + (sk - sq)]
        if not vis:
            o.append([0.0] * d)
            lse.append(-math.inf)
            continue
        s = {j: scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in vis}
        m = max(s.values())
        z = sum(math.exp(s[j] - m) for j in vis)
        lse.append(m + math.log(z))
        o.append([sum(math.exp(s[j] - lse[-1]) * v[j][t] for j in vis) for t in range(d)])
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("sq,sk,causal", [(5, 5, False), (5, 5, True), (4, 6, True), (6, 4, True), (3, 7, False)])
def test_forward_matches_scalar_loops(sq, sk, causal):
    rng = np.random.default_rng(10 + sq * 7 + sk)
    q, k, v = rand(rng, sq, 3), rand(rng, sk, 3), rand(rng, sk, 3)
    o, lse = A.head_forward(q, k, v, 0.7, causal)
    bo, blse = brute_head_forward(q.tolist(), k.tolist(), v.tolist(), 0.7, causal)
    assert np.array_equal(np.isfinite(lse), np.isfinite(blse))
    fin = np.isfinite(blse)
    assert np.max(np.abs(lse[fin] - blse[fin])) <= 1e-12
    assert np.max(np.abs(o - bo)) <= 1e-12


def _torch_mask(sq, sk, causal):
    import torch
    i = torch.arange(sq)[:, None]
    j = torch.arange(sk)[None, :]
    return (j <= i + (sk - sq)) if causal else torch.ones(sq, sk, dtype=torch.bool)


@pytest.mark.parametrize("sq,sk,causal", [(33, 33, False), (33, 33, True), (20, 47, True), (47, 20, True)])
def test_forward_matches_torch_sdpa_float64(sq, sk, causal):
    """torch.nn.functional.scaled_dot_product_attention (CPU, float64) is an
    independent implementation of the same definition."""
    import torch
    rng = np.random.default_rng(3)
    q, k, v = rand(rng, 2, 3, sq, 8), rand(rng, 2, 3, sk, 8), rand(rng, 2, 3, sk, 8)
    mask = _torch_mask(sq, sk, causal)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask, scale=0.4).numpy()
    rows = mask.any(dim=1).numpy()
    for b in range(2):
        for h in range(3):
            o, _ = A.head_forward(q[b, h], k[b, h], v[b, h], 0.4, causal)
            assert np.max(np.abs(o[rows] - ref[b, h][rows])) <= 1e-12
            assert np.all(o[~rows] == 0.0)


def test_golden_worked_examples():
    data = json.load(open(GOLDEN))
    for ex in data["examples"]:
        q, k, v, do = (np.array(ex[n], np.float64) for n in ("q", "k", "v", "do"))
        o, lse = A.head_forward(q, k, v, ex["scale"], ex["causal"])
        want_lse = np.array([-np.inf if x is None else x for x in ex["lse"]])
        assert np.array_equal(np.isfinite(lse), np.isfinite(want_lse)), ex["name"]
        fin = np.isfinite(want_lse)
        assert np.max(np.abs(lse[fin] - want_lse[fin])) <= 1e-14, ex["name"]
        assert np.max(np.abs(o - np.array(ex["o"]))) <= 1e-14, ex["name"]
        dq, dk, dv = A.head_backward(q, k, v, o, do, lse, ex["scale"], ex["causal"])
        for got, key in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            assert np.max(np.abs(got - np.array(ex[key]))) <= 1e-14, (ex["name"], key)


# --------------------------------------------------------------------------
# backward: central finite differences of L = sum(dO * O)
# --------------------------------------------------------------------------

def _fd_case(q, k, v, do, scale, causal, cu_q=None, cu_k=None, window=None):
    """Analytic gradients vs central differences, h = 1e-5, every entry."""
    o, lse = oracle.forward(q, k, v, scale, causal, cu_q, cu_k, window=window)
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, scale, causal, cu_q, cu_k, window=window)

    def loss(qq, kk, vv):
        oo, _ = oracle.forward(qq, kk, vv, scale, causal, cu_q, cu_k, window=window)
        return float(np.sum(do * oo))

    h = 1e-5
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos], args_m[pos] = xp, xm
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = rel_err(g, fd)
        assert err <= 1e-6, (name, err)
    return dq, dk, dv


@pytest.mark.parametrize("sq,sk,causal,scale", [
    (5, 5, False, 1 / math.sqrt(3)),
    (5, 5, True, 1 / math.sqrt(3)),
    (4, 6, True, 1 / math.sqrt(3)),
    (6, 4, True, 1 / math.sqrt(3)),     # rows 0 and 1 see no key
    (5, 5, True, 0.3),
])
def test_backward_finite_differences_dense(sq, sk, causal, scale):
    rng = np.random.default_rng(100 + sq * 10 + sk)
    q, k, v = rand(rng, 1, sq, 1, 3), rand(rng, 1, sk, 1, 3), rand(rng, 1, sk, 1, 3)
    do = rand(rng, 1, sq, 1, 3)
    _fd_case(q, k, v, do, scale, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences_gqa(causal):
    rng = np.random.default_rng(7)
    q, k, v = rand(rng, 1, 5, 4, 3), rand(rng, 1, 5, 2, 3), rand(rng, 1, 5, 2, 3)
    do = rand(rng, 1, 5, 4, 3)
    _fd_case(q, k, v, do, 0.5, causal)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences_varlen(causal):
    rng = np.random.default_rng(8)
    lens = [1, 4, 7]
    cu = np.array([0, 1, 5, 12], np.int32)
    q, k, v = rand(rng, 12, 2, 3), rand(rng, 12, 1, 3), rand(rng, 12, 1, 3)
    do = rand(rng, 12, 2, 3)
    assert sum(lens) == 12
    _fd_case(q, k, v, do, 0.6, causal, cu, cu)


# --------------------------------------------------------------------------
# local (sliding-window) masks
# --------------------------------------------------------------------------

def _window_mask_loops(sq, sk, causal, left, right):
    """The visibility rule written as scalar loops (independent of the oracle's
    vectorised form)."""
    off = sk - sq
    m = np.zeros((sq, sk), bool)
    for i in range(sq):
        for j in range(sk):
            ok = True
            if causal and j > i + off:
                ok = False
            if left >= 0 and j < i + off - left:
                ok = False
            if right >= 0 and j > i + off + right:
                ok = False
            m[i, j] = ok
    return m


@pytest.mark.parametrize("sq,sk", [(9, 9), (6, 11), (11, 6)])
@pytest.mark.parametrize("causal,left,right", [(False, 3, 2), (True, 2, -1), (False, -1, 0), (False, 0, 0),
                                               (True, 4, 1), (False, 1, -1), (False, 40, 40)])
def test_window_visibility_and_special_cases(sq, sk, causal, left, right):
    want = _window_mask_loops(sq, sk, causal, left, right)
    assert np.array_equal(A.visible(sq, sk, causal, (left, right)), want)
    # no window == (-1, -1); causal == the window (-1, 0); a window wider
    # than the keys == no window
    assert np.array_equal(A.visible(sq, sk, causal, (-1, -1)), A.visible(sq, sk, causal))
    assert np.array_equal(A.visible(sq, sk, False, (-1, 0)), A.visible(sq, sk, True))
    assert np.array_equal(A.visible(sq, sk, causal, (sq + sk, sq + sk)), A.visible(sq, sk, causal))


def test_window_zero_width_closed_form():
    """window (0, 0): row i sees only key i + off, so P is one-hot: O_i = V_j,
    dV_j = dO_i, and dQ = dK = 0 (dS = P (dO.V_j - dO.O_i) = 0)."""
    rng = np.random.default_rng(31)
    sq, sk = 7, 10
    q, k, v, do = rand(rng, sq, 5), rand(rng, sk, 5), rand(rng, sk, 5), rand(rng, sq, 5)
    o, lse = A.head_forward(q, k, v, 0.7, False, window=(0, 0))
    off = sk - sq
    assert np.max(np.abs(o - v[off:off + sq])) <= 1e-14
    assert np.max(np.abs(lse - 0.7 * np.sum(q * k[off:off + sq], axis=1))) <= 1e-13
    dq, dk, dv = A.head_backward(q, k, v, o, do, lse, 0.7, False, window=(0, 0))
    assert np.max(np.abs(dq)) <= 1e-13 and np.max(np.abs(dk)) <= 1e-13
    want_dv = np.zeros_like(v)
    want_dv[off:off + sq] = do
    assert np.max(np.abs(dv - want_dv)) <= 1e-14


@pytest.mark.parametrize("causal,window", [(False, (2, 1)), (True, (3, -1)), (False, (0, 4))])
def test_backward_finite_differences_window(causal, window):
    rng = np.random.default_rng(41)
    q, k, v = rand(rng, 1, 9, 2, 3), rand(rng, 1, 7, 1, 3), rand(rng, 1, 7, 1, 3)
    do = rand(rng, 1, 9, 2, 3)
    _fd_case(q, k, v, do, 0.45, causal, window=window)


def test_window_varlen_equals_per_sequence():
    rng = np.random.default_rng(42)
    lens = [5, 1, 12]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v, do = rand(rng, cu[-1], 2, 4), rand(rng, cu[-1], 2, 4), rand(rng, cu[-1], 2, 4), rand(rng, cu[-1], 2, 4)
    o, lse = oracle.forward(q, k, v, 0.5, True, cu, cu, window=(3, -1))
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, 0.5, True, cu, cu, window=(3, -1))
    for bi in range(3):
        sl = slice(cu[bi], cu[bi + 1])
        od, lsed = oracle.forward(q[None, sl], k[None, sl], v[None, sl], 0.5, True, window=(3, -1))
        assert np.max(np.abs(o[sl] - od[0])) <= 1e-12
        dd = oracle.backward(q[None, sl], k[None, sl], v[None, sl], od, do[None, sl], lsed, 0.5, True, window=(3, -1))
        for a_, b_ in zip((dq, dk, dv), dd):
            assert np.max(np.abs(a_[sl] - b_[0])) <= 1e-12


# --------------------------------------------------------------------------
# ALiBi: -slope * |i + off - j| added to the scaled logits
# --------------------------------------------------------------------------

def brute_alibi_forward(q, k, v, scale, causal, slope):
    """Scalar loops: logit_ij = scale q_i.k_j - slope |i + (sk - sq) - j| over
    the visible keys, softmax with math.exp."""
    sq, sk, d = len(q), len(k), len(q[0])
    o, lse = [], []
    for i in range(sq):
        vis = [j for j in range(sk) if (not causal) or j <= i + (sk - sq)]
        if not vis:
            o.append([0.0] * d)
            lse.append(-math.inf)
            continue
        s = {j: scale * sum(q[i][t] * k[j][t] for t in range(d)) - slope * abs(i + (sk - sq) - j) for j in vis}
        m = max(s.values())
        lse.append(m + math.log(sum(math.exp(s[j] - m) for j in vis)))
        o.append([sum(math.exp(s[j] - lse[-1]) * v[j][t] for j in vis) for t in range(d)])
    return np.array(o), np.array(lse)


ALIBI_LOOP_CASES = [(5, 5, False, 0.5), (5, 5, True, 0.25), (4, 7, True, 1.0), (7, 4, True, 0.125),
                    (3, 6, False, 2.0), (6, 3, False, 0.75)]


def _alibi_scalar_loop_pin(sq, sk, causal, slope):
    rng = np.random.default_rng(40 + sq * 7 + sk)
    q, k, v = rand(rng, sq, 3), rand(rng, sk, 3), rand(rng, sk, 3)
    o, lse = A.head_forward(q, k, v, 0.7, causal, alibi=slope)
    bo, blse = brute_alibi_forward(q.tolist(), k.tolist(), v.tolist(), 0.7, causal, slope)
    fin = np.isfinite(blse)
    return (np.array_equal(np.isfinite(lse), fin) and np.max(np.abs(lse[fin] - blse[fin])) <= 1e-12
            and np.max(np.abs(o - bo)) <= 1e-12)


@pytest.mark.parametrize("sq,sk,causal,slope", ALIBI_LOOP_CASES)
def test_alibi_forward_matches_scalar_loops(sq, sk, causal, slope):
    assert _alibi_scalar_loop_pin(sq, sk, causal, slope)


def _alibi_zero_query_pin(sq, sk, causal, slope):
    """Q = 0: the logits are the bias alone, so P_ij = r^|c - j| / Z_i with
    r = exp(-slope), c = i + off the diagonal key, and Z_i the sum of two
    geometric series (keys left and right of c).  dK = s dS^T Q = 0."""
    rng = np.random.default_rng(5)
    q = np.zeros((sq, 4))
    k, v, do = rand(rng, sk, 4), rand(rng, sk, 4), rand(rng, sq, 4)
    o, lse = A.head_forward(q, k, v, 0.9, causal, alibi=slope)
    r = math.exp(-slope)
    ok = True
    for i in range(sq):
        c = i + sk - sq
        lo_key, hi_key = 0, (min(c, sk - 1) if causal else sk - 1)
        if hi_key < lo_key:
            ok &= lse[i] == -math.inf and np.all(o[i] == 0)
            continue
        def run(d0, d1):   # sum of r^d for d = d0 .. d1
            return 0.0 if d1 < d0 else (r ** d0 - r ** (d1 + 1)) / (1 - r)
        # keys at or left of c have distances c - j, those right of it j - c
        l0, l1 = lo_key, min(hi_key, c)
        r0, r1 = max(lo_key, c + 1), hi_key
        z = run(c - l1, c - l0) + run(r0 - c, r1 - c)
        ok &= abs(lse[i] - math.log(z)) <= 1e-12
        w = np.array([r ** abs(c - j) / z if lo_key <= j <= hi_key else 0.0 for j in range(sk)])
        ok &= np.max(np.abs(o[i] - w @ v)) <= 1e-12
    dq, dk, dv = A.head_backward(q, k, v, o, do, lse, 0.9, causal, alibi=slope)
    ok &= np.all(dk == 0.0)
    return bool(ok)


@pytest.mark.parametrize("sq,sk,causal,slope", [(6, 6, False, 0.3), (6, 6, True, 0.7), (4, 9, False, 1.5),
                                                (9, 4, True, 0.2), (9, 4, False, 0.9)])
def test_alibi_zero_query_closed_form(sq, sk, causal, slope):
    assert _alibi_zero_query_pin(sq, sk, causal, slope)


def _alibi_augmented_pin(sq, sk, slope, right_side):
    """On one side of the diagonal |i + off - j| is linear in j, so the bias
    splits into a row constant (cancels in the softmax, shifts LSE) and a
    column term that one extra head dimension carries: [q, 1] . [k, +-slope
    j / s].  The plain path (no ALiBi code) then gives the same O, dQ, dK,
    dV, and LSE shifted by -+slope (i + off).  Left side: causal; right side:
    the window (0, -1)."""
    rng = np.random.default_rng(8)
    d, sc = 5, 0.6
    q, k, v, do = rand(rng, sq, d), rand(rng, sk, d), rand(rng, sk, d), rand(rng, sq, d)
    causal, window = (False, (0, -1)) if right_side else (True, None)
    sign = -1.0 if right_side else 1.0
    jcol = sign * slope * np.arange(sk)[:, None] / sc
    qa = np.concatenate([q, np.ones((sq, 1))], axis=1)
    ka = np.concatenate([k, jcol], axis=1)
    o, lse = A.head_forward(q, k, v, sc, causal, window=window, alibi=slope)
    oa, lsea = A.head_forward(qa, ka, v, sc, causal, window=window)
    c = np.arange(sq) + (sk - sq)
    fin = np.isfinite(lsea)
    ok = np.array_equal(np.isfinite(lse), fin)
    ok &= np.max(np.abs(o - oa)) <= 1e-12
    ok &= np.max(np.abs(lse[fin] - (lsea[fin] - sign * slope * c[fin])), initial=0) <= 1e-11
    dq, dk, dv = A.head_backward(q, k, v, o, do, lse, sc, causal, window=window, alibi=slope)
    dqa, dka, dva = A.head_backward(qa, ka, v, oa, do, lsea, sc, causal, window=window)
    ok &= rel_err(dq, dqa[:, :d]) <= 1e-12 and rel_err(dk, dka[:, :d]) <= 1e-12 and rel_err(dv, dva) <= 1e-12
    return bool(ok)


@pytest.mark.parametrize("sq,sk,slope,right_side", [(9, 9, 0.4, False), (6, 11, 1.1, False), (11, 6, 0.3, False),
                                                    (9, 9, 0.4, True), (6, 11, 0.8, True), (11, 6, 0.5, True)])
def test_alibi_augmented_dimension_equivalence(sq, sk, slope, right_side):
    assert _alibi_augmented_pin(sq, sk, slope, right_side)


def test_alibi_zero_slope_is_plain_attention():
    rng = np.random.default_rng(6)
    q, k, v, do = rand(rng, 7, 4), rand(rng, 9, 4), rand(rng, 9, 4), rand(rng, 7, 4)
    for causal in (False, True):
        o, lse = A.head_forward(q, k, v, 0.5, causal)
        oz, lsez = A.head_forward(q, k, v, 0.5, causal, alibi=0.0)
        assert np.array_equal(o, oz) and np.array_equal(lse, lsez)
        g = A.head_backward(q, k, v, o, do, lse, 0.5, causal)
        gz = A.head_backward(q, k, v, o, do, lse, 0.5, causal, alibi=0.0)
        for a, b in zip(g, gz):
            assert np.array_equal(a, b)


def _fd_alibi(q, k, v, do, scale, causal, slopes, cu=None, window=None):
    o, lse = oracle.forward(q, k, v, scale, causal, cu, cu, window=window, alibi_slopes=slopes)
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, scale, causal, cu, cu, window=window, alibi_slopes=slopes)

    def loss(qq, kk, vv):
        return float(np.sum(do * oracle.forward(qq, kk, vv, scale, causal, cu, cu, window=window,
                                                alibi_slopes=slopes)[0]))

    h = 1e-5
    for pos, g in enumerate((dq, dk, dv)):
        base = [q, k, v]
        fd = np.zeros_like(base[pos])
        for idx in np.ndindex(fd.shape):
            xp, xm = base[pos].copy(), base[pos].copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(base), list(base)
            ap[pos], am[pos] = xp, xm
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        assert rel_err(g, fd) <= 1e-6


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (False, (3, 2))])
def test_alibi_backward_finite_differences(causal, window):
    """Dense GQA (4 q-heads on 2 kv-heads, each q-head its own slope)."""
    rng = np.random.default_rng(21)
    q, k, v, do = rand(rng, 1, 6, 4, 3), rand(rng, 1, 7, 2, 3), rand(rng, 1, 7, 2, 3), rand(rng, 1, 6, 4, 3)
    _fd_alibi(q, k, v, do, 0.5, causal, np.array([0.5, 0.25, 1.0, 0.125]), window=window)


def test_alibi_backward_finite_differences_varlen():
    rng = np.random.default_rng(22)
    cu = np.array([0, 3, 8], np.int32)
    q, k, v, do = rand(rng, 8, 2, 3), rand(rng, 8, 2, 3), rand(rng, 8, 2, 3), rand(rng, 8, 2, 3)
    _fd_alibi(q, k, v, do, 0.6, True, np.array([0.3, 0.9]), cu=cu)


@pytest.mark.parametrize("sq,sk,causal", [(30, 30, False), (20, 37, True), (37, 20, False)])
def test_alibi_backward_matches_torch_autograd_float64(sq, sk, causal):
    """The bias as an explicit float matrix added to the logits in torch float64 autograd."""
    import torch
    rng = np.random.default_rng(13)
    slope = 0.37
    q, k, v, do = rand(rng, sq, 8), rand(rng, sk, 8), rand(rng, sk, 8), rand(rng, sq, 8)
    i = torch.arange(sq, dtype=torch.float64)[:, None]
    j = torch.arange(sk, dtype=torch.float64)[None, :]
    bias = -slope * torch.abs(i + (sk - sq) - j)
    mask = (j <= i + (sk - sq)) if causal else torch.ones(sq, sk, dtype=torch.bool)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = (0.3 * tq @ tk.T + bias).masked_fill(~mask, float("-inf"))
    rows = mask.any(dim=1)
    pr = torch.where(rows[:, None], torch.softmax(torch.where(rows[:, None], s, torch.zeros_like(s)), dim=-1),
                     torch.zeros_like(s))
    out = pr @ tv
    out.backward(torch.from_numpy(do))
    o, lse = A.head_forward(q, k, v, 0.3, causal, alibi=slope)
    assert np.max(np.abs(o - out.detach().numpy())) <= 1e-12
    dq, dk, dv = A.head_backward(q, k, v, o, do, lse, 0.3, causal, alibi=slope)
    assert rel_err(dq, tq.grad.numpy()) <= 1e-12
    assert rel_err(dk, tk.grad.numpy()) <= 1e-12
    assert rel_err(dv, tv.grad.numpy()) <= 1e-12


def _alibi_sign_flipped(sq, sk, slope):
    i = np.arange(sq)[:, None]
    j = np.arange(sk)[None, :]
    return float(slope) * np.abs(i + (sk - sq) - j).astype(np.float64)


def _alibi_top_left(sq, sk, slope):
    i = np.arange(sq)[:, None]
    j = np.arange(sk)[None, :]
    return -float(slope) * np.abs(i - j).astype(np.float64)


def _alibi_no_abs(sq, sk, slope):
    i = np.arange(sq)[:, None]
    j = np.arange(sk)[None, :]
    return -float(slope) * (i + (sk - sq) - j).astype(np.float64)


def _alibi_transposed_distance(sq, sk, slope):
    i = np.arange(sq)[:, None]
    j = np.arange(sk)[None, :]
    return -float(slope) * np.abs(j + (sk - sq) - i).astype(np.float64)


@pytest.mark.parametrize("mutant", [_alibi_sign_flipped, _alibi_top_left, _alibi_no_abs, _alibi_transposed_distance],
                         ids=lambda f: f.__name__)
def test_planted_alibi_mistakes_are_caught(mutant, monkeypatch):
    """Each plausible slip in the bias fails at least one of the ALiBi pins."""
    monkeypatch.setattr(A, "alibi_bias", mutant)
    caught = not all(_alibi_scalar_loop_pin(*c) for c in ALIBI_LOOP_CASES)
    caught |= not _alibi_zero_query_pin(4, 9, False, 1.5)
    caught |= not _alibi_augmented_pin(6, 11, 1.1, False)
    caught |= not _alibi_augmented_pin(6, 11, 0.8, True)
    assert caught, mutant.__name__


# --------------------------------------------------------------------------
# elementwise bias: added to the scaled logits; dBias = dS
# --------------------------------------------------------------------------

def brute_bias_forward(q, k, v, scale, causal, bias):
    """Scalar loops: logit_ij = scale q_i.k_j + bias_ij over the visible keys."""
    sq, sk, d = len(q), len(k), len(q[0])
    o, lse = [], []
    for i in range(sq):
        vis = [j for j in range(sk) if (not causal) or j <= i + (sk - sq)]
        if not vis:
            o.append([0.0] * d)
            lse.append(-math.inf)
            continue
        s = {j: scale * sum(q[i][t] * k[j][t] for t in range(d)) + bias[i][j] for j in vis}
        m = max(s.values())
        lse.append(m + math.log(sum(math.exp(s[j] - m) for j in vis)))
        o.append([sum(math.exp(s[j] - lse[-1]) * v[j][t] for j in vis) for t in range(d)])
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("sq,sk,causal", [(5, 5, False), (4, 7, True), (7, 4, True), (3, 6, False)])
def test_bias_forward_matches_scalar_loops(sq, sk, causal):
    rng = np.random.default_rng(70 + sq * 7 + sk)
    q, k, v, bias = rand(rng, sq, 3), rand(rng, sk, 3), rand(rng, sk, 3), 2.0 * rand(rng, sq, sk)
    o, lse = A.head_forward(q, k, v, 0.7, causal, bias=bias)
    bo, blse = brute_bias_forward(q.tolist(), k.tolist(), v.tolist(), 0.7, causal, bias.tolist())
    fin = np.isfinite(blse)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.max(np.abs(lse[fin] - blse[fin])) <= 1e-12
    assert np.max(np.abs(o - bo)) <= 1e-12


def _fd_bias(q, k, v, do, bias, scale, causal, cu=None):
    """Every gradient, dBias included, against central differences of sum(dO * O)."""
    o, lse = oracle.forward(q, k, v, scale, causal, cu, cu, bias=bias)
    dq, dk, dv, db = oracle.backward(q, k, v, o, do, lse, scale, causal, cu, cu, bias=bias, want_dbias=True)

    def loss(qq, kk, vv, bb):
        return float(np.sum(do * oracle.forward(qq, kk, vv, scale, causal, cu, cu, bias=bb)[0]))

    h = 1e-5
    base = [q, k, v, bias]
    for pos, g in enumerate((dq, dk, dv, db)):
        fd = np.zeros_like(base[pos])
        for idx in np.ndindex(fd.shape):
            xp, xm = base[pos].copy(), base[pos].copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(base), list(base)
            ap[pos], am[pos] = xp, xm
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        # (bias entries outside a sequence's block take no part: both are zero)
        assert rel_err(g, fd) <= 1e-6, ("dq", "dk", "dv", "dbias")[pos]
    return db


@pytest.mark.parametrize("causal", [False, True])
def test_bias_backward_finite_differences(causal):
    """Dense GQA (4 q-heads on 2 kv-heads): dQ, dK, dV and dBias."""
    rng = np.random.default_rng(31)
    q, k, v, do = rand(rng, 1, 5, 4, 3), rand(rng, 1, 6, 2, 3), rand(rng, 1, 6, 2, 3), rand(rng, 1, 5, 4, 3)
    bias = rand(rng, 1, 4, 5, 6)
    _fd_bias(q, k, v, do, bias, 0.5, causal)


def test_bias_backward_finite_differences_varlen():
    rng = np.random.default_rng(32)
    cu = np.array([0, 2, 6], np.int32)
    q, k, v, do = rand(rng, 6, 2, 3), rand(rng, 6, 2, 3), rand(rng, 6, 2, 3), rand(rng, 6, 2, 3)
    bias = rand(rng, 2, 2, 4, 4)
    db = _fd_bias(q, k, v, do, bias, 0.6, True, cu)
    assert np.all(db[0, :, 2:, :] == 0) and np.all(db[0, :, :, 2:] == 0)   # outside sequence 0's 2 x 2 block


@pytest.mark.parametrize("sq,sk,causal", [(30, 30, False), (20, 37, True), (37, 20, False)])
def test_bias_backward_matches_torch_autograd_float64(sq, sk, causal):
    """The bias as a leaf tensor in torch float64 autograd: dQ, dK, dV and dBias."""
    import torch
    rng = np.random.default_rng(14)
    q, k, v, do, bias = (rand(rng, sq, 8), rand(rng, sk, 8), rand(rng, sk, 8), rand(rng, sq, 8),
                         rand(rng, sq, sk))
    i = torch.arange(sq)[:, None]
    j = torch.arange(sk)[None, :]
    mask = (j <= i + (sk - sq)) if causal else torch.ones(sq, sk, dtype=torch.bool)
    tq, tk, tv, tb = (torch.tensor(x, requires_grad=True) for x in (q, k, v, bias))
    s = (0.3 * tq @ tk.T + tb).masked_fill(~mask, float("-inf"))
    rows = mask.any(dim=1)
    pr = torch.where(rows[:, None], torch.softmax(torch.where(rows[:, None], s, torch.zeros_like(s)), dim=-1),
                     torch.zeros_like(s))
    out = pr @ tv
    out.backward(torch.from_numpy(do))
    o, lse = A.head_forward(q, k, v, 0.3, causal, bias=bias)
    assert np.max(np.abs(o - out.detach().numpy())) <= 1e-12
    dq, dk, dv, det = A.head_backward(q, k, v, o, do, lse, 0.3, causal, details=True, bias=bias)
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad), (det["ds"], tb.grad)):
        assert rel_err(got, want.numpy()) <= 1e-12


def test_bias_invariants():
    """A per-row constant bias leaves P (so O, dQ, dK, dV) unchanged and shifts
    LSE by the constant; every row of dBias = dS sums to zero; the ALiBi bias
    given as an elementwise bias gives the ALiBi results."""
    rng = np.random.default_rng(15)
    q, k, v, do = rand(rng, 9, 4), rand(rng, 11, 4), rand(rng, 11, 4), rand(rng, 9, 4)
    c = rand(rng, 9)
    for causal in (False, True):
        o, lse = A.head_forward(q, k, v, 0.5, causal)
        ob, lseb = A.head_forward(q, k, v, 0.5, causal, bias=np.repeat(c[:, None], 11, axis=1))
        assert np.max(np.abs(o - ob)) <= 1e-12
        assert np.max(np.abs((lseb - lse) - c)) <= 1e-12
        g = A.head_backward(q, k, v, o, do, lse, 0.5, causal)
        gb = A.head_backward(q, k, v, ob, do, lseb, 0.5, causal, bias=np.repeat(c[:, None], 11, axis=1))
        for x, y in zip(g, gb):
            assert rel_err(y, x) <= 1e-10
        bias = rand(rng, 9, 11)
        ob, lseb = A.head_forward(q, k, v, 0.5, causal, bias=bias)
        *_, det = A.head_backward(q, k, v, ob, do, lseb, 0.5, causal, details=True, bias=bias)
        assert np.max(np.abs(det["ds"].sum(axis=1))) <= 1e-12
        oa, lsea = A.head_forward(q, k, v, 0.5, causal, alibi=0.3)
        ob, lseb = A.head_forward(q, k, v, 0.5, causal, bias=A.alibi_bias(9, 11, 0.3))
        assert np.max(np.abs(oa - ob)) <= 1e-12


# --------------------------------------------------------------------------
# backward: independent library autograd (torch, float64)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("sq,sk,left,right", [(30, 30, 5, 3), (20, 37, 9, -1), (37, 20, 2, 6)])
def test_window_backward_matches_torch_autograd_float64(sq, sk, left, right):
    """A windowed mask as an explicit boolean mask in torch float64 autograd."""
    import torch
    rng = np.random.default_rng(12)
    q, k, v, do = rand(rng, sq, 8), rand(rng, sk, 8), rand(rng, sk, 8), rand(rng, sq, 8)
    mask = torch.from_numpy(_window_mask_loops(sq, sk, False, left, right))
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = (0.3 * tq @ tk.T).masked_fill(~mask, float("-inf"))
    rows = mask.any(dim=1)
    pr = torch.where(rows[:, None], torch.softmax(torch.where(rows[:, None], s, torch.zeros_like(s)), dim=-1)
                     * mask, torch.zeros_like(s))
    out = pr @ tv
    out.backward(torch.from_numpy(do))
    o, lse = A.head_forward(q, k, v, 0.3, False, window=(left, right))
    assert np.max(np.abs(o - out.detach().numpy())) <= 1e-12
    dq, dk, dv = A.head_backward(q, k, v, o, do, lse, 0.3, False, window=(left, right))
    assert rel_err(dq, tq.grad.numpy()) <= 1e-12
    assert rel_err(dk, tk.grad.numpy()) <= 1e-12
    assert rel_err(dv, tv.grad.numpy()) <= 1e-12


@pytest.mark.parametrize("sq,sk,causal", [(40, 40, True), (40, 40, False), (25, 61, True)])
def test_backward_matches_torch_autograd_float64(sq, sk, causal):
    import torch
    rng = np.random.default_rng(11)
    q, k, v, do = rand(rng, sq, 16), rand(rng, sk, 16), rand(rng, sk, 16), rand(rng, sq, 16)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    mask = _torch_mask(sq, sk, causal)
    s = 0.25 * tq @ tk.T
    s = s.masked_fill(~mask, float("-inf"))
    out = torch.softmax(s, dim=-1) @ tv
    out.backward(torch.from_numpy(do))
    o, lse = A.head_forward(q, k, v, 0.25, causal)
    dq, dk, dv = A.head_backward(q, k, v, o, do, lse, 0.25, causal)
    assert rel_err(dq, tq.grad.numpy()) <= 1e-12
    assert rel_err(dk, tk.grad.numpy()) <= 1e-12
    assert rel_err(dv, tv.grad.numpy()) <= 1e-12


# --------------------------------------------------------------------------
# invariants and closed forms
# --------------------------------------------------------------------------

INVARIANT_SHAPES = [
    # (label, sq, sk, d, causal, scale, do_scale) at the workloads' head dims and lengths
    ("c1_like", 128, 128, 64, False, 1 / 8, 1.0),
    ("c2_like", 1024, 1024, 64, True, 1 / 8, 1.0),
    ("c3_like", 4096, 4096, 128, True, 1 / math.sqrt(128), 0.1),
    ("c3nc_like", 4096, 4096, 128, False, 1 / math.sqrt(128), 0.1),
    ("c4_like", 779, 779, 128, True, 1 / math.sqrt(128), 1.0),
    ("c5_like", 2048, 2048, 128, True, 1 / math.sqrt(128), 1.0),
]


@pytest.mark.parametrize("label,sq,sk,d,causal,scale,do_scale", INVARIANT_SHAPES)
def test_softmax_gradient_invariants(label, sq, sk, d, causal, scale, do_scale):
    """With O and LSE from the oracle's own forward:
    sum_j dS_ij = 0;  D_i = sum_j P_ij dP_ij;  sum_j dK_j = 0;
    sum_j dV_j = sum of dO over rows that see a key."""
    rng = np.random.default_rng(sq + d)
    q, k, v = rand(rng, sq, d), rand(rng, sk, d), rand(rng, sk, d)
    do = do_scale * rand(rng, sq, d)
    o, lse = A.head_forward(q, k, v, scale, causal)
    dq, dk, dv, x = A.head_backward(q, k, v, o, do, lse, scale, causal, details=True)
    assert np.max(np.abs(x["ds"].sum(axis=1))) <= 1e-10, label
    assert rel_err(x["delta"], (x["p"] * x["dp"]).sum(axis=1)) <= 1e-12, label
    assert np.max(np.abs(dk.sum(axis=0))) <= 1e-10 * np.sum(np.abs(dk)), label
    rows = np.isfinite(lse)
    assert rel_err(dv.sum(axis=0), do[rows].sum(axis=0)) <= 1e-12, label


@pytest.mark.parametrize("sq,sk,causal", [(9, 9, False), (9, 9, True), (6, 11, True), (11, 6, True)])
def test_closed_form_constant_keys(sq, sk, causal):
    """All keys equal: P is uniform over the visible keys, so LSE = s q.k + ln n,
    O = mean of the visible values, dV_j = sum over rows seeing j of dO_i / n_i,
    and dQ = 0."""
    rng = np.random.default_rng(5)
    d = 4
    kvec = rand(rng, d)
    q, v, do = rand(rng, sq, d), rand(rng, sk, d), rand(rng, sq, d)
    k = np.tile(kvec, (sk, 1))
    o, lse = A.head_forward(q, k, v, 0.9, causal)
    vis = A.visible(sq, sk, causal)
    n = vis.sum(axis=1)
    for i in range(sq):
        if n[i] == 0:
            assert lse[i] == -np.inf and np.all(o[i] == 0)
            continue
        assert abs(lse[i] - (0.9 * q[i] @ kvec + math.log(n[i]))) <= 1e-12
        assert np.max(np.abs(o[i] - v[vis[i]].mean(axis=0))) <= 1e-12
    dq, dk, dv = A.head_backward(q, k, v, o, do, lse, 0.9, causal)
    want_dv = np.zeros((sk, d))
    for i in range(sq):
        for j in range(sk):
            if vis[i, j]:
                want_dv[j] += do[i] / n[i]
    assert np.max(np.abs(dv - want_dv)) <= 1e-12
    assert np.max(np.abs(dq)) <= 1e-12
    if not causal and sq == sk:
        # column mean of dO broadcast to every key
        assert np.max(np.abs(dv - do.mean(axis=0)[None, :])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_closed_form_constant_values(causal):
    """All values equal: O = v and dP is constant along each row, so dS = 0 and
    dQ = dK = 0."""
    rng = np.random.default_rng(6)
    d = 5
    vvec = rand(rng, d)
    q, k, do = rand(rng, 8, d), rand(rng, 8, d), rand(rng, 8, d)
    v = np.tile(vvec, (8, 1))
    o, lse = A.head_forward(q, k, v, 0.5, causal)
    assert np.max(np.abs(o - vvec)) <= 1e-12
    dq, dk, dv = A.head_backward(q, k, v, o, do, lse, 0.5, causal)
    assert np.max(np.abs(dq)) <= 1e-12
    assert np.max(np.abs(dk)) <= 1e-12


def test_single_key_special_case():
    """Sk = 1: every row puts weight 1 on the only key, so dV_0 = sum_i dO_i and
    dQ = dK = 0; LSE_i = s q_i . k_0."""
    rng = np.random.default_rng(9)
    q, k, v, do = rand(rng, 7, 3), rand(rng, 1, 3), rand(rng, 1, 3), rand(rng, 7, 3)
    o, lse = A.head_forward(q, k, v, 0.8, False)
    assert np.max(np.abs(lse - 0.8 * q @ k[0])) <= 1e-12
    dq, dk, dv = A.head_backward(q, k, v, o, do, lse, 0.8, False)
    assert np.max(np.abs(dv[0] - do.sum(axis=0))) <= 1e-12
    assert np.max(np.abs(dq)) <= 1e-12 and np.max(np.abs(dk)) <= 1e-12


def test_causal_first_row_and_last_key():
    """Causal, Sq = Sk: query 0 sees only key 0 (so dQ_0 = 0) and the last key
    is seen only by the last query (dV_last = P_last,last dO_last)."""
    rng = np.random.default_rng(12)
    q, k, v, do = rand(rng, 10, 4), rand(rng, 10, 4), rand(rng, 10, 4), rand(rng, 10, 4)
    o, lse = A.head_forward(q, k, v, 0.5, True)
    dq, dk, dv, x = A.head_backward(q, k, v, o, do, lse, 0.5, True, details=True)
    assert np.max(np.abs(dq[0])) <= 1e-12
    assert np.max(np.abs(dv[-1] - x["p"][-1, -1] * do[-1])) <= 1e-12


def test_fully_masked_rows():
    """Causal with Sq > Sk: rows i < Sq - Sk see no key; they get LSE = -inf,
    O = 0 and dQ = 0, and do not touch dK or dV."""
    rng = np.random.default_rng(13)
    q, k, v, do = rand(rng, 9, 4), rand(rng, 5, 4), rand(rng, 5, 4), rand(rng, 9, 4)
    o, lse = A.head_forward(q, k, v, 0.5, True)
    assert np.all(lse[:4] == -np.inf) and np.all(np.isfinite(lse[4:]))
    assert np.all(o[:4] == 0)
    dq, dk, dv = A.head_backward(q, k, v, o, do, lse, 0.5, True)
    assert np.all(dq[:4] == 0)
    do2 = do.copy()
    do2[:4] = 1e3 * rand(rng, 4, 4)        # changing dO on empty rows changes nothing
    dq2, dk2, dv2 = A.head_backward(q, k, v, o, do2, lse, 0.5, True)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


# --------------------------------------------------------------------------
# layouts: GQA and varlen reduce to the plain per-head case
# --------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_repeated_heads(causal):
    rng = np.random.default_rng(14)
    b, s, hq, hkv, d = 2, 23, 6, 2, 8
    q, k, v, do = rand(rng, b, s, hq, d), rand(rng, b, s, hkv, d), rand(rng, b, s, hkv, d), rand(rng, b, s, hq, d)
    g = hq // hkv
    kr, vr = np.repeat(k, g, axis=2), np.repeat(v, g, axis=2)
    o, lse = oracle.forward(q, k, v, 0.35, causal)
    o_r, lse_r = oracle.forward(q, kr, vr, 0.35, causal)
    assert np.max(np.abs(o - o_r)) <= 1e-12 and np.max(np.abs(lse - lse_r)) <= 1e-12
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, 0.35, causal)
    dq_r, dk_r, dv_r = oracle.backward(q, kr, vr, o, do, lse, 0.35, causal)
    assert np.max(np.abs(dq - dq_r)) <= 1e-12
    assert np.max(np.abs(dk - dk_r.reshape(b, s, hkv, g, d).sum(axis=3))) <= 1e-12
    assert np.max(np.abs(dv - dv_r.reshape(b, s, hkv, g, d).sum(axis=3))) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_per_sequence_dense(causal):
    rng = np.random.default_rng(15)
    lens = [1, 17, 40, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t, h, d = cu[-1], 3, 8
    q, k, v, do = rand(rng, t, h, d), rand(rng, t, h, d), rand(rng, t, h, d), rand(rng, t, h, d)
    o, lse = oracle.forward(q, k, v, 0.3, causal, cu, cu)
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, 0.3, causal, cu, cu)
    for bi, L in enumerate(lens):
        sl = slice(cu[bi], cu[bi + 1])
        od, lsed = oracle.forward(q[None, sl], k[None, sl], v[None, sl], 0.3, causal)
        assert np.max(np.abs(o[sl] - od[0])) <= 1e-12
        assert np.max(np.abs(lse[:, sl] - lsed[0])) <= 1e-12
        dqd, dkd, dvd = oracle.backward(q[None, sl], k[None, sl], v[None, sl], od, do[None, sl], lsed, 0.3, causal)
        for a, bb in ((dq, dqd), (dk, dkd), (dv, dvd)):
            assert np.max(np.abs(a[sl] - bb[0])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_seqused_equals_truncated_sequences(causal):
    """seqused keeps each sequence's start (cu_seqlens) and shortens it: the
    result on the used rows is the per-sequence dense result of the first
    used rows (causal alignment from the used lengths), and every unused row
    is left at zero."""
    rng = np.random.default_rng(25)
    lens_q, lens_k = [9, 30, 4, 21], [12, 25, 7, 21]
    used_q, used_k = np.array([9, 17, 0, 5], np.int32), np.array([3, 25, 7, 21], np.int32)
    cq = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    h, hkv, d = 4, 2, 8
    q, do = rand(rng, cq[-1], h, d), rand(rng, cq[-1], h, d)
    k, v = rand(rng, ck[-1], hkv, d), rand(rng, ck[-1], hkv, d)
    o, lse = oracle.forward(q, k, v, 0.4, causal, cq, ck, used_q, used_k)
    dq, dk, dv = oracle.backward(q, k, v, o, do, lse, 0.4, causal, cq, ck, used_q, used_k)
    for bi in range(4):
        sq = slice(cq[bi], cq[bi] + used_q[bi])
        sk = slice(ck[bi], ck[bi] + used_k[bi])
        if used_q[bi] and used_k[bi]:
            od, lsed = oracle.forward(q[None, sq], k[None, sk], v[None, sk], 0.4, causal)
            assert np.max(np.abs(o[sq] - od[0])) <= 1e-12
            fin = np.isfinite(lsed[0])
            assert np.array_equal(np.isfinite(lse[:, sq]), fin)
            assert np.max(np.abs(lse[:, sq][fin] - lsed[0][fin]), initial=0) <= 1e-12
            dqd, dkd, dvd = oracle.backward(q[None, sq], k[None, sk], v[None, sk], od, do[None, sq], lsed, 0.4, causal)
            assert np.max(np.abs(dq[sq] - dqd[0])) <= 1e-12
            assert np.max(np.abs(dk[sk] - dkd[0])) <= 1e-12
            assert np.max(np.abs(dv[sk] - dvd[0])) <= 1e-12
        for arr, cu, used in ((dq, cq, used_q), (o, cq, used_q), (dk, ck, used_k), (dv, ck, used_k)):
            assert not np.any(arr[cu[bi] + used[bi]:cu[bi + 1]])
    # seqused equal to the full lengths changes nothing
    full = oracle.backward(q, k, v, o, do, lse, 0.4, causal, cq, ck, np.diff(cq), np.diff(ck))
    plain = oracle.backward(q, k, v, o, do, lse, 0.4, causal, cq, ck)
    for a, bb in zip(full, plain):
        assert np.array_equal(a, bb)


def test_preprocess_delta_layouts_and_definition():
    rng = np.random.default_rng(16)
    o, do = rand(rng, 2, 5, 3, 4), rand(rng, 2, 5, 3, 4)
    dl = oracle.preprocess_delta(o, do)
    assert dl.shape == (2, 3, 5)
    for b in range(2):
        for i in range(5):
            for h in range(3):
                assert abs(dl[b, h, i] - sum(o[b, i, h, t] * do[b, i, h, t] for t in range(4))) <= 1e-13
    ov, dov = o.reshape(10, 3, 4), do.reshape(10, 3, 4)
    dlv = oracle.preprocess_delta(ov, dov, cu_seqlens_q=np.array([0, 5, 10]))
    assert dlv.shape == (3, 10)
    assert np.max(np.abs(dlv - np.transpose(dl, (1, 0, 2)).reshape(3, 10))) <= 1e-15


# --------------------------------------------------------------------------
# dQ postprocess: bfloat16 rounding
# --------------------------------------------------------------------------

def test_bf16_rounding_golden_bit_patterns():
    data = json.load(open(GOLDEN))["bf16_rounding"]["cases"]
    src = np.array([int(a, 16) for a, _, _ in data], np.uint32).view(np.float32)
    want = np.array([int(b, 16) for _, b, _ in data], np.uint16)
    got = A.round_f32_to_bf16_bits(src)
    for (a, b, why), g in zip(data, got):
        assert g == int(b, 16), (a, b, hex(int(g)), why)


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(17)
    x = (rng.standard_normal(1 << 18) * np.exp(rng.uniform(-30, 30, 1 << 18))).astype(np.float32)
    ties = ((rng.integers(0, 1 << 16, 4096).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    got = A.round_f32_to_bf16_bits(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    assert np.array_equal(A.bf16_bits_to_f32(got), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_f16_rounding_golden_bit_patterns():
    data = json.load(open(GOLDEN))["f16_rounding"]["cases"]
    src = np.array([int(a, 16) for a, _, _ in data], np.uint32).view(np.float32)
    got = A.round_f32_to_f16_bits(src)
    for (a, b, why), g in zip(data, got):
        assert g == int(b, 16), (a, b, hex(int(g)), why)


def test_f16_rounding_matches_numpy():
    """numpy's float32 -> float16 conversion is IEEE round-to-nearest-even:
    agreement over normal, subnormal, overflowing and exact-tie inputs."""
    rng = np.random.default_rng(19)
    x = (rng.standard_normal(1 << 18) * np.exp(rng.uniform(-25, 13, 1 << 18))).astype(np.float32)
    # exact ties: odd multiples of half a unit, in normal binades and among subnormals
    e = rng.integers(-14, 16, 4096)
    k = rng.integers(0, 1024, 4096)
    ties_n = np.ldexp(1024.0 + k + 0.5, e - 10).astype(np.float32)
    ties_s = np.ldexp(rng.integers(0, 1024, 4096) + 0.5, -24).astype(np.float32)
    x = np.concatenate([x, ties_n, ties_s, -ties_n, np.float32([np.inf, -np.inf, 0.0, -0.0])])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16)
    got = A.round_f32_to_f16_bits(x)
    assert np.array_equal(got, want.view(np.uint16))
    assert np.array_equal(A.f16_bits_to_f32(got), want.astype(np.float32))
    nan = np.float32([np.nan, -np.nan])
    assert np.all(np.isnan(A.f16_bits_to_f32(A.round_f32_to_f16_bits(nan))))


def test_postprocess_dq_product_in_float32():
    import torch
    rng = np.random.default_rng(18)
    acc = rng.standard_normal((3, 7, 64)).astype(np.float32) * 50
    s = 1 / math.sqrt(128)
    got = oracle.postprocess_dq(acc, s, "bf16")
    want = (torch.from_numpy(acc) * torch.tensor(s, dtype=torch.float32)).to(torch.bfloat16)
    assert np.array_equal(got, want.view(torch.int16).numpy().view(np.uint16))
    got16 = oracle.postprocess_dq(acc, s, "f16")
    assert np.array_equal(got16, (acc * np.float32(s)).astype(np.float16).view(np.uint16))
    got32 = oracle.postprocess_dq(acc, s, "f32")
    assert np.array_equal(got32, acc * np.float32(s))


# --------------------------------------------------------------------------
# planted mistakes: the pins above must catch each of these
# --------------------------------------------------------------------------

def _mutants():
    def drop_delta(q, k, v, o, do, lse, scale, causal):
        p = A._probabilities(q, k, lse, scale, causal)
        ds = p * (do @ v.T)
        return scale * ds @ k, scale * ds.T @ q, p.T @ do

    def wrong_sign(q, k, v, o, do, lse, scale, causal):
        p = A._probabilities(q, k, lse, scale, causal)
        ds = p * ((do @ v.T) + np.sum(do * o, 1)[:, None])
        return scale * ds @ k, scale * ds.T @ q, p.T @ do

    def no_dk_scale(q, k, v, o, do, lse, scale, causal):
        dq, dk, dv = A.head_backward(q, k, v, o, do, lse, scale, causal)
        return dq, dk / scale, dv

    def transposed_p(q, k, v, o, do, lse, scale, causal):
        dq, dk, dv = A.head_backward(q, k, v, o, do, lse, scale, causal)
        p = A._probabilities(q, k, lse, scale, causal)
        return dq, dk, p @ do

    def causal_off_by_one(q, k, v, o, do, lse, scale, causal):
        sq, sk = len(q), len(k)
        ok = A.visible(sq, sk, causal)
        ok = ok & ~np.eye(sq, sk, dtype=bool) if causal else ok
        s = scale * q @ k.T
        p = np.exp(np.where(ok, s - lse[:, None], -np.inf))
        ds = p * ((do @ v.T) - np.sum(do * o, 1)[:, None])
        return scale * ds @ k, scale * ds.T @ q, p.T @ do

    return [drop_delta, wrong_sign, no_dk_scale, transposed_p, causal_off_by_one]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_mistakes_are_caught_by_finite_differences(mutant):
    rng = np.random.default_rng(19)
    q, k, v, do = rand(rng, 5, 3), rand(rng, 5, 3), rand(rng, 5, 3), rand(rng, 5, 3)
    o, lse = A.head_forward(q, k, v, 0.6, True)
    dq, dk, dv = mutant(q, k, v, o, do, lse, 0.6, True)
    good = A.head_backward(q, k, v, o, do, lse, 0.6, True)

    def loss(qq, kk, vv):
        return float(np.sum(do * A.head_forward(qq, kk, vv, 0.6, True)[0]))

    h = 1e-5
    worst = 0.0
    for pos, g in enumerate((dq, dk, dv)):
        base = [q, k, v]
        fd = np.zeros_like(base[pos])
        for idx in np.ndindex(fd.shape):
            xp, xm = base[pos].copy(), base[pos].copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = list(base), list(base)
            ap[pos], am[pos] = xp, xm
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        assert rel_err(good[pos], fd) <= 1e-6
        worst = max(worst, rel_err(g, fd))
    assert worst > 1e-3, mutant.__name__


# --------------------------------------------------------------------------
# the row-blocked forward and the sampled backward (long sequences)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("sq,sk,causal,block", [(7, 9, True, 3), (9, 7, True, 2), (7, 7, False, 4), (5, 8, True, 1)])
def test_row_blocked_forward_matches_scalar_loops(sq, sk, causal, block):
    """head_forward_rows against the scalar-loop definition, with row blocks
    that split the sequence unevenly (rows that see no key included)."""
    rng = np.random.default_rng(300 + sq * 10 + sk)
    q, k, v = rand(rng, sq, 3), rand(rng, sk, 3), rand(rng, sk, 3)
    o, lse = A.head_forward_rows(q, k, v, 0.7, causal, block=block)
    bo, blse = brute_head_forward(q.tolist(), k.tolist(), v.tolist(), 0.7, causal)
    assert np.array_equal(np.isinf(lse), np.isinf(blse))
    fin = np.isfinite(blse)
    assert np.max(np.abs(lse[fin] - blse[fin])) <= 1e-12
    assert np.max(np.abs(o - bo)) <= 1e-12


@pytest.mark.parametrize("window,alibi", [((2, 1), None), (None, 0.3), ((3, -1), 0.5)])
def test_row_blocked_forward_matches_head_forward_windows_alibi(window, alibi):
    rng = np.random.default_rng(31)
    q, k, v = rand(rng, 11, 4), rand(rng, 9, 4), rand(rng, 9, 4)
    for causal in (False, True):
        o, lse = A.head_forward_rows(q, k, v, 0.6, causal, window, alibi, block=4)
        ro, rlse = A.head_forward(q, k, v, 0.6, causal, window, alibi)
        assert np.array_equal(np.isinf(lse), np.isinf(rlse))
        fin = np.isfinite(rlse)
        assert np.max(np.abs(lse[fin] - rlse[fin])) <= 1e-12
        assert np.max(np.abs(o - ro)) <= 1e-12


@pytest.mark.parametrize("sq,sk,causal", [(6, 6, True), (6, 4, True), (4, 7, False), (5, 5, False)])
def test_sampled_backward_finite_differences(sq, sk, causal):
    """head_backward_rows at sampled rows and keys against central finite
    differences of L = sum dO * O(Q, K, V), O from head_forward_rows."""
    rng = np.random.default_rng(400 + sq * 10 + sk)
    q, k, v, do = rand(rng, sq, 3), rand(rng, sk, 3), rand(rng, sk, 3), rand(rng, sq, 3)
    scale = 0.8
    o, lse = A.head_forward_rows(q, k, v, scale, causal, block=2)
    rows, keys = [0, sq - 1, sq // 2], [0, sk - 1, 1]
    dq, dk, dv = A.head_backward_rows(q, k, v, o, do, lse, scale, causal, rows, keys)

    def loss(qq, kk, vv):
        return float(np.sum(do * A.head_forward_rows(qq, kk, vv, scale, causal, block=3)[0]))

    h = 1e-5
    for name, x, g, idx_rows in (("q", q, dq, rows), ("k", k, dk, keys), ("v", v, dv, keys)):
        fd = np.zeros((len(idx_rows), x.shape[1]))
        for a, r in enumerate(idx_rows):
            for t in range(x.shape[1]):
                xp, xm = x.copy(), x.copy()
                xp[r, t] += h
                xm[r, t] -= h
                args_p, args_m = [q, k, v], [q, k, v]
                args_p["qkv".index(name)], args_m["qkv".index(name)] = xp, xm
                fd[a, t] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert rel_err(g, fd) <= 1e-6, (name, rel_err(g, fd))


@pytest.mark.parametrize("window,alibi", [(None, None), ((3, 1), None), (None, 0.25), ((2, -1), 0.4)])
def test_sampled_backward_equals_full_backward(window, alibi):
    """The sampled rows and keys of head_backward_rows equal those rows of
    head_backward (pinned above by finite differences and torch autograd)."""
    rng = np.random.default_rng(57)
    q, k, v, do = rand(rng, 13, 5), rand(rng, 10, 5), rand(rng, 10, 5), rand(rng, 13, 5)
    for causal in (False, True):
        o, lse = A.head_forward(q, k, v, 0.45, causal, window, alibi)
        rows, keys = [0, 3, 12, 7], [9, 0, 4]
        dq, dk, dv = A.head_backward_rows(q, k, v, o, do, lse, 0.45, causal, rows, keys, window, alibi)
        fq, fk, fv = A.head_backward(q, k, v, o, do, lse, 0.45, causal, window=window, alibi=alibi)
        assert np.max(np.abs(dq - fq[rows])) <= 1e-12
        assert np.max(np.abs(dk - fk[keys])) <= 1e-12
        assert np.max(np.abs(dv - fv[keys])) <= 1e-12
