"""Pins of the dropout oracle (``oracle/dropout.py`` and the ``dropout``
arguments of ``oracle/attention.py``), each independent of the code it checks:
the generator's published known-answer vectors, keep-rate and uniformity
statistics, central finite differences of the dropped output under a fixed
mask, torch float64 autograd with the mask applied, the p = 0 special case,
an invariant of the softmax gradient, and planted mistakes that must fail."""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A
from oracle import dropout as DR

KAT = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))


def rand(rng, *shape):
    return rng.standard_normal(shape)


def test_philox_known_answer_vectors():
    for vec in json.load(open(KAT))["vectors"]:
        ctr = np.array([int(x, 16) for x in vec["counter"]], np.uint64)
        key = np.array([int(x, 16) for x in vec["key"]], np.uint64)
        got = DR.philox4x32(ctr, key)
        assert [int(x) for x in got] == [int(x, 16) for x in vec["output"]], vec
    # the same vectors in one broadcast call
    vecs = json.load(open(KAT))["vectors"]
    ctr = np.array([[int(x, 16) for x in v["counter"]] for v in vecs], np.uint64)
    key = np.array([[int(x, 16) for x in v["key"]] for v in vecs], np.uint64)
    out = DR.philox4x32(ctr, key)
    assert [[int(x) for x in row] for row in out] == [[int(x, 16) for x in v["output"]] for v in vecs]


def test_threshold_rounds_p_to_multiples_of_1_256():
    assert DR.dropout_threshold(0.0) == 0
    assert DR.dropout_threshold(0.1) == 26          # 25.6 -> 26
    assert DR.dropout_threshold(0.5) == 128
    assert DR.dropout_threshold(0.999) == 255       # never all dropped
    for bad in (-0.1, 1.0, 1.5):
        with pytest.raises(ValueError):
            DR.dropout_threshold(bad)


def test_bytes_follow_the_block_layout():
    """Element (4a + r, 4b + c) of (sequence, head) index bh is byte c of word
    r of the generator at counter (b, a, bh, offset), key = the seed's halves."""
    seed, offset, bh = 0x0123456789ABCDEF, 77, 5
    by = DR.dropout_bytes(seed, offset, bh, 13, 22)
    assert by.shape == (13, 22) and by.dtype == np.uint8
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint64)
    for a, b in ((0, 0), (1, 3), (3, 5), (2, 1)):
        w = DR.philox4x32(np.array([b, a, bh, offset], np.uint64), key)
        for r in range(4):
            for c in range(4):
                i, j = 4 * a + r, 4 * b + c
                if i < 13 and j < 22:
                    assert by[i, j] == (int(w[r]) >> (8 * c)) & 0xFF


@pytest.mark.parametrize("p", [0.1, 0.3, 0.5, 0.9])
def test_keep_rate_and_uniformity(p):
    """Over 16 (sequence, head) blocks of 256 x 256 (2^20 elements) the kept
    fraction is within 5 sigma of (256 - t) / 256 and the bytes pass a
    chi-square test of uniformity (256 bins, p-value above 1e-6)."""
    from scipy import stats
    seed, offset = 1234, 9
    bytes_ = np.stack([DR.dropout_bytes(seed, offset, bh, 256, 256) for bh in range(16)])
    keep = bytes_ >= DR.dropout_threshold(p)
    n = keep.size
    want = (256 - DR.dropout_threshold(p)) / 256
    sigma = math.sqrt(want * (1 - want) / n)
    assert abs(keep.mean() - want) <= 5 * sigma
    counts = np.bincount(bytes_.reshape(-1), minlength=256)
    assert stats.chisquare(counts).pvalue > 1e-6
    # neighbours along rows and keys are uncorrelated
    x = bytes_.astype(np.float64)
    for a, b in ((x[:, :, 1:], x[:, :, :-1]), (x[:, 1:, :], x[:, :-1, :])):
        assert abs(np.corrcoef(a.reshape(-1), b.reshape(-1))[0, 1]) < 0.01


def test_masks_differ_by_seed_offset_and_head():
    base = DR.dropout_keep(1, 0, 0, 64, 64, 0.5)
    assert np.array_equal(base, DR.dropout_keep(1, 0, 0, 64, 64, 0.5))          # reproducible
    for other in (DR.dropout_keep(2, 0, 0, 64, 64, 0.5), DR.dropout_keep(1, 1, 0, 64, 64, 0.5),
                  DR.dropout_keep(1, 0, 1, 64, 64, 0.5), DR.dropout_keep(1 << 32, 0, 0, 64, 64, 0.5)):
        agree = (other == base).mean()
        assert 0.45 < agree < 0.55   # independent masks agree about half the time at p = 0.5
    # a prefix of the positions does not depend on the extent asked for
    assert np.array_equal(DR.dropout_keep(3, 4, 2, 10, 7, 0.3), DR.dropout_keep(3, 4, 2, 40, 33, 0.3)[:10, :7])


def test_p_zero_is_plain_attention():
    rng = np.random.default_rng(40)
    q, k, v, do = rand(rng, 1, 9, 4, 5), rand(rng, 1, 11, 2, 5), rand(rng, 1, 11, 2, 5), rand(rng, 1, 9, 4, 5)
    for causal in (False, True):
        o, lse = oracle.forward(q, k, v, 0.4, causal)
        od, lsed = oracle.forward(q, k, v, 0.4, causal, dropout=(0.0, 5, 6))
        assert np.array_equal(o, od) and np.array_equal(lse, lsed)
        g = oracle.backward(q, k, v, o, do, lse, 0.4, causal)
        gd = oracle.backward(q, k, v, o, do, lse, 0.4, causal, dropout=(0.0, 5, 6))
        for x, y in zip(g, gd):
            assert np.array_equal(x, y)


def _fd_dropout(q, k, v, do, scale, causal, dropout, cu=None, bias=None, window=None):
    """Central differences (h = 1e-5) of L = sum(dO * O) with the mask fixed
    by (p, seed, offset), against the analytic gradients (and dBias)."""
    o, lse = oracle.forward(q, k, v, scale, causal, cu, cu, window=window, bias=bias, dropout=dropout)
    res = oracle.backward(q, k, v, o, do, lse, scale, causal, cu, cu, window=window, bias=bias,
                          dropout=dropout, want_dbias=bias is not None)

    def loss(qq, kk, vv, bb):
        oo, _ = oracle.forward(qq, kk, vv, scale, causal, cu, cu, window=window, bias=bb, dropout=dropout)
        return float(np.sum(do * oo))

    h = 1e-5
    xs = [q, k, v] + ([bias] if bias is not None else [])
    for pos, (x, g) in enumerate(zip(xs, res)):
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap = list(xs) + ([None] if bias is None else [])
            am = list(xs) + ([None] if bias is None else [])
            ap[pos], am[pos] = xp, xm
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * h)
        assert rel_err(g, fd) <= 1e-6, ("dq", "dk", "dv", "dbias")[pos]
    return res


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_backward_finite_differences_gqa(causal):
    rng = np.random.default_rng(41)
    q, k, v, do = rand(rng, 1, 6, 4, 3), rand(rng, 1, 7, 2, 3), rand(rng, 1, 7, 2, 3), rand(rng, 1, 6, 4, 3)
    _fd_dropout(q, k, v, do, 0.5, causal, (0.4, 99, 3))


def test_dropout_backward_finite_differences_varlen_with_bias():
    rng = np.random.default_rng(42)
    cu = np.array([0, 3, 8], np.int32)
    q, k, v, do = rand(rng, 8, 2, 3), rand(rng, 8, 1, 3), rand(rng, 8, 1, 3), rand(rng, 8, 2, 3)
    bias = rand(rng, 2, 2, 5, 5)
    _fd_dropout(q, k, v, do, 0.6, True, (0.3, 7, 11), cu=cu, bias=bias)


def test_dropout_backward_finite_differences_window():
    rng = np.random.default_rng(43)
    q, k, v, do = rand(rng, 1, 7, 2, 3), rand(rng, 1, 7, 2, 3), rand(rng, 1, 7, 2, 3), rand(rng, 1, 7, 2, 3)
    _fd_dropout(q, k, v, do, 0.5, False, (0.5, 1, 2), window=(2, 1))


@pytest.mark.parametrize("sq,sk,causal", [(30, 30, False), (20, 37, True), (37, 20, True)])
def test_dropout_matches_torch_autograd_float64(sq, sk, causal):
    """torch float64 autograd of ((softmax(S) * keep) / (1 - p)) V with the
    oracle's mask: O, dQ, dK, dV and dBias."""
    import torch
    rng = np.random.default_rng(44)
    q, k, v, do, bias = (rand(rng, sq, 8), rand(rng, sk, 8), rand(rng, sk, 8), rand(rng, sq, 8),
                         rand(rng, sq, sk))
    p = 0.35
    keep = DR.dropout_keep(21, 4, 3, sq, sk, p)
    rp = 1 / (1 - p)
    i = torch.arange(sq)[:, None]
    j = torch.arange(sk)[None, :]
    mask = (j <= i + (sk - sq)) if causal else torch.ones(sq, sk, dtype=torch.bool)
    tq, tk, tv, tb = (torch.tensor(x, requires_grad=True) for x in (q, k, v, bias))
    s = (0.3 * tq @ tk.T + tb).masked_fill(~mask, float("-inf"))
    rows = mask.any(dim=1)
    pr = torch.where(rows[:, None], torch.softmax(torch.where(rows[:, None], s, torch.zeros_like(s)), dim=-1),
                     torch.zeros_like(s))
    out = (pr * torch.from_numpy(keep) * rp) @ tv
    out.backward(torch.from_numpy(do))
    o, lse = A.head_forward(q, k, v, 0.3, causal, bias=bias, dropout=(keep, rp))
    assert np.max(np.abs(o - out.detach().numpy())) <= 1e-12
    dq, dk, dv, det = A.head_backward(q, k, v, o, do, lse, 0.3, causal, details=True, bias=bias,
                                      dropout=(keep, rp))
    for got, want in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad), (det["ds"], tb.grad)):
        assert rel_err(got, want.numpy()) <= 1e-12


def test_dropout_invariants():
    """Rows of dS still sum to zero (sum_j P dP = D for the dropped output);
    dV summed over keys is rp sum_i (sum_j keep P) dO_i; the LSE does not
    depend on the mask."""
    rng = np.random.default_rng(45)
    q, k, v, do = rand(rng, 12, 4), rand(rng, 15, 4), rand(rng, 15, 4), rand(rng, 12, 4)
    keep = DR.dropout_keep(8, 0, 0, 12, 15, 0.5)
    for causal in (False, True):
        o0, lse0 = A.head_forward(q, k, v, 0.5, causal)
        o, lse = A.head_forward(q, k, v, 0.5, causal, dropout=(keep, 2.0))
        assert np.array_equal(lse, lse0)
        dq, dk, dv, det = A.head_backward(q, k, v, o, do, lse, 0.5, causal, details=True, dropout=(keep, 2.0))
        assert np.max(np.abs(det["ds"].sum(axis=1))) <= 1e-12
        kept_mass = (2.0 * np.where(keep, det["p"], 0.0)).sum(axis=1)
        assert np.max(np.abs(dv.sum(axis=0) - (kept_mass[:, None] * do).sum(axis=0))) <= 1e-12


def _mutant_dv_undropped(q, k, v, o, do, lse, scale, causal, details=False, window=None, alibi=None, bias=None,
                         dropout=None):
    """Slip: dV from the undropped P."""
    keep, rp = dropout
    p = A._probabilities(np.asarray(q, float), np.asarray(k, float), np.asarray(lse, float), scale, causal,
                         window, alibi, bias)
    delta = np.sum(do * o, axis=1)
    dp = rp * np.where(keep, do @ np.asarray(v, float).T, 0.0)
    ds = p * (dp - delta[:, None])
    out = (scale * (ds @ k), scale * (ds.T @ q), p.T @ do)
    return out + ({"ds": ds},) if details else out


def _mutant_no_rescale(q, k, v, o, do, lse, scale, causal, details=False, window=None, alibi=None, bias=None,
                       dropout=None):
    """Slip: the mask applied without the 1 / (1 - p) factor."""
    keep, rp = dropout
    return _ORIG_BACKWARD(q, k, v, o, do, lse, scale, causal, details, window, alibi, bias, (keep, 1.0))


def _mutant_mask_on_ds(q, k, v, o, do, lse, scale, causal, details=False, window=None, alibi=None, bias=None,
                       dropout=None):
    """Slip: the mask applied to dS instead of dP (dropped elements get 0, not -P D)."""
    keep, rp = dropout
    res = _ORIG_BACKWARD(q, k, v, o, do, lse, scale, causal, True, window, alibi, bias, dropout)
    ds = np.where(keep, res[3]["ds"], 0.0)
    out = (scale * (ds @ np.asarray(k, float)), scale * (ds.T @ np.asarray(q, float)), res[2])
    return out + ({"ds": ds},) if details else out


_ORIG_BACKWARD = A.head_backward


@pytest.mark.parametrize("mutant", [_mutant_dv_undropped, _mutant_no_rescale, _mutant_mask_on_ds],
                         ids=lambda f: f.__name__)
def test_planted_dropout_mistakes_are_caught(mutant, monkeypatch):
    """Each plausible slip in the dropout gradient fails the finite-difference pin."""
    monkeypatch.setattr(A, "head_backward", mutant)
    rng = np.random.default_rng(46)
    q, k, v, do = rand(rng, 1, 5, 2, 3), rand(rng, 1, 5, 1, 3), rand(rng, 1, 5, 1, 3), rand(rng, 1, 5, 2, 3)
    with pytest.raises(AssertionError):
        _fd_dropout(q, k, v, do, 0.5, False, (0.5, 3, 1))
