"""GPU parity of dropout (Philox4x32-10 keep mask) against the fp64 oracle in
every dQ mode and both backward APIs: the forward's kept positions bit for
bit, O and LSE, dQ/dK/dV (and dBias with a bias), dense, varlen, GQA, windows,
fp32, bf16 and fp16.  Tolerances as in test_gpu_parity."""

import numpy as np
import pytest
import torch

import datagen
import oracle
from _harness import Run, assert_close, to_dev, to_host, small_problem
from exact_attention_backward_amd import api

pytestmark = pytest.mark.gpu

# (dtype, B, Hq, Hkv, Sq, Sk, D, causal, lengths, window, p, bias)
DROP_CASES = [
    ("bf16", 2, 3, 3, 200, 200, 128, True, None, None, 0.1, False),
    ("bf16", 1, 4, 2, 170, 264, 64, False, None, None, 0.5, False),
    ("bf16", 1, 2, 2, 333, 333, 128, True, None, (70, 20), 0.3, True),
    ("f16", 1, 8, 2, 300, 300, 128, True, None, None, 0.2, False),
    ("f16", 2, 2, 2, 130, 130, 64, False, None, None, 0.6, True),
    ("f32", 1, 2, 2, 150, 200, 64, True, None, None, 0.25, False),
    ("f32", 1, 4, 2, 97, 96, 128, False, None, None, 0.4, True),
    ("bf16", 0, 4, 2, 0, 0, 128, True, (1, 64, 300), None, 0.15, False),   # varlen + GQA
    ("f16", 0, 2, 2, 0, 0, 64, False, (7, 129, 40), None, 0.35, True),    # varlen + bias
    ("bf16", 1, 4, 2, 200, 200, 256, True, None, (90, 10), 0.2, True),    # head dim 256, window, bias
]


def _id(c):
    dt, b, hq, hkv, sq, sk, d, causal, lens, win, p, bias = c
    shape = f"lens{'-'.join(map(str, lens))}" if lens else f"b{b}s{sq}x{sk}"
    w = f"-w{win[0]}/{win[1]}" if win else ""
    return f"{dt}-{shape}-h{hq}/{hkv}-d{d}-{'causal' if causal else 'full'}{w}-p{p}{'-bias' if bias else ''}"


def _setup(case, seed=5):
    dt, b, hq, hkv, sq, sk, d, causal, lens, win, p_drop, with_bias = case
    p = small_problem(dt, b, hq, hkv, sq, sk, d, causal, 2000 + seed, lengths=lens)
    r = Run(p, oracle_o_lse=False, window=win)
    p32 = float(np.float32(p_drop))             # the probability the library sees
    drop = (p32, 0x5EED0000ABCD + seed, 17 + seed)
    nb = len(lens) if lens else b
    bias_np = bias_dev = None
    if with_bias:
        bias_np = datagen.draw_bias(p, 93, batch=nb)
        skp = (p.seqlen_k + 7) // 8 * 8          # 16-byte aligned rows (every dQ mode)
        padded = torch.zeros(bias_np.shape[:3] + (skp,), dtype=to_dev(bias_np[:1, :1, :1], dt).dtype,
                             device="cuda")
        padded[..., :p.seqlen_k] = to_dev(bias_np, dt)
        bias_dev = padded[..., :p.seqlen_k]
    return p, r, drop, bias_np, bias_dev, nb


@pytest.mark.parametrize("case", DROP_CASES, ids=_id)
def test_dropout_forward_matches_oracle(case):
    p, r, drop, bias_np, bias_dev, nb = _setup(case)
    cq, ck = r.cu_np
    print(f"dropout forward {_id(case)}", flush=True)
    d = r.dev
    o, lse = api.forward(d["q"], d["k"], d["v"], p.scale, p.causal, window=r.window, bias=bias_dev,
                         dropout=drop, **r.kw())
    torch.cuda.synchronize()
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal, cq, ck, window=r.window,
                              bias=bias_np, dropout=drop)
    assert_close("O", to_host(o), ro, p.dtype)
    g = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(g), fin)
    assert np.max(np.abs(g[fin] - rlse[fin]), initial=0) <= (1e-4 if p.dtype == "f32" else 2e-4)


@pytest.mark.parametrize("algo", ["separate", "stored_ds", "atomic"])
@pytest.mark.parametrize("full", [False, True], ids=["three_calls", "bwd_full"])
@pytest.mark.parametrize("case", DROP_CASES, ids=_id)
def test_dropout_backward_matches_oracle(case, full, algo):
    p, r, drop, bias_np, bias_dev, nb = _setup(case)
    if algo == "stored_ds" and p.dtype == "f32":
        pytest.skip("the stored-dS mode is for 16-bit types")
    cq, ck = r.cu_np
    print(f"dropout backward {_id(case)} full={full} algo={algo}", flush=True)
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal, cq, ck, window=r.window,
                              bias=bias_np, dropout=drop)
    r.set_o_lse(ro, rlse)
    d, kw = r.dev, r.kw()
    dbias = None
    if bias_dev is not None:
        dbias = torch.zeros((nb, p.heads_q, p.seqlen_q, p.seqlen_k), dtype=d["q"].dtype, device="cuda")
    plan = api.BackwardPlan(d["q"], d["k"], p.scale, p.causal, False, dq_algo=algo, window=r.window,
                            bias=bias_dev, dbias=dbias, dropout=drop, **kw)
    dq, dk, dv = (torch.empty_like(d[n]) for n in ("q", "k", "v"))
    (plan.run_full if full else plan.run)(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], dq, dk, dv)
    torch.cuda.synchronize()
    res = oracle.backward(r.x["q"], r.x["k"], r.x["v"], r.o, r.x["do"], r.lse, p.scale, p.causal, cq, ck,
                          window=r.window, bias=bias_np, want_dbias=bias_np is not None, dropout=drop)
    for n, g, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), res):
        assert_close(n, to_host(g), ref, p.dtype)
    if bias_np is not None:
        gdb = to_host(dbias)
        lq = [cq[i + 1] - cq[i] for i in range(nb)] if cq is not None else [p.seqlen_q] * nb
        lk = [ck[i + 1] - ck[i] for i in range(nb)] if ck is not None else [p.seqlen_k] * nb
        inside = np.zeros(gdb.shape, bool)
        for bb in range(nb):
            inside[bb, :, :lq[bb], :lk[bb]] = True
        assert_close("dBias", gdb[inside], res[3][inside], p.dtype)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_dropout_forward_keeps_exactly_the_oracle_positions(dt):
    """With V the identity (Sk = D keys), O[i, j] = P_ij / (1 - p) where kept
    and 0 where dropped: the forward kernel's mask equals the oracle's bit for
    bit, over several 4 x 4 blocks, two sequences and four heads."""
    sq = sk = d = 64
    p = small_problem(dt, 2, 4, 4, sq, sk, d, False, 3000)
    r = Run(p, oracle_o_lse=False)
    v = np.zeros((2, sk, 4, d), np.float32)
    for j in range(sk):
        v[:, j, :, j] = 1.0
    r.x["v"] = v
    r.dev["v"] = to_dev(v, dt)
    for p_drop in (0.3, 0.7):
        drop = (float(np.float32(p_drop)), 123456789, 3)
        o, _ = api.forward(r.dev["q"], r.dev["k"], r.dev["v"], p.scale, False, dropout=drop)
        torch.cuda.synchronize()
        got = to_host(o) != 0.0                        # [b, i, h, j]
        for b in range(2):
            for h in range(4):
                keep = oracle.dropout_keep(drop[1], drop[2], b * 4 + h, sq, sk, drop[0])
                assert np.array_equal(got[b, :, h, :], keep), (b, h, p_drop)


def test_dropout_p_zero_equals_plain():
    case = ("bf16", 1, 2, 2, 200, 200, 128, True, None, None, 0.0, False)
    p, r, drop, _, _, _ = _setup(case)
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal)
    r.set_o_lse(ro, rlse)
    d = r.dev
    outs = []
    for dd in (None, (0.0, 1, 2)):
        plan = api.BackwardPlan(d["q"], d["k"], p.scale, p.causal, False, dq_algo="stored_ds", dropout=dd)
        g = [torch.empty_like(d[n]) for n in ("q", "k", "v")]
        plan.run_full(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], *g)
        outs.append(g)
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)
