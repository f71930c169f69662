"""GPU parity with ALiBi slopes, an elementwise bias (and dBias) and dropout
together: the kernels' bias variants also apply the slopes, and their dropout
variants the bias and the slopes, so these paths only run when the features
meet.  O and LSE of the forward, then dQ/dK/dV and dBias of the backward
(from the oracle's O and LSE) in every dQ mode, against the fp64 oracle.
Bias rows are padded to a multiple of 8 keys with NaN (which would reach the
results if any padding were read).  Tolerances as in test_gpu_parity."""

import numpy as np
import pytest
import torch

import datagen
import oracle
from _harness import Run, assert_close, small_problem, to_dev, to_host
from exact_attention_backward_amd import api

pytestmark = pytest.mark.gpu

# (dtype, B, Hq, Hkv, Sq, Sk, D, causal, lengths, window, dropout p or 0)
COMBINED_CASES = [
    ("bf16", 2, 4, 2, 200, 200, 128, True, None, None, 0.0),
    ("f16", 1, 4, 4, 170, 260, 64, False, None, None, 0.3),
    ("bf16", 0, 4, 2, 0, 0, 128, True, (7, 129, 300), None, 0.2),      # varlen + GQA
    ("bf16", 1, 66, 1, 130, 130, 64, True, None, None, 0.1),         # a group of more than 64 q-heads
    ("bf16", 1, 4, 2, 200, 200, 256, True, None, (64, -1), 0.25),    # head dim 256 with a window
    ("f32", 1, 2, 2, 150, 200, 64, True, None, None, 0.4),
]


def _id(c):
    dt, b, hq, hkv, sq, sk, d, causal, lens, win, pd = c
    shape = f"lens{'-'.join(map(str, lens))}" if lens else f"b{b}s{sq}x{sk}"
    w = f"-w{win[0]}/{win[1]}" if win else ""
    return f"{dt}-{shape}-h{hq}/{hkv}-d{d}-{'causal' if causal else 'full'}{w}-p{pd}"


def _slopes(h):
    return np.array([2.0 ** (-8.0 * (i + 1) / h) for i in range(h)], np.float32)


def _setup(case):
    dt, b, hq, hkv, sq, sk, d, causal, lens, win, pd = case
    p = small_problem(dt, b, hq, hkv, sq, sk, d, causal, 5100 + hq + d, lengths=lens)
    r = Run(p, oracle_o_lse=False, window=win, alibi=_slopes(hq))
    nb = len(lens) if lens else b
    bias_np = datagen.draw_bias(p, 77, batch=nb)
    skp = (p.seqlen_k + 7) // 8 * 8
    elem = to_dev(bias_np[:1, :1, :1], dt).dtype
    padded = torch.full(bias_np.shape[:3] + (skp,), float("nan"), dtype=elem, device="cuda")
    padded[..., :p.seqlen_k] = to_dev(bias_np, dt)
    bias_dev = padded[..., :p.seqlen_k]
    drop = (float(np.float32(pd)), 0xC0FFEE + hq, 5) if pd > 0 else None
    return p, r, nb, bias_np, bias_dev, drop


@pytest.mark.parametrize("case", COMBINED_CASES, ids=_id)
def test_combined_forward_matches_oracle(case):
    p, r, nb, bias_np, bias_dev, drop = _setup(case)
    print(f"combined forward {_id(case)}", flush=True)
    d = r.dev
    o, lse = api.forward(d["q"], d["k"], d["v"], p.scale, p.causal, window=r.window, alibi_slopes=r.slopes,
                         bias=bias_dev, dropout=drop, **r.kw())
    torch.cuda.synchronize()
    cq, ck = r.cu_np
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal, cq, ck, window=r.window,
                              alibi_slopes=r.alibi, bias=bias_np, dropout=drop)
    assert_close("O", to_host(o), ro, p.dtype)
    g = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(g), fin)
    assert np.max(np.abs(g[fin] - rlse[fin]), initial=0) <= (1e-4 if p.dtype == "f32" else 2e-4)


@pytest.mark.parametrize("algo", ["separate", "stored_ds", "atomic", "ordered"])
@pytest.mark.parametrize("case", COMBINED_CASES, ids=_id)
def test_combined_backward_matches_oracle(case, algo):
    p, r, nb, bias_np, bias_dev, drop = _setup(case)
    if algo == "stored_ds" and p.dtype == "f32":
        pytest.skip("the stored-dS mode is for 16-bit types")
    print(f"combined backward {_id(case)} {algo}", flush=True)
    cq, ck = r.cu_np
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal, cq, ck, window=r.window,
                              alibi_slopes=r.alibi, bias=bias_np, dropout=drop)
    r.set_o_lse(ro, rlse)
    d, kw = r.dev, r.kw()
    dbias = torch.full((nb, p.heads_q, p.seqlen_q, p.seqlen_k), 9.0, dtype=d["q"].dtype, device="cuda")
    plan = api.BackwardPlan(d["q"], d["k"], p.scale, p.causal, algo == "ordered",
                            dq_algo="atomic" if algo == "ordered" else algo, window=r.window,
                            alibi_slopes=r.slopes, bias=bias_dev, dbias=dbias, dropout=drop, **kw)
    dq, dk, dv = (torch.empty_like(d[n]) for n in ("q", "k", "v"))
    plan.run_full(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], dq, dk, dv)
    torch.cuda.synchronize()
    if algo == "ordered":
        assert plan.error_flag() == 0
    res = oracle.backward(r.x["q"], r.x["k"], r.x["v"], r.o, r.x["do"], r.lse, p.scale, p.causal, cq, ck,
                          window=r.window, alibi_slopes=r.alibi, bias=bias_np, want_dbias=True, dropout=drop)
    for n, g, ref in zip(("dQ", "dK", "dV"), (dq, dk, dv), res):
        assert_close(n, to_host(g), ref, p.dtype)
    gdb = to_host(dbias)
    lq = [cq[i + 1] - cq[i] for i in range(nb)] if cq is not None else [p.seqlen_q] * nb
    lk = [ck[i + 1] - ck[i] for i in range(nb)] if ck is not None else [p.seqlen_k] * nb
    inside = np.zeros(gdb.shape, bool)
    for bb in range(nb):
        inside[bb, :, :lq[bb], :lk[bb]] = True
    assert_close("dBias", gdb[inside], res[3][inside], p.dtype)
    assert np.all(gdb[~inside] == 9.0)
