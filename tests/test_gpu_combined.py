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


# (dtype, Hq, Hkv, D, causal, lengths_q, lengths_k, used_q, used_k, dropout p or 0)
SEQUSED_COMBINED = [
    ("bf16", 4, 2, 128, True, (70, 300, 129), (90, 260, 129), (70, 211, 100), (33, 260, 64), 0.2),
    ("f16", 2, 2, 64, False, (200, 65), (150, 300), (199, 1), (150, 129), 0.0),
]


@pytest.mark.parametrize("algo", ["separate", "stored_ds", "atomic"])
@pytest.mark.parametrize("case", SEQUSED_COMBINED,
                         ids=lambda c: f"{c[0]}-h{c[1]}/{c[2]}-d{c[3]}-{'causal' if c[4] else 'full'}-p{c[9]}")
def test_combined_with_used_lengths(case, algo):
    """Used lengths with ALiBi, bias/dBias and dropout: used rows and keys
    match the oracle; rows past a used length, and dBias outside each
    sequence's used block, keep what the buffers held."""
    import math
    from _harness import round_like
    dt, hq, hkv, d, causal, lq, lk, uq, uk, pd = case
    p = datagen.Problem(dt, len(lq), hq, hkv, max(lq), max(lk), d, causal, 1 / math.sqrt(d), 91,
                        lengths_q=tuple(lq), lengths_k=tuple(lk), name="seqused_combined")
    x = datagen.draw(p)
    cq, ck = p.cu_seqlens()
    uq_np, uk_np = np.array(uq, np.int32), np.array(uk, np.int32)
    dev = {n: to_dev(v, dt) for n, v in x.items()}
    cu = dict(cu_seqlens_q=torch.from_numpy(cq).cuda(), cu_seqlens_k=torch.from_numpy(ck).cuda(),
              max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k,
              seqused_q=torch.from_numpy(uq_np).cuda(), seqused_k=torch.from_numpy(uk_np).cuda())
    nb = len(lq)
    used_q = np.zeros(cq[-1], bool)
    used_k = np.zeros(ck[-1], bool)
    for b in range(nb):
        used_q[cq[b]:cq[b] + uq[b]] = True
        used_k[ck[b]:ck[b] + uk[b]] = True
    slopes = _slopes(hq)
    slopes_dev = torch.from_numpy(slopes).cuda()
    bias_np = datagen.draw_bias(p, 61, batch=nb)
    skp = (p.seqlen_k + 7) // 8 * 8
    padded = torch.full(bias_np.shape[:3] + (skp,), float("nan"), dtype=dev["q"].dtype, device="cuda")
    padded[..., :p.seqlen_k] = to_dev(bias_np, dt)
    bias_dev = padded[..., :p.seqlen_k]
    drop = (float(np.float32(pd)), 0xBEEF + hq, 3) if pd > 0 else None
    print(f"combined seqused {case} {algo}", flush=True)
    feats = dict(alibi_slopes=slopes, bias=bias_np, dropout=drop)
    ro, rlse = oracle.forward(x["q"], x["k"], x["v"], p.scale, causal, cq, ck, uq_np, uk_np, **feats)
    o, lse = api.forward(dev["q"], dev["k"], dev["v"], p.scale, causal, alibi_slopes=slopes_dev, bias=bias_dev,
                         dropout=drop, **cu)
    torch.cuda.synchronize()
    assert_close("O", to_host(o)[used_q], ro[used_q], dt)
    gl = lse.cpu().numpy().astype(np.float64)[:, used_q]
    fin = np.isfinite(rlse[:, used_q])
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.max(np.abs(gl[fin] - rlse[:, used_q][fin]), initial=0) <= 2e-4
    # backward from the oracle's O and LSE on the used rows
    o_in = round_like(np.where(used_q[:, None, None], ro, 0.0), dt)
    lse_in = np.where(used_q[None, :], rlse, 0.0).astype(np.float32)
    sentinel = 3.0
    dbias = torch.full((nb, hq, p.seqlen_q, p.seqlen_k), sentinel, dtype=dev["q"].dtype, device="cuda")
    plan = api.BackwardPlan(dev["q"], dev["k"], p.scale, causal, False, dq_algo=algo, alibi_slopes=slopes_dev,
                            bias=bias_dev, dbias=dbias, dropout=drop, **cu)
    dq = torch.full_like(dev["q"], sentinel)
    dk = torch.full_like(dev["k"], sentinel)
    dv = torch.full_like(dev["v"], sentinel)
    plan.run_full(dev["q"], dev["k"], dev["v"], to_dev(o_in, dt), dev["do"], torch.from_numpy(lse_in).cuda(),
                  dq, dk, dv)
    torch.cuda.synchronize()
    res = oracle.backward(x["q"], x["k"], x["v"], o_in, x["do"], lse_in.astype(np.float64), p.scale, causal, cq, ck,
                          uq_np, uk_np, want_dbias=True, **feats)
    for n, g, ref, used in (("dQ", dq, res[0], used_q), ("dK", dk, res[1], used_k), ("dV", dv, res[2], used_k)):
        gh = to_host(g)
        assert_close(n, gh[used], ref[used], dt)
        assert np.all(gh[~used] == sentinel), f"{n}: a row past the used length was written"
    gdb = to_host(dbias)
    inside = np.zeros(gdb.shape, bool)
    for bb in range(nb):
        inside[bb, :, :uq[bb], :uk[bb]] = True
    assert_close("dBias", gdb[inside], res[3][inside], dt)
    assert np.all(gdb[~inside] == sentinel)


@pytest.mark.parametrize("case", [COMBINED_CASES[0], COMBINED_CASES[2]], ids=_id)
def test_ordered_mode_reproducible_with_features(case):
    """The ordered (deterministic) mode with ALiBi, bias/dBias and dropout:
    two runs, with other GPU work between them, agree bit for bit."""
    p, r, nb, bias_np, bias_dev, drop = _setup(case)
    if drop is None:
        drop = (0.15, 4242, 1)
    print(f"ordered reproducible {_id(case)}", flush=True)
    cq, ck = r.cu_np
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal, cq, ck, window=r.window,
                              alibi_slopes=r.alibi, bias=bias_np, dropout=drop)
    r.set_o_lse(ro, rlse)
    d, kw = r.dev, r.kw()
    outs = []
    for rep in range(2):
        dbias = torch.zeros((nb, p.heads_q, p.seqlen_q, p.seqlen_k), dtype=d["q"].dtype, device="cuda")
        plan = api.BackwardPlan(d["q"], d["k"], p.scale, p.causal, True, dq_algo="atomic", window=r.window,
                                alibi_slopes=r.slopes, bias=bias_dev, dbias=dbias, dropout=drop, **kw)
        g = [torch.empty_like(d[n]) for n in ("q", "k", "v")]
        plan.run_full(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], *g)
        torch.randn(1 << 20, device="cuda").mul_(2.0)   # other work between the runs
        torch.cuda.synchronize()
        assert plan.error_flag() == 0
        outs.append([t.clone() for t in g] + [dbias])
    for n, a, b in zip(("dQ", "dK", "dV", "dBias"), outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), n


# (dtype, B, H, S, D, varlen lengths)
STRIDED_COMBINED = [
    ("bf16", 2, 3, 260, 128, None),
    ("f16", 1, 4, 333, 64, None),
    ("bf16", 0, 2, 0, 128, (1, 64, 300, 129)),
]


@pytest.mark.parametrize("dq_algo", ["stored_ds", "separate", "ordered"])
@pytest.mark.parametrize("case", STRIDED_COMBINED,
                         ids=lambda c: f"{c[0]}-{'lens' + '-'.join(map(str, c[5])) if c[5] else f'b{c[1]}s{c[3]}'}-h{c[2]}-d{c[4]}")
def test_strided_layouts_with_features_match_contiguous_bitwise(case, dq_algo):
    """Q, K, V as views of one packed [.., 3, H, D] tensor, dO head-major, O in
    a row-padded buffer and dQ/dK/dV in a packed gradient tensor, with ALiBi,
    bias/dBias and dropout: O, LSE, dQ, dK, dV and dBias equal the contiguous
    run's bit for bit (the ordered mode stands for the atomic one, whose
    order of additions varies)."""
    dt, b, h, s_len, d, lens = case
    p = small_problem(dt, b, h, h, s_len, s_len, d, True, 71, lengths=lens)
    r = Run(p, oracle_o_lse=False, alibi=_slopes(h))
    dev, kw = r.dev, r.kw()
    nb = len(lens) if lens else b
    bias_np = datagen.draw_bias(p, 29, batch=nb)
    skp = (p.seqlen_k + 7) // 8 * 8
    padded = torch.full(bias_np.shape[:3] + (skp,), float("nan"), dtype=dev["q"].dtype, device="cuda")
    padded[..., :p.seqlen_k] = to_dev(bias_np, dt)
    bias_dev = padded[..., :p.seqlen_k]
    drop = (float(np.float32(0.2)), 0xABC, 9)
    det = dq_algo == "ordered"
    algo = "atomic" if det else dq_algo
    feats = dict(alibi_slopes=r.slopes, bias=bias_dev, dropout=drop)
    print(f"strided combined {case} {dq_algo}", flush=True)

    def backward(q, k, v, o, do, lse, grads):
        dbias = torch.full((nb, h, p.seqlen_q, p.seqlen_k), 5.0, dtype=dev["q"].dtype, device="cuda")
        plan = api.BackwardPlan(q, k, p.scale, True, det, dq_algo=algo, dbias=dbias, **feats, **kw)
        plan.run_full(q, k, v, o, do, lse, *grads)
        torch.cuda.synchronize()
        if det:
            assert plan.error_flag() == 0
        return dbias

    o_c, lse_c = api.forward(dev["q"], dev["k"], dev["v"], p.scale, True, **feats, **kw)
    ref = [torch.empty_like(dev[n]) for n in ("q", "k", "v")]
    dbias_c = backward(dev["q"], dev["k"], dev["v"], o_c, dev["do"], lse_c, ref)
    lead = dev["q"].shape[:-2]
    nl = len(lead)
    qkv = torch.empty(*lead, 3, h, d, dtype=dev["q"].dtype, device="cuda")
    for slot, n in enumerate(("q", "k", "v")):
        qkv.select(nl, slot).copy_(dev[n])
    q, k, v = (qkv.select(nl, slot) for slot in range(3))
    do = dev["do"].movedim(nl, 0).contiguous().movedim(0, nl)
    o_pad = torch.full((*lead, h, d + 8), -3.0, dtype=dev["q"].dtype, device="cuda")
    o = o_pad[..., :d]
    lse = torch.empty_like(lse_c)
    api.forward(q, k, v, p.scale, True, out=(o, lse), **feats, **kw)
    dqkv = torch.full((*lead, 3, h, d), -3.0, dtype=dev["q"].dtype, device="cuda")
    grads = [dqkv.select(nl, slot) for slot in range(3)]
    dbias_s = backward(q, k, v, o, do, lse, grads)
    assert torch.equal(o.contiguous().view(torch.int16), o_c.view(torch.int16))
    assert torch.equal(lse, lse_c)
    assert bool((o_pad[..., d:] == -3.0).all())
    for n, g, c in zip(("dQ", "dK", "dV"), grads, ref):
        assert torch.equal(g.contiguous().view(torch.int16), c.view(torch.int16)), n
    assert torch.equal(dbias_s.view(torch.int16), dbias_c.view(torch.int16))
