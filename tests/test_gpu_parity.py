"""GPU parity of every entry point against the fp64 oracle, element by element,
at sizes the oracle finishes in seconds that span several tiles and ragged
tails: dense and varlen, causal (bottom-right, with fully masked rows) and not,
local (sliding-window) masks with and without the causal bound, ALiBi, GQA, both
head dims, fp32, bf16 and fp16, every dQ mode (separate pass, stored dS,
atomic, ordered atomic).

Tolerance: max|gpu - ref| / max|ref| per tensor <= 1e-5 (fp32 path),
<= 2e-2 (bf16 path) and <= 2.5e-3 (fp16 path); the dQ postprocess is
bit-exact; the deterministic mode is bitwise reproducible."""

import math

import numpy as np
import pytest
import torch

import oracle
from _harness import Run, assert_close, rel_err, round_like, small_problem, to_dev, to_host, TOL
from exact_attention_backward_amd import api

pytestmark = pytest.mark.gpu

# (dtype, B, Hq, Hkv, Sq, Sk, D, causal, lengths)
CASES = [
    ("bf16", 2, 3, 3, 200, 200, 128, True, None),
    ("bf16", 2, 3, 3, 200, 200, 128, False, None),
    ("bf16", 1, 2, 2, 300, 170, 128, True, None),     # Sq > Sk: rows 0..129 see no key
    ("bf16", 1, 2, 2, 170, 300, 128, True, None),     # Sq < Sk
    ("bf16", 1, 2, 2, 130, 257, 64, False, None),
    ("bf16", 2, 4, 4, 333, 333, 64, True, None),
    ("bf16", 1, 8, 2, 333, 333, 128, True, None),     # GQA, group of 4
    ("bf16", 1, 6, 2, 190, 190, 64, False, None),     # GQA, group of 3
    ("bf16", 0, 4, 4, 0, 0, 128, True, (1, 64, 130, 257, 500)),   # varlen
    ("bf16", 0, 4, 2, 0, 0, 64, False, (7, 128, 129, 300)),       # varlen + GQA
    ("f32", 1, 2, 2, 128, 128, 64, False, None),      # the fp32 workload
    ("f32", 1, 2, 2, 150, 99, 64, True, None),
    ("f32", 1, 4, 2, 97, 200, 128, True, None),
    ("f32", 0, 2, 2, 0, 0, 128, False, (5, 70, 33)),
    ("f16", 2, 3, 3, 200, 200, 128, True, None),
    ("f16", 1, 2, 2, 170, 300, 64, True, None),       # Sq < Sk
    ("f16", 1, 8, 2, 333, 333, 128, False, None),     # GQA, group of 4
    ("f16", 0, 4, 2, 0, 0, 64, True, (7, 128, 129, 300)),         # varlen + GQA
]


def _id(c):
    dt, b, hq, hkv, sq, sk, d, causal, lens = c
    shape = f"lens{'-'.join(map(str, lens))}" if lens else f"b{b}s{sq}x{sk}"
    return f"{dt}-{shape}-h{hq}/{hkv}-d{d}-{'causal' if causal else 'full'}"


def problem(c, seed=0, deterministic=False):
    dt, b, hq, hkv, sq, sk, d, causal, lens = c
    return small_problem(dt, b, hq, hkv, sq, sk, d, causal, 1000 + seed, lengths=lens, deterministic=deterministic)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_forward_matches_oracle(case):
    p = problem(case)
    r = Run(p, oracle_o_lse=False)
    print(f"forward {_id(case)}", flush=True)
    o, lse = r.gpu_forward()
    torch.cuda.synchronize()
    cq, ck = r.cu_np
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal, cq, ck)
    assert_close("O", to_host(o), ro, p.dtype)
    g = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isfinite(g), np.isfinite(rlse))
    fin = np.isfinite(rlse)
    assert np.max(np.abs(g[fin] - rlse[fin])) <= (1e-5 if p.dtype == "f32" else 1e-4)


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds", "atomic"])
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_backward_matches_oracle(case, dq_algo):
    if dq_algo == "stored_ds" and case[0] == "f32":
        pytest.skip("the stored-dS mode is for 16-bit types only (the ABI rejects fp32)")
    p = problem(case)
    r = Run(p)
    print(f"backward {_id(case)} dq={dq_algo}", flush=True)
    dq, dk, dv, plan = r.gpu_backward(dq_algo=dq_algo)
    rdq, rdk, rdv = r.oracle_backward()
    errs = {n: rel_err(to_host(g), ref) for n, g, ref in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv))}
    print("rel errs", errs, flush=True)
    for n, e in errs.items():
        assert e <= TOL[p.dtype], f"{n}: max|gpu-ref|/max|ref| = {e:.3e} > {TOL[p.dtype]}" 
    # D from the preprocess
    cq, _ = r.cu_np
    rd = oracle.preprocess_delta(r.o, r.x["do"], cq)
    assert rel_err(plan.delta.cpu().numpy(), rd) <= (1e-6 if p.dtype == "f32" else 1e-5)


DET_CASES = [CASES[0], CASES[6], CASES[8], CASES[1], CASES[17]]


@pytest.mark.parametrize("dq_algo", ["atomic", "separate", "stored_ds"])
@pytest.mark.parametrize("case", DET_CASES, ids=_id)
def test_deterministic_mode_is_bitwise_reproducible(case, dq_algo):
    """Ordered atomic adds (deterministic atomic mode), the separate dQ pass
    and the stored-dS pass all give bitwise identical results on repeated
    runs."""
    p = problem(case, deterministic=True)
    r = Run(p)
    print(f"deterministic {_id(case)} dq={dq_algo}", flush=True)
    outs = []
    for _ in range(3):
        dq, dk, dv, plan = r.gpu_backward(dq_algo=dq_algo)
        assert plan.error_flag() == 0
        outs.append([t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu() for t in (dq, dk, dv)])
    for rep in outs[1:]:
        for a, b in zip(outs[0], rep):
            assert torch.equal(a, b)
    rdq, rdk, rdv = r.oracle_backward()
    for n, g, ref in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert_close(n, to_host(g), ref, p.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_dq_postprocess_bit_exact(dtype, d):
    """Seeded fp32 accumulator -> dQ, compared bit for bit with the oracle's
    rounding of the same fp32 product."""
    p = small_problem(dtype, 2, 3, 3, 77, 77, d, False, 5)
    r = Run(p, oracle_o_lse=False)
    plan = r.plan()
    rng = np.random.default_rng(77 + d)
    acc = (rng.standard_normal((2, 3, 77, d)) * np.exp(rng.uniform(-8, 8, (2, 3, 77, d)))).astype(np.float32)
    ws = plan.workspace
    ws[: acc.nbytes].copy_(torch.from_numpy(acc.view(np.uint8).reshape(-1)).cuda())
    dq = torch.empty_like(r.dev["q"])
    plan.postprocess(dq)
    torch.cuda.synchronize()
    want = oracle.postprocess_dq(np.transpose(acc, (0, 2, 1, 3)), p.scale, dtype)
    if dtype in ("bf16", "f16"):
        got = dq.view(torch.int16).cpu().numpy().view(np.uint16)
    else:
        got = dq.cpu().numpy()
    assert np.array_equal(got, want)


def test_preprocess_clears_workspace_and_main_accumulates():
    """Atomic mode: running the main kernel twice without the preprocess adds
    dQ twice (the documented contract); with it in between, results repeat."""
    p = small_problem("bf16", 1, 2, 2, 150, 150, 64, True, 9)
    r = Run(p)
    d = r.dev
    plan = r.plan(dq_algo="atomic")
    dq1, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    plan.run(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], dq1, dk, dv)
    plan.main(d["q"], d["k"], d["v"], d["do"], d["lse"], dk, dv)
    dq2 = torch.empty_like(dq1)
    plan.postprocess(dq2)
    torch.cuda.synchronize()
    assert rel_err(to_host(dq2), 2 * to_host(dq1)) <= 1e-2
    plan.run(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], dq2, dk, dv)
    torch.cuda.synchronize()
    assert rel_err(to_host(dq2), to_host(dq1)) <= 1e-2


# local (sliding-window) masks: (dtype, B, Hq, Hkv, Sq, Sk, D, causal, lengths, window)
WINDOW_CASES = [
    ("bf16", 2, 3, 3, 300, 300, 128, False, None, (64, 64)),
    ("bf16", 1, 2, 2, 500, 500, 128, True, None, (100, -1)),       # causal sliding window
    ("bf16", 1, 2, 2, 333, 333, 64, False, None, (-1, 40)),
    ("bf16", 1, 2, 2, 300, 170, 128, False, None, (10, 5)),        # Sq > Sk: rows that see no key
    ("bf16", 1, 2, 2, 170, 600, 128, False, None, (30, 0)),        # Sq < Sk: key tiles no row sees
    ("bf16", 1, 8, 2, 400, 400, 128, True, None, (0, -1)),         # each row sees its diagonal key only
    ("bf16", 1, 2, 2, 260, 260, 64, False, None, (0, 0)),
    ("bf16", 1, 2, 2, 200, 200, 128, False, None, (5000, 5000)),   # wider than the sequence
    ("bf16", 0, 4, 2, 0, 0, 128, True, (1, 64, 300, 513), (128, -1)),   # varlen + GQA
    ("f16", 1, 4, 2, 333, 333, 64, True, None, (77, -1)),
    ("f16", 2, 3, 3, 260, 260, 128, False, None, (200, 3)),
    ("f32", 1, 2, 2, 150, 200, 64, False, None, (20, 30)),
    ("f32", 0, 2, 2, 0, 0, 128, True, (5, 170, 33), (40, -1)),
]


def _winid(c):
    return f"{_id(c[:9])}-w{c[9][0]}/{c[9][1]}"


@pytest.mark.parametrize("case", WINDOW_CASES, ids=_winid)
def test_window_forward_matches_oracle(case):
    p = problem(case[:9])
    r = Run(p, oracle_o_lse=False, window=case[9])
    print(f"window forward {_winid(case)}", flush=True)
    o, lse = r.gpu_forward()
    torch.cuda.synchronize()
    cq, ck = r.cu_np
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal, cq, ck, window=case[9])
    assert_close("O", to_host(o), ro, p.dtype)
    g = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isfinite(g), np.isfinite(rlse))
    fin = np.isfinite(rlse)
    assert np.max(np.abs(g[fin] - rlse[fin]), initial=0) <= (1e-5 if p.dtype == "f32" else 1e-4)


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds", "atomic"])
@pytest.mark.parametrize("case", WINDOW_CASES, ids=_winid)
def test_window_backward_matches_oracle(case, dq_algo):
    if dq_algo == "stored_ds" and case[0] == "f32":
        pytest.skip("the stored-dS mode is for 16-bit types only (the ABI rejects fp32)")
    p = problem(case[:9])
    r = Run(p, window=case[9])
    print(f"window backward {_winid(case)} dq={dq_algo}", flush=True)
    dq, dk, dv, plan = r.gpu_backward(dq_algo=dq_algo)
    rdq, rdk, rdv = r.oracle_backward()
    for n, g, ref in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert_close(n, to_host(g), ref, p.dtype)


@pytest.mark.parametrize("dq_algo", ["atomic", "stored_ds"])
@pytest.mark.parametrize("case", [WINDOW_CASES[1], WINDOW_CASES[4], WINDOW_CASES[8]], ids=_winid)
def test_window_deterministic_mode(case, dq_algo):
    """Ordered dQ accumulation under a window: the key tiles that visit a
    query tile take their turns in order (no wait gives up) and repeated runs
    agree bit for bit."""
    p = problem(case[:9], deterministic=True)
    r = Run(p, window=case[9])
    print(f"window deterministic {_winid(case)} dq={dq_algo}", flush=True)
    outs = []
    for _ in range(2):
        dq, dk, dv, plan = r.gpu_backward(dq_algo=dq_algo)
        assert plan.error_flag() == 0
        outs.append([t.view(torch.int16 if t.element_size() == 2 else torch.int32).cpu() for t in (dq, dk, dv)])
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    rdq, rdk, rdv = r.oracle_backward()
    for n, g, ref in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert_close(n, to_host(g), ref, p.dtype)


def test_window_unbounded_equals_plain_masks():
    """A window with both sides unbounded (-1, -1) gives exactly the plain
    causal and full results (the same kernels' arithmetic, bit for bit)."""
    for causal in (True, False):
        p = small_problem("bf16", 1, 2, 2, 300, 300, 128, causal, 31)
        plain = Run(p)
        loc = Run(p, window=(-1, -1))
        a = plain.gpu_backward(dq_algo="separate")[:3]
        b = loc.gpu_backward(dq_algo="separate")[:3]
        for x, y in zip(a, b):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))


# ALiBi: (dtype, B, Hq, Hkv, Sq, Sk, D, causal, lengths, window); slopes 2^(-8 (h + 1) / Hq)
ALIBI_CASES = [
    ("bf16", 2, 4, 4, 300, 300, 128, True, None, None),
    ("bf16", 1, 4, 4, 333, 333, 64, False, None, None),
    ("bf16", 1, 8, 2, 300, 170, 128, True, None, None),       # Sq > Sk, GQA
    ("bf16", 1, 4, 2, 170, 400, 128, False, None, (50, 20)),  # with a window
    ("bf16", 0, 4, 2, 0, 0, 128, True, (1, 64, 300, 513), (128, -1)),   # varlen
    ("bf16", 1, 66, 1, 130, 130, 64, True, None, None),       # a group of more than 64 q-heads
    ("f16", 1, 4, 4, 260, 260, 128, True, None, None),
    ("f16", 1, 6, 2, 200, 333, 64, False, None, None),
    ("f32", 1, 2, 2, 150, 200, 64, True, None, None),
    ("f32", 0, 2, 2, 0, 0, 128, False, (5, 170, 33), None),
    ("bf16", 1, 4, 2, 200, 260, 256, True, None, (64, -1)),   # head dim 256 with a window
]


def _alibi_slopes(hq):
    return np.array([2.0 ** (-8.0 * (h + 1) / hq) for h in range(hq)], np.float32)


def _alibiid(c):
    w = f"-w{c[9][0]}/{c[9][1]}" if c[9] else ""
    return f"{_id(c[:9])}{w}-alibi"


@pytest.mark.parametrize("case", ALIBI_CASES, ids=_alibiid)
def test_alibi_forward_matches_oracle(case):
    p = problem(case[:9])
    r = Run(p, oracle_o_lse=False, window=case[9], alibi=_alibi_slopes(case[2]))
    print(f"alibi forward {_alibiid(case)}", flush=True)
    o, lse = r.gpu_forward()
    torch.cuda.synchronize()
    cq, ck = r.cu_np
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal, cq, ck, window=case[9],
                              alibi_slopes=r.alibi)
    assert_close("O", to_host(o), ro, p.dtype)
    g = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isfinite(g), np.isfinite(rlse))
    fin = np.isfinite(rlse)
    assert np.max(np.abs(g[fin] - rlse[fin]), initial=0) <= (1e-4 if p.dtype == "f32" else 2e-4)


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds", "atomic"])
@pytest.mark.parametrize("case", ALIBI_CASES, ids=_alibiid)
def test_alibi_backward_matches_oracle(case, dq_algo):
    if dq_algo == "stored_ds" and case[0] == "f32":
        pytest.skip("the stored-dS mode is for 16-bit types only (the ABI rejects fp32)")
    p = problem(case[:9])
    r = Run(p, window=case[9], alibi=_alibi_slopes(case[2]))
    print(f"alibi backward {_alibiid(case)} dq={dq_algo}", flush=True)
    dq, dk, dv, plan = r.gpu_backward(dq_algo=dq_algo)
    rdq, rdk, rdv = r.oracle_backward()
    for n, g, ref in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert_close(n, to_host(g), ref, p.dtype)


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds"])
def test_alibi_zero_slopes_equal_plain(dq_algo):
    """Zero slopes take the ALiBi kernels and give the plain results bit for bit."""
    p = small_problem("bf16", 1, 4, 2, 300, 300, 128, True, 33)
    a = Run(p).gpu_backward(dq_algo=dq_algo)[:3]
    b = Run(p, alibi=np.zeros(4, np.float32)).gpu_backward(dq_algo=dq_algo)[:3]
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds", "atomic"])
@pytest.mark.parametrize("d,s,causal", [(128, 700, False), (128, 700, True), (64, 650, False)])
def test_alibi_negative_slopes_with_padded_rows(d, s, causal, dq_algo):
    """Negative slopes (the logit grows with the distance from the diagonal)
    on a length that leaves padded rows in the last query tile: those rows
    must not reach real keys' gradients (their ALiBi term alone would
    overflow exp2; 0 * inf would be NaN)."""
    p = small_problem("bf16", 1, 4, 2, s, s, d, causal, 44)
    slopes = np.array([-0.075, -0.15, -0.225, -0.3], np.float32)
    assert s % (32 if d == 128 else 64) != 0
    assert float(np.max(-slopes)) * s * 1.4427 > 128      # exp2 of the padded rows' term overflows
    r = Run(p, alibi=slopes)
    print(f"negative alibi d{d} s{s} causal={causal} dq={dq_algo}", flush=True)
    dq, dk, dv, plan = r.gpu_backward(dq_algo=dq_algo)
    rdq, rdk, rdv = r.oracle_backward()
    for n, g, ref in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        h = to_host(g)
        assert np.all(np.isfinite(h)), f"{n} has non-finite values"
        assert_close(n, h, ref, p.dtype)


# attn_bwd_full against the three-call path: (case, window, alibi)
FULL_CASES = [
    (CASES[0], None, False),      # bf16 dense causal D128
    (CASES[3], None, False),      # bf16 Sq < Sk causal
    (CASES[9], None, False),      # bf16 varlen + GQA D64
    (CASES[14], None, False),     # fp16 dense causal D128
    (CASES[15], None, False),     # fp16 Sq < Sk causal D64
    (CASES[17], None, False),     # fp16 varlen + GQA causal
    (CASES[11], None, False),     # fp32 Sq > Sk causal
    (CASES[13], None, False),     # fp32 varlen
    (CASES[6], (100, -1), True),  # bf16 GQA causal window + ALiBi
]


def _fullid(c):
    case, win, alibi = c
    return _id(case) + (f"-w{win[0]}/{win[1]}" if win else "") + ("-alibi" if alibi else "")


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds", "atomic"])
@pytest.mark.parametrize("fc", FULL_CASES, ids=_fullid)
def test_bwd_full_matches_three_calls_bitwise(fc, dq_algo):
    """attn_bwd_full (dQ written by the dQ pass in the I/O type, or through
    the postprocess in the atomic mode) gives the three-call results bit for
    bit (the atomic mode in its deterministic order), and the oracle's."""
    case, win, alibi = fc
    if dq_algo == "stored_ds" and case[0] == "f32":
        pytest.skip("the stored-dS mode is for 16-bit types only (the ABI rejects fp32)")
    p = problem(case, deterministic=dq_algo == "atomic")
    r = Run(p, window=win, alibi=_alibi_slopes(case[2]) if alibi else None)
    print(f"full {_fullid(fc)} dq={dq_algo}", flush=True)
    d = r.dev
    plan = r.plan(dq_algo=dq_algo)
    sentinel = 7.0
    three = [torch.full_like(d[n], sentinel) for n in ("q", "k", "v")]
    plan.run(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], *three)
    full = [torch.full_like(d[n], sentinel) for n in ("q", "k", "v")]
    plan.run_full(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], *full)
    torch.cuda.synchronize()
    if p.deterministic:
        assert plan.error_flag() == 0
    iview = torch.int16 if full[0].element_size() == 2 else torch.int32
    for n, a, b in zip(("dQ", "dK", "dV"), three, full):
        assert torch.equal(a.view(iview), b.view(iview)), n
    rdq, rdk, rdv = r.oracle_backward()
    for n, g, ref in (("dQ", full[0], rdq), ("dK", full[1], rdk), ("dV", full[2], rdv)):
        assert_close(n, to_host(g), ref, p.dtype)


# head dims other than 64 and 128 (padded with zeros to 64, 128 or 256 inside
# the kernels); above 128 the dK/dV kernel runs with four waves and 64 keys
# per workgroup and the atomic mode runs as the separate one
HEADDIM_CASES = [
    ("bf16", 1, 2, 2, 200, 200, 256, True, None),
    ("bf16", 1, 4, 2, 150, 260, 192, False, None),   # GQA, Sq < Sk
    ("f16", 2, 2, 2, 130, 130, 136, True, None),
    ("bf16", 0, 4, 2, 0, 0, 256, True, (7, 128, 129, 300)),   # varlen + GQA
    ("f16", 1, 2, 2, 300, 170, 248, True, None),     # Sq > Sk: rows that see no key
    ("bf16", 1, 2, 2, 200, 200, 8, True, None),
    ("bf16", 1, 3, 3, 150, 260, 40, False, None),
    ("bf16", 2, 4, 2, 130, 130, 72, True, None),     # GQA
    ("bf16", 1, 2, 2, 300, 300, 96, True, None),
    ("f16", 1, 2, 2, 170, 170, 120, False, None),
    ("f16", 0, 4, 2, 0, 0, 80, True, (7, 128, 129, 300)),   # varlen + GQA
    ("f32", 1, 2, 2, 100, 150, 48, True, None),
    ("f32", 1, 2, 2, 100, 100, 112, False, None),
]


@pytest.mark.parametrize("case", HEADDIM_CASES, ids=_id)
def test_head_dim_forward_matches_oracle(case):
    p = problem(case)
    r = Run(p, oracle_o_lse=False)
    print(f"head dim forward {_id(case)}", flush=True)
    o, lse = r.gpu_forward()
    torch.cuda.synchronize()
    cq, ck = r.cu_np
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal, cq, ck)
    assert_close("O", to_host(o), ro, p.dtype)
    g = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(g), fin)
    assert np.max(np.abs(g[fin] - rlse[fin]), initial=0) <= (1e-5 if p.dtype == "f32" else 1e-4)


@pytest.mark.parametrize("full", [False, True], ids=["three_calls", "bwd_full"])
@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds", "atomic"])
@pytest.mark.parametrize("case", HEADDIM_CASES, ids=_id)
def test_head_dim_backward_matches_oracle(case, dq_algo, full):
    if dq_algo == "stored_ds" and case[0] == "f32":
        pytest.skip("the stored-dS mode is for 16-bit types only (the ABI rejects fp32)")
    p = problem(case)
    r = Run(p)
    print(f"head dim backward {_id(case)} dq={dq_algo} full={full}", flush=True)
    d = r.dev
    plan = r.plan(dq_algo=dq_algo)
    dq, dk, dv = (torch.full_like(d[n], 5.0) for n in ("q", "k", "v"))
    (plan.run_full if full else plan.run)(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], dq, dk, dv)
    torch.cuda.synchronize()
    rdq, rdk, rdv = r.oracle_backward()
    for n, g, ref in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert_close(n, to_host(g), ref, p.dtype)


# strided layouts: (dtype, B, H, S, D, varlen lengths) with packed QKV rows
STRIDE_CASES = [
    ("bf16", 2, 3, 260, 128, None),
    ("bf16", 1, 4, 333, 64, None),
    ("f16", 2, 2, 200, 72, None),
    ("bf16", 0, 2, 0, 128, (1, 64, 300, 129)),
    ("f32", 1, 2, 150, 64, None),
]


def _strideid(c):
    dt, b, h, s, d, lens = c
    return f"{dt}-{'lens' + '-'.join(map(str, lens)) if lens else f'b{b}s{s}'}-h{h}-d{d}"


@pytest.mark.parametrize("dq_algo", ["stored_ds", "separate", "atomic"])
@pytest.mark.parametrize("case", STRIDE_CASES, ids=_strideid)
def test_strided_layouts_match_contiguous_bitwise(case, dq_algo):
    """Q, K, V as views of one packed [.., S, 3, H, D] tensor, dO head-major
    ([B, H, S, D] permuted), O in a row-padded buffer, dQ/dK/dV written into
    a packed gradient tensor: every output equals the contiguous run's bit
    for bit (the kernels only address differently), the padding and the
    other slots of the packed outputs are untouched, and dQ/dK/dV match the
    oracle."""
    dt, b, h, s_len, d, lens = case
    if dq_algo == "stored_ds" and dt == "f32":
        pytest.skip("the stored-dS mode is for 16-bit types only (the ABI rejects fp32)")
    causal = True
    p = small_problem(dt, b, h, h, s_len, s_len, d, causal, 61, lengths=lens, deterministic=dq_algo == "atomic")
    r = Run(p, oracle_o_lse=False)
    print(f"strided {_strideid(case)} dq={dq_algo}", flush=True)
    dev, kw = r.dev, r.kw()
    varlen = lens is not None
    # contiguous reference run
    o_c, lse_c = api.forward(dev["q"], dev["k"], dev["v"], p.scale, causal, **kw)
    plan_c = api.BackwardPlan(dev["q"], dev["k"], p.scale, causal, p.deterministic, dq_algo=dq_algo, **kw)
    ref = [torch.empty_like(dev[n]) for n in ("q", "k", "v")]
    plan_c.run_full(dev["q"], dev["k"], dev["v"], o_c, dev["do"], lse_c, *ref)
    # strided copies of the same values
    lead = dev["q"].shape[:-2]                 # (B, S) or (T,)
    nl = len(lead)
    qkv = torch.empty(*lead, 3, h, d, dtype=dev["q"].dtype, device="cuda")
    for slot, n in enumerate(("q", "k", "v")):
        qkv.select(nl, slot).copy_(dev[n])
    q, k, v = (qkv.select(nl, slot) for slot in range(3))
    do_hm = dev["do"].movedim(nl, 0).contiguous()   # [H, B, S, D] or [H, T, D]
    do = do_hm.movedim(0, nl)
    sentinel = -3.0
    o_pad = torch.full((*lead, h, d + 8), sentinel, dtype=dev["q"].dtype, device="cuda")
    o = o_pad[..., :d]
    lse = torch.empty_like(lse_c)
    api.forward(q, k, v, p.scale, causal, out=(o, lse), **kw)
    dqkv = torch.full((*lead, 3, h, d), sentinel, dtype=dev["q"].dtype, device="cuda")
    grads = [dqkv.select(nl, slot) for slot in range(3)]
    plan = api.BackwardPlan(q, k, p.scale, causal, p.deterministic, dq_algo=dq_algo, **kw)
    plan.run_full(q, k, v, o, do, lse, *grads)
    torch.cuda.synchronize()
    iview = torch.int16 if o_c.element_size() == 2 else torch.int32
    assert torch.equal(o.contiguous().view(iview), o_c.view(iview))
    assert torch.equal(lse, lse_c)
    assert bool((o_pad[..., d:] == sentinel).all())
    for n, g, c in zip(("dQ", "dK", "dV"), grads, ref):
        assert torch.equal(g.contiguous().view(iview), c.view(iview)), n
    # the three-call path through the same strided views
    grads3 = [torch.full_like(dev[n], sentinel).movedim(nl, 0).contiguous().movedim(0, nl) for n in ("q", "k", "v")]
    plan.run(q, k, v, o, do, lse, *grads3)
    torch.cuda.synchronize()
    for n, g, c in zip(("dQ", "dK", "dV"), grads3, ref):
        assert torch.equal(g.contiguous().view(iview), c.view(iview)), n + " (three calls)"
    # and the oracle, from the strided run's own O and LSE
    r.set_o_lse(to_host(o.contiguous()), lse.cpu().numpy().astype(np.float64))
    rdq, rdk, rdv = r.oracle_backward()
    for n, g, rr in (("dQ", grads[0], rdq), ("dK", grads[1], rdk), ("dV", grads[2], rdv)):
        assert_close(n, to_host(g.contiguous()), rr, p.dtype)


# elementwise bias + dBias: (dtype, B, Hq, Hkv, Sq, Sk, D, causal, lengths, window, broadcast)
BIAS_CASES = [
    ("bf16", 2, 3, 3, 200, 200, 128, True, None, None, None),
    ("bf16", 1, 4, 2, 170, 260, 64, False, None, None, "heads"),     # one bias for every q-head
    ("bf16", 2, 2, 2, 130, 130, 64, True, None, None, "batch"),      # one bias for every batch entry
    ("f16", 1, 2, 2, 300, 300, 128, True, None, (50, -1), None),
    ("f32", 1, 2, 2, 150, 200, 64, True, None, None, None),
    ("bf16", 0, 4, 2, 0, 0, 128, True, (1, 64, 300), None, None),    # varlen
]


def _biasid(c):
    bc = f"-bcast_{c[10]}" if c[10] else ""
    w = f"-w{c[9][0]}/{c[9][1]}" if c[9] else ""
    return f"{_id(c[:9])}{w}{bc}"


@pytest.mark.parametrize("algo", ["atomic", "separate", "stored_ds"])
@pytest.mark.parametrize("full", [False, True], ids=["three_calls", "bwd_full"])
@pytest.mark.parametrize("case", BIAS_CASES, ids=_biasid)
def test_bias_and_dbias_match_oracle(case, full, algo):
    """O and LSE with the bias, dQ/dK/dV and dBias = dS against the oracle in
    every dQ mode; dBias outside each sequence's block keeps its contents.
    Outside the atomic mode bias rows are 16-byte aligned: the bias is a view
    of rows padded to a multiple of 8 keys."""
    import datagen
    p = problem(case[:9])
    if algo == "stored_ds" and p.dtype == "f32":
        pytest.skip("the stored-dS mode is for 16-bit types")
    win, bcast = case[9], case[10]
    r = Run(p, oracle_o_lse=False, window=win)
    nb = len(case[8]) if case[8] else case[1]
    bias_np = datagen.draw_bias(p, 91, heads=1 if bcast == "heads" else None, batch=1 if bcast == "batch" else nb)
    bias_dev = to_dev(bias_np, p.dtype)
    if algo != "atomic":
        skp = (p.seqlen_k + 7) // 8 * 8
        padded = torch.full(bias_dev.shape[:3] + (skp,), float("nan"), dtype=bias_dev.dtype, device="cuda")
        padded[..., :p.seqlen_k] = bias_dev
        bias_dev = padded[..., :p.seqlen_k]
    bias_dev = bias_dev.expand(nb, p.heads_q, p.seqlen_q, p.seqlen_k)
    bias_full = np.broadcast_to(bias_np, (nb, p.heads_q, p.seqlen_q, p.seqlen_k))
    print(f"bias {_biasid(case)} full={full} algo={algo}", flush=True)
    d, kw = r.dev, r.kw()
    cq, ck = r.cu_np
    o, lse = api.forward(d["q"], d["k"], d["v"], p.scale, p.causal, window=win, bias=bias_dev, **kw)
    torch.cuda.synchronize()
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal, cq, ck, window=win, bias=bias_full)
    assert_close("O", to_host(o), ro, p.dtype)
    fin = np.isfinite(rlse)
    g = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isfinite(g), fin)
    assert np.max(np.abs(g[fin] - rlse[fin]), initial=0) <= (1e-4 if p.dtype == "f32" else 2e-4)
    # backward from the oracle's O and LSE
    r.set_o_lse(ro, rlse)
    sentinel = 9.0
    dbias = torch.full((nb, p.heads_q, p.seqlen_q, p.seqlen_k), sentinel, dtype=d["q"].dtype, device="cuda")
    plan = api.BackwardPlan(d["q"], d["k"], p.scale, p.causal, False, dq_algo=algo, window=win,
                            bias=bias_dev, dbias=dbias, **kw)
    dq, dk, dv = (torch.empty_like(d[n]) for n in ("q", "k", "v"))
    (plan.run_full if full else plan.run)(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], dq, dk, dv)
    torch.cuda.synchronize()
    rdq, rdk, rdv, rdb = oracle.backward(r.x["q"], r.x["k"], r.x["v"], r.o, r.x["do"], r.lse, p.scale, p.causal,
                                         cq, ck, window=win, bias=bias_full, want_dbias=True)
    for n, gg, ref in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert_close(n, to_host(gg), ref, p.dtype)
    gdb = to_host(dbias)
    inside = np.zeros(gdb.shape, bool)
    lq = [cq[i + 1] - cq[i] for i in range(nb)] if cq is not None else [p.seqlen_q] * nb
    lk = [ck[i + 1] - ck[i] for i in range(nb)] if ck is not None else [p.seqlen_k] * nb
    for bb in range(nb):
        inside[bb, :, :lq[bb], :lk[bb]] = True
    assert_close("dBias", gdb[inside], rdb[inside], p.dtype)
    assert np.all(gdb[~inside] == sentinel)


# (dtype, Hq, Hkv, Sq, Sk, D, causal, element offset of the bias view, padded row length)
FWD_BIAS_LAYOUTS = [
    ("bf16", 4, 2, 200, 261, 128, True, 1, 265),    # odd base offset and row stride
    ("f16", 2, 2, 150, 77, 64, False, 0, 80),       # aligned rows, ragged 4-key tail
    ("bf16", 2, 1, 130, 130, 64, True, 2, 134),     # 4-byte aligned base, stride 2 mod 4
    ("f16", 3, 3, 97, 300, 128, False, 3, 303),
]


@pytest.mark.parametrize("case", FWD_BIAS_LAYOUTS, ids=lambda c: f"{c[0]}-s{c[3]}x{c[4]}-d{c[5]}-off{c[7]}-row{c[8]}")
def test_bias_forward_any_row_layout_matches_oracle(case):
    """The forward reads a bias whose rows start anywhere (base and row
    stride not multiples of 4 elements) one element at a time and aligned
    rows four keys per load; no element past a row's keys is read (the
    padding holds NaN, which would reach O)."""
    import datagen
    dt, hq, hkv, sq, sk, d, causal, off, row = case
    p = small_problem(dt, 2, hq, hkv, sq, sk, d, causal, 4100 + off)
    r = Run(p, oracle_o_lse=False)
    bias_np = datagen.draw_bias(p, 97, batch=2)
    big = torch.full((2, hq, sq, row), float("nan"), dtype=to_dev(bias_np[:1, :1, :1], dt).dtype, device="cuda")
    big[..., off:off + sk] = to_dev(bias_np, dt)
    bias_dev = big[..., off:off + sk]
    print(f"forward bias layout {case}", flush=True)
    d_ = r.dev
    o, lse = api.forward(d_["q"], d_["k"], d_["v"], p.scale, p.causal, bias=bias_dev)
    torch.cuda.synchronize()
    ro, rlse = oracle.forward(r.x["q"], r.x["k"], r.x["v"], p.scale, p.causal, bias=bias_np)
    assert_close("O", to_host(o), ro, p.dtype)
    fin = np.isfinite(rlse)
    g = lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isfinite(g), fin)
    assert np.max(np.abs(g[fin] - rlse[fin]), initial=0) <= 2e-4


SEQUSED_CASES = [
    # (dtype, Hq, Hkv, D, causal, lengths_q, lengths_k, used_q, used_k)
    ("bf16", 4, 2, 128, True, (70, 300, 129, 1), (90, 260, 129, 40), (70, 211, 0, 1), (33, 260, 100, 40)),
    ("bf16", 2, 2, 64, False, (200, 65, 130), (150, 300, 130), (199, 1, 130), (150, 129, 64)),
    ("f16", 4, 1, 128, True, (257, 40), (257, 300), (250, 40), (257, 170)),
    # a sequence with no used keys (its rows: LSE -inf, O = dQ = 0) and an
    # empty sequence (cu_seqlens repeats an offset) between two others
    ("bf16", 2, 2, 128, True, (100, 0, 64), (120, 0, 200), (100, 0, 64), (0, 0, 150)),
]


def _sequsedid(c):
    dt, hq, hkv, d, causal, lq, lk, uq, uk = c
    return f"{dt}-h{hq}/{hkv}-d{d}-{'causal' if causal else 'full'}-uq{'-'.join(map(str, uq))}-uk{'-'.join(map(str, uk))}"


@pytest.mark.parametrize("full", [False, True], ids=["three_calls", "bwd_full"])
@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds", "atomic"])
@pytest.mark.parametrize("case", SEQUSED_CASES, ids=_sequsedid)
def test_seqused_matches_oracle_and_leaves_unused_rows(case, dq_algo, full):
    """Varlen with used lengths: the used rows of O, LSE, dQ, dK, dV match the
    oracle; every row past a used length keeps what the buffer held (through
    the three calls and through attn_bwd_full)."""
    import datagen
    from _harness import TORCH_DTYPE, to_dev
    dt, hq, hkv, d, causal, lq, lk, uq, uk = case
    p = datagen.Problem(dt, len(lq), hq, hkv, max(lq), max(lk), d, causal, 1 / math.sqrt(d), 77,
                        lengths_q=tuple(lq), lengths_k=tuple(lk), name="seqused")
    x = datagen.draw(p)
    cq, ck = p.cu_seqlens()
    uq_np, uk_np = np.array(uq, np.int32), np.array(uk, np.int32)
    dev = {n: to_dev(v, dt) for n, v in x.items()}
    cu = dict(cu_seqlens_q=torch.from_numpy(cq).cuda(), cu_seqlens_k=torch.from_numpy(ck).cuda(),
              max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k,
              seqused_q=torch.from_numpy(uq_np).cuda(), seqused_k=torch.from_numpy(uk_np).cuda())
    used_q = np.zeros(cq[-1], bool)
    used_k = np.zeros(ck[-1], bool)
    for b in range(len(lq)):
        used_q[cq[b]:cq[b] + uq[b]] = True
        used_k[ck[b]:ck[b] + uk[b]] = True
    print(f"seqused {_sequsedid(case)} dq={dq_algo} full={full}", flush=True)
    sentinel = 3.0
    # forward: used rows against the oracle, unused rows untouched
    o_buf = torch.full_like(dev["q"], sentinel)
    lse_buf = torch.full((hq, cq[-1]), sentinel, dtype=torch.float32, device="cuda")
    api.forward(dev["q"], dev["k"], dev["v"], p.scale, causal, out=(o_buf, lse_buf), **cu)
    torch.cuda.synchronize()
    ro, rlse = oracle.forward(x["q"], x["k"], x["v"], p.scale, causal, cq, ck, uq_np, uk_np)
    go = to_host(o_buf)
    assert_close("O", go[used_q], ro[used_q], dt)
    assert np.all(go[~used_q] == sentinel)
    gl = lse_buf.cpu().numpy().astype(np.float64)
    assert np.all(gl[:, ~used_q] == sentinel)
    fin = np.isfinite(rlse[:, used_q])
    assert np.array_equal(np.isfinite(gl[:, used_q]), fin)
    assert np.max(np.abs(gl[:, used_q][fin] - rlse[:, used_q][fin]), initial=0) <= 1e-4
    # backward with the oracle's O and LSE on the used rows
    o_in = round_like(np.where(used_q[:, None, None], ro, 0.0), dt)
    lse_in = np.where(used_q[None, :], rlse, 0.0).astype(np.float32)
    dev_o = to_dev(o_in, dt)
    dev_lse = torch.from_numpy(lse_in).cuda()
    plan = api.BackwardPlan(dev["q"], dev["k"], p.scale, causal, False, dq_algo=dq_algo, **cu)
    dq = torch.full_like(dev["q"], sentinel)
    dk = torch.full_like(dev["k"], sentinel)
    dv = torch.full_like(dev["v"], sentinel)
    runner = plan.run_full if full else plan.run
    runner(dev["q"], dev["k"], dev["v"], dev_o, dev["do"], dev_lse, dq, dk, dv)
    torch.cuda.synchronize()
    rdq, rdk, rdv = oracle.backward(x["q"], x["k"], x["v"], o_in, x["do"], lse_in.astype(np.float64), p.scale, causal,
                                    cq, ck, uq_np, uk_np)
    for n, g, ref, used in (("dQ", dq, rdq, used_q), ("dK", dk, rdk, used_k), ("dV", dv, rdv, used_k)):
        gh = to_host(g)
        assert_close(n, gh[used], ref[used], dt)
        assert np.all(gh[~used] == sentinel), f"{n}: a row past the used length was written"
