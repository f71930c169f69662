"""The stored-dS workspace: exact sizing from host copies of cu_seqlens, the
bound without them, the caller's cap (kv-head groups in chunks, or the
separate mode when not one group fits).  Every variant must give the results
of the uncapped, exactly sized run bit for bit (the modes fix their summation
order), and match the fp64 oracle."""

import numpy as np
import pytest
import torch

from _harness import Run, assert_close, small_problem, to_host
from exact_attention_backward_amd import api

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def _run(r, plan, full):
    d = r.dev
    out = [torch.full_like(d["q"], 3.0), torch.full_like(d["k"], 3.0), torch.full_like(d["v"], 3.0)]
    if full:
        plan.run_full(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], *out)
    else:
        plan.run(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], *out)
    torch.cuda.synchronize()
    return out


def _plan(r, dq_algo="stored_ds", **kw):
    d = r.dev
    return api.BackwardPlan(d["q"], d["k"], r.p.scale, r.p.causal, dq_algo=dq_algo, window=r.window, **r.kw(), **kw)


CASES = [
    # dtype, B, Hq, Hkv, S, D, causal, lengths, window
    ("bf16", 2, 8, 4, 333, 128, True, None, None),
    ("bf16", 0, 8, 4, 0, 128, True, (1, 300, 77, 513, 129), None),
    ("f16", 0, 6, 3, 0, 64, True, (200, 65, 31, 400), None),
    ("bf16", 0, 4, 4, 0, 64, False, (100, 260, 3), (70, 20)),
    ("bf16", 1, 4, 2, 700, 128, True, None, (300, -1)),
]


def _id(c):
    dt, b, hq, hkv, s, d, causal, lens, win = c
    shape = f"lens{'-'.join(map(str, lens))}" if lens else f"b{b}s{s}"
    return f"{dt}-{shape}-h{hq}/{hkv}-d{d}-{'causal' if causal else 'full'}-w{win}"


@pytest.mark.parametrize("full", [True, False], ids=["bwd_full", "three_calls"])
@pytest.mark.parametrize("case", CASES, ids=_id)
def test_sizing_and_cap_variants_agree_bitwise(case, full):
    dt, b, hq, hkv, s, d, causal, lens, win = case
    p = small_problem(dt, b, hq, hkv, s, s, d, causal, 77, lengths=lens)
    r = Run(p, window=win)
    print(f"workspace variants {_id(case)} full={full}", flush=True)
    ref_plan = _plan(r)
    ref = _run(r, ref_plan, full)
    exact = ref_plan.workspace.numel()
    variants = {}
    if lens is not None:
        variants["bound (no host offsets)"] = _plan(r, host_offsets=False)
        assert variants["bound (no host offsets)"].workspace.numel() >= exact
    # caps: one kv-head group per launch, hkv - 1 per launch, and below one group
    sep_bytes = _plan(r, dq_algo="separate").workspace.numel()
    per_group = None
    for chunk in (1, hkv - 1):
        if chunk < 1:
            continue
        # find the cap that allows exactly `chunk` groups: the workspace is
        # base + chunk * per_group, with base + hkv * per_group = exact
        if per_group is None:
            one = _plan(r, max_workspace_bytes=exact - 1)     # hkv - 1 groups fit
            per_group = exact - one.workspace.numel()
            assert per_group > 0
        cap = exact - (hkv - chunk) * per_group
        pl = _plan(r, max_workspace_bytes=cap)
        assert pl.workspace.numel() == cap
        variants[f"cap {chunk} group(s)"] = pl
    fb = _plan(r, max_workspace_bytes=exact - hkv * per_group - 1)
    assert fb.workspace.numel() == sep_bytes
    for name, pl in variants.items():
        got = _run(r, pl, full)
        for n, a, e in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(_bits(a), _bits(e)), f"{name}: {n} differs from the exactly sized run"
    # the fallback is the separate mode, bit for bit
    got = _run(r, fb, full)
    sep = _run(r, _plan(r, dq_algo="separate"), full)
    for n, a, e in zip(("dQ", "dK", "dV"), got, sep):
        assert torch.equal(_bits(a), _bits(e)), f"fallback: {n} differs from the separate mode"
    rdq, rdk, rdv = r.oracle_backward()
    for n, g, ref_np in (("dQ", ref[0], rdq), ("dK", ref[1], rdk), ("dV", ref[2], rdv)):
        assert_close(n, to_host(g), ref_np, dt)
