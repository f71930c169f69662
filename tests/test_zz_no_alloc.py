"""attn_bwd_full_noalloc (D and the workspace in the library's fixed scratch
memory) against attn_bwd_preprocess + attn_bwd_full with a workspace the
caller allocates, through the C ABI, on two calls in a row, the second with
a smaller problem (the scratch keeps the first call's contents).  Bitwise
equal in the modes that fix their summation order; within the parity
tolerance in the plain atomic mode.  Both are also checked against the
oracle."""

import numpy as np
import pytest
import torch

from _harness import Run, assert_close, small_problem, to_host
from exact_attention_backward_amd import api

pytestmark = pytest.mark.gpu

# (dtype, dq_algo, deterministic) and two problems per case: (B, Hq, Hkv, S, D, causal, lengths)
CASES = [
    ("bf16", "separate", False),
    ("bf16", "stored_ds", False),
    ("f16", "stored_ds", False),
    ("bf16", "atomic", True),
    ("bf16", "atomic", False),
    ("f32", "separate", False),
    ("f32", "atomic", True),
]
PROBLEMS = [
    (2, 4, 2, 333, 128, True, None),
    (1, 2, 1, 100, 64, False, None),
]
VARLEN = [
    (3, 4, 4, 0, 128, True, (300, 1, 170)),
    (2, 2, 1, 0, 64, True, (65, 40)),
]


def _run_pair(r, dq_algo, det):
    d = r.dev
    p = r.p
    # reference: the existing two-call path with a caller-allocated workspace
    plan = r.plan(det, dq_algo)
    ref = [torch.full_like(d["q"], 7.0), torch.empty_like(d["k"]), torch.empty_like(d["v"])]
    plan.run_full(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], *ref)
    torch.cuda.synchronize()
    # the no-allocation entry point
    got = [torch.full_like(d["q"], 7.0), torch.empty_like(d["k"]), torch.empty_like(d["v"])]
    api.attn_bwd_full_noalloc(plan.shape, d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], *got)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype,dq_algo,det", CASES)
@pytest.mark.parametrize("problems", [PROBLEMS, VARLEN], ids=["dense", "varlen"])
def test_noalloc_matches_full(dtype, dq_algo, det, problems):
    exact = dq_algo != "atomic" or det
    for i, (b, hq, hkv, s, dd, causal, lengths) in enumerate(problems):
        p = small_problem(dtype, b, hq, hkv, s, s, dd, causal, seed=40 + i, lengths=lengths, deterministic=det)
        print(f"noalloc case {dtype} {dq_algo} det={det} call {i}: {p.name} lengths={lengths}", flush=True)
        r = Run(p)
        ref, got = _run_pair(r, dq_algo, det)
        for name, a, b_ in zip(("dQ", "dK", "dV"), got, ref):
            if exact:
                assert torch.equal(a.view(torch.int16 if a.element_size() == 2 else torch.int32),
                                   b_.view(torch.int16 if b_.element_size() == 2 else torch.int32)), \
                    f"{name} differs bitwise from attn_bwd_full (call {i})"
            else:
                assert_close(name + " vs attn_bwd_full", to_host(a), to_host(b_), dtype)
        rdq, rdk, rdv = r.oracle_backward()
        for name, a, ref_np in zip(("dQ", "dK", "dV"), got, (rdq, rdk, rdv)):
            assert_close(name, to_host(a), ref_np, dtype)


def test_noalloc_rejects_problems_larger_than_the_scratch():
    q = torch.zeros(4, 4096, 16, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros_like(q)
    lse = torch.zeros(4, 16, 4096, dtype=torch.float32, device="cuda")
    shape = api.make_shape(q, k, 0.1, True, dq_algo="stored_ds")
    with pytest.raises(api.L.AttnError) as e:
        api.attn_bwd_full_noalloc(shape, q, k, k, q, q, lse, q, k, k)
    assert e.value.status == api.L.ATTN_ERR_SCRATCH
