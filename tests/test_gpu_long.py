"""Long context: B=1, H=8, S=65536, D=128, bf16, causal, in both atomic-free
dQ modes (the stored-dS mode under a workspace cap that runs its kv-heads in
chunks of two).  The fp64 oracle cannot hold the 65536 x 65536 matrices, so
one head is checked on sampled outputs: its O and LSE come from the oracle's
row-blocked forward, and dQ at sampled query rows and dK, dV at sampled keys
from the oracle's sampled backward (each from its definition); the other
heads take the library forward's O and LSE and are not compared."""

import math

import numpy as np
import pytest
import torch

import datagen
import oracle
from _harness import TOL, rel_err, round_like, to_dev, to_host
from exact_attention_backward_amd import api

pytestmark = pytest.mark.gpu

S, H, D, HEAD = 65536, 8, 128, 5
ROWS = [0, 1, 127, 128, 4095, 20000, 32767, 32768, 50001, 65534, 65535]
KEYS = [0, 1, 126, 127, 128, 9999, 32768, 60000, 65407, 65408, 65535]


@pytest.fixture(scope="module")
def case():
    p = datagen.Problem("bf16", 1, H, H, S, S, D, True, 1 / math.sqrt(D), 91, name="long_context")
    x = datagen.draw(p)
    print("long context: oracle forward of one head (row-blocked)", flush=True)
    q, k, v = (x[n][0, :, HEAD] for n in ("q", "k", "v"))
    o, lse = oracle.head_forward_rows(q, k, v, p.scale, True, block=2048)
    o = round_like(o, "bf16")
    lse = lse.astype(np.float32).astype(np.float64)
    dev = {n: to_dev(x[n], "bf16") for n in ("q", "k", "v", "do")}
    go, glse = api.forward(dev["q"], dev["k"], dev["v"], p.scale, True)
    go[0, :, HEAD] = to_dev(o, "bf16")
    glse[0, HEAD] = torch.from_numpy(lse.astype(np.float32)).cuda()
    dev["o"], dev["lse"] = go, glse
    rdq, rdk, rdv = oracle.head_backward_rows(q, k, v, o, x["do"][0, :, HEAD], lse, p.scale, True, ROWS, KEYS)
    return p, dev, (rdq, rdk, rdv)


@pytest.mark.parametrize("dq_algo,cap", [("separate", 0), ("stored_ds", 12 << 30)])
def test_long_context_sampled_parity(case, dq_algo, cap):
    p, d, (rdq, rdk, rdv) = case
    plan = api.BackwardPlan(d["q"], d["k"], p.scale, True, dq_algo=dq_algo, max_workspace_bytes=cap)
    print(f"long context {dq_algo}: workspace {plan.workspace.numel() / 2**30:.2f} GiB", flush=True)
    if dq_algo == "stored_ds":
        assert plan.workspace.numel() <= cap
    dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
    plan.run_full(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], dq, dk, dv)
    torch.cuda.synchronize()
    got = (to_host(dq[0, ROWS, HEAD]), to_host(dk[0, KEYS, HEAD]), to_host(dv[0, KEYS, HEAD]))
    for n, g, ref in zip(("dQ", "dK", "dV"), got, (rdq, rdk, rdv)):
        e = rel_err(g, ref)
        print(f"  {n} sampled rel err {e:.3e}", flush=True)
        assert e <= TOL["bf16"], f"{n}: {e:.3e}"
