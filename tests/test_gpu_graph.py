"""HIP graph capture of the backward: attn_bwd_preprocess + attn_bwd_full
captured on the current stream (the separate mode forks its dQ kernel onto
the library's side stream and joins it back inside the capture), replayed
several times with eager work and synchronisations between the replays;
every replay must reproduce the eager call bit for bit (both modes are
deterministic: no atomics)."""

import numpy as np
import pytest
import torch

import datagen
from exact_attention_backward_amd import api

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds"])
def test_captured_backward_replays_match_eager(dq_algo):
    p = datagen.Problem("bf16", 2, 4, 2, 300, 300, 64, True, 1 / 8, 17, name="graph")
    x = datagen.draw(p)
    dev = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    o, lse = api.forward(dev["q"], dev["k"], dev["v"], p.scale, p.causal)
    plan = api.BackwardPlan(dev["q"], dev["k"], p.scale, p.causal, False, dq_algo=dq_algo)
    outs = [torch.empty_like(dev[n]) for n in ("q", "k", "v")]
    args = (dev["q"], dev["k"], dev["v"], o, dev["do"], lse)
    print(f"graph capture {dq_algo}", flush=True)
    plan.run_full(*args, *outs)   # eager (also creates the side stream before any capture)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on a non-default stream, as capture requires
        plan.run_full(*args, *outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run_full(*args, *outs)
    torch.cuda.synchronize()

    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        for t in outs:
            t.fill_(7.0)
        scratch.mul_(1.0001).add_(0.5)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, a, b in zip(("dQ", "dK", "dV"), outs, ref):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}: {n}"
    assert np.isfinite(ref[0].float().cpu().numpy()).all()
