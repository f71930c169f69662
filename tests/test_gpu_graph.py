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


@pytest.mark.parametrize("bias", [False, True], ids=["plain", "bias_dbias"])
@pytest.mark.parametrize("dropout", [False, True], ids=["no_dropout", "dropout"])
@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds"])
def test_captured_backward_replays_match_eager(dq_algo, dropout, bias):
    """With bias and dBias the clear of dBias's masked elements is captured too;
    with dropout every replay draws the same keep mask (fixed seed and offset)."""
    p = datagen.Problem("bf16", 2, 4, 2, 300, 300, 64, True, 1 / 8, 17, name="graph")
    x = datagen.draw(p)
    dev = {k: torch.from_numpy(v).to(torch.bfloat16).cuda() for k, v in x.items()}
    kw = {}
    dbias = None
    if bias:
        # rows padded to a multiple of 8 keys: 16-byte aligned rows, as the
        # atomic-free modes require of the bias
        bpad = torch.zeros((p.batch, p.heads_q, p.seqlen_q, 304), dtype=torch.bfloat16, device="cuda")
        bpad[..., :p.seqlen_k] = torch.from_numpy(datagen.draw_bias(p, 5)).to(torch.bfloat16).cuda()
        dbias = torch.full_like(bpad, 7.0)[..., :p.seqlen_k]
        kw = dict(bias=bpad[..., :p.seqlen_k], dbias=dbias)
    if dropout:
        kw["dropout"] = (0.2, 0x1234ABCD, 7)
    o, lse = api.forward(dev["q"], dev["k"], dev["v"], p.scale, p.causal, bias=kw.get("bias"),
                         dropout=kw.get("dropout"))
    plan = api.BackwardPlan(dev["q"], dev["k"], p.scale, p.causal, False, dq_algo=dq_algo, **kw)
    outs = [torch.empty_like(dev[n]) for n in ("q", "k", "v")] + ([dbias] if bias else [])
    args = (dev["q"], dev["k"], dev["v"], o, dev["do"], lse)
    print(f"graph capture {dq_algo} bias={bias} dropout={dropout}", flush=True)
    grads = outs[:3]
    plan.run_full(*args, *grads)   # eager (also creates the side stream before any capture)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up on a non-default stream, as capture requires
        plan.run_full(*args, *grads)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run_full(*args, *grads)
    torch.cuda.synchronize()

    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        for t in outs:
            t.fill_(7.0)
        scratch.mul_(1.0001).add_(0.5)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, a, b in zip(("dQ", "dK", "dV", "dBias"), outs, ref):
            assert torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16)), f"replay {rep}: {n}"
    assert np.isfinite(ref[0].float().cpu().numpy()).all()
