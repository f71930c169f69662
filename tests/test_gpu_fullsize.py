"""Parity at the five workloads' full sizes, in the launch configuration the
benchmark times (attn_bwd_preprocess -> attn_bwd_full).

Every (sequence, kv-head) group of every workload is compared element by
element with the fp64 oracle (run in worker processes): the two small
workloads directly; for the three large ones O and LSE of every head come from
the oracle forward (rounded to the I/O type and fp32, written into the device
buffers) and dQ, dK and dV of every group from the oracle backward.  Extra
configurations of the headline shape (a window with ALiBi, packed QKV) are
checked on sampled groups plus the identity sum_j dV_j = sum_i dO_i over every
head.  The deterministic and atomic-free modes are checked bit for bit across
repeated runs."""

import numpy as np
import pytest
import torch

import datagen
import oracle
from _harness import TOL, assert_close, oracle_all_groups, rel_err, round_like, to_dev, to_host

pytestmark = pytest.mark.gpu


def setup(p):
    x = datagen.draw(p)
    dt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[p.dtype]
    dev = {k: torch.from_numpy(v).to(dt).cuda() for k, v in x.items()}
    kw, cu = {}, (None, None)
    if p.varlen:
        cu = p.cu_seqlens()
        kw = dict(cu_seqlens_q=torch.from_numpy(cu[0]).cuda(), cu_seqlens_k=torch.from_numpy(cu[1]).cuda(),
                  max_seqlen_q=p.seqlen_q, max_seqlen_k=p.seqlen_k)
    return x, dev, kw, cu


def run_backward(p, dev, o, lse, kw, deterministic=None, dq_algo="separate", extra=None):
    from exact_attention_backward_amd import api
    det = p.deterministic if deterministic is None else deterministic
    plan = api.BackwardPlan(dev["q"], dev["k"], p.scale, p.causal, det, dq_algo=dq_algo, **kw, **(extra or {}))
    dq, dk, dv = torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"])
    # the two calls the benchmark times: attn_bwd_preprocess, attn_bwd_full
    plan.run_full(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, dq, dk, dv)
    torch.cuda.synchronize()
    if det:
        assert plan.error_flag() == 0
    return dq, dk, dv


def sampled_check(p, samples, deterministic=None, repeats=1, dq_algo="separate", window=None, alibi=None,
                  packed=False):
    """samples: list of (sequence, kv_head).  window / alibi (slopes, one per
    q-head): local mask and ALiBi on both sides; packed: Q, K, V as views of
    one [B, S, 3, H, D] tensor (dense, Hq == Hkv)."""
    from exact_attention_backward_amd import api
    x, dev, kw, cu = setup(p)
    if packed:
        qkv = torch.empty(p.batch, p.seqlen_q, 3, p.heads_q, p.head_dim, dtype=dev["q"].dtype, device="cuda")
        for slot, n in enumerate(("q", "k", "v")):
            qkv[:, :, slot].copy_(dev[n])
            dev[n] = qkv[:, :, slot]
    slopes = None if alibi is None else np.asarray(alibi, np.float32)
    extra = dict(window=window, alibi_slopes=None if slopes is None else torch.from_numpy(slopes).cuda())
    print(f"{p.name}: inputs ready", flush=True)
    o, lse = api.forward(dev["q"], dev["k"], dev["v"], p.scale, p.causal, **kw, **extra)
    torch.cuda.synchronize()
    g = p.heads_q // p.heads_kv
    ranges = []
    for b, hk in samples:
        if p.varlen:
            q0, q1 = int(cu[0][b]), int(cu[0][b + 1])
        else:
            q0, q1 = b * p.seqlen_q, (b + 1) * p.seqlen_q
        ranges.append((q0, q1))
        fw = oracle.group_forward(x["q"], x["k"], x["v"], p.scale, p.causal, b, hk, *cu, window=window,
                                  alibi_slopes=slopes)
        for h, (oh, lh) in fw.items():
            oh = round_like(oh, p.dtype).astype(np.float32)
            lh = lh.astype(np.float32)
            if p.varlen:
                o[q0:q1, h] = torch.from_numpy(oh).to(o.dtype).cuda()
                lse[h, q0:q1] = torch.from_numpy(lh).cuda()
            else:
                o[b, :, h] = torch.from_numpy(oh).to(o.dtype).cuda()
                lse[b, h] = torch.from_numpy(lh).cuda()
    torch.cuda.synchronize()
    outs = [run_backward(p, dev, o, lse, kw, deterministic, dq_algo, extra) for _ in range(repeats)]
    print(f"{p.name}: backward done", flush=True)
    for rep in outs[1:]:
        for a, bb in zip(outs[0], rep):
            assert torch.equal(a.view(torch.int16), bb.view(torch.int16)), "deterministic mode not reproducible"
    dq, dk, dv = outs[0]
    o_h = to_host(o)
    lse_h = lse.cpu().numpy().astype(np.float64)
    for (b, hk), (q0, q1) in zip(samples, ranges):
        rdq, rdk, rdv = oracle.group_backward(x["q"], x["k"], x["v"], o_h, x["do"], lse_h, p.scale, p.causal, b, hk,
                                              *cu, window=window, alibi_slopes=slopes)
        if p.varlen:
            k0, k1 = int(cu[1][b]), int(cu[1][b + 1])
            gk, gv = to_host(dk[k0:k1, hk]), to_host(dv[k0:k1, hk])
            gq = {h: to_host(dq[q0:q1, h]) for h in rdq}
        else:
            gk, gv = to_host(dk[b, :, hk]), to_host(dv[b, :, hk])
            gq = {h: to_host(dq[b, :, h]) for h in rdq}
        errs = {"dK": rel_err(gk, rdk), "dV": rel_err(gv, rdv)}
        errs.update({f"dQ[h{h}]": rel_err(gq[h], rdq[h]) for h in rdq})
        print(f"{p.name} seq {b} kv-head {hk}: {errs}", flush=True)
        for n, e in errs.items():
            assert e <= TOL[p.dtype], f"{n}: {e:.3e}"
    # sum_j dV_j = sum of dO over rows that see a key, for every (sequence, kv-head)
    dv_h, do_h = to_host(dv), x["do"].astype(np.float64)
    if p.varlen:
        for b in range(p.batch):
            q0, q1 = int(cu[0][b]), int(cu[0][b + 1])
            k0, k1 = int(cu[1][b]), int(cu[1][b + 1])
            lhs = dv_h[k0:k1].sum(axis=0)                                  # [Hkv, D]
            rhs = do_h[q0:q1].reshape(q1 - q0, p.heads_kv, g, p.head_dim).sum(axis=(0, 2))
            assert rel_err(lhs, rhs) <= TOL[p.dtype]
    else:
        lhs = dv_h.sum(axis=1)                                             # [B, Hkv, D]
        rhs = do_h.reshape(p.batch, p.seqlen_q, p.heads_kv, g, p.head_dim).sum(axis=(1, 3))
        assert rel_err(lhs, rhs) <= TOL[p.dtype]


_ALL = {}


def all_groups_check(name, dq_algo, deterministic=False, repeats=1):
    """Every (sequence, kv-head) group of workload `name` against the fp64
    oracle: O and LSE of every head from the oracle forward (rounded to the
    I/O type and fp32), the backward in the benchmark's launch configuration,
    dQ, dK and dV of every group compared element by element."""
    from exact_attention_backward_amd import api
    p = datagen.workload(name, deterministic=deterministic)
    x, dev, kw, cu = setup(p)
    if name not in _ALL:
        print(f"{p.name}: oracle on every group", flush=True)
        _ALL.clear()   # keep one workload's results at a time
        _ALL[name] = oracle_all_groups(p, x)
    ref = _ALL[name]
    g = p.heads_q // p.heads_kv
    o = torch.empty_like(dev["q"])
    lse = torch.empty((p.heads_q, p.total_q) if p.varlen else (p.batch, p.heads_q, p.seqlen_q), dtype=torch.float32,
                      device="cuda")
    o_np = np.zeros(dev["q"].shape, np.float32)
    lse_np = np.zeros(lse.shape, np.float32)
    for (b, hk), (heads, _, _) in ref.items():
        for j, (oh, lh, _) in enumerate(heads):
            h = hk * g + j
            if p.varlen:
                q0, q1 = int(cu[0][b]), int(cu[0][b + 1])
                o_np[q0:q1, h], lse_np[h, q0:q1] = oh, lh
            else:
                o_np[b, :, h], lse_np[b, h] = oh, lh
    o.copy_(torch.from_numpy(o_np).to(o.dtype))
    lse.copy_(torch.from_numpy(lse_np))
    outs = [run_backward(p, dev, o, lse, kw, deterministic, dq_algo) for _ in range(repeats)]
    for rep in outs[1:]:
        for a, bb in zip(outs[0], rep):
            assert torch.equal(a.view(torch.int16), bb.view(torch.int16)), "not bitwise reproducible"
    dq, dk, dv = (to_host(t) for t in outs[0])
    worst = {}
    for (b, hk), (heads, rdk, rdv) in ref.items():
        if p.varlen:
            q0, q1, k0, k1 = int(cu[0][b]), int(cu[0][b + 1]), int(cu[1][b]), int(cu[1][b + 1])
            gk, gv = dk[k0:k1, hk], dv[k0:k1, hk]
            gq = [dq[q0:q1, hk * g + j] for j in range(g)]
        else:
            gk, gv = dk[b, :, hk], dv[b, :, hk]
            gq = [dq[b, :, hk * g + j] for j in range(g)]
        errs = {"dK": rel_err(gk, rdk), "dV": rel_err(gv, rdv)}
        for j, (_, _, rdq) in enumerate(heads):
            errs[f"dQ{j}"] = rel_err(gq[j], rdq)
        for n, e in errs.items():
            worst[n[:2]] = max(worst.get(n[:2], 0.0), e)
            assert e <= TOL[p.dtype], f"seq {b} kv-head {hk} {n}: {e:.3e}"
    print(f"{p.name} {dq_algo}: {len(ref)} groups, worst rel err {worst}", flush=True)


@pytest.mark.parametrize("dq_algo", ["stored_ds", "separate"])
def test_headline_window_alibi_sampled(dq_algo):
    """The headline shape with a causal sliding window of 1024 keys and ALiBi."""
    slopes = [2.0 ** (-8.0 * (h + 1) / 16) for h in range(16)]
    sampled_check(datagen.workload("c3"), [(0, 0), (3, 15)], dq_algo=dq_algo, window=(1024, -1), alibi=slopes)


@pytest.mark.parametrize("dq_algo", ["stored_ds", "atomic"])
def test_headline_packed_qkv_sampled(dq_algo):
    """The headline shape with Q, K and V read from one packed [B, S, 3, H, D] tensor."""
    sampled_check(datagen.workload("c3"), [(1, 4)], dq_algo=dq_algo, packed=True)


def test_fp32_workload_full():
    p = datagen.workload("c1")
    x, dev, kw, cu = setup(p)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], p.scale, p.causal)
    o32, lse32 = o.astype(np.float32), lse.astype(np.float32)
    dq, dk, dv = run_backward(p, dev, torch.from_numpy(o32).cuda(), torch.from_numpy(lse32).cuda(), kw)
    rdq, rdk, rdv = oracle.backward(x["q"], x["k"], x["v"], o32, x["do"], lse32, p.scale, p.causal)
    for n, gg, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert_close(n, to_host(gg), r, "f32")


@pytest.mark.parametrize("dq_algo,deterministic",
                         [("separate", False), ("stored_ds", False), ("atomic", False), ("atomic", True)])
def test_bf16_causal_d64_workload_full(dq_algo, deterministic):
    p = datagen.workload("c2", deterministic=deterministic)
    x, dev, kw, cu = setup(p)
    o, lse = oracle.forward(x["q"], x["k"], x["v"], p.scale, p.causal)
    o = round_like(o, "bf16")
    lse = lse.astype(np.float32).astype(np.float64)
    O = to_dev(o, "bf16")
    L = torch.from_numpy(lse.astype(np.float32)).cuda()
    reps = [run_backward(p, dev, O, L, kw, dq_algo=dq_algo) for _ in range(3 if deterministic else 1)]
    for rep in reps[1:]:
        for a, bb in zip(reps[0], rep):
            assert torch.equal(a.view(torch.int16), bb.view(torch.int16))
    dq, dk, dv = reps[0]
    rdq, rdk, rdv = oracle.backward(x["q"], x["k"], x["v"], o, x["do"], lse, p.scale, p.causal)
    for n, gg, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert_close(n, to_host(gg), r, "bf16")


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds", "atomic"])
def test_bf16_causal_d64_workload_end_to_end(dq_algo):
    """The c2 workload as specified, O and LSE from the library forward: the
    GPU chain (attn_fwd, then the backward on its O and LSE) against the
    oracle chain (oracle forward, then the oracle backward on its own fp64 O
    and LSE), so no oracle input comes from the GPU."""
    from exact_attention_backward_amd import api
    p = datagen.workload("c2")
    x, dev, kw, cu = setup(p)
    o_g, lse_g = api.forward(dev["q"], dev["k"], dev["v"], p.scale, p.causal)
    dq, dk, dv = run_backward(p, dev, o_g, lse_g, kw, dq_algo=dq_algo)
    ro, rlse = oracle.forward(x["q"], x["k"], x["v"], p.scale, p.causal)
    assert_close("O", to_host(o_g), ro, "bf16")
    assert np.max(np.abs(lse_g.cpu().numpy().astype(np.float64) - rlse)) <= 2e-4
    rdq, rdk, rdv = oracle.backward(x["q"], x["k"], x["v"], ro, x["do"], rlse, p.scale, p.causal)
    for n, gg, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
        assert_close(n, to_host(gg), r, "bf16")


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds", "atomic"])
def test_headline_causal_all_groups(dq_algo):
    all_groups_check("c3", dq_algo)


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds"])
def test_headline_noncausal_all_groups(dq_algo):
    all_groups_check("c3nc", dq_algo)


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds"])
def test_headline_shape_fp16_all_groups(dq_algo):
    """The causal B=4 H=16 S=4096 D=128 shape with fp16 I/O."""
    all_groups_check("c3h", dq_algo)


@pytest.mark.parametrize("dq_algo", ["separate", "stored_ds"])
def test_varlen_all_groups(dq_algo):
    all_groups_check("c4", dq_algo)


@pytest.mark.parametrize("dq_algo,deterministic,repeats",
                         [("atomic", False, 1), ("atomic", True, 3), ("separate", False, 2), ("stored_ds", False, 2)])
def test_gqa_all_groups(dq_algo, deterministic, repeats):
    """GQA Hq32 Hkv8 S8192 in every dQ mode; the deterministic and the
    atomic-free modes also bitwise reproducible."""
    all_groups_check("c5", dq_algo, deterministic, repeats)
