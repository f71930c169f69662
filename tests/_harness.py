"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on
the same seeded inputs and compare.  Test infrastructure only."""

import math

import numpy as np
import torch

import datagen
import oracle
from exact_attention_backward_amd import api

# max|gpu - oracle| / max|oracle|.  The 16-bit paths round P and dS to the
# operand type before their products and the outputs once more, each a
# relative error of at most u (2^-8 for bf16, 2^-11 for fp16), so the bound
# is five units of the type: 2e-2 for bf16, 2.5e-3 for fp16.  fp32 keeps
# only summation-order differences.
TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2.5e-3}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(TORCH_DTYPE[dtype]).cuda()


def to_host(t):
    return t.float().cpu().numpy().astype(np.float64)


def round_like(x, dtype):
    """Values the GPU will hold for a float64 array stored in `dtype`."""
    x32 = np.asarray(x, np.float64).astype(np.float32)
    if dtype == "bf16":
        return datagen.round_to_bf16(x32).astype(np.float64)
    if dtype == "f16":
        return datagen.round_to_f16(x32).astype(np.float64)
    return x32.astype(np.float64)


def small_problem(dtype, b, hq, hkv, sq, sk, d, causal, seed, lengths=None, deterministic=False, scale=None,
                  do_scale=1.0):
    if lengths is not None:
        lengths = tuple(lengths)
        sq = sk = max(lengths)
    return datagen.Problem(dtype, len(lengths) if lengths else b, hq, hkv, sq, sk, d, causal,
                           scale if scale is not None else 1 / math.sqrt(d), seed, do_scale=do_scale,
                           lengths_q=lengths, lengths_k=lengths, deterministic=deterministic,
                           name=f"test_{dtype}_{hq}_{hkv}_{sq}_{sk}_{d}_{int(causal)}")


class Run:
    """Inputs of a problem on host and device, with O/LSE from the oracle.
    window = (left, right) applies a local mask on both sides; alibi (fp32
    array, one slope per q-head) the ALiBi bias."""

    def __init__(self, p, oracle_o_lse=True, window=None, alibi=None):
        self.p = p
        self.window = window
        self.alibi = None if alibi is None else np.asarray(alibi, np.float32)
        self.x = datagen.draw(p)
        cq, ck = p.cu_seqlens()
        self.cu_np = (cq, ck)
        self.cu = (None, None) if cq is None else (torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda())
        self.dev = {k: to_dev(v, p.dtype) for k, v in self.x.items()}
        self.slopes = None if self.alibi is None else torch.from_numpy(self.alibi).cuda()
        if oracle_o_lse:
            o, lse = oracle.forward(self.x["q"], self.x["k"], self.x["v"], p.scale, p.causal, cq, ck,
                                    window=window, alibi_slopes=self.alibi)
            self.set_o_lse(o, lse)

    def kw(self):
        p = self.p
        if not p.varlen:
            return {}
        return dict(cu_seqlens_q=self.cu[0], cu_seqlens_k=self.cu[1], max_seqlen_q=p.seqlen_q,
                    max_seqlen_k=p.seqlen_k)

    def set_o_lse(self, o, lse):
        """O rounded to the I/O type and LSE to fp32, the values both sides use."""
        self.o = round_like(o, self.p.dtype)
        self.lse = np.asarray(lse, np.float64).astype(np.float32).astype(np.float64)
        self.dev["o"] = to_dev(self.o, self.p.dtype)
        self.dev["lse"] = torch.from_numpy(self.lse.astype(np.float32)).cuda()

    def gpu_forward(self):
        d = self.dev
        return api.forward(d["q"], d["k"], d["v"], self.p.scale, self.p.causal, window=self.window,
                           alibi_slopes=self.slopes, **self.kw())

    def plan(self, deterministic=None, dq_algo="separate"):
        d = self.dev
        det = self.p.deterministic if deterministic is None else deterministic
        return api.BackwardPlan(d["q"], d["k"], self.p.scale, self.p.causal, det, dq_algo=dq_algo,
                                window=self.window, alibi_slopes=self.slopes, **self.kw())

    def gpu_backward(self, deterministic=None, plan=None, dq_algo="separate"):
        d = self.dev
        plan = plan or self.plan(deterministic, dq_algo)
        dq, dk, dv = torch.empty_like(d["q"]), torch.empty_like(d["k"]), torch.empty_like(d["v"])
        plan.run(d["q"], d["k"], d["v"], d["o"], d["do"], d["lse"], dq, dk, dv)
        torch.cuda.synchronize()
        return dq, dk, dv, plan

    def oracle_backward(self):
        cq, ck = self.cu_np
        return oracle.backward(self.x["q"], self.x["k"], self.x["v"], self.o, self.x["do"], self.lse,
                               self.p.scale, self.p.causal, cq, ck, window=self.window, alibi_slopes=self.alibi)


def assert_close(name, got, ref, dtype):
    err = rel_err(got, ref)
    assert err <= TOL[dtype], f"{name}: max|gpu-ref|/max|ref| = {err:.3e} > {TOL[dtype]}"
    return err


# --------------------------------------------------------------------------
# the fp64 oracle on every (sequence, kv-head) group of a full-size workload,
# in worker processes (spawned: no GPU state; one BLAS thread each)
# --------------------------------------------------------------------------

def _oracle_group_job(args):
    """Forward (O rounded to the I/O type, LSE to fp32: the values the GPU is
    given) and backward of one kv-head group of one sequence."""
    q, k, v, do, scale, causal, dtype, window, slopes = args
    import numpy as np
    import oracle as orc
    g = q.shape[1] // k.shape[1]
    outs = []
    dk = np.zeros((k.shape[0], k.shape[2]))
    dv = np.zeros_like(dk)
    for j in range(q.shape[1]):
        slope = None if slopes is None else float(slopes[j])
        o, lse = orc.head_forward(q[:, j], k[:, 0], v[:, 0], scale, causal, window, slope)
        o = round_like(o, dtype)
        lse = lse.astype(np.float32).astype(np.float64)
        dq, dkj, dvj = orc.head_backward(q[:, j], k[:, 0], v[:, 0], o, do[:, j], lse, scale, causal,
                                         window=window, alibi=slope)
        dk += dkj
        dv += dvj
        outs.append((o, lse, dq))
    assert g == len(outs)
    return outs, dk, dv


def oracle_all_groups(p, x, window=None, slopes=None, workers=16):
    """{(sequence, kv_head): ([(o, lse, dq) per q-head of the group], dk, dv)}
    for every group of problem p with inputs x (as datagen.draw returns)."""
    import multiprocessing as mp
    import os
    from concurrent.futures import ProcessPoolExecutor
    g = p.heads_q // p.heads_kv
    cq, ck = p.cu_seqlens()
    jobs, keys = [], []
    for b in range(p.batch):
        for hk in range(p.heads_kv):
            hs = slice(hk * g, (hk + 1) * g)
            if p.varlen:
                q0, q1, k0, k1 = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
                q, do = x["q"][q0:q1, hs], x["do"][q0:q1, hs]
                k, v = x["k"][k0:k1, hk:hk + 1], x["v"][k0:k1, hk:hk + 1]
            else:
                q, do = x["q"][b, :, hs], x["do"][b, :, hs]
                k, v = x["k"][b, :, hk:hk + 1], x["v"][b, :, hk:hk + 1]
            sl = None if slopes is None else np.asarray(slopes)[hs]
            jobs.append((q, k, v, do, p.scale, p.causal, p.dtype, window, sl))
            keys.append((b, hk))
    env = {n: os.environ.get(n) for n in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS")}
    os.environ["OPENBLAS_NUM_THREADS"] = os.environ["OMP_NUM_THREADS"] = "1"
    try:
        n = max(1, min(workers, len(jobs), os.cpu_count() or 1))
        with ProcessPoolExecutor(n, mp_context=mp.get_context("spawn")) as ex:
            res = {}
            for i, r in enumerate(ex.map(_oracle_group_job, jobs, timeout=1500)):
                res[keys[i]] = r
                if (i + 1) % 16 == 0 or i + 1 == len(jobs):
                    print(f"  oracle groups {i + 1}/{len(jobs)}", flush=True)
    finally:
        for k_, v_ in env.items():
            if v_ is None:
                os.environ.pop(k_, None)
            else:
                os.environ[k_] = v_
    return res
