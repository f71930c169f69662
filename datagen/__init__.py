"""Seeded synthetic inputs for attention backward: the only code shared by the
oracle side and the HIP side of every test and of the benchmark.

It holds no attention arithmetic: it draws normal samples, rounds them to the
storage type, and packs varlen sequences.  Inputs are drawn with numpy's PCG64
generator (``numpy.random.default_rng(seed)``) in the order Q, K, V, dO (for
varlen, the sequence lengths first), as float32, then rounded to bfloat16 or
IEEE binary16 with round-to-nearest-even for the bf16 and fp16 workloads, so
both sides see identical values.

Workloads (sizes of the five configurations the method is measured on):
  c1  fp32, non-causal, B=1 H=2 S=128 D=64
  c2  bf16, causal, B=2 H=8 S=1024 D=64
  c3  bf16, B=4 H=16 S=4096 D=128, causal and non-causal; dO scaled by 0.1
  c4  bf16, causal, varlen: 8 sequences, lengths uniform in [128, 8192], H=32 D=128
  c5  bf16, causal, GQA: B=1 Hq=32 Hkv=8 S=8192 D=128
  c3h the c3 causal shape with fp16 I/O (the same draws, rounded to fp16)
"""

import math
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

__all__ = ["Problem", "WORKLOADS", "workload", "draw", "round_to_bf16", "round_to_f16", "varlen_lengths"]


@dataclass(frozen=True)
class Problem:
    """Shape and flags of one attention-backward problem."""
    dtype: str            # "f32", "bf16" or "f16"
    batch: int            # dense batch, or number of sequences when varlen
    heads_q: int
    heads_kv: int
    seqlen_q: int         # dense length, or max length when varlen
    seqlen_k: int
    head_dim: int
    causal: bool
    scale: float
    seed: int
    do_scale: float = 1.0
    lengths_q: Optional[tuple] = None   # varlen: per-sequence lengths
    lengths_k: Optional[tuple] = None
    deterministic: bool = False
    name: str = ""
    length_range: Optional[tuple] = None  # varlen: (lo, hi) the lengths were drawn from

    @property
    def varlen(self):
        return self.lengths_q is not None

    @property
    def total_q(self):
        return sum(self.lengths_q) if self.varlen else self.batch * self.seqlen_q

    @property
    def total_k(self):
        return sum(self.lengths_k) if self.varlen else self.batch * self.seqlen_k

    def flops(self):
        """Algorithmic FLOPs of the backward: 10 * Sq * Sk * D per (sequence,
        q-head), halved when causal (the square-causal convention)."""
        if self.varlen:
            pairs = sum(lq * lk for lq, lk in zip(self.lengths_q, self.lengths_k))
        else:
            pairs = self.batch * self.seqlen_q * self.seqlen_k
        f = 10.0 * pairs * self.heads_q * self.head_dim
        return f / 2 if self.causal else f

    def cu_seqlens(self):
        """(cu_q, cu_k) int32 arrays for varlen problems, else (None, None)."""
        if not self.varlen:
            return None, None
        cq = np.concatenate([[0], np.cumsum(self.lengths_q)]).astype(np.int32)
        ck = np.concatenate([[0], np.cumsum(self.lengths_k)]).astype(np.int32)
        return cq, ck


def varlen_lengths(rng, nseq, lo, hi):
    """Sequence lengths uniform in [lo, hi] (the first draw from the seed)."""
    return tuple(int(x) for x in rng.integers(lo, hi + 1, nseq))


def _c4():
    lens = varlen_lengths(np.random.default_rng(4), 8, 128, 8192)
    return Problem("bf16", 8, 32, 32, max(lens), max(lens), 128, True, 1 / math.sqrt(128), 4,
                   lengths_q=lens, lengths_k=lens, name="c4_varlen_causal",
                   length_range=(128, 8192))


WORKLOADS = {
    "c1": Problem("f32", 1, 2, 2, 128, 128, 64, False, 1 / 8, 1, name="c1_f32_noncausal"),
    "c2": Problem("bf16", 2, 8, 8, 1024, 1024, 64, True, 1 / 8, 2, name="c2_bf16_causal"),
    "c3": Problem("bf16", 4, 16, 16, 4096, 4096, 128, True, 1 / math.sqrt(128), 3, do_scale=0.1,
                  name="c3_bf16_causal"),
    "c3nc": Problem("bf16", 4, 16, 16, 4096, 4096, 128, False, 1 / math.sqrt(128), 3, do_scale=0.1,
                    name="c3_bf16_noncausal"),
    "c4": _c4(),
    "c5": Problem("bf16", 1, 32, 8, 8192, 8192, 128, True, 1 / math.sqrt(128), 5,
                  name="c5_bf16_gqa_causal"),
    "c3h": Problem("f16", 4, 16, 16, 4096, 4096, 128, True, 1 / math.sqrt(128), 3, do_scale=0.1,
                   name="c3_f16_causal"),
    # head dim 256 at the headline's FLOPs (half the heads)
    "c3w": Problem("bf16", 4, 8, 8, 4096, 4096, 256, True, 1 / 16, 3, do_scale=0.1,
                   name="c3_bf16_causal_d256"),
}


def workload(name, **overrides):
    """A named workload, optionally with fields replaced (e.g. deterministic=True)."""
    p = WORKLOADS[name]
    return replace(p, **overrides) if overrides else p


def round_to_bf16(x):
    """float32 array -> float32 array holding the nearest bfloat16 values (RNE),
    using torch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def round_to_f16(x):
    """float32 array -> float32 array holding the nearest binary16 values
    (RNE), using torch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float16).to(torch.float32).numpy()


def draw(p: Problem):
    """Seeded Q, K, V, dO for a problem, as float32 arrays holding values
    exactly representable in the problem's dtype.

    dense : q, do [B, Sq, Hq, D]; k, v [B, Sk, Hkv, D]
    varlen: q, do [Tq, Hq, D];    k, v [Tk, Hkv, D]
    """
    rng = np.random.default_rng(p.seed)
    if p.varlen:
        if p.length_range is not None:
            # the lengths are the first draw from the same seed
            lens = varlen_lengths(rng, len(p.lengths_q), *p.length_range)
            assert lens == tuple(p.lengths_q)
        qs = (p.total_q, p.heads_q, p.head_dim)
        ks = (p.total_k, p.heads_kv, p.head_dim)
    else:
        qs = (p.batch, p.seqlen_q, p.heads_q, p.head_dim)
        ks = (p.batch, p.seqlen_k, p.heads_kv, p.head_dim)
    q = rng.standard_normal(qs, dtype=np.float32)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = rng.standard_normal(ks, dtype=np.float32)
    do = rng.standard_normal(qs, dtype=np.float32)
    if p.do_scale != 1.0:
        do = do * np.float32(p.do_scale)
    if p.dtype == "bf16":
        q, k, v, do = (round_to_bf16(x) for x in (q, k, v, do))
    elif p.dtype == "f16":
        q, k, v, do = (round_to_f16(x) for x in (q, k, v, do))
    return {"q": q, "k": k, "v": v, "do": do}


def draw_bias(p: Problem, seed, heads=None, batch=None):
    """A seeded elementwise bias [nseq or B, H, Sq, Sk] (Sq, Sk the longest
    lengths) of standard normal values times 2, exactly representable in the
    problem's dtype.  heads / batch = 1 give a bias to broadcast over them."""
    rng = np.random.default_rng(seed)
    shape = (batch if batch is not None else p.batch, heads if heads is not None else p.heads_q,
             p.seqlen_q, p.seqlen_k)
    b = (2.0 * rng.standard_normal(shape)).astype(np.float32)
    if p.dtype == "bf16":
        b = round_to_bf16(b)
    elif p.dtype == "f16":
        b = round_to_f16(b)
    return b
