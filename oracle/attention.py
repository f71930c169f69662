"""Plain fp64 CPU oracle for exact softmax attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` use it.  It shares no code with the HIP library.

What it computes is the textbook definition of softmax attention and of its
gradient, written out per (batch, head) with no tiling, no fusion and no
reordering beyond what the definition states.  A matrix product (numpy ``@``)
is the only library primitive used.

The backward follows the stage order of the Composable Kernel page
"block_fmha_bwd_dq_dk_dv_pipeline_trload_kr_ktr_vr.hpp Source File"
(``BlockFmhaBwdDQDKDVPipelineTrLoadKRKTRVR::run``):

  STAGE 1  S = Q K^T, scaled by the softmax scale s
  STAGE 2  P recomputed from S and the saved log-sum-exp (natural log; the page
           multiplies it by log2(e) before taking exp2, which is the same value)
  STAGE 4  dP = dO V^T
  STAGE 3  dV = P^T dO
  STAGE 5  dS = P * (dP - D), D the per-row sum of dO * O
  STAGE 6  dK = dS^T Q, multiplied by s at the end ("Results Scale")
  STAGE 7  dQ = dS K, multiplied by s ("QGrad Scale")

Readings taken where the pages are silent (each is listed in the design notes):

* Causal masking is aligned to the bottom-right corner: key j is visible to
  query i iff ``j <= i + (Sk - Sq)``.  The pages only show that an
  out-of-bound test exists (``mask.IsOutOfBound``), not its formula.
* A query row that sees no key has LSE = -inf, O = 0 and contributes nothing
  to any gradient.  The same page maps LSE = -inf to 0 (``get_validated_lse``)
  so that such rows give P = exp(-inf) = 0.
* D is computed from the O it is given (``D`` is only consumed on the pages).
* ALiBi: the composable-kernel page applies a position encoding to each
  scaled logit from its (row, column) position only (``position_encoding.
  update`` after ``s_acc *= scale``, before the exponential), without its
  formula.  Reading taken: the linear-bias definition on the same
  bottom-right-aligned diagonal as the masks, ``-slope_h * |i + off - j|``
  (off = Sk - Sq) added to ``s * q_i . k_j`` in natural-log units, one slope
  per q-head.
* Elementwise bias: the composable-kernel page adds a bias tile to the scaled
  logits (times log2e in its base-2 arithmetic, i.e. in natural-log units)
  and writes dBias as dS cast to the bias type.  The gradient of the loss
  with respect to the logit s q_i . k_j + bias_ij is exactly dS_ij, so dBias
  = dS; a bias broadcast over batch or heads is not summed here (the page
  writes one dBias tile per (batch, head) tile).
* Dropout (``dropout`` arguments): P is computed as without dropout (the
  LSE keeps every visible key); the output uses Z P / (1 - p) with Z the
  keep mask of ``oracle.dropout``.  The gradient of that output is
  dV = (Z P)^T dO / (1 - p), dP = Z (dO V^T) / (1 - p), dS = P (dP - D) with
  D = rowsum(dO * O) of the dropped output.  The composable-kernel page forms
  dS from the sign-marked P as P (dP' - D') on kept and -P D' on dropped
  elements and then scales dS-derived results by rp_undrop; that is this
  same gradient when its D' is D (1 - p), the reading taken for the D it
  consumes but does not define.
* GQA groups are contiguous: q-head h reads kv-head ``h // (Hq // Hkv)``, as in
  the head mapping of ``CollectiveEpilogueBwdGQA::store`` on the
  FlashAttention-3 page "flash-attention/hopper/epilogue_bwd.hpp"; dK and dV of
  a kv-head are summed over its q-heads.

Layouts (all numpy arrays, any float dtype, computed in float64):
  dense : q, o, do [B, Sq, Hq, D];  k, v [B, Sk, Hkv, D];  lse, delta [B, Hq, Sq]
  varlen: q, o, do [Tq, Hq, D];     k, v [Tk, Hkv, D];     lse, delta [Hq, Tq]
          with ``cu_seqlens_q``/``cu_seqlens_k`` (length nseq + 1) giving the
          row range of each sequence.
"""

import numpy as np

from .dropout import dropout_keep

__all__ = [
    "visible",
    "alibi_bias",
    "head_forward",
    "head_backward",
    "head_forward_rows",
    "head_backward_rows",
    "forward",
    "backward",
    "group_forward",
    "group_backward",
    "preprocess_delta",
    "round_f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "round_f32_to_f16_bits",
    "f16_bits_to_f32",
    "postprocess_dq",
]


# --------------------------------------------------------------------------
# one (batch, head) pair
# --------------------------------------------------------------------------

def visible(sq, sk, causal, window=None):
    """Boolean [sq, sk]: True where query i may attend to key j.

    Non-causal: every key.  Causal: ``j <= i + (sk - sq)`` (bottom-right
    alignment; for sq == sk this is the usual lower triangle).

    ``window = (left, right)``: a local (sliding-window) mask on the same
    bottom-right-aligned diagonal, ``i + off - left <= j <= i + off + right``
    with off = sk - sq; a negative side is unbounded.  The composable-kernel
    page only shows that the pipeline asks the mask for each tile's key range
    and for out-of-bound elements; these bounds are the reading taken, and
    they combine with the causal bound by intersection.
    """
    i = np.arange(sq)[:, None]
    j = np.arange(sk)[None, :]
    off = sk - sq
    ok = np.ones((sq, sk), dtype=bool)
    if causal:
        ok &= j <= i + off
    if window is not None:
        left, right = window
        if left >= 0:
            ok &= j >= i + off - left
        if right >= 0:
            ok &= j <= i + off + right
    return ok


def alibi_bias(sq, sk, slope):
    """[sq, sk] float64 ALiBi bias of one head: ``-slope * |i + (sk - sq) - j|``
    (zero on the bottom-right-aligned diagonal, falling linearly with the
    distance from it on both sides)."""
    i = np.arange(sq)[:, None]
    j = np.arange(sk)[None, :]
    return -float(slope) * np.abs(i + (sk - sq) - j).astype(np.float64)


def _logits(q, k, scale, alibi, bias=None):
    """Stage 1: s * Q K^T, plus the ALiBi bias when a slope is given and the
    elementwise bias [sq, sk] when one is given."""
    s = scale * (q @ k.T)
    if alibi is not None:
        s = s + alibi_bias(q.shape[0], k.shape[0], alibi)
    if bias is not None:
        s = s + np.asarray(bias, np.float64)
    return s


def head_forward(q, k, v, scale, causal, window=None, alibi=None, bias=None, dropout=None):
    """Softmax attention for one head.

    q [sq, d], k [sk, d], v [sk, d] -> (o [sq, d], lse [sq]), float64.
    ``lse_i = log(sum_j exp(s * q_i . k_j + b_ij))`` over the visible keys
    (b the ALiBi bias of slope ``alibi``, or 0), ``o_i = sum_j softmax_ij
    v_j``.  Rows with no visible key give lse = -inf and o = 0.
    ``dropout = (keep [sq, sk] bool, rp)``: ``o_i = rp sum_j keep_ij
    softmax_ij v_j`` (the LSE is unchanged).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    sq, sk = q.shape[0], k.shape[0]
    ok = visible(sq, sk, causal, window)
    s = _logits(q, k, scale, alibi, bias)
    has_key = ok.any(axis=1)
    # row maximum over visible keys (0 for empty rows, never used)
    row_max = np.max(np.where(ok, s, -np.inf), axis=1, initial=-np.inf)
    row_max = np.where(has_key, row_max, 0.0)
    e = np.exp(np.where(ok, s - row_max[:, None], -np.inf))
    total = e.sum(axis=1)
    lse = np.full(sq, -np.inf)
    lse[has_key] = row_max[has_key] + np.log(total[has_key])
    p = np.zeros_like(s)
    p[has_key] = e[has_key] / total[has_key, None]
    if dropout is not None:
        keep, rp = dropout
        p = rp * np.where(keep, p, 0.0)
    o = p @ v
    return o, lse


def _probabilities(q, k, lse, scale, causal, window=None, alibi=None, bias=None):
    """P recomputed from the saved LSE (stages 1-2): exp(s q_i.k_j + b_ij - lse_i)."""
    sq, sk = q.shape[0], k.shape[0]
    ok = visible(sq, sk, causal, window) & np.isfinite(lse)[:, None]
    s = _logits(q, k, scale, alibi, bias)
    safe_lse = np.where(np.isfinite(lse), lse, 0.0)
    return np.exp(np.where(ok, s - safe_lse[:, None], -np.inf))


def head_backward(q, k, v, o, do, lse, scale, causal, details=False, window=None, alibi=None, bias=None,
                  dropout=None):
    """Gradient of attention for one head, given O and LSE as saved by a forward.

    Returns (dq [sq, d], dk [sk, d], dv [sk, d]) in float64; with
    ``details=True`` also a dict holding P, dP, dS and D.  The ALiBi and
    elementwise biases only enter through P (they do not depend on Q or K);
    the gradient of the elementwise bias is dS (``details["ds"]``).
    ``dropout = (keep [sq, sk] bool, rp)`` as in head_forward: dV =
    rp (keep P)^T dO and dP = rp keep (dO V^T).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    o = np.asarray(o, np.float64)
    do = np.asarray(do, np.float64)
    lse = np.asarray(lse, np.float64)
    p = _probabilities(q, k, lse, scale, causal, window, alibi, bias)  # stages 1-2
    delta = np.sum(do * o, axis=1)                        # D = rowsum(dO * O)
    dp = do @ v.T                                         # stage 4
    if dropout is None:
        dv = p.T @ do                                     # stage 3
    else:
        keep, rp = dropout
        dv = (rp * np.where(keep, p, 0.0)).T @ do         # stage 3 on the kept P
        dp = rp * np.where(keep, dp, 0.0)
    ds = p * (dp - delta[:, None])                        # stage 5
    dk = scale * (ds.T @ q)                               # stage 6 + final scale
    dq = scale * (ds @ k)                                 # stage 7 + dQ scale
    if details:
        return dq, dk, dv, {"p": p, "dp": dp, "ds": ds, "delta": delta}
    return dq, dk, dv


# --------------------------------------------------------------------------
# one head at lengths where the [sq, sk] matrices do not fit: the same
# definitions, evaluated a slice of rows (or single rows / keys) at a time
# --------------------------------------------------------------------------

def _row_logits(q_rows, rows, k, scale, causal, window, alibi, sq):
    """Logits s q_i . k_j (+ ALiBi) of the given global rows i (q_rows their
    queries) against every key, and their visibility mask."""
    sk = k.shape[0]
    i = np.asarray(rows)[:, None]
    j = np.arange(sk)[None, :]
    off = sk - sq
    ok = np.ones((len(rows), sk), dtype=bool)
    if causal:
        ok &= j <= i + off
    if window is not None:
        left, right = window
        if left >= 0:
            ok &= j >= i + off - left
        if right >= 0:
            ok &= j <= i + off + right
    s = scale * (q_rows @ k.T)
    if alibi is not None:
        s = s - float(alibi) * np.abs(i + off - j).astype(np.float64)
    return s, ok


def head_forward_rows(q, k, v, scale, causal, window=None, alibi=None, block=1024):
    """head_forward for one head, computed ``block`` query rows at a time
    (each row's logits, LSE and output are those of head_forward: rows are
    independent).  Returns (o [sq, d], lse [sq]) in float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    sq = q.shape[0]
    o = np.zeros((sq, v.shape[1]))
    lse = np.full(sq, -np.inf)
    for r0 in range(0, sq, block):
        rows = np.arange(r0, min(r0 + block, sq))
        s, ok = _row_logits(q[rows], rows, k, scale, causal, window, alibi, sq)
        has_key = ok.any(axis=1)
        row_max = np.max(np.where(ok, s, -np.inf), axis=1, initial=-np.inf)
        row_max = np.where(has_key, row_max, 0.0)
        e = np.exp(np.where(ok, s - row_max[:, None], -np.inf))
        total = e.sum(axis=1)
        lse[rows[has_key]] = row_max[has_key] + np.log(total[has_key])
        p = np.zeros_like(s)
        p[has_key] = e[has_key] / total[has_key, None]
        o[rows] = p @ v
    return o, lse


def head_backward_rows(q, k, v, o, do, lse, scale, causal, q_rows, k_rows, window=None, alibi=None):
    """head_backward's dQ at the query rows ``q_rows`` and dK, dV at the keys
    ``k_rows``, each from its definition: dQ_i = s sum_j dS_ij k_j needs row i
    of P and dP; dK_j = s sum_i dS_ij q_i and dV_j = sum_i P_ij dO_i need
    column j, i.e. P_ij = exp(s q_i . k_j - LSE_i) and dP_ij = dO_i . v_j for
    every row i (and D_i = dO_i . O_i).  Returns (dq [len(q_rows), d],
    dk [len(k_rows), d], dv [len(k_rows), d]) in float64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    o = np.asarray(o, np.float64)
    do = np.asarray(do, np.float64)
    lse = np.asarray(lse, np.float64)
    sq, sk = q.shape[0], k.shape[0]
    delta = np.sum(do * o, axis=1)                 # D for every row
    finite = np.isfinite(lse)
    safe_lse = np.where(finite, lse, 0.0)
    # dQ rows
    rows = np.asarray(q_rows)
    s, ok = _row_logits(q[rows], rows, k, scale, causal, window, alibi, sq)
    ok &= finite[rows][:, None]
    p = np.exp(np.where(ok, s - safe_lse[rows][:, None], -np.inf))
    dp = do[rows] @ v.T
    ds = p * (dp - delta[rows][:, None])
    dq = scale * (ds @ k)
    # dK, dV keys: their columns of P and dP over every row
    keys = np.asarray(k_rows)
    all_rows = np.arange(sq)
    s, ok = _row_logits(q, all_rows, k[keys], scale, False, None, None, sq)   # s q_i . k_j, no mask yet
    i = all_rows[:, None]
    j = keys[None, :]
    off = sk - sq
    if causal:
        ok &= j <= i + off
    if window is not None:
        left, right = window
        if left >= 0:
            ok &= j >= i + off - left
        if right >= 0:
            ok &= j <= i + off + right
    if alibi is not None:
        s = s - float(alibi) * np.abs(i + off - j).astype(np.float64)
    ok &= finite[:, None]
    p = np.exp(np.where(ok, s - safe_lse[:, None], -np.inf))     # [sq, len(keys)]
    dp = do @ v[keys].T
    ds = p * (dp - delta[:, None])
    dk = scale * (ds.T @ q)
    dv = p.T @ do
    return dq, dk, dv


# --------------------------------------------------------------------------
# batched / grouped / varlen layouts
# --------------------------------------------------------------------------

def _ranges(nseq, sq, sk, cu_q, cu_k, used_q=None, used_k=None):
    """Row ranges (q0, q1, k0, k1) of every sequence.

    Varlen only: ``used_q``/``used_k`` (one length per sequence) replace the
    length cu[b+1] - cu[b] while the sequence still starts at cu[b], as the
    sequence-length helper of the FlashAttention-3 backward epilogue page does
    with ``seqused``; rows past the used length take no part in anything.
    """
    if cu_q is None:
        if used_q is not None or used_k is not None:
            raise ValueError("seqused needs cu_seqlens")
        return [(b * sq, (b + 1) * sq, b * sk, (b + 1) * sk) for b in range(nseq)]
    cu_q = np.asarray(cu_q, np.int64)
    cu_k = np.asarray(cu_k, np.int64)
    out = []
    for b in range(nseq):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if used_q is not None:
            if not 0 <= int(used_q[b]) <= q1 - q0:
                raise ValueError("seqused_q out of range")
            q1 = q0 + int(used_q[b])
        if used_k is not None:
            if not 0 <= int(used_k[b]) <= k1 - k0:
                raise ValueError("seqused_k out of range")
            k1 = k0 + int(used_k[b])
        out.append((q0, q1, k0, k1))
    return out


def _flat(x, varlen):
    """View [B, S, H, D] as [B*S, H, D]; varlen tensors already are [T, H, D]."""
    x = np.asarray(x)
    return x if varlen else x.reshape(-1, x.shape[2], x.shape[3])


def _geometry(q, k, cu_q, cu_k):
    varlen = cu_q is not None
    if varlen:
        nseq = len(cu_q) - 1
        sq = sk = None
        hq, hkv = q.shape[1], k.shape[1]
    else:
        nseq, sq, hq = q.shape[0], q.shape[1], q.shape[2]
        sk, hkv = k.shape[1], k.shape[2]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return varlen, nseq, sq, sk, hq, hkv


def _lse_view(lse, varlen, nseq, hq, sq):
    """LSE/delta as [H, rows] over the flattened row index."""
    lse = np.asarray(lse)
    if varlen:
        return lse
    # [B, H, Sq] -> [H, B*Sq]
    return np.transpose(lse, (1, 0, 2)).reshape(hq, nseq * sq)


def _slope(alibi_slopes, h):
    return None if alibi_slopes is None else float(np.asarray(alibi_slopes, np.float64)[h])


def _bias_block(bias, seq, h, len_q, len_k):
    """The [len_q, len_k] bias of one (sequence, q-head), or None."""
    return None if bias is None else np.asarray(bias)[seq, h, :len_q, :len_k]


def _dropout_block(dropout, seq, h, hq, len_q, len_k):
    """(keep mask, 1 / (1 - p)) of one (sequence, q-head) for ``dropout =
    (p, seed, offset)``, or None."""
    if dropout is None:
        return None
    p, seed, offset = dropout
    return dropout_keep(seed, offset, seq * hq + h, len_q, len_k, p), 1.0 / (1.0 - float(p))


def group_forward(q, k, v, scale, causal, seq, kv_head, cu_seqlens_q=None, cu_seqlens_k=None,
                  seqused_q=None, seqused_k=None, window=None, alibi_slopes=None, bias=None, dropout=None):
    """Forward for the q-heads of one kv-head group of one sequence.

    Returns {q_head: (o [len_q, d], lse [len_q])}.  ``alibi_slopes``: one
    slope per q-head, or None.  ``bias``: [nseq, Hq, Sq, Sk] (Sq, Sk the
    longest lengths), each sequence's block at its top left, or None.
    ``dropout``: (p, seed, offset) or None; the keep mask of (sequence, q-head)
    uses index sequence * Hq + q-head and the sequence's own row and key
    positions.
    """
    varlen, nseq, sq, sk, hq, hkv = _geometry(q, k, cu_seqlens_q, cu_seqlens_k)
    g = hq // hkv
    q0, q1, k0, k1 = _ranges(nseq, sq, sk, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k)[seq]
    qf, kf, vf = _flat(q, varlen), _flat(k, varlen), _flat(v, varlen)
    out = {}
    for h in range(kv_head * g, (kv_head + 1) * g):
        out[h] = head_forward(qf[q0:q1, h], kf[k0:k1, kv_head], vf[k0:k1, kv_head], scale, causal, window,
                              _slope(alibi_slopes, h), _bias_block(bias, seq, h, q1 - q0, k1 - k0),
                              _dropout_block(dropout, seq, h, hq, q1 - q0, k1 - k0))
    return out


def group_backward(q, k, v, o, do, lse, scale, causal, seq, kv_head,
                   cu_seqlens_q=None, cu_seqlens_k=None, seqused_q=None, seqused_k=None, window=None,
                   alibi_slopes=None, bias=None, dbias_out=None, dropout=None):
    """Backward for one kv-head group of one sequence.

    Returns (dq {q_head: [len_q, d]}, dk [len_k, d], dv [len_k, d]); dk and dv
    are summed over the group's q-heads in ascending head order.  With
    ``dbias_out`` ([nseq, Hq, Sq, Sk]) each q-head's dS is written into its
    block (top left of the sequence's slot).
    """
    varlen, nseq, sq, sk, hq, hkv = _geometry(q, k, cu_seqlens_q, cu_seqlens_k)
    g = hq // hkv
    q0, q1, k0, k1 = _ranges(nseq, sq, sk, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k)[seq]
    qf, kf, vf = _flat(q, varlen), _flat(k, varlen), _flat(v, varlen)
    of, dof = _flat(o, varlen), _flat(do, varlen)
    lf = _lse_view(lse, varlen, nseq, hq, sq)
    d = qf.shape[2]
    dk = np.zeros((k1 - k0, d))
    dv = np.zeros((k1 - k0, d))
    dq = {}
    for h in range(kv_head * g, (kv_head + 1) * g):
        dqh, dkh, dvh, det = head_backward(qf[q0:q1, h], kf[k0:k1, kv_head], vf[k0:k1, kv_head],
                                           of[q0:q1, h], dof[q0:q1, h], lf[h, q0:q1], scale, causal, details=True,
                                           window=window, alibi=_slope(alibi_slopes, h),
                                           bias=_bias_block(bias, seq, h, q1 - q0, k1 - k0),
                                           dropout=_dropout_block(dropout, seq, h, hq, q1 - q0, k1 - k0))
        if dbias_out is not None:
            dbias_out[seq, h, :q1 - q0, :k1 - k0] = det["ds"]
        dq[h] = dqh
        dk += dkh
        dv += dvh
    return dq, dk, dv


def forward(q, k, v, scale, causal, cu_seqlens_q=None, cu_seqlens_k=None, seqused_q=None, seqused_k=None,
            window=None, alibi_slopes=None, bias=None, dropout=None):
    """Full forward.  Returns (o, lse) in the layouts given in the module doc
    (rows past a sequence's used length are left at zero)."""
    varlen, nseq, sq, sk, hq, hkv = _geometry(q, k, cu_seqlens_q, cu_seqlens_k)
    qf = _flat(q, varlen)
    o = np.zeros(qf.shape, np.float64)
    lse = np.zeros((hq, qf.shape[0]), np.float64)
    for b, (q0, q1, _, _) in enumerate(_ranges(nseq, sq, sk, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k)):
        for g in range(hkv):
            for h, (oh, lh) in group_forward(q, k, v, scale, causal, b, g, cu_seqlens_q, cu_seqlens_k,
                                             seqused_q, seqused_k, window, alibi_slopes, bias,
                                             dropout).items():
                o[q0:q1, h] = oh
                lse[h, q0:q1] = lh
    if varlen:
        return o, lse
    return o.reshape(q.shape), np.transpose(lse.reshape(hq, nseq, sq), (1, 0, 2)).copy()


def backward(q, k, v, o, do, lse, scale, causal, cu_seqlens_q=None, cu_seqlens_k=None,
             seqused_q=None, seqused_k=None, window=None, alibi_slopes=None, bias=None, want_dbias=False,
             dropout=None):
    """Full backward.  Returns (dq, dk, dv) shaped like q, k, v (float64);
    rows past a sequence's used length are left at zero.  With
    ``want_dbias`` also dBias [nseq, Hq, Sq, Sk] (dS of each head; zero
    outside each sequence's block)."""
    varlen, nseq, sq, sk, hq, hkv = _geometry(q, k, cu_seqlens_q, cu_seqlens_k)
    qf, kf = _flat(q, varlen), _flat(k, varlen)
    dq = np.zeros(qf.shape, np.float64)
    dk = np.zeros(kf.shape, np.float64)
    dv = np.zeros(kf.shape, np.float64)
    ranges = _ranges(nseq, sq, sk, cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k)
    dbias = None
    if want_dbias:
        msq = max(r[1] - r[0] for r in ranges) if varlen else sq
        msk = max(r[3] - r[2] for r in ranges) if varlen else sk
        if bias is not None:
            msq, msk = np.asarray(bias).shape[2], np.asarray(bias).shape[3]
        dbias = np.zeros((nseq, hq, msq, msk), np.float64)
    for b, (q0, q1, k0, k1) in enumerate(ranges):
        for g in range(hkv):
            dqg, dkg, dvg = group_backward(q, k, v, o, do, lse, scale, causal, b, g, cu_seqlens_q, cu_seqlens_k,
                                           seqused_q, seqused_k, window, alibi_slopes, bias, dbias, dropout)
            for h, x in dqg.items():
                dq[q0:q1, h] = x
            dk[k0:k1, g] = dkg
            dv[k0:k1, g] = dvg
    if varlen:
        out = (dq, dk, dv)
    else:
        out = (dq.reshape(q.shape), dk.reshape(k.shape), dv.reshape(k.shape))
    return out + (dbias,) if want_dbias else out


def preprocess_delta(o, do, cu_seqlens_q=None):
    """D = rowsum(dO * O) per (head, row), in the LSE layout, float64."""
    o = np.asarray(o, np.float64)
    do = np.asarray(do, np.float64)
    d = np.sum(o * do, axis=-1)              # [B, Sq, H] or [T, H]
    if cu_seqlens_q is not None:
        return d.T.copy()                    # [H, T]
    return np.transpose(d, (0, 2, 1)).copy()  # [B, H, Sq]


# --------------------------------------------------------------------------
# dQ postprocess: fp32 accumulator -> output dtype, times the softmax scale
# --------------------------------------------------------------------------

def round_f32_to_bf16_bits(x):
    """bfloat16 bit patterns (uint16) of float32 values, round to nearest even.

    Written from the definition: bfloat16 keeps the top 16 bits of the binary32
    pattern; the discarded low 16 bits round the kept part to the nearest
    representable value, ties going to the even one.  NaN stays a (quiet) NaN.
    """
    u = np.ascontiguousarray(np.asarray(x, np.float32)).view(np.uint32).astype(np.uint64)
    low = u & 0xFFFF
    kept = u >> 16
    half = 0x8000
    round_up = (low > half) | ((low == half) & ((kept & 1) == 1))
    out = (kept + round_up.astype(np.uint64)) & 0xFFFF
    is_nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    out = np.where(is_nan, (kept | 0x0040) & 0xFFFF, out)
    return out.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """float32 values of bfloat16 bit patterns (exact)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def round_f32_to_f16_bits(x):
    """IEEE 754 binary16 bit patterns (uint16) of float32 values, round to
    nearest, ties to even.

    Written from the format's definition: 1 sign bit, 5 exponent bits (bias
    15), 10 fraction bits; normal numbers from 2^-14 have a last-place unit of
    2^(e - 10) for |x| in [2^e, 2^(e+1)), subnormals a unit of 2^-24.  The
    value is rounded to a whole number of its unit (float64 holds every
    float32 exactly, and scaling by a power of two is exact, so ``rint`` sees
    the exact quotient); a result of 2^16 or more is infinity.  NaN becomes a
    quiet NaN keeping the top fraction bits.
    """
    x32 = np.ascontiguousarray(np.asarray(x, np.float32))
    u = x32.view(np.uint32)
    a = np.abs(x32.astype(np.float64))
    sign = ((u >> 16) & 0x8000).astype(np.uint32)
    _, ex = np.frexp(a)                         # a = f 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1                 # a in [2^e, 2^(e+1)) for a > 0
    unit = np.where(e >= -14, e - 10, -24)      # exponent of the last-place unit
    val = np.ldexp(np.rint(np.ldexp(a, -unit)), unit)
    over = ~(val < 65536.0)                     # overflow, infinities and NaN
    val = np.where(over, 0.0, val)
    normal = val >= 2.0 ** -14
    fn, en = np.frexp(np.where(normal, val, 1.0))
    bits_normal = ((en.astype(np.int64) - 1 + 15) << 10) + (np.ldexp(fn, 11).astype(np.int64) - 1024)
    bits_sub = np.ldexp(val, 24).astype(np.int64)          # whole units of 2^-24 (1024 = 2^-14)
    mag = np.where(normal, bits_normal, bits_sub)
    mag = np.where(over, 0x7C00, mag)
    is_nan = np.isnan(a)
    mag = np.where(is_nan, 0x7E00 | ((u >> 13) & 0x3FF), mag)
    return (sign | mag.astype(np.uint32)).astype(np.uint16)


def f16_bits_to_f32(bits):
    """float32 values of binary16 bit patterns (exact), from the definition."""
    b = np.asarray(bits, np.uint16).astype(np.int64)
    sgn = np.where(b & 0x8000, -1.0, 1.0)
    ex = (b >> 10) & 0x1F
    fr = b & 0x3FF
    val = np.where(ex == 0, np.ldexp(fr.astype(np.float64), -24),
                   np.ldexp((1024 + fr).astype(np.float64), ex - 25))
    val = np.where(ex == 31, np.where(fr == 0, np.inf, np.nan), val)
    return (sgn * val).astype(np.float32)


def postprocess_dq(dq_accum, scale, out_dtype):
    """dQ = out_dtype(scale * dQaccum), the product taken in float32.

    Follows ``FlashAttentionBackwardPostprocess`` on the page
    "flash_bwd_postprocess.py": the fp32 accumulator is multiplied by the
    scale and converted to the output type.  ``out_dtype`` is "bf16" or "f16"
    (returns uint16 bit patterns) or "f32" (returns float32).
    """
    prod = np.asarray(dq_accum, np.float32) * np.float32(scale)
    if out_dtype == "bf16":
        return round_f32_to_bf16_bits(prod)
    if out_dtype == "f16":
        return round_f32_to_f16_bits(prod)
    if out_dtype == "f32":
        return prod.astype(np.float32)
    raise ValueError(out_dtype)
