"""Python binding of the C ABI: the same entry points, taking torch tensors.

PyTorch only supplies device memory and the current HIP stream; every step of
the computation runs in the library's kernels.  Tensors must be on the GPU
with the index order of include/attn_bwd.h:

  dense : q, o, do, dq [B, Sq, Hq, D];  k, v, dk, dv [B, Sk, Hkv, D];  lse, delta [B, Hq, Sq]
  varlen: q, o, do, dq [Tq, Hq, D];     k, v, dk, dv [Tk, Hkv, D];     lse, delta [Hq, Tq]

The head dimension must be contiguous; the batch, row and head strides of
every tensor are passed to the library as they are (views such as the q, k
and v slices of a packed [B, S, 3, H, D] tensor need no copy).  LSE, D and
the workspace must be contiguous.
"""

import ctypes

import torch

from . import _lib as L

__all__ = [
    "make_shape",
    "attn_bwd_workspace_bytes",
    "attn_fwd",
    "attn_bwd_preprocess",
    "attn_bwd",
    "attn_bwd_dq_postprocess",
    "attn_bwd_full",
    "attn_bwd_full_noalloc",
    "forward",
    "backward",
    "BackwardPlan",
]

_DTYPES = {torch.bfloat16: L.ATTN_DTYPE_BF16, torch.float16: L.ATTN_DTYPE_F16, torch.float32: L.ATTN_DTYPE_F32}


def _ptr(t):
    """Pointer of a tensor the library reads or writes with its own
    (contiguous) layout: LSE, D, the workspace."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("lse, delta and the workspace must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _tptr(t):
    """Pointer of a strided Q/K/V/O/dO/dQ/dK/dV tensor (head dim contiguous)."""
    if t.stride(-1) != 1 and t.shape[-1] > 1:
        raise ValueError("the head dimension must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


DQ_ALGOS = {"separate": L.ATTN_DQ_SEPARATE, "atomic": L.ATTN_DQ_ATOMIC, "stored_ds": L.ATTN_DQ_STORED_DS}


def make_shape(q, k, scale, causal, deterministic=False, cu_seqlens_q=None, cu_seqlens_k=None,
               max_seqlen_q=None, max_seqlen_k=None, dq_algo="separate", seqused_q=None, seqused_k=None,
               window=None, alibi_slopes=None, bias=None, dbias=None, max_workspace_bytes=0,
               cu_seqlens_host=None, dropout=None):
    """attn_shape_t for the given tensors (the dtype is q's).  dq_algo is
    "separate" (query-stationary dQ pass recomputing S and dP, no atomics),
    "stored_ds" (dS stored in the 16-bit I/O type by the dK/dV kernel, then
    dQ = dS K; bf16 and fp16 only, workspace grows with Sq x Sk) or "atomic".
    seqused_q / seqused_k (varlen only): int32 device tensors of per-sequence
    used lengths.  window = (left, right) selects the local mask: query i sees
    key j iff i + off - left <= j <= i + off + right (off = len_k - len_q, -1
    for an unbounded side), intersected with the causal bound when causal.
    alibi_slopes: fp32 device tensor [Hq]; the logits get -slope_h |i + off - j|.
    bias / dbias: tensors indexed [b, h, i, j] (b the sequence for varlen;
    keys contiguous, batch/head/row strides of 0 broadcast the bias); the
    bias is added to the logits and dbias receives dS.  Outside the atomic
    dQ mode the bias needs 16-byte aligned rows and base (pad the key axis
    to a multiple of 8 for 16-bit types).  dropout = (p, seed, offset): drop
    probability p in [0, 1) with the library's Philox4x32-10 keep mask (seed
    the 64-bit key, offset the 32-bit counter word); forward and backward
    must get the same triple.  max_workspace_bytes caps the stored-dS workspace (kv-head groups in
    chunks, or the separate mode when not even one fits).  cu_seqlens_host =
    (cu_q, cu_k): contiguous int32 CPU tensors holding the offsets, kept
    alive by the caller while the shape is used; with them the stored-dS
    workspace is sized exactly."""
    s = L.AttnShape()
    if q.dtype not in _DTYPES:
        s.dtype = -1
    else:
        s.dtype = _DTYPES[q.dtype]
    if cu_seqlens_q is None:
        s.batch, s.seqlen_q, s.num_heads_q, s.head_dim = q.shape
        s.seqlen_k, s.num_heads_kv = k.shape[1], k.shape[2]
        s.total_q, s.total_k = s.batch * s.seqlen_q, s.batch * s.seqlen_k
    else:
        s.total_q, s.num_heads_q, s.head_dim = q.shape
        s.total_k, s.num_heads_kv = k.shape[0], k.shape[1]
        s.batch = cu_seqlens_q.numel() - 1
        s.seqlen_q, s.seqlen_k = int(max_seqlen_q), int(max_seqlen_k)
        s.cu_seqlens_q = cu_seqlens_q.data_ptr()
        s.cu_seqlens_k = cu_seqlens_k.data_ptr()
    if seqused_q is not None:
        s.seqused_q = seqused_q.data_ptr()
    if seqused_k is not None:
        s.seqused_k = seqused_k.data_ptr()
    if window is not None:
        s.local = 1
        s.window_left, s.window_right = int(window[0]), int(window[1])
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != q.shape[-2]:
            raise ValueError("alibi_slopes must be a float32 tensor with one slope per q-head")
        s.alibi_slopes = alibi_slopes.data_ptr()
    for name, t in (("bias", bias), ("dbias", dbias)):
        if t is None:
            continue
        if t.dim() != 4 or (t.stride(3) != 1 and t.shape[3] > 1) or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a 4-d [b, h, i, j] tensor of q's dtype with contiguous keys")
        setattr(s, name, t.data_ptr())
        st = getattr(s, name + "_strides")
        st.batch, st.head, st.row = t.stride(0), t.stride(1), t.stride(2)
    if cu_seqlens_host is not None:
        for name, t in zip(("cu_seqlens_q_host", "cu_seqlens_k_host"), cu_seqlens_host):
            if t.device.type != "cpu" or t.dtype != torch.int32 or not t.is_contiguous():
                raise ValueError("host cu_seqlens must be contiguous int32 CPU tensors")
            setattr(s, name, t.data_ptr())
    s.max_workspace_bytes = int(max_workspace_bytes)
    if dropout is not None:
        p, seed, offset = dropout
        s.dropout_p = float(p)
        s.dropout_seed = int(seed) & 0xFFFFFFFFFFFFFFFF
        s.dropout_offset = int(offset) & 0xFFFFFFFF
    s.softmax_scale = float(scale)
    s.causal = int(bool(causal))
    s.deterministic = int(bool(deterministic))
    s.dq_algo = DQ_ALGOS[dq_algo] if isinstance(dq_algo, str) else int(dq_algo)
    return s


def _strides(shape, tensors):
    """attn_strides_t of the given tensors (the others keep the contiguous
    layout)."""
    varlen = bool(shape.cu_seqlens_q)
    st = L.Strides()
    d = shape.head_dim
    for name in L.STRIDE_TENSORS:
        is_k = name in ("k", "v", "dk", "dv")
        heads = shape.num_heads_kv if is_k else shape.num_heads_q
        seq = shape.seqlen_k if is_k else shape.seqlen_q
        t = tensors.get(name)
        x = getattr(st, name)
        if t is None:
            x.row, x.head = heads * d, d
            x.batch = 0 if varlen else seq * heads * d
        elif varlen:
            x.batch, x.row, x.head = 0, t.stride(0), t.stride(1)
        else:
            x.batch, x.row, x.head = t.stride(0), t.stride(1), t.stride(2)
    return st


def _call(name, shape, tensors, *args):
    """Call entry point `name` with shape.strides pointing at the strides of
    `tensors` for the duration of the call only."""
    st = _strides(shape, tensors)
    shape.strides = ctypes.addressof(st)
    try:
        return L.check(name, getattr(L.lib(), name)(ctypes.byref(shape), *args))
    finally:
        shape.strides = None


def attn_bwd_workspace_bytes(shape):
    return int(L.lib().attn_bwd_workspace_bytes(ctypes.byref(shape)))


def attn_fwd(shape, q, k, v, o, lse):
    return _call("attn_fwd", shape, dict(q=q, k=k, v=v, o=o),
                 _tptr(q), _tptr(k), _tptr(v), _tptr(o), _ptr(lse), _stream())


def attn_bwd_preprocess(shape, o, do, delta, workspace):
    return _call("attn_bwd_preprocess", shape, dict(o=o, dout=do),
                 _tptr(o), _tptr(do), _ptr(delta), _ptr(workspace), workspace.numel(), _stream())


def attn_bwd(shape, q, k, v, do, lse, delta, workspace, dk, dv):
    return _call("attn_bwd", shape, dict(q=q, k=k, v=v, dout=do, dk=dk, dv=dv),
                 _tptr(q), _tptr(k), _tptr(v), _tptr(do), _ptr(lse), _ptr(delta), _ptr(workspace),
                 workspace.numel(), _tptr(dk), _tptr(dv), _stream())


def attn_bwd_dq_postprocess(shape, workspace, dq, scale):
    return _call("attn_bwd_dq_postprocess", shape, dict(dq=dq),
                 _ptr(workspace), workspace.numel(), _tptr(dq), ctypes.c_float(scale), _stream())


def attn_bwd_full(shape, q, k, v, do, lse, delta, workspace, dq, dk, dv):
    return _call("attn_bwd_full", shape, dict(q=q, k=k, v=v, dout=do, dq=dq, dk=dk, dv=dv),
                 _tptr(q), _tptr(k), _tptr(v), _tptr(do), _ptr(lse), _ptr(delta), _ptr(workspace),
                 workspace.numel(), _tptr(dq), _tptr(dk), _tptr(dv), _stream())


def attn_bwd_full_noalloc(shape, q, k, v, o, do, lse, dq, dk, dv):
    """attn_bwd_preprocess + attn_bwd_full with D and the workspace in the
    library's fixed scratch memory (no allocation, no workspace argument)."""
    return _call("attn_bwd_full_noalloc", shape, dict(q=q, k=k, v=v, o=o, dout=do, dq=dq, dk=dk, dv=dv),
                 _tptr(q), _tptr(k), _tptr(v), _tptr(o), _tptr(do), _ptr(lse), _tptr(dq), _tptr(dk), _tptr(dv),
                 _stream())


def _lse_shape(shape, varlen):
    if varlen:
        return (shape.num_heads_q, shape.total_q)
    return (shape.batch, shape.num_heads_q, shape.seqlen_q)


def forward(q, k, v, scale, causal, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None,
            seqused_q=None, seqused_k=None, out=None, window=None, alibi_slopes=None, bias=None, dropout=None):
    """Plain forward: returns (o, lse).  ``out`` = (o, lse) writes into given
    buffers (rows past the used lengths keep their contents).  ``dropout`` =
    (p, seed, offset): see make_shape."""
    shape = make_shape(q, k, scale, causal, False, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                       seqused_q=seqused_q, seqused_k=seqused_k, window=window, alibi_slopes=alibi_slopes,
                       bias=bias, dropout=dropout)
    if out is not None:
        o, lse = out
    else:
        o = torch.empty_like(q)
        lse = torch.empty(_lse_shape(shape, cu_seqlens_q is not None), dtype=torch.float32, device=q.device)
    attn_fwd(shape, q, k, v, o, lse)
    return o, lse


class BackwardPlan:
    """Shape, workspace and D buffer of one backward problem, for repeated calls.

    ``run`` enqueues the three backward kernels (preprocess, main, dQ
    postprocess) on the current stream and writes dq, dk, dv.
    """

    def __init__(self, q, k, scale, causal, deterministic=False, cu_seqlens_q=None, cu_seqlens_k=None,
                 max_seqlen_q=None, max_seqlen_k=None, dq_algo="separate", seqused_q=None, seqused_k=None,
                 window=None, alibi_slopes=None, bias=None, dbias=None, max_workspace_bytes=0,
                 host_offsets=True, dropout=None):
        # host copies of the offsets size the stored-dS workspace exactly
        host = None
        if cu_seqlens_q is not None and host_offsets:
            host = (cu_seqlens_q.to("cpu", torch.int32).contiguous(), cu_seqlens_k.to("cpu", torch.int32).contiguous())
        self.shape = make_shape(q, k, scale, causal, deterministic, cu_seqlens_q, cu_seqlens_k,
                                max_seqlen_q, max_seqlen_k, dq_algo, seqused_q, seqused_k, window, alibi_slopes,
                                bias, dbias, max_workspace_bytes, host, dropout)
        self._keep = (cu_seqlens_q, cu_seqlens_k, seqused_q, seqused_k, alibi_slopes, bias, dbias, host)
        self.scale = float(scale)
        nbytes = attn_bwd_workspace_bytes(self.shape)
        if nbytes == 0:
            raise L.AttnError("attn_bwd_workspace_bytes", L.ATTN_ERR_BAD_SHAPE, "invalid shape")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
        self.delta = torch.empty(_lse_shape(self.shape, cu_seqlens_q is not None), dtype=torch.float32,
                                 device=q.device)

    def preprocess(self, o, do):
        attn_bwd_preprocess(self.shape, o, do, self.delta, self.workspace)

    def main(self, q, k, v, do, lse, dk, dv):
        attn_bwd(self.shape, q, k, v, do, lse, self.delta, self.workspace, dk, dv)

    def postprocess(self, dq):
        attn_bwd_dq_postprocess(self.shape, self.workspace, dq, self.scale)

    def run(self, q, k, v, o, do, lse, dq, dk, dv):
        """The three calls in order (dQ through the fp32 accumulator)."""
        self.preprocess(o, do)
        self.main(q, k, v, do, lse, dk, dv)
        self.postprocess(dq)

    def main_full(self, q, k, v, do, lse, dq, dk, dv):
        """attn_bwd_full: dK, dV and dQ in one call (dQ written straight in the
        I/O type by the separate and stored-dS modes)."""
        attn_bwd_full(self.shape, q, k, v, do, lse, self.delta, self.workspace, dq, dk, dv)

    def run_full(self, q, k, v, o, do, lse, dq, dk, dv):
        """Two calls: attn_bwd_preprocess, then attn_bwd_full."""
        self.preprocess(o, do)
        self.main_full(q, k, v, do, lse, dq, dk, dv)

    def error_flag(self):
        """Non-zero if an ordered (deterministic) wait gave up; reads the
        workspace's status word (synchronises the stream).  The status words
        are the last 256 bytes of the workspace prefix every dQ mode shares,
        which is the whole workspace of the separate mode."""
        base = L.AttnShape.from_buffer_copy(self.shape)
        base.dq_algo = L.ATTN_DQ_SEPARATE
        end = attn_bwd_workspace_bytes(base)
        return int(self.workspace[end - 256:end].view(torch.int32)[0].item())


def backward(q, k, v, o, do, lse, scale, causal, deterministic=False, cu_seqlens_q=None, cu_seqlens_k=None,
             max_seqlen_q=None, max_seqlen_k=None, dq_algo="separate", seqused_q=None, seqused_k=None,
             window=None, alibi_slopes=None, bias=None, dbias=None, dropout=None):
    """Full backward: returns (dq, dk, dv) (and fills dbias when given)."""
    plan = BackwardPlan(q, k, scale, causal, deterministic, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                        dq_algo, seqused_q, seqused_k, window, alibi_slopes, bias, dbias, dropout=dropout)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    plan.run(q, k, v, o, do, lse, dq, dk, dv)
    return dq, dk, dv
