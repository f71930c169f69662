"""ctypes binding of libattnbwd.so (the C ABI declared in include/attn_bwd.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind these symbols.  There is no fallback: if the shared library is
missing, loading raises.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; ATTN_BWD_LIB may name another build of the same sources
LIB_PATH = os.environ.get("ATTN_BWD_LIB") or os.path.join(_PKG, "libattnbwd.so")

ATTN_OK = 0
ATTN_ERR_NULL_ARG = 1
ATTN_ERR_BAD_SHAPE = 2
ATTN_ERR_UNSUPPORTED = 3
ATTN_ERR_MISALIGNED = 4
ATTN_ERR_HIP = 5
ATTN_ERR_SCRATCH = 6

# bytes of the no-allocation entry point's scratch memory (per GPU)
NOALLOC_SCRATCH_BYTES = 64 << 20

ATTN_DTYPE_F32 = 0
ATTN_DTYPE_BF16 = 1
ATTN_DTYPE_F16 = 2

ATTN_DQ_SEPARATE = 0
ATTN_DQ_ATOMIC = 1
ATTN_DQ_STORED_DS = 2

EXPORTS = (
    "attn_status_string",
    "attn_bwd_workspace_bytes",
    "attn_fwd",
    "attn_bwd_preprocess",
    "attn_bwd",
    "attn_bwd_dq_postprocess",
    "attn_bwd_full",
    "attn_bwd_full_noalloc",
)


class TensorStrides(ctypes.Structure):
    """Mirror of attn_tensor_strides_t (elements)."""
    _fields_ = [("batch", ctypes.c_int64), ("row", ctypes.c_int64), ("head", ctypes.c_int64)]


STRIDE_TENSORS = ("q", "k", "v", "o", "dout", "dq", "dk", "dv")


class Strides(ctypes.Structure):
    """Mirror of attn_strides_t."""
    _fields_ = [(n, TensorStrides) for n in STRIDE_TENSORS]


class AttnShape(ctypes.Structure):
    """Mirror of attn_shape_t."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads_q", ctypes.c_int32),
        ("num_heads_kv", ctypes.c_int32),
        ("seqlen_q", ctypes.c_int32),
        ("seqlen_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("total_k", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("softmax_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("deterministic", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("dq_algo", ctypes.c_int32),
        ("seqused_q", ctypes.c_void_p),
        ("seqused_k", ctypes.c_void_p),
        ("local", ctypes.c_int32),
        ("window_left", ctypes.c_int32),
        ("window_right", ctypes.c_int32),
        ("alibi_slopes", ctypes.c_void_p),
        ("strides", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("bias_strides", TensorStrides),
        ("dbias", ctypes.c_void_p),
        ("dbias_strides", TensorStrides),
        ("max_workspace_bytes", ctypes.c_int64),
        ("cu_seqlens_q_host", ctypes.c_void_p),
        ("cu_seqlens_k_host", ctypes.c_void_p),
        ("dropout_seed", ctypes.c_uint64),
        ("dropout_p", ctypes.c_float),
        ("dropout_offset", ctypes.c_uint32),
    ]


class AttnError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: {text} (status {status})")
        self.status = status


_lib = None


def lib():
    """The loaded library (loaded once).  Raises OSError if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise OSError(f"{LIB_PATH} not found: build it with `python -m exact_attention_backward_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        sp = ctypes.POINTER(AttnShape)
        L.attn_status_string.argtypes = [i32]
        L.attn_status_string.restype = ctypes.c_char_p
        L.attn_bwd_workspace_bytes.argtypes = [sp]
        L.attn_bwd_workspace_bytes.restype = sz
        L.attn_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp]
        L.attn_fwd.restype = i32
        L.attn_bwd_preprocess.argtypes = [sp, vp, vp, vp, vp, sz, vp]
        L.attn_bwd_preprocess.restype = i32
        L.attn_bwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.attn_bwd.restype = i32
        L.attn_bwd_dq_postprocess.argtypes = [sp, vp, sz, vp, ctypes.c_float, vp]
        L.attn_bwd_dq_postprocess.restype = i32
        L.attn_bwd_full.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp]
        L.attn_bwd_full.restype = i32
        if hasattr(L, "attn_bwd_full_noalloc"):   # absent from builds that predate it
            L.attn_bwd_full_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
            L.attn_bwd_full_noalloc.restype = i32
        _lib = L
    return _lib


def status_string(status):
    return lib().attn_status_string(int(status)).decode()


def check(fn, status):
    if status != ATTN_OK:
        raise AttnError(fn, status, status_string(status))
    return status
