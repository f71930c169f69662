"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments before any HIP call."""

import ctypes
from pathlib import Path
import os
import re

import pytest

from exact_attention_backward_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_bwd.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|size_t|int)\s+(attn_\w+)\s*\(", text, re.M)))


def test_header_declares_the_exports():
    assert declared_functions() == sorted(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = L.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert L.status_string(L.ATTN_OK) == "ok"
    for code in (1, 2, 3, 4, 5, 6):
        assert L.status_string(code) not in ("ok", "unknown status")
    assert L.status_string(99) == "unknown status"


def shape(**kw):
    s = L.AttnShape()
    base = dict(batch=2, num_heads_q=4, num_heads_kv=2, seqlen_q=100, seqlen_k=90, head_dim=128,
                total_q=0, total_k=0, softmax_scale=0.125, causal=1, deterministic=0, dtype=L.ATTN_DTYPE_BF16)
    base.update(kw)
    for k, v in base.items():
        setattr(s, k, v)
    return s


def ws_bytes(s):
    return L.lib().attn_bwd_workspace_bytes(ctypes.byref(s))


def test_workspace_size_formula():
    s = shape()
    # dQ accumulator [B, Hq, Sq, D] fp32, counters [B, Hq, ceil(Sq/64)] int32, 256 B status
    acc = 2 * 4 * 100 * 128 * 4
    acc = (acc + 255) // 256 * 256
    sem = (2 * 4 * 2 * 4 + 255) // 256 * 256
    assert ws_bytes(s) == acc + sem + 256
    # stored dS: + the block table + Hq x (visible (query tile, key tile) pairs) blocks of 32 x 128 bf16
    s = shape(dq_algo=L.ATTN_DQ_STORED_DS)
    table = 256                       # (batch + 1 + query tiles) int32
    # Sq = 100, Sk = 90 causal (off = -10): each 32-row tile's rows 10.. see key tile 0
    blocks = 4 * (2 * 4) * 1 * 32 * 128 * 2
    assert ws_bytes(s) == acc + sem + 256 + table + blocks
    # fp16 I/O: the same sizes (the accumulator is fp32, dS blocks 16-bit)
    assert ws_bytes(shape(dtype=L.ATTN_DTYPE_F16)) == acc + sem + 256
    assert ws_bytes(shape(dq_algo=L.ATTN_DQ_STORED_DS, dtype=L.ATTN_DTYPE_F16)) == acc + sem + 256 + table + blocks


def _visible_tile_pairs(lq, lk, bm, causal, window):
    """(query tile of bm rows, 128-key tile) pairs in which some query row sees
    some key, counted by brute force from the visibility rule of the header:
    key j is visible to row i iff i + off - left <= j <= i + off + right
    (off = lk - lq; causal sets right = 0; -1 / no window: unbounded)."""
    import numpy as np
    off = lk - lq
    big = 1 << 40
    left = window[0] if window is not None and window[0] >= 0 else big
    right = 0 if causal else (window[1] if window is not None and window[1] >= 0 else big)
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    vis = (j >= i + off - left) & (j <= i + off + right)
    nq, nk = -(-lq // bm), -(-lk // 128)
    pad = np.zeros((nq * bm, nk * 128), bool)
    pad[:lq, :lk] = vis
    return int(pad.reshape(nq, bm, nk, 128).any(axis=(1, 3)).sum())


@pytest.mark.parametrize("d,causal,window,lens", [
    (128, True, None, None),
    (64, True, None, None),
    (128, False, None, None),
    (128, False, (100, 40), None),
    (64, True, (300, -1), None),
    (128, True, None, ((300, 300), (1, 1), (700, 650), (0, 0), (129, 400))),
    (64, True, (70, -1), ((65, 90), (200, 200), (33, 31))),
])
def test_stored_ds_workspace_is_exactly_the_visible_blocks(d, causal, window, lens):
    """The stored-dS workspace holds one 32 x 128 block per 32-row block of
    each (query tile, key tile) pair with a visible element, per q-head: dense
    shapes, and varlen shapes whose offsets are also given in host memory."""
    bm = 32 if d == 128 else 64
    hq, hkv = 6, 3
    kw = dict(num_heads_q=hq, num_heads_kv=hkv, head_dim=d, causal=int(causal), dq_algo=L.ATTN_DQ_STORED_DS)
    if window is not None:
        kw.update(local=1, window_left=window[0], window_right=window[1])
    keep = []
    if lens is None:
        kw.update(batch=2, seqlen_q=700, seqlen_k=650)
        seqs = [(700, 650)] * 2
    else:
        seqs = list(lens)
        cq = (ctypes.c_int32 * (len(seqs) + 1))(*[sum(a for a, _ in seqs[:b]) for b in range(len(seqs) + 1)])
        ck = (ctypes.c_int32 * (len(seqs) + 1))(*[sum(b_ for _, b_ in seqs[:b]) for b in range(len(seqs) + 1)])
        keep += [cq, ck]
        kw.update(batch=len(seqs), seqlen_q=max(a for a, _ in seqs), seqlen_k=max(b_ for _, b_ in seqs),
                  total_q=cq[len(seqs)], total_k=ck[len(seqs)], cu_seqlens_q=0x1000, cu_seqlens_k=0x2000,
                  cu_seqlens_q_host=ctypes.addressof(cq), cu_seqlens_k_host=ctypes.addressof(ck))
    s = shape(**kw)
    base = shape(**dict(kw, dq_algo=L.ATTN_DQ_SEPARATE))
    pairs = sum(_visible_tile_pairs(a, b_, bm, causal, window) for a, b_ in seqs)
    tiles = len(seqs) * -(-kw["seqlen_q"] // bm) if lens is None else s.total_q // bm + len(seqs)
    table = (4 * (len(seqs) + 1 + tiles) + 255) // 256 * 256
    assert ws_bytes(s) == ws_bytes(base) + table + hq * pairs * (bm // 32) * 32 * 128 * 2
    if lens is not None:
        # without the host offsets: every sequence's full rectangle, bounded
        s.cu_seqlens_q_host = None
        bound = (s.total_q // 32 + (bm // 32) * len(seqs)) * -(-s.seqlen_k // 128)
        assert ws_bytes(s) == ws_bytes(base) + table + hq * bound * 32 * 128 * 2


def test_workspace_cap_chunks_kv_heads_or_falls_back():
    """max_workspace_bytes: the stored-dS blocks of as many whole kv-head
    groups as fit, or the separate mode's workspace when not one does."""
    kw = dict(batch=2, num_heads_q=8, num_heads_kv=4, seqlen_q=1000, seqlen_k=1000, causal=1,
              dq_algo=L.ATTN_DQ_STORED_DS)
    full = ws_bytes(shape(**kw))
    sep = ws_bytes(shape(**dict(kw, dq_algo=L.ATTN_DQ_SEPARATE)))
    pairs = 2 * _visible_tile_pairs(1000, 1000, 32, True, None)
    per_group = 2 * pairs * 32 * 128 * 2          # G = 2 q-heads per kv-head
    base = full - 4 * per_group
    assert base > sep
    assert ws_bytes(shape(**kw, max_workspace_bytes=full)) == full
    assert ws_bytes(shape(**kw, max_workspace_bytes=full - 1)) == base + 3 * per_group
    assert ws_bytes(shape(**kw, max_workspace_bytes=base + per_group)) == base + per_group
    assert ws_bytes(shape(**kw, max_workspace_bytes=base + per_group - 1)) == sep
    assert ws_bytes(shape(**kw, max_workspace_bytes=1)) == sep
    assert ws_bytes(shape(**kw, max_workspace_bytes=-1)) == 0    # invalid


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=100), L.ATTN_ERR_UNSUPPORTED),
    (dict(head_dim=264), L.ATTN_ERR_UNSUPPORTED),
    (dict(head_dim=136, dtype=L.ATTN_DTYPE_F32), L.ATTN_ERR_UNSUPPORTED),   # fp32: up to 128
    (dict(head_dim=0), L.ATTN_ERR_UNSUPPORTED),
    (dict(dtype=7), L.ATTN_ERR_UNSUPPORTED),
    (dict(num_heads_kv=3), L.ATTN_ERR_BAD_SHAPE),
    (dict(batch=0), L.ATTN_ERR_BAD_SHAPE),
    (dict(seqlen_q=-1), L.ATTN_ERR_BAD_SHAPE),
    (dict(causal=2), L.ATTN_ERR_BAD_SHAPE),
    (dict(softmax_scale=float("nan")), L.ATTN_ERR_BAD_SHAPE),
    (dict(batch=1, seqlen_q=(1 << 23) + 1, num_heads_q=16, num_heads_kv=16), L.ATTN_ERR_BAD_SHAPE),
    (dict(dq_algo=5), L.ATTN_ERR_UNSUPPORTED),
    (dict(local=2), L.ATTN_ERR_BAD_SHAPE),
    (dict(local=1, window_left=-2, window_right=3), L.ATTN_ERR_BAD_SHAPE),
    (dict(local=1, window_left=3, window_right=-7), L.ATTN_ERR_BAD_SHAPE),
    (dict(dq_algo=L.ATTN_DQ_STORED_DS, dtype=L.ATTN_DTYPE_F32), L.ATTN_ERR_UNSUPPORTED),
])
def test_invalid_shapes_rejected(kw, status):
    s = shape(**kw)
    assert ws_bytes(s) == 0
    fake = ctypes.c_void_p(0x1000)
    rc = L.lib().attn_bwd(ctypes.byref(s), fake, fake, fake, fake, fake, fake, fake, 1 << 40, fake, fake, None)
    assert rc == status


def test_seqused_needs_varlen_and_alignment():
    assert ws_bytes(shape(seqused_q=0x1000)) == 0
    assert ws_bytes(shape(seqused_k=0x1000)) == 0
    s = shape(cu_seqlens_q=0x1000, cu_seqlens_k=0x2000, total_q=500, total_k=400, seqused_q=0x3000, seqused_k=0x4000)
    assert ws_bytes(s) == ws_bytes(shape(cu_seqlens_q=0x1000, cu_seqlens_k=0x2000, total_q=500, total_k=400))
    fake = ctypes.c_void_p(0x1000)
    s = shape(cu_seqlens_q=0x1000, cu_seqlens_k=0x2000, total_q=500, total_k=400, seqused_q=0x3002)
    rc = L.lib().attn_bwd(ctypes.byref(s), fake, fake, fake, fake, fake, fake, fake, 1 << 40, fake, fake, None)
    assert rc == L.ATTN_ERR_MISALIGNED
    s = shape(seqused_k=0x3000)
    rc = L.lib().attn_bwd(ctypes.byref(s), fake, fake, fake, fake, fake, fake, fake, 1 << 40, fake, fake, None)
    assert rc == L.ATTN_ERR_BAD_SHAPE


def test_head_dims_accepted_and_workspace_padded():
    """Any multiple of 8 up to 256 (fp32: 128); the accumulator is sized for
    the padded head dim (64, 128 or 256); above 128 the atomic mode runs (and
    is sized) as the separate one."""
    for d, pad in ((8, 64), (40, 64), (64, 64), (72, 128), (96, 128), (128, 128), (136, 256), (200, 256),
                   (256, 256)):
        assert ws_bytes(shape(head_dim=d)) == ws_bytes(shape(head_dim=pad))
    assert ws_bytes(shape(head_dim=256)) > ws_bytes(shape(head_dim=128))
    for d in (136, 256):
        assert ws_bytes(shape(head_dim=d, dq_algo=L.ATTN_DQ_ATOMIC)) == ws_bytes(shape(head_dim=d))


def _strides(**over):
    st = L.Strides()
    for name in L.STRIDE_TENSORS:
        x = getattr(st, name)
        heads = 2 if name in ("k", "v", "dk", "dv") else 4
        seq = 90 if name in ("k", "v", "dk", "dv") else 100
        x.batch, x.row, x.head = seq * heads * 128, heads * 128, 128
    for key, (b, r, h) in over.items():
        x = getattr(st, key)
        x.batch, x.row, x.head = b, r, h
    return st


def test_strides_validated():
    fake = ctypes.c_void_p(0x1000)
    lib = L.lib()

    def call(st):
        s = shape()
        s.strides = ctypes.addressof(st)
        return lib.attn_bwd(ctypes.byref(s), fake, fake, fake, fake, fake, fake, fake, 1 << 40, fake, fake, None)

    def ws(st):
        s = shape()
        s.strides = ctypes.addressof(st)
        return ws_bytes(s)

    base = ws_bytes(shape())
    # packed QKV rows (3 H D) and a head-major dO: accepted, same workspace
    assert ws(_strides(q=(100 * 3 * 4 * 128, 3 * 4 * 128, 128), dout=(4 * 100 * 128, 128, 100 * 128))) == base
    assert call(_strides(q=(-8, 512, 128))) == L.ATTN_ERR_BAD_SHAPE
    assert call(_strides(dk=(8, -512, 128))) == L.ATTN_ERR_BAD_SHAPE
    assert call(_strides(v=(100, 256, 128))) == L.ATTN_ERR_MISALIGNED     # batch stride not 16-byte aligned
    assert call(_strides(dq=(0, 516, 128))) == L.ATTN_ERR_MISALIGNED      # row stride not 16-byte aligned
    assert call(_strides(o=(0, 512, 132))) == L.ATTN_ERR_MISALIGNED       # head stride not 16-byte aligned
    assert call(_strides(q=(0, 1 << 24, 128))) == L.ATTN_ERR_BAD_SHAPE    # a sequence's rows past 2 GiB


def test_window_sizes_accepted():
    base = ws_bytes(shape())
    for left, right in [(-1, -1), (0, 0), (5, -1), (-1, 7), (1 << 30, (1 << 31) - 1)]:
        for causal in (0, 1):
            assert ws_bytes(shape(local=1, window_left=left, window_right=right, causal=causal)) == base
    # the window fields are ignored without local
    assert ws_bytes(shape(local=0, window_left=-9, window_right=-9)) == base


def test_alibi_slopes_alignment():
    base = ws_bytes(shape())
    assert ws_bytes(shape(alibi_slopes=0x1000)) == base
    s = shape(alibi_slopes=0x1002)
    assert ws_bytes(s) == 0
    fake = ctypes.c_void_p(0x1000)
    rc = L.lib().attn_bwd(ctypes.byref(s), fake, fake, fake, fake, fake, fake, fake, 1 << 40, fake, fake, None)
    assert rc == L.ATTN_ERR_MISALIGNED


def test_bias_alignment_and_range_by_dq_mode():
    """Every dQ mode takes a bias and dBias; outside the atomic mode the bias
    is copied in 16-byte chunks (base, batch, head and row steps 16-byte
    aligned) and 64 rows of bias or dBias must stay inside a 32-bit offset."""
    fake = ctypes.c_void_p(0x1000)
    for algo in (L.ATTN_DQ_ATOMIC, L.ATTN_DQ_SEPARATE, L.ATTN_DQ_STORED_DS):
        base = ws_bytes(shape(dq_algo=algo))
        s = shape(dq_algo=algo, bias=0x1000, dbias=0x2000)
        s.bias_strides.row = s.dbias_strides.row = 96
        s.bias_strides.head = s.dbias_strides.head = 96 * 100
        assert ws_bytes(s) == base
        for field, value, aligned_ok in (("bias", 0x1008, False), ("dbias", 0x1002, True)):
            s = shape(dq_algo=algo, **{field: value})
            getattr(s, field + "_strides").row = 96
            assert (ws_bytes(s) == base) == (algo == L.ATTN_DQ_ATOMIC or aligned_ok), (algo, field)
        s = shape(dq_algo=algo, bias=0x1000)
        s.bias_strides.row = 90   # 180 bytes: not a multiple of 16
        want_ok = algo == L.ATTN_DQ_ATOMIC
        assert (ws_bytes(s) == base) == want_ok
        if not want_ok:
            rc = L.lib().attn_bwd(ctypes.byref(s), fake, fake, fake, fake, fake, fake, fake, 1 << 40, fake, fake, None)
            assert rc == L.ATTN_ERR_MISALIGNED
        s = shape(dq_algo=algo, dbias=0x1000)
        s.dbias_strides.row = 1 << 24   # 64 rows of 32 MiB
        assert (ws_bytes(s) == base) == (algo == L.ATTN_DQ_ATOMIC)
    s = shape(dq_algo=L.ATTN_DQ_ATOMIC, bias=0x1001)
    assert ws_bytes(s) == 0   # misaligned for bf16
    s = shape(dq_algo=L.ATTN_DQ_ATOMIC, dbias=0x1000)
    s.dbias_strides.row = -4
    assert ws_bytes(s) == 0


def test_dropout_probability_validated():
    base = ws_bytes(shape())
    for p_drop, ok in ((0.0, True), (0.5, True), (0.999, True), (1.0, False), (-0.1, False), (float("nan"), False)):
        s = shape(dropout_p=p_drop, dropout_seed=(1 << 63) + 5, dropout_offset=7)
        assert (ws_bytes(s) == base) == ok, p_drop
    fake = ctypes.c_void_p(0x1000)
    s = shape(dropout_p=1.5)
    assert L.lib().attn_fwd(ctypes.byref(s), fake, fake, fake, fake, fake, None) == L.ATTN_ERR_BAD_SHAPE


def test_shape_struct_layout_matches_header(tmp_path):
    """The ctypes mirror of attn_shape_t has the C layout (compiled from the header)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    fields = [f[0] for f in L.AttnShape._fields_]
    sub = {"bias_strides": ("batch", "row", "head"), "dbias_strides": ("batch", "row", "head")}
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "attn_bwd.h"\nint main(void) {\n'
                   '    printf("%zu\\n", sizeof(attn_shape_t));\n'
                   + "".join(f'    printf("%zu\\n", offsetof(attn_shape_t, {f}));\n' for f in fields)
                   + "".join(f'    printf("%zu\\n", offsetof(attn_shape_t, {f}.{g}));\n' for f in sub for g in sub[f])
                   + "    return 0;\n}\n")
    exe = tmp_path / "layout"
    inc = Path(__file__).resolve().parents[1] / "include"
    subprocess.run(["gcc", "-std=c99", "-I", str(inc), str(src), "-o", str(exe)], check=True)
    out = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()]
    assert out[0] == ctypes.sizeof(L.AttnShape)
    want = [getattr(L.AttnShape, f).offset for f in fields]
    want += [getattr(L.AttnShape, f).offset + getattr(L.TensorStrides, g).offset for f in sub for g in sub[f]]
    assert out[1:] == want


def test_varlen_needs_both_offsets_and_totals():
    s = shape(cu_seqlens_q=0x1000)
    assert ws_bytes(s) == 0
    s = shape(cu_seqlens_q=0x1000, cu_seqlens_k=0x2000, total_q=0, total_k=5)
    assert ws_bytes(s) == 0
    s = shape(cu_seqlens_q=0x1000, cu_seqlens_k=0x2000, total_q=500, total_k=400)
    assert ws_bytes(s) > 0


def test_null_and_misaligned_pointers_rejected():
    s = shape()
    fake = ctypes.c_void_p(0x1000)
    bad = ctypes.c_void_p(0x1004)
    lib = L.lib()
    assert lib.attn_bwd(ctypes.byref(s), None, fake, fake, fake, fake, fake, fake, 1 << 40, fake, fake,
                        None) == L.ATTN_ERR_NULL_ARG
    assert lib.attn_bwd(ctypes.byref(s), fake, fake, fake, fake, fake, fake, None, 1 << 40, fake, fake,
                        None) == L.ATTN_ERR_NULL_ARG
    assert lib.attn_bwd(ctypes.byref(s), bad, fake, fake, fake, fake, fake, fake, 1 << 40, fake, fake,
                        None) == L.ATTN_ERR_MISALIGNED
    assert lib.attn_bwd_preprocess(ctypes.byref(s), fake, fake, fake, fake, 16, None) == L.ATTN_ERR_BAD_SHAPE
    assert lib.attn_bwd_dq_postprocess(ctypes.byref(s), None, 1 << 40, fake, ctypes.c_float(1.0),
                                       None) == L.ATTN_ERR_NULL_ARG
    assert lib.attn_fwd(ctypes.byref(s), fake, fake, fake, bad, fake, None) == L.ATTN_ERR_MISALIGNED
    assert lib.attn_fwd(None, fake, fake, fake, fake, fake, None) == L.ATTN_ERR_NULL_ARG
    # attn_bwd_full: dq is required and aligned like the other tensors
    assert lib.attn_bwd_full(ctypes.byref(s), fake, fake, fake, fake, fake, fake, fake, 1 << 40, None, fake, fake,
                             None) == L.ATTN_ERR_NULL_ARG
    assert lib.attn_bwd_full(ctypes.byref(s), fake, fake, fake, fake, fake, fake, fake, 1 << 40, bad, fake, fake,
                             None) == L.ATTN_ERR_MISALIGNED
    assert lib.attn_bwd_full(ctypes.byref(s), fake, fake, fake, fake, fake, fake, fake, 16, fake, fake, fake,
                             None) == L.ATTN_ERR_BAD_SHAPE


def test_noalloc_entry_point_validates_before_any_hip_call():
    """attn_bwd_full_noalloc: null and misaligned pointers, and problems
    larger than its fixed scratch, are rejected before any HIP call."""
    lib = L.lib()
    fake = ctypes.c_void_p(0x1000)
    bad = ctypes.c_void_p(0x1008)
    s = shape(dq_algo=L.ATTN_DQ_SEPARATE)
    args = [fake] * 9
    for i in range(9):
        a = list(args)
        a[i] = None
        assert lib.attn_bwd_full_noalloc(ctypes.byref(s), *a, None) == L.ATTN_ERR_NULL_ARG, i
        a[i] = bad
        assert lib.attn_bwd_full_noalloc(ctypes.byref(s), *a, None) == L.ATTN_ERR_MISALIGNED, i
    assert lib.attn_bwd_full_noalloc(None, *args, None) == L.ATTN_ERR_NULL_ARG
    # D alone of 2^24 (row, head) pairs fills the 64 MiB scratch
    big = shape(batch=64, seqlen_q=1 << 15, seqlen_k=1 << 15, num_heads_q=8, num_heads_kv=8,
                dq_algo=L.ATTN_DQ_SEPARATE)
    assert 4 * 64 * (1 << 15) * 8 >= L.NOALLOC_SCRATCH_BYTES
    assert lib.attn_bwd_full_noalloc(ctypes.byref(big), *args, None) == L.ATTN_ERR_SCRATCH
    # the stored-dS blocks of B4 H16 S4096 (1 GiB) do not fit either, nor the
    # atomic mode's accumulator at that size (128 MiB)
    for algo in (L.ATTN_DQ_STORED_DS, L.ATTN_DQ_ATOMIC):
        hs = shape(batch=4, seqlen_q=4096, seqlen_k=4096, num_heads_q=16, num_heads_kv=16, dq_algo=algo)
        assert lib.attn_bwd_full_noalloc(ctypes.byref(hs), *args, None) == L.ATTN_ERR_SCRATCH
    # invalid shapes keep their own status
    assert lib.attn_bwd_full_noalloc(ctypes.byref(shape(head_dim=100)), *args, None) == L.ATTN_ERR_UNSUPPORTED
    assert L.status_string(L.ATTN_ERR_SCRATCH) != "unknown status"
