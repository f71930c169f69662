"""Dropout on the attention probabilities: a counter-based random keep mask.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``.

The composable-kernel page ("block_fmha_bwd_dq_dk_dv_pipeline_trload_kr_ktr_vr.hpp
Source File", ``run``, STAGE 2 "Scale, Add bias, Mask, Softmax, Dropout")
drops elements of P after the softmax (``dropout.template Run``), feeds the
kept P to dV = P^T dO, marks dropped elements by their sign when forming dS,
and rescales dV, dK, dQ (and dBias) by ``rp_undrop`` = 1 / (1 - p).  The
pages give neither the random generator nor how its output maps to (row,
key) positions.  Readings taken (listed in the design notes):

* Generator: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random
  Numbers: As Easy as 1, 2, 3", SC 2011): a 128-bit counter and a 64-bit key,
  ten rounds; each round multiplies counter words 0 and 2 by 0xD2511F53 and
  0xCD9E8D57 into 64-bit products and forms (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1,
  lo0); the key grows by (0x9E3779B9, 0xBB67AE85) between rounds.
* One call covers a 4 x 4 block of (row, key) positions of one (sequence,
  q-head): counter = (key // 4, row // 4, sequence * Hq + q-head, offset),
  key = (seed mod 2^32, seed div 2^32).  Element (row r, key c) of the block
  takes byte c % 4 (least significant first) of output word r % 4.
* An element is kept iff its byte is >= t, t = round(256 p) (p in [0, 1);
  t <= 255), so the keep probability is (256 - t) / 256; kept values are
  scaled by 1 / (1 - p) with the p given.
"""

import numpy as np

__all__ = ["philox4x32", "dropout_threshold", "dropout_bytes", "dropout_keep"]

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32(counter, key, rounds=10):
    """Philox4x32 with ``rounds`` rounds.  counter: uint32 [..., 4]; key:
    uint32 [..., 2] (broadcast against counter's leading axes).  Returns
    uint32 [..., 4]."""
    c = np.asarray(counter, np.uint64) & _MASK32
    k = np.asarray(key, np.uint64) & _MASK32
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = k[..., 0], k[..., 1]
    for r in range(rounds):
        if r > 0:
            k0 = (k0 + np.uint64(_W0)) & _MASK32
            k1 = (k1 + np.uint64(_W1)) & _MASK32
        p0 = np.uint64(_M0) * c0          # < 2^64: exact in uint64
        p1 = np.uint64(_M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def dropout_threshold(p):
    """The byte threshold t = round(256 p) for a drop probability p in [0, 1)."""
    p = float(p)
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return min(255, int(np.floor(256.0 * p + 0.5)))


def dropout_bytes(seed, offset, bh, sq, sk):
    """uint8 [sq, sk]: the random byte of every (row, key) position of the
    (sequence, q-head) with index ``bh`` = sequence * Hq + q-head."""
    i4 = np.arange((sq + 3) // 4, dtype=np.uint64)
    j4 = np.arange((sk + 3) // 4, dtype=np.uint64)
    ctr = np.zeros((len(i4), len(j4), 4), np.uint64)
    ctr[..., 0] = j4[None, :]
    ctr[..., 1] = i4[:, None]
    ctr[..., 2] = np.uint64(bh)
    ctr[..., 3] = np.uint64(int(offset) & 0xFFFFFFFF)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    key = np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint64)
    words = philox4x32(ctr, key)                                  # [i4, j4, 4 words]
    # byte c of word r -> element (4 i4 + r, 4 j4 + c)
    b = words[..., :, None] >> (8 * np.arange(4, dtype=np.uint32))[None, None, None, :]
    b = (b & 0xFF).astype(np.uint8)                               # [i4, j4, r, c]
    full = b.transpose(0, 2, 1, 3).reshape(4 * len(i4), 4 * len(j4))
    return full[:sq, :sk]


def dropout_keep(seed, offset, bh, sq, sk, p):
    """Boolean [sq, sk] keep mask of one (sequence, q-head) for drop probability p."""
    return dropout_bytes(seed, offset, bh, sq, sk) >= dropout_threshold(p)
