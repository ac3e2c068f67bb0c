"""Dropout masks for the PTB layer from a counter-based generator, in plain
numpy.

TEST INFRASTRUCTURE. Only the test-suite, the package's smoke entry and the
benchmark's CPU-baseline leg may import or run this module; it shares no code
with the HIP path, which implements the same published generator on its own.

Page followed: [MS] Zhongzhu Zhou, "MegaScale: ByteDance 如何在 12,288 块 GPU 上
实现 55% MFU 的大规模 LLM 训练", section 1.3: MegaScale fuses dropout into its
normalisation kernel, and selective recompute keeps the activations of the
cheap operators, dropout's among them.  The page names neither the generator
nor where the dropout sits; the readings taken:

* where: on the block's branch output, before the residual add.  Parallel
  block (eq (4)): y = x + M * (Attn(LN x) W_o + MLP(LN x)), one mask over
  [T, h]; the two branches are summed in one accumulator ([O | FC2] is one
  product), so the branch output of the block is that sum.  Serial block
  (eq (3)): x1 = x + M1 * (Attn(LN1 x) W_o), y = x1 + M2 * MLP(LN2 x1).
  M holds 0 for a dropped element and 1 / (1 - p) for a kept one.
* the generator: Philox-4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror,
  D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11): a
  keyed bijection of a 128-bit counter, ten rounds, so that every mask bit is
  a pure function of (seed, stream, element) and the backward can regenerate
  the mask instead of storing it ("kept" as the key that reproduces it).
* element e = t h + c of a [T, h] tensor: key (seed mod 2^32, seed >> 32),
  counter (e >> 2, stream, 0, 0), output word e & 3; kept iff that word is
  >= floor(p 2^32) with p the fp32 dropout rate; stream = 2 * layer for the
  parallel block's mask and the serial block's attention branch, 2 * layer + 1
  for the serial block's MLP branch.
* the scale 1 / (1 - p) of kept elements is computed from the same fp32 p.
"""
from __future__ import annotations

import numpy as np

# Philox-4x32 constants (Salmon et al., SC'11): the two round multipliers and
# the two Weyl increments of the key schedule.
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox-4x32 with 10 rounds on arrays of counters (four 32-bit words)
    under the key (k0, k1).  A round multiplies counter words 0 and 2 by the
    two round constants into 64-bit products and forms the new counter
    (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); between
    rounds the key words advance by the two Weyl constants (mod 2^32).
    Returns the four output words as uint32 arrays."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3)]
    k = [np.uint64(int(k0) & 0xFFFFFFFF), np.uint64(int(k1) & 0xFFFFFFFF)]
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for rnd in range(10):
        if rnd:
            k = [(k[0] + np.uint64(PHILOX_W0)) & _MASK32, (k[1] + np.uint64(PHILOX_W1)) & _MASK32]
        p0 = m0 * c[0]            # < 2^64: exact in uint64
        p1 = m1 * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ k[0], p1 & _MASK32,
             (p0 >> np.uint64(32)) ^ c[3] ^ k[1], p0 & _MASK32]
    return [x.astype(np.uint32) for x in c]


def dropout_threshold(p) -> int:
    """floor(p * 2^32) of the fp32 rate p, 0 <= p < 1 (exact: p has at most 24
    significant bits)."""
    p32 = float(np.float32(p))
    if not 0.0 <= p32 < 1.0:
        raise ValueError("dropout rate must be in [0, 1)")
    return int(np.floor(p32 * 4294967296.0))


def dropout_scale(p) -> float:
    """1 / (1 - p) of the fp32 rate p, in fp64."""
    return 1.0 / (1.0 - float(np.float32(p)))


def dropout_keep(n: int, seed: int, stream: int, p) -> np.ndarray:
    """Boolean keep mask of elements 0 .. n-1 of one stream."""
    if n == 0:
        return np.zeros(0, dtype=bool)
    groups = (n + 3) // 4
    j = np.arange(groups, dtype=np.uint64)
    words = philox4x32_10(j, np.full(groups, stream, dtype=np.uint64), 0, 0,
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.stack(words, axis=1).reshape(-1)[:n]       # element e -> word e & 3 of group e >> 2
    return w >= np.uint32(dropout_threshold(p))


def dropout_multiplier(shape, seed: int, stream: int, p) -> np.ndarray:
    """The multiplier M of a [T, h] branch output: 1 / (1 - p) where kept, 0
    where dropped (all ones for p = 0)."""
    n = int(np.prod(shape))
    keep = dropout_keep(n, seed, stream, p)
    return np.where(keep, dropout_scale(p), 0.0).reshape(shape)


def layer_stream(layer: int, branch: int = 0) -> int:
    """Generator stream of a layer's mask: 2 * layer for the parallel block
    (and the serial block's attention branch), + 1 for the serial MLP branch."""
    return 2 * layer + branch
