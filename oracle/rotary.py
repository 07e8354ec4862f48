"""CPU oracle for attention with rotary position embeddings, in float64.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the library never does.

"TLX Block Attention" (summary; the section on why the kernel is bound by memory
bandwidth) fuses rotary embeddings into the block attention kernels and names
the avoided memory traffic as the gain, without defining the embedding. Readings
taken here, each the common form of rotary position embedding:
  * Query and key rows are rotated by their token position before the scores
    are formed; values are not rotated. The attention is then the plain
    block-diagonal attention of the rotated rows.
  * Column pairs are (i, i + D/2) for i < D/2 (the half-split form), with angle
    pos * theta_i and theta_i = base ** (-2 i / D): a pair (x1, x2) becomes
    (x1 cos a - x2 sin a, x2 cos a + x1 sin a).
  * The position of a token is its index inside its own sequence.
  * The backward returns gradients with respect to the unrotated query and key
    rows: the gradients of the rotated rows, rotated back by the same angles.
  * The same embedding applies to jagged self-attention (causal or not): the
    attention of the rotated rows over the original offsets.
"""
from __future__ import annotations

import numpy as np

from .attention import block_diag_backward, block_diag_forward, jagged_backward, jagged_forward


def rope_freqs(head_dim, base):
    """theta_i = base ** (-2 i / D) for i in [0, D/2)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * i / head_dim)


def token_positions(offsets):
    """Index of every token inside its own sequence, [T] int64."""
    off = np.asarray(offsets, dtype=np.int64)
    pos = np.empty(int(off[-1]), dtype=np.int64)
    for s, e in zip(off[:-1], off[1:]):
        pos[s:e] = np.arange(e - s)
    return pos


def rope(x, positions, base, inverse=False):
    """Rotate the rows of x [T, H, D] by the angles of their positions.

    inverse=True applies the transposed rotation (angle negated), which undoes it
    and maps a gradient of the rotated rows back to the unrotated ones.
    """
    d = x.shape[-1]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_freqs(d, base)[None, :]
    if inverse:
        ang = -ang
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def block_diag_rope_forward(q, k, v, offsets, scale, base, block=64):
    """Block-diagonal attention of the rotated queries and keys -> out [T,H,D]."""
    pos = token_positions(offsets)
    return block_diag_forward(rope(q, pos, base), rope(k, pos, base), v, offsets, scale, block)


def block_diag_rope_backward(q, k, v, do, offsets, scale, base, block=64):
    """(dq, dk, dv) with respect to the unrotated q and k."""
    pos = token_positions(offsets)
    dqr, dkr, dv = block_diag_backward(rope(q, pos, base), rope(k, pos, base), v, do, offsets,
                                       scale, block)
    return rope(dqr, pos, base, inverse=True), rope(dkr, pos, base, inverse=True), dv


def jagged_rope_forward(q, k, v, offsets, scale, base, causal=False, window=0):
    """Jagged attention of the rotated queries and keys -> (out, lse)."""
    pos = token_positions(offsets)
    return jagged_forward(rope(q, pos, base), rope(k, pos, base), v, offsets, scale, causal, window)


def jagged_rope_backward(q, k, v, do, offsets, scale, base, causal=False, window=0):
    """(dq, dk, dv) with respect to the unrotated q and k."""
    pos = token_positions(offsets)
    dqr, dkr, dv = jagged_backward(rope(q, pos, base), rope(k, pos, base), v, do, offsets, scale,
                                   causal, window)
    return rope(dqr, pos, base, inverse=True), rope(dkr, pos, base, inverse=True), dv
