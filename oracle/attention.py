"""CPU oracle for jagged attention, forward and backward, in float64.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the library never does.

What it computes is the plain definition of exact softmax attention, which the
flash formulation reaches up to rounding order (the online-softmax loop with its
running row max, running row sum and correction factor, shown in "TLX Block
Attention", section 2, reproduces softmax(S) V exactly). So the oracle evaluates
the definition directly, one sequence at a time, with no tiling beyond splitting
very long sequences into independent blocks of query rows (each block sees all of
its keys, so nothing is rescaled or merged).

Readings of points the pages leave open:
  * S = scale * Q K^T with scale an argument (the pages' loop shows no scale).
  * Natural-exponent softmax; the saved log-sum-exp is lse = m + ln(l)
    ("TLX Block Attention", section 2: L = m + log(l) kept for the backward).
  * Causal means: inside a sequence, query i attends keys j <= i.
  * Sliding window (named by the pages as a modelling variant, never defined):
    a causal window of W keys, query i attends keys j with i - W < j <= i.
  * Backward: P is rebuilt from Q and K, Di = rowsum(dO * O) ("TLX Block
    Attention", sections 2 and 4), dS = P * (dP - Di), dQ = scale dS K,
    dK = scale dS^T Q, dV = P^T dO.
  * Broadcast-Q: one dense Q is shared by every sequence, so dQ is the sum over
    sequences of each sequence's dQ ("Jagged Flash Attention for GEM",
    backward / dQ section).
  * Block-diagonal: the sequence is split into fixed 64-token groups that attend
    only within themselves ("TLX Block Attention", section 1), i.e. jagged
    attention over offsets refined to every 64 tokens; no lse is produced.
  * A broadcast sequence with no keys yields out = 0, lse = -inf, and adds nothing
    to dQ (convention; the pages do not cover it).
  * Block-sparse (the pages name block-sparse patterns as a modelling variant and
    contrast a 256-token minimum tile with the 64-token blocks their models need,
    "TLX Block Attention", section 1; "Jagged Flash Attention for GEM", the
    section on generative models): each sequence is cut into 64-token blocks
    (the last one partial), and a boolean matrix per sequence says which key
    blocks each query block attends; query i attends key j of its own sequence
    iff mask[i // 64][j // 64], and with causal also only if j <= i (the
    generative-model case the GEM page names). A query row that keeps no key
    gets out = 0 and lse = -inf and contributes nothing to the gradients (the
    same convention as an empty broadcast sequence).

Layouts: packed tensors are [T, H, D] (token-major, no padding) with int32
offsets [B+1]; jagged lse is [H, T]; broadcast Q/dQ are [Lq, H, D], broadcast
out/dO are [B, Lq, H, D] and broadcast lse is [B, H, Lq]. Block-sparse masks are
a list with one [n_b, n_b] boolean array per sequence, n_b = ceil(L_b / 64); the
flat form concatenates them row-major (uint8).
All array arguments are float64 (bf16 inputs widened exactly).
"""
from __future__ import annotations

import numpy as np

ROW_BLOCK = 1024
SPARSE_BLOCK = 64


def _row_blocks(n):
    for r0 in range(0, n, ROW_BLOCK):
        yield r0, min(n, r0 + ROW_BLOCK)


def _probs(q_blk, k, scale, causal, r0, window=0, bmask=None):
    """Softmax probabilities P [rows, Lk] and the row max / row sum.

    Rows are queries r0..r0+rows-1 of the sequence; with causal, query i keeps
    keys j <= i only, and with a window W > 0 also only keys j > i - W. With a
    block mask, query i keeps key j iff bmask[i // 64, j // 64]. A row that keeps
    no key has P = 0, max -inf and sum 0.
    """
    s = scale * (q_blk @ k.T)
    i = np.arange(r0, r0 + q_blk.shape[0])[:, None]
    j = np.arange(k.shape[0])[None, :]
    if causal:
        keep = j <= i
        if window:
            keep &= j > i - window
        s = np.where(keep, s, -np.inf)
    if bmask is not None:
        s = np.where(bmask[i // SPARSE_BLOCK, j // SPARSE_BLOCK], s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - np.where(np.isfinite(m), m, 0.0)[:, None])
    l = e.sum(axis=1)
    return e / np.where(l > 0, l, 1.0)[:, None], m, l


def seq_forward(q, k, v, scale, causal=False, window=0, bmask=None):
    """One sequence, one head. q [Lq,D], k/v [Lk,D] -> out [Lq,D], lse [Lq]."""
    Lq, Lk = q.shape[0], k.shape[0]
    out = np.zeros((Lq, v.shape[1]))
    lse = np.full(Lq, -np.inf)
    if Lq == 0 or Lk == 0:
        return out, lse
    for r0, r1 in _row_blocks(Lq):
        p, m, l = _probs(q[r0:r1], k, scale, causal, r0, window, bmask)
        out[r0:r1] = p @ v
        with np.errstate(divide="ignore"):
            lse[r0:r1] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out, lse


def seq_backward(q, k, v, do, scale, causal=False, window=0, bmask=None):
    """Gradients of <out, dO> for one sequence and head -> dq, dk, dv."""
    Lq, Lk = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if Lq == 0 or Lk == 0:
        return dq, dk, dv
    for r0, r1 in _row_blocks(Lq):
        p, _, _ = _probs(q[r0:r1], k, scale, causal, r0, window, bmask)
        o = p @ v
        d_o = do[r0:r1]
        di = np.sum(d_o * o, axis=1)            # Di = rowsum(dO * O)
        dv += p.T @ d_o                          # dV = P^T dO
        dp = d_o @ v.T                           # dP = dO V^T
        ds = p * (dp - di[:, None])              # dS = P * (dP - Di)
        dq[r0:r1] = scale * (ds @ k)             # dQ = scale dS K
        dk += scale * (ds.T @ q[r0:r1])          # dK = scale dS^T Q
    return dq, dk, dv


def _seqs(offsets):
    off = np.asarray(offsets, dtype=np.int64)
    return [(int(off[b]), int(off[b + 1])) for b in range(len(off) - 1)]


def jagged_forward(q, k, v, offsets, scale, causal=False, window=0):
    """Packed self-attention: q/k/v [T,H,D] -> out [T,H,D], lse [H,T]."""
    T, H, D = q.shape
    out = np.zeros((T, H, v.shape[2]))
    lse = np.full((H, T), -np.inf)
    for s, e in _seqs(offsets):
        for h in range(H):
            o, l = seq_forward(q[s:e, h], k[s:e, h], v[s:e, h], scale, causal, window)
            out[s:e, h] = o
            lse[h, s:e] = l
    return out, lse


def jagged_backward(q, k, v, do, offsets, scale, causal=False, window=0):
    """Packed self-attention gradients -> dq, dk, dv, each [T,H,D]."""
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    H = q.shape[1]
    for s, e in _seqs(offsets):
        for h in range(H):
            a, b_, c = seq_backward(q[s:e, h], k[s:e, h], v[s:e, h], do[s:e, h], scale, causal,
                                    window)
            dq[s:e, h], dk[s:e, h], dv[s:e, h] = a, b_, c
    return dq, dk, dv


def broadcast_forward(qd, k, v, offsets, scale):
    """Dense Q [Lq,H,D] against every jagged K/V sequence.

    -> out [B,Lq,H,D], lse [B,H,Lq].
    """
    Lq, H, D = qd.shape
    seqs = _seqs(offsets)
    out = np.zeros((len(seqs), Lq, H, v.shape[2]))
    lse = np.full((len(seqs), H, Lq), -np.inf)
    for b, (s, e) in enumerate(seqs):
        for h in range(H):
            o, l = seq_forward(qd[:, h], k[s:e, h], v[s:e, h], scale, False)
            out[b, :, h] = o
            lse[b, h] = l
    return out, lse


def broadcast_backward(qd, k, v, do, offsets, scale):
    """-> dq [Lq,H,D] (summed over sequences in order b = 0..B-1), dk, dv [T,H,D]."""
    Lq, H, D = qd.shape
    dq = np.zeros_like(qd)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b, (s, e) in enumerate(_seqs(offsets)):
        for h in range(H):
            a, b_, c = seq_backward(qd[:, h], k[s:e, h], v[s:e, h], do[b, :, h], scale, False)
            dq[:, h] += a
            dk[s:e, h], dv[s:e, h] = b_, c
    return dq, dk, dv


def sparse_masks(offsets, flat):
    """Per-sequence block masks ([n_b, n_b] bool, n_b = ceil(L_b / 64)) from the
    flat row-major concatenation."""
    flat = np.asarray(flat).reshape(-1)
    masks, pos = [], 0
    for s, e in _seqs(offsets):
        n = -(-(e - s) // SPARSE_BLOCK)
        masks.append(flat[pos:pos + n * n].reshape(n, n).astype(bool))
        pos += n * n
    if pos != flat.size:
        raise ValueError("flat mask size does not match the offsets")
    return masks


def block_sparse_forward(q, k, v, offsets, scale, masks, causal=False):
    """Block-sparse self-attention: q/k/v [T,H,D], one block mask per sequence
    -> out [T,H,D], lse [H,T]."""
    T, H, D = q.shape
    out = np.zeros((T, H, v.shape[2]))
    lse = np.full((H, T), -np.inf)
    for (s, e), bm in zip(_seqs(offsets), masks):
        for h in range(H):
            o, l = seq_forward(q[s:e, h], k[s:e, h], v[s:e, h], scale, causal, bmask=bm)
            out[s:e, h] = o
            lse[h, s:e] = l
    return out, lse


def block_sparse_backward(q, k, v, do, offsets, scale, masks, causal=False):
    """Block-sparse self-attention gradients -> dq, dk, dv, each [T,H,D]."""
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    H = q.shape[1]
    for (s, e), bm in zip(_seqs(offsets), masks):
        for h in range(H):
            a, b_, c = seq_backward(q[s:e, h], k[s:e, h], v[s:e, h], do[s:e, h], scale, causal,
                                    bmask=bm)
            dq[s:e, h], dk[s:e, h], dv[s:e, h] = a, b_, c
    return dq, dk, dv


def refine_offsets(offsets, block=64):
    """Offsets split at every `block` tokens inside each sequence.

    Every sequence length must be a multiple of `block`.
    """
    out = [0]
    for s, e in _seqs(offsets):
        if (e - s) % block:
            raise ValueError("sequence length is not a multiple of the block size")
        out.extend(range(s + block, e + 1, block))
    return np.asarray(out, dtype=np.int64)


def block_diag_forward(q, k, v, offsets, scale, block=64):
    """64-token block-diagonal attention -> out [T,H,D] (no lse)."""
    out, _ = jagged_forward(q, k, v, refine_offsets(offsets, block), scale, False)
    return out


def block_diag_backward(q, k, v, do, offsets, scale, block=64):
    return jagged_backward(q, k, v, do, refine_offsets(offsets, block), scale, False)


# ---------------------------------------------------------------- counters
def pair_count(lengths, causal=False, lq=0, block=0, masks=None):
    """Number of unmasked (query, key) pairs the attention evaluates.

    self-attention: sum L^2 (causal: sum L(L+1)/2); broadcast: sum Lq*L;
    block-diagonal: block * sum L; block-sparse: the pairs of every allowed
    (query block, key block), the last block of a sequence counting its own rows.
    """
    L = np.asarray(lengths, dtype=np.int64)
    if masks is not None:
        total = 0
        for n, bm in zip(L, masks):
            nb = bm.shape[0]
            rows = np.full(nb, SPARSE_BLOCK, dtype=np.int64)
            if nb:
                rows[-1] = n - SPARSE_BLOCK * (nb - 1)
            if causal:
                # below the diagonal blocks whole; on it the block's own causal count
                m = np.tril(bm, -1).astype(np.int64)
                total += int(rows @ m @ rows)
                total += int(sum(int(r) * (int(r) + 1) // 2 for r, d in zip(rows, np.diag(bm)) if d))
            else:
                total += int(rows @ bm.astype(np.int64) @ rows)
        return total
    if block:
        return int(block * L.sum())
    if lq:
        return int(lq * L.sum())
    if causal:
        return int((L * (L + 1) // 2).sum())
    return int((L * L).sum())
