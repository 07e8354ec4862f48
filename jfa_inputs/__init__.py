"""Seeded synthetic inputs for jagged attention: sequence lengths, offsets and
bf16 Q/K/V/dO values.

This module is data only. It draws lengths and normal values and rounds them to
bf16; it contains none of the attention arithmetic. Both the HIP path and the
CPU oracle consume what it produces, so it is the one thing they share.

Every draw comes from its own numpy stream keyed by
(workload id, seed, stream id, sequence index), so any single sequence can be
regenerated without generating the others (the oracle uses this to check a
sample of a large workload without holding it all in memory).

Workloads (restated from the jagged-attention pages' GEM and block-attention
shapes, see "Jagged Flash Attention for GEM" intro and "TLX Block Attention"
section 1):

  tiny        B=4, L ~ U{1..96} with sequence 1 forced to length 1, H=2, D=64,
              sigma 1, non-causal.
  gem         B=256, L log-uniform int in [16,4096], H=8, D=128, sigma 0.5,
              causal and non-causal.
  broadcast   one dense Q [256,8,128] shared by B=1024 sequences, K/V lengths
              log-uniform int in [32,2048], sigma 0.5, non-causal.
  block64     B=1152, L = 64*U{1..64}, H=4, D in {64,128}, sigma 1,
              64-token block-diagonal.
  imbalance   B=2048: 102 lengths U{8192..16384} and 1946 lengths U{8..64},
              shuffled; H=16, D=128, sigma 0.5, non-causal.
  gem_padded  the gem batch with every sequence as long as its longest one (the
              padded-dense layout the jagged one avoids), causal and non-causal;
              for timing the work a padded-dense run executes.
  sparse      block-sparse self-attention over 64-token blocks: B=1152, L ~
              U{1..4096} (the last block of a sequence partial), H=4, D in
              {64,128}, sigma 1; each query block attends its own key block and
              each other key block of its sequence with probability 0.3, about
              70% of the block pairs of a long sequence masked (the sparsity the
              block-attention page reports for its workloads, section 1); at
              D=128 also causal (the same masks, keys after the query dropped).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

# stream ids
S_LENGTHS, S_Q, S_K, S_V, S_DO, S_QDENSE, S_MASK = 0, 1, 2, 3, 4, 5, 6
SPARSE_BLOCK = 64

# gem_padded shares gem's id, so its lengths are the gem draw padded to the maximum
WORKLOAD_IDS = {"tiny": 1, "gem": 2, "broadcast": 3, "block64": 4, "imbalance": 5,
                "gem_padded": 2, "sparse": 6}


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_heads: int
    head_dim: int
    sigma: float
    kind: str = "jagged"        # "jagged" | "broadcast" | "block" (block-diagonal) | "sparse"
    causal: bool = False
    lq: int = 0                 # dense Q rows for "broadcast"
    seed: int = 0
    # length law
    law: str = "uniform"        # "uniform" | "loguniform" | "blocks" | "mix" | "fixed"
    lo: int = 1
    hi: int = 1
    force_first_short: bool = False   # tiny: lengths[1] = 1
    mix_long_frac: float = 0.0
    mix_long_lo: int = 0
    mix_long_hi: int = 0
    fixed_lengths: tuple = ()
    pad_to_max: bool = False          # every length replaced by the largest drawn
    rope_base: float = 0.0            # rotary embeddings with this base (0: none)
    window: int = 0                   # causal sliding window of this many keys (0: none)
    block: int = 64                   # kind "block": tokens per diagonal block
    density: float = 0.0              # kind "sparse": chance of each off-diagonal block pair

    @property
    def wid(self) -> int:
        return WORKLOAD_IDS.get(self.name, 99)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def standard_workloads():
    """The five reference workloads (block64 and gem in both of their variants)."""
    return {
        "tiny": Workload("tiny", 4, 2, 64, 1.0, law="uniform", lo=1, hi=96,
                         force_first_short=True),
        "gem": Workload("gem", 256, 8, 128, 0.5, law="loguniform", lo=16, hi=4096),
        "gem_causal": Workload("gem", 256, 8, 128, 0.5, law="loguniform", lo=16, hi=4096,
                               causal=True),
        "broadcast": Workload("broadcast", 1024, 8, 128, 0.5, kind="broadcast", lq=256,
                              law="loguniform", lo=32, hi=2048),
        "block64_d64": Workload("block64", 1152, 4, 64, 1.0, kind="block", law="blocks",
                                lo=1, hi=64),
        "block64_d128": Workload("block64", 1152, 4, 128, 1.0, kind="block", law="blocks",
                                 lo=1, hi=64),
        # other block sizes, lengths drawn so that the batch holds as many tokens
        "block32_d128": Workload("block64", 1152, 4, 128, 1.0, kind="block", law="blocks",
                                 lo=1, hi=128, block=32),
        "block128_d128": Workload("block64", 1152, 4, 128, 1.0, kind="block", law="blocks",
                                  lo=1, hi=32, block=128),
        "block256_d128": Workload("block64", 1152, 4, 128, 1.0, kind="block", law="blocks",
                                  lo=1, hi=16, block=256),
        # the same batches with rotary embeddings fused in (same seeds and values)
        "block64_rope_d64": Workload("block64", 1152, 4, 64, 1.0, kind="block",
                                     law="blocks", lo=1, hi=64, rope_base=10000.0),
        "block64_rope_d128": Workload("block64", 1152, 4, 128, 1.0, kind="block",
                                      law="blocks", lo=1, hi=64, rope_base=10000.0),
        "imbalance": Workload("imbalance", 2048, 16, 128, 0.5, law="mix", lo=8, hi=64,
                              mix_long_frac=0.05, mix_long_lo=8192, mix_long_hi=16384),
        "gem_padded": Workload("gem_padded", 256, 8, 128, 0.5, law="loguniform", lo=16,
                               hi=4096, pad_to_max=True),
        # the gem batches with rotary embeddings (same seeds and values)
        "gem_rope": Workload("gem", 256, 8, 128, 0.5, law="loguniform", lo=16, hi=4096,
                             rope_base=10000.0),
        "gem_rope_causal": Workload("gem", 256, 8, 128, 0.5, law="loguniform", lo=16, hi=4096,
                                    causal=True, rope_base=10000.0),
        # the causal gem batch with a sliding window of 512 keys (same seeds and values)
        "gem_window": Workload("gem", 256, 8, 128, 0.5, law="loguniform", lo=16, hi=4096,
                               causal=True, window=512),
        "gem_padded_causal": Workload("gem_padded", 256, 8, 128, 0.5, law="loguniform", lo=16,
                                      hi=4096, pad_to_max=True, causal=True),
        "sparse_d128": Workload("sparse", 1152, 4, 128, 1.0, kind="sparse", law="uniform",
                                lo=1, hi=4096, density=0.3),
        "sparse_d64": Workload("sparse", 1152, 4, 64, 1.0, kind="sparse", law="uniform",
                               lo=1, hi=4096, density=0.3),
        # the sparse_d128 batch (same seeds, values and masks) with causal masking
        "sparse_d128_causal": Workload("sparse", 1152, 4, 128, 1.0, kind="sparse",
                                       law="uniform", lo=1, hi=4096, density=0.3, causal=True),
    }


def _rng(w: Workload, stream: int, b: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([w.wid, w.seed, stream, b]))


def lengths(w: Workload) -> np.ndarray:
    """Sequence lengths (int64 [B])."""
    rng = _rng(w, S_LENGTHS)
    B = w.num_seqs
    if w.law == "fixed":
        L = np.asarray(w.fixed_lengths, dtype=np.int64)
        assert L.shape == (B,)
        return L
    if w.law == "uniform":
        L = rng.integers(w.lo, w.hi + 1, size=B, dtype=np.int64)
    elif w.law == "loguniform":
        # P(L = n) proportional to ln((n+1)/n) on [lo, hi]
        u = rng.uniform(math.log(w.lo), math.log(w.hi + 1), size=B)
        L = np.clip(np.floor(np.exp(u)).astype(np.int64), w.lo, w.hi)
    elif w.law == "blocks":
        L = w.block * rng.integers(w.lo, w.hi + 1, size=B, dtype=np.int64)
    elif w.law == "mix":
        n_long = int(round(w.mix_long_frac * B))
        long_ = rng.integers(w.mix_long_lo, w.mix_long_hi + 1, size=n_long, dtype=np.int64)
        short = rng.integers(w.lo, w.hi + 1, size=B - n_long, dtype=np.int64)
        L = np.concatenate([long_, short])
        rng.shuffle(L)
    else:
        raise ValueError(w.law)
    if w.force_first_short and B > 1:
        L[1] = 1
    if w.pad_to_max and B > 0:
        L[:] = L.max()
    return L


def offsets_from_lengths(L) -> np.ndarray:
    """int32 exclusive prefix sum, shape [B+1]."""
    L = np.asarray(L, dtype=np.int64)
    off = np.zeros(L.shape[0] + 1, dtype=np.int64)
    np.cumsum(L, out=off[1:])
    assert off[-1] < 2**31
    return off.astype(np.int32)


def sparse_mask_seq(w: Workload, b: int, L: int) -> np.ndarray:
    """Block mask of sequence b (uint8 [n, n], n = ceil(L / 64)): row = query
    block, column = key block; the diagonal always set, every other entry set with
    probability w.density."""
    n = -(-int(L) // SPARSE_BLOCK)
    m = (_rng(w, S_MASK, b).random((n, n)) < w.density)
    m |= np.eye(n, dtype=bool)
    return m.astype(np.uint8)


def sparse_mask_flat(w: Workload, L) -> np.ndarray:
    """Every sequence's block mask, row-major, concatenated (uint8)."""
    parts = [sparse_mask_seq(w, b, int(n)).ravel() for b, n in enumerate(L)]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.uint8)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def seq_values(w: Workload, stream: int, b: int, rows: int) -> np.ndarray:
    """bf16 bits [rows, H, D] for one sequence (or one dense block) of one tensor."""
    rng = _rng(w, stream, b)
    x = rng.standard_normal(rows * w.num_heads * w.head_dim, dtype=np.float32)
    x *= np.float32(w.sigma)
    return f32_to_bf16_bits(x).reshape(rows, w.num_heads, w.head_dim)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def packed_values(w: Workload, stream: int, L: np.ndarray, rows_per_seq=None) -> np.ndarray:
    """bf16 bits [sum(rows), H, D]: sequences concatenated with no padding."""
    L = np.asarray(L, dtype=np.int64)
    rows = L if rows_per_seq is None else np.full_like(L, rows_per_seq)
    off = np.zeros(len(rows) + 1, dtype=np.int64)
    np.cumsum(rows, out=off[1:])
    out = np.empty((int(off[-1]), w.num_heads, w.head_dim), dtype=np.uint16)

    def one(b):
        if rows[b]:
            out[off[b]:off[b + 1]] = seq_values(w, stream, b, int(rows[b]))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(len(rows))))
    return out


@dataclass
class Case:
    """All host-side inputs of one workload draw (bf16 values as uint16 bits)."""
    w: Workload
    lengths: np.ndarray
    offsets: np.ndarray
    q: np.ndarray       # [T,H,D] or dense [Lq,H,D] for broadcast
    k: np.ndarray       # [T,H,D]
    v: np.ndarray       # [T,H,D]
    do: np.ndarray      # [T,H,D] or [B,Lq,H,D] for broadcast
    scale: float        # float32 value of 1/sqrt(D)
    mask: np.ndarray = None  # kind "sparse": the flat block masks (uint8)

    @property
    def max_len(self) -> int:
        return int(self.lengths.max()) if len(self.lengths) else 0


def softmax_scale(D: int) -> float:
    return float(np.float32(1.0) / np.sqrt(np.float32(D)))


def make_case(w: Workload, with_do: bool = True) -> Case:
    L = lengths(w)
    off = offsets_from_lengths(L)
    if w.kind == "broadcast":
        q = seq_values(w, S_QDENSE, 0, w.lq)
        do = (packed_values(w, S_DO, L, rows_per_seq=w.lq).reshape(
            len(L), w.lq, w.num_heads, w.head_dim) if with_do else None)
    else:
        q = packed_values(w, S_Q, L)
        do = packed_values(w, S_DO, L) if with_do else None
    k = packed_values(w, S_K, L)
    v = packed_values(w, S_V, L)
    mask = sparse_mask_flat(w, L) if w.kind == "sparse" else None
    return Case(w, L, off, q, k, v, do, softmax_scale(w.head_dim), mask)


def custom(lengths_, num_heads, head_dim, sigma=1.0, seed=0, kind="jagged", causal=False,
           lq=0, name="custom", rope_base=0.0, window=0, block=64, density=0.0) -> Workload:
    """A workload with explicitly given lengths (edge cases, small tests)."""
    L = tuple(int(x) for x in lengths_)
    return Workload(name, len(L), num_heads, head_dim, sigma, kind=kind, causal=causal,
                    lq=lq, seed=seed, law="fixed", fixed_lengths=L, rope_base=rope_base,
                    window=window, block=block, density=density)


def to_torch_bf16(bits: np.ndarray):
    """uint16 bits -> torch.bfloat16 tensor (CPU), sharing no arithmetic."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
