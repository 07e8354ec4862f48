// Block-sparse step lists on the device: the walk over the entries of one of a
// tile's two 64-token blocks. A tile's entries (one int32 each) hold the other
// side's block index in bits 0..kSpBit-1 and, in bits kSpBit and kSpBit + 1,
// whether the tile's block 2t or 2t + 1 pairs with it; each wave pair of a
// block-sparse kernel walks the entries of its own block.
#pragma once

#include "jfa_internal.h"
#include "jfa_device.h"

namespace jfa_dev {

// The blocks one 64-token block of a tile pairs with, in list order: the tile's
// entries that carry that block's bit (kSpBit for block 2t, kSpBit + 1 for block
// 2t + 1), read 64 at a time (one per lane) and taken from the ballot of the bit.
struct BlockWalk {
  const int32_t* ent;  // the tile's entries
  int n_ent, bit, lane;
  int base;            // index of the loaded chunk's first entry
  uint64_t left;       // entries of the chunk with the bit, not yet taken
  int v;               // the lane's entry of the chunk
  __device__ __forceinline__ void load(int b0) {
    base = b0;
    const int e = b0 + lane;
    v = e < n_ent ? ent[e] : 0;
    left = __builtin_amdgcn_ballot_w64((v >> bit) & 1);
  }
  // the next block index (only called while one is left; 0 past the list)
  __device__ __forceinline__ int next() {
    while (left == 0 && base + 64 < n_ent) load(base + 64);
    if (left == 0) return 0;
    const int i = __builtin_ctzll(left);
    left &= left - 1;
    return __builtin_amdgcn_readlane(v, i) & jfa::kSpIdx;
  }
};

// Number of the tile's entries that carry bit `bit` (uniform).
__device__ __forceinline__ int count_bit(const int32_t* ent, int n_ent, int bit, int lane) {
  int n = 0;
  for (int b0 = 0; b0 < n_ent; b0 += 64) {
    const int e = b0 + lane;
    const int v = e < n_ent ? ent[e] : 0;
    n += __builtin_popcountll(__builtin_amdgcn_ballot_w64((v >> bit) & 1));
  }
  return n;
}

}  // namespace jfa_dev
