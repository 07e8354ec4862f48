// Rotary-embedding helpers for the jagged kernels.
//
// A row at position p (its index inside its sequence) has its column pair
// (i, i + D/2), i < D/2, turned by the angle p * base^(-2i/D) ("TLX Block
// Attention" fuses rotary embeddings into its kernels; the embedding itself is
// the common rotary position embedding). The host fills RopeTab with the angle
// of one position step in revolutions; positions on the jagged path reach tens of
// thousands, so p * rev is formed in double precision (a single-precision product
// would be off by up to ~1e-3 rad there), reduced to half a revolution, and only
// then handed to the single-precision hardware sine and cosine, which take
// revolutions.
#pragma once

#include "jfa_device.h"
#include "jfa_internal.h"

namespace jfa_dev {

__device__ __forceinline__ void rope_cs_rev(double rev, float& c, float& s) {
  const float f = float(rev - __builtin_rint(rev));
  c = __builtin_amdgcn_cosf(f);
  s = __builtin_amdgcn_sinf(f);
}

// Turn gradients of rotated rows back (the transposed rotation) in an
// accumulator set whose tile nb holds columns nb*32 + (r/4)*8 + 4g + r%4 of this
// lane's row (position p) at register r: pair partners sit in tiles nb and
// nb + NB/2 of the same lane. `tab` is the angle table copied to LDS (read where
// it is needed, so that no register holds the table across the main loop).
template <int D>
__device__ __forceinline__ void rope_back_rows(f32x16 (&a)[D / 32], int p, int g,
                                               const double* tab) {
  constexpr int NB = D / 32;
  const double pd = double(p);
  const double* tg = tab + 4 * g;
#pragma unroll
  for (int nb = 0; nb < NB / 2; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const double rv = tg[nb * 32 + (r / 4) * 8 + (r % 4)];
      float c, s;
      rope_cs_rev(pd * rv, c, s);
      const float x1 = a[nb][r], x2 = a[nb + NB / 2][r];
      a[nb][r] = x1 * c + x2 * s;
      a[nb + NB / 2][r] = x2 * c - x1 * s;
    }
}

}  // namespace jfa_dev
