// Rotary embeddings on the jagged path: one pass writes the rows of q and k,
// rotated by their position inside their sequence, to the workspace, and the
// attention kernels read those copies. The keys are streamed past every query
// tile of their sequence, so rotating them once here and reading them back costs
// one extra trip through HBM, where rotating them inside the attention loop would
// repeat the work for every query tile and sit on the matrix-core critical path.
// The backward turns dQ and dK back inside its own epilogues (jfa_bwd.hip).
//
// The pass walks the forward schedule: every (token, head) row lies in exactly
// one forward tile (b, h, t), rows [t*128, t*128 + 128) of sequence b, so every
// row is rotated once and its position is its row index in the tile's sequence.
#include <cmath>

#include "jfa_internal.h"
#include "jfa_rope.h"

using namespace jfa_dev;

namespace {

struct RopeRowsParams {
  const uint16_t* q; const uint16_t* k; uint16_t* qr; uint16_t* kr;
  const int32_t* offsets; const int32_t* slot_ptr; const int32_t* tiles;
  int32_t num_slots, H;
  jfa::RopeTab tab;
};

template <int D>
__device__ __forceinline__ void rotate_chunk(const uint16_t* x, uint16_t* y, const float (&cs)[8],
                                             const float (&sn)[8]) {
  const u32x4 a = ld16(x), b = ld16(x + D / 2);
  u32x4 ya, yb;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float a0 = bf16_lo(a[j]), a1 = bf16_hi(a[j]), b0 = bf16_lo(b[j]), b1 = bf16_hi(b[j]);
    const float c0 = cs[2 * j], c1 = cs[2 * j + 1], s0 = sn[2 * j], s1 = sn[2 * j + 1];
    ya[j] = pack_bf16(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
    yb[j] = pack_bf16(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
  }
  st16(y, ya);
  st16(y + D / 2, yb);
}

// Items of a tile are (row, 8-column chunk of the first half) in row order, so
// a wave covers the first halves of 64 / (D/16) consecutive rows with one load
// and their second halves with the other.
template <int D>
__global__ void __launch_bounds__(256) rope_rows_kernel(RopeRowsParams P) {
  constexpr int CH = D / 16;
  constexpr int ITEMS = jfa::kFwdBM * CH;
  __shared__ double rev[D / 2];
  if (threadIdx.x < D / 2) rev[threadIdx.x] = P.tab.rev[threadIdx.x];
  __syncthreads();
  const int n = P.slot_ptr[P.num_slots];
  const int64_t rstride = int64_t(P.H) * D;
  for (int ti = blockIdx.x; ti < n; ti += gridDim.x) {
    const int b = sload(P.tiles + 4 * ti + 0), h = sload(P.tiles + 4 * ti + 1);
    const int t = sload(P.tiles + 4 * ti + 2);
    const int kv0 = sload(P.offsets + b);
    const int L = sload(P.offsets + b + 1) - kv0;
    for (int it = threadIdx.x; it < ITEMS; it += 256) {
      const int r = t * jfa::kFwdBM + it / CH, c = it % CH;
      if (r >= L) break;  // later items of this thread lie further down the tile
      float cs[8], sn[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) rope_cs_rev(double(r) * rev[c * 8 + e], cs[e], sn[e]);
      const int64_t e0 = (int64_t(kv0) + r) * rstride + int64_t(h) * D + c * 8;
      rotate_chunk<D>(P.q + e0, P.qr + e0, cs, sn);
      rotate_chunk<D>(P.k + e0, P.kr + e0, cs, sn);
    }
  }
}

template <int D>
jfa_status launch_t(const jfa::RopeRowsLaunch& a) {
  RopeRowsParams P{};
  P.q = static_cast<const uint16_t*>(a.q);
  P.k = static_cast<const uint16_t*>(a.k);
  P.qr = static_cast<uint16_t*>(a.qr);
  P.kr = static_cast<uint16_t*>(a.kr);
  P.offsets = a.offsets;
  P.slot_ptr = a.slot_ptr;
  P.tiles = a.tiles;
  P.num_slots = a.num_slots;
  P.H = a.num_heads;
  P.tab = a.tab;
  // a forward tile holds up to 128 rows of one head: at most H * (T/128 + B) tiles
  const int64_t max_tiles = int64_t(a.num_heads) * (a.total_kv / jfa::kFwdBM + a.num_seqs);
  const unsigned grid = unsigned(max_tiles < 4096 ? (max_tiles > 0 ? max_tiles : 1) : 4096);
  hipLaunchKernelGGL(rope_rows_kernel<D>, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(a.stream), P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("rotary launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

}  // namespace

namespace jfa {

RopeTab rope_table(float base, int head_dim) {
  RopeTab t{};
  for (int i = 0; i < head_dim / 2; ++i)
    t.rev[i] = std::pow(double(base), -2.0 * i / head_dim) / (2.0 * M_PI);
  return t;
}

jfa_status launch_rope_rows(const RopeRowsLaunch& a) {
  return a.head_dim == 128 ? launch_t<128>(a) : launch_t<64>(a);
}

}  // namespace jfa
