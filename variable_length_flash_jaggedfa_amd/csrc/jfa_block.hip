// 64-token block-diagonal attention for gfx950 ("TLX Block Attention").
//
// Every 64-token group attends only within itself, so one query tile meets
// exactly one key tile (section 2): the 64x64 score tile is complete after one
// product, the row max and row sum are exact at once (no correction factor), the
// output is one fresh product (accumulators start from zero), and no log-sum-exp
// is stored: the backward rebuilds the softmax statistics itself and computes Di
// inline (sections 2 and 4). One workgroup of two waves handles one
// (64-token block, head) unit; each wave owns 32 query rows in the score phase
// and 32 keys in the dK/dV phase. The kernels are bound by HBM traffic (the page
// puts the arithmetic intensity far below the ridge point), so each unit reads
// its operands once and writes its outputs once.
//
// 32-token blocks run on the same kernels: a 64-token unit then holds two blocks
// (block boundaries fall on multiples of 32 tokens everywhere), and each wave,
// whose 32 query rows are one block, masks the other block's keys; the last unit
// may hold a single block. Blocks of 128 or 256 tokens run on the jagged kernels,
// except the whole backward of 128-token blocks without rotary, which runs as one
// single-tile kernel below.
//
// With rotary embeddings (the page fuses them into these kernels) the rows of Q
// and K are rotated inside the kernel after they arrive in LDS, and the backward
// turns dQ and dK back before storing them, so the rotated rows never travel
// through memory.
#include <cmath>

#include "jfa_internal.h"
#include "jfa_tiles.h"

using namespace jfa_dev;

namespace {

constexpr int kBS = jfa::kBlock;  // 64

template <int D>
struct BlkCfg {
  static constexpr int NW = 2;        // waves: 32 query rows (then 32 keys) each
  static constexpr int NT = 64 * NW;
  static constexpr int DS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int TILE = kBS * D;  // one 64 x D tile
};

// Rotary angles. A row at position p has its column pair (i, i + D/2), i < D/2,
// turned by p * theta_i with theta_i = base^(-2i/D). The scores and gradients
// depend only on position differences, and two rows meet only inside one 64-token
// group, so p counts from the start of the group (0..63): the same results as
// positions counted from the start of the sequence, with small angles. Angles are
// kept in revolutions, the unit of the hardware sine and cosine:
// p * 2^(i * kr + kc) with kr = -2 log2(base) / D and kc = -log2(2 pi).
struct Rope {
  float kr, kc;
};

struct BlkParams {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; const uint16_t* o; const uint16_t* dout;
  uint16_t* out; uint16_t* dq; uint16_t* dk; uint16_t* dv;
  int32_t H;
  int32_t rows;  // tokens T (the last 32-token-block unit may hold 32 of them)
  float c;       // scale * log2(e)
  float scale;
  Rope rope;     // rotary kernels only
};

// Rows of this unit that exist: 64, or with 32-token blocks up to 64.
template <int BS>
__device__ __forceinline__ int unit_rows(int rows, int blk) {
  return BS == kBS ? kBS : min(kBS, rows - blk * kBS);
}

// With 32-token blocks, a wave's queries (its block) meet only their own keys.
template <int BS>
__device__ __forceinline__ void mask_other_block(f32x16 (&s)[2], int w) {
  if (BS == 32) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      if (kb != w) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = -INFINITY;
      }
  }
}

__device__ __forceinline__ void rope_cs(float p, int i, const Rope& R, float& c, float& s) {
  float rev = p * exp2_fast(float(i) * R.kr + R.kc);
  rev -= rintf(rev);  // within half a revolution of zero
  c = __builtin_amdgcn_cosf(rev);
  s = __builtin_amdgcn_sinf(rev);
}

// Rotate the 64 rows of two swizzled 64 x D LDS tiles in place. Lane l takes row
// l; the waves deal the 8-column chunks of the first half of a row between them,
// each with its partner chunk D/2 columns on. Sixteen lanes read sixteen
// consecutive rows at one logical chunk, the conflict-free pattern of the tiles.
template <int D, int NW>
__device__ __forceinline__ void rope_tiles(uint16_t* ta, uint16_t* tb, const Rope& R, int w, int lane) {
  constexpr int CH = D / 16;
  static_assert(CH % NW == 0, "chunks split evenly over the waves");
  const float p = float(lane);
#pragma unroll
  for (int k = 0; k < CH / NW; ++k) {
    const int c = w + k * NW;
    float cs[8], sn[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rope_cs(p, c * 8 + e, R, cs[e], sn[e]);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      uint16_t* tile = t ? tb : ta;
      uint16_t* pa = tile + Swz<D>::chunk(lane, c);
      uint16_t* pb = tile + Swz<D>::chunk(lane, c + CH);
      const u32x4 a = ld16(pa), b = ld16(pb);
      u32x4 ya, yb;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a0 = bf16_lo(a[j]), a1 = bf16_hi(a[j]), b0 = bf16_lo(b[j]), b1 = bf16_hi(b[j]);
        const float c0 = cs[2 * j], c1 = cs[2 * j + 1], s0 = sn[2 * j], s1 = sn[2 * j + 1];
        ya[j] = pack_bf16(a0 * c0 - b0 * s0, a1 * c1 - b1 * s1);
        yb[j] = pack_bf16(b0 * c0 + a0 * s0, b1 * c1 + a1 * s1);
      }
      st16(pa, ya);
      st16(pb, yb);
    }
  }
}

// Turn gradients of rotated rows back (the transposed rotation) in an
// accumulator set: tile nb holds columns nb*32 + (r/4)*8 + 4g + r%4 of this
// lane's row at register r, so pair partners sit in tiles nb and nb + NB/2.
template <int D>
__device__ __forceinline__ void rope_back(f32x16 (&a)[D / 32], float p, int g, const Rope& R) {
  constexpr int NB = D / 32;
#pragma unroll
  for (int nb = 0; nb < NB / 2; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float c, s;
      rope_cs(p, nb * 32 + (r / 4) * 8 + 4 * g + (r % 4), R, c, s);
      const float x1 = a[nb][r], x2 = a[nb + NB / 2][r];
      a[nb][r] = x1 * c + x2 * s;
      a[nb + NB / 2][r] = x2 * c - x1 * s;
    }
}

// The (64-token block, head) unit of this workgroup. At D = 128 neighbouring
// workgroups take the heads of one block (together they read whole contiguous
// rows of all heads); at D = 64 they take neighbouring blocks of one head. Each
// order measured faster at its head dimension on the block-diagonal workload.
template <int D>
__device__ __forceinline__ void unit_of(int H, int& blk, int& h) {
  if (D == 128) {
    blk = blockIdx.x / H;
    h = blockIdx.x % H;
  } else {
    const int nblk = gridDim.x / H;
    blk = blockIdx.x % nblk;
    h = blockIdx.x / nblk;
  }
}

// Exact softmax of one 64-key tile held as S^T (keys along the registers, one
// query per lane pair): returns P packed to bf16 as MFMA operands (keys in the
// order of an accumulator tile) and keeps P in `s`.
__device__ __forceinline__ void tile_softmax(f32x16 (&s)[2], float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = pair_max(mx) * c;  // scale > 0, so the max commutes with it
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(__builtin_fmaf(s[kb][r], c, -mx));
      s[kb][r] = p;
      rs += p;
    }
  const float inv = 1.f / pair_sum(rs);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] *= inv;
}

template <int D, bool ROPE, int BS>
__global__ void __launch_bounds__(128) block_fwd_kernel(BlkParams P) {
  using C = BlkCfg<D>;
  // K, V, then the two waves' output staging tiles (32 x D each; with ROPE they
  // first hold the Q tile, wave w's half being its own 32 query rows)
  __shared__ __attribute__((aligned(1024))) uint16_t lds[3 * C::TILE];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
  int blk, h;
  unit_of<D>(P.H, blk, h);
  const int64_t rstride = int64_t(P.H) * D;
  const int64_t base = int64_t(blk) * kBS * rstride + int64_t(h) * D;
  const int rowbytes = int(rstride * 2);
  const int nrows = unit_rows<BS>(P.rows, blk);
  tile_load<D, kBS, C::NW>(lds, rows_rsrc<D, kBS>(P.k + base, rstride, nrows), rowbytes, w, lane);
  tile_load<D, kBS, C::NW>(lds + C::TILE, rows_rsrc<D, kBS>(P.v + base, rstride, nrows), rowbytes, w, lane);
  u32x4 qf[C::DS];
  if (ROPE) {
    uint16_t* Qt = lds + 2 * C::TILE;
    tile_load<D, kBS, C::NW>(Qt, rows_rsrc<D, kBS>(P.q + base, rstride, nrows), rowbytes, w, lane);
    wait_vmem();
    __syncthreads();
    rope_tiles<D, C::NW>(lds, Qt, P.rope, w, lane);
    __syncthreads();
#pragma unroll
    for (int d = 0; d < C::DS; ++d) qf[d] = frag_rows<D>(Qt, w * 32, d, li, g);
  } else {
    const uint16_t* qrow = P.q + base + int64_t(w * 32 + li) * rstride;
    const bool ok = w * 32 + li < nrows;
#pragma unroll
    for (int d = 0; d < C::DS; ++d) qf[d] = ok ? ld16(qrow + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
    wait_vmem();
    __syncthreads();
  }
  // S^T = K Q^T for the 64 keys and this wave's 32 queries, fresh accumulators
  f32x16 s[2];
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int d = 0; d < C::DS; ++d)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(frag_rows<D>(lds, kb * 32, d, li, g), qf[d], s[kb]);
  mask_other_block<BS>(s, w);
  // one tile: the row max and sum are exact at once, nothing is rescaled
  tile_softmax(s, P.c);
  u32x4 pf[4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) pf[kb * 2 + r / 8][(r % 8) / 2] = pack_bf16(s[kb][r], s[kb][r + 1]);
  f32x16 o[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    o[nb] = f32x16{};
#pragma unroll
    for (int st = 0; st < 4; ++st) o[nb] = mfma32(frag_cols<D>(lds + C::TILE, st * 16, nb * 32, lane), pf[st], o[nb]);
  }
  store_rows<D>(lds + 2 * C::TILE + w * (C::TILE / 2), o, 1.f, P.out + base + int64_t(w * 32) * rstride,
                rstride, nrows - w * 32, lane);
}

template <int D, bool ROPE, int BS>
__global__ void __launch_bounds__(128) block_bwd_kernel(BlkParams P) {
  using C = BlkCfg<D>;
  // K, V, Q, dO tiles (64 x D) and P^T, dS^T tiles (64 queries x 64 keys)
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * C::TILE + 2 * kBS * kBS];
  uint16_t* Kt = lds;
  uint16_t* Vt = Kt + C::TILE;
  uint16_t* Qt = Vt + C::TILE;
  uint16_t* dOt = Qt + C::TILE;
  uint16_t* Pt = dOt + C::TILE;
  uint16_t* dSt = Pt + kBS * kBS;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
  int blk, h;
  unit_of<D>(P.H, blk, h);
  const int64_t rstride = int64_t(P.H) * D;
  const int64_t base = int64_t(blk) * kBS * rstride + int64_t(h) * D;
  const int rowbytes = int(rstride * 2);
  const int nrows = unit_rows<BS>(P.rows, blk);
  tile_load<D, kBS, C::NW>(Kt, rows_rsrc<D, kBS>(P.k + base, rstride, nrows), rowbytes, w, lane);
  tile_load<D, kBS, C::NW>(Vt, rows_rsrc<D, kBS>(P.v + base, rstride, nrows), rowbytes, w, lane);
  tile_load<D, kBS, C::NW>(Qt, rows_rsrc<D, kBS>(P.q + base, rstride, nrows), rowbytes, w, lane);
  tile_load<D, kBS, C::NW>(dOt, rows_rsrc<D, kBS>(P.dout + base, rstride, nrows), rowbytes, w, lane);
  // out fragments of this lane's query row, for Di = rowsum(dO * out)
  const int i = w * 32 + li;
  u32x4 of[C::DS];
  const uint16_t* orow = P.o + base + int64_t(i) * rstride;
#pragma unroll
  for (int d = 0; d < C::DS; ++d) of[d] = i < nrows ? ld16(orow + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
  wait_vmem();
  __syncthreads();
  if (ROPE) {
    // every product below then reads the rotated rows of Q and K
    rope_tiles<D, C::NW>(Kt, Qt, P.rope, w, lane);
    __syncthreads();
  }

  // ---- query side (lane = query): S^T, dP^T, exact softmax, dS^T, dQ^T
  f32x16 s[2], dp[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
    dp[kb] = f32x16{};
  }
  float di = 0.f;
#pragma unroll
  for (int d = 0; d < C::DS; ++d) {
    const u32x4 qf = frag_rows<D>(Qt, w * 32, d, li, g);
    const u32x4 dof = frag_rows<D>(dOt, w * 32, d, li, g);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      di += bf16_lo(dof[e2]) * bf16_lo(of[d][e2]) + bf16_hi(dof[e2]) * bf16_hi(of[d][e2]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = mfma32(frag_rows<D>(Kt, kb * 32, d, li, g), qf, s[kb]);
      dp[kb] = mfma32(frag_rows<D>(Vt, kb * 32, d, li, g), dof, dp[kb]);
    }
  }
  di = pair_sum(di);
  mask_other_block<BS>(s, w);
  tile_softmax(s, P.c);  // statistics recomputed here: no lse is stored or read
  u32x4 pds[4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float dsv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) dsv[e] = s[kb][q4 * 4 + e] * (dp[kb][q4 * 4 + e] - di);
      const uint32_t p01 = pack_bf16(s[kb][q4 * 4 + 0], s[kb][q4 * 4 + 1]);
      const uint32_t p23 = pack_bf16(s[kb][q4 * 4 + 2], s[kb][q4 * 4 + 3]);
      const uint32_t d01 = pack_bf16(dsv[0], dsv[1]), d23 = pack_bf16(dsv[2], dsv[3]);
      const int st = kb * 2 + q4 / 2, hw = (q4 % 2) * 2;
      pds[st][hw] = d01;
      pds[st][hw + 1] = d23;
      // P^T and dS^T rows (query i, keys j0..j0+3) for the key-side products
      const int j0 = kb * 32 + q4 * 8 + g * 4;
      st8(Pt + Swz<kBS>::chunk(i, j0 >> 3) + (j0 & 7), u32x2{p01, p23});
      st8(dSt + Swz<kBS>::chunk(i, j0 >> 3) + (j0 & 7), u32x2{d01, d23});
    }
  }
  f32x16 dqa[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    dqa[nb] = f32x16{};
#pragma unroll
    for (int st = 0; st < 4; ++st) dqa[nb] = mfma32(frag_cols<D>(Kt, st * 16, nb * 32, lane), pds[st], dqa[nb]);
  }
  __syncthreads();
  // dQ and dK of the rotated rows, turned back: row i of this lane is query i
  // here and key i below, at the same position
  if (ROPE) rope_back<D>(dqa, float(i), g, P.rope);
  // K and V are not read after this point: their tiles stage the outputs (each
  // wave a private 32 x D half of K for dQ, and of V for dV, then dK)
  store_rows<D>(Kt + w * (C::TILE / 2), dqa, P.scale, P.dq + base + int64_t(w * 32) * rstride, rstride,
                nrows - w * 32, lane);

  // ---- key side (lane = key): dV^T = dO^T P, dK^T = Q^T dS
  u32x4 pb[4], db[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    pb[st] = frag_cols<kBS>(Pt, st * 16, w * 32, lane);
    db[st] = frag_cols<kBS>(dSt, st * 16, w * 32, lane);
  }
  f32x16 av[C::NB], ak[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    av[nb] = f32x16{};
    ak[nb] = f32x16{};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      av[nb] = mfma32(frag_cols<D>(dOt, st * 16, nb * 32, lane), pb[st], av[nb]);
      ak[nb] = mfma32(frag_cols<D>(Qt, st * 16, nb * 32, lane), db[st], ak[nb]);
    }
  }
  uint16_t* vst = Vt + w * (C::TILE / 2);
  store_rows<D>(vst, av, 1.f, P.dv + base + int64_t(w * 32) * rstride, rstride, nrows - w * 32, lane);
  if (ROPE) rope_back<D>(ak, float(i), g, P.rope);
  store_rows<D>(vst, ak, P.scale, P.dk + base + int64_t(w * 32) * rstride, rstride, nrows - w * 32, lane);
}

Rope rope_consts(float base, int D) {
  Rope R;
  R.kr = float(-2.0 * std::log2(double(base)) / D);
  R.kc = float(-std::log2(2.0 * M_PI));
  return R;
}

template <int D>
jfa_status launch_fwd_t(const jfa::FwdLaunch& a) {
  BlkParams P{};
  P.q = static_cast<const uint16_t*>(a.q);
  P.k = static_cast<const uint16_t*>(a.k);
  P.v = static_cast<const uint16_t*>(a.v);
  P.out = static_cast<uint16_t*>(a.out);
  P.H = a.num_heads;
  P.c = a.scale * kLog2e;
  P.scale = a.scale;
  const bool rope = a.flags & JFA_ROTARY;
  if (rope) P.rope = rope_consts(a.rope_base, D);
  P.rows = int32_t(a.total_kv);
  const int64_t units = ((a.total_kv + kBS - 1) / kBS) * a.num_heads;
  if (units > INT32_MAX) return jfa::fail(JFA_ERR_INVALID_ARG, "too many block units");
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const dim3 grid{unsigned(units)}, block{unsigned(BlkCfg<D>::NT)};
  if (a.block == 32) {
    if (rope) hipLaunchKernelGGL((block_fwd_kernel<D, true, 32>), grid, block, 0, st, P);
    else hipLaunchKernelGGL((block_fwd_kernel<D, false, 32>), grid, block, 0, st, P);
  } else {
    if (rope) hipLaunchKernelGGL((block_fwd_kernel<D, true, kBS>), grid, block, 0, st, P);
    else hipLaunchKernelGGL((block_fwd_kernel<D, false, kBS>), grid, block, 0, st, P);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("block fwd launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

template <int D>
jfa_status launch_bwd_t(const jfa::BwdLaunch& a) {
  BlkParams P{};
  P.q = static_cast<const uint16_t*>(a.q);
  P.k = static_cast<const uint16_t*>(a.k);
  P.v = static_cast<const uint16_t*>(a.v);
  P.o = static_cast<const uint16_t*>(a.out);
  P.dout = static_cast<const uint16_t*>(a.dout);
  P.dq = static_cast<uint16_t*>(a.dq);
  P.dk = static_cast<uint16_t*>(a.dk);
  P.dv = static_cast<uint16_t*>(a.dv);
  P.H = a.num_heads;
  P.c = a.scale * kLog2e;
  P.scale = a.scale;
  const bool rope = a.flags & JFA_ROTARY;
  if (rope) P.rope = rope_consts(a.rope_base, D);
  P.rows = int32_t(a.total_kv);
  const int64_t units = ((a.total_kv + kBS - 1) / kBS) * a.num_heads;
  if (units > INT32_MAX) return jfa::fail(JFA_ERR_INVALID_ARG, "too many block units");
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const dim3 grid{unsigned(units)}, block{unsigned(BlkCfg<D>::NT)};
  if (a.block == 32) {
    if (rope) hipLaunchKernelGGL((block_bwd_kernel<D, true, 32>), grid, block, 0, st, P);
    else hipLaunchKernelGGL((block_bwd_kernel<D, false, 32>), grid, block, 0, st, P);
  } else {
    if (rope) hipLaunchKernelGGL((block_bwd_kernel<D, true, kBS>), grid, block, 0, st, P);
    else hipLaunchKernelGGL((block_bwd_kernel<D, false, kBS>), grid, block, 0, st, P);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("block bwd launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

// 128-token blocks: the single-tile backward above with four waves ("TLX Block
// Attention", sections 2 and 4: one tile per block, statistics recomputed exactly,
// Di inline, no lse read, no atomics). Wave w owns query rows 32w..32w+31 on the
// query side (its score tile spans all 128 keys) and keys 32w..32w+31 on the key
// side. K, V, Q and dO stay in LDS. Once every wave has its dQ, the P^T and dS^T
// tiles (128 queries x 128 keys, bf16) are written: at D = 128 over K and V (the
// same size, and no longer read), at D = 64 to LDS of their own.
template <int D>
struct Blk128Cfg {
  static constexpr int BS = 128;
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int DS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int KB = BS / 32;                    // 32-key blocks of a score tile
  static constexpr int TILE = BS * D;                   // one 128 x D tile
  static constexpr int PT = BS * BS;                    // one 128 x 128 tile
  static constexpr int EXTRA = D == 128 ? 0 : 2 * PT;   // P^T, dS^T beyond the four tiles
};

// Exact softmax over the KB 32-key blocks of a score tile held as S^T (one query
// per lane pair); P is left in `s`.
template <int KB>
__device__ __forceinline__ void tile_softmax_kb(f32x16 (&s)[KB], float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = pair_max(mx) * c;  // scale > 0, so the max commutes with it
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(__builtin_fmaf(s[kb][r], c, -mx));
      s[kb][r] = p;
      rs += p;
    }
  const float inv = 1.f / pair_sum(rs);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] *= inv;
}

template <int D>
__global__ void __launch_bounds__(256) block128_bwd_kernel(BlkParams P) {
  using C = Blk128Cfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[4 * C::TILE + C::EXTRA];
  uint16_t* Kt = lds;
  uint16_t* Vt = Kt + C::TILE;
  uint16_t* Qt = Vt + C::TILE;
  uint16_t* dOt = Qt + C::TILE;
  uint16_t* Pt = D == 128 ? Kt : lds + 4 * C::TILE;  // written only after K and V are done
  uint16_t* dSt = Pt + C::PT;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
  int blk, h;
  unit_of<D>(P.H, blk, h);
  const int64_t rstride = int64_t(P.H) * D;
  const int64_t base = int64_t(blk) * C::BS * rstride + int64_t(h) * D;
  const int rowbytes = int(rstride * 2);
  const int nrows = min(C::BS, P.rows - blk * C::BS);  // 128: every length is a multiple of it
  tile_load<D, C::BS, C::NW>(Kt, rows_rsrc<D, C::BS>(P.k + base, rstride, nrows), rowbytes, w, lane);
  tile_load<D, C::BS, C::NW>(Vt, rows_rsrc<D, C::BS>(P.v + base, rstride, nrows), rowbytes, w, lane);
  tile_load<D, C::BS, C::NW>(Qt, rows_rsrc<D, C::BS>(P.q + base, rstride, nrows), rowbytes, w, lane);
  tile_load<D, C::BS, C::NW>(dOt, rows_rsrc<D, C::BS>(P.dout + base, rstride, nrows), rowbytes, w, lane);
  // out fragments of this lane's query row, for Di = rowsum(dO * out)
  const int i = w * 32 + li;
  u32x4 of[C::DS];
  const uint16_t* orow = P.o + base + int64_t(i) * rstride;
#pragma unroll
  for (int d = 0; d < C::DS; ++d) of[d] = i < nrows ? ld16(orow + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
  wait_vmem();
  __syncthreads();

  // ---- query side (lane = query): S^T, dP^T over all 128 keys, exact softmax,
  // dS^T = P (dP - Di), dQ^T = K^T dS^T
  f32x16 s[C::KB], dp[C::KB];
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    s[kb] = f32x16{};
    dp[kb] = f32x16{};
  }
  float di = 0.f;
#pragma unroll
  for (int d = 0; d < C::DS; ++d) {
    const u32x4 qf = frag_rows<D>(Qt, w * 32, d, li, g);
    const u32x4 dof = frag_rows<D>(dOt, w * 32, d, li, g);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      di += bf16_lo(dof[e2]) * bf16_lo(of[d][e2]) + bf16_hi(dof[e2]) * bf16_hi(of[d][e2]);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      s[kb] = mfma32(frag_rows<D>(Kt, kb * 32, d, li, g), qf, s[kb]);
      dp[kb] = mfma32(frag_rows<D>(Vt, kb * 32, d, li, g), dof, dp[kb]);
    }
  }
  di = pair_sum(di);
  tile_softmax_kb<C::KB>(s, P.c);
  // P and dS packed to bf16 with keys in accumulator order: operand st holds keys
  // st*16 .. st*16+15 of this lane's query
  u32x4 pps[2 * C::KB], pds[2 * C::KB];
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      float dsv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) dsv[e] = s[kb][q4 * 4 + e] * (dp[kb][q4 * 4 + e] - di);
      const int st = kb * 2 + q4 / 2, hw = (q4 % 2) * 2;
      pps[st][hw] = pack_bf16(s[kb][q4 * 4 + 0], s[kb][q4 * 4 + 1]);
      pps[st][hw + 1] = pack_bf16(s[kb][q4 * 4 + 2], s[kb][q4 * 4 + 3]);
      pds[st][hw] = pack_bf16(dsv[0], dsv[1]);
      pds[st][hw + 1] = pack_bf16(dsv[2], dsv[3]);
    }
  f32x16 dqa[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    dqa[nb] = f32x16{};
#pragma unroll
    for (int st = 0; st < 2 * C::KB; ++st)
      dqa[nb] = mfma32(frag_cols<D>(Kt, st * 16, nb * 32, lane), pds[st], dqa[nb]);
  }
  __syncthreads();  // every wave is done reading K and V
  // dQ rows leave through this wave's 32 x D quarter of the K tile
  store_rows<D>(Kt + w * 32 * D, dqa, P.scale, P.dq + base + int64_t(w * 32) * rstride, rstride,
                nrows - w * 32, lane);
  __syncthreads();  // the staging is read back before P^T overwrites it
  // P^T and dS^T rows: query i, keys j0..j0+3
#pragma unroll
  for (int st = 0; st < 2 * C::KB; ++st)
#pragma unroll
    for (int hw = 0; hw < 4; hw += 2) {
      const int j0 = (st / 2) * 32 + ((st % 2) * 2 + hw / 2) * 8 + g * 4;
      st8(Pt + Swz<C::BS>::chunk(i, j0 >> 3) + (j0 & 7), u32x2{pps[st][hw], pps[st][hw + 1]});
      st8(dSt + Swz<C::BS>::chunk(i, j0 >> 3) + (j0 & 7), u32x2{pds[st][hw], pds[st][hw + 1]});
    }
  __syncthreads();

  // ---- key side (lane = key): dV^T = dO^T P, dK^T = Q^T dS over all 128 queries
  f32x16 av[C::NB], ak[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    av[nb] = f32x16{};
    ak[nb] = f32x16{};
  }
#pragma unroll
  for (int st = 0; st < 2 * C::KB; ++st) {
    const u32x4 pb = frag_cols<C::BS>(Pt, st * 16, w * 32, lane);
    const u32x4 db = frag_cols<C::BS>(dSt, st * 16, w * 32, lane);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      av[nb] = mfma32(frag_cols<D>(dOt, st * 16, nb * 32, lane), pb, av[nb]);
      ak[nb] = mfma32(frag_cols<D>(Qt, st * 16, nb * 32, lane), db, ak[nb]);
    }
  }
  __syncthreads();  // every wave is done with P^T and dS^T before the staging below
  uint16_t* vst = Vt + w * 32 * D;
  store_rows<D>(vst, av, 1.f, P.dv + base + int64_t(w * 32) * rstride, rstride, nrows - w * 32, lane);
  store_rows<D>(vst, ak, P.scale, P.dk + base + int64_t(w * 32) * rstride, rstride, nrows - w * 32, lane);
}

template <int D>
jfa_status launch_b128_t(const jfa::BwdLaunch& a) {
  BlkParams P{};
  P.q = static_cast<const uint16_t*>(a.q);
  P.k = static_cast<const uint16_t*>(a.k);
  P.v = static_cast<const uint16_t*>(a.v);
  P.o = static_cast<const uint16_t*>(a.out);
  P.dout = static_cast<const uint16_t*>(a.dout);
  P.dq = static_cast<uint16_t*>(a.dq);
  P.dk = static_cast<uint16_t*>(a.dk);
  P.dv = static_cast<uint16_t*>(a.dv);
  P.H = a.num_heads;
  P.c = a.scale * kLog2e;
  P.scale = a.scale;
  P.rows = int32_t(a.total_kv);
  const int64_t units = (a.total_kv / Blk128Cfg<D>::BS) * a.num_heads;
  if (units > INT32_MAX) return jfa::fail(JFA_ERR_INVALID_ARG, "too many block units");
  hipLaunchKernelGGL((block128_bwd_kernel<D>), dim3(unsigned(units)), dim3(Blk128Cfg<D>::NT), 0,
                     static_cast<hipStream_t>(a.stream), P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("128-block bwd launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

__global__ void __launch_bounds__(256) block_offsets_kernel(int32_t* out, int32_t n, int32_t block) {
  const int i = int(blockIdx.x) * 256 + int(threadIdx.x);
  if (i <= n) out[i] = i * block;
}

}  // namespace

namespace jfa {

jfa_status launch_block_offsets(int32_t* out, int64_t n, int32_t block, void* stream) {
  if (n >= INT32_MAX) return fail(JFA_ERR_INVALID_ARG, "too many blocks");
  hipLaunchKernelGGL(block_offsets_kernel, dim3(unsigned(n / 256 + 1)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), out, int32_t(n), block);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(JFA_ERR_HIP, std::string("block offsets launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

jfa_status launch_block_fwd(const FwdLaunch& a) {
  return a.head_dim == 128 ? launch_fwd_t<128>(a) : launch_fwd_t<64>(a);
}

jfa_status launch_block_bwd(const BwdLaunch& a) {
  return a.head_dim == 128 ? launch_bwd_t<128>(a) : launch_bwd_t<64>(a);
}

jfa_status launch_block128_bwd(const BwdLaunch& a) {
  return a.head_dim == 128 ? launch_b128_t<128>(a) : launch_b128_t<64>(a);
}

}  // namespace jfa
