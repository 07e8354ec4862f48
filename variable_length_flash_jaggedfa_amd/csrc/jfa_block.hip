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
#include "jfa_device.h"
#include "jfa_internal.h"

using namespace jfa_dev;

namespace {

constexpr int kBS = jfa::kBlock;  // 64

template <int D>
struct BlkCfg {
  static constexpr int NT = 128;          // two waves
  static constexpr int TS = kBS + 8;      // row stride of transposed tiles [D][64]
  static constexpr int DS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int CH = D / 8;
  static constexpr int GRP = (kBS / 4) * CH;   // (4-row group, chunk) pairs of a tile
};

struct BlkParams {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; const uint16_t* o; const uint16_t* dout;
  uint16_t* out; uint16_t* dq; uint16_t* dk; uint16_t* dv;
  int32_t H;
  float c;      // scale * log2(e)
  float scale;
};

// Write a 64 x D bf16 tile (rows tok0.., head h) transposed into LDS as [D][64],
// keys permuted by kperm inside each 16-group.
template <int D>
__device__ __forceinline__ void load_transposed(uint16_t* dst, const uint16_t* base, int64_t rstride,
                                                int tid) {
  using C = BlkCfg<D>;
  for (int pidx = tid; pidx < C::GRP; pidx += C::NT) {
    const int jg = pidx % (kBS / 4), cc = pidx / (kBS / 4);
    u32x4 x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = ld16(base + int64_t(4 * jg + r) * rstride + cc * 8);
    const int col = kperm(4 * jg);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x2 wv;
      wv[0] = half_of(x[0], e) | (half_of(x[1], e) << 16);
      wv[1] = half_of(x[2], e) | (half_of(x[3], e) << 16);
      st8(dst + (cc * 8 + e) * C::TS + col, wv);
    }
  }
}

template <int D>
__global__ void __launch_bounds__(128) block_fwd_kernel(BlkParams P) {
  using C = BlkCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * C::TS];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int blk = blockIdx.x / P.H, h = blockIdx.x % P.H;
  const int64_t rstride = int64_t(P.H) * D;
  const int64_t base = int64_t(blk) * kBS * rstride + int64_t(h) * D;

  load_transposed<D>(vt, P.v + base, rstride, tid);
  u32x4 qf[C::DS];
#pragma unroll
  for (int d = 0; d < C::DS; ++d) qf[d] = ld16(P.q + base + int64_t(w * 32 + li) * rstride + d * 16 + g * 8);
  // S^T = K Q^T (64 keys x this wave's 32 queries), fresh accumulators
  f32x16 s[2];
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int d = 0; d < C::DS; ++d) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 a = ld16(P.k + base + int64_t(kb * 32 + li) * rstride + d * 16 + g * 8);
      s[kb] = mfma32(a, qf[d], s[kb]);
    }
  }
  // exact softmax of the one tile: no running max, no correction factor
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = pair_max(mx) * P.c;
  float rs = 0.f;
  u32x4 pf[4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = exp2_fast(s[kb][r] * P.c - mx);
      const float p1 = exp2_fast(s[kb][r + 1] * P.c - mx);
      rs += p0 + p1;
      pf[kb * 2 + r / 8][(r % 8) / 2] = pack_bf16(p0, p1);
    }
  }
  const float inv = 1.f / pair_sum(rs);
  __syncthreads();
  // O^T = V^T P^T, one fresh product per 32-column block
  uint16_t* orow = P.out + base + int64_t(w * 32 + li) * rstride;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    f32x16 o = f32x16{};
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      const u32x4 a = ld16(vt + (nb * 32 + li) * C::TS + step * 16 + g * 8);
      o = mfma32(a, pf[step], o);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 wv;
      wv[0] = pack_bf16(o[q4 * 4 + 0] * inv, o[q4 * 4 + 1] * inv);
      wv[1] = pack_bf16(o[q4 * 4 + 2] * inv, o[q4 * 4 + 3] * inv);
      st8(orow + nb * 32 + q4 * 8 + g * 4, wv);
    }
  }
}

template <int D>
__global__ void __launch_bounds__(128) block_bwd_kernel(BlkParams P) {
  using C = BlkCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[3 * D * C::TS + 2 * kBS * C::TS];
  uint16_t* KT = lds;
  uint16_t* QT = KT + D * C::TS;
  uint16_t* dOT = QT + D * C::TS;
  uint16_t* Pm = dOT + D * C::TS;      // P as [key][query], queries permuted by kperm
  uint16_t* dSm = Pm + kBS * C::TS;    // dS as [key][query]
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int blk = blockIdx.x / P.H, h = blockIdx.x % P.H;
  const int64_t rstride = int64_t(P.H) * D;
  const int64_t base = int64_t(blk) * kBS * rstride + int64_t(h) * D;

  load_transposed<D>(KT, P.k + base, rstride, tid);
  load_transposed<D>(QT, P.q + base, rstride, tid);
  load_transposed<D>(dOT, P.dout + base, rstride, tid);

  // ---- phase 1: this wave's 32 query rows (lane = query)
  const int i = w * 32 + li;
  u32x4 qf[C::DS], dof[C::DS];
  float di = 0.f;
#pragma unroll
  for (int d = 0; d < C::DS; ++d) {
    qf[d] = ld16(P.q + base + int64_t(i) * rstride + d * 16 + g * 8);
    dof[d] = ld16(P.dout + base + int64_t(i) * rstride + d * 16 + g * 8);
    const u32x4 of = ld16(P.o + base + int64_t(i) * rstride + d * 16 + g * 8);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      di += bf16_lo(dof[d][e2]) * bf16_lo(of[e2]) + bf16_hi(dof[d][e2]) * bf16_hi(of[e2]);
  }
  di = pair_sum(di);  // Di = rowsum(dO * out), computed inline
  f32x16 s[2], dp[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
    dp[kb] = f32x16{};
  }
#pragma unroll
  for (int d = 0; d < C::DS; ++d) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 ak = ld16(P.k + base + int64_t(kb * 32 + li) * rstride + d * 16 + g * 8);
      s[kb] = mfma32(ak, qf[d], s[kb]);
      const u32x4 av = ld16(P.v + base + int64_t(kb * 32 + li) * rstride + d * 16 + g * 8);
      dp[kb] = mfma32(av, dof[d], dp[kb]);
    }
  }
  // recompute the exact softmax statistics of the tile (no stored lse)
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = pair_max(mx) * P.c;
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(s[kb][r] * P.c - mx);
      s[kb][r] = p;
      rs += p;
    }
  const float inv = 1.f / pair_sum(rs);
  u32x4 pdsT[4];
  const int ip = kperm(i);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = s[kb][r] * inv, p1 = s[kb][r + 1] * inv;
      const float d0 = p0 * (dp[kb][r] - di), d1 = p1 * (dp[kb][r + 1] - di);
      const uint32_t pk = pack_bf16(p0, p1), dk2 = pack_bf16(d0, d1);
      pdsT[kb * 2 + r / 8][(r % 8) / 2] = dk2;
      // P and dS to LDS as [key][query] for the key-side products
      const int j0 = kb * 32 + (r / 4) * 8 + g * 4 + (r % 4);
      Pm[j0 * C::TS + ip] = uint16_t(pk & 0xffffu);
      Pm[(j0 + 1) * C::TS + ip] = uint16_t(pk >> 16);
      dSm[j0 * C::TS + ip] = uint16_t(dk2 & 0xffffu);
      dSm[(j0 + 1) * C::TS + ip] = uint16_t(dk2 >> 16);
    }
  }
  __syncthreads();
  // dQ^T = K^T dS^T (32-column blocks), dq = scale * dQ
  uint16_t* dqrow = P.dq + base + int64_t(i) * rstride;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      const u32x4 a = ld16(KT + (nb * 32 + li) * C::TS + step * 16 + g * 8);
      acc = mfma32(a, pdsT[step], acc);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 wv;
      wv[0] = pack_bf16(acc[q4 * 4 + 0] * P.scale, acc[q4 * 4 + 1] * P.scale);
      wv[1] = pack_bf16(acc[q4 * 4 + 2] * P.scale, acc[q4 * 4 + 3] * P.scale);
      st8(dqrow + nb * 32 + q4 * 8 + g * 4, wv);
    }
  }

  // ---- phase 2: this wave's 32 keys (lane = key): dV^T = dO^T P, dK^T = Q^T dS
  const int j = w * 32 + li;
  uint16_t* dvrow = P.dv + base + int64_t(j) * rstride;
  uint16_t* dkrow = P.dk + base + int64_t(j) * rstride;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    f32x16 av = f32x16{}, ak = f32x16{};
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      const u32x4 bp = ld16(Pm + j * C::TS + step * 16 + g * 8);
      const u32x4 bd = ld16(dSm + j * C::TS + step * 16 + g * 8);
      av = mfma32(ld16(dOT + (nb * 32 + li) * C::TS + step * 16 + g * 8), bp, av);
      ak = mfma32(ld16(QT + (nb * 32 + li) * C::TS + step * 16 + g * 8), bd, ak);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 a, bb;
      a[0] = pack_bf16(av[q4 * 4 + 0], av[q4 * 4 + 1]);
      a[1] = pack_bf16(av[q4 * 4 + 2], av[q4 * 4 + 3]);
      bb[0] = pack_bf16(ak[q4 * 4 + 0] * P.scale, ak[q4 * 4 + 1] * P.scale);
      bb[1] = pack_bf16(ak[q4 * 4 + 2] * P.scale, ak[q4 * 4 + 3] * P.scale);
      st8(dvrow + nb * 32 + q4 * 8 + g * 4, a);
      st8(dkrow + nb * 32 + q4 * 8 + g * 4, bb);
    }
  }
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
  const int64_t units = (a.total_kv / kBS) * a.num_heads;
  if (units > INT32_MAX) return jfa::fail(JFA_ERR_INVALID_ARG, "too many block units");
  hipLaunchKernelGGL(block_fwd_kernel<D>, dim3(unsigned(units)), dim3(128), 0,
                     static_cast<hipStream_t>(a.stream), P);
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
  const int64_t units = (a.total_kv / kBS) * a.num_heads;
  if (units > INT32_MAX) return jfa::fail(JFA_ERR_INVALID_ARG, "too many block units");
  hipLaunchKernelGGL(block_bwd_kernel<D>, dim3(unsigned(units)), dim3(128), 0,
                     static_cast<hipStream_t>(a.stream), P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("block bwd launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

}  // namespace

namespace jfa {

jfa_status launch_block_fwd(const FwdLaunch& a) {
  return a.head_dim == 128 ? launch_fwd_t<128>(a) : launch_fwd_t<64>(a);
}

jfa_status launch_block_bwd(const BwdLaunch& a) {
  return a.head_dim == 128 ? launch_bwd_t<128>(a) : launch_bwd_t<64>(a);
}

}  // namespace jfa
