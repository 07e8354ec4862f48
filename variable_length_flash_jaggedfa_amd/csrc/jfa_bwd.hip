// Jagged flash attention backward for gfx950 (persistent, MFMA bf16).
//
// A tile is 128 keys of one (sequence, head); each of the 4 waves keeps 32 keys
// of K and V in registers together with its dK^T and dV^T accumulators. The
// workgroup walks the 64-row query steps that can attend those keys. Per step:
//   - Q, dO (row-major and transposed) go to LDS; Di = rowsum(dO * out) is summed
//     while they are staged, so no separate preprocessing pass runs ("TLX Block
//     Attention", sections 2 and 4);
//   - S = Q K^T and dP = dO V^T (lane = key, registers = query rows);
//   - P = 2^(S*scale*log2e - lse*log2e) rebuilt from the saved lse;
//     dS = P * (dP - Di);
//   - dV^T += dO^T P and dK^T += Q^T dS, P and dS fed from the accumulators;
//   - dS goes to LDS so the whole workgroup forms dQ = dS K over its 128 keys
//     (the staging of the dQ partial before the global sum), and one fp32 atomic
//     per element adds it into the dQ accumulator ("Jagged Flash Attention for
//     GEM", backward / dQ section). For broadcast-Q every tile of a head adds into
//     the same [Lq, D] slice.
// A finalize pass converts the accumulator to bf16 and applies the scale.
#include "jfa_device.h"
#include "jfa_internal.h"

using namespace jfa_dev;

namespace {

template <int D>
struct BwdCfg {
  static constexpr int BN = jfa::kBwdBN;  // 128 keys per tile
  static constexpr int BM = jfa::kBwdBM;  // 64 query rows per step
  static constexpr int NT = 256;
  static constexpr int QS = D + 8;        // row stride of Q / dO tiles [BM][D]
  static constexpr int TS = BM + 8;       // row stride of Q^T / dO^T tiles [D][BM]
  static constexpr int SS = BN + 8;       // row stride of the dS tile [BM][BN]
  static constexpr int KS = D + 8;        // row stride of the K staging tile [BN][D]
  static constexpr int DS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int CH = D / 8;
  static constexpr int GRP = (BM / 4) * CH;       // (4-row group, chunk) pairs of a step
  // LDS carve-up (elements of 16 bits)
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = OFF_Q + BM * QS;
  static constexpr int OFF_QT = OFF_DO + BM * QS;
  static constexpr int OFF_DOT = OFF_QT + D * TS;
  static constexpr int OFF_DS = OFF_DOT + D * TS;
  static constexpr int OFF_F32 = OFF_DS + BM * SS;        // lse[BM], Di[2][BM] as floats
  static constexpr int ELEMS = OFF_F32 + 2 * 3 * BM;
  static_assert(BN * KS <= OFF_DS, "K staging tile must fit below the dS tile");
  // dQ work split: (BM/32) x NB blocks of 32x32 over 4 waves
  static constexpr int DQ_BLOCKS = (BM / 32) * NB / 4;
};

struct BwdParams {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; const uint16_t* o; const uint16_t* dout;
  const float* lse;
  const int32_t* offsets; const int32_t* slot_ptr; const int32_t* tiles;
  uint16_t* dk; uint16_t* dv;
  float* dq_acc;
  int32_t H, lq, total_kv;
  float c;      // scale * log2(e)
  float scale;
};

template <int D, bool CAUSAL, bool BCAST>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
bwd_kernel(BwdParams P) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::ELEMS];
  uint16_t* Qs = lds + C::OFF_Q;
  uint16_t* dOs = lds + C::OFF_DO;
  uint16_t* QTs = lds + C::OFF_QT;
  uint16_t* dOTs = lds + C::OFF_DOT;
  uint16_t* dSs = lds + C::OFF_DS;
  float* lse_s = reinterpret_cast<float*>(lds + C::OFF_F32);
  float* di_s = lse_s + C::BM;  // two buffers of BM

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int slot = xcd_slot(blockIdx.x, gridDim.x);
  const int t_begin = P.slot_ptr[slot], t_end = P.slot_ptr[slot + 1];
  const int64_t rstride = int64_t(P.H) * D;

  for (int ti = t_begin; ti < t_end; ++ti) {
    const int b = P.tiles[4 * ti + 0], h = P.tiles[4 * ti + 1], n = P.tiles[4 * ti + 2];
    const int kv0 = P.offsets[b];
    const int L = P.offsets[b + 1] - kv0;
    const int key0 = n * C::BN;
    const int rows_total = BCAST ? P.lq : L;
    const int jw = key0 + w * 32 + li;  // this lane's key (inside the sequence)
    const bool key_ok = jw < L;
    const uint16_t* kbase = P.k + int64_t(kv0) * rstride + int64_t(h) * D;
    const uint16_t* vbase = P.v + int64_t(kv0) * rstride + int64_t(h) * D;

    // resident K / V fragments (B operands of S = Q K^T and dP = dO V^T)
    u32x4 kf[C::DS], vf[C::DS];
#pragma unroll
    for (int d = 0; d < C::DS; ++d) {
      kf[d] = key_ok ? ld16(kbase + int64_t(jw) * rstride + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
      vf[d] = key_ok ? ld16(vbase + int64_t(jw) * rstride + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
    }
    // K tile through LDS to build the K^T-side fragments of dQ = dS K
    for (int c = tid; c < C::BN * C::CH; c += C::NT) {
      const int j = c / C::CH, cc = c % C::CH;
      const int row = key0 + j;
      st16(lds + j * C::KS + cc * 8,
           row < L ? ld16(kbase + int64_t(row) * rstride + cc * 8) : u32x4{0, 0, 0, 0});
    }
    __syncthreads();
    // dQ blocks of this wave: column block db of D, row blocks ib0 .. ib0+DQ_BLOCKS-1
    const int dq_db = w % C::NB;
    const int dq_ib0 = (w / C::NB) * C::DQ_BLOCKS;
    u32x4 ktf[C::BN / 16];
#pragma unroll
    for (int s = 0; s < C::BN / 16; ++s) {
      u32x4 f;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int j0 = s * 16 + g * 8 + 2 * e2;
        const uint32_t lo = lds[j0 * C::KS + dq_db * 32 + li];
        const uint32_t hi = lds[(j0 + 1) * C::KS + dq_db * 32 + li];
        f[e2] = lo | (hi << 16);
      }
      ktf[s] = f;
    }
    __syncthreads();

    f32x16 dvacc[C::NB], dkacc[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      dvacc[nb] = f32x16{};
      dkacc[nb] = f32x16{};
    }

    const int qt_lo = CAUSAL ? key0 / C::BM : 0;
    const int qt_hi = ceil_div(rows_total, C::BM);
    for (int qt = qt_lo; qt < qt_hi; ++qt) {
      const int par = (qt - qt_lo) & 1;
      float* di_cur = di_s + par * C::BM;
      const int q_first = qt * C::BM;
      // ---- stage Q, dO (row-major + transposed), lse, Di into LDS. The CH chunks
      // of a 4-row group sit on CH consecutive lanes of one wave, so each row's Di
      // is reduced with fixed-order lane swaps (deterministic, no atomics).
      for (int pidx = tid; pidx < C::GRP; pidx += C::NT) {
        const int cc = pidx % C::CH, jg = pidx / C::CH;
        u32x4 qv[4], dv4[4];
        float di_part[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qpos = q_first + 4 * jg + r;
          const bool ok = qpos < rows_total;
          const int64_t qrow = BCAST ? int64_t(qpos) : int64_t(kv0) + qpos;
          const int64_t orow = BCAST ? int64_t(b) * P.lq + qpos : int64_t(kv0) + qpos;
          qv[r] = ok ? ld16(P.q + qrow * rstride + int64_t(h) * D + cc * 8) : u32x4{0, 0, 0, 0};
          dv4[r] = ok ? ld16(P.dout + orow * rstride + int64_t(h) * D + cc * 8) : u32x4{0, 0, 0, 0};
          const u32x4 ov = ok ? ld16(P.o + orow * rstride + int64_t(h) * D + cc * 8) : u32x4{0, 0, 0, 0};
          float acc = 0.f;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            acc += bf16_lo(dv4[r][e2]) * bf16_lo(ov[e2]);
            acc += bf16_hi(dv4[r][e2]) * bf16_hi(ov[e2]);
          }
#pragma unroll
          for (int m = 1; m < C::CH; m <<= 1) acc += __shfl_xor(acc, m);
          di_part[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          st16(Qs + (4 * jg + r) * C::QS + cc * 8, qv[r]);
          st16(dOs + (4 * jg + r) * C::QS + cc * 8, dv4[r]);
        }
        if (cc == 0) *reinterpret_cast<f32x4*>(di_cur + 4 * jg) = f32x4{di_part[0], di_part[1], di_part[2], di_part[3]};
        const int col = kperm(4 * jg);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          u32x2 a, bb;
          a[0] = half_of(qv[0], e) | (half_of(qv[1], e) << 16);
          a[1] = half_of(qv[2], e) | (half_of(qv[3], e) << 16);
          bb[0] = half_of(dv4[0], e) | (half_of(dv4[1], e) << 16);
          bb[1] = half_of(dv4[2], e) | (half_of(dv4[3], e) << 16);
          st8(QTs + (cc * 8 + e) * C::TS + col, a);
          st8(dOTs + (cc * 8 + e) * C::TS + col, bb);
        }
      }
      if (tid < C::BM) {
        const int qpos = q_first + tid;
        float x = INFINITY;  // rows past the end get P = 0
        if (qpos < rows_total)
          x = (BCAST ? P.lse[(int64_t(b) * P.H + h) * P.lq + qpos]
                     : P.lse[int64_t(h) * P.total_kv + kv0 + qpos]) * kLog2e;
        lse_s[tid] = x;
      }
      __syncthreads();

      // ---- S = Q K^T, dP = dO V^T for this wave's 32 keys
      f32x16 sacc[2], dpacc[2];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
        sacc[ib] = f32x16{};
        dpacc[ib] = f32x16{};
      }
#pragma unroll 2
      for (int d = 0; d < C::DS; ++d) {
#pragma unroll
        for (int ib = 0; ib < 2; ++ib) {
          const u32x4 aq = ld16(Qs + (ib * 32 + li) * C::QS + d * 16 + g * 8);
          sacc[ib] = mfma32(aq, kf[d], sacc[ib]);
          const u32x4 ad = ld16(dOs + (ib * 32 + li) * C::QS + d * 16 + g * 8);
          dpacc[ib] = mfma32(ad, vf[d], dpacc[ib]);
        }
      }

      const bool mask = (CAUSAL && q_first < key0 + C::BN) || (key0 + C::BN > L);
      u32x4 pp[4], pds[4];
#pragma unroll
      for (int ib = 0; ib < 2; ++ib) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int i0 = ib * 32 + q4 * 8 + g * 4;
          const f32x4 lse4 = *reinterpret_cast<const f32x4*>(lse_s + i0);
          const f32x4 di4 = *reinterpret_cast<const f32x4*>(di_cur + i0);
          float pv[4], dsv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = q4 * 4 + e;
            float p = exp2_fast(sacc[ib][r] * P.c - lse4[e]);
            if (mask) {
              const int qpos = q_first + i0 + e;
              const bool dead = !key_ok || (CAUSAL && jw > qpos);
              p = dead ? 0.f : p;
            }
            pv[e] = p;
            dsv[e] = p * (dpacc[ib][r] - di4[e]);
          }
          // step s = ib*2 + q4/2 covers rows ib*32 + 16*(q4/2) .. +15
          const int s = ib * 2 + q4 / 2;
          const int hw = (q4 % 2) * 2;
          pp[s][hw] = pack_bf16(pv[0], pv[1]);
          pp[s][hw + 1] = pack_bf16(pv[2], pv[3]);
          pds[s][hw] = pack_bf16(dsv[0], dsv[1]);
          pds[s][hw + 1] = pack_bf16(dsv[2], dsv[3]);
        }
      }
      // ---- dV^T += dO^T P, dK^T += Q^T dS
#pragma unroll 2
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const u32x4 a = ld16(dOTs + (nb * 32 + li) * C::TS + s * 16 + g * 8);
          dvacc[nb] = mfma32(a, pp[s], dvacc[nb]);
          const u32x4 aq = ld16(QTs + (nb * 32 + li) * C::TS + s * 16 + g * 8);
          dkacc[nb] = mfma32(aq, pds[s], dkacc[nb]);
        }
      }
      // ---- dS tile to LDS as [row i][key j]
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          // register pair x of step s holds rows (s/2)*32 + ((s%2)*2 + x/2)*8 + g*4 + 2*(x%2) + {0,1}
          const int i0 = (s / 2) * 32 + ((s % 2) * 2 + x / 2) * 8 + g * 4 + 2 * (x % 2);
          dSs[i0 * C::SS + w * 32 + li] = uint16_t(pds[s][x] & 0xffffu);
          dSs[(i0 + 1) * C::SS + w * 32 + li] = uint16_t(pds[s][x] >> 16);
        }
      }
      __syncthreads();

      // ---- dQ partial over the workgroup's 128 keys, then fp32 atomics
#pragma unroll
      for (int x = 0; x < C::DQ_BLOCKS; ++x) {
        const int ib = dq_ib0 + x;
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < C::BN / 16; ++s) {
          const u32x4 a = ld16(dSs + (ib * 32 + li) * C::SS + s * 16 + g * 8);
          acc = mfma32(a, ktf[s], acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = ib * 32 + (r / 4) * 8 + g * 4 + (r % 4);
          const int qpos = q_first + i;
          if (qpos < rows_total) {
            const int64_t row = BCAST ? int64_t(qpos) : int64_t(kv0) + qpos;
            unsafeAtomicAdd(P.dq_acc + row * rstride + int64_t(h) * D + dq_db * 32 + li, acc[r]);
          }
        }
      }
    }
    __syncthreads();  // the next tile reuses the Q/dO region for its K staging

    // ---- dK = scale * dK^T, dV = dV^T (bf16)
    if (key_ok) {
      uint16_t* dkrow = P.dk + (int64_t(kv0) + jw) * rstride + int64_t(h) * D;
      uint16_t* dvrow = P.dv + (int64_t(kv0) + jw) * rstride + int64_t(h) * D;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 a, bb;
          a[0] = pack_bf16(dkacc[nb][q4 * 4 + 0] * P.scale, dkacc[nb][q4 * 4 + 1] * P.scale);
          a[1] = pack_bf16(dkacc[nb][q4 * 4 + 2] * P.scale, dkacc[nb][q4 * 4 + 3] * P.scale);
          bb[0] = pack_bf16(dvacc[nb][q4 * 4 + 0], dvacc[nb][q4 * 4 + 1]);
          bb[1] = pack_bf16(dvacc[nb][q4 * 4 + 2], dvacc[nb][q4 * 4 + 3]);
          st8(dkrow + nb * 32 + q4 * 8 + g * 4, a);
          st8(dvrow + nb * 32 + q4 * 8 + g * 4, bb);
        }
      }
    }
  }
}

// zero a float buffer (n is a multiple of 4)
__global__ void __launch_bounds__(256) zero_kernel(float* __restrict__ x, int64_t n4) {
  for (int64_t i = blockIdx.x * int64_t(256) + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256)
    reinterpret_cast<f32x4*>(x)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// dq = bf16(scale * acc), 4 elements per thread step
__global__ void __launch_bounds__(256) dq_finalize_kernel(const float* __restrict__ acc,
                                                         uint16_t* __restrict__ dq, int64_t n4,
                                                         float scale) {
  for (int64_t i = blockIdx.x * int64_t(256) + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256) {
    const f32x4 a = reinterpret_cast<const f32x4*>(acc)[i];
    u32x2 o;
    o[0] = pack_bf16(a[0] * scale, a[1] * scale);
    o[1] = pack_bf16(a[2] * scale, a[3] * scale);
    reinterpret_cast<u32x2*>(dq)[i] = o;
  }
}

int grid_for(int64_t n4) {
  const int64_t g = (n4 + 255) / 256;
  return int(g < 8192 ? (g > 0 ? g : 1) : 8192);
}

template <int D, bool CAUSAL, bool BCAST>
jfa_status launch_t(const jfa::BwdLaunch& a) {
  BwdParams P;
  P.q = static_cast<const uint16_t*>(a.q);
  P.k = static_cast<const uint16_t*>(a.k);
  P.v = static_cast<const uint16_t*>(a.v);
  P.o = static_cast<const uint16_t*>(a.out);
  P.dout = static_cast<const uint16_t*>(a.dout);
  P.lse = a.lse;
  P.offsets = a.offsets;
  P.slot_ptr = a.slot_ptr;
  P.tiles = a.tiles;
  P.dk = static_cast<uint16_t*>(a.dk);
  P.dv = static_cast<uint16_t*>(a.dv);
  P.dq_acc = a.dq_acc;
  P.H = a.num_heads;
  P.lq = a.lq;
  P.total_kv = int32_t(a.total_kv);
  P.c = a.scale * kLog2e;
  P.scale = a.scale;
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const int64_t rows = BCAST ? int64_t(a.lq) : a.total_kv;
  const int64_t n4 = rows * a.num_heads * D / 4;
  if (n4 > 0) hipLaunchKernelGGL(zero_kernel, dim3(grid_for(n4)), dim3(256), 0, st, a.dq_acc, n4);
  if (a.total_kv > 0)
    hipLaunchKernelGGL((bwd_kernel<D, CAUSAL, BCAST>), dim3(a.num_slots), dim3(256), 0, st, P);
  if (n4 > 0)
    hipLaunchKernelGGL(dq_finalize_kernel, dim3(grid_for(n4)), dim3(256), 0, st, a.dq_acc,
                       static_cast<uint16_t*>(a.dq), n4, a.scale);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("bwd launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

template <int D, bool CAUSAL, bool BCAST>
int occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, bwd_kernel<D, CAUSAL, BCAST>, 256, 0) !=
      hipSuccess)
    return 0;
  return n;
}

}  // namespace

namespace jfa {

jfa_status launch_bwd(const BwdLaunch& a) {
  const bool causal = a.flags & JFA_CAUSAL, bq = a.flags & JFA_BROADCAST_Q;
  if (a.head_dim == 128) {
    if (bq) return launch_t<128, false, true>(a);
    return causal ? launch_t<128, true, false>(a) : launch_t<128, false, false>(a);
  }
  if (bq) return launch_t<64, false, true>(a);
  return causal ? launch_t<64, true, false>(a) : launch_t<64, false, false>(a);
}

jfa_status bwd_slots_per_cu(int head_dim, uint32_t flags, int* per_cu) {
  const bool causal = flags & JFA_CAUSAL, bq = flags & JFA_BROADCAST_Q;
  int n;
  if (head_dim == 128)
    n = bq ? occupancy<128, false, true>() : causal ? occupancy<128, true, false>() : occupancy<128, false, false>();
  else
    n = bq ? occupancy<64, false, true>() : causal ? occupancy<64, true, false>() : occupancy<64, false, false>();
  if (n <= 0) return fail(JFA_ERR_HIP, "occupancy query failed for the backward kernel");
  *per_cu = n;
  return JFA_OK;
}

}  // namespace jfa
