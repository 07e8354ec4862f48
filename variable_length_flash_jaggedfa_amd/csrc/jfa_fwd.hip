// Jagged flash attention forward for gfx950 (persistent, MFMA bf16).
//
// One workgroup per persistent slot walks the tiles the host scheduler dealt to
// it ("Jagged Flash Attention for GEM": persistent kernel fed by a zigzag deal of
// KV-work-sorted tiles). A tile is 128 query rows of one (sequence, head); each
// of the 4 waves owns 32 rows. Keys stream through a double-buffered LDS ring in
// steps of 64. Per step the wave computes S^T = K Q^T (so every lane holds the
// scores of one query row and the softmax statistics stay lane-local apart from
// one swap with lane ^ 32), applies the online softmax in base 2 with the scale
// folded into the exponent ("TLX Block Attention", section 2 and Fig. 1: running
// max, correction factor, exp2), and accumulates O^T = V^T P^T, feeding the
// probability tile straight from the accumulator registers. Key steps that need
// no mask run in a separate unmasked loop; the tail step and the causal diagonal
// run masked ("Jagged Flash Attention for GEM": loop peeling).
#include "jfa_device.h"
#include "jfa_internal.h"

using namespace jfa_dev;

namespace {

template <int D>
struct FwdCfg {
  static constexpr int BM = jfa::kFwdBM;  // 128 query rows per tile
  static constexpr int BN = jfa::kFwdBN;  // 64 keys per step
  static constexpr int NT = 256;          // threads (4 waves)
  static constexpr int KS = D + 8;        // LDS row stride of the K tile (elements)
  static constexpr int VS = BN + 8;       // LDS row stride of the V^T tile
  static constexpr int K_ELEMS = BN * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr int DS = D / 16;       // MFMA k-steps over the head dim
  static constexpr int NB = D / 32;       // 32-column blocks of the head dim
  static constexpr int CH = D / 8;        // 16-byte chunks per row
  static constexpr int K_LD = BN * CH / NT;        // K chunks per thread
  static constexpr int V_GRP = (BN / 4) * CH;      // (4-row group, chunk) pairs
  static constexpr int V_LD = (V_GRP + NT - 1) / NT;
};

struct FwdParams {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  const int32_t* offsets; const int32_t* slot_ptr; const int32_t* tiles;
  uint16_t* out; float* lse;
  int32_t H, lq, total_kv;
  float c;  // scale * log2(e)
};

// Registers holding one K/V step in flight between global memory and LDS.
template <int D>
struct Stage {
  u32x4 k[FwdCfg<D>::K_LD];
  u32x4 v[FwdCfg<D>::V_LD][4];
};

template <int D>
__device__ __forceinline__ void stage_load(Stage<D>& st, const uint16_t* kbase, const uint16_t* vbase,
                                           int64_t rstride, int row0, int L, int tid) {
  using C = FwdCfg<D>;
#pragma unroll
  for (int i = 0; i < C::K_LD; ++i) {
    const int c = tid + i * C::NT;
    const int j = c / C::CH, cc = c % C::CH;
    const int row = row0 + j;
    st.k[i] = row < L ? ld16(kbase + row * rstride + cc * 8) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < C::V_LD; ++i) {
    const int pidx = tid + i * C::NT;
    const int jg = pidx % (C::BN / 4), cc = pidx / (C::BN / 4);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 4 * jg + r;
      st.v[i][r] = (pidx < C::V_GRP && row < L) ? ld16(vbase + row * rstride + cc * 8)
                                                 : u32x4{0, 0, 0, 0};
    }
  }
}

template <int D>
__device__ __forceinline__ void stage_store(const Stage<D>& st, uint16_t* buf, int tid) {
  using C = FwdCfg<D>;
  uint16_t* ks = buf;
  uint16_t* vt = buf + C::K_ELEMS;
#pragma unroll
  for (int i = 0; i < C::K_LD; ++i) {
    const int c = tid + i * C::NT;
    const int j = c / C::CH, cc = c % C::CH;
    st16(ks + j * C::KS + cc * 8, st.k[i]);
  }
#pragma unroll
  for (int i = 0; i < C::V_LD; ++i) {
    const int pidx = tid + i * C::NT;
    if (pidx >= C::V_GRP) continue;
    const int jg = pidx % (C::BN / 4), cc = pidx / (C::BN / 4);
    const int col = kperm(4 * jg);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      u32x2 w;
      w[0] = half_of(st.v[i][0], e) | (half_of(st.v[i][1], e) << 16);
      w[1] = half_of(st.v[i][2], e) | (half_of(st.v[i][3], e) << 16);
      st8(vt + (cc * 8 + e) * C::VS + col, w);
    }
  }
}

// One 64-key step for one wave: S^T, online softmax, O^T += V^T P^T.
template <int D, bool MASK, bool CAUSAL>
__device__ __forceinline__ void fwd_step(const uint16_t* buf, const u32x4 (&qf)[FwdCfg<D>::DS],
                                         f32x16 (&oacc)[FwdCfg<D>::NB], float& m, float& l,
                                         float c, int li, int g, int key0, int n_keys, int qpos) {
  using C = FwdCfg<D>;
  const uint16_t* ks = buf;
  const uint16_t* vt = buf + C::K_ELEMS;
  f32x16 s[2];
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int d = 0; d < C::DS; ++d) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 a = ld16(ks + (kb * 32 + li) * C::KS + d * 16 + g * 8);
      s[kb] = mfma32(a, qf[d], s[kb]);
    }
  }
  // scale to the log2 domain, mask, row max
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[kb][r] * c;
      if (MASK) {
        const int key = key0 + kb * 32 + (r / 4) * 8 + g * 4 + (r % 4);
        const bool dead = key >= n_keys || (CAUSAL && key > qpos);
        x = dead ? -INFINITY : x;
      }
      s[kb][r] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = pair_max(mx);
  const float m_new = fmaxf(m, mx);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = exp2_fast(m - m_use);
  m = m_new;
  float rs = 0.f;
  u32x4 pf[4];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = exp2_fast(s[kb][r] - m_use);
      const float p1 = exp2_fast(s[kb][r + 1] - m_use);
      rs += p0 + p1;
      const int step = kb * 2 + r / 8;
      pf[step][(r % 8) / 2] = pack_bf16(p0, p1);
    }
  }
  l = alpha * l + rs;
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) oacc[nb] *= alpha;
#pragma unroll
  for (int step = 0; step < 4; ++step) {
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      const u32x4 a = ld16(vt + (nb * 32 + li) * C::VS + step * 16 + g * 8);
      oacc[nb] = mfma32(a, pf[step], oacc[nb]);
    }
  }
}

template <int D, bool CAUSAL, bool BCAST>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2)))
fwd_kernel(FwdParams P) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * C::BUF];
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, g = lane >> 5, li = lane & 31;
  const int slot = xcd_slot(blockIdx.x, gridDim.x);
  const int t_begin = P.slot_ptr[slot], t_end = P.slot_ptr[slot + 1];
  const int64_t rstride = int64_t(P.H) * D;  // elements between consecutive tokens

  for (int ti = t_begin; ti < t_end; ++ti) {
    const int b = P.tiles[4 * ti + 0], h = P.tiles[4 * ti + 1], t = P.tiles[4 * ti + 2];
    const int kv0 = P.offsets[b];
    const int L = P.offsets[b + 1] - kv0;
    const int rows_total = BCAST ? P.lq : L;
    const int q_first = t * C::BM;
    const int q_rows = min(C::BM, rows_total - q_first);
    const int n_keys = CAUSAL ? min(L, q_first + q_rows) : L;
    const int n_steps = ceil_div(n_keys, C::BN);
    const int n_free = min(n_steps, (CAUSAL ? q_first : L) / C::BN);  // steps without a mask
    const int i_loc = w * 32 + li;
    const bool row_ok = i_loc < q_rows;
    const bool wave_on = w * 32 < q_rows;
    const int qpos = q_first + i_loc;  // query position (inside the sequence / dense Q)

    const uint16_t* kbase = P.k + int64_t(kv0) * rstride + int64_t(h) * D;
    const uint16_t* vbase = P.v + int64_t(kv0) * rstride + int64_t(h) * D;
    const int64_t qrow = BCAST ? int64_t(qpos) : int64_t(kv0) + qpos;

    u32x4 qf[C::DS];
#pragma unroll
    for (int d = 0; d < C::DS; ++d)
      qf[d] = row_ok ? ld16(P.q + qrow * rstride + int64_t(h) * D + d * 16 + g * 8)
                     : u32x4{0, 0, 0, 0};

    f32x16 oacc[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) oacc[nb] = f32x16{};
    float m = -INFINITY, l = 0.f;

    Stage<D> st;
    if (n_steps > 0) {
      stage_load<D>(st, kbase, vbase, rstride, 0, L, tid);
      stage_store<D>(st, lds, tid);
    }
    __syncthreads();
    for (int kt = 0; kt < n_steps; ++kt) {
      const bool more = kt + 1 < n_steps;
      if (more) stage_load<D>(st, kbase, vbase, rstride, (kt + 1) * C::BN, L, tid);
      const uint16_t* buf = lds + (kt & 1) * C::BUF;
      if (wave_on) {
        if (kt < n_free)
          fwd_step<D, false, CAUSAL>(buf, qf, oacc, m, l, P.c, li, g, kt * C::BN, n_keys, qpos);
        else
          fwd_step<D, true, CAUSAL>(buf, qf, oacc, m, l, P.c, li, g, kt * C::BN, n_keys, qpos);
      }
      if (more) stage_store<D>(st, lds + ((kt + 1) & 1) * C::BUF, tid);
      __syncthreads();
    }

    // epilogue: out = O / l (bf16), lse = (m + log2 l) * ln 2
    const float lt = pair_sum(l);
    if (row_ok) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      uint16_t* orow = BCAST ? P.out + ((int64_t(b) * P.lq + qpos) * P.H + h) * D
                             : P.out + qrow * rstride + int64_t(h) * D;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          u32x2 wv;
          wv[0] = pack_bf16(oacc[nb][q4 * 4 + 0] * inv, oacc[nb][q4 * 4 + 1] * inv);
          wv[1] = pack_bf16(oacc[nb][q4 * 4 + 2] * inv, oacc[nb][q4 * 4 + 3] * inv);
          st8(orow + nb * 32 + q4 * 8 + g * 4, wv);
        }
      }
      if (g == 0) {
        const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
        if (BCAST)
          P.lse[(int64_t(b) * P.H + h) * P.lq + qpos] = lse;
        else
          P.lse[int64_t(h) * P.total_kv + kv0 + qpos] = lse;
      }
    }
  }
}

template <int D, bool CAUSAL, bool BCAST>
jfa_status launch_t(const jfa::FwdLaunch& a) {
  FwdParams P;
  P.q = static_cast<const uint16_t*>(a.q);
  P.k = static_cast<const uint16_t*>(a.k);
  P.v = static_cast<const uint16_t*>(a.v);
  P.offsets = a.offsets;
  P.slot_ptr = a.slot_ptr;
  P.tiles = a.tiles;
  P.out = static_cast<uint16_t*>(a.out);
  P.lse = a.lse;
  P.H = a.num_heads;
  P.lq = a.lq;
  P.total_kv = int32_t(a.total_kv);
  P.c = a.scale * kLog2e;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, BCAST>), dim3(a.num_slots), dim3(256), 0,
                     static_cast<hipStream_t>(a.stream), P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("fwd launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

template <int D, bool CAUSAL, bool BCAST>
int occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_kernel<D, CAUSAL, BCAST>, 256, 0) !=
      hipSuccess)
    return 0;
  return n;
}

}  // namespace

namespace jfa {

jfa_status launch_fwd(const FwdLaunch& a) {
  const bool causal = a.flags & JFA_CAUSAL, bq = a.flags & JFA_BROADCAST_Q;
  if (a.head_dim == 128) {
    if (bq) return launch_t<128, false, true>(a);
    return causal ? launch_t<128, true, false>(a) : launch_t<128, false, false>(a);
  }
  if (bq) return launch_t<64, false, true>(a);
  return causal ? launch_t<64, true, false>(a) : launch_t<64, false, false>(a);
}

jfa_status fwd_slots_per_cu(int head_dim, uint32_t flags, int* per_cu) {
  const bool causal = flags & JFA_CAUSAL, bq = flags & JFA_BROADCAST_Q;
  int n;
  if (head_dim == 128)
    n = bq ? occupancy<128, false, true>() : causal ? occupancy<128, true, false>() : occupancy<128, false, false>();
  else
    n = bq ? occupancy<64, false, true>() : causal ? occupancy<64, true, false>() : occupancy<64, false, false>();
  if (n <= 0) return fail(JFA_ERR_HIP, "occupancy query failed for the forward kernel");
  *per_cu = n;
  return JFA_OK;
}

}  // namespace jfa
