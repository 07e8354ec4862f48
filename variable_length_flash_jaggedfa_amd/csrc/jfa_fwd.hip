// Jagged flash attention forward for gfx950 (persistent, MFMA bf16).
//
// One workgroup per persistent slot walks the tiles the host scheduler dealt to
// it ("Jagged Flash Attention for GEM": persistent kernel fed by a zigzag deal of
// KV-work-sorted tiles). A tile is 128 query rows of one (sequence, head); each
// of the 4 waves owns 32 rows and two workgroups share a compute unit, so one
// wave's softmax overlaps another wave's MFMAs on the same SIMD. Keys stream in
// steps of 64 through a double-buffered LDS ring filled by direct global->LDS
// loads issued one step ahead. Per step a
// wave computes S^T = K Q^T (each lane holds the scores of one query row, so the
// softmax statistics stay in the lane apart from one swap with lane ^ 32),
// applies the online softmax in base 2 with the scale folded into the exponent
// ("TLX Block Attention", section 2 and Fig. 1: running max, correction factor,
// exp2) and accumulates O^T = V^T P^T with P taken straight from the score
// registers and V^T read through the LDS transpose path. The accumulator rescale
// is skipped when no row max moved. Steps that need no mask run separately from
// the tail step and the causal diagonal ("Jagged Flash Attention for GEM": loop
// peeling).
#include "jfa_internal.h"
#include "jfa_tiles.h"

using namespace jfa_dev;

namespace {

template <int D>
struct FwdCfg {
  static constexpr int BM = jfa::kFwdBM;  // 128 query rows per tile
  static constexpr int QB = 1;            // 32-row blocks per wave
  static constexpr int BN = D == 128 ? 32 : 64;  // keys per step
  static constexpr int KB = BN / 32;      // 32-key blocks per step
  static constexpr int NW = BM / (32 * QB);  // waves
  static constexpr int NT = 64 * NW;
  static constexpr int NS = 3;            // LDS ring stages (prefetch distance 2)
  static constexpr int DS = D / 16;       // MFMA k-steps over the head dim
  static constexpr int NB = D / 32;       // 32-column blocks of the head dim
  static constexpr int TILE = BN * D;     // elements of one K or V tile
  static constexpr int STAGE = 2 * TILE;  // K then V
  static constexpr int LOADS = 2 * TILE / 8 / 64 / NW;  // load instructions per wave per stage
};

// Probabilities are formed against a per-row reference max that only moves when
// the running max exceeds it by more than this (log2 units), so P <= 2^8 and the
// accumulator rescale runs rarely.
constexpr float kRescaleSlack = 8.f;

struct FwdParams {
  const uint16_t* q; const uint16_t* k; const uint16_t* v;
  const int32_t* offsets; const int32_t* slot_ptr; const int32_t* tiles;
  uint16_t* out; float* lse;
  int32_t H, lq, total_kv;
  float c;  // scale * log2(e)
};

// One step of BN keys for one wave: S^T = K Q^T, online softmax, O^T += V^T P^T.
template <int D, bool MASK, bool CAUSAL>
__device__ __forceinline__ void fwd_step(const uint16_t* ks, const uint16_t* vs,
                                         const u32x4 (&qf)[FwdCfg<D>::QB][FwdCfg<D>::DS],
                                         f32x16 (&o)[FwdCfg<D>::QB][FwdCfg<D>::NB],
                                         float (&m)[FwdCfg<D>::QB], float (&l)[FwdCfg<D>::QB],
                                         float c, int lane, int key0, int n_keys, int qpos0) {
  using C = FwdCfg<D>;
  constexpr int KB = C::KB, QB = C::QB;
  const int g = lane >> 5, li = lane & 31;
  f32x16 s[QB][KB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) s[qb][kb] = f32x16{};
  // S^T: K fragments are read one k-step ahead of the MFMAs that use them
  u32x4 kf[2][KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) kf[0][kb] = frag_rows<D>(ks, kb * 32, 0, li, g);
#pragma unroll
  for (int d = 0; d < C::DS; ++d) {
    if (d + 1 < C::DS) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) kf[(d + 1) & 1][kb] = frag_rows<D>(ks, kb * 32, d + 1, li, g);
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32(kf[d & 1][kb], qf[qb][d], s[qb][kb]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // masks, step max, reference-max update
  float mx[QB];
  bool move = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float x = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (MASK) {
          const int key = key0 + kb * 32 + (r / 4) * 8 + g * 4 + (r % 4);
          const bool dead = key >= n_keys || (CAUSAL && key > qpos0 + qb * 32);
          s[qb][kb][r] = dead ? -INFINITY : s[qb][kb][r];
        }
        x = fmaxf(x, s[qb][kb][r]);
      }
    }
    mx[qb] = pair_max(x) * c;
    move = move || (mx[qb] > m[qb] + kRescaleSlack);
  }
  if (__builtin_amdgcn_ballot_w64(move)) {
    asm volatile("" ::: "memory");  // keep this rare path a branch, not a select
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_new = fmaxf(m[qb], mx[qb]);
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m[qb] - m_new);
      m[qb] = m_new;
      l[qb] *= alpha;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) o[qb][nb] *= alpha;
    }
  }
  u32x4 pf[QB][2 * KB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float m_use = m[qb] == -INFINITY ? 0.f : m[qb];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = exp2_fast(__builtin_fmaf(s[qb][kb][r], c, -m_use));
        const float p1 = exp2_fast(__builtin_fmaf(s[qb][kb][r + 1], c, -m_use));
        rs += p0 + p1;
        pf[qb][kb * 2 + r / 8][(r % 8) / 2] = pack_bf16(p0, p1);
      }
    }
    l[qb] += rs;
  }
  // O^T += V^T P^T: V^T fragments one (step, block) ahead of their MFMAs
  constexpr int NX = 2 * KB * C::NB;
  u32x4 vf[2];
  vf[0] = frag_cols<D>(vs, 0, 0, lane);
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int st = x / C::NB, nb = x % C::NB;
    if (x + 1 < NX) vf[(x + 1) & 1] = frag_cols<D>(vs, ((x + 1) / C::NB) * 16, ((x + 1) % C::NB) * 32, lane);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) o[qb][nb] = mfma32(vf[x & 1], pf[qb][st], o[qb][nb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D, bool CAUSAL, bool BCAST>
__global__ void __launch_bounds__(FwdCfg<D>::NT)
__attribute__((amdgpu_waves_per_eu(FwdCfg<D>::QB == 1 ? 2 : 1)))
fwd_kernel(FwdParams P) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::NS * C::STAGE];
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
    const int qpos0 = q_first + w * 32 * C::QB + li;  // query position of block 0 in this lane
    const uint16_t* kbase = P.k + int64_t(kv0) * rstride + int64_t(h) * D;
    const uint16_t* vbase = P.v + int64_t(kv0) * rstride + int64_t(h) * D;
    const int rowbytes = int(rstride * 2);
    // stage st holds keys [st*BN, st*BN + BN): a resource starting at that row,
    // covering the rest of the sequence (keys past the end read as zero)
    auto load_stage = [&](int st, uint16_t* buf) {
      const int64_t r0 = int64_t(st) * C::BN * rstride;
      tile_load<D, C::BN, C::NW>(buf, rows_rsrc<D>(kbase + r0, rstride, L - st * C::BN), rowbytes, w, lane);
      tile_load<D, C::BN, C::NW>(buf + C::TILE, rows_rsrc<D>(vbase + r0, rstride, L - st * C::BN),
                                 rowbytes, w, lane);
    };

    // Q fragments first, then the first two K/V stages (older loads complete first)
    u32x4 qf[C::QB][C::DS];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const int qpos = qpos0 + qb * 32;
      const bool ok = qpos < rows_total;
      const int64_t qrow = BCAST ? int64_t(qpos) : int64_t(kv0) + qpos;
#pragma unroll
      for (int d = 0; d < C::DS; ++d)
        qf[qb][d] = ok ? ld16(P.q + qrow * rstride + int64_t(h) * D + d * 16 + g * 8)
                       : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int st = 0; st < C::NS - 1; ++st) {
      if (st < n_steps) load_stage(st, lds + st * C::STAGE);
    }
    f32x16 o[C::QB][C::NB];
    float m[C::QB], l[C::QB];
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      m[qb] = -INFINITY;
      l[qb] = 0.f;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) o[qb][nb] = f32x16{};
    }

    for (int kt = 0; kt < n_steps; ++kt) {
      if (C::NS > 2 && kt + 1 < n_steps)
        wait_vmem_le<C::LOADS>();  // stage kt landed; stage kt+1 may still be in flight
      else
        wait_vmem();
      __syncthreads();
      if (kt + C::NS - 1 < n_steps) {
        const int nk = kt + C::NS - 1;
        load_stage(nk, lds + (nk % C::NS) * C::STAGE);
      }
      const uint16_t* cur = lds + (kt % C::NS) * C::STAGE;
      if (kt < n_free)
        fwd_step<D, false, CAUSAL>(cur, cur + C::TILE, qf, o, m, l, P.c, lane, kt * C::BN, n_keys, qpos0);
      else
        fwd_step<D, true, CAUSAL>(cur, cur + C::TILE, qf, o, m, l, P.c, lane, kt * C::BN, n_keys, qpos0);
    }

    // epilogue: out = O / l (bf16), lse = (m + log2 l) * ln 2
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) {
      const int qpos = qpos0 + qb * 32;
      const float lt = pair_sum(l[qb]);
      if (qpos < rows_total) {
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        uint16_t* orow = BCAST ? P.out + ((int64_t(b) * P.lq + qpos) * P.H + h) * D
                               : P.out + (int64_t(kv0) + qpos) * rstride + int64_t(h) * D;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            u32x2 wv;
            wv[0] = pack_bf16(o[qb][nb][q4 * 4 + 0] * inv, o[qb][nb][q4 * 4 + 1] * inv);
            wv[1] = pack_bf16(o[qb][nb][q4 * 4 + 2] * inv, o[qb][nb][q4 * 4 + 3] * inv);
            st8(orow + nb * 32 + q4 * 8 + g * 4, wv);
          }
        }
        if (g == 0) {
          const float lse = lt > 0.f ? (m[qb] + __log2f(lt)) * kLn2 : -INFINITY;
          if (BCAST)
            P.lse[(int64_t(b) * P.H + h) * P.lq + qpos] = lse;
          else
            P.lse[int64_t(h) * P.total_kv + kv0 + qpos] = lse;
        }
      }
    }
    __syncthreads();  // the next tile's first loads overwrite the first stages
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
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, BCAST>), dim3(a.num_slots), dim3(FwdCfg<D>::NT), 0,
                     static_cast<hipStream_t>(a.stream), P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("fwd launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

template <int D, bool CAUSAL, bool BCAST>
int occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_kernel<D, CAUSAL, BCAST>,
                                                   FwdCfg<D>::NT, 0) != hipSuccess)
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
