// Jagged flash attention backward for gfx950 (MFMA bf16), without atomics.
//
// The backward rebuilds P from Q, K and the saved lse, forms Di = rowsum(dO*out)
// inline ("TLX Block Attention", sections 2 and 4) and produces dQ, dK and dV.
// It runs as two passes over the same tiles the host scheduler deals
// ("Jagged Flash Attention for GEM", backward / dQ section):
//
//   dQ pass (query-tile outer, forward schedule). Each wave keeps 32 query rows
//     of Q and dO in registers, computes Di for them, and streams the keys of
//     its sequence through a 4-stage LDS ring: S^T = K Q^T and dP^T = V dO^T,
//     P = 2^(S*scale*log2e - lse*log2e), dS = P * (dP - Di), dQ^T += K^T dS^T.
//     dQ stays in registers and is written once; Di is written for the other pass.
//   dK/dV pass (key-tile outer, backward schedule). Each 32-key block of a tile
//     belongs to a pair of waves that stream the query rows (Q, dO, -lse/scale,
//     -Di) through a 3-stage LDS ring: one wave keeps K and dV^T (S = Q K^T, P,
//     dV^T += dO^T P), the other V and dK^T (dP = dO V^T, dS = P (dP - Di) with
//     the P its partner leaves in LDS, dK^T += Q^T dS).
//
// Each pass recomputes S and dP, so the backward runs 7 matrix products instead
// of 5; in exchange no partial result is ever summed through memory atomics.
// For broadcast-Q every sequence adds into the same dQ: the dQ pass gives each
// workgroup a (query tile, head, group of sequences), accumulates on chip over
// the group, stores one float32 partial per group, and a last kernel sums the
// partials in a fixed order.
//
// With rotary embeddings the passes read rotated copies of Q and K and turn dQ
// (dQ pass) and dK (dK/dV pass) back to the unrotated rows in registers just
// before their rows are stored.
#include <type_traits>

#include "jfa_internal.h"
#include "jfa_rope.h"
#include "jfa_sparse.h"
#include "jfa_tiles.h"

using namespace jfa_dev;

namespace {

template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------- dQ pass
// NW waves of 32 query rows each: 4 for the jagged pass (the forward tiles of 128
// rows), 8 for broadcast-Q (256 dense query rows share one key stream).
template <int D, int NW_ = jfa::kFwdBM / 32>
struct DqCfg {
  static constexpr int NW = NW_;                 // waves, 32 rows each
  static constexpr int BM = 32 * NW;             // query rows per tile
  static constexpr int NT = 64 * NW;
  static constexpr int BN = D == 128 ? 32 : 64;  // keys per step
  static constexpr int KB = BN / 32;
  static constexpr int NS = 4;                   // LDS ring stages
  static constexpr int DS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int NX = 2 * KB * NB;         // dQ products per step
  static constexpr int TILE = BN * D;
  static constexpr int STAGE = 2 * TILE;         // K then V
  static constexpr int LOADS = 2 * TILE / 8 / 64 / NW;
};

struct DqParams {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; const uint16_t* o; const uint16_t* dout;
  const float* lse;
  float* di;                  // -Di out, same layout as lse
  float* nls;                 // -lse / scale out, same layout as lse
  const int32_t* offsets; const int32_t* slot_ptr; const int32_t* tiles;
  uint16_t* dq;               // jagged: bf16 dQ
  float* dq_part;             // broadcast: [groups][Lq][H][D] float32 partials
  int32_t H, lq, total_kv, num_seqs, groups;
  float c, scale;
  int32_t window;             // causal sliding window (WIN kernels)
  jfa::RopeTab rope;          // rotary kernels only
  const int32_t* sp_base; const int32_t* sp_ptr; const int32_t* sp_ent;  // SPARSE kernels
};

// S^T = K Q^T and dP^T - Di = V dO^T - Di for one step of BN keys (lane = query
// row): the first dP product takes `ndi` (every element -Di of the lane's row)
// as its accumulator input, so dS = P * dP' needs no subtraction.
template <int D>
__device__ __forceinline__ void dq_scores(uint32_t ks, const LaneOffsets<D>& lo,
                                          const u32x4 (&qf)[DqCfg<D>::DS],
                                          const u32x4 (&dof)[DqCfg<D>::DS], const f32x16& ndi,
                                          f32x16 (&s)[DqCfg<D>::KB], f32x16 (&dp)[DqCfg<D>::KB]) {
  using C = DqCfg<D>;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) s[kb] = f32x16{};
  // row fragments are read one k-step ahead of their MFMAs; the K and V
  // fragments of one k-step share their address (the V tile follows the K tile
  // at a fixed distance, an immediate offset), one add per k-step
  u32x4 ka[2][C::KB], va[2][C::KB];
  auto read = [&](int d, int bf) {
    const uint32_t a = ks + lo.row[d];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      ka[bf][kb] = lds_ld16(a + uint32_t(kb * 32 * D * 2));
      va[bf][kb] = lds_ld16(a + uint32_t(C::TILE * 2 + kb * 32 * D * 2));
    }
  };
  read(0, 0);
#pragma unroll
  for (int d = 0; d < C::DS; ++d) {
    if (d + 1 < C::DS) read(d + 1, (d + 1) & 1);
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      s[kb] = mfma32(ka[d & 1][kb], qf[d], s[kb]);
      dp[kb] = mfma32(va[d & 1][kb], dof[d], d == 0 ? ndi : dp[kb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// dQ^T += K^T dS^T for one step whose dS is packed with keys along the registers.
template <int D>
__device__ __forceinline__ void dq_accumulate(uint32_t ks, const LaneOffsets<D>& lo,
                                              const u32x4 (&pds)[2 * DqCfg<D>::KB],
                                              f32x16 (&acc)[DqCfg<D>::NB]) {
  using C = DqCfg<D>;
  // one address per column block and half, shared by the step's 16-key groups
  // (whose distance is an immediate offset)
  uint32_t a[C::NB][2];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) {
    a[nb][0] = ks + lo.col[nb][0];
    a[nb][1] = ks + lo.col[nb][1];
  }
#pragma unroll
  for (int x = 0; x < C::NX; ++x) {
    const int st = x / C::NB, nb = x % C::NB;
    const uint32_t off = uint32_t(st * 16 * D * 2);
    const u32x2 lo2 = lds_tr8(a[nb][0] + off), hi2 = lds_tr8(a[nb][1] + off);
    acc[nb] = mfma32(u32x4{lo2[0], lo2[1], hi2[0], hi2[1]}, pds[st], acc[nb]);
  }
}

// P = 2^(S c - lse2) and dS = P dP' (dP' = dP - Di) for one step, packed to bf16 (keys past
// the sequence end or, with CAUSAL, after the lane's query masked; with WIN also
// keys at or before qpos - win). With PREV the dQ products of the previous step
// are issued in the same region so that these VALU instructions run under them.
template <int D, bool MASK, bool CAUSAL, bool PREV, bool WIN = false>
__device__ __forceinline__ void dq_softmax(const f32x16 (&s)[DqCfg<D>::KB],
                                           const f32x16 (&dp)[DqCfg<D>::KB], float lse2,
                                           float c, int g, int key0, int n_keys, int qpos,
                                           u32x4 (&pds)[2 * DqCfg<D>::KB], uint32_t ks_prev,
                                           const LaneOffsets<D>& lo,
                                           const u32x4 (&pds_prev)[2 * DqCfg<D>::KB],
                                           f32x16 (&acc)[DqCfg<D>::NB], int win = 0) {
  using C = DqCfg<D>;
  if (PREV) dq_accumulate<D>(ks_prev, lo, pds_prev, acc);
  // Register r of block kb holds key key0 + 4g + e, e = kb*32 + (r/4)*8 + r%4 (a
  // constant). The key is dead past the sequence end or, with CAUSAL, after the
  // query (e > hi), and with WIN at or before qpos - win (e <= wl).
  const int kbase = key0 + 4 * g;
  const int hi = (CAUSAL ? min(n_keys - 1, qpos) : n_keys - 1) - kbase;
  const int wl = qpos - win - kbase;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0 = exp2_fast(__builtin_fmaf(s[kb][r], c, -lse2));
      float p1 = exp2_fast(__builtin_fmaf(s[kb][r + 1], c, -lse2));
      if (MASK) {
        const int e = kb * 32 + (r / 4) * 8 + (r % 4);
        p0 = (e > hi || (WIN && e <= wl)) ? 0.f : p0;
        p1 = (e + 1 > hi || (WIN && e + 1 <= wl)) ? 0.f : p1;
      }
      pds[kb * 2 + r / 8][(r % 8) / 2] = pack_bf16(p0 * dp[kb][r], p1 * dp[kb][r + 1]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Stream the keys [0, n_keys) of one (sequence, head) past one query tile. Step kt
// reads the rows of stage kt and the columns of stage kt-1 of a four-stage ring,
// so the load issued at step kt (stage kt+2) goes to the buffer of stage kt-2.
// Steps [0, n_lo) (window edge) and [n_free, n_steps) (tail, diagonal) are masked.
// The wave computes steps [0, n_own) only and meets the barriers and issues its
// loads for the rest.
// Stage st of the key stream: keys [st*BN, st*BN + BN) of K and V into ring
// buffer st % NS, through buffer->LDS copies issued by all NW waves (keys at or
// past L arrive as zeros).
template <int D, int NW>
__device__ __forceinline__ void dq_load_stage(uint16_t* lds, const uint16_t* kbase,
                                              const uint16_t* vbase, int64_t rstride, int L, int st,
                                              int w, int lane) {
  using C = DqCfg<D, NW>;
  uint16_t* buf = lds + (st % C::NS) * C::STAGE;
  const int64_t r0 = int64_t(st) * C::BN * rstride;
  const int rowbytes = int(rstride * 2);
  tile_load<D, C::BN, C::NW>(buf, rows_rsrc<D, C::BN>(kbase + r0, rstride, L - st * C::BN), rowbytes,
                             w, lane);
  tile_load<D, C::BN, C::NW>(buf + C::TILE, rows_rsrc<D, C::BN>(vbase + r0, rstride, L - st * C::BN),
                             rowbytes, w, lane);
}

// The first NS - 2 stages of a key stream, issued ahead of dq_stream<..., true>
// so that their latency overlaps the caller's own loads (the query rows).
template <int D, int NW>
__device__ __forceinline__ void dq_stream_issue(uint16_t* lds, const uint16_t* kbase,
                                                const uint16_t* vbase, int64_t rstride, int L,
                                                int n_keys, int w, int lane) {
  using C = DqCfg<D, NW>;
  const int n_steps = ceil_div(n_keys, C::BN);
#pragma unroll
  for (int st = 0; st < C::NS - 2; ++st)
    if (st < n_steps) dq_load_stage<D, NW>(lds, kbase, vbase, rstride, L, st, w, lane);
}

template <int D, bool CAUSAL, bool WIN = false, int NW = DqCfg<D>::NW, bool PRE = false>
__device__ __forceinline__ void dq_stream(uint16_t* lds, const uint16_t* kbase, const uint16_t* vbase,
                                          int64_t rstride, int L, int n_keys, int n_lo, int n_free,
                                          int n_own, int win,
                                          const u32x4 (&qf)[DqCfg<D>::DS],
                                          const u32x4 (&dof)[DqCfg<D>::DS],
                                          f32x16 (&acc)[DqCfg<D>::NB], float lse2, float di,
                                          float c, int w, int lane, int qpos,
                                          const LaneOffsets<D>& lo) {
  using C = DqCfg<D, NW>;
  static_assert(C::NS == 4, "the ring below assumes four stages");
  const int g = lane >> 5;
  const int n_steps = ceil_div(n_keys, C::BN);
  const uint32_t lds0 = lds_addr(lds);
  auto load_stage = [&](int st) {
    dq_load_stage<D, NW>(lds, kbase, vbase, rstride, L, st, w, lane);
  };
  auto ks_of = [&](int st) { return lds0 + uint32_t((st % C::NS) * C::STAGE * 2); };
  auto arrive = [&](int st) {
    if (st + 1 < n_steps) wait_vmem_le<C::LOADS>();
    else wait_vmem();
    __syncthreads();
  };
  if (!PRE) dq_stream_issue<D, NW>(lds, kbase, vbase, rstride, L, n_keys, w, lane);
  if (n_steps > 0) {
    f32x16 s[C::KB], dp[C::KB];
    u32x4 pds[2 * C::KB], pdv[2 * C::KB];
    f32x16 ndi;  // -Di of the lane's row, the first dP product's accumulator input
#pragma unroll
    for (int r = 0; r < 16; ++r) ndi[r] = -di;
    arrive(0);
    if (C::NS - 2 < n_steps) load_stage(C::NS - 2);
    dq_scores<D>(ks_of(0), lo, qf, dof, ndi, s, dp);
    if (n_lo > 0 || n_free == 0)
      dq_softmax<D, true, CAUSAL, false, WIN>(s, dp, lse2, c, g, 0, n_keys, qpos, pds, 0, lo, pdv,
                                              acc, win);
    else
      dq_softmax<D, false, CAUSAL, false, WIN>(s, dp, lse2, c, g, 0, n_keys, qpos, pds, 0, lo, pdv,
                                               acc, win);
    auto step = [&](int kt, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
      for (int x = 0; x < 2 * C::KB; ++x) pdv[x] = pds[x];
      arrive(kt);  // also: every wave is done with stage kt-2
      if (kt + C::NS - 2 < n_steps) load_stage(kt + C::NS - 2);
      const uint32_t ks = ks_of(kt);
      // the MFMA-only phase runs at raised priority: on a shared SIMD it issues
      // ahead of the other wave's softmax
      __builtin_amdgcn_s_setprio(1);
      dq_scores<D>(ks, lo, qf, dof, ndi, s, dp);
      __builtin_amdgcn_s_setprio(0);
      dq_softmax<D, MASK, CAUSAL, true, WIN>(s, dp, lse2, c, g, kt * C::BN, n_keys, qpos, pds,
                                             ks_of(kt - 1), lo, pdv, acc, win);
    };
    int kt = 1;
    if (WIN)
      for (; kt < min(n_lo, n_own); ++kt) step(kt, std::true_type{});
    for (; kt < min(n_free, n_own); ++kt) step(kt, std::false_type{});
    for (; kt < n_own; ++kt) step(kt, std::true_type{});
    dq_accumulate<D>(ks_of(n_own - 1), lo, pds, acc);
    for (; kt < n_steps; ++kt) {  // the steps this wave leaves out
      arrive(kt);
      if (kt + C::NS - 2 < n_steps) load_stage(kt + C::NS - 2);
    }
  }
  __syncthreads();  // the next stream's first loads overwrite the first stages
}

// dO fragments of one query row (zero past the end) and its Di = rowsum(dO * out).
template <int D>
__device__ __forceinline__ float load_do_row(const uint16_t* orow, const uint16_t* dorow, bool ok,
                                             int g, u32x4 (&dof)[DqCfg<D>::DS]) {
  float di = 0.f;
#pragma unroll
  for (int d = 0; d < DqCfg<D>::DS; ++d) {
    dof[d] = ok ? ld16(dorow + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
    const u32x4 of = ok ? ld16(orow + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      di += bf16_lo(dof[d][e2]) * bf16_lo(of[e2]) + bf16_hi(dof[d][e2]) * bf16_hi(of[e2]);
  }
  return pair_sum(di);
}

// Q and dO fragments of one query row (zero past the end) and its Di.
template <int D>
__device__ __forceinline__ float load_row(const uint16_t* qrow, const uint16_t* orow,
                                          const uint16_t* dorow, bool ok, int g,
                                          u32x4 (&qf)[DqCfg<D>::DS], u32x4 (&dof)[DqCfg<D>::DS]) {
  float di = 0.f;
#pragma unroll
  for (int d = 0; d < DqCfg<D>::DS; ++d) {
    qf[d] = ok ? ld16(qrow + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
    dof[d] = ok ? ld16(dorow + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
    const u32x4 of = ok ? ld16(orow + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      di += bf16_lo(dof[d][e2]) * bf16_lo(of[e2]) + bf16_hi(dof[d][e2]) * bf16_hi(of[e2]);
  }
  return pair_sum(di);  // Di = rowsum(dO * out)
}

// SPARSE (block-sparse attention): each wave pair walks the key blocks its own
// query block attends (the entries of the tile's step list that carry its bit),
// every step masked as in the forward.
template <int D, bool CAUSAL, bool ROPE, bool WIN, bool SPARSE = false>
__global__ void __launch_bounds__(DqCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(2)))
dq_kernel(DqParams P) {
  using C = DqCfg<D>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::NS * C::STAGE];
  __shared__ double rope_tab[ROPE ? D / 2 : 1];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5;
  const LaneOffsets<D> lo(lane);
  // the main loop's barriers order this copy before the first epilogue reads it
  if (ROPE && tid < D / 2) rope_tab[tid] = P.rope.rev[tid];
  const int slot = xcd_slot(blockIdx.x, gridDim.x);
  const int t_begin = P.slot_ptr[slot], t_end = P.slot_ptr[slot + 1];
  const int64_t rstride = int64_t(P.H) * D;
  for (int ti = t_begin; ti < t_end; ++ti) {
    const int b = sload(P.tiles + 4 * ti + 0), h = sload(P.tiles + 4 * ti + 1);
    const int t = sload(P.tiles + 4 * ti + 2);
    const int kv0 = sload(P.offsets + b);
    const int L = sload(P.offsets + b + 1) - kv0;
    const int q_first = t * C::BM;
    const int q_rows = min(C::BM, L - q_first);
    // with a sliding window the keys are streamed from ks0, the start of the step
    // holding key q_first - W + 1 (as in the forward), and counted from there
    const int ks0 = WIN ? max(0, q_first - P.window + 1) / C::BN * C::BN : 0;
    const int n_keys = (CAUSAL ? min(L, q_first + q_rows) : L) - ks0;
    int e_first = 0, n_ent = 0;
    if (SPARSE) {
      const int u = sload(P.sp_base + b) + t;
      e_first = sload(P.sp_ptr + u);
      n_ent = sload(P.sp_ptr + u + 1) - e_first;
    }
    const int n_steps = SPARSE ? n_ent * (jfa::kSpBlock / C::BN) : ceil_div(n_keys, C::BN);
    const int lo_edge = WIN ? q_first + C::BM - P.window - ks0 : 0;
    const int n_lo = lo_edge > 0 ? min(n_steps, ceil_div(lo_edge, C::BN)) : 0;
    const int n_free =
        SPARSE ? 0 : max(n_lo, min(n_steps, ((CAUSAL ? q_first : L) - ks0) / C::BN));
    const int qpos = q_first + w * 32 + (lane & 31);
    const bool ok = qpos < L;
    // steps this wave computes: all, or one when the tile has no row for it
    // (nothing of it is stored)
    const int n_own = w * 32 < q_rows ? n_steps : 1;
    const int64_t row = int64_t(kv0) + qpos;
    const int64_t eoff = row * rstride + int64_t(h) * D;
    const uint16_t* kbase = P.k + (int64_t(kv0) + ks0) * rstride + int64_t(h) * D;
    const uint16_t* vbase = P.v + (int64_t(kv0) + ks0) * rstride + int64_t(h) * D;
    // SPARSE: the wave pair pr = w / 2 holds query block 2t + pr and walks only
    // the key blocks that block attends, SPB steps each, on ring stages 2pr and
    // 2pr + 1 (loaded by the pair's two waves); the pairs meet at every step's
    // barrier
    constexpr int SPB = jfa::kSpBlock / C::BN;
    const int pr = w >> 1;
    int n_all = 0, n_mine = 0, blk = 0;
    BlockWalk walk{P.sp_ent + e_first, n_ent, jfa::kSpBit + pr, lane, 0, 0, 0};
    auto load_pair = [&](int st, int key) {
      uint16_t* buf = lds + (2 * pr + (st & 1)) * C::STAGE;
      const int64_t r0 = int64_t(key) * rstride;
      const int rowbytes = int(rstride * 2);
      tile_load<D, C::BN, 2>(buf, rows_rsrc<D, C::BN>(kbase + r0, rstride, L - key), rowbytes, w & 1,
                             lane);
      tile_load<D, C::BN, 2>(buf + C::TILE, rows_rsrc<D, C::BN>(vbase + r0, rstride, L - key),
                             rowbytes, w & 1, lane);
    };
    if (SPARSE) {
      const int n0 = count_bit(P.sp_ent + e_first, n_ent, jfa::kSpBit, lane) * SPB;
      const int n1 = count_bit(P.sp_ent + e_first, n_ent, jfa::kSpBit + 1, lane) * SPB;
      n_all = max(n0, n1);
      n_mine = pr ? n1 : n0;
      walk.load(0);
      if (n_mine > 0) {
        blk = walk.next();
        load_pair(0, blk * jfa::kSpBlock);
      }
    } else {
      // the first key stages are in flight while the query rows load
      dq_stream_issue<D, C::NW>(lds, kbase, vbase, rstride, L - ks0, n_keys, w, lane);
    }
    u32x4 qf[C::DS], dof[C::DS];
    const float di = load_row<D>(P.q + eoff, P.o + eoff, P.dout + eoff, ok, g, qf, dof);
    const int64_t vidx = int64_t(h) * P.total_kv + row;
    const float lse = ok ? P.lse[vidx] : 0.f;
    const float lse2 = lse * kLog2e;
    if (ok && g == 0) {
      P.di[vidx] = -di;
      P.nls[vidx] = -lse / P.scale;
    }
    f32x16 acc[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) acc[nb] = f32x16{};
    if (SPARSE) {
      // a step: wait for the pair's stage, barrier (every wave is done with the
      // previous step, whose stages the next loads reuse), load the pair's next
      // step, then S, dP, dS and the dQ products of this one
      const bool own = w * 32 < q_rows;  // the wave holds rows of the tile
      f32x16 ndi;  // -Di of the lane's row, the first dP product's accumulator input
#pragma unroll
      for (int r = 0; r < 16; ++r) ndi[r] = -di;
      const uint32_t lds0 = lds_addr(lds);
      for (int st = 0; st < n_all; ++st) {
        wait_vmem();
        __syncthreads();
        const int key = blk * jfa::kSpBlock + (st % SPB) * C::BN;
        if (st + 1 < n_mine) {
          if ((st + 1) % SPB == 0) blk = walk.next();
          load_pair(st + 1, blk * jfa::kSpBlock + ((st + 1) % SPB) * C::BN);
        }
        if (st < n_mine && own) {
          const uint32_t kst = lds0 + uint32_t((2 * pr + (st & 1)) * C::STAGE * 2);
          f32x16 sc[C::KB], dp[C::KB];
          u32x4 pds[2 * C::KB];
          __builtin_amdgcn_s_setprio(1);
          dq_scores<D>(kst, lo, qf, dof, ndi, sc, dp);
          __builtin_amdgcn_s_setprio(0);
          // masked only where a key can be past the end or after a query (as in
          // the forward)
          if (key + C::BN > L || (CAUSAL && key + C::BN - 1 > q_first + w * 32))
            dq_softmax<D, true, CAUSAL, false>(sc, dp, lse2, P.c, g, key, L, qpos, pds, 0, lo, pds, acc);
          else
            dq_softmax<D, false, CAUSAL, false>(sc, dp, lse2, P.c, g, key, L, qpos, pds, 0, lo, pds, acc);
          dq_accumulate<D>(kst, lo, pds, acc);
        }
      }
      __syncthreads();  // every wave is done with the ring before it stages the rows
    } else {
      dq_stream<D, CAUSAL, WIN, C::NW, true>(lds, kbase, vbase, rstride, L - ks0, n_keys, n_lo,
                                             n_free, n_own, P.window, qf, dof, acc, lse2, di, P.c,
                                             w, lane, qpos - ks0, lo);
    }
    // the key stream ended with a barrier: the ring is free to stage the output rows
    if (ROPE) rope_back_rows<D>(acc, qpos, g, rope_tab);
    const int row0 = q_first + w * 32;
    store_rows<D>(lds + w * 32 * D, acc, P.scale,
                  P.dq + (int64_t(kv0) + row0) * rstride + int64_t(h) * D, rstride, L - row0, lane);
    // the staging tiles lie in ring stages 0 and 1, which the next tile's first
    // loads (issued by every wave) overwrite: no wave may start them before all
    // waves have read their rows back
    __syncthreads();
  }
}

// Waves per broadcast-Q dQ workgroup: four (128 query rows), two workgroups per
// compute unit, so that one workgroup's waits at a sequence boundary (its dO rows,
// then its first key stages) run under the other's products.
constexpr int kBcastDqWaves = 4;

// First b in [0, B] with offsets[b] >= target (offsets non-decreasing, offsets[B]
// >= target): a 64-way search by the whole wave, one round of loads per level.
__device__ __forceinline__ int lower_bound_wave(const int32_t* off, int B, int64_t target, int lane) {
  int lo = 0, hi = B;  // the answer lies in [lo, hi]
  while (lo < hi) {
    const int n = hi - lo;
    const int stride = (n + 63) / 64;
    const int idx = lo + lane * stride;
    const bool ge = idx >= hi || int64_t(off[idx]) >= target;
    const uint64_t m = __builtin_amdgcn_ballot_w64(ge);  // set from the first lane on
    const int first = m ? __builtin_ctzll(m) : 64;
    if (first == 0) {
      hi = lo;
    } else {
      const int before = lo + (first - 1) * stride;  // off[before] < target
      hi = first < 64 ? min(hi, lo + first * stride) : hi;
      lo = before + 1;
    }
  }
  return lo;
}

// Broadcast-Q dQ: workgroup (query tile of BM = 32 NW rows, head, sequence
// group). The waves own 32 dense query rows each and share one key stream; Q is
// loaded once per workgroup, and per sequence the waves load their dO and out
// rows (Di) and lse. The sequences are split into `groups` contiguous groups
// holding about the same number of keys (group g: the sequences whose first key
// lies in [g T / G, (g+1) T / G)), so the workgroups carry similar work; each
// writes one float32 partial of dQ. The query tiles of one (head, group) get
// neighbouring workgroup numbers on one XCD (workgroup w runs on XCD w % 8), so
// they stream the same K and V side by side through one L2.
template <int D, int NW>
__global__ void __launch_bounds__((DqCfg<D, NW>::NT)) __attribute__((amdgpu_waves_per_eu(2)))
dq_bcast_kernel(DqParams P) {
  using C = DqCfg<D, NW>;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::NS * C::STAGE];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5;
  const LaneOffsets<D> lo(lane);
  const int n_qt = ceil_div(P.lq, C::BM);
  const int u = xcd_slot(blockIdx.x, gridDim.x);  // consecutive u share an XCD
  const int t = u % n_qt, h = (u / n_qt) % P.H, grp = u / (n_qt * P.H);
  const int64_t T = P.total_kv;
  const int b0 = uniform(lower_bound_wave(P.offsets, P.num_seqs, int64_t(grp) * T / P.groups, lane));
  const int b1 = grp + 1 == P.groups
                     ? P.num_seqs
                     : uniform(lower_bound_wave(P.offsets, P.num_seqs,
                                                int64_t(grp + 1) * T / P.groups, lane));
  const int64_t rstride = int64_t(P.H) * D;
  const int qpos = t * C::BM + w * 32 + (lane & 31);
  const bool ok = qpos < P.lq;
  u32x4 qf[C::DS];
  {
    const uint16_t* qrow = P.q + int64_t(qpos) * rstride + int64_t(h) * D;
#pragma unroll
    for (int d = 0; d < C::DS; ++d) qf[d] = ok ? ld16(qrow + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
  }
  // waves with no query row compute one step per sequence (nothing of it is kept)
  const bool own = t * C::BM + w * 32 < P.lq;
  f32x16 acc[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb) acc[nb] = f32x16{};
  for (int b = b0; b < b1; ++b) {
    const int kv0 = sload(P.offsets + b);
    const int L = sload(P.offsets + b + 1) - kv0;
    const int64_t oeff = (int64_t(b) * P.lq + qpos) * rstride + int64_t(h) * D;
    const uint16_t* kbase = P.k + int64_t(kv0) * rstride + int64_t(h) * D;
    const uint16_t* vbase = P.v + int64_t(kv0) * rstride + int64_t(h) * D;
    // the sequence's first key stages are in flight while its dO and out rows load
    dq_stream_issue<D, NW>(lds, kbase, vbase, rstride, L, L, w, lane);
    u32x4 dof[C::DS];
    const float di = load_do_row<D>(P.o + oeff, P.dout + oeff, ok, g, dof);
    const int64_t vidx = (int64_t(b) * P.H + h) * P.lq + qpos;
    const float lse = ok ? P.lse[vidx] : 0.f;
    if (ok && g == 0) {
      P.di[vidx] = -di;
      P.nls[vidx] = -lse / P.scale;
    }
    if (L > 0)
      dq_stream<D, false, false, NW, true>(lds, kbase, vbase, rstride, L, L, 0,
                                    L / C::BN, own ? ceil_div(L, C::BN) : 1, 0, qf, dof, acc,
                                    lse * kLog2e, di, P.c, w, lane, qpos, lo);
  }
  if (ok) {
    float* prow = P.dq_part + ((int64_t(grp) * P.lq + qpos) * P.H + h) * D;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<f32x4*>(prow + nb * 32 + q4 * 8 + g * 4) =
            f32x4{acc[nb][q4 * 4 + 0], acc[nb][q4 * 4 + 1], acc[nb][q4 * 4 + 2], acc[nb][q4 * 4 + 3]};
  }
}

// dq = bf16(scale * sum over groups of the partials), groups summed in order.
__global__ void __launch_bounds__(256) dq_reduce_kernel(const float* __restrict__ part,
                                                       uint16_t* __restrict__ dq, int64_t n4,
                                                       int groups, float scale) {
  for (int64_t i = blockIdx.x * int64_t(256) + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256) {
    f32x4 a = reinterpret_cast<const f32x4*>(part)[i];
    for (int gi = 1; gi < groups; ++gi) a += reinterpret_cast<const f32x4*>(part)[gi * n4 + i];
    u32x2 o;
    o[0] = pack_bf16(a[0] * scale, a[1] * scale);
    o[1] = pack_bf16(a[2] * scale, a[3] * scale);
    reinterpret_cast<u32x2*>(dq)[i] = o;
  }
}

// ---------------------------------------------------------------- dK/dV pass
//
// A tile is BN keys of one (sequence, head); it walks the query rows in steps of
// BM. Each 32-key block of the tile belongs to a pair of waves that split the four
// products of a step between them:
//   P wave:  S' = Q K^T - lse/scale, P = 2^(c S'), dV^T += dO^T P;
//   dS wave: dP' = dO V^T - Di, dS = P dP' (P handed over through LDS),
//            dK^T += Q^T dS.
// Each wave holds one 32-key operand (K or V) and one accumulator (dV^T or dK^T),
// which lets two waves share a SIMD. The dS wave works one step behind its
// partner, and the two alternate between MFMA work and VALU work: while the P
// wave runs its products the dS wave forms dS, and while the P wave forms P the
// dS wave runs its products.
template <int D>
struct KvCfg {
  static constexpr int BN = jfa::kBwdBN;  // keys per tile
  static constexpr int NP = BN / 32;      // wave pairs, 32 keys each
  static constexpr int NW = 2 * NP;       // P waves 0..NP-1, dS waves NP..2NP-1
  static constexpr int NT = 64 * NW;
  static constexpr int BM = jfa::kBwdBM;  // query rows per step
  static constexpr int IB = BM / 32;
  static constexpr int NS = 3;            // ring stages
  static constexpr int DS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int NX = 2 * IB * NB;  // dV (or dK) products per step
  static constexpr int PK = 2 * IB;       // packed P (or dS) operands per step
  static constexpr int TILE = BM * D;     // elements of one Q or dO tile
  static constexpr int TB = TILE * 2;     // its bytes
};

struct KvParams {
  const uint16_t* q; const uint16_t* k; const uint16_t* v; const uint16_t* dout;
  const float* nls; const float* di;  // -lse / scale and -Di from the dQ pass
  const int32_t* offsets; const int32_t* slot_ptr; const int32_t* tiles;
  uint16_t* dk; uint16_t* dv;
  int32_t H, lq, total_kv;
  float c, scale;
  int32_t window;     // causal sliding window (WIN kernels)
  jfa::RopeTab rope;  // rotary kernels only
  const int32_t* sp_base; const int32_t* sp_ptr; const int32_t* sp_ent;  // SPARSE kernels
};

typedef __attribute__((address_space(3))) u32x4 lds_u32x4_rw_t;
typedef __attribute__((address_space(3))) const f32x4 lds_f32x4_t;

// Per-lane LDS addresses of one wave of a pair for the current tile. The wave
// reads row fragments of one tensor and column fragments of the other (P wave:
// rows of Q, columns of dO; dS wave: rows of dO, columns of Q); every access to
// ring stage S adds S*TB, a compile-time offset.
template <int D>
struct KvAddr {
  uint32_t row[D / 16];     // row fragments, k-chunk kc, rows 0..31 of stage 0
  uint32_t col[D / 32][2];  // column fragments, column block nb, rows 0..7 / 8..15
  uint32_t xch;             // this lane's slot of the pair's exchange, stage 0
  uint32_t vec;             // this lane's rows of the stage-0 vector
};

// Scores of one step with lane = key: S' = Q K^T - lse/scale (P wave, `op` = K)
// or dP' = dO V^T - Di (dS wave, `op` = V), from ring stage S. The accumulators
// start from the per-row constant the dQ pass left in the stage's vector; row
// fragments are read one k-step ahead of their MFMAs.
template <int D, int S>
__device__ __forceinline__ void kv_scores(const KvAddr<D>& a, const u32x4 (&op)[KvCfg<D>::DS],
                                          f32x16 (&s)[KvCfg<D>::IB]) {
  using C = KvCfg<D>;
#pragma unroll
  for (int ib = 0; ib < C::IB; ++ib)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      // register q4*4 + e holds row ib*32 + q4*8 + 4g + e
      const f32x4 v = *(lds_f32x4_t*)(size_t)(a.vec + uint32_t((S * 2 * C::BM + ib * 32 + q4 * 8) * 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) s[ib][q4 * 4 + e] = v[e];
    }
  u32x4 fr[2][C::IB];
  auto read = [&](int d, int buf) {
#pragma unroll
    for (int ib = 0; ib < C::IB; ++ib)
      fr[buf][ib] = lds_ld16(a.row[d] + uint32_t(S * C::TB + ib * 32 * D * 2));
  };
  read(0, 0);
#pragma unroll
  for (int d = 0; d < C::DS; ++d) {
    if (d + 1 < C::DS) read(d + 1, (d + 1) & 1);
#pragma unroll
    for (int ib = 0; ib < C::IB; ++ib) s[ib] = mfma32(fr[d & 1][ib], op[d], s[ib]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// acc^T += X^T Y for the step in ring stage S: X = dO (P wave: acc = dV, Y = P)
// or Q (dS wave: acc = dK, Y = dS), Y packed with query rows along the registers.
// Column fragments are read two products ahead of their MFMAs.
template <int D, int S>
__device__ __forceinline__ void kv_products(const KvAddr<D>& a, const u32x4 (&y)[KvCfg<D>::PK],
                                            f32x16 (&acc)[KvCfg<D>::NB]) {
  using C = KvCfg<D>;
  constexpr int AH = 2;
  u32x4 f[AH + 1];
  auto read = [&](int x) {
    const int st = x / C::NB, nb = x % C::NB;
    const uint32_t off = uint32_t(S * C::TB + st * 16 * D * 2);
    const u32x2 lo = lds_tr8(a.col[nb][0] + off), hi = lds_tr8(a.col[nb][1] + off);
    f[x % (AH + 1)] = u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
#pragma unroll
  for (int x = 0; x < AH; ++x) read(x);
#pragma unroll
  for (int x = 0; x < C::NX; ++x) {
    if (x + AH < C::NX) read(x + AH);
    acc[x % C::NB] = mfma32(f[x % (AH + 1)], y[x / C::NB], acc[x % C::NB]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// P = 2^(c S') packed to bf16 (keys after the query masked with MASK). Operand st
// element k holds rows (st%2)*8 + 2k, +1 of 32-row block st/2.
template <int D, bool MASK, bool WIN = false>
__device__ __forceinline__ void kv_probs(const f32x16 (&s)[KvCfg<D>::IB], float c, int g, int q0,
                                         int jw, u32x4 (&pk)[KvCfg<D>::PK], int win = 0) {
  using C = KvCfg<D>;
  // Register r of block ib holds query q0 + 4g + e, e = ib*32 + (r/4)*8 + r%4 (a
  // constant). It is masked when the key comes after the query (e < dk) and,
  // with a window, when the query is win or more rows after the key (e >= dw):
  // one compare with a constant per element.
  const int dk = jw - q0 - 4 * g, dw = dk + win;
#pragma unroll
  for (int st = 0; st < C::PK; ++st)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int ib = st / 2, r = (st % 2) * 8 + 2 * k;
      const int e = ib * 32 + (r / 4) * 8 + r % 4;
      float p0 = exp2_fast(s[ib][r] * c), p1 = exp2_fast(s[ib][r + 1] * c);
      if (MASK) {
        p0 = (e < dk || (WIN && e >= dw)) ? 0.f : p0;
        p1 = (e + 1 < dk || (WIN && e + 1 >= dw)) ? 0.f : p1;
      }
      pk[st][k] = pack_bf16(p0, p1);
    }
}

// dS = P dP' packed to bf16, from the partner's packed P (same layout).
template <int D>
__device__ __forceinline__ void kv_dsoft(const f32x16 (&dp)[KvCfg<D>::IB],
                                         const u32x4 (&pp)[KvCfg<D>::PK],
                                         u32x4 (&pk)[KvCfg<D>::PK]) {
  using C = KvCfg<D>;
#pragma unroll
  for (int st = 0; st < C::PK; ++st)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int ib = st / 2, r = (st % 2) * 8 + 2 * k;
      pk[st][k] = pack_bf16(bf16_lo(pp[st][k]) * dp[ib][r], bf16_hi(pp[st][k]) * dp[ib][r + 1]);
    }
}

template <int D, int S>
__device__ __forceinline__ void xch_put(const KvAddr<D>& a, const u32x4 (&pk)[KvCfg<D>::PK]) {
  using C = KvCfg<D>;
#pragma unroll
  for (int x = 0; x < C::PK; ++x)
    *(lds_u32x4_rw_t*)(size_t)(a.xch + uint32_t((S * C::NP * C::PK + x) * 64 * 16)) = pk[x];
}
template <int D, int S>
__device__ __forceinline__ void xch_get(const KvAddr<D>& a, u32x4 (&pp)[KvCfg<D>::PK]) {
  using C = KvCfg<D>;
#pragma unroll
  for (int x = 0; x < C::PK; ++x)
    pp[x] = lds_ld16(a.xch + uint32_t((S * C::NP * C::PK + x) * 64 * 16));
}

// SPARSE (block-sparse attention): a tile's steps are the 64-row query blocks of
// its step list, in ascending order; a pair whose 64-key block a step's query
// block does not attend skips that step's products (its SIMD's matrix core serves
// the other waves meanwhile); a tile whose list is empty stores zeros.
template <int D, bool CAUSAL, bool BCAST, bool ROPE, bool WIN, bool SPARSE = false>
__global__ void __launch_bounds__(KvCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(2)))
dkdv_kernel(KvParams P) {
  using C = KvCfg<D>;
  static_assert(!SPARSE || (C::BM == jfa::kSpBlock && C::BN == 2 * jfa::kSpBlock),
                "a sparse step is one query block and a tile two key blocks");
  static_assert(C::NS == 3, "the ring below loads one stage ahead and unrolls by three");
  // Q ring then dO ring; the output rows are staged over both at the end of a tile
  __shared__ __attribute__((aligned(1024))) uint16_t ring[2 * C::NS * C::TILE];
  __shared__ __attribute__((aligned(16))) float vecs[C::NS][2][C::BM];  // -lse/scale, -Di per stage
  __shared__ u32x4 xch[C::NS][C::NP][C::PK * 64];  // packed P per stage and pair
  __shared__ double rope_tab[ROPE ? D / 2 : 1];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
  // the main loop's barriers order this copy before the first epilogue reads it
  if (ROPE && tid < D / 2) rope_tab[tid] = P.rope.rev[tid];
  const bool pwave = w < C::NP;
  const int kw = pwave ? w : w - C::NP;  // 32-key block of the pair
  const int slot = xcd_slot(blockIdx.x, gridDim.x);
  const int t_begin = P.slot_ptr[slot], t_end = P.slot_ptr[slot + 1];
  const int64_t rstride = int64_t(P.H) * D;
  const int rowbytes = int(rstride * 2);

  // what every wave derives from a tile of the schedule
  struct Entry {  // what the schedule and the offsets give for a tile
    int b, h, kv0, L, key0;
  };
  struct Tile : Entry {
    int e_first;  // SPARSE: the tile's step list starts here (n_steps entries)
    int rows_total, qs_lo, n_steps, n_mask, n_hi;
    const uint16_t* qbase;
    const uint16_t* dobase;
    int64_t voff;
  };
  auto entry_of = [&](int ti) {
    Entry E;
    E.b = sload(P.tiles + 4 * ti + 0);
    E.h = sload(P.tiles + 4 * ti + 1);
    E.key0 = sload(P.tiles + 4 * ti + 2) * C::BN;
    E.kv0 = sload(P.offsets + E.b);
    E.L = sload(P.offsets + E.b + 1) - E.kv0;
    return E;
  };
  auto tile_of = [&](const Entry& E) {
    Tile T;
    static_cast<Entry&>(T) = E;
    T.rows_total = BCAST ? P.lq : T.L;
    T.qbase = BCAST ? P.q + int64_t(T.h) * D : P.q + int64_t(T.kv0) * rstride + int64_t(T.h) * D;
    T.dobase = BCAST ? P.dout + int64_t(T.b) * P.lq * rstride + int64_t(T.h) * D
                     : P.dout + int64_t(T.kv0) * rstride + int64_t(T.h) * D;
    T.voff = BCAST ? (int64_t(T.b) * P.H + T.h) * P.lq : int64_t(T.h) * P.total_kv + T.kv0;
    T.qs_lo = CAUSAL ? T.key0 / C::BM : 0;
    // every tile has at least one step (lq >= 1; a causal tile starts on the
    // diagonal of its own keys); with a sliding window the queries past
    // key0 + BN - 1 + W reach none of the tile's keys
    const int q_end = WIN ? min(T.rows_total, T.key0 + C::BN - 1 + P.window) : T.rows_total;
    T.n_steps = ceil_div(q_end, C::BM) - T.qs_lo;
    // causal steps that reach the diagonal need a mask, and with a window the
    // steps from the one holding query key0 + W on (rows past the end read as
    // zeros and contribute nothing)
    T.n_mask = CAUSAL ? min(T.n_steps, C::BN / C::BM) : 0;
    T.n_hi = WIN ? max(0, (T.key0 + P.window) / C::BM - T.qs_lo) : T.n_steps;
    T.e_first = 0;
    if (SPARSE) {  // the tile's step list (possibly empty)
      const int u = sload(P.sp_base + T.b) + T.key0 / C::BN;
      T.e_first = sload(P.sp_ptr + u);
      T.n_steps = T.n_hi = sload(P.sp_ptr + u + 1) - T.e_first;
    }
    return T;
  };
  // SPARSE: entry st of a tile's step list
  auto sp_entry = [&](const Tile& T, int st) { return sload(P.sp_ent + T.e_first + st); };
  auto load_stage = [&](const Tile& T, int st) {
    const int q_first =
        SPARSE ? (sp_entry(T, st) & jfa::kSpIdx) * jfa::kSpBlock : (T.qs_lo + st) * C::BM;
    const int left = T.rows_total - q_first;
    const int sl = st % C::NS;
    tile_load<D, C::BM, C::NW>(ring + sl * C::TILE,
                               rows_rsrc<D, C::BM>(T.qbase + int64_t(q_first) * rstride, rstride, left),
                               rowbytes, w, lane);
    tile_load<D, C::BM, C::NW>(ring + (C::NS + sl) * C::TILE,
                               rows_rsrc<D, C::BM>(T.dobase + int64_t(q_first) * rstride, rstride, left),
                               rowbytes, w, lane);
    if (w < 2) {
      const float* src = (w == 0 ? P.nls : P.di) + T.voff + q_first;
      vec64_load(vecs[sl][w], vec_rsrc<C::BM>(src, left), lane);
    }
  };

  // One role per wave, each walking all the slot's tiles; both meet the same
  // barriers. Step it: wait for stage it, barrier (every wave is done with step
  // it-1, so the buffers of stage it-2 are free and the P of step it-1 is in
  // LDS); stage it+1 is loaded during the step. The next tile's key operand is
  // loaded once the last scores have read the current one: its 32 rows x 32
  // bytes per load instruction are the tile's costliest accesses for the CU's
  // vector memory path, and issued in the epilogue they queued up behind every
  // wave's stage loads and stores there. With broadcast-Q (EARLY), where a tile
  // has only lq/64 steps and the epilogue is a large share of it, they are
  // issued inside the last step, under its products (dK/dV pass 8% faster on
  // 4-step tiles); otherwise after the step loop, under the tail (a test in
  // every step cost the long self-attention tiles 3-5%; after the loop the
  // causal pass gains 3%). The next tile's first stage is loaded before this
  // tile's output rows are stored, so its latency runs under the stores.
  auto run = [&](auto role) {
    constexpr bool PW = decltype(role)::value;
    constexpr bool EARLY = BCAST;
    const uint16_t* kvsrc = PW ? P.k : P.v;  // the wave's 32-key operand: K or V
    auto load_op = [&](const Entry& T, u32x4 (&op)[C::DS]) {
      const int jw = T.key0 + kw * 32 + li;
      const uint16_t* obase = kvsrc + int64_t(T.kv0) * rstride + int64_t(T.h) * D;
#pragma unroll
      for (int d = 0; d < C::DS; ++d)
        op[d] = jw < T.L ? ld16(obase + int64_t(jw) * rstride + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
    };
    u32x4 op[C::DS];
    Tile T{};
    if (t_begin < t_end) {
      T = tile_of(entry_of(t_begin));
      load_op(T, op);
      if (!SPARSE || T.n_steps > 0) load_stage(T, 0);
    }
    for (int ti = t_begin; ti < t_end; ++ti) {
      // The next tile's schedule entry, read at the start of this one and kept
      // in vector registers (scalar ones are all taken by the steps). Its scalar
      // loads are waited for here: left outstanding into the steps, they would
      // turn every counted wait for the steps' LDS reads into a full wait
      // (scalar loads return out of order on the same counter).
      Entry En{};
      if (ti + 1 < t_end) En = entry_of(ti + 1);
      asm volatile("" : "+v"(En.b), "+v"(En.h), "+v"(En.kv0), "+v"(En.L), "+v"(En.key0));
      const int row0 = T.key0 + kw * 32;
      const int jw = row0 + li;  // this lane's key
      // lane-dependent addresses are derived afresh for each tile (otherwise the
      // compiler computes them once, before the tile loop, and keeps them live)
      int ln = lane;
      asm volatile("" : "+v"(ln));
      KvAddr<D> ad;
      {
        const LaneOffsets<D> lo(ln);
        const uint32_t rows_t = lds_addr(ring) + uint32_t(PW ? 0 : C::NS * C::TB);
        const uint32_t cols_t = lds_addr(ring) + uint32_t(PW ? C::NS * C::TB : 0);
#pragma unroll
        for (int kc = 0; kc < C::DS; ++kc) ad.row[kc] = rows_t + lo.row[kc];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          ad.col[nb][0] = cols_t + lo.col[nb][0];
          ad.col[nb][1] = cols_t + lo.col[nb][1];
        }
        ad.xch = lds_addr(xch) + uint32_t((kw * C::PK * 64 + ln) * 16);
        ad.vec = lds_addr(vecs) + uint32_t((PW ? 0 : C::BM) * 4 + (ln >> 5) * 16);
        // Keep each tensor's ring offset inside these registers. Left visible,
        // the compiler moves it into the immediate of every read, and for the
        // dO ring's later stages (48 KB + stage offset) that immediate no
        // longer fits the 16-bit field, so each read gets an add of its own.
#pragma unroll
        for (int kc = 0; kc < C::DS; ++kc) asm volatile("" : "+v"(ad.row[kc]));
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) asm volatile("" : "+v"(ad.col[nb][0]), "+v"(ad.col[nb][1]));
      }
      f32x16 acc[C::NB];
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) acc[nb] = f32x16{};
      // Take delivery of the key operand here, before the steps. Otherwise the
      // compiler, which cannot see the buffer->LDS copies, places its wait for
      // these loads inside the step loop, where it also drains the copy of the
      // next stage issued just before.
#pragma unroll
      for (int d = 0; d < C::DS; ++d) asm volatile("" ::"v"(op[d]));
      f32x16 s[C::IB];
      u32x4 pk[C::PK];
      // the next tile's key operand (op is dead once the last scores are in);
      // after the slot's last tile En is all zeros, so no lane loads
      auto next_op = [&]() { load_op(En, op); };
      auto step = [&](int it, auto stage) {
        constexpr int S = decltype(stage)::value, SP = (S + C::NS - 1) % C::NS;
        const bool prev = S != 0 || it > 0;
        // the first stage of a tile may still have the previous tile's D/16
        // output stores behind it
        if (S == 0 && it == 0 && ti > t_begin) wait_vmem_le<D / 16>();
        else wait_vmem();
        __syncthreads();
        // each role's MFMA section runs at raised priority, its VALU section at
        // the normal one
        // SPARSE: whether the pair's key block pairs with the query block of this
        // step (cur) and of the previous one (was); the others are skipped
        const bool cur = !SPARSE || ((sp_entry(T, it) >> (jfa::kSpBit + kw / 2)) & 1);
        const bool was = prev && (!SPARSE || ((sp_entry(T, it - 1) >> (jfa::kSpBit + kw / 2)) & 1));
        if (PW) {
          __builtin_amdgcn_s_setprio(1);
          if (cur) kv_scores<D, S>(ad, op, s);
          if (EARLY && it + 1 == T.n_steps) next_op();
          if (was) kv_products<D, SP>(ad, pk, acc);
          __builtin_amdgcn_s_setprio(0);
          // the P waves issue their share of the next stage's loads after their
          // products, the dS waves at the start of the step: the buffer->LDS
          // traffic is spread over the step
          if (it + 1 < T.n_steps) load_stage(T, it + 1);
          const int q0 = SPARSE ? (sp_entry(T, it) & jfa::kSpIdx) * jfa::kSpBlock
                                : (T.qs_lo + it) * C::BM;
          if (cur) {
            if (CAUSAL && (it < T.n_mask || (WIN && it >= T.n_hi)))
              kv_probs<D, true, WIN>(s, P.c, g, q0, jw, pk, P.window);
            else
              kv_probs<D, false>(s, P.c, g, q0, jw, pk);
            xch_put<D, S>(ad, pk);
          }
        } else {
          if (was) {
            u32x4 pp[C::PK];
            xch_get<D, SP>(ad, pp);
            kv_dsoft<D>(s, pp, pk);
          }
          if (it + 1 < T.n_steps) load_stage(T, it + 1);
          __builtin_amdgcn_s_setprio(1);
          if (cur) kv_scores<D, S>(ad, op, s);
          if (EARLY && it + 1 == T.n_steps) next_op();
          if (was) kv_products<D, SP>(ad, pk, acc);
          __builtin_amdgcn_s_setprio(0);
        }
      };
      // the last step's products, once its P is in LDS
      auto tail = [&](auto stage) {
        constexpr int S = decltype(stage)::value;
        __syncthreads();
        // SPARSE: no query block attends the tile's keys (no step): zero dK, dV
        if (SPARSE && (T.n_steps == 0 ||
                       !((sp_entry(T, T.n_steps - 1) >> (jfa::kSpBit + kw / 2)) & 1)))
          return;
        if (PW) {
          kv_products<D, S>(ad, pk, acc);
        } else {
          u32x4 pp[C::PK];
          xch_get<D, S>(ad, pp);
          kv_dsoft<D>(s, pp, pk);
          kv_products<D, S>(ad, pk, acc);
        }
      };
      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, 1>;
      using S2 = std::integral_constant<int, 2>;
      if (row0 >= T.L) {
        // no key of the sequence in this pair's block (last tile of a sequence):
        // the pair only meets the barriers and issues its share of the loads;
        // its zero accumulators are stored range-checked, i.e. not at all
        for (int it = 0; it < T.n_steps; ++it) {
          if (it == 0 && ti > t_begin) wait_vmem_le<D / 16>();
          else wait_vmem();
          __syncthreads();
          if (it + 1 < T.n_steps) load_stage(T, it + 1);
        }
        next_op();
        __syncthreads();  // the tail's barrier
      } else {
        for (int it = 0; it < T.n_steps; it += 3) {
          step(it, S0{});
          if (it + 1 < T.n_steps) step(it + 1, S1{});
          if (it + 2 < T.n_steps) step(it + 2, S2{});
        }
        if (!EARLY) next_op();
        const int last = (T.n_steps - 1) % C::NS;  // -1 (the last branch) with no step
        if (last == 0) tail(S0{});
        else if (last == 1) tail(S1{});
        else tail(S2{});
      }
      __syncthreads();  // every wave is done with the ring and the exchange
      const Tile Tc = T;
      if (ti + 1 < t_end) {
        T = tile_of(Entry{uniform(En.b), uniform(En.h), uniform(En.kv0), uniform(En.L),
                          uniform(En.key0)});
        if (!SPARSE || T.n_steps > 0) load_stage(T, 0);
      }
      // output rows staged in ring stages 1 and 2 (stage 0 is filling); the next
      // tile's first barrier orders these reads before its loads of stage 1. The
      // stores are counted (no other vector memory operation follows them before
      // the next tile's first wait), so that wait need not drain them.
      if (ROPE && !PW) rope_back_rows<D>(acc, row0 + li, g, rope_tab);  // dK of the rotated keys
      uint16_t* stg = ring + ((PW ? 0 : C::NS) + 1 + kw / 2) * C::TILE + (kw % 2) * 32 * D;
      const int64_t e0 = (int64_t(Tc.kv0) + row0) * rstride + int64_t(Tc.h) * D;
      store_rows_counted<D>(stg, acc, PW ? 1.f : P.scale, (PW ? P.dv : P.dk) + e0, rstride,
                            Tc.L - row0, lane);
    }
  };
  if (pwave) run(std::true_type{});
  else run(std::false_type{});
}

int grid_for(int64_t n4) {
  const int64_t g = (n4 + 255) / 256;
  return int(g < 8192 ? (g > 0 ? g : 1) : 8192);
}

template <int D, bool CAUSAL, bool BCAST, bool ROPE, bool WIN, bool SPARSE = false>
jfa_status launch_t(const jfa::BwdLaunch& a) {
  hipStream_t st = static_cast<hipStream_t>(a.stream);
  const float c = a.scale * kLog2e;
  DqParams dp{};
  dp.q = static_cast<const uint16_t*>(a.q);
  dp.k = static_cast<const uint16_t*>(a.k);
  dp.v = static_cast<const uint16_t*>(a.v);
  dp.o = static_cast<const uint16_t*>(a.out);
  dp.dout = static_cast<const uint16_t*>(a.dout);
  dp.lse = a.lse;
  dp.di = a.di;
  dp.nls = a.nls;
  dp.offsets = a.offsets;
  dp.slot_ptr = a.q_slot_ptr;
  dp.tiles = a.q_tiles;
  dp.dq = static_cast<uint16_t*>(a.dq);
  dp.dq_part = a.dq_part;
  dp.H = a.num_heads;
  dp.lq = a.lq;
  dp.total_kv = int32_t(a.total_kv);
  dp.num_seqs = a.num_seqs;
  dp.groups = a.groups;
  dp.c = c;
  dp.scale = a.scale;
  dp.window = a.window;
  dp.sp_base = a.q_sp_base;
  dp.sp_ptr = a.q_sp_ptr;
  dp.sp_ent = a.q_sp_ent;
  if (ROPE) dp.rope = *a.rope;
  const bool run_dq = a.passes & JFA_PASS_DQ, run_kv = a.passes & JFA_PASS_DKDV;
  if (!run_dq) {
  } else if (BCAST) {
    using BC = DqCfg<D, kBcastDqWaves>;
    const int n_qt = (a.lq + BC::BM - 1) / BC::BM;
    hipLaunchKernelGGL((dq_bcast_kernel<D, kBcastDqWaves>), dim3(n_qt * a.num_heads * a.groups),
                       dim3(BC::NT), 0, st, dp);
    const int64_t n4 = int64_t(a.lq) * a.num_heads * D / 4;
    hipLaunchKernelGGL(dq_reduce_kernel, dim3(grid_for(n4)), dim3(256), 0, st, a.dq_part,
                       static_cast<uint16_t*>(a.dq), n4, a.groups, a.scale);
  } else if (a.total_kv > 0) {
    hipLaunchKernelGGL((dq_kernel<D, CAUSAL, ROPE, WIN, SPARSE>), dim3(a.q_num_slots),
                       dim3(DqCfg<D>::NT), 0, st, dp);
  }
  if (run_kv && a.total_kv > 0) {
    KvParams kp{};
    kp.q = dp.q;
    kp.k = dp.k;
    kp.v = dp.v;
    kp.dout = dp.dout;
    kp.nls = a.nls;
    kp.di = a.di;
    kp.offsets = a.offsets;
    kp.slot_ptr = a.kv_slot_ptr;
    kp.tiles = a.kv_tiles;
    kp.dk = static_cast<uint16_t*>(a.dk);
    kp.dv = static_cast<uint16_t*>(a.dv);
    kp.H = a.num_heads;
    kp.lq = a.lq;
    kp.total_kv = int32_t(a.total_kv);
    kp.c = c;
    kp.scale = a.scale;
    kp.window = a.window;
    kp.sp_base = a.kv_sp_base;
    kp.sp_ptr = a.kv_sp_ptr;
    kp.sp_ent = a.kv_sp_ent;
    if (ROPE) kp.rope = *a.rope;
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL, BCAST, ROPE, WIN, SPARSE>), dim3(a.kv_num_slots),
                       dim3(KvCfg<D>::NT), 0, st, kp);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("bwd launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

template <int D, bool CAUSAL, bool BCAST>
int occupancy_kv() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, dkdv_kernel<D, CAUSAL, BCAST, false, false>,
                                                   KvCfg<D>::NT, 0) != hipSuccess)
    return 0;
  return n;
}

}  // namespace

namespace jfa {

template <int D>
jfa_status launch_bwd_d(const BwdLaunch& a) {
  const bool causal = a.flags & JFA_CAUSAL, bq = a.flags & JFA_BROADCAST_Q, rope = a.rope != nullptr,
             win = a.window > 0;
  if (bq) return launch_t<D, false, true, false, false>(a);
  if (a.flags & JFA_BLOCK_SPARSE)
    return causal ? launch_t<D, true, false, false, false, true>(a)
                  : launch_t<D, false, false, false, false, true>(a);
  if (win)  // a window comes with CAUSAL
    return rope ? launch_t<D, true, false, true, true>(a) : launch_t<D, true, false, false, true>(a);
  if (rope)
    return causal ? launch_t<D, true, false, true, false>(a) : launch_t<D, false, false, true, false>(a);
  return causal ? launch_t<D, true, false, false, false>(a) : launch_t<D, false, false, false, false>(a);
}

jfa_status launch_bwd(const BwdLaunch& a) {
  return a.head_dim == 128 ? launch_bwd_d<128>(a) : launch_bwd_d<64>(a);
}

jfa_status bwd_slots_per_cu(int head_dim, uint32_t flags, int* per_cu) {
  const bool causal = flags & JFA_CAUSAL, bq = flags & JFA_BROADCAST_Q;
  int n;
  if (head_dim == 128)
    n = bq ? occupancy_kv<128, false, true>() : causal ? occupancy_kv<128, true, false>() : occupancy_kv<128, false, false>();
  else
    n = bq ? occupancy_kv<64, false, true>() : causal ? occupancy_kv<64, true, false>() : occupancy_kv<64, false, false>();
  if (n <= 0) return fail(JFA_ERR_HIP, "occupancy query failed for the dK/dV kernel");
  *per_cu = n;
  return JFA_OK;
}

}  // namespace jfa
