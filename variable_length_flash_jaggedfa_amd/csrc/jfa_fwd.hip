// Jagged flash attention forward for gfx950 (persistent, MFMA bf16).
//
// One workgroup per persistent slot walks the tiles the host scheduler dealt to
// it ("Jagged Flash Attention for GEM": persistent kernel fed by a zigzag deal of
// KV-work-sorted tiles). A tile is 128 query rows of one (sequence, head); each
// of the 4 waves owns 32 rows and two workgroups share a compute unit, so one
// wave's LDS and memory waits are covered by the other wave on its SIMD (its
// MFMA and VALU work barely overlap: kept lean, not hidden). Keys stream in
// steps of 32 (D = 128) or 64 (D = 64) through a four-stage LDS ring filled by
// direct buffer->LDS loads issued three steps ahead. Per step a
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
#include "jfa_sparse.h"
#include "jfa_tiles.h"

using namespace jfa_dev;

namespace {

template <int D>
struct FwdCfg {
  static constexpr int BM = jfa::kFwdBM;  // 128 query rows per tile
  static constexpr int BN = D == 128 ? 32 : 64;  // keys per step
  static constexpr int KB = BN / 32;      // 32-key blocks per step
  static constexpr int NW = BM / 32;      // waves, 32 query rows each
  static constexpr int NT = 64 * NW;
  static constexpr int NS = 4;            // LDS ring stages
  static constexpr int DS = D / 16;       // MFMA k-steps over the head dim
  static constexpr int NB = D / 32;       // 32-column blocks of the head dim
  static constexpr int NX = 2 * KB * NB;  // P V products per step
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
  int32_t window;  // causal sliding window (WIN kernels)
  const int32_t* sp_base; const int32_t* sp_ptr; const int32_t* sp_ent;  // SPARSE kernels
};

// Scores of one step whose keys fall past the sequence end or, with CAUSAL,
// after the lane's query position (with WIN also at or before qpos - win) are
// set to -inf.
template <int D, bool CAUSAL, bool WIN>
__device__ __forceinline__ void mask_scores(f32x16 (&s)[FwdCfg<D>::KB], int g, int key0, int n_keys,
                                            int qpos, int win) {
#pragma unroll
  for (int kb = 0; kb < FwdCfg<D>::KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + kb * 32 + (r / 4) * 8 + g * 4 + (r % 4);
      const bool dead = key >= n_keys || (CAUSAL && key > qpos) || (WIN && key <= qpos - win);
      s[kb][r] = dead ? -INFINITY : s[kb][r];
    }
}

// Row max of one step's scores (raw, before scaling), per lane pair.
template <int D>
__device__ __forceinline__ float row_max(const f32x16 (&s)[FwdCfg<D>::KB]) {
  float x = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < FwdCfg<D>::KB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) x = fmaxf(x, s[kb][r]);
  return x;
}

// S^T = K Q^T for one step with no other work to overlap (the first step).
template <int D>
__device__ __forceinline__ void scores(const uint16_t* ks, const u32x4 (&qf)[FwdCfg<D>::DS],
                                       f32x16 (&s)[FwdCfg<D>::KB], int li, int g) {
  using C = FwdCfg<D>;
  u32x4 kf[C::KB][C::DS];
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
    for (int d = 0; d < C::DS; ++d) kf[kb][d] = frag_rows<D>(ks, kb * 32, d, li, g);
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
    s[kb] = f32x16{};
#pragma unroll
    for (int d = 0; d < C::DS; ++d) s[kb] = mfma32(kf[kb][d], qf[d], s[kb]);
  }
}

// Move the reference max of each row if the new step's max exceeds it by more
// than the slack, rescaling l and O by the correction factor 2^(m_old - m_new).
template <int D>
__device__ __forceinline__ void update_max(float mx, float& m, float& l,
                                           f32x16 (&o)[FwdCfg<D>::NB]) {
  if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack)) {
    asm volatile("" ::: "memory");  // keep this rare path a branch, not a select
    const float m_new = fmaxf(m, mx);
    const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int nb = 0; nb < FwdCfg<D>::NB; ++nb) o[nb] *= alpha;
  }
}

// One pipelined step for one wave. On entry `sc` holds this step's scores and m
// its (already moved) reference max. The step
//   A: reads this step's V^T fragments and the next step's K fragments from LDS,
//      then issues the next step's S^T = K Q^T MFMAs interleaved with the exp2
//      and bf16 packing of this step's probabilities;
//   B: issues O^T += V^T P^T interleaved with the masking and row max of the
//      next step's scores.
// Returns the next step's scaled row max (or -inf when there is no next step).
template <int D, bool NEXT, bool MASK_NEXT, bool CAUSAL, bool WIN>
__device__ __forceinline__ float fwd_step(const uint16_t* vs, const uint16_t* ks_next,
                                          const u32x4 (&qf)[FwdCfg<D>::DS],
                                          const f32x16 (&sc)[FwdCfg<D>::KB],
                                          f32x16 (&sn)[FwdCfg<D>::KB], f32x16 (&o)[FwdCfg<D>::NB],
                                          float m, float& l, float c, int lane, int key_next,
                                          int n_keys, int qpos, int win) {
  using C = FwdCfg<D>;
  const int g = lane >> 5, li = lane & 31;
  // --- A. The step runs at raised wave priority: of the two waves sharing a
  // SIMD, the one inside its step issues first, the other one's update and
  // barrier wait go underneath.
  __builtin_amdgcn_s_setprio(1);
  u32x4 kf[C::KB][C::DS];
  if (NEXT) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int d = 0; d < C::DS; ++d) kf[kb][d] = frag_rows<D>(ks_next, kb * 32, d, li, g);
  }
  const float m_use = m == -INFINITY ? 0.f : m;
  u32x4 pf[2 * C::KB];
  float rs = 0.f;
#pragma unroll
  for (int kb = 0; kb < C::KB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = exp2_fast(__builtin_fmaf(sc[kb][r], c, -m_use));
      const float p1 = exp2_fast(__builtin_fmaf(sc[kb][r + 1], c, -m_use));
      rs += p0 + p1;
      pf[kb * 2 + r / 8][(r % 8) / 2] = pack_bf16(p0, p1);
    }
  }
  l += rs;
  if (NEXT) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      sn[kb] = f32x16{};
#pragma unroll
      for (int d = 0; d < C::DS; ++d) sn[kb] = mfma32(kf[kb][d], qf[d], sn[kb]);
    }
  }
  // V^T fragments: the first two are read at the end of A, the rest in B, each
  // two MFMAs ahead of its use
  u32x4 vf[C::NX];
#pragma unroll
  for (int x = 0; x < 2; ++x)
    vf[x] = frag_cols<D>(vs, (x / C::NB) * 16, (x % C::NB) * 32, lane);
  if (NEXT) {
    // all K reads first (their latency is paid once), then each MFMA with a
    // share of the VALU work, then the first V reads
    constexpr int NK = C::KB * C::DS;
    __builtin_amdgcn_sched_group_barrier(0x100, NK, 0);
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6 * C::KB, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // --- B
#pragma unroll
  for (int x = 2; x < C::NX; ++x)
    vf[x] = frag_cols<D>(vs, (x / C::NB) * 16, (x % C::NB) * 32, lane);
#pragma unroll
  for (int x = 0; x < C::NX; ++x) o[x % C::NB] = mfma32(vf[x], pf[x / C::NB], o[x % C::NB]);
  float mx = -INFINITY;
  if (NEXT) {
    if (MASK_NEXT) mask_scores<D, CAUSAL, WIN>(sn, g, key_next, n_keys, qpos, win);
    mx = row_max<D>(sn);
  }
#pragma unroll
  for (int i = 0; i < C::NX; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (NEXT) __builtin_amdgcn_sched_group_barrier(0x002, MASK_NEXT ? 6 * C::KB : 2 * C::KB, 0);
    if (i + 2 < C::NX) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  return NEXT ? pair_max(mx) * c : -INFINITY;
}

template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// SPARSE (block-sparse attention over 64-token blocks): instead of the whole
// sequence, each wave pair of a tile walks the key blocks its own query block
// attends (the entries of the tile's step list that carry its bit), in
// ascending order; every step is masked (past the sequence end and, with
// CAUSAL, after the query).
template <int D, bool CAUSAL, bool BCAST, bool WIN, bool SPARSE = false>
__global__ void __launch_bounds__(FwdCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(2)))
fwd_kernel(FwdParams P) {
  using C = FwdCfg<D>;
  static_assert(C::NS == 4, "the waits below assume a four-stage ring");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::NS * C::STAGE];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 5, li = lane & 31;
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
    // With a sliding window the steps start at the step holding key
    // q_first - W + 1, the first key any row of the tile attends; keys, the key
    // count and the query position used by the masks are counted from that
    // step's first key, ks0. The first n_lo steps meet the window's lower edge
    // and are masked like the diagonal ones.
    const int ks0 = WIN ? max(0, q_first - P.window + 1) / C::BN * C::BN : 0;
    const int n_keys = (CAUSAL ? min(L, q_first + q_rows) : L) - ks0;
    // SPARSE: the tile's entries [e_first, e_first + n_ent), SPB steps each
    // (the union of the two query blocks' lists, a bit per block)
    constexpr int SPB = SPARSE ? jfa::kSpBlock / C::BN : 1;
    int e_first = 0, n_ent = 0;
    if (SPARSE) {
      const int u = sload(P.sp_base + b) + t;
      e_first = sload(P.sp_ptr + u);
      n_ent = sload(P.sp_ptr + u + 1) - e_first;
    }
    const int n_steps = ceil_div(n_keys, C::BN);  // dense kernels
    const int lo_edge = WIN ? q_first + C::BM - P.window - ks0 : 0;
    const int n_lo = lo_edge > 0 ? min(n_steps, ceil_div(lo_edge, C::BN)) : 0;
    // steps without a mask: [n_lo, n_free)
    const int n_free = max(n_lo, min(n_steps, ((CAUSAL ? q_first : L) - ks0) / C::BN));
    const int qpos = q_first + w * 32 + li;  // query position of this lane
    const int qm = qpos - ks0;                // the same, counted from key ks0
    // Steps this wave computes: all, or one when the tile has no row for it
    // (last tile of a sequence; nothing of it is stored). A wave that computes
    // fewer still meets the workgroup's barriers and issues its share of every
    // stage's loads. Causal kernels compute every step: stopping causal waves
    // after their own diagonal step saves no time, because the waves of a
    // workgroup move in lock-step and a step lasts as long as its busiest wave.
    const int n_own = CAUSAL || w * 32 < q_rows ? n_steps : 1;
    const uint16_t* kbase = P.k + (int64_t(kv0) + ks0) * rstride + int64_t(h) * D;
    const uint16_t* vbase = P.v + (int64_t(kv0) + ks0) * rstride + int64_t(h) * D;
    const int Lk = L - ks0;
    const int rowbytes = int(rstride * 2);
    // stage st holds keys [st*BN, st*BN + BN): a resource starting at that row,
    // covering the rest of the sequence (keys past the end read as zero)
    auto load_stage = [&](int st) {
      uint16_t* buf = lds + (st % C::NS) * C::STAGE;
      const int key = st * C::BN;
      const int64_t r0 = int64_t(key) * rstride;
      tile_load<D, C::BN, C::NW>(buf, rows_rsrc<D, C::BN>(kbase + r0, rstride, Lk - key), rowbytes, w, lane);
      tile_load<D, C::BN, C::NW>(buf + C::TILE, rows_rsrc<D, C::BN>(vbase + r0, rstride, Lk - key),
                                 rowbytes, w, lane);
    };
    auto stage_ptr = [&](int st) { return lds + (st % C::NS) * C::STAGE; };

    // Q fragments first, then the first three K/V stages (older loads complete first)
    u32x4 qf[C::DS];
    {
      const bool ok = qpos < rows_total;
      const int64_t qrow = BCAST ? int64_t(qpos) : int64_t(kv0) + qpos;
#pragma unroll
      for (int d = 0; d < C::DS; ++d)
        qf[d] = ok ? ld16(P.q + qrow * rstride + int64_t(h) * D + d * 16 + g * 8) : u32x4{0, 0, 0, 0};
    }
    f32x16 o[C::NB];
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) o[nb] = f32x16{};
    float m = -INFINITY, l = 0.f;

    if (SPARSE) {
      // The wave pair p = w / 2 holds query block 2t + p (rows 64p .. 64p + 63 of
      // the tile) and walks only the key blocks that block attends, SPB steps
      // each, on ring stages 2p and 2p + 1; the two pairs meet at every step's
      // barrier. A step: wait for the pair's stage, barrier (every wave is done
      // with the previous step, whose stages the next loads reuse), load the
      // pair's next step, then the scores, mask, row max, probabilities and
      // products of this one.
      const int pr = w >> 1, wp = w & 1;
      const int32_t* ent = P.sp_ent + e_first;
      const int n0 = count_bit(ent, n_ent, jfa::kSpBit, lane) * SPB;
      const int n1 = count_bit(ent, n_ent, jfa::kSpBit + 1, lane) * SPB;
      const int n_all = max(n0, n1), n_mine = pr ? n1 : n0;
      const bool own = CAUSAL || w * 32 < q_rows;  // the wave holds rows of the tile
      BlockWalk walk{ent, n_ent, jfa::kSpBit + pr, lane, 0, 0, 0};
      walk.load(0);
      auto load_pair = [&](int st, int key) {
        uint16_t* buf = lds + (2 * pr + (st & 1)) * C::STAGE;
        const int64_t r0 = int64_t(key) * rstride;
        tile_load<D, C::BN, 2>(buf, rows_rsrc<D, C::BN>(kbase + r0, rstride, Lk - key), rowbytes, wp,
                               lane);
        tile_load<D, C::BN, 2>(buf + C::TILE, rows_rsrc<D, C::BN>(vbase + r0, rstride, Lk - key),
                               rowbytes, wp, lane);
      };
      int blk = n_mine > 0 ? walk.next() : 0;
      if (n_mine > 0) load_pair(0, blk * jfa::kSpBlock);
      for (int st = 0; st < n_all; ++st) {
        wait_vmem();
        __syncthreads();
        const int key = blk * jfa::kSpBlock + (st % SPB) * C::BN;
        if (st + 1 < n_mine) {
          if ((st + 1) % SPB == 0) blk = walk.next();
          load_pair(st + 1, blk * jfa::kSpBlock + ((st + 1) % SPB) * C::BN);
        }
        if (st < n_mine && own) {
          const uint16_t* stage = lds + (2 * pr + (st & 1)) * C::STAGE;
          f32x16 sc[C::KB], sn[C::KB];
          scores<D>(stage, qf, sc, li, g);
          // only the sequence's last block holds keys past its end, and with
          // CAUSAL only a step reaching past the wave's first row holds keys
          // after a query: the other steps need no mask
          if (key + C::BN > L || (CAUSAL && key + C::BN - 1 > q_first + w * 32))
            mask_scores<D, CAUSAL, false>(sc, g, key, L, qm, 0);
          const float mx = pair_max(row_max<D>(sc)) * P.c;
          update_max<D>(mx, m, l, o);
          fwd_step<D, false, false, CAUSAL, false>(stage + C::TILE, nullptr, qf, sc, sn, o, m, l, P.c,
                                                   lane, 0, L, qm, 0);
        }
      }
    } else {
#pragma unroll
      for (int st = 0; st < C::NS - 1; ++st)
        if (st < n_steps) load_stage(st);

      if (n_steps > 0) {
        // first step's scores: wait for stage 0 only
        if (n_steps >= 3) wait_vmem_le<2 * C::LOADS>();
        else if (n_steps == 2) wait_vmem_le<C::LOADS>();
        else wait_vmem();
        __syncthreads();
        f32x16 sc[C::KB], sn[C::KB];
        scores<D>(stage_ptr(0), qf, sc, li, g);
        if (n_lo > 0 || n_free == 0) mask_scores<D, CAUSAL, WIN>(sc, g, 0, n_keys, qm, P.window);
        m = pair_max(row_max<D>(sc)) * P.c;

        // before step kt (kt + 1 < n_steps): stage kt+1 must have landed, stage
        // kt+2 may still be in flight; the barrier also means every wave is done
        // with stage kt-1, whose buffer the load of stage kt+3 reuses
        auto advance = [&](int kt) {
          if (kt + 2 < n_steps) wait_vmem_le<C::LOADS>();
          else wait_vmem();
          __syncthreads();
          if (kt + C::NS - 1 < n_steps) load_stage(kt + C::NS - 1);
        };
        int kt = 0;
        const int n_free_own = CAUSAL ? n_free : min(n_free, n_own);
        if (WIN) {
          for (; kt + 1 < n_lo; ++kt) {  // the next step meets the window's lower edge
            advance(kt);
            const float mx = fwd_step<D, true, true, CAUSAL, WIN>(
                stage_ptr(kt) + C::TILE, stage_ptr(kt + 1), qf, sc, sn, o, m, l, P.c, lane,
                (kt + 1) * C::BN, n_keys, qm, P.window);
            update_max<D>(mx, m, l, o);
#pragma unroll
            for (int kb = 0; kb < C::KB; ++kb) sc[kb] = sn[kb];
          }
        }
        // two unmasked steps per iteration, the score registers swapping roles
        for (; kt + 2 < n_free_own; kt += 2) {
          advance(kt);
          float mx = fwd_step<D, true, false, CAUSAL, WIN>(stage_ptr(kt) + C::TILE, stage_ptr(kt + 1),
                                                     qf, sc, sn, o, m, l, P.c, lane,
                                                     (kt + 1) * C::BN, n_keys, qm, P.window);
          update_max<D>(mx, m, l, o);
          advance(kt + 1);
          mx = fwd_step<D, true, false, CAUSAL, WIN>(stage_ptr(kt + 1) + C::TILE, stage_ptr(kt + 2),
                                               qf, sn, sc, o, m, l, P.c, lane,
                                               (kt + 2) * C::BN, n_keys, qm, P.window);
          update_max<D>(mx, m, l, o);
        }
        for (; kt + 1 < n_free_own; ++kt) {  // the next step needs no mask
          advance(kt);
          const float mx = fwd_step<D, true, false, CAUSAL, WIN>(stage_ptr(kt) + C::TILE, stage_ptr(kt + 1),
                                                           qf, sc, sn, o, m, l, P.c, lane,
                                                           (kt + 1) * C::BN, n_keys, qm, P.window);
          update_max<D>(mx, m, l, o);
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) sc[kb] = sn[kb];
        }
        for (; kt + 1 < (CAUSAL ? n_steps : n_own); ++kt) {  // the next step is the tail or on the diagonal
          advance(kt);
          const float mx = fwd_step<D, true, true, CAUSAL, WIN>(stage_ptr(kt) + C::TILE, stage_ptr(kt + 1),
                                                          qf, sc, sn, o, m, l, P.c, lane,
                                                          (kt + 1) * C::BN, n_keys, qm, P.window);
          update_max<D>(mx, m, l, o);
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) sc[kb] = sn[kb];
        }
        fwd_step<D, false, false, CAUSAL, WIN>(stage_ptr(kt) + C::TILE, nullptr, qf, sc, sn, o, m, l, P.c,
                                          lane, 0, n_keys, qm, P.window);
        if (!CAUSAL)
          for (; kt + 1 < n_steps; ++kt) advance(kt);  // the steps this wave leaves out
      }
    }

    // epilogue: out = O / l (bf16) through the wave's LDS staging tile, lse =
    // (m + log2 l) * ln 2. The barrier makes the ring free for the staging.
    const float lt = pair_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    __syncthreads();
    {
      const int row0 = q_first + w * 32;
      uint16_t* orow0 = BCAST ? P.out + ((int64_t(b) * P.lq + row0) * P.H + h) * D
                              : P.out + (int64_t(kv0) + row0) * rstride + int64_t(h) * D;
      // 1/l belongs to the lane's row: fold it in before staging
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) o[nb] *= inv;
      store_rows<D>(lds + w * 32 * D, o, 1.f, orow0, rstride, rows_total - row0, lane);
    }
    if (qpos < rows_total && g == 0) {
      const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
      if (BCAST)
        P.lse[(int64_t(b) * P.H + h) * P.lq + qpos] = lse;
      else
        P.lse[int64_t(h) * P.total_kv + kv0 + qpos] = lse;
    }
    __syncthreads();  // the next tile's first loads overwrite the first stages
  }
}

template <int D, bool CAUSAL, bool BCAST, bool WIN, bool SPARSE = false>
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
  P.window = a.window;
  P.sp_base = a.sp_base;
  P.sp_ptr = a.sp_ptr;
  P.sp_ent = a.sp_ent;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, BCAST, WIN, SPARSE>), dim3(a.num_slots), dim3(FwdCfg<D>::NT), 0,
                     static_cast<hipStream_t>(a.stream), P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return jfa::fail(JFA_ERR_HIP, std::string("fwd launch: ") + hipGetErrorString(e));
  return JFA_OK;
}

template <int D, bool CAUSAL, bool BCAST>
int occupancy() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_kernel<D, CAUSAL, BCAST, false>,
                                                   FwdCfg<D>::NT, 0) != hipSuccess)
    return 0;
  return n;
}

}  // namespace

namespace jfa {

jfa_status launch_fwd(const FwdLaunch& a) {
  const bool causal = a.flags & JFA_CAUSAL, bq = a.flags & JFA_BROADCAST_Q, win = a.window > 0;
  if (a.flags & JFA_BLOCK_SPARSE) {
    if (a.head_dim == 128)
      return causal ? launch_t<128, true, false, false, true>(a) : launch_t<128, false, false, false, true>(a);
    return causal ? launch_t<64, true, false, false, true>(a) : launch_t<64, false, false, false, true>(a);
  }
  if (a.head_dim == 128) {
    if (bq) return launch_t<128, false, true, false>(a);
    if (win) return launch_t<128, true, false, true>(a);
    return causal ? launch_t<128, true, false, false>(a) : launch_t<128, false, false, false>(a);
  }
  if (bq) return launch_t<64, false, true, false>(a);
  if (win) return launch_t<64, true, false, true>(a);
  return causal ? launch_t<64, true, false, false>(a) : launch_t<64, false, false, false>(a);
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
