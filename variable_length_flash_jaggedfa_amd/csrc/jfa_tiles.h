// LDS tile helpers for the gfx950 kernels: swizzled row-major tiles filled by
// direct global->LDS loads, and the two ways an MFMA fragment is read back.
//
// A tile holds ROWS x D bf16 values row-major with no padding. Each row is D/8
// chunks of 16 bytes; chunk c of row r is stored at position c ^ f(r), with f
// chosen so that both fragment reads below are free of bank conflicts.
//
// Fragment reads (lane = 32*g + li, see jfa_device.h):
//   frag_rows: 8 consecutive columns (chunk 2*kc+g) of row r0+li -- an A or B
//     operand whose 32-index runs down the rows and whose k runs along a row.
//   frag_cols: rows k0..k0+15 of column c0+li, in the order an accumulator tile
//     hands its rows to the next product (row (e/4)*8 + 4*g + e%4 for element e),
//     built from two ds_read_b64_tr_b16. That instruction works on groups of 16
//     lanes: if lane s of a group loads the 4 values X[a + s/4][b + 4*(s%4) .. +3],
//     lane j of the group receives X[a + e][b + j] for e = 0..3.
#pragma once

#include "jfa_device.h"

namespace jfa_dev {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;
typedef __fp16 f16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) f16x4_t lds_f16x4_t;

template <int D>
struct Swz {
  static_assert(D == 64 || D == 128, "rows of 64 or 128 bf16");
  static constexpr int CPR = D / 8;  // 16-byte chunks per row
  // The gfx950 LDS has 64 four-byte banks (256 bytes per cycle). A 16-byte read
  // is served 16 lanes at a time and frag_rows gives those lanes 16 consecutive
  // rows (aligned to 16) and one logical chunk, so the 16 rows must land on 16
  // distinct 16-byte slots mod 256 bytes. A transpose read serves 32 lanes at a
  // time: 4 consecutive rows (aligned to 4) x 4 consecutive chunks (aligned to
  // 4) x 8 bytes, so the 4 rows must put their aligned block of 4 chunks on 4
  // distinct 64-byte quarters mod 256 bytes. f depends on r mod 16 only.
  //   D = 128 (one row per 256 bytes): f = (r1 r0 r3 r2), a bijection on r mod
  //     16, whose bits 2-3 take 4 values over 4 aligned rows.
  //   D = 64 (two rows per 256 bytes, r0 picks the half): f = (r1 r3 r2), a
  //     bijection on the 8 rows of each parity, whose bit 2 differs between
  //     rows r and r+2.
  __device__ static __forceinline__ int f(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
  }
  // element offset of logical chunk c of row r
  __device__ static __forceinline__ int chunk(int r, int c) { return r * D + ((c ^ f(r)) << 3); }
};

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource (four scalar words): base address, stride 0, size in bytes and
// the configuration word for raw dword access. Loads at offsets >= nbytes return
// zeros.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(int32_t(uint32_t(a)));
  r[1] = __builtin_amdgcn_readfirstlane(int32_t(uint32_t(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(nbytes);
  r[3] = 0x00020000;
  return r;
}

// Buffer resource over rows [0, min(nrows, ROWS)) of a bf16 matrix whose rows
// are `rstride` elements apart and D elements wide. ROWS is the tile the caller
// addresses through it: `nrows` may be the rest of a long sequence, whose span
// would not fit the 32-bit size word, while the tile's own span always does
// (the host rejects problems whose ROWS rows of all heads reach 2^31 bytes).
template <int D, int ROWS>
__device__ __forceinline__ i32x4 rows_rsrc(const uint16_t* base, int64_t rstride, int nrows) {
  const int n = nrows < ROWS ? nrows : ROWS;
  return make_rsrc(base, n > 0 ? int((int64_t(n - 1) * rstride + D) * 2) : 0);
}

// Buffer resource over min(n, N) floats (N: the entries the caller addresses).
template <int N>
__device__ __forceinline__ i32x4 vec_rsrc(const float* base, int n) {
  return make_rsrc(base, n > 0 ? (n < N ? n : N) * 4 : 0);
}

// LDS byte address of a pointer into __shared__ memory: the low 32 bits of its
// generic address (the shared aperture keeps the LDS offset there).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(p)));
}

// Direct buffer->LDS copies: lane i of the wave writes its 16 (4) loaded bytes to
// LDS at dst + 16*i (dst + 4*i). They are issued from inline assembly on purpose:
// the compiler orders LDS reads after an LDS-writing load it knows of by waiting
// for every outstanding vector memory operation, which would stall each pipeline
// step on the prefetch it has just issued. Completion is instead awaited
// explicitly by the kernels (s_waitcnt vmcnt, then a workgroup barrier) before a
// stage is read. The LDS base goes in M0 (set by the compiler from the operand).
// The compiler cannot see the vector memory instruction inside the assembly, so
// it does not pad the hazards that instruction has on its scalar operands: the
// descriptor words may have just been written by v_readfirstlane (a VALU write
// of an SGPR needs 5 wait states before a vector memory instruction reads it)
// and M0 by s_mov. s_nop 4 provides those 5 wait states.
__device__ __forceinline__ void dma16(const i32x4& rsrc, void* dst, int voffset) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds_addr(dst))
               : "memory");
}
__device__ __forceinline__ void dma4(const i32x4& rsrc, void* dst, int voffset) {
  asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "{m0}"(lds_addr(dst))
               : "memory");
}

// Fill a ROWS x D tile from the rows [0, ROWS) of `rsrc` with direct buffer->LDS
// 16-byte loads issued by the NW waves of the workgroup (rows the resource does
// not cover arrive as zeros).
template <int D, int ROWS, int NW>
__device__ __forceinline__ void tile_load(uint16_t* lds_tile, const i32x4& rsrc, int rowbytes,
                                          int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int INSTR = ROWS * CPR / 64;  // one instruction moves 64 chunks
  static_assert(INSTR % NW == 0, "tile must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < INSTR / NW; ++i) {
    const int blk = wave * (INSTR / NW) + i;
    const int q = blk * 64 + lane;  // LDS chunk index within the tile
    const int r = q / CPR;
    const int c = (q % CPR) ^ Swz<D>::f(r);
    dma16(rsrc, lds_tile + blk * 512, r * rowbytes + c * 16);
  }
}

// 64 floats (entries [0, 64) of `rsrc`) with direct 4-byte loads by one wave.
__device__ __forceinline__ void vec64_load(float* lds_vec, const i32x4& rsrc, int lane) {
  dma4(rsrc, lds_vec, lane * 4);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Row-major fragment: row r0 + li, columns (2*kc + g)*8 .. +7.
template <int D>
__device__ __forceinline__ u32x4 frag_rows(const uint16_t* tile, int r0, int kc, int li, int g) {
  return ld16(tile + Swz<D>::chunk(r0 + li, 2 * kc + g));
}

__device__ __forceinline__ u32x2 ld_tr(const uint16_t* p) {
  const f16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_f16x4_t*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Column fragment: rows k0 + (e/4)*8 + 4*g + e%4 (e = 0..7) of column c0 + li.
template <int D>
__device__ __forceinline__ u32x4 frag_cols(const uint16_t* tile, int k0, int c0, int lane) {
  const int G = lane >> 4, j = lane & 15, g = lane >> 5;
  const int col = c0 + (G & 1) * 16 + 4 * (j & 3);
  const int r = k0 + g * 4 + (j >> 2);
  const int cc = col >> 3, within = col & 7;
  const u32x2 lo = ld_tr(tile + Swz<D>::chunk(r, cc) + within);
  const u32x2 hi = ld_tr(tile + Swz<D>::chunk(r + 8, cc) + within);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// ---- fragment reads from precomputed per-lane byte offsets
//
// f depends on r mod 16 only, so for blocks that start at a row that is a
// multiple of 16 the swizzled position of a fragment is a per-lane part, the
// same for every such block, plus the block's row offset. The kernels compute
// the lane parts once; every read is then one address add and an immediate.
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4_t;

template <int D>
struct LaneOffsets {
  static constexpr int DS = D / 16, NB = D / 32;
  uint32_t row[DS];     // frag_rows, k-chunk kc, rows 0..31 of a block
  uint32_t col[NB][2];  // frag_cols, column block nb, rows 0..7 and 8..15 of a k-block
  __device__ __forceinline__ explicit LaneOffsets(int lane) {
    const int g = lane >> 5, li = lane & 31;
#pragma unroll
    for (int kc = 0; kc < DS; ++kc) row[kc] = uint32_t(Swz<D>::chunk(li, 2 * kc + g) * 2);
    const int G = lane >> 4, j = lane & 15;
    const int r = g * 4 + (j >> 2);
    const int cin = (G & 1) * 2 + ((j & 3) >> 1), within = 4 * (j & 1);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      col[nb][0] = uint32_t((Swz<D>::chunk(r, nb * 4 + cin) + within) * 2);
      col[nb][1] = uint32_t((Swz<D>::chunk(r + 8, nb * 4 + cin) + within) * 2);
    }
  }
};

__device__ __forceinline__ u32x4 lds_ld16(uint32_t addr) {
  return *(lds_u32x4_t*)(size_t)addr;
}
__device__ __forceinline__ u32x2 lds_tr8(uint32_t addr) {
  const f16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_f16x4_t*)(size_t)addr);
  return __builtin_bit_cast(u32x2, v);
}

// frag_rows of a tile at LDS byte address tb (r0 a multiple of 16).
template <int D>
__device__ __forceinline__ u32x4 rows_at(uint32_t tb, const LaneOffsets<D>& lo, int r0, int kc) {
  return lds_ld16(tb + lo.row[kc] + uint32_t(r0 * D * 2));
}
// frag_cols of a tile at LDS byte address tb (k0 a multiple of 16, c0 of 32).
template <int D>
__device__ __forceinline__ u32x4 cols_at(uint32_t tb, const LaneOffsets<D>& lo, int k0, int c0) {
  const int nb = c0 / 32;
  const u32x2 x = lds_tr8(tb + lo.col[nb][0] + uint32_t(k0 * D * 2));
  const u32x2 y = lds_tr8(tb + lo.col[nb][1] + uint32_t(k0 * D * 2));
  return u32x4{x[0], x[1], y[0], y[1]};
}

// ---- output rows through LDS
//
// The output of one wave is 32 rows x D, one row per lane pair, held as D/32
// transposed 32 x 32 accumulator blocks (lane li has row li; register r is column
// nb*32 + (r/4)*8 + 4g + r%4). Stored straight from the registers, every store
// instruction would touch 16 bytes in each of 32 rows; instead the rows go
// through a wave-private swizzled LDS tile (32 x D bf16) and leave as whole rows,
// 16 bytes per lane. `stage` is the wave's LDS tile (nothing else may use it
// meanwhile), `row0` the global address of the wave's first row, `rstride`
// elements between rows; rows >= nrows are not written.
template <int D>
__device__ __forceinline__ void store_rows(uint16_t* stage, const f32x16 (&a)[D / 32], float mul,
                                           uint16_t* row0, int64_t rstride, int nrows, int lane) {
  // derive the addresses here, not before the caller's main loop (where the
  // compiler would otherwise hoist them and keep them live across it)
  asm volatile("" : "+v"(lane));
  const int g = lane >> 5, li = lane & 31;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 wv;
      wv[0] = pack_bf16(a[nb][q4 * 4 + 0] * mul, a[nb][q4 * 4 + 1] * mul);
      wv[1] = pack_bf16(a[nb][q4 * 4 + 2] * mul, a[nb][q4 * 4 + 3] * mul);
      st8(stage + Swz<D>::chunk(li, nb * 4 + q4) + g * 4, wv);
    }
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per store instruction
  const int c = lane % CPR, r = lane / CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = i * RPI + r;
    const u32x4 v = ld16(stage + Swz<D>::chunk(row, c));
    if (row < nrows) st16(row0 + int64_t(row) * rstride + c * 8, v);
  }
}

// store_rows through buffer stores whose resource covers rows [0, min(nrows, 32)): rows
// past the end fall outside it and are dropped by the hardware, so every wave
// issues exactly D/16 store instructions whatever nrows is (a caller may count
// them in s_waitcnt vmcnt).
template <int D>
__device__ __forceinline__ void store_rows_counted(uint16_t* stage, const f32x16 (&a)[D / 32],
                                                   float mul, uint16_t* row0, int64_t rstride,
                                                   int nrows, int lane) {
  asm volatile("" : "+v"(lane));
  const int g = lane >> 5, li = lane & 31;
#pragma unroll
  for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      u32x2 wv;
      wv[0] = pack_bf16(a[nb][q4 * 4 + 0] * mul, a[nb][q4 * 4 + 1] * mul);
      wv[1] = pack_bf16(a[nb][q4 * 4 + 2] * mul, a[nb][q4 * 4 + 3] * mul);
      st8(stage + Swz<D>::chunk(li, nb * 4 + q4) + g * 4, wv);
    }
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per store instruction
  const int c = lane % CPR, r = lane / CPR;
  // only the wave's 32 rows are addressed: the resource never spans more
  const int nr = nrows < 32 ? nrows : 32;
  const int nbytes = nr > 0 ? int((int64_t(nr - 1) * rstride + D) * 2) : 0;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      row0, (short)0, __builtin_amdgcn_readfirstlane(nbytes), 0x00020000);
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int row = i * RPI + r;
    const u32x4 v = ld16(stage + Swz<D>::chunk(row, c));
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, int(row * rstride * 2) + c * 16, 0, 0);
  }
}
static_assert(32 / (64 / (128 / 8)) == 128 / 16 && 32 / (64 / (64 / 8)) == 64 / 16,
              "store_rows_counted issues D/16 stores");

}  // namespace jfa_dev
