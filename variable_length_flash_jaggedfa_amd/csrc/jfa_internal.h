// Internal declarations shared by the host-side translation units of libjfa.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/jfa.h"

namespace jfa {

// Tile shapes the kernels are compiled for.
constexpr int kFwdBM = 128;    // query rows per forward tile (4 waves x 32 rows)
constexpr int kFwdBN = 64;     // keys per forward KV step
constexpr int kBwdBN = 128;    // key rows per backward tile (4 waves x 32 keys)
constexpr int kBwdBM = 64;     // query rows per backward query step
constexpr int kBlock = 64;     // block-diagonal group size
constexpr int kXcds = 8;       // accelerator complex dies (separate L2s) on MI355X
// Block-sparse step lists: an entry is the other side's 64-token block index in
// the low bits and, in bits kSpBit and kSpBit + 1, which of the tile's two
// blocks pair with it.
constexpr int kSpBlock = 64;
constexpr int kSpBit = 28;
constexpr int32_t kSpIdx = (1 << kSpBit) - 1;

// thread-local error text
void set_error(const std::string& msg);
jfa_status fail(jfa_status s, const std::string& msg);

// host validation of the problem descriptor (no HIP calls)
jfa_status check_problem(const jfa_problem* p);

// Tokens per diagonal block of a validated problem (0 if not block-diagonal).
inline int block_size(const jfa_problem* p) {
  if (p->flags & JFA_BLOCK_DIAG) return p->block;
  return (p->flags & JFA_BLOCK_DIAG64) ? kBlock : 0;
}
// blocks that one single-tile unit covers (32 or 64 tokens): no schedule, no lse
inline bool unit_blocks(const jfa_problem* p) {
  const int bs = block_size(p);
  return bs > 0 && bs <= kBlock;
}
// blocks run as jagged attention over the blocks (128 or 256 tokens)
inline bool tiled_blocks(const jfa_problem* p) { return block_size(p) > kBlock; }
// bytes of the block offsets of a tiled-block problem (rounded up to 256), else 0
size_t block_offsets_bytes(const jfa_problem* p);

// Rotary angle of one position step, in revolutions: rev[i] = base^(-2i/D) / (2 pi)
// for i < D/2 (the jagged kernels form p * rev[i] in double precision).
struct RopeTab {
  double rev[64];
};
RopeTab rope_table(float base, int head_dim);

// kernel launchers (defined in the .hip files); all arguments already validated
struct FwdLaunch {
  const void* q; const void* k; const void* v;
  const int32_t* offsets; const int32_t* slot_ptr; const int32_t* tiles;
  int32_t num_slots;
  void* out; float* lse;
  int32_t num_seqs, num_heads, head_dim, lq;
  int64_t total_kv;
  float scale;
  uint32_t flags;
  float rope_base;  // ROTARY only
  int32_t window;   // causal sliding window (0: none)
  int32_t block;    // single-tile block kernels: tokens per block (32 or 64)
  // BLOCK_SPARSE: the forward step lists (seq_base [B+1], list_ptr, entries)
  const int32_t* sp_base; const int32_t* sp_ptr; const int32_t* sp_ent;
  void* stream;
};

struct BwdLaunch {
  const void* q; const void* k; const void* v; const void* out; const void* dout;
  const float* lse;
  const int32_t* offsets;
  const int32_t* q_slot_ptr; const int32_t* q_tiles; int32_t q_num_slots;    // forward tiles
  const int32_t* kv_slot_ptr; const int32_t* kv_tiles; int32_t kv_num_slots; // backward tiles
  void* dq; void* dk; void* dv;
  float* di;        // workspace: -Di, laid out like lse
  float* nls;       // workspace: -lse / scale, laid out like lse
  float* dq_part;   // workspace: broadcast-Q dQ partials [groups][Lq][H][D]
  int32_t groups;   // broadcast-Q sequence groups
  int32_t num_seqs, num_heads, head_dim, lq;
  int64_t total_kv;
  float scale;
  uint32_t flags;
  float rope_base;  // ROTARY only
  int32_t window;   // causal sliding window (0: none)
  int32_t block;    // single-tile block kernels: tokens per block (32 or 64)
  uint32_t passes;  // JFA_PASS_* mask
  const RopeTab* rope;  // jagged ROTARY: q and k are the rotated copies, dq and dk
                        // are turned back in the epilogues; otherwise NULL
  // BLOCK_SPARSE: the step lists of the query tiles (dQ pass) and of the key
  // tiles (dK/dV pass): seq_base [B+1], list_ptr, entries
  const int32_t* q_sp_base; const int32_t* q_sp_ptr; const int32_t* q_sp_ent;
  const int32_t* kv_sp_base; const int32_t* kv_sp_ptr; const int32_t* kv_sp_ent;
  void* stream;
};

// Rotary pre-pass of the jagged path: q, k [T,H,D] -> rotated copies qr, kr,
// walking the tiles of a forward schedule.
struct RopeRowsLaunch {
  const void* q; const void* k; void* qr; void* kr;
  const int32_t* offsets; const int32_t* slot_ptr; const int32_t* tiles;
  int32_t num_slots, num_seqs, num_heads, head_dim;
  int64_t total_kv;
  RopeTab tab;
  void* stream;
};

// broadcast-Q backward: sequences are split into this many contiguous groups
int bcast_groups(int num_seqs);
// bytes of the Di part of the backward workspace (rounded up to 256)
size_t di_bytes(const jfa_problem* p);
// bytes of one rotated [T,H,D] bf16 copy (rounded up to 256); 0 unless jagged ROTARY
size_t rot_bytes(const jfa_problem* p);

jfa_status launch_fwd(const FwdLaunch& a);
jfa_status launch_bwd(const BwdLaunch& a);
jfa_status launch_block_fwd(const FwdLaunch& a);
jfa_status launch_block_bwd(const BwdLaunch& a);
jfa_status launch_block128_bwd(const BwdLaunch& a);  // whole backward, 128-token blocks, no rotary
jfa_status launch_rope_rows(const RopeRowsLaunch& a);
// offsets of consecutive blocks of `block` tokens: out[i] = i * block, i <= n
jfa_status launch_block_offsets(int32_t* out, int64_t n, int32_t block, void* stream);
jfa_status fwd_slots_per_cu(int head_dim, uint32_t flags, int* per_cu);
jfa_status bwd_slots_per_cu(int head_dim, uint32_t flags, int* per_cu);

}  // namespace jfa
