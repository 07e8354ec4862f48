// C ABI entry points jfa_fwd, jfa_bwd and jfa_default_slots: argument checks on
// the host (nothing is enqueued when a check fails), then kernel launches.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "jfa_internal.h"

using namespace jfa;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

jfa_status need(const void* p, const char* name, uintptr_t align = 16) {
  if (!p) return fail(JFA_ERR_INVALID_ARG, std::string(name) + " is NULL");
  if (!aligned(p, align))
    return fail(JFA_ERR_INVALID_ARG, std::string(name) + " is not " + std::to_string(align) +
                                         "-byte aligned");
  return JFA_OK;
}

// rows of Q / out for the problem (dense Q rows for broadcast-Q)
int64_t q_rows(const jfa_problem* p) {
  return (p->flags & JFA_BROADCAST_Q) ? int64_t(p->lq) : p->total_kv;
}

jfa_status check_schedule_args(const jfa_problem* p, const int32_t* offsets, const int32_t* slot_ptr,
                               const int32_t* tiles, int32_t num_slots) {
  if (jfa_status s = need(offsets, "offsets_dev", 4)) return s;
  if (jfa_status s = need(slot_ptr, "slot_ptr_dev", 4)) return s;
  if (jfa_status s = need(tiles, "tiles_dev", 16)) return s;
  if (num_slots < 1) return fail(JFA_ERR_INVALID_ARG, "num_slots < 1");
  (void)p;
  return JFA_OK;
}

jfa_status check_workspace(void* workspace, size_t workspace_bytes, size_t ws) {
  if (ws == 0) return JFA_OK;
  if (!workspace || workspace_bytes < ws)
    return fail(JFA_ERR_WORKSPACE, "workspace needs " + std::to_string(ws) + " bytes, got " +
                                       std::to_string(workspace_bytes));
  if (!aligned(workspace, 256)) return fail(JFA_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  return JFA_OK;
}

// ---- diagnostics switched on by the environment (read on every call)
//   JFA_VALIDATE=1  before launching, copy the device offsets and schedule back
//                   (a stream synchronisation and blocking copies) and check the
//                   precondition the kernels rely on: under these device offsets
//                   the tiles cover every (sequence, head, tile index) exactly once;
//                   block-sparse step lists are checked against the offsets too.
//   JFA_LOG=1       one line per entry-point call on stderr.
bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v && *v && std::strcmp(v, "0") != 0;
}

void log_call(const char* what, const jfa_problem* p, int32_t slots_a, int32_t slots_b,
              uint32_t passes) {
  if (!env_on("JFA_LOG")) return;
  std::fprintf(stderr,
               "jfa: %s B=%d H=%d D=%d T=%lld lq=%d flags=0x%x window=%d block=%d slots=%d/%d "
               "passes=%u\n",
               what, p->num_seqs, p->num_heads, p->head_dim, (long long)p->total_kv, p->lq,
               p->flags, p->window, p->block, slots_a, slots_b, passes);
}

// Checks one device schedule of `kind` against the device offsets (see above).
// Runs before anything is enqueued, so a failure leaves the stream untouched.
jfa_status validate_schedule(const jfa_problem* p, const int32_t* offsets_dev,
                             const int32_t* slot_ptr_dev, const int32_t* tiles_dev,
                             int32_t num_slots, int32_t kind, void* stream) {
  const char* which = kind == JFA_KIND_FWD ? "forward" : "backward";
  auto bad = [&](const std::string& m) {
    return fail(JFA_ERR_INVALID_ARG, std::string("JFA_VALIDATE: ") + which + " schedule: " + m);
  };
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(JFA_ERR_HIP, "JFA_VALIDATE: stream synchronisation failed");
  const int64_t B = p->num_seqs;
  std::vector<int32_t> off(size_t(B) + 1), sp(size_t(num_slots) + 1);
  if (hipMemcpy(off.data(), offsets_dev, off.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(sp.data(), slot_ptr_dev, sp.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(JFA_ERR_HIP, "JFA_VALIDATE: copy of offsets or slot_ptr failed");
  if (off[0] != 0) return bad("offsets[0] != 0");
  for (int64_t b = 0; b < B; ++b) {
    const int64_t L = int64_t(off[b + 1]) - off[b];
    if (L < 0) return bad("offsets decrease at sequence " + std::to_string(b));
    if (L > p->max_len) return bad("sequence " + std::to_string(b) + " longer than max_len");
    if (block_size(p) > 0 && L % block_size(p))
      return bad("sequence " + std::to_string(b) + " is not a whole number of blocks");
  }
  if (off[B] != p->total_kv) return bad("offsets[B] != total_kv");
  if (sp[0] != 0) return bad("slot_ptr[0] != 0");
  for (int32_t s = 0; s < num_slots; ++s)
    if (sp[s + 1] < sp[s]) return bad("slot_ptr decreases at slot " + std::to_string(s));
  const int64_t n = sp[num_slots];
  std::vector<int32_t> tl(size_t(n) * 4);
  if (n > 0 && hipMemcpy(tl.data(), tiles_dev, tl.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(JFA_ERR_HIP, "JFA_VALIDATE: copy of tiles failed");
  // 128- and 256-token blocks are scheduled over the blocks as sequences
  const bool tb = tiled_blocks(p);
  const int64_t nseq = tb ? p->total_kv / p->block : B;
  const int32_t rows = jfa_tile_rows(kind, p->head_dim, tb ? JFA_BLOCK_DIAG : p->flags);
  const bool dense_q = (p->flags & JFA_BROADCAST_Q) && kind == JFA_KIND_FWD;
  // tiles each (sequence, head) needs under these offsets, as prefix sums
  std::vector<int64_t> first(size_t(nseq) + 1, 0);
  for (int64_t b = 0; b < nseq; ++b) {
    const int64_t L = tb ? p->block : int64_t(off[b + 1]) - off[b];
    first[b + 1] = first[b] + ((dense_q ? p->lq : L) + rows - 1) / rows;
  }
  if (first[nseq] * p->num_heads != n)
    return bad(std::to_string(n) + " tiles where the offsets need " +
               std::to_string(first[nseq] * p->num_heads));
  std::vector<char> seen(size_t(n), 0);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t b = tl[4 * i], h = tl[4 * i + 1], t = tl[4 * i + 2];
    if (b < 0 || b >= nseq || h < 0 || h >= p->num_heads || t < 0)
      return bad("tile " + std::to_string(i) + " names a sequence or head that does not exist");
    const int64_t have = first[b + 1] - first[b];
    if (t >= have)
      return bad("tile " + std::to_string(i) + " (sequence " + std::to_string(b) + ", index " +
                 std::to_string(t) + ") lies past the sequence's rows");
    char& mark = seen[size_t(h * first[nseq] + first[b] + t)];
    if (mark) return bad("tile " + std::to_string(i) + " appears twice");
    mark = 1;
  }
  return JFA_OK;
}

// JFA_VALIDATE for block-sparse step lists of `kind` on the device: copied back
// and checked against the device offsets for what the kernels rely on: seq_base
// holds each sequence's first unit (two 64-token blocks per unit), list_ptr
// starts at 0 and never decreases, and every entry carries one or both block
// bits, no other high bit, a block of its own sequence (and bit kSpBit + 1 only
// where the unit has a second block), ascending within its list.
jfa_status validate_lists(const jfa_problem* p, const int32_t* offsets_dev,
                          const jfa_sparse_lists_dev* sp, int32_t kind, void* stream) {
  const char* which = kind == JFA_KIND_FWD ? "forward" : "backward";
  auto bad = [&](const std::string& m) {
    return fail(JFA_ERR_INVALID_ARG, std::string("JFA_VALIDATE: ") + which + " step lists: " + m);
  };
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess)
    return fail(JFA_ERR_HIP, "JFA_VALIDATE: stream synchronisation failed");
  const int64_t B = p->num_seqs;
  std::vector<int32_t> off(size_t(B) + 1), base(size_t(B) + 1);
  if (hipMemcpy(off.data(), offsets_dev, off.size() * 4, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(base.data(), sp->seq_base, base.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(JFA_ERR_HIP, "JFA_VALIDATE: copy of offsets or seq_base failed");
  int64_t units = 0;
  for (int64_t b = 0; b < B; ++b) {
    if (base[b] != units) return bad("seq_base[" + std::to_string(b) + "] is not the sequence's first unit");
    units += (int64_t(off[b + 1]) - off[b] + 2 * kSpBlock - 1) / (2 * kSpBlock);
  }
  if (base[B] != units) return bad("seq_base[B] is not the number of units");
  std::vector<int32_t> lp(size_t(units) + 1);
  if (hipMemcpy(lp.data(), sp->list_ptr, lp.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(JFA_ERR_HIP, "JFA_VALIDATE: copy of list_ptr failed");
  if (lp[0] != 0) return bad("list_ptr[0] != 0");
  // a list names each block of its sequence at most once: bound every list (and
  // so the entries copied below) before reading any entry
  for (int64_t b = 0, u = 0; b < B; ++b) {
    const int64_t nb = (int64_t(off[b + 1]) - off[b] + kSpBlock - 1) / kSpBlock;
    for (int64_t t = 0; t < (nb + 1) / 2; ++t, ++u) {
      if (lp[u + 1] < lp[u]) return bad("list_ptr decreases at unit " + std::to_string(u));
      if (lp[u + 1] - lp[u] > nb)
        return bad("the list of unit " + std::to_string(u) + " is longer than its sequence's blocks");
    }
  }
  std::vector<int32_t> ent(static_cast<size_t>(lp[units]));
  if (!ent.empty() &&
      hipMemcpy(ent.data(), sp->entries, ent.size() * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(JFA_ERR_HIP, "JFA_VALIDATE: copy of entries failed");
  int64_t u = 0;
  for (int64_t b = 0; b < B; ++b) {
    const int64_t nb = (int64_t(off[b + 1]) - off[b] + kSpBlock - 1) / kSpBlock;
    for (int64_t t = 0; t < (nb + 1) / 2; ++t, ++u)
      for (int32_t e = lp[u]; e < lp[u + 1]; ++e) {
        const int32_t x = ent[size_t(e)], blk = x & kSpIdx, bits = (x >> kSpBit) & 3;
        if ((x >> (kSpBit + 2)) != 0 || bits == 0 || blk >= nb || ((bits & 2) && 2 * t + 1 >= nb))
          return bad("entry " + std::to_string(e) + " of unit " + std::to_string(u) +
                     " does not name a block pair of its sequence");
        if (e > lp[u] && blk <= (ent[size_t(e) - 1] & kSpIdx))
          return bad("the list of unit " + std::to_string(u) + " is not ascending");
      }
  }
  return JFA_OK;
}

// ROTARY on the tiled path: rotated copies of q and k into `rot` (two rot_bytes
// regions), walking the forward schedule given over `num_seqs` sequences.
jfa_status rotate_qk(const jfa_problem* p, const void* q, const void* k, char* rot,
                     const int32_t* offsets_dev, int32_t num_seqs, const int32_t* slot_ptr_dev,
                     const int32_t* tiles_dev, int32_t num_slots, void* stream) {
  RopeRowsLaunch r{q, k, rot, rot + rot_bytes(p), offsets_dev, slot_ptr_dev, tiles_dev, num_slots,
                   num_seqs, p->num_heads, p->head_dim, p->total_kv,
                   rope_table(p->rope_base, p->head_dim), stream};
  return launch_rope_rows(r);
}

// 128- and 256-token blocks run as the jagged problem whose sequences are the
// blocks: their offsets go to the head of `ws`, and the launch reads them.
template <typename Launch>
jfa_status as_block_sequences(const jfa_problem* p, char*& ws, Launch& a, void* stream) {
  const int64_t nb = p->total_kv / p->block;
  int32_t* boff = reinterpret_cast<int32_t*>(ws);
  if (jfa_status s = launch_block_offsets(boff, nb, p->block, stream)) return s;
  ws += block_offsets_bytes(p);
  a.offsets = boff;
  a.num_seqs = int32_t(nb);
  a.flags &= ~(JFA_BLOCK_DIAG | JFA_BLOCK_DIAG64);
  return JFA_OK;
}

}  // namespace

extern "C" jfa_status jfa_default_slots(int32_t kind, int32_t head_dim, uint32_t flags,
                                        int32_t device, int32_t* num_slots) {
  set_error("");
  if (!num_slots) return fail(JFA_ERR_INVALID_ARG, "num_slots is NULL");
  if (kind != JFA_KIND_FWD && kind != JFA_KIND_BWD) return fail(JFA_ERR_INVALID_ARG, "bad kind");
  if (head_dim != 64 && head_dim != 128) return fail(JFA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (flags & JFA_BLOCK_DIAG64) return fail(JFA_ERR_UNSUPPORTED, "BLOCK_DIAG64 runs without a schedule");
  int cus = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess || cus <= 0)
    return fail(JFA_ERR_HIP, std::string("device query failed: ") + hipGetErrorString(e));
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return fail(JFA_ERR_HIP, "hipGetDevice failed");
  if (cur != device && hipSetDevice(device) != hipSuccess) return fail(JFA_ERR_HIP, "hipSetDevice failed");
  int per_cu = 0;
  jfa_status s = kind == JFA_KIND_FWD ? fwd_slots_per_cu(head_dim, flags, &per_cu)
                                      : bwd_slots_per_cu(head_dim, flags, &per_cu);
  if (cur != device) (void)hipSetDevice(cur);
  if (s) return s;
  *num_slots = cus * per_cu;
  return JFA_OK;
}

namespace {

// device step lists of a BLOCK_SPARSE problem: present exactly when the flag is
jfa_status check_lists(const jfa_problem* p, const jfa_sparse_lists_dev* sp, const char* which) {
  const bool sparse = p->flags & JFA_BLOCK_SPARSE;
  if (!sparse && sp) return fail(JFA_ERR_INVALID_ARG, std::string(which) + " given without BLOCK_SPARSE");
  if (!sparse) return JFA_OK;
  if (!sp) return fail(JFA_ERR_INVALID_ARG, std::string("BLOCK_SPARSE needs ") + which);
  if (jfa_status s = need(sp->seq_base, "seq_base", 4)) return s;
  if (jfa_status s = need(sp->list_ptr, "list_ptr", 4)) return s;
  return need(sp->entries, "entries", 4);
}

jfa_status fwd_impl(const jfa_problem* p, const void* q, const void* k, const void* v,
                    const int32_t* offsets_dev, const jfa_sparse_lists_dev* sp,
                    const int32_t* slot_ptr_dev, const int32_t* tiles_dev, int32_t num_slots,
                    void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (jfa_status s = check_problem(p)) return s;
  const bool blk = unit_blocks(p);
  if (p->num_seqs == 0 || (q_rows(p) == 0 && p->total_kv == 0)) return JFA_OK;  // nothing to do
  if (q_rows(p) > 0) {
    if (jfa_status s = need(q, "q")) return s;
    if (jfa_status s = need(out, "out")) return s;
  }
  if (p->total_kv > 0) {
    if (jfa_status s = need(k, "k")) return s;
    if (jfa_status s = need(v, "v")) return s;
  }
  if (jfa_status s = check_lists(p, sp, "forward step lists")) return s;
  log_call("fwd", p, num_slots, 0, 0);
  FwdLaunch a{};
  a.q = q; a.k = k; a.v = v;
  a.offsets = offsets_dev; a.slot_ptr = slot_ptr_dev; a.tiles = tiles_dev; a.num_slots = num_slots;
  a.out = out; a.lse = lse;
  a.num_seqs = p->num_seqs; a.num_heads = p->num_heads; a.head_dim = p->head_dim; a.lq = p->lq;
  a.total_kv = p->total_kv; a.scale = p->scale; a.flags = p->flags; a.rope_base = p->rope_base;
  a.window = p->window; a.block = block_size(p);
  if (sp) {
    a.sp_base = sp->seq_base; a.sp_ptr = sp->list_ptr; a.sp_ent = sp->entries;
  }
  a.stream = stream;
  if (blk) {
    if (lse) return fail(JFA_ERR_INVALID_ARG, "lse must be NULL for blocks of 32 or 64 tokens (no lse is stored)");
    if (p->total_kv == 0) return JFA_OK;
    return launch_block_fwd(a);
  }
  if (jfa_status s = need(lse, "lse", 4)) return s;
  if (jfa_status s = check_schedule_args(p, offsets_dev, slot_ptr_dev, tiles_dev, num_slots)) return s;
  if (jfa_status s = check_workspace(workspace, workspace_bytes, jfa_fwd_workspace_bytes(p))) return s;
  if (env_on("JFA_VALIDATE")) {
    if (jfa_status s = validate_schedule(p, offsets_dev, slot_ptr_dev, tiles_dev, num_slots,
                                         JFA_KIND_FWD, stream))
      return s;
    if (sp) {
      if (jfa_status s = validate_lists(p, offsets_dev, sp, JFA_KIND_FWD, stream)) return s;
    }
  }
  char* ws = static_cast<char*>(workspace);
  if (tiled_blocks(p) && p->total_kv > 0) {
    if (jfa_status s = as_block_sequences(p, ws, a, stream)) return s;
  }
  if (rot_bytes(p) > 0 && p->total_kv > 0) {
    if (jfa_status s = rotate_qk(p, q, k, ws, a.offsets, a.num_seqs, slot_ptr_dev, tiles_dev,
                                 num_slots, stream))
      return s;
    a.q = ws;
    a.k = ws + rot_bytes(p);
  }
  return launch_fwd(a);
}

}  // namespace

extern "C" jfa_status jfa_fwd(const jfa_problem* p, const void* q, const void* k, const void* v,
                              const int32_t* offsets_dev, const int32_t* slot_ptr_dev,
                              const int32_t* tiles_dev, int32_t num_slots, void* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream) {
  set_error("");
  return fwd_impl(p, q, k, v, offsets_dev, nullptr, slot_ptr_dev, tiles_dev, num_slots, out, lse,
                  workspace, workspace_bytes, stream);
}

extern "C" jfa_status jfa_fwd_sparse(const jfa_problem* p, const void* q, const void* k,
                                     const void* v, const int32_t* offsets_dev,
                                     const jfa_sparse_lists_dev* lists, const int32_t* slot_ptr_dev,
                                     const int32_t* tiles_dev, int32_t num_slots, void* out,
                                     float* lse, void* stream) {
  set_error("");
  if (!lists) return fail(JFA_ERR_INVALID_ARG, "lists is NULL");
  return fwd_impl(p, q, k, v, offsets_dev, lists, slot_ptr_dev, tiles_dev, num_slots, out, lse,
                  nullptr, 0, stream);
}

namespace {

jfa_status bwd_impl(const jfa_problem* p, const void* q, const void* k, const void* v,
                    const void* out, const void* dout, const float* lse, const int32_t* offsets_dev,
                    const jfa_sparse_lists_dev* q_sp, const int32_t* q_slot_ptr_dev,
                    const int32_t* q_tiles_dev, int32_t q_num_slots,
                    const jfa_sparse_lists_dev* kv_sp, const int32_t* kv_slot_ptr_dev,
                    const int32_t* kv_tiles_dev, int32_t kv_num_slots, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, uint32_t passes, void* stream) {
  if (jfa_status s = check_problem(p)) return s;
  if (passes == 0 || (passes & ~JFA_PASS_ALL))
    return fail(JFA_ERR_INVALID_ARG, "passes must be a non-zero mask of JFA_PASS_DQ | JFA_PASS_DKDV");
  if (unit_blocks(p) && passes != JFA_PASS_ALL)
    return fail(JFA_ERR_INVALID_ARG,
                "blocks of 32 or 64 tokens run one fused backward kernel: passes must be JFA_PASS_ALL");
  const bool blk = unit_blocks(p);
  const bool bq = p->flags & JFA_BROADCAST_Q;
  if (p->num_seqs == 0) return JFA_OK;
  if (q_rows(p) > 0) {
    if (jfa_status s = need(q, "q")) return s;
    if (jfa_status s = need(out, "out")) return s;
    if (jfa_status s = need(dout, "dout")) return s;
    if (jfa_status s = need(dq, "dq")) return s;
  }
  if (p->total_kv > 0) {
    if (jfa_status s = need(k, "k")) return s;
    if (jfa_status s = need(v, "v")) return s;
    if (jfa_status s = need(dk, "dk")) return s;
    if (jfa_status s = need(dv, "dv")) return s;
  }
  if (jfa_status s = check_lists(p, q_sp, "query-tile step lists")) return s;
  if (jfa_status s = check_lists(p, kv_sp, "key-tile step lists")) return s;
  log_call("bwd", p, q_num_slots, kv_num_slots, passes);
  BwdLaunch a{};
  if (q_sp) {
    a.q_sp_base = q_sp->seq_base; a.q_sp_ptr = q_sp->list_ptr; a.q_sp_ent = q_sp->entries;
  }
  if (kv_sp) {
    a.kv_sp_base = kv_sp->seq_base; a.kv_sp_ptr = kv_sp->list_ptr; a.kv_sp_ent = kv_sp->entries;
  }
  a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse;
  a.offsets = offsets_dev;
  a.q_slot_ptr = q_slot_ptr_dev; a.q_tiles = q_tiles_dev; a.q_num_slots = q_num_slots;
  a.kv_slot_ptr = kv_slot_ptr_dev; a.kv_tiles = kv_tiles_dev; a.kv_num_slots = kv_num_slots;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.num_seqs = p->num_seqs; a.num_heads = p->num_heads; a.head_dim = p->head_dim; a.lq = p->lq;
  a.total_kv = p->total_kv; a.scale = p->scale; a.flags = p->flags; a.rope_base = p->rope_base;
  a.window = p->window;
  a.block = block_size(p);
  a.passes = passes;
  a.stream = stream;
  if (blk) {
    if (lse) return fail(JFA_ERR_INVALID_ARG, "lse must be NULL for blocks of 32 or 64 tokens (no lse is read)");
    if (p->total_kv == 0) return JFA_OK;
    return launch_block_bwd(a);
  }
  if (q_rows(p) > 0 && !lse) return fail(JFA_ERR_INVALID_ARG, "lse is NULL");
  if (lse && !aligned(lse, 4)) return fail(JFA_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  if (jfa_status s = check_workspace(workspace, workspace_bytes, jfa_bwd_workspace_bytes(p))) return s;
  if (p->total_kv > 0) {
    if (jfa_status s = check_schedule_args(p, offsets_dev, kv_slot_ptr_dev, kv_tiles_dev, kv_num_slots))
      return s;
    if (!bq) {
      if (jfa_status s = check_schedule_args(p, offsets_dev, q_slot_ptr_dev, q_tiles_dev, q_num_slots))
        return s;
    }
  } else if (bq) {
    if (jfa_status s = need(offsets_dev, "offsets_dev", 4)) return s;
  }
  if (q_rows(p) == 0 && p->total_kv == 0) return JFA_OK;
  if (env_on("JFA_VALIDATE") && p->total_kv > 0) {
    if (jfa_status s = validate_schedule(p, offsets_dev, kv_slot_ptr_dev, kv_tiles_dev,
                                         kv_num_slots, JFA_KIND_BWD, stream))
      return s;
    if (!bq) {
      if (jfa_status s = validate_schedule(p, offsets_dev, q_slot_ptr_dev, q_tiles_dev,
                                           q_num_slots, JFA_KIND_FWD, stream))
        return s;
    }
    if (q_sp) {
      if (jfa_status s = validate_lists(p, offsets_dev, q_sp, JFA_KIND_FWD, stream)) return s;
    }
    if (kv_sp) {
      if (jfa_status s = validate_lists(p, offsets_dev, kv_sp, JFA_KIND_BWD, stream)) return s;
    }
  }
  a.di = static_cast<float*>(workspace);
  a.nls = reinterpret_cast<float*>(static_cast<char*>(workspace) + di_bytes(p));
  a.groups = bcast_groups(p->num_seqs);
  a.dq_part = bq ? reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * di_bytes(p)) : nullptr;
  char* ws = static_cast<char*>(workspace) + 2 * di_bytes(p);  // after -Di and -lse/scale
  // The whole backward of 128-token blocks without rotary is one single-tile
  // kernel (a block is one tile: no lse read, no workspace used); the arguments
  // are checked as for the two passes, which a caller may still run apart.
  if (block_size(p) == 128 && !(p->flags & JFA_ROTARY) && passes == JFA_PASS_ALL &&
      p->total_kv > 0)
    return launch_block128_bwd(a);
  if (tiled_blocks(p) && p->total_kv > 0) {
    if (jfa_status s = as_block_sequences(p, ws, a, stream)) return s;
  }
  RopeTab tab;
  if (rot_bytes(p) > 0 && p->total_kv > 0) {
    // the dQ pass rotates q and k into the workspace; the dK/dV pass reads the
    // copies it left there
    char* rot = ws;
    if (passes & JFA_PASS_DQ) {
      if (jfa_status s = rotate_qk(p, q, k, rot, a.offsets, a.num_seqs, q_slot_ptr_dev, q_tiles_dev,
                                   q_num_slots, stream))
        return s;
    }
    tab = rope_table(p->rope_base, p->head_dim);
    a.q = rot;
    a.k = rot + rot_bytes(p);
    a.rope = &tab;
  }
  return launch_bwd(a);
}

}  // namespace

extern "C" jfa_status jfa_bwd_passes(const jfa_problem* p, const void* q, const void* k,
                                     const void* v, const void* out, const void* dout,
                                     const float* lse, const int32_t* offsets_dev,
                                     const int32_t* q_slot_ptr_dev, const int32_t* q_tiles_dev,
                                     int32_t q_num_slots, const int32_t* kv_slot_ptr_dev,
                                     const int32_t* kv_tiles_dev, int32_t kv_num_slots, void* dq,
                                     void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                     uint32_t passes, void* stream) {
  set_error("");
  return bwd_impl(p, q, k, v, out, dout, lse, offsets_dev, nullptr, q_slot_ptr_dev, q_tiles_dev,
                  q_num_slots, nullptr, kv_slot_ptr_dev, kv_tiles_dev, kv_num_slots, dq, dk, dv,
                  workspace, workspace_bytes, passes, stream);
}

extern "C" jfa_status jfa_bwd_sparse(const jfa_problem* p, const void* q, const void* k,
                                     const void* v, const void* out, const void* dout,
                                     const float* lse, const int32_t* offsets_dev,
                                     const jfa_sparse_lists_dev* q_lists,
                                     const int32_t* q_slot_ptr_dev, const int32_t* q_tiles_dev,
                                     int32_t q_num_slots, const jfa_sparse_lists_dev* kv_lists,
                                     const int32_t* kv_slot_ptr_dev, const int32_t* kv_tiles_dev,
                                     int32_t kv_num_slots, void* dq, void* dk, void* dv,
                                     void* workspace, size_t workspace_bytes, uint32_t passes,
                                     void* stream) {
  set_error("");
  if (!q_lists || !kv_lists) return fail(JFA_ERR_INVALID_ARG, "q_lists or kv_lists is NULL");
  return bwd_impl(p, q, k, v, out, dout, lse, offsets_dev, q_lists, q_slot_ptr_dev, q_tiles_dev,
                  q_num_slots, kv_lists, kv_slot_ptr_dev, kv_tiles_dev, kv_num_slots, dq, dk, dv,
                  workspace, workspace_bytes, passes, stream);
}

extern "C" jfa_status jfa_bwd(const jfa_problem* p, const void* q, const void* k, const void* v,
                              const void* out, const void* dout, const float* lse,
                              const int32_t* offsets_dev, const int32_t* q_slot_ptr_dev,
                              const int32_t* q_tiles_dev, int32_t q_num_slots,
                              const int32_t* kv_slot_ptr_dev, const int32_t* kv_tiles_dev,
                              int32_t kv_num_slots, void* dq, void* dk, void* dv, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return jfa_bwd_passes(p, q, k, v, out, dout, lse, offsets_dev, q_slot_ptr_dev, q_tiles_dev,
                        q_num_slots, kv_slot_ptr_dev, kv_tiles_dev, kv_num_slots, dq, dk, dv,
                        workspace, workspace_bytes, JFA_PASS_ALL, stream);
}
