// Host tile scheduler ("Jagged Flash Attention for GEM", GEM-specific
// optimisations): enumerate the tiles of a jagged problem with their KV work,
// sort them by that work in descending order and deal them zigzag over the
// persistent workgroups. Pure host code; no HIP call.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>
#include <queue>
#include <string>
#include <vector>

#include "jfa_internal.h"

namespace jfa {

namespace {
thread_local std::string g_error;
}

void set_error(const std::string& msg) { g_error = msg; }

jfa_status fail(jfa_status s, const std::string& msg) {
  g_error = msg;
  return s;
}

jfa_status check_problem(const jfa_problem* p) {
  if (!p) return fail(JFA_ERR_INVALID_ARG, "problem descriptor is NULL");
  if (p->num_seqs < 0) return fail(JFA_ERR_INVALID_ARG, "num_seqs < 0");
  if (p->num_heads < 1) return fail(JFA_ERR_INVALID_ARG, "num_heads < 1");
  if (p->max_len < 0) return fail(JFA_ERR_INVALID_ARG, "max_len < 0");
  if (p->total_kv < 0) return fail(JFA_ERR_INVALID_ARG, "total_kv < 0");
  if (!(std::isfinite(p->scale) && p->scale > 0.f))
    return fail(JFA_ERR_INVALID_ARG, "scale must be finite and > 0");
  const uint32_t known =
      JFA_CAUSAL | JFA_BROADCAST_Q | JFA_BLOCK_DIAG64 | JFA_ROTARY | JFA_BLOCK_DIAG | JFA_BLOCK_SPARSE;
  if (p->flags & ~known) return fail(JFA_ERR_INVALID_ARG, "unknown flag bits");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(JFA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const bool causal = p->flags & JFA_CAUSAL, bq = p->flags & JFA_BROADCAST_Q,
             blk = p->flags & (JFA_BLOCK_DIAG64 | JFA_BLOCK_DIAG);
  if (causal && bq) return fail(JFA_ERR_UNSUPPORTED, "CAUSAL with BROADCAST_Q");
  if (blk && (causal || bq)) return fail(JFA_ERR_UNSUPPORTED, "block-diagonal with other flags");
  if (p->flags & JFA_BLOCK_SPARSE) {
    if (p->flags & ~(JFA_BLOCK_SPARSE | JFA_CAUSAL))
      return fail(JFA_ERR_UNSUPPORTED, "BLOCK_SPARSE combines with CAUSAL only");
    if (p->window != 0) return fail(JFA_ERR_UNSUPPORTED, "BLOCK_SPARSE with a sliding window");
    if (p->block != kSpBlock) return fail(JFA_ERR_INVALID_ARG, "BLOCK_SPARSE needs block = 64");
  } else if (p->flags & JFA_BLOCK_DIAG) {
    if (p->block != 32 && p->block != 64 && p->block != 128 && p->block != 256)
      return fail(JFA_ERR_UNSUPPORTED, "BLOCK_DIAG needs block 32, 64, 128 or 256");
    if ((p->flags & JFA_BLOCK_DIAG64) && p->block != 64)
      return fail(JFA_ERR_INVALID_ARG, "BLOCK_DIAG64 with a block other than 64");
  } else if ((p->flags & JFA_BLOCK_DIAG64) ? (p->block != 0 && p->block != 64) : p->block != 0) {
    return fail(JFA_ERR_INVALID_ARG, "block must be 0 (or 64 with BLOCK_DIAG64) without BLOCK_DIAG");
  }
  if (p->window < 0) return fail(JFA_ERR_INVALID_ARG, "window < 0");
  if (p->window > 0 && !causal)
    return fail(JFA_ERR_UNSUPPORTED, "a sliding window needs CAUSAL (jagged self-attention)");
  if (p->flags & JFA_ROTARY) {
    if (bq) return fail(JFA_ERR_UNSUPPORTED, "ROTARY with BROADCAST_Q (the dense Q rows have no positions)");
    if (!(std::isfinite(p->rope_base) && p->rope_base > 1.f && p->rope_base <= 1e9f))
      return fail(JFA_ERR_INVALID_ARG, "ROTARY needs rope_base finite and in (1, 1e9]");
  } else if (p->rope_base != 0.f) {
    return fail(JFA_ERR_INVALID_ARG, "rope_base must be 0 without ROTARY");
  }
  if (bq && p->lq < 1) return fail(JFA_ERR_INVALID_ARG, "BROADCAST_Q needs lq >= 1");
  if (!bq && p->lq != 0) return fail(JFA_ERR_INVALID_ARG, "lq must be 0 without BROADCAST_Q");
  if (blk && (p->total_kv % block_size(p)))
    return fail(JFA_ERR_INVALID_ARG, "block-diagonal needs total_kv to be a multiple of the block");
  // element counts must stay addressable with 64-bit offsets and tiles in int32
  const double elems = double(std::max<int64_t>(p->total_kv, p->lq)) * p->num_heads * p->head_dim;
  if (elems > 4.0e15) return fail(JFA_ERR_INVALID_ARG, "problem too large");
  if (bq && double(p->num_seqs) * p->lq * p->num_heads * p->head_dim > 4.0e15)
    return fail(JFA_ERR_INVALID_ARG, "problem too large (broadcast-Q out rows)");
  if (p->total_kv > INT32_MAX) return fail(JFA_ERR_INVALID_ARG, "total_kv exceeds int32");
  // The kernels address one tile of at most 256 rows of one head through a
  // buffer resource whose size and offsets are 32-bit: 256 token rows of all
  // heads (256 * H * D bf16 values) must stay below 2^31 bytes.
  if (int64_t(p->num_heads) * p->head_dim * 2 * 256 >= (int64_t(1) << 31))
    return fail(JFA_ERR_UNSUPPORTED, "num_heads * head_dim too large: 256 token rows of all heads "
                                     "must span less than 2^31 bytes");
  return JFA_OK;
}

namespace {

struct Tile {
  int32_t b, h, t, work;
};

int32_t ceil_div(int64_t a, int64_t b) { return int32_t((a + b - 1) / b); }

jfa_status check_offsets(const jfa_problem* p, const int32_t* off) {
  if (p->num_seqs > 0 && !off) return fail(JFA_ERR_INVALID_ARG, "offsets_host is NULL");
  if (!off) return p->total_kv == 0 ? JFA_OK : fail(JFA_ERR_INVALID_ARG, "offsets_host is NULL");
  if (off[0] != 0) return fail(JFA_ERR_INVALID_ARG, "offsets[0] != 0");
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    const int64_t L = int64_t(off[b + 1]) - off[b];
    if (L < 0) return fail(JFA_ERR_INVALID_ARG, "offsets decrease at sequence " + std::to_string(b));
    if (L > p->max_len)
      return fail(JFA_ERR_INVALID_ARG, "sequence " + std::to_string(b) + " longer than max_len");
    if (block_size(p) > 0 && (L % block_size(p)))
      return fail(JFA_ERR_INVALID_ARG, "block-diagonal: length of sequence " + std::to_string(b) +
                                           " is not a multiple of the block size");
  }
  if (off[p->num_seqs] != p->total_kv) return fail(JFA_ERR_INVALID_ARG, "offsets[B] != total_kv");
  return JFA_OK;
}

// Tiles in generation order (b, then h, then t). With `sp_ptr` and `sp_ent`
// (block-sparse step lists, one list per (b, t) in that order, see sparse_lists)
// a key tile's work is its list's length times the 64 query rows of each entry,
// and a query tile's the 64 keys times the larger number of entries that carry
// one of its two blocks' bits (its two wave pairs walk those side by side).
std::vector<Tile> enumerate(const jfa_problem* p, const int32_t* off, int32_t kind,
                            const int32_t* sp_ptr = nullptr, const int32_t* sp_ent = nullptr) {
  const bool causal = p->flags & JFA_CAUSAL;
  const int32_t lq = (p->flags & JFA_BROADCAST_Q) ? p->lq : 0;
  const int32_t rows = jfa_tile_rows(kind, p->head_dim, p->flags);
  std::vector<Tile> tiles;
  int64_t u0 = 0;  // first (b, t) unit of sequence b
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    const int32_t L = off[b + 1] - off[b];
    if (sp_ptr) {
      const int32_t n = ceil_div(L, rows);
      std::vector<int32_t> work(size_t(n > 0 ? n : 0));
      for (int32_t t = 0; t < n; ++t) {
        const int32_t lo = sp_ptr[u0 + t], hi = sp_ptr[u0 + t + 1];
        int32_t steps = hi - lo;
        if (kind == JFA_KIND_FWD) {
          int32_t c0 = 0, c1 = 0;
          for (int32_t e = lo; e < hi; ++e) {
            c0 += (sp_ent[e] >> kSpBit) & 1;
            c1 += (sp_ent[e] >> (kSpBit + 1)) & 1;
          }
          steps = std::max(c0, c1);
        }
        work[size_t(t)] = steps * kSpBlock;
      }
      for (int32_t h = 0; h < p->num_heads; ++h)
        for (int32_t t = 0; t < n; ++t) tiles.push_back({b, h, t, work[size_t(t)]});
      u0 += n;
      continue;
    }
    for (int32_t h = 0; h < p->num_heads; ++h) {
      if (kind == JFA_KIND_FWD) {
        if (lq) {
          for (int32_t t = 0, n = ceil_div(lq, rows); t < n; ++t) tiles.push_back({b, h, t, L});
        } else {
          for (int32_t t = 0, n = ceil_div(L, rows); t < n; ++t) {
            const int64_t end = int64_t(t + 1) * rows;
            int64_t work = causal ? std::min<int64_t>(L, end) : L;
            // a causal window leaves the keys from t*rows - W + 1 on
            if (p->window > 0) work -= std::max<int64_t>(0, int64_t(t) * rows - p->window + 1);
            tiles.push_back({b, h, t, int32_t(work)});
          }
        }
      } else {
        for (int32_t n = 0, m = ceil_div(L, rows); n < m; ++n) {
          int64_t work = lq ? lq : (causal ? L - n * rows : L);
          // a causal window: the queries from n*rows to (n+1)*rows - 1 + W reach it
          if (p->window > 0)
            work = std::min<int64_t>(L, int64_t(n + 1) * rows - 1 + p->window) - int64_t(n) * rows;
          tiles.push_back({b, h, n, int32_t(work)});
        }
      }
    }
  }
  return tiles;
}

// Indices 0..n-1 ordered by descending key, ties in ascending index (a stable
// sort). Keys are KV work, non-negative and bounded by the longest sequence (or
// Lq), so a counting sort over the key range does it in linear time; a range
// beyond 2^22 falls back to a comparison sort.
std::vector<int32_t> order_by_desc(const std::vector<int32_t>& key) {
  const size_t n = key.size();
  std::vector<int32_t> idx(n);
  int32_t mx = 0;
  for (int32_t k : key) mx = std::max(mx, k);
  if (mx > (1 << 22)) {
    std::iota(idx.begin(), idx.end(), 0);
    std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return key[a] > key[b]; });
    return idx;
  }
  // start[k]: first output position of key k, larger keys first
  std::vector<int64_t> start(size_t(mx) + 2, 0);
  for (int32_t k : key) ++start[size_t(mx - k) + 1];
  for (size_t i = 1; i < start.size(); ++i) start[i] += start[i - 1];
  for (size_t i = 0; i < n; ++i) idx[size_t(start[size_t(mx - key[i])]++)] = int32_t(i);
  return idx;
}

}  // namespace
}  // namespace jfa

using namespace jfa;

extern "C" int32_t jfa_tile_rows(int32_t kind, int32_t head_dim, uint32_t flags) {
  if (head_dim != 64 && head_dim != 128) return -1;
  if (flags & JFA_BLOCK_DIAG64) return kBlock;
  if (kind == JFA_KIND_FWD) return kFwdBM;
  if (kind == JFA_KIND_BWD) return kBwdBN;
  return -1;
}

extern "C" jfa_status jfa_schedule_count(const jfa_problem* p, const int32_t* offsets_host,
                                         int32_t kind, int64_t* num_tiles) {
  set_error("");
  if (jfa_status s = check_problem(p)) return s;
  if (!num_tiles) return fail(JFA_ERR_INVALID_ARG, "num_tiles is NULL");
  if (kind != JFA_KIND_FWD && kind != JFA_KIND_BWD) return fail(JFA_ERR_INVALID_ARG, "bad kind");
  if (jfa_status s = check_offsets(p, offsets_host)) return s;
  if (unit_blocks(p)) {  // (64-token unit, head) pairs; 32-token blocks pair up in a unit
    const int64_t n = ((p->total_kv + kBlock - 1) / kBlock) * p->num_heads;
    if (n > INT32_MAX) return fail(JFA_ERR_INVALID_ARG, "too many tiles");
    *num_tiles = n;
    return JFA_OK;
  }
  if (tiled_blocks(p)) {  // the jagged tiles of the blocks
    const int32_t rows = jfa_tile_rows(kind, p->head_dim, JFA_BLOCK_DIAG);
    const int64_t n = (p->total_kv / p->block) * p->num_heads * ceil_div(p->block, rows);
    if (n > INT32_MAX) return fail(JFA_ERR_INVALID_ARG, "too many tiles");
    *num_tiles = n;
    return JFA_OK;
  }
  const bool lqmode = (p->flags & JFA_BROADCAST_Q) && kind == JFA_KIND_FWD;
  const int32_t rows = jfa_tile_rows(kind, p->head_dim, p->flags);
  int64_t n = 0;
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    const int64_t L = int64_t(offsets_host[b + 1]) - offsets_host[b];
    n += int64_t(p->num_heads) * ceil_div(lqmode ? p->lq : L, rows);
  }
  if (n > INT32_MAX) return fail(JFA_ERR_INVALID_ARG, "too many tiles");
  *num_tiles = n;
  return JFA_OK;
}

namespace {

jfa_status deal(const jfa_problem* p, const std::vector<Tile>& tiles, int32_t order,
                int32_t num_slots, int32_t* slot_ptr, int32_t* tiles_out);

jfa_status check_deal_args(int64_t count, int32_t order, int32_t num_slots, int32_t* slot_ptr,
                           int32_t* tiles_out, int64_t capacity) {
  if (order != JFA_ORDER_INORDER && order != JFA_ORDER_ZIGZAG && order != JFA_ORDER_XCD_ZIGZAG &&
      order != JFA_ORDER_FOLDED_ZIGZAG && order != JFA_ORDER_XCD_INORDER)
    return fail(JFA_ERR_INVALID_ARG, "bad order");
  if (num_slots < 1) return fail(JFA_ERR_INVALID_ARG, "num_slots < 1");
  if (!slot_ptr) return fail(JFA_ERR_INVALID_ARG, "slot_ptr is NULL");
  if (count > 0 && !tiles_out) return fail(JFA_ERR_INVALID_ARG, "tiles is NULL");
  if (capacity < count) return fail(JFA_ERR_INVALID_ARG, "tiles capacity too small");
  return JFA_OK;
}

// Blocks of a sequence of L tokens, and its mask's first byte in the flat array.
int64_t sp_blocks(int64_t L) { return (L + kSpBlock - 1) / kSpBlock; }

jfa_status check_sparse(const jfa_problem* p, const int32_t* off, const uint8_t* mask,
                        int64_t mask_bytes, int32_t kind) {
  if (jfa_status s = check_problem(p)) return s;
  if (!(p->flags & JFA_BLOCK_SPARSE)) return fail(JFA_ERR_INVALID_ARG, "problem is not BLOCK_SPARSE");
  if (kind != JFA_KIND_FWD && kind != JFA_KIND_BWD) return fail(JFA_ERR_INVALID_ARG, "bad kind");
  if (jfa_status s = check_offsets(p, off)) return s;
  int64_t need = 0;
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    const int64_t n = sp_blocks(int64_t(off[b + 1]) - off[b]);
    need += n * n;
  }
  if (mask_bytes != need)
    return fail(JFA_ERR_INVALID_ARG, "mask_bytes is " + std::to_string(mask_bytes) + ", the offsets need " +
                                         std::to_string(need) + " (sum of n_b^2)");
  if (need > 0 && !mask) return fail(JFA_ERR_INVALID_ARG, "mask_host is NULL");
  return JFA_OK;
}

// The step lists of `kind` (see jfa_sparse_lists); with null outputs only counts.
void sparse_lists(const jfa_problem* p, const int32_t* off, const uint8_t* mask, int32_t kind,
                  int32_t* seq_base, int32_t* list_ptr, int32_t* entries, int64_t* n_units,
                  int64_t* n_entries) {
  const int32_t rows = jfa_tile_rows(kind, p->head_dim, p->flags);  // two 64-token blocks
  const bool causal = p->flags & JFA_CAUSAL;  // no key block after the query block
  int64_t u = 0, e = 0, m0 = 0;
  if (list_ptr) list_ptr[0] = 0;
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    const int64_t L = int64_t(off[b + 1]) - off[b], n = sp_blocks(L);
    const uint8_t* mb = mask + m0;
    if (seq_base) seq_base[b] = int32_t(u);
    for (int64_t t = 0, nt = (L + rows - 1) / rows; t < nt; ++t, ++u) {
      const int64_t a0 = 2 * t, a1 = 2 * t + 1;  // the unit's two blocks
      for (int64_t c = 0; c < n; ++c) {
        // FWD: key block c for query blocks a0, a1; BWD: query block c for key blocks a0, a1
        const bool fwd = kind == JFA_KIND_FWD;
        const bool x0 = (fwd ? mb[a0 * n + c] : mb[c * n + a0]) && !(causal && (fwd ? c > a0 : c < a0));
        const bool x1 = a1 < n && (fwd ? mb[a1 * n + c] : mb[c * n + a1]) &&
                        !(causal && (fwd ? c > a1 : c < a1));
        if (!x0 && !x1) continue;
        if (entries) entries[e] = int32_t(c) | (int32_t(x0) << kSpBit) | (int32_t(x1) << (kSpBit + 1));
        ++e;
      }
      if (list_ptr) list_ptr[u + 1] = int32_t(e);
    }
    m0 += n * n;
  }
  if (seq_base) seq_base[p->num_seqs] = int32_t(u);
  *n_units = u;
  *n_entries = e;
}

}  // namespace

extern "C" jfa_status jfa_sparse_lists_count(const jfa_problem* p, const int32_t* offsets_host,
                                             const uint8_t* mask_host, int64_t mask_bytes,
                                             int32_t kind, int64_t* num_units,
                                             int64_t* num_entries) {
  set_error("");
  if (jfa_status s = check_sparse(p, offsets_host, mask_host, mask_bytes, kind)) return s;
  if (!num_units || !num_entries) return fail(JFA_ERR_INVALID_ARG, "num_units or num_entries is NULL");
  sparse_lists(p, offsets_host, mask_host, kind, nullptr, nullptr, nullptr, num_units, num_entries);
  if (*num_entries > INT32_MAX || *num_units > INT32_MAX)
    return fail(JFA_ERR_INVALID_ARG, "too many step-list entries");
  return JFA_OK;
}

extern "C" jfa_status jfa_sparse_lists(const jfa_problem* p, const int32_t* offsets_host,
                                       const uint8_t* mask_host, int64_t mask_bytes, int32_t kind,
                                       int32_t* seq_base, int32_t* list_ptr, int32_t* entries,
                                       int64_t entries_capacity) {
  int64_t nu = 0, ne = 0;
  if (jfa_status s = jfa_sparse_lists_count(p, offsets_host, mask_host, mask_bytes, kind, &nu, &ne))
    return s;
  if (!seq_base || !list_ptr || (ne > 0 && !entries))
    return fail(JFA_ERR_INVALID_ARG, "seq_base, list_ptr or entries is NULL");
  if (entries_capacity < ne) return fail(JFA_ERR_INVALID_ARG, "entries capacity too small");
  sparse_lists(p, offsets_host, mask_host, kind, seq_base, list_ptr, entries, &nu, &ne);
  return JFA_OK;
}

extern "C" jfa_status jfa_schedule_sparse(const jfa_problem* p, const int32_t* offsets_host,
                                          const int32_t* list_ptr_host, const int32_t* entries_host,
                                          int32_t kind, int32_t order, int32_t num_slots,
                                          int32_t* slot_ptr, int32_t* tiles_out, int64_t capacity) {
  set_error("");
  if (jfa_status s = check_problem(p)) return s;
  if (!(p->flags & JFA_BLOCK_SPARSE)) return fail(JFA_ERR_INVALID_ARG, "problem is not BLOCK_SPARSE");
  int64_t count = 0;
  if (jfa_status s = jfa_schedule_count(p, offsets_host, kind, &count)) return s;
  if (jfa_status s = check_deal_args(count, order, num_slots, slot_ptr, tiles_out, capacity)) return s;
  if (!list_ptr_host) return fail(JFA_ERR_INVALID_ARG, "list_ptr_host is NULL");
  // the units (two blocks each) of the offsets: list_ptr_host has one more
  // entry; a list names each block of its sequence at most once
  const int32_t rows = jfa_tile_rows(kind, p->head_dim, p->flags);
  if (list_ptr_host[0] != 0) return fail(JFA_ERR_INVALID_ARG, "list_ptr[0] != 0");
  int64_t units = 0;
  for (int32_t b = 0; b < p->num_seqs; ++b) {
    const int64_t L = int64_t(offsets_host[b + 1]) - offsets_host[b];
    for (int64_t t = 0, n = ceil_div(L, rows); t < n; ++t, ++units) {
      const int64_t len = int64_t(list_ptr_host[units + 1]) - list_ptr_host[units];
      if (len < 0) return fail(JFA_ERR_INVALID_ARG, "list_ptr decreases at unit " + std::to_string(units));
      if (len > sp_blocks(L))
        return fail(JFA_ERR_INVALID_ARG, "the list of unit " + std::to_string(units) +
                                             " is longer than its sequence's blocks");
    }
  }
  if (kind == JFA_KIND_FWD && list_ptr_host[units] > 0 && !entries_host)
    return fail(JFA_ERR_INVALID_ARG, "entries_host is NULL");
  return deal(p, enumerate(p, offsets_host, kind, list_ptr_host, entries_host), order, num_slots,
              slot_ptr, tiles_out);
}

extern "C" jfa_status jfa_schedule(const jfa_problem* p, const int32_t* offsets_host, int32_t kind,
                                   int32_t order, int32_t num_slots, int32_t* slot_ptr,
                                   int32_t* tiles_out, int64_t capacity) {
  int64_t count = 0;
  if (jfa_status s = jfa_schedule_count(p, offsets_host, kind, &count)) return s;
  if (unit_blocks(p))
    return fail(JFA_ERR_UNSUPPORTED, "blocks of 32 or 64 tokens run without a schedule");
  if (p->flags & JFA_BLOCK_SPARSE)
    return fail(JFA_ERR_INVALID_ARG, "BLOCK_SPARSE schedules come from jfa_schedule_sparse");
  if (jfa_status s = check_deal_args(count, order, num_slots, slot_ptr, tiles_out, capacity)) return s;

  // 128- and 256-token blocks: the tiles of the jagged problem whose sequences are
  // the blocks, in order
  jfa_problem pb = *p;
  std::vector<int32_t> boff;
  if (tiled_blocks(p)) {
    const int32_t nb = int32_t(p->total_kv / p->block);
    boff.resize(size_t(nb) + 1);
    for (int32_t i = 0; i <= nb; ++i) boff[i] = i * p->block;
    pb.num_seqs = nb;
    pb.max_len = p->block;
    pb.flags = p->flags & ~(JFA_BLOCK_DIAG | JFA_BLOCK_DIAG64);
    pb.block = 0;
  }
  return deal(p, tiled_blocks(p) ? enumerate(&pb, boff.data(), kind) : enumerate(p, offsets_host, kind),
              order, num_slots, slot_ptr, tiles_out);
}

namespace {

// Deal the tiles (generation order) over the slots by `order` (see jfa_schedule).
jfa_status deal(const jfa_problem* p, const std::vector<Tile>& tiles, int32_t order,
                int32_t num_slots, int32_t* slot_ptr, int32_t* tiles_out) {
  std::vector<int32_t> idx;      // tiles in dealing order
  std::vector<int32_t> slot_of;  // slot of idx[j]
  if (order == JFA_ORDER_XCD_INORDER) {
    // (sequence, head) units in generation order, each to the group of slots
    // (one group per XCD; one group of all slots when their number is not a
    // multiple of 8) with the least work dealt so far, the lower group on ties;
    // the unit's tiles, in order, each to the least-loaded slot of that group,
    // the lower slot on ties.
    const int32_t X = num_slots % kXcds ? 1 : kXcds;
    const int32_t sx = num_slots / X;
    using Load = std::pair<int64_t, int32_t>;  // (work dealt, slot)
    std::vector<std::priority_queue<Load, std::vector<Load>, std::greater<Load>>> free_slot(X);
    for (int32_t x = 0; x < X; ++x)
      for (int32_t i = 0; i < sx; ++i) free_slot[x].push({0, x * sx + i});
    std::vector<int64_t> group_work(X, 0);
    size_t u0 = 0;
    while (u0 < tiles.size()) {
      size_t u1 = u0 + 1;
      while (u1 < tiles.size() && tiles[u1].b == tiles[u0].b && tiles[u1].h == tiles[u0].h) ++u1;
      int32_t x = 0;
      for (int32_t y = 1; y < X; ++y)
        if (group_work[y] < group_work[x]) x = y;
      for (size_t i = u0; i < u1; ++i) {
        const Load l = free_slot[x].top();
        free_slot[x].pop();
        free_slot[x].push({l.first + tiles[i].work, l.second});
        group_work[x] += tiles[i].work;
        idx.push_back(int32_t(i));
        slot_of.push_back(l.second);
      }
      u0 = u1;
    }
  } else if (order == JFA_ORDER_XCD_ZIGZAG) {
    constexpr int32_t X = kXcds;
    if (num_slots % X) return fail(JFA_ERR_INVALID_ARG, "XCD_ZIGZAG needs num_slots % 8 == 0");
    const int32_t sx = num_slots / X;
    // units = (sequence, head) pairs, in generation order, with their total work
    std::vector<int32_t> unit_first, unit_work;
    for (size_t i = 0; i < tiles.size(); ++i) {
      if (i == 0 || tiles[i].b != tiles[i - 1].b || tiles[i].h != tiles[i - 1].h) {
        unit_first.push_back(int32_t(i));
        unit_work.push_back(0);
      }
      unit_work.back() += tiles[i].work;
    }
    unit_first.push_back(int32_t(tiles.size()));
    const int32_t nu = int32_t(unit_work.size());
    const std::vector<int32_t> uorder = order_by_desc(unit_work);
    std::vector<int32_t> group_of(nu);
    for (int32_t j = 0; j < nu; ++j) {
      const int32_t pass = j / X, r = j % X;
      group_of[uorder[j]] = (pass & 1) ? X - 1 - r : r;
    }
    for (int32_t x = 0; x < X; ++x) {
      std::vector<int32_t> g0;  // this group's tiles, generation order
      for (int32_t u = 0; u < nu; ++u)
        if (group_of[u] == x)
          for (int32_t i = unit_first[u]; i < unit_first[u + 1]; ++i) g0.push_back(i);
      std::vector<int32_t> gw(g0.size());
      for (size_t j = 0; j < g0.size(); ++j) gw[j] = tiles[g0[j]].work;
      std::vector<int32_t> gt(g0.size());
      {
        const std::vector<int32_t> o = order_by_desc(gw);
        for (size_t j = 0; j < o.size(); ++j) gt[j] = g0[o[j]];
      }
      for (size_t j = 0; j < gt.size(); ++j) {
        const int64_t pass = int64_t(j) / sx;
        const int32_t r = int32_t(int64_t(j) % sx);
        idx.push_back(gt[j]);
        slot_of.push_back(x * sx + ((pass & 1) ? sx - 1 - r : r));
      }
    }
  } else if (order == JFA_ORDER_FOLDED_ZIGZAG) {
    // items: with CAUSAL, tiles a and n-1-a of one (sequence, head) form one item
    // (the middle tile of an odd count stands alone); otherwise one tile each.
    // Items in generation order of their first tile, stable-sorted by their
    // summed work, descending, and dealt zigzag; an item's tiles go to one slot.
    const bool fold = p->flags & JFA_CAUSAL;
    std::vector<int32_t> item_first, item_tiles, item_work;  // CSR of tile indices
    size_t u0 = 0;
    while (u0 < tiles.size()) {
      size_t u1 = u0 + 1;
      while (u1 < tiles.size() && tiles[u1].b == tiles[u0].b && tiles[u1].h == tiles[u0].h) ++u1;
      const int32_t n = int32_t(u1 - u0);
      if (fold) {
        for (int32_t a = 0; a < n / 2; ++a) {
          item_first.push_back(int32_t(item_tiles.size()));
          item_tiles.push_back(int32_t(u0) + a);
          item_tiles.push_back(int32_t(u0) + n - 1 - a);
          item_work.push_back(tiles[u0 + a].work + tiles[u0 + n - 1 - a].work);
        }
        if (n % 2) {
          item_first.push_back(int32_t(item_tiles.size()));
          item_tiles.push_back(int32_t(u0) + n / 2);
          item_work.push_back(tiles[u0 + n / 2].work);
        }
      } else {
        for (int32_t a = 0; a < n; ++a) {
          item_first.push_back(int32_t(item_tiles.size()));
          item_tiles.push_back(int32_t(u0) + a);
          item_work.push_back(tiles[u0 + a].work);
        }
      }
      u0 = u1;
    }
    const int32_t ni = int32_t(item_work.size());
    item_first.push_back(int32_t(item_tiles.size()));
    const std::vector<int32_t> iorder = order_by_desc(item_work);
    for (int32_t j = 0; j < ni; ++j) {
      const int32_t pass = j / num_slots, r = j % num_slots;
      const int32_t sl = (pass & 1) ? num_slots - 1 - r : r;
      const int32_t it = iorder[j];
      for (int32_t k = item_first[it]; k < item_first[it + 1]; ++k) {
        idx.push_back(item_tiles[k]);
        slot_of.push_back(sl);
      }
    }
  } else {
    // descending work; ties keep generation order
    if (order == JFA_ORDER_ZIGZAG) {
      std::vector<int32_t> w(tiles.size());
      for (size_t j = 0; j < tiles.size(); ++j) w[j] = tiles[j].work;
      idx = order_by_desc(w);
    } else {
      idx.resize(tiles.size());
      std::iota(idx.begin(), idx.end(), 0);
    }
    // deal: sorted position j -> pass j / S, rank r = j % S
    slot_of.resize(idx.size());
    for (size_t j = 0; j < idx.size(); ++j) {
      const int64_t pass = int64_t(j) / num_slots;
      const int32_t r = int32_t(int64_t(j) % num_slots);
      slot_of[j] = (order == JFA_ORDER_ZIGZAG && (pass & 1)) ? num_slots - 1 - r : r;
    }
  }
  std::vector<int32_t> count_of(num_slots, 0);
  for (int32_t sl : slot_of) ++count_of[sl];
  slot_ptr[0] = 0;
  for (int32_t s = 0; s < num_slots; ++s) slot_ptr[s + 1] = slot_ptr[s] + count_of[s];
  std::vector<int32_t> fill(slot_ptr, slot_ptr + num_slots);
  for (size_t j = 0; j < idx.size(); ++j) {
    const Tile& t = tiles[idx[j]];
    int32_t* dst = tiles_out + 4 * int64_t(fill[slot_of[j]]++);
    dst[0] = t.b; dst[1] = t.h; dst[2] = t.t; dst[3] = t.work;
  }
  return JFA_OK;
}

}  // namespace

namespace jfa {

int bcast_groups(int num_seqs) { return num_seqs < 1 ? 1 : (num_seqs < 128 ? num_seqs : 128); }

size_t di_bytes(const jfa_problem* p) {
  const int64_t n = (p->flags & JFA_BROADCAST_Q) ? int64_t(p->num_seqs) * p->num_heads * p->lq
                                                 : int64_t(p->num_heads) * p->total_kv;
  return (size_t(n) * sizeof(float) + 255) / 256 * 256;
}

size_t rot_bytes(const jfa_problem* p) {
  if (!(p->flags & JFA_ROTARY) || unit_blocks(p)) return 0;
  return (size_t(p->total_kv) * p->num_heads * p->head_dim * 2 + 255) / 256 * 256;
}

size_t block_offsets_bytes(const jfa_problem* p) {
  if (!tiled_blocks(p)) return 0;
  return (size_t(p->total_kv / p->block + 1) * sizeof(int32_t) + 255) / 256 * 256;
}

}  // namespace jfa

extern "C" size_t jfa_bwd_workspace_bytes(const jfa_problem* p) {
  if (!p || check_problem(p) != JFA_OK) return 0;
  if (unit_blocks(p)) return 0;
  size_t bytes = 2 * di_bytes(p) + block_offsets_bytes(p);  // -Di, -lse/scale; block offsets
  if (p->flags & JFA_BROADCAST_Q)
    bytes += size_t(bcast_groups(p->num_seqs)) * p->lq * p->num_heads * p->head_dim * sizeof(float);
  return bytes + 2 * rot_bytes(p);  // rotated q and k (ROTARY)
}

extern "C" size_t jfa_fwd_workspace_bytes(const jfa_problem* p) {
  if (!p || check_problem(p) != JFA_OK) return 0;
  return block_offsets_bytes(p) + 2 * rot_bytes(p);
}

extern "C" const char* jfa_status_string(jfa_status s) {
  switch (s) {
    case JFA_OK: return "ok";
    case JFA_ERR_INVALID_ARG: return "invalid argument";
    case JFA_ERR_UNSUPPORTED: return "unsupported";
    case JFA_ERR_WORKSPACE: return "workspace too small";
    case JFA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

extern "C" const char* jfa_last_error(void) { return jfa::g_error.c_str(); }
