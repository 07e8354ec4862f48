/*
 * jfa.h -- C ABI of the MI355X (gfx950) jagged flash attention library (libjfa.so).
 *
 * The library computes exact softmax attention, forward and backward, directly on
 * packed bf16 Q/K/V whose sequences are concatenated with no padding and whose
 * boundaries are given by an int32 offsets array ("Jagged Flash Attention for GEM",
 * introduction; the packed-tensor-plus-offsets layout). Besides plain jagged
 * self-attention it covers:
 *   - broadcast-Q: one dense Q shared by every sequence, so dQ is a sum over the
 *     batch ("Jagged Flash Attention for GEM", backward / dQ section);
 *   - 64-token block-diagonal attention, where each 64-token group attends only
 *     within itself, with a single-tile path that keeps no running statistics and
 *     stores no log-sum-exp ("TLX Block Attention", sections 1, 2 and 4); 32-token
 *     blocks run on the same single-tile kernels, 128- and 256-token blocks as
 *     jagged attention over the blocks (the page contrasts 64-token blocks with a
 *     256-token minimum tile elsewhere);
 *   - rotary position embeddings of Q and K ("TLX Block Attention", summary and
 *     the section on the memory-bandwidth bound, where they are fused into the
 *     attention kernels): inside the block-diagonal kernels the rotated rows never
 *     travel through memory; on the jagged path one pass writes rotated copies of
 *     q and k to the workspace and the backward turns dQ and dK back in its
 *     epilogues;
 *   - a host scheduler that sorts tiles by KV work and deals them zigzag over the
 *     persistent workgroups ("Jagged Flash Attention for GEM", section on the
 *     GEM-specific optimisations).
 *
 * Conventions for every entry point
 *   Layouts     q, k, v, out, dout, dq, dk, dv: bf16, contiguous, 16-byte aligned.
 *               Jagged: [T, H, D] token-major, T = offsets[B].
 *               Broadcast-Q: q and dq [Lq, H, D]; out and dout [B, Lq, H, D];
 *               k, v, dk, dv [T, H, D].
 *               lse (float32): jagged [H, T]; broadcast-Q [B, H, Lq]; no lse for
 *               the block-diagonal mode. lse is the natural-log log-sum-exp of
 *               each query row's scaled scores.
 *               offsets: int32 [B + 1], offsets[0] = 0, non-decreasing.
 *   Maths       S = scale * Q K^T, P = softmax(S) per query row, out = P V.
 *               Causal: inside a sequence, query i attends keys j <= i; with a
 *               window W > 0 only keys i - W < j <= i (a causal sliding window,
 *               a modelling variant the pages name without defining).
 *               Rotary: S = scale * rot(Q) rot(K)^T with the rows of Q and K
 *               rotated by their token position p (index inside the sequence):
 *               column pairs (i, i + D/2), i < D/2, turn by the angle
 *               p * rope_base^(-2i/D), (x1, x2) -> (x1 cos a - x2 sin a,
 *               x2 cos a + x1 sin a); V is not rotated, and dq, dk are the
 *               gradients with respect to the unrotated q and k. The scores
 *               depend only on position differences, so the block-diagonal
 *               kernels count positions from the start of each 64-token group.
 *   Ownership   The caller allocates every host and device buffer (schedule arrays
 *               and workspace included). The library allocates nothing, keeps no
 *               pointer after a call returns, and enqueues work only on `stream`
 *               (a hipStream_t; NULL is the default stream).
 *   Async       jfa_fwd / jfa_bwd return once their kernels are enqueued.
 *   Errors      Return codes only; nothing throws across the ABI. Arguments are
 *               checked on the host before any HIP call, so on any error nothing
 *               is enqueued. jfa_last_error() gives a thread-local message.
 *   Threads     Calls are thread-safe; calls on one stream execute in order.
 *   Diagnostics Read from the environment on every call:
 *               JFA_VALIDATE=1  jfa_fwd / jfa_bwd / jfa_bwd_passes (and the
 *                 sparse calls) first synchronise `stream`, copy the device offsets
 *                 and schedules back and check the precondition the kernels rely on
 *                 (offsets start at 0, never decrease, end at total_kv, no length
 *                 above max_len; the tiles cover every (sequence, head, tile index)
 *                 exactly once; block-sparse step lists: seq_base gives each
 *                 sequence's first unit, list_ptr starts at 0 and never decreases,
 *                 every entry names a block pair of its sequence, ascending within
 *                 its list). A mismatch
 *                 returns JFA_ERR_INVALID_ARG with nothing enqueued. Costs a
 *                 synchronisation and blocking copies: for debugging.
 *               JFA_LOG=1  one line per call of those entry points on stderr.
 */
#ifndef JFA_H
#define JFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum jfa_status {
  JFA_OK = 0,
  JFA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size, bad offsets */
  JFA_ERR_UNSUPPORTED = 2,  /* head_dim or flag combination not implemented */
  JFA_ERR_WORKSPACE = 3,    /* workspace missing or too small */
  JFA_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed */
} jfa_status;

/* problem flags */
#define JFA_CAUSAL       1u  /* causal mask inside each sequence (jagged self-attention only) */
#define JFA_BROADCAST_Q  2u  /* one dense Q [Lq,H,D] shared by every sequence (non-causal) */
#define JFA_BLOCK_DIAG64 4u  /* 64-token block-diagonal self-attention (non-causal) */
#define JFA_ROTARY       8u  /* rotary embeddings of Q and K (not with BROADCAST_Q) */
#define JFA_BLOCK_DIAG  16u  /* block-diagonal self-attention with blocks of
                                jfa_problem.block tokens (32, 64, 128 or 256) */
#define JFA_BLOCK_SPARSE 32u /* block-sparse self-attention over 64-token blocks
                                (jfa_problem.block = 64; CAUSAL the only other
                                flag): see the jfa_sparse_* entry points */

/* schedule kinds and dealing orders */
#define JFA_KIND_FWD 0
#define JFA_KIND_BWD 1
#define JFA_ORDER_INORDER 0  /* tiles in generation order, tile j to slot j mod S */
#define JFA_ORDER_ZIGZAG  1  /* sorted by KV work, descending; zigzag deal */
#define JFA_ORDER_XCD_ZIGZAG 2 /* the same deal inside each of the 8 XCDs, after whole
                                  (sequence, head) units are dealt zigzag by total
                                  work over the XCDs; num_slots % 8 == 0 */
#define JFA_ORDER_FOLDED_ZIGZAG 3 /* ZIGZAG over items; with CAUSAL an item is the pair
                                     of tiles a and n-1-a of one (sequence, head) */
#define JFA_ORDER_XCD_INORDER 4 /* (sequence, head) units in generation order, each to
                                   the XCD (group of num_slots / 8 consecutive slots;
                                   one group of all slots if num_slots % 8 != 0) with
                                   the least work dealt so far, its tiles in order each
                                   to that group's least-loaded slot; ties to the lower
                                   group or slot. Keeps the tiles of a unit together in
                                   time and on one L2 while balancing the slots */

typedef struct jfa_problem {
  int32_t num_seqs;   /* B >= 0 */
  int32_t num_heads;  /* H >= 1 */
  int32_t head_dim;   /* D: 64 or 128 */
  int32_t max_len;    /* >= every sequence length (checked by jfa_schedule_count) */
  int32_t lq;         /* BROADCAST_Q: rows of the dense Q (>= 1); otherwise 0 */
  uint32_t flags;     /* JFA_CAUSAL | JFA_BROADCAST_Q | JFA_BLOCK_DIAG64 | JFA_ROTARY |
                         JFA_BLOCK_DIAG, or JFA_BLOCK_SPARSE [| JFA_CAUSAL] */
  int64_t total_kv;   /* T = offsets[B], tokens in the packed K/V */
  float scale;        /* softmax scale applied to Q K^T, finite and > 0 */
  float rope_base;    /* ROTARY: base of the rotary frequencies, finite, in (1, 1e9];
                         otherwise must be 0 */
  int32_t window;     /* CAUSAL only: W > 0 restricts query i to keys i - W < j <= i
                         (a causal sliding window); 0 = no window; 0 with
                         BLOCK_SPARSE */
  int32_t block;      /* BLOCK_DIAG: tokens per block, 32, 64, 128 or 256; with
                         BLOCK_DIAG64 alone 0 or 64; BLOCK_SPARSE: 64; otherwise 0 */
} jfa_problem;

/* Rows of Q per forward tile (kind FWD) or of K/V per backward tile (kind BWD)
 * that the kernels use for this head_dim and flags; -1 if unsupported.
 * BLOCK_DIAG64: 64 (the single-tile unit); BLOCK_DIAG: the jagged tile rows, which
 * the 128- and 256-token blocks use. */
int32_t jfa_tile_rows(int32_t kind, int32_t head_dim, uint32_t flags);

/* Number of persistent workgroups (slots) the schedule should be dealt over on
 * `device`: compute units times resident workgroups per compute unit. Writes
 * *num_slots. Queries the HIP device (the only host entry point that does). */
jfa_status jfa_default_slots(int32_t kind, int32_t head_dim, uint32_t flags, int32_t device,
                             int32_t* num_slots);

/* Validate the host offsets against the problem and count the tiles of `kind`.
 * Checks: offsets[0] == 0, non-decreasing, offsets[B] == total_kv, every length
 * <= max_len, and for block-diagonal problems every length a multiple of the
 * block size. For blocks of 32 or 64 tokens the count is the number of (64-token
 * unit, head) pairs the single-tile kernels run (no schedule is needed); for
 * blocks of 128 or 256 tokens it is the number of tiles of the jagged problem
 * whose sequences are the blocks (in order), which jfa_schedule deals. The
 * argument `offsets_host` is host memory, B+1 ints. */
jfa_status jfa_schedule_count(const jfa_problem* p, const int32_t* offsets_host, int32_t kind,
                              int64_t* num_tiles);

/* Build the tile schedule on the host ("Jagged Flash Attention for GEM",
 * GEM-specific optimisations: sort by KV work, deal zigzag).
 *   Forward tile (b,h,t): query rows [t*BM, t*BM+BM) of sequence b (of the dense
 *     Q for BROADCAST_Q), head h; work = keys visited: L_b, or with CAUSAL
 *     min(L_b, (t+1)*BM), less max(0, t*BM - W + 1) with a window W.
 *   Backward tile (b,h,n): key rows [n*BN, n*BN+BN) of sequence b, head h;
 *     work = query rows that attend them: L_b (Lq for BROADCAST_Q), or with
 *     CAUSAL L_b - n*BN, or with a window min(L_b, (n+1)*BN - 1 + W) - n*BN.
 *   Generation order is b, then h, then t. ZIGZAG: stable sort by descending
 *   work, sorted position j goes to pass j / S, rank r = j % S, slot r on even
 *   passes and S-1-r on odd ones. INORDER: tile j goes to slot j % S.
 *   XCD_ZIGZAG: the (b, h) units, with work = sum of their tiles' work, are
 *   stable-sorted by descending work and dealt zigzag over 8 groups; group x
 *   owns slots [x*S/8, (x+1)*S/8) (the kernels run those slots on XCD x, so the
 *   tiles of one sequence share an L2), and its tiles are dealt with the ZIGZAG
 *   rule over those slots.
 *   FOLDED_ZIGZAG (an MI355X refinement for causal problems): the tiles of one
 *   (b, h), indices 0..n-1 in generation order, are folded into items {a, n-1-a}
 *   for a < n/2, plus {n/2} when n is odd, each with the summed work; without
 *   CAUSAL every tile is its own item. Items in generation order of their first
 *   tile are dealt with the ZIGZAG rule, and an item's tiles go to one slot in
 *   that order. Under CAUSAL the items of one (b, h) have nearly equal work, so
 *   the sort keeps them adjacent and they run side by side on neighbouring
 *   slots, sharing the sequence's K/V (or Q/dO) in L2, where the plain ZIGZAG
 *   spreads its tiles, whose works differ, over the whole kernel.
 * Outputs (host memory, caller-allocated):
 *   slot_ptr [num_slots + 1]: tiles of slot s are tiles[slot_ptr[s] .. slot_ptr[s+1]).
 *   tiles    [capacity][4] int32 (b, h, t, work), grouped by slot in dealing order.
 * `capacity` must be >= the count from jfa_schedule_count. Not valid for
 * BLOCK_DIAG64 or for blocks of 32 or 64 tokens (UNSUPPORTED). For 128- and
 * 256-token blocks the tiles' b is the block index (sequences in order, blocks in
 * order inside each). Host only; no HIP call. */
jfa_status jfa_schedule(const jfa_problem* p, const int32_t* offsets_host, int32_t kind,
                        int32_t order, int32_t num_slots, int32_t* slot_ptr, int32_t* tiles,
                        int64_t capacity);

/* Bytes of device workspace jfa_bwd needs: two float32 row vectors laid out like
 * lse, each rounded up to 256 bytes (-Di and -lse/scale, written by the dQ pass
 * and read by the dK/dV pass) and, for BROADCAST_Q, float32 dQ partials of
 * [G][Lq][H][D] where the B sequences are split into G = min(B, 128) contiguous
 * groups (each holding about T/G keys); for 128- or 256-token blocks also the block offsets, (T/block + 1)
 * int32 rounded up to 256 bytes; for ROTARY (except on blocks of 32 or 64
 * tokens) also two bf16 [T, H, D] regions, each rounded up to 256 bytes, for the
 * rotated copies of q and k; 0 for blocks of 32 or 64 tokens. 0 for an invalid
 * problem. */
size_t jfa_bwd_workspace_bytes(const jfa_problem* p);

/* Bytes of device workspace jfa_fwd needs: for 128- or 256-token blocks the block
 * offsets, (T/block + 1) int32 rounded up to 256 bytes; for ROTARY (except on
 * blocks of 32 or 64 tokens) two bf16 [T, H, D] regions, each rounded up to 256
 * bytes, that receive the rotated copies of q and k; 0 otherwise and for an
 * invalid problem. */
size_t jfa_fwd_workspace_bytes(const jfa_problem* p);

/* Forward ("TLX Block Attention", section 2: the online-softmax loop; section 3,
 * pipeline order load -> Q K^T -> exp2 softmax -> P V -> epilogue).
 *   q, k, v      device, bf16, layouts above.
 *   offsets_dev  device copy of the offsets the schedule was built from.
 *   slot_ptr_dev, tiles_dev, num_slots: device copy of a FWD schedule
 *                (ignored, may be NULL, for blocks of 32 or 64 tokens).
 *   out          device, bf16, written for every valid query row.
 *   lse          device float32; must be NULL for blocks of 32 or 64 tokens,
 *                non-NULL otherwise ([H, T] for 128- and 256-token blocks).
 *   workspace    device, >= jfa_fwd_workspace_bytes(p) bytes, 256-byte aligned;
 *                contents on entry are ignored and clobbered (jagged ROTARY: the
 *                rotated q and k). May be NULL when the size is 0.
 * A broadcast-Q sequence with no keys gets out = 0 and lse = -inf.
 * Precondition (not checked on the device; JFA_VALIDATE=1 checks it on the host):
 * offsets_dev equals the host offsets the schedule was built from. */
jfa_status jfa_fwd(const jfa_problem* p, const void* q, const void* k, const void* v,
                   const int32_t* offsets_dev, const int32_t* slot_ptr_dev,
                   const int32_t* tiles_dev, int32_t num_slots, void* out, float* lse,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Backward ("TLX Block Attention", sections 2 and 4; "Jagged Flash Attention for
 * GEM", backward / dQ section): P is rebuilt from Q, K and lse, Di = rowsum(dO*out)
 * is computed inside the kernels, dS = P * (dP - Di), dV = P^T dO,
 * dK = scale dS^T Q, dQ = scale dS K (summed over sequences for BROADCAST_Q).
 * No memory atomics are used: dQ is produced by a pass over query tiles and
 * dK/dV by a pass over key tiles, so dK and dV (and dQ) are bitwise reproducible.
 *   out, dout    device bf16 (out as written by jfa_fwd).
 *   lse          device float32 from jfa_fwd; NULL for blocks of 32 or 64 tokens
 *                (that path recomputes the softmax statistics instead).
 *   q_slot_ptr_dev, q_tiles_dev, q_num_slots: device copy of a FWD schedule; the
 *                dQ pass walks these query tiles. Ignored for BROADCAST_Q and for
 *                blocks of 32 or 64 tokens (may be NULL).
 *   kv_slot_ptr_dev, kv_tiles_dev, kv_num_slots: device copy of a BWD schedule;
 *                the dK/dV pass walks these key tiles. Ignored for blocks of 32 or
 *                64 tokens.
 *   dq, dk, dv   device bf16 outputs (dq is [Lq,H,D] for BROADCAST_Q).
 *   workspace    device, >= jfa_bwd_workspace_bytes(p) bytes, 256-byte aligned;
 *                contents on entry are ignored and clobbered. May be NULL when the
 *                size is 0. */
jfa_status jfa_bwd(const jfa_problem* p, const void* q, const void* k, const void* v,
                   const void* out, const void* dout, const float* lse,
                   const int32_t* offsets_dev, const int32_t* q_slot_ptr_dev,
                   const int32_t* q_tiles_dev, int32_t q_num_slots,
                   const int32_t* kv_slot_ptr_dev, const int32_t* kv_tiles_dev,
                   int32_t kv_num_slots, void* dq, void* dk, void* dv, void* workspace,
                   size_t workspace_bytes, void* stream);

/* The two passes of the backward, for jfa_bwd_passes. */
#define JFA_PASS_DQ   1u  /* dQ pass over query tiles; also writes Di into the workspace */
#define JFA_PASS_DKDV 2u  /* dK/dV pass over key tiles; reads Di from the workspace */
#define JFA_PASS_ALL  3u

/* jfa_bwd restricted to some of its passes, so that each can be timed or
 * overlapped on its own. Same arguments as jfa_bwd plus `passes`, a non-zero
 * mask of JFA_PASS_*. JFA_PASS_DKDV alone is valid only after a JFA_PASS_DQ call
 * with the same problem, inputs and workspace on the same stream (it reads the Di,
 * and for ROTARY the rotated q and k, that pass left in the workspace); the
 * library cannot check this. Blocks of 32 or 64 tokens run one fused kernel and
 * accept JFA_PASS_ALL only (JFA_ERR_INVALID_ARG otherwise). For 128-token blocks
 * without ROTARY, JFA_PASS_ALL runs one single-tile kernel ("TLX Block
 * Attention", sections 2 and 4: lse and workspace are checked but not read),
 * while the passes called apart run the two jagged passes; the two agree within
 * rounding, not bit for bit. jfa_bwd(...) is jfa_bwd_passes(..., JFA_PASS_ALL, stream). */
jfa_status jfa_bwd_passes(const jfa_problem* p, const void* q, const void* k, const void* v,
                          const void* out, const void* dout, const float* lse,
                          const int32_t* offsets_dev, const int32_t* q_slot_ptr_dev,
                          const int32_t* q_tiles_dev, int32_t q_num_slots,
                          const int32_t* kv_slot_ptr_dev, const int32_t* kv_tiles_dev,
                          int32_t kv_num_slots, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, uint32_t passes, void* stream);

/* ---- Block-sparse attention (JFA_BLOCK_SPARSE)
 * The pages name block-sparse patterns as a modelling variant and contrast a
 * 256-token minimum tile with the 64-token blocks their models need ("TLX Block
 * Attention", section 1; "Jagged Flash Attention for GEM", the section on
 * generative models). Here each sequence b of L_b tokens is cut into
 * n_b = ceil(L_b / 64) blocks of 64 tokens (the last one partial) and an
 * n_b x n_b byte matrix says which key blocks each query block attends: query i
 * attends key j of its own sequence iff mask_b[i / 64][j / 64] != 0, and with
 * JFA_CAUSAL also j <= i (the block mask and the causal rule both hold). The mask
 * (host memory) holds every sequence's matrix row-major (row = query block),
 * concatenated in sequence order: sum of n_b^2 bytes. A query row that attends no
 * key gets out = 0 and lse = -inf, and adds nothing to the gradients. The problem
 * has flags = JFA_BLOCK_SPARSE, optionally | JFA_CAUSAL, block = 64, window = 0;
 * its tiles are those of jagged self-attention (jfa_schedule_count).
 *
 * The kernels walk step lists built on the host from the mask. A unit is (b, t)
 * for each sequence b and tile index t (128 query rows for kind FWD, 128 keys for
 * kind BWD: the 64-token blocks 2t and 2t+1), units in order of b, then t.
 *   seq_base [B + 1]      first unit of sequence b (seq_base[B] = units).
 *   list_ptr [units + 1]  unit u's entries are entries[list_ptr[u] .. list_ptr[u+1]).
 *   entries               int32: bits 0..27 the other side's block index (FWD: key
 *                         block c; BWD: query block r), ascending; bit 28 set when
 *                         the unit's block 2t pairs with it (FWD: mask[2t][c];
 *                         BWD: mask[r][2t]), bit 29 likewise for block 2t+1.
 *                         With CAUSAL a bit is also cleared where the causal
 *                         rule masks the whole block pair (FWD: bit 28 when
 *                         c > 2t, bit 29 when c > 2t+1; BWD: bit 28 when r < 2t,
 *                         bit 29 when r < 2t+1). Blocks paired with neither are
 *                         left out. */
typedef struct jfa_sparse_lists_dev {
  const int32_t* seq_base;  /* device copies of the arrays above, 4-byte aligned */
  const int32_t* list_ptr;
  const int32_t* entries;
} jfa_sparse_lists_dev;

/* Sizes of the step lists of `kind`: *num_units = seq_base[B] (the units) and
 * *num_entries. Checks the problem (BLOCK_SPARSE), the offsets as
 * jfa_schedule_count does, and mask_bytes == sum of n_b^2. Host only. */
jfa_status jfa_sparse_lists_count(const jfa_problem* p, const int32_t* offsets_host,
                                  const uint8_t* mask_host, int64_t mask_bytes, int32_t kind,
                                  int64_t* num_units, int64_t* num_entries);

/* Build the step lists of `kind` from the host mask into caller-allocated host
 * arrays: seq_base [B + 1], list_ptr [num_units + 1], entries [num_entries]
 * (entries_capacity >= num_entries). Host only; no HIP call. */
jfa_status jfa_sparse_lists(const jfa_problem* p, const int32_t* offsets_host,
                            const uint8_t* mask_host, int64_t mask_bytes, int32_t kind,
                            int32_t* seq_base, int32_t* list_ptr, int32_t* entries,
                            int64_t entries_capacity);

/* jfa_schedule for a BLOCK_SPARSE problem: the same tiles, orders and outputs.
 * list_ptr_host and entries_host are the lists of the same kind from
 * jfa_sparse_lists (entries_host may be NULL for kind BWD). A BWD tile's work is
 * 64 times its list's length (the dK/dV pass walks the whole list); a FWD tile's
 * is 64 times the larger number of its entries that carry bit 28 or bit 29 (the
 * forward and the dQ pass walk the two blocks' entries side by side). Returns
 * INVALID_ARG if list_ptr_host[0] != 0, the list pointers decrease or a list is
 * longer than its sequence has 64-token blocks. Host only. */
jfa_status jfa_schedule_sparse(const jfa_problem* p, const int32_t* offsets_host,
                               const int32_t* list_ptr_host, const int32_t* entries_host,
                               int32_t kind, int32_t order, int32_t num_slots, int32_t* slot_ptr,
                               int32_t* tiles, int64_t capacity);

/* Block-sparse forward: as jfa_fwd with the FWD step lists (device) and no
 * workspace; a tile visits only the key blocks its list names. Preconditions as
 * for jfa_fwd, and the lists are those of the offsets and mask the schedule was
 * built from (not checked on the device; JFA_VALIDATE=1 checks their structure). */
jfa_status jfa_fwd_sparse(const jfa_problem* p, const void* q, const void* k, const void* v,
                          const int32_t* offsets_dev, const jfa_sparse_lists_dev* lists,
                          const int32_t* slot_ptr_dev, const int32_t* tiles_dev,
                          int32_t num_slots, void* out, float* lse, void* stream);

/* Block-sparse backward: as jfa_bwd_passes with the FWD step lists (q_lists, for
 * the dQ pass over the FWD schedule) and the BWD step lists (kv_lists, for the
 * dK/dV pass over the BWD schedule); workspace of jfa_bwd_workspace_bytes(p). */
jfa_status jfa_bwd_sparse(const jfa_problem* p, const void* q, const void* k, const void* v,
                          const void* out, const void* dout, const float* lse,
                          const int32_t* offsets_dev, const jfa_sparse_lists_dev* q_lists,
                          const int32_t* q_slot_ptr_dev, const int32_t* q_tiles_dev,
                          int32_t q_num_slots, const jfa_sparse_lists_dev* kv_lists,
                          const int32_t* kv_slot_ptr_dev, const int32_t* kv_tiles_dev,
                          int32_t kv_num_slots, void* dq, void* dk, void* dv, void* workspace,
                          size_t workspace_bytes, uint32_t passes, void* stream);

/* Bytes of the static device scratch array jfa_bwd_noalloc uses as its workspace
 * (32 MiB, held by every GPU the library runs on until the process ends). */
#define JFA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* jfa_bwd without a workspace argument, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that forbid
 * allocation): the workspace is a static device array of
 * JFA_NOALLOC_SCRATCH_BYTES bytes in the library, and nothing is allocated.
 * Same arguments, results and errors as jfa_bwd otherwise; the caller still
 * provides every input and output buffer. A problem whose
 * jfa_bwd_workspace_bytes exceeds JFA_NOALLOC_SCRATCH_BYTES is rejected with
 * JFA_ERR_WORKSPACE before anything is enqueued (jagged problems up to about
 * H * T = 4M query rows fit; broadcast-Q up to about
 * 2 * B * H * Lq + min(B, 128) * Lq * H * D floats). Each GPU has one array,
 * shared by every call on it: calls that overlap on one GPU (different streams
 * or threads) race, calls on one stream do not. Nothing in it needs clearing
 * between calls (the backward writes every workspace entry before reading it).
 * The first call on a device looks up that device's copy of the array. */
jfa_status jfa_bwd_noalloc(const jfa_problem* p, const void* q, const void* k, const void* v,
                           const void* out, const void* dout, const float* lse,
                           const int32_t* offsets_dev, const int32_t* q_slot_ptr_dev,
                           const int32_t* q_tiles_dev, int32_t q_num_slots,
                           const int32_t* kv_slot_ptr_dev, const int32_t* kv_tiles_dev,
                           int32_t kv_num_slots, void* dq, void* dk, void* dv, void* stream);

/* Matrix-core probe (measurement only; not a step of the attention path): a
 * kernel of `workgroups` workgroups of four waves, each wave running four
 * independent chains of `iters` bf16 32x32x16 MFMAs (32768 FLOP each) on
 * register operands, so the benchmark can report the MFMA rate the chip
 * sustains and its core clock beside the published dense peak.
 *   iters       1 .. 2^24
 *   workgroups  1 .. 65536 (at most one is resident per compute unit; one per
 *               compute unit puts one wave on every SIMD)
 *   sink        device float32 [workgroups * 256], written (keeps the products live)
 *   clocks      device uint64 [workgroups * 4]: per workgroup, the core-clock
 *               counter (s_memtime) and the constant-rate counter
 *               (s_memrealtime) elapsed over wave 0's loop, then the
 *               constant-rate counter's values at the loop's start and end
 * Host checks only (INVALID_ARG on a bad count, a NULL or a misaligned
 * pointer); asynchronous on `stream`. FLOP per call = workgroups*4*4*iters*32768. */
jfa_status jfa_probe_mfma(int32_t iters, int32_t workgroups, float* sink, uint64_t* clocks,
                         void* stream);

/* HBM copy probe (measurement only; not a step of the attention path): copies
 * `bytes` bytes from `src` to `dst` (device memory, 16-byte aligned, bytes a
 * multiple of 16) with 16-byte non-temporal loads and stores, `workgroups`
 * workgroups of 256 threads striding over the buffers, so the benchmark can
 * report the bandwidth a plain stream sustains beside the published 8 TB/s.
 * Host checks only (INVALID_ARG); asynchronous on `stream`. */
jfa_status jfa_probe_copy(const void* src, void* dst, uint64_t bytes, int32_t workgroups,
                          void* stream);

/* Static text for a status code. */
const char* jfa_status_string(jfa_status s);

/* Message describing the last error raised on the calling thread ("" if none). */
const char* jfa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* JFA_H */
