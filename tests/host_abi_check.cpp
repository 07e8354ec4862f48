// Host-only check of libjfa's host code (argument validation, the tile
// scheduler, the JFA_VALIDATE schedule check and the workspace arithmetic),
// built together with schedule.cpp and api.cpp under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitized.py. No GPU and no HIP
// runtime take part: the kernel launchers and the few HIP runtime calls the host
// code makes are replaced below by stubs that record what would have been
// launched ("device" buffers are host arrays here, so the validation copies are
// plain memcpy). The process exits with status 0 only if every check holds;
// any out-of-bounds access or undefined behaviour aborts it.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "../include/jfa.h"
#include "../variable_length_flash_jaggedfa_amd/csrc/jfa_internal.h"

// ---------------------------------------------------------------- stubs
static int g_launches = 0;

namespace jfa {
jfa_status launch_fwd(const FwdLaunch&) { ++g_launches; return JFA_OK; }
jfa_status launch_bwd(const BwdLaunch&) { ++g_launches; return JFA_OK; }
jfa_status launch_block_fwd(const FwdLaunch&) { ++g_launches; return JFA_OK; }
jfa_status launch_block_bwd(const BwdLaunch&) { ++g_launches; return JFA_OK; }
jfa_status launch_block128_bwd(const BwdLaunch&) { ++g_launches; return JFA_OK; }
jfa_status launch_rope_rows(const RopeRowsLaunch&) { ++g_launches; return JFA_OK; }
jfa_status launch_block_offsets(int32_t*, int64_t, int32_t, void*) { ++g_launches; return JFA_OK; }
jfa_status fwd_slots_per_cu(int, uint32_t, int* n) { *n = 2; return JFA_OK; }
jfa_status bwd_slots_per_cu(int, uint32_t, int* n) { *n = 1; return JFA_OK; }
RopeTab rope_table(float, int) { return RopeTab{}; }
}  // namespace jfa

extern "C" {
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }
hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }
hipError_t hipSetDevice(int) { return hipSuccess; }
}

// ---------------------------------------------------------------- checks
static int g_failed = 0;
#define CHECK(cond, ...)                                           \
  do {                                                             \
    if (!(cond)) {                                                 \
      ++g_failed;                                                  \
      std::fprintf(stderr, "FAIL %s:%d: %s | ", __FILE__, __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                           \
      std::fprintf(stderr, " | %s\n", jfa_last_error());           \
    }                                                              \
  } while (0)

static jfa_problem make(int B, int H, int D, int max_len, int64_t T, uint32_t flags, int lq = 0,
                        int window = 0, int block = 0, float rope = 0.f) {
  jfa_problem p{};
  p.num_seqs = B; p.num_heads = H; p.head_dim = D; p.max_len = max_len; p.lq = lq;
  p.flags = flags; p.total_kv = T; p.scale = 0.125f; p.rope_base = rope; p.window = window;
  p.block = block;
  return p;
}

// Every tile exactly once, slot lists consistent, works as the rule states.
static void check_schedule(const jfa_problem& p, const std::vector<int32_t>& off, int32_t kind,
                           int32_t order, int32_t S, std::mt19937& rng) {
  int64_t n = -1;
  jfa_status st = jfa_schedule_count(&p, off.data(), kind, &n);
  CHECK(st == JFA_OK, "count B=%d", p.num_seqs);
  if (st) return;
  std::vector<int32_t> sp(size_t(S) + 1, -7), tl(size_t(std::max<int64_t>(n, 1)) * 4, -7);
  st = jfa_schedule(&p, off.data(), kind, order, S, sp.data(), tl.data(), n);
  if (order == JFA_ORDER_XCD_ZIGZAG && S % 8) {
    CHECK(st == JFA_ERR_INVALID_ARG, "xcd with S=%d", S);
    return;
  }
  CHECK(st == JFA_OK, "schedule order %d S %d", order, S);
  if (st) return;
  CHECK(sp[0] == 0 && sp[S] == n, "slot_ptr ends");
  for (int s = 0; s < S; ++s) CHECK(sp[s + 1] >= sp[s], "slot_ptr monotone");
  const int32_t rows = jfa_tile_rows(kind, p.head_dim, p.flags);
  const bool dense_q = (p.flags & JFA_BROADCAST_Q) && kind == JFA_KIND_FWD;
  std::vector<std::vector<char>> seen(p.num_seqs);
  int64_t expect = 0;
  for (int b = 0; b < p.num_seqs; ++b) {
    const int64_t L = off[b + 1] - off[b];
    const int64_t nt = ((dense_q ? p.lq : L) + rows - 1) / rows;
    seen[b].assign(size_t(nt) * p.num_heads, 0);
    expect += nt * p.num_heads;
  }
  CHECK(expect == n, "count %lld vs %lld", (long long)expect, (long long)n);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t b = tl[4 * i], h = tl[4 * i + 1], t = tl[4 * i + 2];
    if (b < 0 || b >= p.num_seqs || h < 0 || h >= p.num_heads || t < 0) {
      CHECK(false, "tile %lld out of range", (long long)i);
      continue;
    }
    const size_t nt = seen[b].size() / p.num_heads;
    if (size_t(t) >= nt) {
      CHECK(false, "tile index past the sequence");
      continue;
    }
    CHECK(!seen[b][size_t(h) * nt + t], "tile twice");
    seen[b][size_t(h) * nt + t] = 1;
  }
  (void)rng;
}

static void fuzz_scheduler() {
  std::mt19937 rng(1234);
  for (int it = 0; it < 400; ++it) {
    const int B = int(rng() % 40);
    const int H = 1 + int(rng() % 4);
    const int D = (rng() % 2) ? 64 : 128;
    std::vector<int32_t> off(size_t(B) + 1, 0);
    int maxL = 0;
    for (int b = 0; b < B; ++b) {
      const int r = int(rng() % 10);
      const int L = r == 0 ? 0 : r < 8 ? int(rng() % 300) : int(rng() % 3000);
      off[b + 1] = off[b] + L;
      maxL = std::max(maxL, L);
    }
    const uint32_t fl[] = {0u, JFA_CAUSAL, JFA_BROADCAST_Q};
    const uint32_t flags = fl[rng() % 3];
    const int lq = (flags & JFA_BROADCAST_Q) ? 1 + int(rng() % 400) : 0;
    const int window = (flags & JFA_CAUSAL) && rng() % 2 ? 1 + int(rng() % 600) : 0;
    jfa_problem p = make(B, H, D, maxL, off[B], flags, lq, window);
    const int32_t S = 1 + int(rng() % 600);
    for (int32_t kind : {JFA_KIND_FWD, JFA_KIND_BWD})
      for (int32_t order : {JFA_ORDER_INORDER, JFA_ORDER_ZIGZAG, JFA_ORDER_XCD_ZIGZAG,
                            JFA_ORDER_FOLDED_ZIGZAG, JFA_ORDER_XCD_INORDER})
        check_schedule(p, off, kind, order, order == JFA_ORDER_XCD_ZIGZAG ? S / 8 * 8 + 8 * (S < 8) : S,
                       rng);
    // a bad order, too small a capacity, and broken offsets are rejected
    std::vector<int32_t> sp(size_t(S) + 1), tl(4);
    int64_t n = 0;
    jfa_schedule_count(&p, off.data(), JFA_KIND_FWD, &n);
    CHECK(jfa_schedule(&p, off.data(), JFA_KIND_FWD, 9, S, sp.data(), tl.data(), 1 << 30) ==
              JFA_ERR_INVALID_ARG, "bad order");
    if (n > 1)
      CHECK(jfa_schedule(&p, off.data(), JFA_KIND_FWD, JFA_ORDER_ZIGZAG, S, sp.data(), tl.data(),
                         n - 1) == JFA_ERR_INVALID_ARG, "capacity");
    if (B > 1 && off[B] > 0) {
      std::vector<int32_t> bad = off;
      bad[1] = off[B] + 1;  // a sequence past the end, then a negative one
      CHECK(jfa_schedule_count(&p, bad.data(), JFA_KIND_FWD, &n) == JFA_ERR_INVALID_ARG,
            "broken offsets");
    }
  }
}

// Valid and invalid calls of jfa_fwd / jfa_bwd_passes with host arrays as
// "device" buffers; the validation decides, the stubs count the launches.
static void entry_points() {
  const int B = 5, H = 3, D = 128;
  std::vector<int32_t> off = {0, 100, 100, 229, 230, 500};
  const int64_t T = off[B];
  jfa_problem p = make(B, H, D, 270, T, JFA_CAUSAL);
  int32_t S = 16;
  int64_t nf = 0, nb = 0;
  CHECK(jfa_schedule_count(&p, off.data(), JFA_KIND_FWD, &nf) == JFA_OK, "count fwd");
  CHECK(jfa_schedule_count(&p, off.data(), JFA_KIND_BWD, &nb) == JFA_OK, "count bwd");
  std::vector<int32_t> spf(S + 1), tf(nf * 4), spb(S + 1), tb(nb * 4);
  CHECK(jfa_schedule(&p, off.data(), JFA_KIND_FWD, JFA_ORDER_FOLDED_ZIGZAG, S, spf.data(),
                     tf.data(), nf) == JFA_OK, "sched fwd");
  CHECK(jfa_schedule(&p, off.data(), JFA_KIND_BWD, JFA_ORDER_ZIGZAG, S, spb.data(), tb.data(), nb) ==
            JFA_OK, "sched bwd");
  alignas(256) static uint16_t buf[8][16];  // stand-in tensors (never dereferenced)
  alignas(256) static float lse[16];
  const size_t wsb = jfa_bwd_workspace_bytes(&p);
  CHECK(wsb == 2 * ((size_t(H) * T * 4 + 255) / 256 * 256), "bwd workspace %zu", wsb);
  std::vector<char> wsv(wsb + 256);
  void* ws = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(wsv.data()) + 255) / 256 * 256);

  int before = g_launches;
  CHECK(jfa_fwd(&p, buf[0], buf[1], buf[2], off.data(), spf.data(), tf.data(), S, buf[3], lse,
                nullptr, 0, nullptr) == JFA_OK, "fwd ok");
  CHECK(g_launches == before + 1, "fwd launched once");
  before = g_launches;
  CHECK(jfa_bwd_passes(&p, buf[0], buf[1], buf[2], buf[3], buf[4], lse, off.data(), spf.data(),
                       tf.data(), S, spb.data(), tb.data(), S, buf[5], buf[6], buf[7], ws, wsb,
                       JFA_PASS_ALL, nullptr) == JFA_OK, "bwd ok");
  CHECK(g_launches == before + 1, "bwd launched once");

  // each invalid argument: an error and nothing launched
  before = g_launches;
  CHECK(jfa_fwd(&p, nullptr, buf[1], buf[2], off.data(), spf.data(), tf.data(), S, buf[3], lse,
                nullptr, 0, nullptr) == JFA_ERR_INVALID_ARG, "null q");
  CHECK(jfa_fwd(&p, reinterpret_cast<char*>(buf[0]) + 2, buf[1], buf[2], off.data(), spf.data(),
                tf.data(), S, buf[3], lse, nullptr, 0, nullptr) == JFA_ERR_INVALID_ARG, "misaligned");
  CHECK(jfa_fwd(&p, buf[0], buf[1], buf[2], off.data(), spf.data(), tf.data(), 0, buf[3], lse,
                nullptr, 0, nullptr) == JFA_ERR_INVALID_ARG, "no slots");
  CHECK(jfa_fwd(&p, buf[0], buf[1], buf[2], off.data(), spf.data(), tf.data(), S, buf[3], nullptr,
                nullptr, 0, nullptr) == JFA_ERR_INVALID_ARG, "no lse");
  CHECK(jfa_bwd_passes(&p, buf[0], buf[1], buf[2], buf[3], buf[4], lse, off.data(), spf.data(),
                       tf.data(), S, spb.data(), tb.data(), S, buf[5], buf[6], buf[7], ws, wsb - 1,
                       JFA_PASS_ALL, nullptr) == JFA_ERR_WORKSPACE, "small workspace");
  CHECK(jfa_bwd_passes(&p, buf[0], buf[1], buf[2], buf[3], buf[4], lse, off.data(), spf.data(),
                       tf.data(), S, spb.data(), tb.data(), S, buf[5], buf[6], buf[7], ws, wsb, 0,
                       nullptr) == JFA_ERR_INVALID_ARG, "passes 0");
  CHECK(jfa_bwd_passes(&p, buf[0], buf[1], buf[2], buf[3], buf[4], lse, off.data(), spf.data(),
                       tf.data(), S, spb.data(), tb.data(), S, buf[5], buf[6], nullptr, ws, wsb,
                       JFA_PASS_ALL, nullptr) == JFA_ERR_INVALID_ARG, "null dv");
  CHECK(g_launches == before, "nothing launched on errors");

  // JFA_VALIDATE: the good schedules pass, corrupted ones are refused before launch
  setenv("JFA_VALIDATE", "1", 1);
  before = g_launches;
  CHECK(jfa_fwd(&p, buf[0], buf[1], buf[2], off.data(), spf.data(), tf.data(), S, buf[3], lse,
                nullptr, 0, nullptr) == JFA_OK, "validated fwd");
  CHECK(jfa_bwd_passes(&p, buf[0], buf[1], buf[2], buf[3], buf[4], lse, off.data(), spf.data(),
                       tf.data(), S, spb.data(), tb.data(), S, buf[5], buf[6], buf[7], ws, wsb,
                       JFA_PASS_ALL, nullptr) == JFA_OK, "validated bwd");
  CHECK(g_launches == before + 2, "validated calls launch");
  before = g_launches;
  {
    std::vector<int32_t> t2 = tf;
    t2[0] = B;  // a sequence that does not exist
    CHECK(jfa_fwd(&p, buf[0], buf[1], buf[2], off.data(), spf.data(), t2.data(), S, buf[3], lse,
                  nullptr, 0, nullptr) == JFA_ERR_INVALID_ARG, "validate b");
    t2 = tf;
    t2[2] = 1000;  // a tile index past the sequence
    CHECK(jfa_fwd(&p, buf[0], buf[1], buf[2], off.data(), spf.data(), t2.data(), S, buf[3], lse,
                  nullptr, 0, nullptr) == JFA_ERR_INVALID_ARG, "validate t");
    std::vector<int32_t> o2 = off;
    o2[1] = 10;  // device offsets that differ from the schedule's: sequence 0 shrinks
    CHECK(jfa_bwd_passes(&p, buf[0], buf[1], buf[2], buf[3], buf[4], lse, o2.data(), spf.data(),
                         tf.data(), S, spb.data(), tb.data(), S, buf[5], buf[6], buf[7], ws, wsb,
                         JFA_PASS_ALL, nullptr) == JFA_ERR_INVALID_ARG, "validate offsets");
    std::vector<int32_t> s2 = spb;
    s2[1] = -1;
    CHECK(jfa_bwd_passes(&p, buf[0], buf[1], buf[2], buf[3], buf[4], lse, off.data(), spf.data(),
                         tf.data(), S, s2.data(), tb.data(), S, buf[5], buf[6], buf[7], ws, wsb,
                         JFA_PASS_ALL, nullptr) == JFA_ERR_INVALID_ARG, "validate slot_ptr");
  }
  CHECK(g_launches == before, "nothing launched on validation errors");

  // JFA_VALIDATE with block-sparse step lists: good lists pass; a decreasing list
  // pointer, an over-long list (checked before any entry is read, so the copy
  // stays inside the entries array) and an entry past its sequence are refused
  {
    const std::vector<int32_t> so = {0, 130, 130, 450};
    jfa_problem sp_p = make(3, 2, 64, 320, 450, JFA_BLOCK_SPARSE, 0, 0, 64);
    std::vector<uint8_t> mk;
    for (int64_t nb : {3, 0, 5})
      for (int64_t i = 0; i < nb * nb; ++i) mk.push_back(uint8_t((i * 7) % 3 != 0));
    int64_t nu = 0, ne = 0;
    CHECK(jfa_sparse_lists_count(&sp_p, so.data(), mk.data(), int64_t(mk.size()), JFA_KIND_FWD, &nu,
                                 &ne) == JFA_OK, "validate sparse count");
    std::vector<int32_t> sb(4), lp(size_t(nu) + 1), en(size_t(std::max<int64_t>(ne, 1)));
    CHECK(jfa_sparse_lists(&sp_p, so.data(), mk.data(), int64_t(mk.size()), JFA_KIND_FWD, sb.data(),
                           lp.data(), en.data(), ne) == JFA_OK, "validate sparse lists");
    int64_t nt = 0;
    jfa_schedule_count(&sp_p, so.data(), JFA_KIND_FWD, &nt);
    const int32_t SS = 4;
    std::vector<int32_t> ssp(SS + 1), stl(size_t(std::max<int64_t>(nt, 1)) * 4);
    CHECK(jfa_schedule_sparse(&sp_p, so.data(), lp.data(), en.data(), JFA_KIND_FWD,
                              JFA_ORDER_XCD_INORDER, SS, ssp.data(), stl.data(), nt) == JFA_OK,
          "validate sparse schedule");
    auto fwd_with = [&](const std::vector<int32_t>& l, const std::vector<int32_t>& e) {
      jfa_sparse_lists_dev d{sb.data(), l.data(), e.data()};
      return jfa_fwd_sparse(&sp_p, buf[0], buf[1], buf[2], so.data(), &d, ssp.data(), stl.data(), SS,
                            buf[3], lse, nullptr);
    };
    before = g_launches;
    CHECK(fwd_with(lp, en) == JFA_OK, "validated sparse fwd");
    CHECK(g_launches == before + 1, "validated sparse call launches");
    before = g_launches;
    std::vector<int32_t> l2 = lp;
    l2[1] = l2[2] + 1;
    CHECK(fwd_with(l2, en) == JFA_ERR_INVALID_ARG, "validate decreasing list_ptr");
    l2 = lp;
    for (size_t i = 1; i < l2.size(); ++i) l2[i] += 1000;  // every later list 1000 longer
    l2[0] = 0;
    CHECK(fwd_with(l2, en) == JFA_ERR_INVALID_ARG, "validate over-long list");
    std::vector<int32_t> e2 = en;
    e2[0] = (e2[0] & ~((1 << 28) - 1)) | 7;  // block 7 of a 3-block sequence
    CHECK(fwd_with(lp, e2) == JFA_ERR_INVALID_ARG, "validate entry past its sequence");
    CHECK(g_launches == before, "nothing launched on list validation errors");
  }
  unsetenv("JFA_VALIDATE");

  // broadcast-Q, block-diagonal and rotary problems: workspace sizes and launches
  {
    std::vector<int32_t> o = {0, 64, 64, 320};
    jfa_problem pb = make(3, 2, 64, 256, 320, JFA_BROADCAST_Q, 100);
    const size_t w = jfa_bwd_workspace_bytes(&pb);
    CHECK(w == 2 * ((size_t(3) * 2 * 100 * 4 + 255) / 256 * 256) + size_t(3) * 100 * 2 * 64 * 4,
          "bcast workspace %zu", w);
    jfa_problem pk = make(3, 2, 64, 256, 320, JFA_BLOCK_DIAG64);
    CHECK(jfa_bwd_workspace_bytes(&pk) == 0 && jfa_fwd_workspace_bytes(&pk) == 0, "block ws");
    before = g_launches;
    CHECK(jfa_fwd(&pk, buf[0], buf[1], buf[2], o.data(), nullptr, nullptr, 0, buf[3], nullptr,
                  nullptr, 0, nullptr) == JFA_OK, "block fwd");
    CHECK(jfa_fwd(&pk, buf[0], buf[1], buf[2], o.data(), nullptr, nullptr, 0, buf[3], lse, nullptr,
                  0, nullptr) == JFA_ERR_INVALID_ARG, "block fwd with lse");
    CHECK(g_launches == before + 1, "block launches");
    jfa_problem pr = make(3, 2, 128, 256, 320, JFA_CAUSAL | JFA_ROTARY, 0, 0, 0, 10000.f);
    CHECK(jfa_fwd_workspace_bytes(&pr) == 2 * ((size_t(320) * 2 * 128 * 2 + 255) / 256 * 256),
          "rope fwd ws");
  }
  // the probe and the default slot count (stubs: 256 CUs)
  int32_t n = 0;
  CHECK(jfa_default_slots(JFA_KIND_FWD, 128, 0, 0, &n) == JFA_OK && n == 512, "slots %d", n);
  CHECK(jfa_default_slots(JFA_KIND_BWD, 96, 0, 0, &n) == JFA_ERR_UNSUPPORTED, "slots D");
  for (int s = 0; s < 6; ++s) CHECK(jfa_status_string(jfa_status(s)) != nullptr, "status string");
}

// Problems at the limits of the 32-bit addressing and of the counts.
static void limits() {
  std::vector<int32_t> off = {0, 8};
  int64_t n = 0;
  jfa_problem p = make(1, 32768, 128, 8, 8, 0);
  CHECK(jfa_schedule_count(&p, off.data(), JFA_KIND_FWD, &n) == JFA_ERR_UNSUPPORTED, "H*D");
  p = make(1, 32767, 128, 8, 8, 0);
  CHECK(jfa_schedule_count(&p, off.data(), JFA_KIND_FWD, &n) == JFA_OK && n == 32767, "H*D ok");
  std::vector<int32_t> lo = {0, (1 << 20) + 1};
  p = make(1, 16, 128, (1 << 20) + 1, (1 << 20) + 1, 0);
  CHECK(jfa_schedule_count(&p, lo.data(), JFA_KIND_BWD, &n) == JFA_OK && n == 16 * 8193, "long");
  p = make(1, 1, 64, 8, int64_t(INT32_MAX) + 1, 0);
  CHECK(jfa_schedule_count(&p, off.data(), JFA_KIND_FWD, &n) == JFA_ERR_INVALID_ARG, "T > int32");
  p = make(0, 1, 64, 0, 0, 0);
  CHECK(jfa_schedule_count(&p, off.data(), JFA_KIND_FWD, &n) == JFA_OK && n == 0, "empty");
  CHECK(jfa_fwd(&p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr,
                nullptr, 0, nullptr) == JFA_OK, "empty fwd is a no-op");
  CHECK(jfa_schedule_count(nullptr, off.data(), JFA_KIND_FWD, &n) == JFA_ERR_INVALID_ARG, "null");
}

// Block-sparse lists and schedules on random masks: the counts agree with the
// lists, every list is ascending with only valid bits, every tile is dealt once,
// and a query tile's work is 64 x the longer of its two blocks' lists.
static void fuzz_sparse() {
  std::mt19937 rng(99);
  for (int it = 0; it < 200; ++it) {
    const int B = int(rng() % 12);
    const int H = 1 + int(rng() % 3);
    std::vector<int32_t> off(size_t(B) + 1, 0);
    int maxL = 0;
    int64_t mbytes = 0;
    for (int b = 0; b < B; ++b) {
      const int L = (rng() % 5 == 0) ? 0 : 1 + int(rng() % 900);
      off[b + 1] = off[b] + L;
      maxL = std::max(maxL, L);
      const int64_t nb = (L + 63) / 64;
      mbytes += nb * nb;
    }
    std::vector<uint8_t> mask(size_t(std::max<int64_t>(mbytes, 1)));
    const int density = int(rng() % 101);
    for (auto& x : mask) x = uint8_t(int(rng() % 100) < density);
    const uint32_t flags = JFA_BLOCK_SPARSE | ((rng() % 2) ? JFA_CAUSAL : 0u);
    jfa_problem p = make(B, H, 128, maxL, off[B], flags, 0, 0, 64);
    for (int32_t kind : {JFA_KIND_FWD, JFA_KIND_BWD}) {
      int64_t nu = -1, ne = -1;
      CHECK(jfa_sparse_lists_count(&p, off.data(), mask.data(), mbytes, kind, &nu, &ne) == JFA_OK,
            "sparse count");
      if (nu < 0) continue;
      std::vector<int32_t> sb(size_t(B) + 1), lp(size_t(nu) + 1), ent(size_t(std::max<int64_t>(ne, 1)));
      CHECK(jfa_sparse_lists(&p, off.data(), mask.data(), mbytes, kind, sb.data(), lp.data(),
                             ent.data(), ne) == JFA_OK, "sparse lists");
      CHECK(lp[0] == 0 && lp[nu] == ne && sb[B] == nu, "list ends");
      for (int64_t u = 0; u < nu; ++u)
        for (int32_t e = lp[u]; e < lp[u + 1]; ++e) {
          CHECK((ent[e] >> 30) == 0 && (ent[e] >> 28) != 0, "entry bits");
          if (e > lp[u]) CHECK((ent[e] & 0x0FFFFFFF) > (ent[e - 1] & 0x0FFFFFFF), "ascending");
        }
      int64_t n = 0;
      jfa_schedule_count(&p, off.data(), kind, &n);
      const int32_t S = 1 + int(rng() % 100);
      for (int32_t order : {JFA_ORDER_INORDER, JFA_ORDER_ZIGZAG, JFA_ORDER_FOLDED_ZIGZAG,
                            JFA_ORDER_XCD_INORDER}) {
        std::vector<int32_t> sp(size_t(S) + 1), tl(size_t(std::max<int64_t>(n, 1)) * 4);
        CHECK(jfa_schedule_sparse(&p, off.data(), lp.data(), ent.data(), kind, order, S, sp.data(),
                                  tl.data(), n) == JFA_OK, "sparse schedule order %d", order);
        CHECK(sp[0] == 0 && sp[S] == n, "sparse slot_ptr ends");
        int64_t work = 0, want = 0;
        for (int64_t i = 0; i < n; ++i) work += tl[4 * i + 3];
        for (int64_t u = 0; u < nu; ++u) {
          int32_t c0 = 0, c1 = 0;
          for (int32_t e = lp[u]; e < lp[u + 1]; ++e) {
            c0 += (ent[e] >> 28) & 1;
            c1 += (ent[e] >> 29) & 1;
          }
          want += int64_t(H) * 64 * (kind == JFA_KIND_FWD ? std::max(c0, c1) : lp[u + 1] - lp[u]);
        }
        CHECK(work == want, "sparse work %lld vs %lld", (long long)work, (long long)want);
      }
    }
  }
}

int main() {
  fuzz_scheduler();
  fuzz_sparse();
  entry_points();
  limits();
  if (g_failed) {
    std::fprintf(stderr, "%d checks failed\n", g_failed);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
