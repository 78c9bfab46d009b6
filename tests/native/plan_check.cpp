// Host-only check of the attention planner in lra_api.cpp.  The kernel launchers are
// replaced by stubs that record each launch's argument block, and the checks cover what the
// kernels rely on: every request is launched exactly once; in the shared-context decode
// launches the members of a unit are consecutive, read the same base rows, share the split
// count and never exceed the member cap; the first member owns the unit's work items and
// the others carry INT32_MAX; the lookup the kernels use (the last request whose work start
// is <= w) maps every work item into its unit; a unit has no more key splits than its
// members alone (the workspace query plans without grouping); and the plain decode kernel
// runs when no two requests share base rows or grouping is switched off.
#include <cassert>
#include <cstdio>
#include <cstdlib>
#include <set>
#include <algorithm>
#include <vector>
#include "lra.h"
#include "lra_internal.h"

struct Rec { lra::AttnArgs a; int kind; int grid; bool expand; int min_rank = -1; };   // 0 prefill, 1 decode, 2 decode shared, 3 combine, 4 f32
static std::vector<Rec> g_recs;
static std::vector<lra::ExpandArgs> g_expand;
static std::vector<lra::AppendArgs> g_append;
namespace lra {
hipError_t launch_prefill_bf16(const AttnArgs& a, int, int, int grid, hipStream_t, bool ex, int min_rank) { g_recs.push_back({a, 0, grid, ex, min_rank}); return hipSuccess; }
hipError_t launch_decode_bf16(const AttnArgs& a, int, int, int, hipStream_t, bool ex) { g_recs.push_back({a, 1, 0, ex}); return hipSuccess; }
hipError_t launch_expand_bf16(const ExpandArgs& a, int, int, hipStream_t) { g_expand.push_back(a); return hipSuccess; }
hipError_t launch_decode_shared_bf16(const AttnArgs& a, int, int, int, hipStream_t) { g_recs.push_back({a, 2, 0, false}); return hipSuccess; }
hipError_t launch_combine_bf16(const AttnArgs& a, int, hipStream_t) { g_recs.push_back({a, 3, 0, false}); return hipSuccess; }
hipError_t launch_attn_f32(const AttnArgs& a, int, int, hipStream_t) { g_recs.push_back({a, 4, 0, false}); return hipSuccess; }
hipError_t launch_precompute_bf16(const PrecomputeArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_precompute_f32(const PrecomputeArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t) { g_append.push_back(a); return hipSuccess; }
hipError_t launch_append_f32(const AppendArgs&, hipStream_t) { return hipSuccess; }
}

static int check(int batch, int Hq, int Hkv, const std::vector<int>& ks, const std::vector<int>& kl,
                 const std::vector<int>& ag, const std::vector<int>& ranks, bool expect_shared) {
  g_recs.clear();
  std::vector<const void*> L(ranks.size(), (void*)0x100000), B(ranks.size(), (void*)0x200000);
  std::vector<int64_t> ldl(ranks.size(), 64);
  const int64_t kv_rows = 1 << 22;
  size_t wsb = lra_attn_workspace_bytes(LRA_DTYPE_BF16, 1, batch, nullptr, kl.data(), Hq, Hkv, 128, 64);
  int rc = lra_attn_decode(LRA_DTYPE_BF16, batch, Hq, Hkv, 128, ks.data(), kl.data(), ag.data(),
                           (void*)0x1000, (void*)0x2000, (void*)0x3000, kv_rows, (int)ranks.size(),
                           ranks.data(), L.data(), ldl.data(), B.data(), (void*)0x4000,
                           wsb ? (void*)0x5000 : nullptr, wsb, nullptr);
  if (rc) { printf("rc %d: %s\n", rc, lra_last_error()); return 1; }
  const int G = Hq / Hkv;
  const int cap = std::min(lra::kMaxMembers, 16 / G);
  std::multiset<int> seen;
  bool any_shared = false;
  for (const Rec& r : g_recs) {
    if (r.kind == 3) continue;
    const lra::AttnArgs& a = r.a;
    any_shared |= r.kind == 2;
    int64_t work = 0;
    for (int i = 0; i < a.n_req; ++i) {
      const lra::ReqDesc& q = a.reqs[i];
      seen.insert(q.q_start);
      if (q.n_members > 0) {
        assert(q.work_start == work);
        assert(q.n_members <= (r.kind == 2 ? cap : 1));
        for (int m = 1; m < q.n_members; ++m) {
          const lra::ReqDesc& o = a.reqs[i + m];
          assert(o.n_members == 0 && o.work_start == INT32_MAX);
          // one first row; the first member is the longest (it sets the key range)
          assert(o.k_start == q.k_start && o.k_len <= q.k_len && o.n_split == q.n_split);
        }
        // never more splits than alone (the workspace is sized without grouping)
        const int alone = std::max(1, std::min({(q.k_len + 1023) / 1024, (q.k_len + 63) / 64, 64}));
        assert(q.n_split >= 1 && q.n_split <= alone);
        if (q.n_split > 1) assert(q.part_base >= 0);
        work += (int64_t)Hkv * q.n_rt * q.n_split;
      } else {
        assert(r.kind == 2 && q.work_start == INT32_MAX);
      }
    }
    assert(work == a.n_work);
    // the kernel's lookup: last request with work_start <= w
    for (int w = 0; w < a.n_work; ++w) {
      int u = -1;
      for (int i = 0; i < a.n_req; ++i) if (a.reqs[i].work_start <= w) u = i;
      assert(u >= 0 && a.reqs[u].n_members > 0);
      assert(w - a.reqs[u].work_start < Hkv * a.reqs[u].n_split);
    }
  }
  assert((int)seen.size() == batch);
  for (int b = 0; b < batch; ++b) assert(seen.count(b) == 1);
  assert(any_shared == expect_shared);
  return 0;
}

// bf16 prefill launches: several requests are sorted by descending keys per work item
// (ceil(k_len / n_split)) and dealt over the XCDs (grid_per_xcd == 0); a single request
// keeps the XCD-major mapping.  Either way the kernel's block -> item map covers every
// work item exactly once, and every request appears exactly once.
static int check_prefill_order(const std::vector<int>& ql, const std::vector<int>& kl,
                               const std::vector<int>& ranks = {16},
                               const std::vector<int>& agents = {}) {
  g_recs.clear();
  const int batch = (int)ql.size(), Hq = 32, Hkv = 8;
  std::vector<int> qs(batch), ks(batch), ag(batch, 0);
  for (int b = 0; b < batch && !agents.empty(); ++b) ag[b] = agents[b];
  int64_t q_rows = 0, kv_rows = 0;
  for (int b = 0; b < batch; ++b) { qs[b] = (int)q_rows; q_rows += ql[b]; ks[b] = (int)kv_rows; kv_rows += kl[b]; }
  std::vector<const void*> L(ranks.size(), (void*)0x100000), B(ranks.size(), (void*)0x200000);
  std::vector<int64_t> ldl(ranks.size(), 64);
  const size_t wsb = lra_attn_workspace_bytes(LRA_DTYPE_BF16, 0, batch, ql.data(), kl.data(), Hq, Hkv, 128, 64);
  int rc = lra_attn_prefill(LRA_DTYPE_BF16, batch, Hq, Hkv, 128, qs.data(), ql.data(), ks.data(),
                            kl.data(), ag.data(), (void*)0x1000, q_rows, (void*)0x2000, (void*)0x3000,
                            kv_rows, (int)ranks.size(), ranks.data(), L.data(), ldl.data(), B.data(),
                            (void*)0x4000, wsb ? (void*)0x10000000 : nullptr, wsb, nullptr);
  if (rc) { printf("rc %d: %s\n", rc, lra_last_error()); return 1; }
  std::multiset<int> seen;
  for (const Rec& r : g_recs) {
    if (r.kind != 0) continue;
    const lra::AttnArgs& a = r.a;
    int64_t work = 0, prev = INT64_MAX;
    for (int i = 0; i < a.n_req; ++i) {
      const lra::ReqDesc& q = a.reqs[i];
      seen.insert(q.q_start);
      assert(q.work_start == work);
      work += (int64_t)Hkv * q.n_rt * q.n_split;
      const int64_t keys = (q.k_len + q.n_split - 1) / q.n_split;
      if (a.n_req > 1) assert(keys <= prev);
      prev = keys;
    }
    assert(work == a.n_work);
    assert((a.n_req > 1) == (a.grid_per_xcd == 0));
    // the launch reports its smallest rank (the kernel then runs each item at its own width)
    int lo = 1 << 30;
    for (int i = 0; i < a.n_req; ++i) lo = std::min(lo, a.agents[a.reqs[i].agent].rank);
    assert(r.min_rank == lo);
    std::vector<int> hit(a.n_work, 0);
    for (int bid = 0; bid < r.grid; ++bid) {
      const int w = a.grid_per_xcd > 0
                        ? (bid & 7) * a.grid_per_xcd + (bid >> 3)
                        : ((bid >> 3) / lra::kDealChunk) * (8 * lra::kDealChunk) +
                              (bid & 7) * lra::kDealChunk + (bid >> 3) % lra::kDealChunk;
      if (w < a.n_work) ++hit[w];
    }
    for (int w = 0; w < a.n_work; ++w) assert(hit[w] == 1);
  }
  for (int b = 0; b < batch; ++b) assert(seen.count(qs[b]) == 1);
  return 0;
}

// Validation paths of every entry point: each malformed or unsupported call returns its
// status with a message and launches nothing; a valid call clears the message.
static void expect(int rc, int want, const char* what) {
  if (rc != want) { printf("%s: rc %d, want %d (%s)\n", what, rc, want, lra_last_error()); abort(); }
  if (want != LRA_OK && lra_last_error()[0] == '\0') { printf("%s: no message\n", what); abort(); }
  if (want == LRA_OK && lra_last_error()[0] != '\0') { printf("%s: stale message\n", what); abort(); }
}

struct PrefillCall {
  int dtype = LRA_DTYPE_BF16, batch = 2, Hq = 8, Hkv = 2, D = 128;
  std::vector<int> qs = {0, 10}, ql = {10, 5}, ks = {0, 0}, kl = {100, 50}, ag = {0, 1};
  int64_t q_rows = 15, kv_rows = 100;
  std::vector<int> ranks = {16, 8};
  std::vector<const void*> L = {(void*)0x100000, (void*)0x101000};
  std::vector<int64_t> ldl = {16, 8};
  std::vector<const void*> B = {(void*)0x200000, (void*)0x202000};
  size_t ws_bytes = (size_t)1 << 30;
  int run() {
    g_recs.clear();
    const int rc = lra_attn_prefill(dtype, batch, Hq, Hkv, D, qs.data(), ql.data(), ks.data(),
                                    kl.data(), ag.data(), (void*)0x1000, q_rows, (void*)0x2000,
                                    (void*)0x3000, kv_rows, (int)ranks.size(), ranks.data(),
                                    L.data(), ldl.data(), B.data(), (void*)0x4000,
                                    (void*)0x10000000, ws_bytes, nullptr);
    if (rc != LRA_OK) assert(g_recs.empty());
    return rc;
  }
};

static void check_validation() {
  expect(PrefillCall().run(), LRA_OK, "valid prefill");
  { PrefillCall c; c.dtype = 7; expect(c.run(), LRA_ERR_INVALID, "dtype"); }
  { PrefillCall c; c.batch = -1; expect(c.run(), LRA_ERR_INVALID, "negative batch"); }
  { PrefillCall c; c.batch = LRA_MAX_BATCH + 1; expect(c.run(), LRA_ERR_UNSUPPORTED, "batch cap"); }
  { PrefillCall c; c.Hq = 6; c.Hkv = 4; expect(c.run(), LRA_ERR_INVALID, "Hq % Hkv"); }
  { PrefillCall c; c.Hq = 32; c.Hkv = 2; expect(c.run(), LRA_ERR_UNSUPPORTED, "group > 8"); }
  { PrefillCall c; c.D = 96; expect(c.run(), LRA_ERR_UNSUPPORTED, "head_dim"); }
  { PrefillCall c; c.ql[1] = 60; expect(c.run(), LRA_ERR_INVALID, "q_len > k_len"); }
  { PrefillCall c; c.qs[1] = 5; expect(c.run(), LRA_ERR_INVALID, "overlapping query rows"); }
  { PrefillCall c; c.ks[0] = 1; expect(c.run(), LRA_ERR_INVALID, "key rows past kv_rows"); }
  { PrefillCall c; c.ag[1] = 2; expect(c.run(), LRA_ERR_INVALID, "agent index"); }
  { PrefillCall c; c.ranks[0] = 12; expect(c.run(), LRA_ERR_UNSUPPORTED, "rank % 8"); }
  { PrefillCall c; c.ranks[0] = 72; c.ldl[0] = 72; expect(c.run(), LRA_ERR_UNSUPPORTED, "rank cap"); }
  { PrefillCall c; c.ldl[0] = 8; expect(c.run(), LRA_ERR_INVALID, "ldl < rank"); }
  { PrefillCall c; c.ldl[0] = 20; expect(c.run(), LRA_ERR_INVALID, "ldl % 8"); }
  { PrefillCall c; c.L[1] = (void*)0x101004; expect(c.run(), LRA_ERR_INVALID, "L alignment"); }
  { PrefillCall c; c.ws_bytes = 16; c.kl = {3000, 50}; c.kv_rows = 3000;
    // few row tiles over many keys: the planner splits the keys, which needs a workspace
    const size_t need = lra_attn_workspace_bytes(LRA_DTYPE_BF16, 0, 2, c.ql.data(), c.kl.data(), 8, 2, 128, 16);
    assert(need > 16);
    expect(c.run(), LRA_ERR_WORKSPACE, "workspace too small");
    c.ws_bytes = need;
    expect(c.run(), LRA_OK, "workspace of the queried size"); }
  { PrefillCall c; c.ql = {0, 0}; expect(c.run(), LRA_OK, "empty requests"); assert(g_recs.empty()); }
  assert(lra_attn_workspace_bytes(LRA_DTYPE_BF16, 0, 1, nullptr, nullptr, 8, 2, 128, 16) == (size_t)-1);
  { const int ql = 5, kl = 4;
    assert(lra_attn_workspace_bytes(LRA_DTYPE_BF16, 0, 1, &ql, &kl, 8, 2, 128, 16) == (size_t)-1); }
  // decode
  { const int ks[2] = {0, 0}, kl[2] = {10, 0}, ag[2] = {0, 0}, r = 16;
    const void* L = (void*)0x100000; const void* B = (void*)0x200000; const int64_t ldl = 16;
    expect(lra_attn_decode(LRA_DTYPE_BF16, 2, 8, 2, 128, ks, kl, ag, (void*)0x1000, (void*)0x2000,
                           (void*)0x3000, 100, 1, &r, &L, &ldl, &B, (void*)0x4000, nullptr, 0, nullptr),
           LRA_ERR_INVALID, "decode with an empty context"); }
  // precompute and append
  const int ranks[3] = {64, 64, 64};
  void* outs[3] = {(void*)0x100000, (void*)0x200000, (void*)0x300000};
  const int64_t ldl[3] = {64, 64, 64};
  expect(lra_precompute_lr(LRA_DTYPE_BF16, 100, 4096, (void*)0x1000, 4096, (void*)0x2000, 192, 3,
                           ranks, outs, ldl, nullptr), LRA_OK, "valid precompute");
  expect(lra_precompute_lr(LRA_DTYPE_BF16, 100, 100, (void*)0x1000, 104, (void*)0x2000, 192, 3,
                           ranks, outs, ldl, nullptr), LRA_ERR_UNSUPPORTED, "d_model % 8");
  expect(lra_precompute_lr(LRA_DTYPE_BF16, 100, 4096, (void*)0x1000, 4000, (void*)0x2000, 192, 3,
                           ranks, outs, ldl, nullptr), LRA_ERR_INVALID, "ldx < d_model");
  expect(lra_precompute_lr(LRA_DTYPE_BF16, 100, 4096, (void*)0x1000, 4096, (void*)0x2000, 100, 3,
                           ranks, outs, ldl, nullptr), LRA_ERR_INVALID, "lda < sum of ranks");
  { const int big[5] = {64, 64, 64, 64, 64}; void* o5[5] = {outs[0], outs[1], outs[2], outs[0], outs[1]};
    const int64_t l5[5] = {64, 64, 64, 64, 64};
    expect(lra_precompute_lr(LRA_DTYPE_BF16, 100, 4096, (void*)0x1000, 4096, (void*)0x2000, 320, 5,
                             big, o5, l5, nullptr), LRA_ERR_UNSUPPORTED, "sum of ranks > 256"); }
  { const int rows[3] = {5, 9, 5};
    expect(lra_append_lr(LRA_DTYPE_BF16, 3, 4096, (void*)0x1000, 4096, (void*)0x2000, 192, 3, ranks,
                         outs, ldl, rows, 100, nullptr, 0, nullptr), LRA_ERR_INVALID, "duplicate append rows"); }
  { const int rows[2] = {5, 100};
    expect(lra_append_lr(LRA_DTYPE_BF16, 2, 4096, (void*)0x1000, 4096, (void*)0x2000, 192, 3, ranks,
                         outs, ldl, rows, 100, nullptr, 0, nullptr), LRA_ERR_INVALID, "append row out of range"); }
  { std::vector<int> rows(LRA_MAX_BATCH + 1);
    for (size_t i = 0; i < rows.size(); ++i) rows[i] = (int)i;
    expect(lra_append_lr(LRA_DTYPE_BF16, (int)rows.size(), 4096, (void*)0x1000, 4096, (void*)0x2000,
                         192, 3, ranks, outs, ldl, rows.data(), 1 << 20, nullptr, 0, nullptr),
           LRA_ERR_UNSUPPORTED, "append batch cap"); }
  { const int rows[2] = {5, 9};
    const size_t wsb = lra_append_workspace_bytes(LRA_DTYPE_BF16, 2, 4096, 3, ranks);
    assert(wsb > 0 && wsb != (size_t)-1);
    assert(lra_append_workspace_bytes(LRA_DTYPE_F32, 2, 4096, 3, ranks) == 0);
    assert(lra_append_workspace_bytes(LRA_DTYPE_BF16, -1, 4096, 3, ranks) == (size_t)-1);
    expect(lra_append_lr(LRA_DTYPE_BF16, 2, 4096, (void*)0x1000, 4096, (void*)0x2000, 192, 3, ranks,
                         outs, ldl, rows, 100, nullptr, 0, nullptr), LRA_ERR_WORKSPACE,
           "append without workspace");
    expect(lra_append_lr(LRA_DTYPE_BF16, 2, 4096, (void*)0x1000, 4096, (void*)0x2000, 192, 3, ranks,
                         outs, ldl, rows, 100, (void*)0x8000, wsb - 4, nullptr), LRA_ERR_WORKSPACE,
           "append with a short workspace");
    expect(lra_append_lr(LRA_DTYPE_BF16, 2, 4096, (void*)0x1000, 4096, (void*)0x2000, 192, 3, ranks,
                         outs, ldl, rows, 100, (void*)0x8000, wsb, nullptr), LRA_OK, "valid append");
    expect(lra_append_lr(LRA_DTYPE_F32, 2, 4096, (void*)0x1000, 4096, (void*)0x2000, 192, 3, ranks,
                         outs, ldl, rows, 100, nullptr, 0, nullptr), LRA_OK, "fp32 append, no workspace"); }
}

// The bf16 append's split of d_model: slices of whole 256-value rounds that cover d_model
// exactly once, partial blocks of 64 x 64 that cover the launch's tokens and columns, about
// sixteen workgroups when that many rounds exist, and a workspace query that bounds every
// launch of a call (batches above 256 tokens take several launches).
static void check_append_plan() {
  for (int64_t T : {1, 37, 64, 65, 256})
    for (int64_t dm : {64, 128, 320, 512, 4096, 16384})
      for (int64_t R : {8, 64, 192, 256}) {
        const lra::AppendPlan p = lra::plan_append(T, dm, R);
        const int nk = (int)(dm / 32);
        assert(p.slice_chunks % 8 == 0 && p.slice_chunks > 0);
        assert(p.n_slices >= 1 && p.n_slices <= lra::kAppendMaxSlices);
        assert((int64_t)p.n_slices * p.slice_chunks >= nk);
        assert((int64_t)(p.n_slices - 1) * p.slice_chunks < nk);   // no empty slice
        assert(p.t_pad % 64 == 0 && p.t_pad >= T && p.t_pad < T + 64);
        assert(p.r_pad % 64 == 0 && p.r_pad >= R && p.r_pad < R + 64);
        const int64_t items = (int64_t)p.n_slices * (p.t_pad / 64) * (p.r_pad / 64);
        assert(items >= std::min<int64_t>(16, (int64_t)((nk + 7) / 8) * (p.t_pad / 64) * (p.r_pad / 64)) / 2);
      }
  const lra::AppendPlan w = lra::plan_append(64, 4096, 64);   // the decode batch's append
  assert(w.n_slices == 16 && w.slice_chunks == 8 && w.bytes() == 16 * 64 * 64 * 4);
  const int ranks[6] = {0, 40, 24, 64, 64, 64};
  void* outs[6] = {nullptr, (void*)0x10000, (void*)0x20000, (void*)0x30000, (void*)0x40000, (void*)0x50000};
  const int64_t ldl[6] = {0, 40, 24, 64, 64, 64};
  std::vector<int> rows(300);
  for (int i = 0; i < 300; ++i) rows[i] = 2 * i;
  const size_t wsb = lra_append_workspace_bytes(LRA_DTYPE_BF16, 300, 256, 6, ranks);
  g_append.clear();
  expect(lra_append_lr(LRA_DTYPE_BF16, 300, 256, (void*)0x1000, 256, (void*)0x2000, 256, 6, ranks,
                       outs, ldl, rows.data(), 700, (void*)0x8000, wsb, nullptr), LRA_OK,
         "append in two launches");
  assert(g_append.size() == 2 && g_append[0].p.T == 256 && g_append[1].p.T == 44);
  for (const lra::AppendArgs& a : g_append) {
    const lra::AppendPlan p{a.n_slices, a.slice_chunks, a.t_pad, a.r_pad};
    assert(a.part == (float*)0x8000 && (size_t)p.bytes() <= wsb);
    assert(a.rows[0] == (a.p.T == 256 ? 0 : 512));
  }
}

// The comparators: the in-tile expansion decode never groups shared contexts and launches
// the expanding kernel; lra_expand_values splits spans into chunks of kExpandRows per kv
// head, at most kReqsPerLaunch spans per launch, and refuses overlapping spans.
static void check_comparators() {
  std::vector<int> ks(8, 0), kl(8, 4096), ag = {0, 1, 0, 1, 0, 1, 0, 1};
  const int ranks[2] = {16, 64};
  const void* L[2] = {(void*)0x100000, (void*)0x200000};
  const void* B[2] = {(void*)0x300000, (void*)0x400000};
  const int64_t ldl[2] = {16, 64};
  const size_t wsb = lra_attn_workspace_bytes(LRA_DTYPE_BF16, 1, 8, nullptr, kl.data(), 32, 8, 128, 64);
  g_recs.clear();
  expect(lra_attn_decode_expand(LRA_DTYPE_BF16, 8, 32, 8, 128, ks.data(), kl.data(), ag.data(),
                                (void*)0x1000, (void*)0x2000, (void*)0x3000, 4096, 2, ranks, L,
                                ldl, B, (void*)0x4000, (void*)0x10000000, wsb, nullptr),
         LRA_OK, "decode, in-tile expansion");
  bool any = false;
  for (const Rec& r : g_recs) {
    assert(r.kind != 2);
    if (r.kind == 1) { assert(r.expand); any = true; }
  }
  assert(any);
  expect(lra_attn_decode_expand(LRA_DTYPE_F32, 8, 32, 8, 128, ks.data(), kl.data(), ag.data(),
                                (void*)0x1000, (void*)0x2000, (void*)0x3000, 4096, 2, ranks, L,
                                ldl, B, (void*)0x4000, (void*)0x10000000, wsb, nullptr),
         LRA_ERR_UNSUPPORTED, "in-tile expansion in fp32");
  // 70 spans (two launches), one empty, lengths around the chunk size
  std::vector<int> st, ln, sa;
  int row = 0;
  for (int i = 0; i < 70; ++i) {
    const int n = i == 5 ? 0 : 1 + (i * 397) % 1500;
    st.push_back(row); ln.push_back(n); sa.push_back(i % 2); row += n + (i % 3);
  }
  g_expand.clear();
  expect(lra_expand_values(LRA_DTYPE_BF16, 70, st.data(), ln.data(), sa.data(), (void*)0x1000, row,
                           8, 128, 2, ranks, L, ldl, B, (void*)0x2000, nullptr),
         LRA_OK, "expand values");
  assert(g_expand.size() == 2);
  int seen = 0;
  for (const lra::ExpandArgs& a : g_expand) {
    int64_t work = 0;
    for (int i = 0; i < a.n_span; ++i) {
      const lra::ExpandSpan& sp = a.spans[i];
      assert(sp.len > 0 && sp.work_start == work);
      assert(a.rows_per_item % 32 == 0 && a.rows_per_item >= 32 && a.rows_per_item <= lra::kExpandRows);
      work += (int64_t)((sp.len + a.rows_per_item - 1) / a.rows_per_item) * 8;
      ++seen;
    }
    assert(work == a.n_work && a.n_span <= lra::kReqsPerLaunch);
  }
  assert(seen == 69);
  st[3] = st[2] + 1;   // overlaps span 2
  expect(lra_expand_values(LRA_DTYPE_BF16, 70, st.data(), ln.data(), sa.data(), (void*)0x1000, row,
                           8, 128, 2, ranks, L, ldl, B, (void*)0x2000, nullptr),
         LRA_ERR_INVALID, "overlapping spans");
  expect(lra_expand_values(LRA_DTYPE_F32, 1, st.data(), ln.data(), sa.data(), (void*)0x1000, row,
                           8, 128, 2, ranks, L, ldl, B, (void*)0x2000, nullptr),
         LRA_ERR_UNSUPPORTED, "expand values in fp32");
}

int main() {
  check_validation();
  check_comparators();
  check_append_plan();
  // prefill: a mixed batch (one launch), 100 requests (two launches), one request
  {
    std::vector<int> ql, kl;
    for (int i = 0; i < 32; ++i) { ql.push_back(1 + (i * 97) % 512); kl.push_back(ql.back() + 2048 + (i * 4441) % 14336); }
    assert(!check_prefill_order(ql, kl));
    ql.clear(); kl.clear();
    for (int i = 0; i < 100; ++i) { ql.push_back(1 + (i * 37) % 300); kl.push_back(ql.back() + (i * 911) % 5000); }
    assert(!check_prefill_order(ql, kl));
    assert(!check_prefill_order({1024}, {9216}));
    // agents of ranks 8, 64 and 0 in one launch
    {
      std::vector<int> mq, mk, ma;
      for (int i = 0; i < 12; ++i) { mq.push_back(1 + (i * 53) % 300); mk.push_back(mq.back() + 500 + (i * 977) % 4000); ma.push_back(i % 3); }
      assert(!check_prefill_order(mq, mk, {8, 64, 0}, ma));
    }
  }
  // 16 contexts x 4 agents, G = 4: units of 4
  {
    std::vector<int> ks, kl, ag;
    for (int c = 0; c < 16; ++c) for (int a = 0; a < 4; ++a) { ks.push_back(c * 16384); kl.push_back(16384); ag.push_back(a); }
    assert(!check(64, 32, 8, ks, kl, ag, {16, 16, 16, 16}, true));
  }
  // interleaved order, 7 requests per context (units 4 + 3), G = 2 (cap 4), 150 requests (3 launches)
  {
    std::vector<int> ks, kl, ag;
    for (int i = 0; i < 150; ++i) { ks.push_back((i % 22) * 1000); kl.push_back(900 + (i % 22)); ag.push_back(i % 3); }
    assert(!check(150, 16, 8, ks, kl, ag, {8, 64, 0}, true));
  }
  // G = 8: cap 2
  {
    std::vector<int> ks(10, 0), kl(10, 5000), ag(10, 1);
    assert(!check(10, 64, 8, ks, kl, ag, {16, 32}, true));
  }
  // distinct contexts: no unit, the plain kernel
  {
    std::vector<int> ks, kl, ag;
    for (int i = 0; i < 70; ++i) { ks.push_back(i * 100); kl.push_back(100); ag.push_back(0); }
    assert(!check(70, 32, 8, ks, kl, ag, {16}, false));
  }
  // same start, different lengths (agents that have seen different lengths of one
  // context): grouped when their solo split counts agree, longest first
  {
    std::vector<int> ks(4, 0), kl = {100, 200, 300, 400}, ag(4, 0);
    assert(!check(4, 32, 8, ks, kl, ag, {16}, true));
  }
  // ... and not across different split counts (1, 2 and 3 splits of 1024 keys)
  {
    std::vector<int> ks(3, 0), kl = {1000, 2000, 3000}, ag(3, 0);
    assert(!check(3, 32, 8, ks, kl, ag, {16}, false));
  }
  // grouping switched off
  {
    setenv("LRA_DECODE_GROUP", "0", 1);
    std::vector<int> ks(8, 0), kl(8, 4096), ag(8, 0);
    assert(!check(8, 32, 8, ks, kl, ag, {16}, false));
    unsetenv("LRA_DECODE_GROUP");
  }
  printf("planner checks passed\n");
  return 0;
}
