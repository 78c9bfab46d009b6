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

struct Rec { lra::AttnArgs a; int kind; int grid; };   // 0 prefill, 1 decode, 2 decode shared, 3 combine, 4 f32
static std::vector<Rec> g_recs;
namespace lra {
hipError_t launch_prefill_bf16(const AttnArgs& a, int, int, int grid, hipStream_t) { g_recs.push_back({a, 0, grid}); return hipSuccess; }
hipError_t launch_decode_bf16(const AttnArgs& a, int, int, int, hipStream_t) { g_recs.push_back({a, 1, 0}); return hipSuccess; }
hipError_t launch_decode_shared_bf16(const AttnArgs& a, int, int, int, hipStream_t) { g_recs.push_back({a, 2, 0}); return hipSuccess; }
hipError_t launch_combine_bf16(const AttnArgs& a, int, hipStream_t) { g_recs.push_back({a, 3, 0}); return hipSuccess; }
hipError_t launch_attn_f32(const AttnArgs& a, int, int, hipStream_t) { g_recs.push_back({a, 4, 0}); return hipSuccess; }
hipError_t launch_precompute_bf16(const PrecomputeArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_precompute_f32(const PrecomputeArgs&, hipStream_t) { return hipSuccess; }
hipError_t launch_append_bf16(const AppendArgs&, hipStream_t) { return hipSuccess; }
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
          assert(o.k_start == q.k_start && o.k_len == q.k_len && o.n_split == q.n_split);
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
static int check_prefill_order(const std::vector<int>& ql, const std::vector<int>& kl) {
  g_recs.clear();
  const int batch = (int)ql.size(), Hq = 32, Hkv = 8;
  std::vector<int> qs(batch), ks(batch), ag(batch, 0);
  int64_t q_rows = 0, kv_rows = 0;
  for (int b = 0; b < batch; ++b) { qs[b] = (int)q_rows; q_rows += ql[b]; ks[b] = (int)kv_rows; kv_rows += kl[b]; }
  std::vector<int> ranks = {16};
  std::vector<const void*> L = {(void*)0x100000}, B = {(void*)0x200000};
  std::vector<int64_t> ldl = {16};
  const size_t wsb = lra_attn_workspace_bytes(LRA_DTYPE_BF16, 0, batch, ql.data(), kl.data(), Hq, Hkv, 128, 16);
  int rc = lra_attn_prefill(LRA_DTYPE_BF16, batch, Hq, Hkv, 128, qs.data(), ql.data(), ks.data(),
                            kl.data(), ag.data(), (void*)0x1000, q_rows, (void*)0x2000, (void*)0x3000,
                            kv_rows, 1, ranks.data(), L.data(), ldl.data(), B.data(), (void*)0x4000,
                            wsb ? (void*)0x10000000 : nullptr, wsb, nullptr);
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

int main() {
  // prefill: a mixed batch (one launch), 100 requests (two launches), one request
  {
    std::vector<int> ql, kl;
    for (int i = 0; i < 32; ++i) { ql.push_back(1 + (i * 97) % 512); kl.push_back(ql.back() + 2048 + (i * 4441) % 14336); }
    assert(!check_prefill_order(ql, kl));
    ql.clear(); kl.clear();
    for (int i = 0; i < 100; ++i) { ql.push_back(1 + (i * 37) % 300); kl.push_back(ql.back() + (i * 911) % 5000); }
    assert(!check_prefill_order(ql, kl));
    assert(!check_prefill_order({1024}, {9216}));
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
  // same start, different lengths: not grouped
  {
    std::vector<int> ks(4, 0), kl = {100, 200, 300, 400}, ag(4, 0);
    assert(!check(4, 32, 8, ks, kl, ag, {16}, false));
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
