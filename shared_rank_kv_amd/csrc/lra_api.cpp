// C-ABI front end of liblra.so: argument validation (host only, before any HIP call),
// work planning, workspace sizing and kernel dispatch.  Declarations and the contract of
// every entry point are in include/lra.h.
#include "lra.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <utility>
#include <vector>

#include "lra_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return LRA_OK;
}

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shared-context decode grouping is on unless LRA_DECODE_GROUP=0 (kept for comparisons).
bool group_decode_enabled() {
  const char* v = std::getenv("LRA_DECODE_GROUP");
  return !(v && v[0] == '0' && v[1] == '\0');
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  int x = std::atoi(v);
  return x > 0 ? x : dflt;
}

// ---------------------------------------------------------------------------------------
// Validation
// ---------------------------------------------------------------------------------------

struct AttnShape {
  int dtype, batch, Hq, Hkv, D;
};

int check_shape(const AttnShape& s) {
  if (s.dtype != LRA_DTYPE_F32 && s.dtype != LRA_DTYPE_BF16)
    return fail(LRA_ERR_INVALID, "dtype %d is neither LRA_DTYPE_F32 nor LRA_DTYPE_BF16", s.dtype);
  if (s.batch < 0) return fail(LRA_ERR_INVALID, "batch %d < 0", s.batch);
  if (s.batch > LRA_MAX_BATCH)
    return fail(LRA_ERR_UNSUPPORTED, "batch %d > LRA_MAX_BATCH (%d)", s.batch, LRA_MAX_BATCH);
  if (s.Hq <= 0 || s.Hkv <= 0)
    return fail(LRA_ERR_INVALID, "head counts must be positive (n_q_heads %d, n_kv_heads %d)",
                s.Hq, s.Hkv);
  if (s.Hq % s.Hkv != 0)
    return fail(LRA_ERR_INVALID, "n_q_heads %d is not a multiple of n_kv_heads %d", s.Hq, s.Hkv);
  if (s.Hq / s.Hkv > LRA_MAX_GROUP)
    return fail(LRA_ERR_UNSUPPORTED, "group size %d > LRA_MAX_GROUP (%d)", s.Hq / s.Hkv,
                LRA_MAX_GROUP);
  if (s.D <= 0) return fail(LRA_ERR_INVALID, "head_dim %d <= 0", s.D);
  if (s.D != 64 && s.D != 128)
    return fail(LRA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", s.D);
  // the bf16 kernels address a 64-row tile of K/V rows (and B's rank rows) with 32-bit
  // byte offsets
  if (s.dtype == LRA_DTYPE_BF16 && (int64_t)s.Hkv * s.D * 2 * 64 >= ((int64_t)1 << 31))
    return fail(LRA_ERR_UNSUPPORTED, "bf16 K/V rows of %lld bytes: 64 of them must stay below "
                "2 GiB", (long long)s.Hkv * s.D * 2);
  return LRA_OK;
}

struct Adapters {
  int32_t n_agents;
  const int32_t* ranks;
  const void* const* L;
  const int64_t* ldl;
  const void* const* B;
};

int check_adapters(int dtype, const Adapters& ad, int64_t kv_rows) {
  if (ad.n_agents <= 0) return fail(LRA_ERR_INVALID, "n_agents %d <= 0", ad.n_agents);
  if (ad.n_agents > LRA_MAX_AGENTS)
    return fail(LRA_ERR_UNSUPPORTED, "n_agents %d > LRA_MAX_AGENTS (%d)", ad.n_agents,
                LRA_MAX_AGENTS);
  if (!ad.ranks || !ad.L || !ad.ldl || !ad.B)
    return fail(LRA_ERR_INVALID, "ranks, L, ldl and B must be non-null host arrays");
  const int ldl_mult = dtype == LRA_DTYPE_BF16 ? 8 : 4;
  for (int a = 0; a < ad.n_agents; ++a) {
    const int r = ad.ranks[a];
    if (r < 0) return fail(LRA_ERR_INVALID, "ranks[%d] = %d < 0", a, r);
    if (r > LRA_MAX_RANK || r % 8 != 0)
      return fail(LRA_ERR_UNSUPPORTED, "ranks[%d] = %d: ranks must be multiples of 8 up to %d",
                  a, r, LRA_MAX_RANK);
    if (r == 0) continue;
    if (!ad.L[a] || !ad.B[a]) return fail(LRA_ERR_INVALID, "L[%d] / B[%d] is null", a, a);
    if (ad.ldl[a] < r) return fail(LRA_ERR_INVALID, "ldl[%d] = %lld < rank %d", a,
                                   (long long)ad.ldl[a], r);
    if (ad.ldl[a] % ldl_mult != 0)
      return fail(LRA_ERR_INVALID, "ldl[%d] = %lld is not a multiple of %d elements", a,
                  (long long)ad.ldl[a], ldl_mult);
    // the bf16 kernels address a 64-row tile of LR rows with 32-bit byte offsets
    if (dtype == LRA_DTYPE_BF16 && ad.ldl[a] * 2 * 64 >= ((int64_t)1 << 31))
      return fail(LRA_ERR_UNSUPPORTED, "ldl[%d] = %lld: 64 bf16 LR rows must stay below 2 GiB",
                  a, (long long)ad.ldl[a]);
    if (!aligned(ad.L[a], 16) || !aligned(ad.B[a], 16))
      return fail(LRA_ERR_INVALID, "L[%d] / B[%d] not 16-byte aligned", a, a);
    (void)kv_rows;
  }
  return LRA_OK;
}

struct Requests {
  const int32_t* q_start;
  const int32_t* q_len;
  const int32_t* k_start;
  const int32_t* k_len;
  const int32_t* agent;
};

int check_requests(int batch, const Requests& rq, int64_t q_rows, int64_t kv_rows,
                   int32_t n_agents) {
  if (batch == 0) return LRA_OK;
  if (!rq.q_start || !rq.q_len || !rq.k_start || !rq.k_len || !rq.agent)
    return fail(LRA_ERR_INVALID, "request arrays must be non-null host arrays");
  if (q_rows < 0 || kv_rows < 0) return fail(LRA_ERR_INVALID, "q_rows / kv_rows < 0");
  std::vector<std::pair<int64_t, int64_t>> spans;
  for (int b = 0; b < batch; ++b) {
    const int64_t qs = rq.q_start[b], ql = rq.q_len[b], ks = rq.k_start[b], kl = rq.k_len[b];
    if (ql < 0 || kl < 0) return fail(LRA_ERR_INVALID, "request %d: negative length", b);
    if (ql == 0) continue;
    if (ql > kl)
      return fail(LRA_ERR_INVALID, "request %d: q_len %lld > k_len %lld", b, (long long)ql,
                  (long long)kl);
    if (qs < 0 || qs + ql > q_rows)
      return fail(LRA_ERR_INVALID, "request %d: query rows [%lld, %lld) outside [0, %lld)", b,
                  (long long)qs, (long long)(qs + ql), (long long)q_rows);
    if (ks < 0 || ks + kl > kv_rows)
      return fail(LRA_ERR_INVALID, "request %d: key rows [%lld, %lld) outside [0, %lld)", b,
                  (long long)ks, (long long)(ks + kl), (long long)kv_rows);
    if (rq.agent[b] < 0 || rq.agent[b] >= n_agents)
      return fail(LRA_ERR_INVALID, "request %d: agent_idx %d outside [0, %d)", b, rq.agent[b],
                  n_agents);
    spans.emplace_back(qs, qs + ql);
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second)
      return fail(LRA_ERR_INVALID, "query/output rows of two requests overlap at row %lld",
                  (long long)spans[i].first);
  return LRA_OK;
}

// ---------------------------------------------------------------------------------------
// Planning (deterministic: the workspace query and the call agree)
// ---------------------------------------------------------------------------------------

struct Plan {
  std::vector<int> active;     // requests with q_len > 0, in order
  std::vector<int> n_rt, n_split;
  std::vector<int64_t> part_base;
  int64_t part_rows = 0;
  size_t ws_bytes = 0;
};

size_t part_bytes(int64_t part_rows, int D) {
  return (size_t)part_rows * (size_t)(D + 2) * sizeof(float);
}

Plan make_plan(const AttnShape& s, bool decode, const int32_t* q_len, const int32_t* k_len) {
  Plan p;
  const int G = s.Hq / s.Hkv;
  for (int b = 0; b < s.batch; ++b) {
    const int ql = decode ? 1 : q_len[b];
    if (ql <= 0) continue;
    p.active.push_back(b);
  }
  const size_t n = p.active.size();
  p.n_rt.resize(n);
  p.n_split.assign(n, 1);
  p.part_base.assign(n, -1);
  if (s.dtype == LRA_DTYPE_F32) {
    for (size_t i = 0; i < n; ++i) {
      const int ql = decode ? 1 : q_len[p.active[i]];
      p.n_rt[i] = (int)ceil_div(ql, 16);   // 16 query rows per fp32 workgroup
    }
    return p;
  }
  int64_t total_wg = 0;
  for (size_t i = 0; i < n; ++i) {
    const int ql = decode ? 1 : q_len[p.active[i]];
    p.n_rt[i] = (int)ceil_div((int64_t)ql * G, decode ? lra::kTileRows : lra::kPrefillRows);
    total_wg += (int64_t)s.Hkv * p.n_rt[i];
  }
  if (decode) {
    const int chunk = env_int("LRA_DECODE_CHUNK", 1024);
    for (size_t i = 0; i < n; ++i) {
      const int64_t kl = k_len[p.active[i]];
      const int64_t tiles = ceil_div(kl, lra::kTileKeys);
      p.n_split[i] = (int)std::max<int64_t>(1, std::min<int64_t>({ceil_div(kl, chunk), tiles, 64}));
    }
  } else {
    // one workgroup per CU: split keys until the launch covers the 256 CUs
    const int target = env_int("LRA_PREFILL_TARGET_WG", 256);
    if (total_wg < target) {
      const int64_t factor = ceil_div(target, std::max<int64_t>(total_wg, 1));
      for (size_t i = 0; i < n; ++i) {
        const int64_t tiles = ceil_div(k_len[p.active[i]], lra::kTileKeys);
        p.n_split[i] = (int)std::max<int64_t>(1, std::min<int64_t>({factor, tiles / 8, 64}));
      }
    }
  }
  for (size_t i = 0; i < n; ++i) {
    if (p.n_split[i] <= 1) continue;
    const int ql = decode ? 1 : q_len[p.active[i]];
    p.part_base[i] = p.part_rows;
    p.part_rows += (int64_t)p.n_split[i] * ql * s.Hq;
  }
  p.ws_bytes = p.part_rows ? part_bytes(p.part_rows, s.D) + 256 : 0;
  return p;
}

// ---------------------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------------------

// expand: the in-tile expansion comparator instead of the regrouped LR term (bf16 only;
// every request is its own work unit, since one expanded V tile serves one agent).
int run_attention(const AttnShape& s, bool decode, const Requests& rq, const void* Q,
                  const void* K, const void* V, const Adapters& ad, void* O, void* ws,
                  size_t ws_bytes, hipStream_t stream, bool expand = false) {
  const int32_t* q_len_arg = decode ? nullptr : rq.q_len;
  Plan p = make_plan(s, decode, q_len_arg, rq.k_len);
  if (p.active.empty()) return ok();
  if (p.ws_bytes > 0) {
    if (!ws) return fail(LRA_ERR_WORKSPACE, "workspace is null; %zu bytes needed", p.ws_bytes);
    if (ws_bytes < p.ws_bytes)
      return fail(LRA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, p.ws_bytes);
  }
  const int G = s.Hq / s.Hkv;
  lra::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  if (p.part_rows) {
    uintptr_t base = (reinterpret_cast<uintptr_t>(ws) + 255) & ~uintptr_t(255);
    a.ws_o = reinterpret_cast<float*>(base);
    a.ws_ml = a.ws_o + p.part_rows * s.D;
  }
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = G;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)s.D));
  for (int i = 0; i < ad.n_agents; ++i) {
    a.agents[i].L = ad.L[i];
    a.agents[i].B = ad.B[i];
    a.agents[i].ldl = ad.ldl[i];
    a.agents[i].rank = ad.ranks[i];
  }
  const size_t n = p.active.size();
  // Units: requests that one work item serves together.  Decode requests whose base rows
  // start at the same row share every K/V tile of the shorter one's rows (one context read
  // by several agents, some of which have seen more of it), so they are grouped, up to
  // kMaxMembers (and 16 / G query columns) per unit, members consecutive in launch order and
  // longest first: the unit streams the first member's rows once, and each member's query
  // columns are masked past its own length.  Members also share their key-split count when
  // planned alone, so the unit's splits fit every member's share of the workspace.  Every
  // other request is a unit of its own.
  std::vector<int> unit_size(n, 1);
  if (decode && s.dtype == LRA_DTYPE_BF16 && !expand && group_decode_enabled()) {
    const int cap = std::min(lra::kMaxMembers, 16 / G);
    bool fits = cap >= 2;
    for (size_t i = 0; i < n && fits; ++i) {
      const int b = p.active[i];
      const int a = rq.agent[b];
      if (ad.ranks[a] > 0 && (int64_t)rq.k_len[b] * ad.ldl[a] * 2 >= ((int64_t)1 << 31))
        fits = false;   // the kernel addresses one request's LR rows with 32-bit offsets
    }
    if (fits) {
      std::map<std::pair<int32_t, int32_t>, std::vector<size_t>> groups;
      std::vector<std::pair<int32_t, int32_t>> first_seen;
      for (size_t i = 0; i < n; ++i) {
        const int b = p.active[i];
        const auto key = std::make_pair(rq.k_start[b], p.n_split[i]);
        auto it = groups.find(key);
        if (it == groups.end()) {
          first_seen.push_back(key);
          groups[key].push_back(i);
        } else {
          it->second.push_back(i);
        }
      }
      for (auto& kv : groups)   // longest first (stable: equal lengths keep batch order)
        std::stable_sort(kv.second.begin(), kv.second.end(), [&](size_t x, size_t y) {
          return rq.k_len[p.active[x]] > rq.k_len[p.active[y]];
        });
      std::vector<size_t> order;
      unit_size.clear();
      for (const auto& key : first_seen) {
        const auto& mem = groups[key];
        for (size_t j = 0; j < mem.size(); j += cap) {
          const size_t cnt = std::min(mem.size() - j, (size_t)cap);
          unit_size.push_back((int)cnt);
          for (size_t k = 0; k < cnt; ++k) order.push_back(mem[j + k]);
        }
      }
      Plan q = p;
      for (size_t i = 0; i < n; ++i) {
        p.active[i] = q.active[order[i]];
        p.n_rt[i] = q.n_rt[order[i]];
        p.n_split[i] = q.n_split[order[i]];
        p.part_base[i] = q.part_base[order[i]];
      }
      // A unit's work item streams its K/V once for every member, so it takes about
      // `members` times the keys of a single request's split: the fixed cost of a work
      // item (first loads in flight, the merge) is spread over more work.  At least two
      // work items per CU remain, and a unit never has more splits than its members would
      // alone, so the workspace size (which the query computes without grouping) and the
      // members' partial-row ranges still hold.
      const int chunk = env_int("LRA_DECODE_CHUNK", 1024);
      std::vector<int> split_u(unit_size.size());
      int64_t items = 0;
      for (size_t u = 0, i = 0; u < unit_size.size(); i += unit_size[u++]) {
        const int64_t kl = rq.k_len[p.active[i]];
        split_u[u] = unit_size[u] < 2 ? p.n_split[i]
                     : (int)std::max<int64_t>(1, std::min<int64_t>(
                           p.n_split[i], ceil_div(kl, (int64_t)chunk * unit_size[u])));
        items += (int64_t)s.Hkv * split_u[u];
      }
      const int64_t min_items = 2 * 256;
      if (items < min_items) {
        const int64_t f = ceil_div(min_items, std::max<int64_t>(items, 1));
        for (size_t u = 0, i = 0; u < unit_size.size(); i += unit_size[u++])
          if (unit_size[u] > 1)
            split_u[u] = (int)std::min<int64_t>(p.n_split[i], (int64_t)split_u[u] * f);
      }
      for (size_t u = 0, i = 0; u < unit_size.size(); i += unit_size[u++])
        for (int k = 0; k < unit_size[u]; ++k) p.n_split[i + k] = split_u[u];
    }
  }
  // bf16 prefill with several requests: longest work items first (their keys per item,
  // ceil(k_len / n_split)), so that the launch does not end on a few long workgroups; the
  // kernel then deals the items round-robin over the XCDs (grid_per_xcd = 0).  The order
  // of requests does not change any result.
  const bool longest_first = !decode && s.dtype == LRA_DTYPE_BF16 && n > 1;
  if (longest_first) {
    std::vector<size_t> ord(n);
    for (size_t i = 0; i < n; ++i) ord[i] = i;
    auto keys = [&](size_t i) { return ceil_div(rq.k_len[p.active[i]], p.n_split[i]); };
    std::stable_sort(ord.begin(), ord.end(), [&](size_t x, size_t y) { return keys(x) > keys(y); });
    Plan q = p;
    for (size_t i = 0; i < n; ++i) {
      p.active[i] = q.active[ord[i]];
      p.n_rt[i] = q.n_rt[ord[i]];
      p.n_split[i] = q.n_split[ord[i]];
      p.part_base[i] = q.part_base[ord[i]];
    }
  }
  const int heads_per_item = s.dtype == LRA_DTYPE_F32 ? s.Hq : s.Hkv;
  size_t c0 = 0, u0 = 0;
  while (c0 < n) {
    // whole units, at most kReqsPerLaunch requests per launch
    size_t c1 = c0, u1 = u0;
    bool shared = false;
    while (u1 < unit_size.size() && c1 - c0 + unit_size[u1] <= (size_t)lra::kReqsPerLaunch) {
      shared |= unit_size[u1] > 1;
      c1 += unit_size[u1++];
    }
    int64_t work = 0, comb = 0;
    a.n_req = (int)(c1 - c0);
    size_t next_leader = c0;
    size_t u = u0;
    for (size_t i = c0; i < c1; ++i) {
      const int b = p.active[i];
      lra::ReqDesc& r = a.reqs[i - c0];
      r.q_start = decode ? b : rq.q_start[b];
      r.q_len = decode ? 1 : rq.q_len[b];
      r.k_start = rq.k_start[b];
      r.k_len = rq.k_len[b];
      r.agent = rq.agent[b];
      r.n_rt = p.n_rt[i];
      r.n_split = p.n_split[i];
      r.part_base = (int)p.part_base[i];
      r.comb_start = (int)comb;
      if (i == next_leader) {   // first member of unit u: owns the unit's work items
        r.work_start = (int)work;
        r.n_members = unit_size[u];
        work += (int64_t)heads_per_item * r.n_rt * r.n_split;
        next_leader += unit_size[u++];
      } else {
        r.work_start = INT32_MAX;
        r.n_members = 0;
      }
      if (r.n_split > 1) comb += (int64_t)r.q_len * s.Hq;
    }
    if (work > INT32_MAX / 2) return fail(LRA_ERR_UNSUPPORTED, "launch too large");
    a.n_work = (int)work;
    a.n_comb = (int)comb;
    hipError_t e;
    if (s.dtype == LRA_DTYPE_BF16) {
      const bool dealt = longest_first && c1 - c0 > 1;
      const int64_t round = dealt ? 8 * lra::kDealChunk : 8;
      const int grid = (int)(ceil_div(work, round) * round);
      a.grid_per_xcd = dealt ? 0 : grid / 8;
      int max_rank = 0, min_rank = LRA_MAX_RANK;
      for (size_t i = c0; i < c1; ++i) {
        max_rank = std::max(max_rank, ad.ranks[rq.agent[p.active[i]]]);
        min_rank = std::min(min_rank, ad.ranks[rq.agent[p.active[i]]]);
      }
      if (!decode)
        e = lra::launch_prefill_bf16(a, s.D, max_rank, grid, stream, expand, min_rank);
      else if (shared)
        e = lra::launch_decode_shared_bf16(a, s.D, max_rank, grid, stream);
      else
        e = lra::launch_decode_bf16(a, s.D, max_rank, grid, stream, expand);
      if (e == hipSuccess && comb > 0) e = lra::launch_combine_bf16(a, s.D, stream);
    } else {
      a.grid_per_xcd = 0;
      e = lra::launch_attn_f32(a, s.D, (int)work, stream);
    }
    if (e != hipSuccess) return fail(LRA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    c0 = c1;
    u0 = u1;
  }
  return ok();
}

// Arguments shared by the LR precompute and the decode-step append (T rows of X), filled
// into `a` on success; *R_out receives the sum of ranks.
int check_lr_args(int dtype, int64_t T, int64_t d_model, const void* X, int64_t ldx,
                  const void* A_cat, int64_t lda, int32_t n_agents, const int32_t* ranks,
                  void* const* L_out, const int64_t* ldl, lra::PrecomputeArgs* a,
                  int64_t* R_out) {
  if (dtype != LRA_DTYPE_F32 && dtype != LRA_DTYPE_BF16)
    return fail(LRA_ERR_INVALID, "dtype %d is neither LRA_DTYPE_F32 nor LRA_DTYPE_BF16", dtype);
  if (T < 0 || d_model <= 0) return fail(LRA_ERR_INVALID, "T %lld < 0 or d_model %lld <= 0",
                                         (long long)T, (long long)d_model);
  if (n_agents <= 0) return fail(LRA_ERR_INVALID, "n_agents %d <= 0", n_agents);
  if (n_agents > LRA_MAX_AGENTS)
    return fail(LRA_ERR_UNSUPPORTED, "n_agents %d > LRA_MAX_AGENTS (%d)", n_agents, LRA_MAX_AGENTS);
  if (!ranks || !L_out || !ldl) return fail(LRA_ERR_INVALID, "ranks, L_out, ldl must be non-null");
  int64_t R = 0;
  for (int i = 0; i < n_agents; ++i) {
    if (ranks[i] < 0) return fail(LRA_ERR_INVALID, "ranks[%d] = %d < 0", i, ranks[i]);
    if (ranks[i] > LRA_MAX_RANK || ranks[i] % 8 != 0)
      return fail(LRA_ERR_UNSUPPORTED, "ranks[%d] = %d: ranks must be multiples of 8 up to %d", i,
                  ranks[i], LRA_MAX_RANK);
    if (ranks[i] > 0) {
      if (!L_out[i]) return fail(LRA_ERR_INVALID, "L_out[%d] is null", i);
      if (ldl[i] < ranks[i]) return fail(LRA_ERR_INVALID, "ldl[%d] < ranks[%d]", i, i);
      if (!aligned(L_out[i], 4)) return fail(LRA_ERR_INVALID, "L_out[%d] not 4-byte aligned", i);
    }
    R += ranks[i];
  }
  if (d_model % 8 != 0) return fail(LRA_ERR_UNSUPPORTED, "d_model %lld %% 8 != 0", (long long)d_model);
  if (dtype == LRA_DTYPE_BF16 && d_model % 64 != 0)
    return fail(LRA_ERR_UNSUPPORTED, "bf16 d_model %lld %% 64 != 0", (long long)d_model);
  if (ldx < d_model || ldx % 8 != 0)
    return fail(LRA_ERR_INVALID, "ldx %lld must be >= d_model and a multiple of 8", (long long)ldx);
  if (lda < R) return fail(LRA_ERR_INVALID, "lda %lld < sum of ranks %lld", (long long)lda,
                           (long long)R);
  *R_out = R;
  if (T == 0 || R == 0) return LRA_OK;
  if (!X || !A_cat) return fail(LRA_ERR_INVALID, "X and A_cat must be non-null");
  if (!aligned(X, 16) || !aligned(A_cat, dtype == LRA_DTYPE_BF16 ? 16 : 4))
    return fail(LRA_ERR_INVALID, "X must be 16-byte aligned, A_cat %d-byte aligned",
                dtype == LRA_DTYPE_BF16 ? 16 : 4);
  if (dtype == LRA_DTYPE_BF16 && (lda % 8 != 0))
    return fail(LRA_ERR_INVALID, "lda %lld must be a multiple of 8 for bf16", (long long)lda);
  if (R > 256) return fail(LRA_ERR_UNSUPPORTED, "sum of ranks %lld > 256", (long long)R);
  // the bf16 kernels address 64 rows of X, or all of A_cat, with 32-bit offsets
  if (dtype == LRA_DTYPE_BF16 && (ldx >= (1 << 24) || d_model * lda * 2 >= ((int64_t)1 << 31)))
    return fail(LRA_ERR_UNSUPPORTED, "bf16 ldx %lld must be below 2^24 and A_cat below 2 GiB",
                (long long)ldx);
  std::memset(a, 0, sizeof(*a));
  a->X = X;
  a->A = A_cat;
  a->T = T;
  a->d_model = d_model;
  a->ldx = ldx;
  a->lda = lda;
  a->R = (int)R;
  a->n_agents = n_agents;
  int32_t off = 0;
  for (int i = 0; i < n_agents; ++i) {
    a->Lout[i] = L_out[i];
    a->ldl[i] = ldl[i];
    a->col_start[i] = off;
    off += ranks[i];
  }
  a->col_start[n_agents] = off;
  return LRA_OK;
}

// The attention entry points; expand selects the in-tile expansion comparator.
int attn_prefill_impl(bool expand, int dtype, int32_t batch, int32_t n_q_heads,
                      int32_t n_kv_heads, int32_t head_dim, const int32_t* q_start,
                      const int32_t* q_len, const int32_t* k_start, const int32_t* k_len,
                      const int32_t* agent_idx, const void* Q, int64_t q_rows,
                      const void* K_base, const void* V_base, int64_t kv_rows,
                      int32_t n_agents, const int32_t* ranks, const void* const* L,
                      const int64_t* ldl, const void* const* B, void* O, void* workspace,
                      size_t workspace_bytes, void* stream) {
  AttnShape s{dtype, batch, n_q_heads, n_kv_heads, head_dim};
  int rc = check_shape(s);
  if (rc) return rc;
  if (expand && dtype != LRA_DTYPE_BF16)
    return fail(LRA_ERR_UNSUPPORTED, "the in-tile expansion variant is bf16 only");
  Adapters ad{n_agents, ranks, L, ldl, B};
  if ((rc = check_adapters(dtype, ad, kv_rows))) return rc;
  Requests rq{q_start, q_len, k_start, k_len, agent_idx};
  if ((rc = check_requests(batch, rq, q_rows, kv_rows, n_agents))) return rc;
  bool any = false;
  for (int b = 0; b < batch; ++b) any |= q_len[b] > 0;
  if (!any) return ok();
  if (!Q || !K_base || !V_base || !O)
    return fail(LRA_ERR_INVALID, "Q, K_base, V_base and O must be non-null");
  if (!aligned(Q, 16) || !aligned(K_base, 16) || !aligned(V_base, 16) || !aligned(O, 16))
    return fail(LRA_ERR_INVALID, "Q, K_base, V_base and O must be 16-byte aligned");
  return run_attention(s, false, rq, Q, K_base, V_base, ad, O, workspace, workspace_bytes,
                       (hipStream_t)stream, expand);
}

int attn_decode_impl(bool expand, int dtype, int32_t batch, int32_t n_q_heads,
                     int32_t n_kv_heads, int32_t head_dim, const int32_t* k_start,
                     const int32_t* k_len, const int32_t* agent_idx, const void* Q,
                     const void* K_base, const void* V_base, int64_t kv_rows, int32_t n_agents,
                     const int32_t* ranks, const void* const* L, const int64_t* ldl,
                     const void* const* B, void* O, void* workspace, size_t workspace_bytes,
                     void* stream) {
  AttnShape s{dtype, batch, n_q_heads, n_kv_heads, head_dim};
  int rc = check_shape(s);
  if (rc) return rc;
  if (expand && dtype != LRA_DTYPE_BF16)
    return fail(LRA_ERR_UNSUPPORTED, "the in-tile expansion variant is bf16 only");
  Adapters ad{n_agents, ranks, L, ldl, B};
  if ((rc = check_adapters(dtype, ad, kv_rows))) return rc;
  if (batch == 0) return ok();
  if (!k_start || !k_len || !agent_idx)
    return fail(LRA_ERR_INVALID, "request arrays must be non-null host arrays");
  std::vector<int32_t> qs(batch), ql(batch, 1);
  for (int b = 0; b < batch; ++b) qs[b] = b;
  Requests rq{qs.data(), ql.data(), k_start, k_len, agent_idx};
  if ((rc = check_requests(batch, rq, batch, kv_rows, n_agents))) return rc;
  if (!Q || !K_base || !V_base || !O)
    return fail(LRA_ERR_INVALID, "Q, K_base, V_base and O must be non-null");
  if (!aligned(Q, 16) || !aligned(K_base, 16) || !aligned(V_base, 16) || !aligned(O, 16))
    return fail(LRA_ERR_INVALID, "Q, K_base, V_base and O must be 16-byte aligned");
  return run_attention(s, true, rq, Q, K_base, V_base, ad, O, workspace, workspace_bytes,
                       (hipStream_t)stream, expand);
}

}  // namespace

namespace lra {
int report_error(int code, const char* msg) { return fail(code, "%s", msg); }

// One bf16 append launch: 64 x 64 output blocks, and d_model cut into slices of whole
// 256-value rounds so that the launch has about kAppendItems workgroups (a slice is never
// shorter than one round).  Every X and A_cat element is read by exactly one workgroup
// when the tokens fit one block and the columns one block (64 tokens, 64 columns).
constexpr int kAppendItems = kAppendMaxSlices;   // so that a launch has at most that many slices
AppendPlan plan_append(int64_t T, int64_t d_model, int64_t R) {
  AppendPlan p;
  const int tbn = (int)ceil_div(T, 64), cbn = (int)ceil_div(R, 64);
  const int nk = (int)(d_model / 32);
  const int rounds = (int)ceil_div(nk, 8);
  const int want = std::max(1, kAppendItems / (tbn * cbn));
  const int per = (int)ceil_div(rounds, std::min(want, rounds));   // rounds per slice
  p.slice_chunks = per * 8;
  p.n_slices = (int)ceil_div(nk, p.slice_chunks);
  p.t_pad = tbn * 64;
  p.r_pad = cbn * 64;
  return p;
}
}  // namespace lra

namespace {
// Workspace of an append call: the largest of its launches' partial buffers (the launches
// run one after another on the call's stream and reuse it).
size_t append_workspace(int32_t batch, int64_t d_model, int64_t R) {
  int64_t most = 0;
  for (int b0 = 0; b0 < batch; b0 += lra::kAppendRows) {
    const int n = std::min(batch - b0, lra::kAppendRows);
    most = std::max(most, lra::plan_append(n, d_model, R).bytes());
  }
  return (size_t)most;
}
}  // namespace

extern "C" {

const char* lra_last_error(void) { return g_err; }

size_t lra_attn_workspace_bytes(int dtype, int is_decode, int32_t batch, const int32_t* q_len,
                                const int32_t* k_len, int32_t n_q_heads, int32_t n_kv_heads,
                                int32_t head_dim, int32_t max_rank) {
  AttnShape s{dtype, batch, n_q_heads, n_kv_heads, head_dim};
  if (check_shape(s) != LRA_OK) return (size_t)-1;
  if (max_rank < 0 || max_rank > LRA_MAX_RANK) return (size_t)-1;
  if (batch > 0 && (!k_len || (!is_decode && !q_len))) return (size_t)-1;
  for (int b = 0; b < batch; ++b) {
    if (k_len[b] < 0 || (!is_decode && (q_len[b] < 0 || q_len[b] > k_len[b]))) return (size_t)-1;
    if (is_decode && k_len[b] < 1) return (size_t)-1;
  }
  return make_plan(s, is_decode != 0, q_len, k_len).ws_bytes;
}

int lra_attn_prefill(int dtype, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                     int32_t head_dim, const int32_t* q_start, const int32_t* q_len,
                     const int32_t* k_start, const int32_t* k_len, const int32_t* agent_idx,
                     const void* Q, int64_t q_rows, const void* K_base, const void* V_base,
                     int64_t kv_rows, int32_t n_agents, const int32_t* ranks,
                     const void* const* L, const int64_t* ldl, const void* const* B, void* O,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return attn_prefill_impl(false, dtype, batch, n_q_heads, n_kv_heads, head_dim, q_start, q_len,
                           k_start, k_len, agent_idx, Q, q_rows, K_base, V_base, kv_rows,
                           n_agents, ranks, L, ldl, B, O, workspace, workspace_bytes, stream);
}

int lra_attn_prefill_expand(int dtype, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, const int32_t* q_start, const int32_t* q_len,
                            const int32_t* k_start, const int32_t* k_len,
                            const int32_t* agent_idx, const void* Q, int64_t q_rows,
                            const void* K_base, const void* V_base, int64_t kv_rows,
                            int32_t n_agents, const int32_t* ranks, const void* const* L,
                            const int64_t* ldl, const void* const* B, void* O, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return attn_prefill_impl(true, dtype, batch, n_q_heads, n_kv_heads, head_dim, q_start, q_len,
                           k_start, k_len, agent_idx, Q, q_rows, K_base, V_base, kv_rows,
                           n_agents, ranks, L, ldl, B, O, workspace, workspace_bytes, stream);
}

int lra_attn_decode(int dtype, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                    int32_t head_dim, const int32_t* k_start, const int32_t* k_len,
                    const int32_t* agent_idx, const void* Q, const void* K_base,
                    const void* V_base, int64_t kv_rows, int32_t n_agents, const int32_t* ranks,
                    const void* const* L, const int64_t* ldl, const void* const* B, void* O,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return attn_decode_impl(false, dtype, batch, n_q_heads, n_kv_heads, head_dim, k_start, k_len,
                          agent_idx, Q, K_base, V_base, kv_rows, n_agents, ranks, L, ldl, B, O,
                          workspace, workspace_bytes, stream);
}

int lra_attn_decode_expand(int dtype, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                           int32_t head_dim, const int32_t* k_start, const int32_t* k_len,
                           const int32_t* agent_idx, const void* Q, const void* K_base,
                           const void* V_base, int64_t kv_rows, int32_t n_agents,
                           const int32_t* ranks, const void* const* L, const int64_t* ldl,
                           const void* const* B, void* O, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return attn_decode_impl(true, dtype, batch, n_q_heads, n_kv_heads, head_dim, k_start, k_len,
                          agent_idx, Q, K_base, V_base, kv_rows, n_agents, ranks, L, ldl, B, O,
                          workspace, workspace_bytes, stream);
}

int lra_expand_values(int dtype, int32_t n_spans, const int32_t* start, const int32_t* len,
                      const int32_t* agent_idx, const void* V_base, int64_t kv_rows,
                      int32_t n_kv_heads, int32_t head_dim, int32_t n_agents,
                      const int32_t* ranks, const void* const* L, const int64_t* ldl,
                      const void* const* B, void* V_full, void* stream) {
  if (dtype != LRA_DTYPE_BF16 && dtype != LRA_DTYPE_F32)
    return fail(LRA_ERR_INVALID, "dtype %d is neither LRA_DTYPE_F32 nor LRA_DTYPE_BF16", dtype);
  if (dtype != LRA_DTYPE_BF16) return fail(LRA_ERR_UNSUPPORTED, "lra_expand_values is bf16 only");
  if (n_spans < 0) return fail(LRA_ERR_INVALID, "n_spans %d < 0", n_spans);
  if (n_spans > LRA_MAX_BATCH)
    return fail(LRA_ERR_UNSUPPORTED, "n_spans %d > LRA_MAX_BATCH (%d)", n_spans, LRA_MAX_BATCH);
  if (n_kv_heads <= 0) return fail(LRA_ERR_INVALID, "n_kv_heads %d <= 0", n_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(LRA_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", head_dim);
  Adapters ad{n_agents, ranks, L, ldl, B};
  int rc = check_adapters(dtype, ad, kv_rows);
  if (rc) return rc;
  if (n_spans == 0) return ok();
  if (!start || !len || !agent_idx)
    return fail(LRA_ERR_INVALID, "span arrays must be non-null host arrays");
  std::vector<std::pair<int64_t, int64_t>> rows;
  for (int i = 0; i < n_spans; ++i) {
    if (start[i] < 0 || len[i] < 0 || (int64_t)start[i] + len[i] > kv_rows)
      return fail(LRA_ERR_INVALID, "span %d: rows [%d, %lld) outside [0, %lld)", i, start[i],
                  (long long)start[i] + len[i], (long long)kv_rows);
    if (agent_idx[i] < 0 || agent_idx[i] >= n_agents)
      return fail(LRA_ERR_INVALID, "span %d: agent_idx %d outside [0, %d)", i, agent_idx[i],
                  n_agents);
    if (len[i] > 0) rows.emplace_back(start[i], (int64_t)start[i] + len[i]);
  }
  std::sort(rows.begin(), rows.end());
  for (size_t i = 1; i < rows.size(); ++i)
    if (rows[i].first < rows[i - 1].second)
      return fail(LRA_ERR_INVALID, "two spans overlap at row %lld", (long long)rows[i].first);
  if (rows.empty()) return ok();
  if (!V_base || !V_full) return fail(LRA_ERR_INVALID, "V_base and V_full must be non-null");
  if (!aligned(V_base, 16) || !aligned(V_full, 16))
    return fail(LRA_ERR_INVALID, "V_base and V_full must be 16-byte aligned");
  lra::ExpandArgs a;
  std::memset(&a, 0, sizeof(a));
  a.V = V_base;
  a.Vout = V_full;
  a.Hkv = n_kv_heads;
  for (int i = 0; i < n_agents; ++i) {
    a.agents[i].L = L[i];
    a.agents[i].B = B[i];
    a.agents[i].ldl = ldl[i];
    a.agents[i].rank = ranks[i];
  }
  // rows per work item: enough items to cover the CUs several times over (at least 2048
  // when the rows allow it), at most kExpandRows, in whole 32-row tiles
  int64_t total_rows = 0;
  for (int i = 0; i < n_spans; ++i) total_rows += len[i];
  const int64_t want = ceil_div(total_rows * n_kv_heads, 2048);
  a.rows_per_item = (int)std::min<int64_t>(lra::kExpandRows, std::max<int64_t>(32, ceil_div(want, 32) * 32));
  int i0 = 0;
  while (i0 < n_spans) {
    int64_t work = 0;
    int n = 0, max_rank = 0;
    for (; i0 < n_spans && n < lra::kReqsPerLaunch; ++i0) {
      if (len[i0] == 0) continue;
      lra::ExpandSpan& sp = a.spans[n++];
      sp.start = start[i0];
      sp.len = len[i0];
      sp.agent = agent_idx[i0];
      sp.work_start = (int)work;
      work += ceil_div(len[i0], a.rows_per_item) * n_kv_heads;
      max_rank = std::max(max_rank, ranks[agent_idx[i0]]);
    }
    if (n == 0) break;
    if (work > INT32_MAX / 2) return fail(LRA_ERR_UNSUPPORTED, "launch too large");
    a.n_span = n;
    a.n_work = (int)work;
    hipError_t e = lra::launch_expand_bf16(a, head_dim, max_rank, (hipStream_t)stream);
    if (e != hipSuccess) return fail(LRA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

int lra_precompute_lr(int dtype, int64_t T, int64_t d_model, const void* X, int64_t ldx,
                      const void* A_cat, int64_t lda, int32_t n_agents, const int32_t* ranks,
                      void* const* L_out, const int64_t* ldl, void* stream) {
  lra::PrecomputeArgs a;
  int64_t R = 0;
  int rc = check_lr_args(dtype, T, d_model, X, ldx, A_cat, lda, n_agents, ranks, L_out, ldl,
                         &a, &R);
  if (rc != LRA_OK) return rc;
  if (T == 0 || R == 0) return ok();
  hipError_t e = dtype == LRA_DTYPE_BF16 ? lra::launch_precompute_bf16(a, (hipStream_t)stream)
                                         : lra::launch_precompute_f32(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(LRA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int lra_append_lr(int dtype, int32_t batch, int64_t d_model, const void* X, int64_t ldx,
                  const void* A_cat, int64_t lda, int32_t n_agents, const int32_t* ranks,
                  void* const* L_out, const int64_t* ldl, const int32_t* rows, int64_t l_rows,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 0) return fail(LRA_ERR_INVALID, "batch %d < 0", batch);
  if (batch > LRA_MAX_BATCH)
    return fail(LRA_ERR_UNSUPPORTED, "batch %d > LRA_MAX_BATCH (%d)", batch, LRA_MAX_BATCH);
  lra::AppendArgs a;
  std::memset(&a, 0, sizeof(a));
  int64_t R = 0;
  int rc = check_lr_args(dtype, batch, d_model, X, ldx, A_cat, lda, n_agents, ranks, L_out, ldl,
                         &a.p, &R);
  if (rc != LRA_OK) return rc;
  if (batch == 0) return ok();
  if (!rows) return fail(LRA_ERR_INVALID, "rows must be a non-null host array");
  std::vector<int32_t> sorted(rows, rows + batch);
  std::sort(sorted.begin(), sorted.end());
  for (int b = 0; b < batch; ++b) {
    if (sorted[b] < 0 || sorted[b] >= l_rows)
      return fail(LRA_ERR_INVALID, "rows: %d outside [0, %lld)", sorted[b], (long long)l_rows);
    if (b > 0 && sorted[b] == sorted[b - 1])
      return fail(LRA_ERR_INVALID, "rows: row %d appears twice", sorted[b]);
  }
  if (R == 0) return ok();
  const bool bf16 = dtype == LRA_DTYPE_BF16;
  const size_t need = bf16 ? append_workspace(batch, d_model, R) : 0;
  if (need > 0 && !workspace)
    return fail(LRA_ERR_WORKSPACE, "workspace is null; %zu bytes needed", need);
  if (workspace_bytes < need)
    return fail(LRA_ERR_WORKSPACE, "workspace of %zu bytes < %zu needed", workspace_bytes, need);
  if (need > 0 && !aligned(workspace, 16))
    return fail(LRA_ERR_INVALID, "workspace must be 16-byte aligned");
  const char* Xb = static_cast<const char*>(X);
  const int64_t esz = bf16 ? 2 : 4;
  for (int b0 = 0; b0 < batch; b0 += lra::kAppendRows) {
    const int n = std::min(batch - b0, lra::kAppendRows);
    a.p.X = Xb + (int64_t)b0 * ldx * esz;
    a.p.T = n;
    for (int i = 0; i < n; ++i) a.rows[i] = rows[b0 + i];
    if (bf16) {
      const lra::AppendPlan pl = lra::plan_append(n, d_model, R);
      a.part = static_cast<float*>(workspace);
      a.n_slices = pl.n_slices;
      a.slice_chunks = pl.slice_chunks;
      a.t_pad = pl.t_pad;
      a.r_pad = pl.r_pad;
    }
    hipError_t e = bf16 ? lra::launch_append_bf16(a, (hipStream_t)stream)
                        : lra::launch_append_f32(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(LRA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

size_t lra_append_workspace_bytes(int dtype, int32_t batch, int64_t d_model, int32_t n_agents,
                                  const int32_t* ranks) {
  if ((dtype != LRA_DTYPE_F32 && dtype != LRA_DTYPE_BF16) || batch < 0 ||
      batch > LRA_MAX_BATCH || d_model <= 0 || n_agents <= 0 || n_agents > LRA_MAX_AGENTS ||
      !ranks)
    return (size_t)-1;
  // the rank and size rules of lra_append_lr, so that no size is given for a call it refuses
  int64_t R = 0;
  for (int i = 0; i < n_agents; ++i) {
    if (ranks[i] < 0 || ranks[i] > LRA_MAX_RANK || ranks[i] % 8 != 0) return (size_t)-1;
    R += ranks[i];
  }
  if (R > 256 || d_model % 8 != 0 || (dtype == LRA_DTYPE_BF16 && d_model % 64 != 0))
    return (size_t)-1;
  if (dtype != LRA_DTYPE_BF16 || batch == 0 || R == 0) return 0;
  return append_workspace(batch, d_model, R);
}

}  // extern "C"
