// Internal interface between the C-ABI front end (lra_api.cpp) and the HIP kernels.
// Kernel arguments are passed by value; per-request and per-agent tables live inside the
// argument block and kernels read them through the kernarg segment pointer, so nothing
// has to be copied to device memory before a launch.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace lra {

constexpr int kMaxAgents = 16;
constexpr int kMaxRank = 64;
constexpr int kReqsPerLaunch = 64;   // larger batches are split into several launches

// Tile geometry of the bf16 attention kernel (see fla_bf16.hip).
constexpr int kTileRows = 128;       // (query, head-in-group) rows per workgroup
constexpr int kTileKeys = 64;        // keys per LDS tile
constexpr int kPrefillRows = 256;    // rows per workgroup of the ping-pong prefill kernel
constexpr int kThreads = 256;        // 4 waves of 64

struct AgentDesc {
  const void* L;      // [kv_rows, ldl] LR cache (device)
  const void* B;      // [rank, Hkv*D] up-projection (device)
  int64_t ldl;        // row stride of L in elements
  int32_t rank;
  int32_t pad_;
};

// One request of a launch.  In the prefill kernel the work items of a request are
// numbered ((g * n_split + split) * n_rt + rt) with rt (row tile) fastest; in the decode
// kernel (n_rt = 1) they are numbered (split * Hkv + g).
struct ReqDesc {
  int32_t q_start, q_len, k_start, k_len;
  int32_t agent;
  int32_t n_rt;        // row tiles per kv head
  int32_t n_split;     // key-range splits (1: the attention kernel writes O directly)
  int32_t work_start;  // first work item of this request within the launch
  int32_t part_base;   // first partial row in the workspace (split requests), else -1
  int32_t comb_start;  // first combine row of this request within the launch
  // Shared-context decode: requests that read the same base rows are grouped into units
  // of consecutive entries.  The first entry of a unit owns its work items and holds the
  // member count; the other members hold 0 here and work_start = INT32_MAX.
  int32_t n_members;
};

// Members per unit of the shared-context decode kernel (at most 16 / G: the members'
// query heads share the 16 columns of one MFMA tile).
constexpr int kMaxMembers = 4;

// Consecutive work items per XCD turn in the longest-first prefill mapping (grid_per_xcd
// == 0); the grid is then a multiple of 8 * kDealChunk.
constexpr int kDealChunk = 4;

struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* ws_o;         // [part_rows, D]  unnormalised P·V_base + (P·L)·B of a key split
  float* ws_ml;        // [part_rows, 2]  (running max in log2 units, row sum)
  int32_t Hq, Hkv, G;
  int32_t n_req;
  int32_t n_work;      // work items (workgroups that do work) in this launch
  // Workgroup -> work item.  > 0: XCD-major, XCD x (blockIdx % 8) takes the contiguous
  // items [x * grid_per_xcd, (x + 1) * grid_per_xcd), so the items of one kv head share
  // that XCD's L2.  0 (bf16 prefill with several requests, sorted longest first): the items
  // are dealt round-robin over the XCDs in chunks of kDealChunk, so every XCD starts on
  // long items and ends on short ones.
  int32_t grid_per_xcd;
  int32_t n_comb;      // combine rows in this launch
  float scale_log2;    // log2(e) / sqrt(D)
  AgentDesc agents[kMaxAgents];
  ReqDesc reqs[kReqsPerLaunch];
};

// Precompute: L_a[t, :] = X[t, :] · A_cat[:, off_a : off_a + r_a].
struct PrecomputeArgs {
  const void* X;
  const void* A;
  int64_t T, d_model, ldx, lda;
  int32_t R;           // total columns (sum of ranks)
  int32_t n_agents;
  int32_t n_row_tiles;
  int32_t grid_per_xcd;
  void* Lout[kMaxAgents];
  int64_t ldl[kMaxAgents];
  int32_t col_start[kMaxAgents + 1];
};

// Decode-step append: the LR rows of up to kAppendRows new tokens per launch.  Token t of
// the launch goes to row rows[t] of every agent's cache.  bf16: d_model is cut into
// n_slices slices of slice_chunks 32-value chunks; slice s leaves its fp32 partial sums in
// part[s][t][c] ([n_slices][t_pad][r_pad] in the workspace, t_pad and r_pad multiples of 64).
constexpr int kAppendRows = 256;
constexpr int kAppendMaxSlices = 16;
struct AppendArgs {
  PrecomputeArgs p;    // X holds the launch's tokens (T of them), A_cat, the agents' caches
  float* part;
  int32_t n_slices, slice_chunks, t_pad, r_pad;
  int32_t rows[kAppendRows];
};
// The split of one bf16 append launch of T tokens (T <= kAppendRows) and R columns.
struct AppendPlan {
  int32_t n_slices, slice_chunks, t_pad, r_pad;
  int64_t bytes() const { return (int64_t)n_slices * t_pad * r_pad * 4; }
};
AppendPlan plan_append(int64_t T, int64_t d_model, int64_t R);

// Naive value expansion (the comparator of the regrouped kernels): span i covers rows
// [start, start + len) of V_base, expanded with agent `agent`'s L and B into the same rows
// of V_full.  Work items: (chunk of rows_per_item rows, kv head) with the kv head fastest;
// rows_per_item is a multiple of 32 up to kExpandRows.
constexpr int kExpandRows = 512;
struct ExpandSpan {
  int64_t start;
  int32_t len, agent, work_start, pad_;
};
struct ExpandArgs {
  const void* V;
  void* Vout;
  int32_t Hkv, n_span, n_work, rows_per_item;
  AgentDesc agents[kMaxAgents];
  ExpandSpan spans[kReqsPerLaunch];
};

// Sets the calling thread's lra_last_error() message and returns `code`.
int report_error(int code, const char* msg);

// Launchers (return the HIP status of the launch).
// min_rank: the smallest rank among the launch's requests (-1: not known); a launch whose
// ranks span LR widths runs each work item at its own width.
hipError_t launch_prefill_bf16(const AttnArgs& a, int head_dim, int max_rank, int n_grid,
                               hipStream_t s, bool expand = false, int min_rank = -1);
hipError_t launch_decode_shared_bf16(const AttnArgs& a, int head_dim, int max_rank, int n_grid,
                                     hipStream_t s);
// expand: the in-tile expansion comparator (each V_base tile expanded with L·B_g in LDS
// before P·V) instead of the regrouped LR term.
hipError_t launch_decode_bf16(const AttnArgs& a, int head_dim, int max_rank, int n_grid,
                              hipStream_t s, bool expand = false);
hipError_t launch_combine_bf16(const AttnArgs& a, int head_dim, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, int n_blocks, hipStream_t s);
hipError_t launch_precompute_bf16(const PrecomputeArgs& a, hipStream_t s);
hipError_t launch_precompute_f32(const PrecomputeArgs& a, hipStream_t s);
hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t s);
hipError_t launch_append_f32(const AppendArgs& a, hipStream_t s);
hipError_t launch_expand_bf16(const ExpandArgs& a, int head_dim, int max_rank, hipStream_t s);

}  // namespace lra
