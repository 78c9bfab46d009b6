// lra_attn_decode_noalloc: lra_attn_decode with its split-key scratch in a fixed device
// array of this library, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// `scratch` is a file-scope device array: in host code its name is a host-side stand-in,
// never a device address.  The first call on a device, with that device current, looks up
// the array's address there with hipGetSymbolAddress and keeps it per device; every later
// call on that device passes that address to the kernels as their workspace.  Each device
// holds its own copy of the array until the process ends.
#include <cstdio>
#include <mutex>

#include "lra.h"
#include "lra_internal.h"

namespace {

constexpr size_t kScratchBytes = (size_t)LRA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch`, per device (null: not yet)

// Address of this device's copy of `scratch` (nullptr and a message on failure).
void* device_scratch(char* msg, size_t n) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    snprintf(msg, n, "hipGetDevice failed: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    snprintf(msg, n, "device %d is beyond the %d devices this library tracks", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      snprintf(msg, n, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
               hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int lra_attn_decode_noalloc(int dtype, int32_t batch, int32_t n_q_heads,
                                       int32_t n_kv_heads, int32_t head_dim,
                                       const int32_t* k_start, const int32_t* k_len,
                                       const int32_t* agent_idx, const void* Q,
                                       const void* K_base, const void* V_base, int64_t kv_rows,
                                       int32_t n_agents, const int32_t* ranks,
                                       const void* const* L, const int64_t* ldl,
                                       const void* const* B, void* O, void* stream) {
  int max_rank = 0;
  if (ranks && n_agents > 0 && n_agents <= LRA_MAX_AGENTS)
    for (int a = 0; a < n_agents; ++a) max_rank = ranks[a] > max_rank ? ranks[a] : max_rank;
  const size_t need = lra_attn_workspace_bytes(dtype, 1, batch, nullptr, k_len, n_q_heads,
                                               n_kv_heads, head_dim, max_rank);
  char msg[256];
  if (need != (size_t)-1 && need > kScratchBytes) {
    snprintf(msg, sizeof(msg),
             "this decode needs %zu bytes of split-key scratch, more than the %zu bytes of the "
             "library's fixed scratch; call lra_attn_decode with a workspace instead",
             need, kScratchBytes);
    return lra::report_error(LRA_ERR_WORKSPACE, msg);
  }
  // (invalid arguments make the query return (size_t)-1; lra_attn_decode reports why)
  void* ws = device_scratch(msg, sizeof(msg));
  if (!ws) return lra::report_error(LRA_ERR_HIP, msg);
  return lra_attn_decode(dtype, batch, n_q_heads, n_kv_heads, head_dim, k_start, k_len,
                         agent_idx, Q, K_base, V_base, kv_rows, n_agents, ranks, L, ldl, B, O,
                         ws, kScratchBytes, stream);
}
