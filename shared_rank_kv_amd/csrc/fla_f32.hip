// Flash-LoRA-Attention, fp32 storage and fp32 arithmetic throughout (no reduced precision),
// for gfx950.  Same computation as the bf16 path (LRAgent summary, section
// "3. Flash-LoRA-Attention": O = P·V_base + (P·L_a)·B_a with one online softmax), written
// as a plain kernel: it serves exactness checks, not throughput.
//
// Workgroup = 256 threads = 16 query rows of one (request, q head) x 4 head_dim quarters x
// 4 key groups: thread (row, quarter, group) holds a quarter of the row's query and output
// lanes and of its LR accumulator, and runs its own online softmax over the keys
// k = 4 j + group (eight at a time), reading K, V_base and L straight from memory (L2).
// The four key groups' states of a row are merged through LDS at the end (weights
// exp(m_g - M)), then B_g is applied once.  Scores use accurate expf.
#include "lra_device.h"

namespace lra {
namespace {

constexpr int kF32Rows = 16;

template <int D>
__global__ __launch_bounds__(256) void fla_attn_f32(const AttnArgs args) {
  const AttnArgs* A = (const AttnArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int DP = D / 4;            // head_dim lanes per thread
  constexpr int RP = 16;               // LR lanes per thread (rank <= 64)
  constexpr int NK = 8;                // keys per step of a thread
  __shared__ float st_acc[4][kF32Rows][D];
  __shared__ float st_l[4][kF32Rows][64];
  __shared__ float st_ml[4][kF32Rows][2];

  const int w = blockIdx.x;
  const int b = find_request(A, w);
  const ReqDesc& R = A->reqs[b];
  const int local = w - R.work_start;
  const int rt = local % R.n_rt, h = local / R.n_rt;
  const int Hq = A->Hq, Hkv = A->Hkv, G = A->G, g = h / G;
  const int Lq = R.q_len, Lk = R.k_len;
  const AgentDesc& AG = A->agents[R.agent];
  const int rank = AG.rank;
  const float* Lsrc = rank ? (const float*)AG.L + (int64_t)R.k_start * AG.ldl : nullptr;

  const int tid = threadIdx.x;
  const int r = tid & 15, q4 = (tid >> 4) & 3, kg = tid >> 6;   // row, quarter, key group
  const int t = rt * kF32Rows + r;
  const bool valid = t < Lq;
  const int pos = valid ? Lk - Lq + t : -1;   // last visible key (none for padding rows)
  const float scale = 1.0f / sqrtf((float)D);
  const int64_t kv_stride = (int64_t)Hkv * D;
  const float* Kg = (const float*)A->K + ((int64_t)R.k_start * Hkv + g) * D + q4 * DP;
  const float* Vg = (const float*)A->V + ((int64_t)R.k_start * Hkv + g) * D + q4 * DP;

  float q[DP], acc[DP], accl[RP];
  const float* qrow = (const float*)A->Q + ((int64_t)(R.q_start + t) * Hq + h) * D + q4 * DP;
#pragma unroll
  for (int i = 0; i < DP; i += 4) {
    const float4 v = valid ? *(const float4*)(qrow + i) : float4{0.f, 0.f, 0.f, 0.f};
    q[i] = v.x, q[i + 1] = v.y, q[i + 2] = v.z, q[i + 3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < DP; ++i) acc[i] = 0.f;
#pragma unroll
  for (int i = 0; i < RP; ++i) accl[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  // the workgroup's last visible key bounds every thread's loop (uniform trip count; the
  // four quarter-threads of a row must meet in the same shuffles)
  const int t_last = min(rt * kF32Rows + kF32Rows - 1, Lq - 1);
  const int kend = Lk - Lq + t_last + 1;
  for (int k0 = 0; k0 < kend; k0 += 4 * NK) {
    float sc[NK];
    float mx = m;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int key = k0 + 4 * j + kg;
      const bool in = key < kend;
      const float* kr = Kg + (int64_t)(in ? key : 0) * kv_stride;
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < DP; i += 4) {
        const float4 kv = *(const float4*)(kr + i);
        part = fmaf(q[i], kv.x, part);
        part = fmaf(q[i + 1], kv.y, part);
        part = fmaf(q[i + 2], kv.z, part);
        part = fmaf(q[i + 3], kv.w, part);
      }
      // sum over the row's four quarters (lanes 16 apart within the wave)
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      const float v = key <= pos ? part * scale : -INFINITY;
      sc[j] = v;
      mx = fmaxf(mx, v);
    }
    if (mx == -INFINITY) continue;     // nothing visible yet (uniform per row)
    const float alpha = m == -INFINITY ? 0.f : expf(m - mx);
    m = mx;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < DP; ++i) acc[i] *= alpha;
#pragma unroll
    for (int i = 0; i < RP; ++i) accl[i] *= alpha;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int key = k0 + 4 * j + kg;
      if (sc[j] == -INFINITY) continue;
      const float pj = expf(sc[j] - m);
      l += pj;
      const float* vr = Vg + (int64_t)key * kv_stride;
#pragma unroll
      for (int i = 0; i < DP; i += 4) {
        const float4 vv = *(const float4*)(vr + i);
        acc[i] = fmaf(pj, vv.x, acc[i]);
        acc[i + 1] = fmaf(pj, vv.y, acc[i + 1]);
        acc[i + 2] = fmaf(pj, vv.z, acc[i + 2]);
        acc[i + 3] = fmaf(pj, vv.w, acc[i + 3]);
      }
      if (rank > q4 * RP) {   // this quarter's LR columns q4*16 .. +16 (zero past the rank)
        const float* lr = Lsrc + (int64_t)key * AG.ldl + q4 * RP;
#pragma unroll
        for (int i = 0; i < RP; i += 4) {
          const float4 lv = q4 * RP + i < rank ? *(const float4*)(lr + i)
                                               : float4{0.f, 0.f, 0.f, 0.f};
          accl[i] = fmaf(pj, lv.x, accl[i]);
          accl[i + 1] = fmaf(pj, lv.y, accl[i + 1]);
          accl[i + 2] = fmaf(pj, lv.z, accl[i + 2]);
          accl[i + 3] = fmaf(pj, lv.w, accl[i + 3]);
        }
      }
    }
  }

  // merge the four key groups of each row: O = Σ_g e^(m_g - M) acc_g / Σ_g e^(m_g - M) l_g
#pragma unroll
  for (int i = 0; i < DP; ++i) st_acc[kg][r][q4 * DP + i] = acc[i];
#pragma unroll
  for (int i = 0; i < RP; ++i) st_l[kg][r][q4 * RP + i] = accl[i];
  if (q4 == 0) {
    st_ml[kg][r][0] = m;
    st_ml[kg][r][1] = l;
  }
  __syncthreads();
  if (kg != 0 || !valid) return;
  float M = -INFINITY;
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) M = fmaxf(M, st_ml[gg][r][0]);
  float wgt[4], lt = 0.f;
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) {
    wgt[gg] = st_ml[gg][r][0] == -INFINITY ? 0.f : expf(st_ml[gg][r][0] - M);
    lt += wgt[gg] * st_ml[gg][r][1];
  }
  float out[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    float v = 0.f;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) v = fmaf(wgt[gg], st_acc[gg][r][q4 * DP + i], v);
    out[i] = v;
  }
  // epilogue: O = (acc + accl · B_g) / l, B applied once to the merged LR term
  const float* Bg = (const float*)AG.B + g * D + q4 * DP;
  for (int rho = 0; rho < rank; ++rho) {
    float c = 0.f;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) c = fmaf(wgt[gg], st_l[gg][r][rho], c);
    const float* brow = Bg + (int64_t)rho * kv_stride;
#pragma unroll
    for (int i = 0; i < DP; ++i) out[i] = fmaf(c, brow[i], out[i]);
  }
  const float inv = 1.f / lt;
  float* orow = (float*)A->O + ((int64_t)(R.q_start + t) * Hq + h) * D + q4 * DP;
#pragma unroll
  for (int i = 0; i < DP; ++i) orow[i] = out[i] * inv;
}

}  // namespace

hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, int n_blocks, hipStream_t s) {
  if (head_dim == 128)
    hipLaunchKernelGGL(fla_attn_f32<128>, dim3(n_blocks), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(fla_attn_f32<64>, dim3(n_blocks), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace lra
