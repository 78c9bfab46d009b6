// Flash-LoRA-Attention, fp32 storage and fp32 arithmetic throughout (no reduced precision),
// for gfx950.  Same computation as the bf16 path (LRAgent summary, section
// "3. Flash-LoRA-Attention": O = P·V_base + (P·L_a)·B_a with one online softmax), written
// as a plain tiled kernel: it serves exactness checks, not throughput.
//
// Workgroup = 256 threads = 64 query rows of one (request, q head) x 4 threads per row;
// each thread holds a quarter of the row's head_dim lanes and of its LR accumulator.
// K/V_base/L tiles of 32 keys are staged in LDS; scores use accurate expf.
#include "lra_device.h"

namespace lra {
namespace {

template <int D>
__global__ __launch_bounds__(256) void fla_attn_f32(const AttnArgs args) {
  const AttnArgs* A = (const AttnArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int DP = D / 4;            // head_dim lanes per thread
  constexpr int RP = 16;               // LR lanes per thread (rank <= 64)
  constexpr int TK = 32;               // keys per tile
  __shared__ float Ks[TK][D];
  __shared__ float Vs[TK][D];
  __shared__ float Ls[TK][64];
  __shared__ float rowL[64][65];

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

  const int tid = threadIdx.x, r = tid >> 2, sub = tid & 3;
  const int t = rt * 64 + r;
  const bool valid = t < Lq;
  const int pos = valid ? Lk - Lq + t : Lk - 1;
  const int t_last = min(rt * 64 + 63, Lq - 1);
  const int kend = Lk - Lq + t_last + 1;
  const float scale = 1.0f / sqrtf((float)D);

  float q[DP], acc[DP], accl[RP];
  const float* qrow = (const float*)A->Q + ((int64_t)(R.q_start + t) * Hq + h) * D + sub * DP;
#pragma unroll
  for (int i = 0; i < DP; ++i) {
    q[i] = valid ? qrow[i] : 0.f;
    acc[i] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < RP; ++i) accl[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int k0 = 0; k0 < kend; k0 += TK) {
    __syncthreads();
    for (int e = tid; e < TK * D; e += 256) {
      const int kk = e / D, d = e % D;
      const int key = k0 + kk;
      const bool in = key < kend;
      const int64_t off = ((int64_t)(R.k_start + key) * Hkv + g) * D + d;
      Ks[kk][d] = in ? ((const float*)A->K)[off] : 0.f;
      Vs[kk][d] = in ? ((const float*)A->V)[off] : 0.f;
    }
    for (int e = tid; e < TK * 64; e += 256) {
      const int kk = e / 64, c = e % 64;
      const int key = k0 + kk;
      Ls[kk][c] = (key < kend && c < rank) ? Lsrc[(int64_t)key * AG.ldl + c] : 0.f;
    }
    __syncthreads();
    float sc[TK];
    float mx = m;
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < DP; ++i) part = fmaf(q[i], Ks[kk][sub * DP + i], part);
      part += __shfl_xor(part, 1);
      part += __shfl_xor(part, 2);
      float v = part * scale;
      if (k0 + kk > pos) v = -INFINITY;
      sc[kk] = v;
      mx = fmaxf(mx, v);
    }
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mx);
    m = mx;
    l *= alpha;
#pragma unroll
    for (int i = 0; i < DP; ++i) acc[i] *= alpha;
#pragma unroll
    for (int i = 0; i < RP; ++i) accl[i] *= alpha;
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      const float p = (sc[kk] == -INFINITY) ? 0.f : expf(sc[kk] - m);
      l += p;
#pragma unroll
      for (int i = 0; i < DP; ++i) acc[i] = fmaf(p, Vs[kk][sub * DP + i], acc[i]);
#pragma unroll
      for (int i = 0; i < RP; ++i) accl[i] = fmaf(p, Ls[kk][sub * RP + i], accl[i]);
    }
  }

  // epilogue: O = acc / l + (accl / l) · B_g
#pragma unroll
  for (int i = 0; i < RP; ++i) rowL[r][sub * RP + i] = accl[i];
  __syncthreads();
  if (!valid) return;
  const float inv = 1.f / l;
  float out[DP];
#pragma unroll
  for (int i = 0; i < DP; ++i) out[i] = acc[i];
  const float* Bg = (const float*)AG.B + g * D + sub * DP;
  for (int rho = 0; rho < rank; ++rho) {
    const float c = rowL[r][rho];
    const float* brow = Bg + (int64_t)rho * Hkv * D;
#pragma unroll
    for (int i = 0; i < DP; ++i) out[i] = fmaf(c, brow[i], out[i]);
  }
  float* orow = (float*)A->O + ((int64_t)(R.q_start + t) * Hq + h) * D + sub * DP;
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
