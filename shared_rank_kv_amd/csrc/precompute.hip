// PreLRShared LR precompute for gfx950: L_a = X·A_a for every agent in one pass over X
// (PReCache abstract on the arxivdaily page, PreLRShared; LRAgent summary, section 2: the
// LR cache holds the LoRA down-projection activations X·A_i).
//
// bf16 path: a tall-skinny GEMM L_cat[T, R] = X[T, d_model]·A_cat[d_model, R] with
// R = sum of ranks <= 256.  The work is bound by reading X once from HBM (R = 192 gives
// ~180 FLOP per byte, under the MI355X ridge), so every workgroup owns 128 rows of X and
// ALL R columns, and X never passes through LDS: each lane loads its MFMA A-operand
// fragment (8 consecutive d_model values of one row) straight from HBM into registers,
// two 64-wide d_model chunks ahead of use.  A_cat chunks (64 x R) are shared by the
// workgroup through a padded LDS tile and read as B operands with ds_read_b64_tr_b16.
// Four waves split the 128 x R tile 2 x 2 (64 rows x R/2 columns each) with
// v_mfma_f32_32x32x16_bf16; the epilogue rounds to bf16 and scatters column blocks to
// each agent's L_a.
//
// fp32 path: a plain LDS-tiled fp32 GEMM (exactness, not throughput).
#include "lra_internal.h"

namespace lra {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr int KC = 64;          // d_model chunk
constexpr int TM = 128;         // rows per workgroup

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 join(i16x4 lo, i16x4 hi) {
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int NBW>
__global__ __launch_bounds__(256, 1) void lr_precompute_bf16(const PrecomputeArgs args) {
  const PrecomputeArgs* P = (const PrecomputeArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int NBT = 2 * NBW;                 // 32-column blocks in the padded tile
  constexpr int RS = NBT * 32 * 2 + 16;        // LDS row stride (bytes), padded
  constexpr int CHUNKS = KC * NBT * 4;         // 16-byte chunks of one A_cat tile
  constexpr int CPT = CHUNKS / 256;            // per thread (= NBT)
  __shared__ __attribute__((aligned(16))) char smem_raw[2 * KC * RS];
  LDS char* smem = (LDS char*)smem_raw;

  const int tile = blockIdx.x;
  const int64_t row0 = (int64_t)tile * TM;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int hi = lane >> 5;
  const int64_t T = P->T, dm = P->d_model, ldx = P->ldx, lda = P->lda;
  const int R = P->R;
  const int nk = (int)((dm + KC - 1) / KC);
  const bf16* X = (const bf16*)P->X;
  const bf16* Ac = (const bf16*)P->A;

  // X fragments: xs[stage][mb][ks], lane = (row lane&31 of m-block mb, k-half hi)
  bf16x8 xs[3][2][4];
  int64_t xrow[2];
  bool xok[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int64_t r = row0 + wm * 64 + mb * 32 + (lane & 31);
    xok[mb] = r < T;
    xrow[mb] = xok[mb] ? r : 0;
  }
  auto load_x = [&](bf16x8 (&dst)[2][4], int kc) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int64_t k = (int64_t)kc * KC + ks * 16 + hi * 8;
        dst[mb][ks] = (xok[mb] && k < dm) ? *(const bf16x8*)(X + xrow[mb] * ldx + k) : bf16x8{};
      }
  };
  u32x4 areg[CPT];
  auto load_a = [&](int kc) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + 256 * i;
      const int k = ch / (NBT * 4), c = ch % (NBT * 4);
      const int64_t kk = (int64_t)kc * KC + k;
      areg[i] = (kk < dm && c * 8 < R) ? *(const u32x4*)(Ac + kk * lda + c * 8) : u32x4{};
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + 256 * i;
      const int k = ch / (NBT * 4), c = ch % (NBT * 4);
      *(LDS u32x4*)(smem + buf * KC * RS + k * RS + c * 16) = areg[i];
    }
  };

  f32x16 acc[2][NBW];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x16{};

  load_a(0);
  load_x(xs[0], 0);
  if (nk > 1) load_x(xs[1], 1);
  store_a(0);
  __syncthreads();

  const int g16 = lane >> 4, jj = lane & 15;
  for (int kc0 = 0; kc0 < nk; kc0 += 3) {
#pragma unroll
    for (int st = 0; st < 3; ++st) {
      const int kc = kc0 + st;
      if (kc < nk) {
        if (kc + 2 < nk) load_x(xs[(st + 2) % 3], kc + 2);
        if (kc + 1 < nk) load_a(kc + 1);
        const LDS char* at = smem + (kc & 1) * KC * RS;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) {
            const int n = (wn * NBW + nb) * 32 + (g16 & 1) * 16 + (jj & 3) * 4;
            const int k = ks * 16 + (g16 >> 1) * 8 + (jj >> 2);
            i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(at + k * RS + n * 2));
            i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(at + (k + 4) * RS + n * 2));
            const bf16x8 bf = join(lo, hi4);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) acc[mb][nb] = mfma32(xs[st][mb][ks], bf, acc[mb][nb]);
          }
        }
        if (kc + 1 < nk) {
          store_a((kc + 1) & 1);
        }
        __syncthreads();
      }
    }
  }

  // epilogue: round to bf16 and scatter columns to their agent's LR cache
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    const int colg = (wn * NBW + nb) * 32 + (lane & 31);
    if (colg >= R) continue;
    int a = 0;
    while (a + 1 < P->n_agents && P->col_start[a + 1] <= colg) ++a;
    bf16* Lp = (bf16*)P->Lout[a];
    const int64_t ld = P->ldl[a];
    const int c = colg - P->col_start[a];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t r = row0 + wm * 64 + mb * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
        if (r < T) Lp[r * ld + c] = (bf16)acc[mb][nb][e];
      }
  }
}

__global__ __launch_bounds__(256) void lr_precompute_f32(const PrecomputeArgs args) {
  const PrecomputeArgs* P = (const PrecomputeArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  __shared__ float Xs[64][17];
  __shared__ float As[16][64];
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int tid = threadIdx.x, tr = (tid >> 4) * 4, tc = (tid & 15) * 4;
  const float* X = (const float*)P->X;
  const float* Ac = (const float*)P->A;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < P->d_model; k0 += 16) {
    __syncthreads();
    for (int e = tid; e < 64 * 16; e += 256) {
      const int r = e / 16, k = e % 16;
      const int64_t gr = r0 + r, gk = k0 + k;
      Xs[r][k] = (gr < P->T && gk < P->d_model) ? X[gr * P->ldx + gk] : 0.f;
    }
    for (int e = tid; e < 16 * 64; e += 256) {
      const int k = e / 64, c = e % 64;
      const int64_t gk = k0 + k;
      As[k][c] = (gk < P->d_model && c0 + c < P->R) ? Ac[gk * P->lda + c0 + c] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(Xs[tr + i][k], As[k][tc + j], acc[i][j]);
  }
  for (int j = 0; j < 4; ++j) {
    const int col = c0 + tc + j;
    if (col >= P->R) continue;
    int a = 0;
    while (a + 1 < P->n_agents && P->col_start[a + 1] <= col) ++a;
    float* Lp = (float*)P->Lout[a];
    const int c = col - P->col_start[a];
    for (int i = 0; i < 4; ++i) {
      const int64_t r = r0 + tr + i;
      if (r < P->T) Lp[r * P->ldl[a] + c] = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_precompute_bf16(const PrecomputeArgs& a, hipStream_t s) {
  const int tiles = (int)((a.T + TM - 1) / TM);
  const int nbt = (a.R + 31) / 32;
  const int nbw = (nbt + 1) / 2;
  switch (nbw) {
    case 1: hipLaunchKernelGGL(lr_precompute_bf16<1>, dim3(tiles), dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(lr_precompute_bf16<2>, dim3(tiles), dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL(lr_precompute_bf16<3>, dim3(tiles), dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(lr_precompute_bf16<4>, dim3(tiles), dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_precompute_f32(const PrecomputeArgs& a, hipStream_t s) {
  const int rt = (int)((a.T + 63) / 64);
  const int ct = (a.R + 63) / 64;
  hipLaunchKernelGGL(lr_precompute_f32, dim3(rt, ct), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lra
