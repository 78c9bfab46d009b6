// PreLRShared LR precompute for gfx950: L_a = X·A_a for every agent in one pass over X
// (PReCache abstract on the arxivdaily page, PreLRShared; LRAgent summary, section 2: the
// LR cache holds the LoRA down-projection activations X·A_i).
//
// bf16 path: a tall-skinny GEMM L_cat[T, R] = X[T, d_model]·A_cat[d_model, R] with
// R = sum of ranks <= 256.  The work is bound by reading X once from HBM (R = 192 gives
// ~180 FLOP per byte, under the MI355X ridge), so every workgroup owns 128 rows of X and
// ALL R columns, reading X from HBM exactly once.  X chunks (128 rows x 64 d_model values,
// whole 128-byte row segments per 8-lane group) and A_cat chunks (64 x R) are loaded two
// chunks ahead into registers and stored into LDS tiles (X swizzled, A_cat padded); the
// B operands are read with ds_read_b64_tr_b16.  Four waves split the 128 x R tile 2 x 2 (64 rows x R/2 columns
// each) with v_mfma_f32_32x32x16_bf16; the epilogue rounds to bf16 and scatters column
// blocks to each agent's L_a.
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
constexpr int PF = 2;           // chunks in flight in registers ahead of the LDS tiles

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
  constexpr int NBT = 2 * NBW;                 // 32-column blocks in the padded A_cat tile
  constexpr int RS = NBT * 32 * 2 + 16;        // A_cat LDS row stride (bytes), padded
  constexpr int CPT = NBT;                     // 16-byte A_cat chunks per thread per tile
  constexpr int XS = 2;                        // X LDS stages
  constexpr int XTILE = TM * KC * 2;           // 16 KB: 128 rows x 64 d_model values
  constexpr int UX = XTILE / 1024 / 4;         // X direct loads per wave per chunk (4)
  constexpr int ATILE = KC * RS;
  __shared__ __attribute__((aligned(1024))) char smem_raw[XS * XTILE + 2 * ATILE];
  LDS char* xlds = (LDS char*)smem_raw;
  LDS char* alds = xlds + XS * XTILE;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int hi = lane >> 5;
  const int64_t T = P->T, ldx = P->ldx, lda = P->lda;
  const int R = P->R;
  const int nk = (int)(P->d_model / KC);       // d_model % 64 == 0 (checked by the host)
  const int nk_pad = (nk + PF - 1) / PF * PF;   // padded chunks meet zero rows of A_cat
  const int64_t row0 = (int64_t)blockIdx.x * TM;

  // X chunk (128 rows x 128 bytes): each lane loads 16-byte units, 8 whole rows per wave
  // instruction, two chunks ahead into registers, and stores them into an LDS tile where
  // unit p of row r holds global unit p ^ ((r >> 1) & 7); that makes the operand reads
  // below (32 consecutive rows at one unit) bank-conflict free.  Rows past T repeat row T-1
  // (their results are never stored).  (Register staging measured faster here than direct
  // global->LDS loads.)
  const char* xsrc[UX];
#pragma unroll
  for (int i = 0; i < UX; ++i) {
    const int u = wave + 4 * i;
    const int row = u * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    xsrc[i] = (const char*)P->X + (min(row0 + row, T - 1) * ldx + c * 8) * 2;
  }
  // Workgroups start their d_model sweep at different chunks so that they do not all read
  // the same 128-byte column of the 8 KB rows at once.
  const int rot = (int)(blockIdx.x % nk);
  auto chunk = [&](int kc) { return kc < nk ? (kc + rot) % nk : nk - 1; };
  u32x4 xr[PF][UX];
  auto load_x = [&](u32x4 (&dst)[UX], int kc) {
    const int64_t koff = (int64_t)chunk(kc) * KC * 2;
#pragma unroll
    for (int i = 0; i < UX; ++i) dst[i] = *(const u32x4*)(xsrc[i] + koff);
  };
  auto store_x = [&](const u32x4 (&src)[UX], int kc) {
    LDS char* dst = xlds + (kc % XS) * XTILE;
#pragma unroll
    for (int i = 0; i < UX; ++i) *(LDS u32x4*)(dst + (wave + 4 * i) * 1024 + lane * 16) = src[i];
  };
  // A operand (row lane&31 of m-block mb, d_model values ks*16 + hi*8 ..) from the X tile
  int xoff[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int row = wm * 64 + mb * 32 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) xoff[mb][ks] = row * 128 + (((2 * ks + hi) ^ ((row >> 1) & 7)) << 4);
  }
  // A_cat tile (64 d_model rows x NBT*32 columns), staged through registers into a padded
  // LDS tile; columns past R and padded chunks are stored as zeros.
  u32x4 areg[PF][CPT];
  uint32_t aoff[CPT];
  int a_ok[CPT], lds_off[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int ch = tid + 256 * i;
    const int k = ch / (NBT * 4), c = ch % (NBT * 4);
    a_ok[i] = c * 8 < R;
    aoff[i] = (uint32_t)((k * lda + min(c, R / 8 - 1) * 8) * 2);
    lds_off[i] = k * RS + c * 16;
  }
  const char* Abase = (const char*)P->A;
  auto load_a = [&](u32x4 (&dst)[CPT], int kc) {
    const char* base = Abase + (int64_t)chunk(kc) * KC * lda * 2;
#pragma unroll
    for (int i = 0; i < CPT; ++i) dst[i] = *(const u32x4*)(base + aoff[i]);
  };
  auto store_a = [&](const u32x4 (&src)[CPT], int buf, int kc) {
    const bool chunk_ok = kc < nk;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      *(LDS u32x4*)(alds + buf * ATILE + lds_off[i]) = (chunk_ok && a_ok[i]) ? src[i] : u32x4{};
  };
  const int g16 = lane >> 4, jj = lane & 15;
  int boff[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb)
    boff[nb] = ((g16 >> 1) * 8 + (jj >> 2)) * RS + ((wn * NBW + nb) * 32 + (g16 & 1) * 16 + (jj & 3) * 4) * 2;

  f32x16 acc[2][NBW];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = f32x16{};

#pragma unroll
  for (int i = 0; i < PF; ++i) {
    load_a(areg[i], i);
    load_x(xr[i], i);
  }
  store_a(areg[0], 0, 0);
  store_x(xr[0], 0);
  __syncthreads();

  // Chunk c travels global -> register slot c % PF (issued in iteration c - PF) -> LDS
  // (stored at the end of iteration c - 1) -> MFMA operands (iteration c).  The loop is
  // unrolled by PF so every slot index is static and the wait counts are exact.
  for (int kc0 = 0; kc0 < nk_pad; kc0 += PF) {
#pragma unroll
    for (int st = 0; st < PF; ++st) {
      const int kc = kc0 + st;
      // slot st held chunk kc, already in LDS: refill it with chunk kc + PF
      load_a(areg[st], kc + PF);
      load_x(xr[st], kc + PF);
      const LDS char* xt = xlds + (kc % XS) * XTILE;
      const LDS char* at = alds + (kc & 1) * ATILE;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 af[2], bf[NBW];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) af[mb] = *(const LDS bf16x8*)(xt + xoff[mb][ks]);
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
          const LDS char* p = at + boff[nb] + ks * 16 * RS;
          bf[nb] = join(__builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)p),
                        __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(p + 4 * RS)));
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < NBW; ++nb) acc[mb][nb] = mfma32(af[mb], bf[nb], acc[mb][nb]);
      }
      store_a(areg[(st + 1) % PF], (kc + 1) & 1, kc + 1);
      store_x(xr[(st + 1) % PF], kc + 1);
      __syncthreads();
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
