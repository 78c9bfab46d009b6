// Naive value expansion, bf16 storage / fp32 accumulation, for gfx950 (MI355X): the
// computation Flash-LoRA-Attention avoids (LRAgent summary, section "3. Flash-LoRA-
// Attention": rebuilding an agent's values from its LR cache expands L·B to the full
// value width, O(L·r·d_out) work and a full-width cache per agent).  For every row s of a
// span of agent a and every kv head g:
//     V_full[s, g, :] = V_base[s, g, :] + L_a[s, :] · B_a[:, g*D : (g+1)*D]
// rounded to bf16.  It exists to measure the regrouping against (a full-width V_full
// followed by plain attention with no adapter), not as part of the regrouped path.
//
// A workgroup (4 waves) owns one kv head and up to rows_per_item rows (at most 512) of one
// span, in tiles of 32 rows.  The product is an MFMA contraction over the rank: wave w computes the
// transposed block (L·B_g)ᵀ[32w .. 32w+31, rows] = B_gᵀ·Lᵀ with v_mfma_f32_32x32x16_bf16,
// its B_gᵀ fragments held in registers for the whole work item and the L rows loaded
// straight into the other operand.  The fp32 block goes through LDS so that the V_base
// read and the V_full write are whole 16-byte chunks of each row (coalesced), and the next
// tile's V_base chunks are in flight while the current tile is computed.
#include "lra_internal.h"

namespace lra {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr int kRowsPerTile = 32;

// Span that owns work item w (wave-uniform): lane i compares span i's first item.
__device__ __forceinline__ int find_span(const ExpandArgs* A, int w) {
  const int lane = threadIdx.x & 63;
  const int start = lane < A->n_span ? A->spans[lane].work_start : 0x7fffffff;
  return __builtin_amdgcn_readfirstlane(__popcll(__ballot(start <= w)) - 1);
}

template <int D, int NK>   // NK: 16-wide rank steps (the launch's largest rank, rounded up)
__global__ __launch_bounds__(256) void lr_expand_bf16(const ExpandArgs args) {
  const ExpandArgs* A = (const ExpandArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int CPR = D / 8;                       // 16-byte chunks per row of one head
  constexpr int NP = kRowsPerTile * CPR / 256;     // chunks per thread per tile
  constexpr int PAD = D + 4;                       // fp32 LDS row (16-byte skew per row)
  __shared__ __attribute__((aligned(16))) float tile[kRowsPerTile * PAD];

  const int w = blockIdx.x;
  if (w >= A->n_work) return;
  const int si = find_span(A, w);
  const ExpandSpan& S = A->spans[si];
  const int Hkv = A->Hkv;
  const int local = w - S.work_start;
  const int g = local % Hkv;
  const int64_t r_begin = S.start + (int64_t)(local / Hkv) * A->rows_per_item;
  const int64_t r_end = min(S.start + (int64_t)S.len, r_begin + A->rows_per_item);
  const AgentDesc& AG = A->agents[S.agent];
  const int rank = AG.rank;
  const int64_t kv_stride = (int64_t)Hkv * D;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool mma_wave = NK > 0 && wave * 32 < D && rank > 0;
  const int col = lane & 31, half = lane >> 5;

  // B_gᵀ fragments: lane (col, half) holds B[ks*16 + half*8 + j][g*D + wave*32 + col]
  bf16x8 bfr[NK > 0 ? NK : 1];
  if (mma_wave) {
    const bf16* Bc = (const bf16*)AG.B + g * D + wave * 32 + col;
#pragma unroll
    for (int ks = 0; ks < NK; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = ks * 16 + half * 8 + j;
        bfr[ks][j] = k < rank ? Bc[(int64_t)k * kv_stride] : (bf16)0.f;
      }
  }
  const bf16* Lb = rank > 0 ? (const bf16*)AG.L : nullptr;
  const int64_t ldl = AG.ldl;
  const bf16* Vg = (const bf16*)A->V + (int64_t)g * D;
  bf16* Og = (bf16*)A->Vout + (int64_t)g * D;

  auto load_v = [&](int64_t r0, u32x4* v) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int u = tid + 256 * p;
      const int64_t row = r0 + u / CPR;
      v[p] = row < r_end ? *(const u32x4*)(Vg + row * kv_stride + (u % CPR) * 8) : u32x4{};
    }
  };
  u32x4 vcur[NP], vnext[NP];
  load_v(r_begin, vcur);
  for (int64_t r0 = r_begin; r0 < r_end; r0 += kRowsPerTile) {
    if (r0 + kRowsPerTile < r_end) load_v(r0 + kRowsPerTile, vnext);
    if (mma_wave) {
      const int64_t row = r0 + col;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NK; ++ks) {
        const int k = ks * 16 + half * 8;
        const u32x4 lv = (row < r_end && k < rank) ? *(const u32x4*)(Lb + row * ldl + k) : u32x4{};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ks], __builtin_bit_cast(bf16x8, lv),
                                                      acc, 0, 0, 0);
      }
      // lane holds row `col` of the tile and head lanes wave*32 + 8i + 4*half .. +3
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(LDS f32x4*)((LDS float*)tile + col * PAD + wave * 32 + 8 * i + 4 * half) =
            f32x4{acc[4 * i], acc[4 * i + 1], acc[4 * i + 2], acc[4 * i + 3]};
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int u = tid + 256 * p;
      const int rl = u / CPR, c = u % CPR;
      const int64_t row = r0 + rl;
      if (row < r_end) {
        const bf16x8 vb = __builtin_bit_cast(bf16x8, vcur[p]);
        bf16x8 o;
        if (rank > 0) {
          const f32x4 a0 = *(const LDS f32x4*)((const LDS float*)tile + rl * PAD + c * 8);
          const f32x4 a1 = *(const LDS f32x4*)((const LDS float*)tile + rl * PAD + c * 8 + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            o[j] = (bf16)((float)vb[j] + a0[j]);
            o[4 + j] = (bf16)((float)vb[4 + j] + a1[j]);
          }
        } else {
          o = vb;
        }
        *(bf16x8*)(Og + row * kv_stride + c * 8) = o;
      }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < NP; ++p) vcur[p] = vnext[p];
  }
}

}  // namespace

hipError_t launch_expand_bf16(const ExpandArgs& a, int head_dim, int max_rank, hipStream_t s) {
  const int nk = max_rank > 32 ? 4 : max_rank > 16 ? 2 : max_rank > 0 ? 1 : 0;
#define LRA_LAUNCH(D, NK) \
  hipLaunchKernelGGL((lr_expand_bf16<D, NK>), dim3(a.n_work), dim3(256), 0, s, a)
  if (head_dim == 128) {
    if (nk == 0) LRA_LAUNCH(128, 0);
    else if (nk == 1) LRA_LAUNCH(128, 1);
    else if (nk == 2) LRA_LAUNCH(128, 2);
    else LRA_LAUNCH(128, 4);
  } else {
    if (nk == 0) LRA_LAUNCH(64, 0);
    else if (nk == 1) LRA_LAUNCH(64, 1);
    else if (nk == 2) LRA_LAUNCH(64, 2);
    else LRA_LAUNCH(64, 4);
  }
#undef LRA_LAUNCH
  return hipGetLastError();
}

}  // namespace lra
