// Flash-LoRA-Attention, bf16 storage / fp32 accumulation, for gfx950 (MI355X).
//
// Computes, per request and query row of agent a (LRAgent summary, section
// "3. Flash-LoRA-Attention"):
//     O = P·V_base + (P·L_a)·B_a,   P = causal softmax(Q·K_baseᵀ / sqrt(D))
// with ONE online softmax shared by both products; L_a stays r wide inside the key loop
// and B_a is applied once per tile of query rows, after the loop.
//
// Workgroup = 4 waves.  It owns one kv head g of one request and a tile of 128
// (query, head-in-group) rows, row = t*G + h_local, so all q heads that share K/V_base
// read each LDS tile (GQA-aware).  Each wave owns 32 rows and keeps its scores
// TRANSPOSED, Sᵀ = K·Qᵀ: with v_mfma_f32_32x32x16_bf16 a lane then holds one query row's
// scores for 16 keys, the row max/sum need a single cross-half permlane32 swap, and the
// score accumulator is already laid out as the B operand of the next products
// Oᵀ += V_baseᵀ·Pᵀ and (P·L)ᵀ += Lᵀ·Pᵀ (keys are permuted identically on both sides).
// K, V_base and L tiles of 64 keys stream HBM -> LDS with direct (VGPR-free)
// global_load_lds_dwordx4, double-buffered, one barrier per tile; K/V rows are
// XOR-swizzled in 16-byte chunks against LDS bank conflicts.  V_base and L are read
// with ds_read_b64_tr_b16, which transposes 4x16 blocks inside 16-lane groups, so the
// caches keep their natural token-major layout in HBM and LDS.
//
// When the planner splits a request's key range over several workgroups (to fill the
// 256 CUs), each writes its unnormalised partial state (m, l, P·V_base, P·L) to the
// workspace and fla_combine_bf16 merges them and applies B once per row.  Decode is the
// same kernel with one query per request and many key splits.
#include "lra_internal.h"

namespace lra {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr float kNegBig = -1.0e30f;   // finite start value of the running max

__device__ __forceinline__ float half_max(float x) {
  // max over lanes l and l^32 (the two halves of a wave hold the same query row)
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i16x4 tr_read(const LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)p);
}

__device__ __forceinline__ bf16x8 join(i16x4 lo, i16x4 hi) {
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 64 rows x D bf16 from a strided source into LDS (row = D*2 bytes, 16-byte chunk c of
// row k stored at position c ^ (k % (D/8))).  Rows at or past `valid` repeat row valid-1
// so the tile holds only finite data; the caller masks them.
template <int D>
__device__ __forceinline__ void load_rows(const bf16* src, int64_t stride, int r0, int valid,
                                          LDS char* dst, int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int RPU = 64 / CPR;        // rows per 1 KB unit
  constexpr int UNITS = 64 / RPU;
#pragma unroll
  for (int u = wave; u < UNITS; u += 4) {
    const int row = u * RPU + lane / CPR;
    const int c = (lane % CPR) ^ (row % CPR);
    const int key = min(r0 + row, valid - 1);
    __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)key * stride + c * 8),
                                     (LDS void*)(dst + u * 1024), 16, 0, 0);
  }
}

// 64 rows x rank bf16 of an LR cache, rows packed densely (rank*2 bytes) in LDS.
__device__ __forceinline__ void load_lr(const bf16* src, int64_t ldl, int rank, int r0, int valid,
                                        LDS char* dst, int wave, int lane) {
  const int row_bytes = rank * 2;
  const int units = rank / 8;
  for (int u = wave; u < units; u += 4) {
    const int off = u * 1024 + lane * 16;
    const int row = off / row_bytes;
    const int c = (off - row * row_bytes) >> 4;
    const int key = min(r0 + row, valid - 1);
    __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)key * ldl + c * 8),
                                     (LDS void*)(dst + u * 1024), 16, 0, 0);
  }
}

// A operand (rows = D lanes of block db, k = 16 keys of step st) of Oᵀ += Vᵀ·Pᵀ from a
// swizzled 64 x D tile.  Key order within the step matches pfrag().
template <int D>
__device__ __forceinline__ bf16x8 vfrag(const LDS char* tile, int st, int db, int lane) {
  constexpr int CPR = D / 8;
  const int g16 = lane >> 4, jj = lane & 15;
  const int key = (st >> 1) * 32 + (st & 1) * 16 + (g16 >> 1) * 4 + (jj >> 2);
  const int d = db * 32 + (g16 & 1) * 16 + (jj & 3) * 4;
  const int c = d >> 3, sub = (d & 7) * 2;
  const int k1 = key + 8;
  i16x4 lo = tr_read(tile + key * (D * 2) + ((c ^ (key % CPR)) << 4) + sub);
  i16x4 hi = tr_read(tile + k1 * (D * 2) + ((c ^ (k1 % CPR)) << 4) + sub);
  return join(lo, hi);
}

// A operand of (P·L)ᵀ += Lᵀ·Pᵀ: rows = rank lanes rb*32.., zero for rows >= rank.
__device__ __forceinline__ bf16x8 lfrag(const LDS char* tile, int rank, int st, int rb, int lane) {
  const int g16 = lane >> 4, jj = lane & 15;
  const int key = (st >> 1) * 32 + (st & 1) * 16 + (g16 >> 1) * 4 + (jj >> 2);
  int rho = rb * 32 + (g16 & 1) * 16 + (jj & 3) * 4;
  if (rho >= rank) rho = 0;                               // keep the read in bounds
  i16x4 lo = tr_read(tile + key * (rank * 2) + rho * 2);
  i16x4 hi = tr_read(tile + (key + 8) * (rank * 2) + rho * 2);
  bf16x8 v = join(lo, hi);
  const int my_rho = rb * 32 + (lane & 31);
  if (my_rho >= rank) v = bf16x8{};
  return v;
}

// B operand for key step st (16 keys) from the transposed score/probability block.
__device__ __forceinline__ bf16x8 pfrag(const f32x16& s, int half) {
  bf16x8 r;
#pragma unroll
  for (int q = 0; q < 8; ++q) r[q] = (bf16)s[half * 8 + q];
  return r;
}

template <int D>
__global__ __launch_bounds__(256, 2) void fla_attn_bf16(const AttnArgs args) {
  const AttnArgs* A = (const AttnArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int DB = D / 32;           // 32-row blocks of the transposed output
  constexpr int KS = D / 16;           // k-steps of the score product
  constexpr int CPR = D / 8;
  constexpr int TILE_KV = 64 * D * 2;  // bytes of one K or V tile
  constexpr int TILE_L = 64 * 64 * 2;  // bytes of one LR tile (max rank)
  constexpr int BUF = 2 * TILE_KV + TILE_L;
  __shared__ __attribute__((aligned(1024))) char smem_raw[2 * BUF];
  LDS char* smem = (LDS char*)smem_raw;

  // ---- work item -> (request, kv head, key split, row tile); XCD-major numbering keeps
  // the row tiles of one (request, kv head, split) on one XCD, sharing its L2.
  const int bid = blockIdx.x;
  const int w = (bid & 7) * A->grid_per_xcd + (bid >> 3);
  if (w >= A->n_work) return;
  int b = 0;
  while (b + 1 < A->n_req && A->reqs[b + 1].work_start <= w) ++b;
  const ReqDesc& R = A->reqs[b];
  const int q_start = R.q_start, Lq = R.q_len, k_start = R.k_start, Lk = R.k_len;
  const int n_rt = R.n_rt, n_split = R.n_split;
  int local = w - R.work_start;
  const int rt = local % n_rt;
  local /= n_rt;
  const int sp = local % n_split;
  const int g = local / n_split;
  const int G = A->G, Hq = A->Hq, Hkv = A->Hkv;
  const AgentDesc& AG = A->agents[R.agent];
  const int rank = AG.rank;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, hi = lane >> 5;
  const int rows_total = Lq * G;
  const int row0 = rt * kTileRows;
  const int my_row = row0 + wave * 32 + col;
  const bool valid = my_row < rows_total;
  const int t = valid ? my_row / G : 0;
  const int hl = valid ? my_row - t * G : 0;
  const int pos = valid ? Lk - Lq + t : Lk - 1;
  const bool wave_active = row0 + wave * 32 < rows_total;

  // key range of this workgroup: its split, cut at the causal end of its last row
  const int last_row = min(row0 + kTileRows, rows_total) - 1;
  const int kend_causal = Lk - Lq + last_row / G + 1;
  const int kmask_from = Lk - Lq + row0 / G + 1;      // first key hidden from some row
  const int n_tiles_req = (Lk + kTileKeys - 1) / kTileKeys;
  const int tps = (n_tiles_req + n_split - 1) / n_split;
  const int kb = sp * tps * kTileKeys;
  const int ke = min(min(Lk, kb + tps * kTileKeys), kend_causal);
  const int n_tiles = ke > kb ? (ke - kb + kTileKeys - 1) / kTileKeys : 0;
  const int mask_from = min(kmask_from, ke);

  const int64_t kv_stride = (int64_t)Hkv * D;
  const bf16* Kg = (const bf16*)A->K + ((int64_t)k_start * Hkv + g) * D;
  const bf16* Vg = (const bf16*)A->V + ((int64_t)k_start * Hkv + g) * D;
  const bf16* Lg = rank ? (const bf16*)AG.L + (int64_t)k_start * AG.ldl : nullptr;

  // ---- Q fragments (B operand of Sᵀ = K·Qᵀ): lane holds Q[row col][ks*16 + hi*8 .. +7]
  bf16x8 qf[KS];
  {
    const bf16* qrow = (const bf16*)A->Q + ((int64_t)(q_start + t) * Hq + g * G + hl) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = valid ? *(const bf16x8*)(qrow + ks * 16 + hi * 8) : bf16x8{};
  }

  f32x16 accV[DB];
  f32x16 accL[2];
#pragma unroll
  for (int i = 0; i < DB; ++i) accV[i] = f32x16{};
  accL[0] = accL[1] = f32x16{};
  float m_run = kNegBig, l_run = 0.f;
  const float sl2 = A->scale_log2;
  const int RB = rank > 32 ? 2 : (rank > 0 ? 1 : 0);

  if (n_tiles > 0) {
    load_rows<D>(Kg, kv_stride, kb, ke, smem, wave, lane);
    load_rows<D>(Vg, kv_stride, kb, ke, smem + TILE_KV, wave, lane);
    if (rank) load_lr(Lg, AG.ldl, rank, kb, ke, smem + 2 * TILE_KV, wave, lane);
  }
  wait_loads();
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int k0 = kb + j * kTileKeys;
    LDS char* cur = smem + (j & 1) * BUF;
    if (j + 1 < n_tiles) {
      LDS char* nxt = smem + ((j + 1) & 1) * BUF;
      load_rows<D>(Kg, kv_stride, k0 + kTileKeys, ke, nxt, wave, lane);
      load_rows<D>(Vg, kv_stride, k0 + kTileKeys, ke, nxt + TILE_KV, wave, lane);
      if (rank) load_lr(Lg, AG.ldl, rank, k0 + kTileKeys, ke, nxt + 2 * TILE_KV, wave, lane);
    }
    if (wave_active) {
      // -- Sᵀ = K·Qᵀ for 64 keys (two 32-key blocks)
      f32x16 s[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        s[kb2] = f32x16{};
        const int krow = kb2 * 32 + col;
        const LDS char* rowp = cur + krow * (D * 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = ks * 2 + hi;
          bf16x8 kf = *(const LDS bf16x8*)(rowp + ((c ^ (krow % CPR)) << 4));
          s[kb2] = mfma32(kf, qf[ks], s[kb2]);
        }
      }
      // -- scale, causal mask, online softmax (one running max/sum per query row)
      const bool need_mask = k0 + kTileKeys > mask_from;
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float v = s[kb2][e] * sl2;
          if (need_mask) {
            const int key = k0 + kb2 * 32 + (e >> 2) * 8 + hi * 4 + (e & 3);
            if (key > pos || key >= ke) v = -INFINITY;
          }
          s[kb2][e] = v;
          mx = fmaxf(mx, v);
        }
      mx = half_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      float psum = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(s[kb2][e] - m_new);
          s[kb2][e] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
#pragma unroll
      for (int i = 0; i < DB; ++i) accV[i] *= alpha;
      accL[0] *= alpha;
      accL[1] *= alpha;

      // -- Oᵀ += V_baseᵀ·Pᵀ and (P·L)ᵀ += Lᵀ·Pᵀ with the same P
      const LDS char* vt = cur + TILE_KV;
      const LDS char* lt = cur + 2 * TILE_KV;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 pf = pfrag(s[st >> 1], st & 1);
#pragma unroll
        for (int db = 0; db < DB; ++db) accV[db] = mfma32(vfrag<D>(vt, st, db, lane), pf, accV[db]);
        if (RB > 0) accL[0] = mfma32(lfrag(lt, rank, st, 0, lane), pf, accL[0]);
        if (RB > 1) accL[1] = mfma32(lfrag(lt, rank, st, 1, lane), pf, accL[1]);
      }
    }
    wait_loads();
    __syncthreads();
  }

  const float l_tot = half_sum(l_run);
  if (n_split == 1) {
    // ---- epilogue: O = P·V_base / l + ((P·L)/l)·B_g, B applied once for the row tile
    const float inv = 1.f / l_tot;
#pragma unroll
    for (int i = 0; i < DB; ++i) accV[i] *= inv;
    if (rank) {
      // B_g = B[:, g*D : (g+1)*D] is a "value tile" whose rows are the rank index.
      load_rows<D>((const bf16*)AG.B + g * D, kv_stride, 0, rank, smem + TILE_KV, wave, lane);
      wait_loads();
      __syncthreads();
      if (wave_active) {
        const int nst = (rank + 15) / 16;
        for (int st = 0; st < nst; ++st) {
          const f32x16 lsc = accL[st >> 1] * inv;
          const bf16x8 pf = pfrag(lsc, st & 1);
#pragma unroll
          for (int db = 0; db < DB; ++db)
            accV[db] = mfma32(vfrag<D>(smem + TILE_KV, st, db, lane), pf, accV[db]);
        }
      }
    }
    if (valid) {
      bf16* orow = (bf16*)A->O + ((int64_t)(q_start + t) * Hq + g * G + hl) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          bf16x4 o;
#pragma unroll
          for (int j2 = 0; j2 < 4; ++j2) o[j2] = (bf16)accV[db][i * 4 + j2];
          *(bf16x4*)(orow + db * 32 + i * 8 + hi * 4) = o;
        }
    }
  } else if (valid) {
    // ---- partial state of this key split for the combine pass
    const int64_t pr = (int64_t)R.part_base + ((int64_t)sp * Lq + t) * Hq + g * G + hl;
    float* po = A->ws_o + pr * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 v = {accV[db][i * 4], accV[db][i * 4 + 1], accV[db][i * 4 + 2], accV[db][i * 4 + 3]};
        *(f32x4*)(po + db * 32 + i * 8 + hi * 4) = v;
      }
    float* pl = A->ws_l + pr * 64;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 v = {accL[rb][i * 4], accL[rb][i * 4 + 1], accL[rb][i * 4 + 2], accL[rb][i * 4 + 3]};
        *(f32x4*)(pl + rb * 32 + i * 8 + hi * 4) = v;
      }
    if (hi == 0) {
      A->ws_ml[pr * 2] = m_run;
      A->ws_ml[pr * 2 + 1] = l_tot;
    }
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Merge the key-split partial states of one output row (one wave per row):
//   M = max m_s, w_s = 2^(m_s - M),
//   O = (Σ w_s·(P·V_base)_s + (Σ w_s·(P·L)_s)·B_g) / Σ w_s·l_s
// B is linear, so applying it once after the merge equals applying it per split.
template <int D>
__global__ __launch_bounds__(256) void fla_combine_bf16(const AttnArgs args) {
  const AttnArgs* A = (const AttnArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= A->n_comb) return;
  int b = -1;
  for (int i = 0; i < A->n_req; ++i)
    if (A->reqs[i].n_split > 1 && A->reqs[i].comb_start <= row) b = i;
  const ReqDesc& R = A->reqs[b];
  const int Hq = A->Hq, G = A->G, Hkv = A->Hkv;
  const int local = row - R.comb_start;
  const int t = local / Hq, h = local - t * Hq, g = h / G;
  const int S = R.n_split;
  const AgentDesc& AG = A->agents[R.agent];
  const int rank = AG.rank;
  auto prow = [&](int s) { return (int64_t)R.part_base + ((int64_t)s * R.q_len + t) * Hq + h; };

  float m_s = kNegBig, l_s = 0.f;
  if (lane < S) {
    m_s = A->ws_ml[prow(lane) * 2];
    l_s = A->ws_ml[prow(lane) * 2 + 1];
  }
  const float M = wave_max(m_s);
  const float w_s = lane < S ? __builtin_amdgcn_exp2f(m_s - M) : 0.f;
  const float l = wave_sum(w_s * l_s);

  constexpr int DPL = D / 64;
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  float al = 0.f;
  for (int s = 0; s < S; ++s) {
    const float ws = __shfl(w_s, s);
    const int64_t pr = prow(s);
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] += ws * A->ws_o[pr * D + lane + 64 * i];
    al += ws * A->ws_l[pr * 64 + lane];
  }
  const bf16* Bg = (const bf16*)AG.B + g * D;
  for (int rho = 0; rho < rank; ++rho) {
    const float c = __shfl(al, rho);
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] += c * (float)Bg[(int64_t)rho * Hkv * D + lane + 64 * i];
  }
  const float inv = 1.f / l;
  bf16* orow = (bf16*)A->O + ((int64_t)(R.q_start + t) * Hq + h) * D;
#pragma unroll
  for (int i = 0; i < DPL; ++i) orow[lane + 64 * i] = (bf16)(o[i] * inv);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, int n_grid, hipStream_t s) {
  if (head_dim == 128)
    hipLaunchKernelGGL(fla_attn_bf16<128>, dim3(n_grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(fla_attn_bf16<64>, dim3(n_grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine_bf16(const AttnArgs& a, int head_dim, hipStream_t s) {
  const int grid = (a.n_comb + 3) / 4;
  if (head_dim == 128)
    hipLaunchKernelGGL(fla_combine_bf16<128>, dim3(grid), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(fla_combine_bf16<64>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace lra
