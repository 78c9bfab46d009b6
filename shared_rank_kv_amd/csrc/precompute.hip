// PreLRShared LR precompute for gfx950: L_a = X·A_a for every agent in one pass over X
// (PReCache abstract on the arxivdaily page, PreLRShared; LRAgent summary, section 2: the
// LR cache holds the LoRA down-projection activations X·A_i).
//
// bf16 path: a tall-skinny GEMM L_cat[T, R] = X[T, d_model]·A_cat[d_model, R] with
// R = sum of ranks <= 256.  The work is bound by reading X once from HBM (R = 192 gives
// ~180 FLOP per byte, under the MI355X ridge).  The kernel computes the transposed tile
// L_catᵀ = A_catᵀ·Xᵀ with v_mfma_f32_16x16x32_bf16, so that X is the B operand: in that
// operand a lane holds eight consecutive d_model values of one token, which is 16
// contiguous bytes of an X row.  X therefore streams from HBM straight into MFMA operand
// registers and never touches LDS; each step issues one 64-value chunk (128 bytes of each
// row), four chunks ahead.  A_cat (small, L2-resident) is the A
// operand: it travels by direct buffer->LDS loads into a ring of four LDS tiles, three
// chunks ahead, and is read back with the transposing LDS read.  Each workgroup owns 128
// tokens and all R columns, so X is read from HBM exactly once; the epilogue rounds to
// bf16 and scatters column blocks to each agent's L_a.
//
// fp32 path: a plain LDS-tiled fp32 GEMM (exactness, not throughput).
#include "lra_internal.h"

namespace lra {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr int KC = 64;                        // d_model values per chunk
constexpr int TM = 128;                       // tokens per workgroup
constexpr int kBufferFlags = 0x00020000;      // raw buffer resource, dword format
constexpr int kOutOfRange = 0x7ffffff0;       // a buffer offset past every record count

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 join(i16x4 lo, i16x4 hi) {
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ i16x4 tr_read(const LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)p);
}

// s_waitcnt vmcnt(N): all but the N most recently issued vector-memory operations are done
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Barrier for LDS data: waits for this wave's own LDS operations only (direct
// buffer->LDS loads are waited for with wait_vm by the wave that issued them).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte buffer load into registers (zero past the resource's record count)
__device__ __forceinline__ u32x4 load_b128(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// 16-byte direct buffer->LDS load: lane l's bytes land at dst + 16 l
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, LDS char* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)dst, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}

// Row k of an A_cat chunk sits in LDS row a_row(k).  Inside each 32-row block the bits of
// k = 8g + 4h + e become 16h + 4g + e: the two transposing reads of lane group g (LDS rows
// 4g + e, then 16 + 4g + e, e = 0..3) then return A_cat rows 8g .. 8g + 7, the same eight
// consecutive d_model values that the lane holds of its X row.  a_k inverts it.
__device__ __forceinline__ int a_k(int rho) {
  return (rho & ~31) | (((rho >> 2) & 3) << 3) | (((rho >> 4) & 1) << 2) | (rho & 3);
}

// 16-byte unit p of LDS tile row rho holds A_cat unit p ^ a_swz(rho).  The transposing read
// of a lane group fetches rows 4g + e (e = 0..3) x 32 bytes; a quarter-wave (one g) must
// fall on distinct 32-byte slots of a 128-byte bank cycle and a half-wave (g and g + 1) on
// distinct slots of a 256-byte cycle.  Rows of 256 or 512 bytes all start at bank 0: the
// swizzle takes eight slots (an involution inside aligned groups of 16 units).  Rows of 128
// or 384 bytes alternate between the halves of the 256-byte cycle: four slots per row
// parity, permuted with g so that rows 4g + e and 4(g + 1) + e differ (groups of 8 units).
// Row offsets that are multiples of 16 (the second read, later k-steps) leave it unchanged.
template <int NCB>
__device__ __forceinline__ int a_swz(int rho) {
  return NCB % 8 == 0 ? 2 * (rho & 7) : 2 * ((rho & 3) ^ ((rho >> 2) & 1));
}

// NCB: 16-column blocks of A_cat (R padded up to 64, 128, 192 or 256 columns).
template <int NCB>
__global__ __launch_bounds__(256, 1) void lr_precompute_bf16(const PrecomputeArgs args) {
  const PrecomputeArgs* P = (const PrecomputeArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int RB = NCB * 32;                 // bytes per LDS tile row (NCB * 16 columns)
  constexpr int ATILE = KC * RB;               // bytes per A_cat chunk tile
  constexpr int NAW = ATILE / 1024 / 4;        // 1 KB direct loads per wave per chunk
  constexpr int NB = 2;                        // 16-token blocks per wave (32 tokens)
  constexpr int MB = NCB;                      // 16-column blocks (all of R)
  constexpr int XN = NB * 2;                   // X loads per wave per chunk (2 k-steps)
  constexpr int XV = 4;                        // granularity of the per-XCD chunk rotation
  constexpr int NT = 4;                        // A_cat tiles in the LDS ring
  constexpr int UNROLL = 8;                    // chunk steps per loop pass (X ring slots)
  static_assert(NAW * 4 * 1024 == ATILE, "tile split over four waves");
  static_assert(UNROLL % NT == 0, "static tile indices");
  // A_cat ring: chunk kc lives in tile kc % NT.  Separate arrays let the compiler see that
  // the tile being filled by direct loads is not the one being read.
  __shared__ __attribute__((aligned(1024))) char sa0[ATILE];
  __shared__ __attribute__((aligned(1024))) char sa1[ATILE];
  __shared__ __attribute__((aligned(1024))) char sa2[ATILE];
  __shared__ __attribute__((aligned(1024))) char sa3[ATILE];
  LDS char* const tiles[NT] = {(LDS char*)sa0, (LDS char*)sa1, (LDS char*)sa2, (LDS char*)sa3};

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: base pointers stay scalar
  const int grp = lane >> 4, col = lane & 15;
  const int64_t T = P->T, ldx = P->ldx, lda = P->lda;
  const int R = P->R;
  const int nk = (int)(P->d_model / KC);       // d_model % 64 == 0 (checked by the host)
  const int nk_pad = (nk + UNROLL - 1) / UNROLL * UNROLL;   // padded chunks read zeros
  const int64_t t0 = (int64_t)blockIdx.x * TM + wave * 16 * NB;   // first token of this wave

  // X operand (token block nb, k-step ks of a chunk): lane (grp, col) holds d_model values
  // 32 ks + 8 grp .. + 8 of the chunk, of token t0 + 16 nb + col.  Tokens past T read zeros
  // (their results are not stored); chunks past d_model read zeros through an empty
  // resource.
  const int64_t left = T - t0;
  const int x_rows = left <= 0 ? 0 : (left < 16 * NB ? (int)left : 16 * NB);
  const __amdgpu_buffer_rsrc_t x_rsrc =
      make_rsrc((const char*)P->X + t0 * ldx * 2, (int)(x_rows * ldx * 2));
  const __amdgpu_buffer_rsrc_t none = make_rsrc(P->X, 0);
  int xoff[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) xoff[nb] = (int)((nb * 16 + col) * ldx * 2) + grp * 16;
  // The workgroups of one XCD sweep d_model in the same order, so each A_cat chunk is read
  // into that XCD's L2 once and serves all of them; the eight XCDs start an eighth of
  // d_model apart (rounded down to four chunks).
  const int rot = (int)(blockIdx.x & 7) * (nk >> 3) & ~(XV - 1);
  auto chunk = [&](int kc) { return kc < nk ? (kc + rot < nk ? kc + rot : kc + rot - nk) : 0; };
  u32x4 xop[UNROLL][NB][2];
  auto load_x = [&](u32x4 (&dst)[NB][2], int kc) {
    __amdgpu_buffer_rsrc_t r = none;
    if (kc < nk) r = x_rsrc;
    const int soff = chunk(kc) * KC * 2;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) dst[nb][ks] = load_b128(r, xoff[nb] + ks * 64, soff);
  };

  // A_cat chunk -> LDS tile: the 1 KB unit i of this wave covers tile units
  // (wave * NAW + i) * 64 + lane; columns past R read zeros.
  int aoff_g[NAW];
#pragma unroll
  for (int i = 0; i < NAW; ++i) {
    const int u = (wave * NAW + i) * 64 + lane;
    const int rho = u / (2 * NCB), c = (u % (2 * NCB)) ^ a_swz<NCB>(rho);
    aoff_g[i] = c * 8 < R ? (int)((a_k(rho) * lda + c * 8) * 2) : kOutOfRange;
  }
  const char* Abase = (const char*)P->A;
  const int a_bytes = (int)(KC * lda * 2);
  auto load_a = [&](LDS char* tile, int kc) {
    const __amdgpu_buffer_rsrc_t r =
        make_rsrc(Abase + (int64_t)chunk(kc) * KC * lda * 2, kc < nk ? a_bytes : 0);
#pragma unroll
    for (int i = 0; i < NAW; ++i)
      load_lds16(r, tile + (wave * NAW + i) * 1024, aoff_g[i]);
  };

  // A operand (column block cb, k-step ks): lane (grp, e = col / 4, q = col % 4) points the
  // transposing read at LDS row 32 ks + 4 grp + e (then + 16), columns 16 cb + 4 q .. + 4;
  // the read hands lane (grp, col) column 16 cb + col.
  int aoff[MB];
  {
    const int e = col >> 2, q = col & 3;
#pragma unroll
    for (int cb = 0; cb < MB; ++cb)
      aoff[cb] = (4 * grp + e) * RB + ((2 * cb + (q >> 1)) ^ a_swz<NCB>(4 * grp + e)) * 16 +
                 (q & 1) * 8;
  }

  f32x4 acc[NB][MB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int cb = 0; cb < MB; ++cb) acc[nb][cb] = f32x4{};

  // Issue order per chunk step kc, before its MFMAs: A_cat chunk kc + 3 (into the tile chunk
  // kc - 1 used), then the X operands of chunk kc + 4, so X streams as a sliding window of
  // four chunks.  At the end of step kc the tile and the X operands of chunk kc + 1 must be
  // complete; both precede A_cat chunk kc + 1 in issue order, which was followed by X of
  // kc + 2, A of kc + 2, X of kc + 3, A of kc + 3 and X of kc + 4: those may stay in flight.
  // (Issuing X a whole visit of four chunks at a time made each visit's wait cover all four
  // chunks at once; measured 2-3 % slower.)  The prologue issues X(0) A(0) X(1) A(1) X(2)
  // A(2) X(3).
#pragma unroll
  for (int i = 0; i < NT - 1; ++i) {
    load_x(xop[i], i);
    load_a(tiles[i], i);
  }
  load_x(xop[NT - 1], NT - 1);
  wait_vm<3 * XN + 2 * NAW>();
  lds_barrier();

  for (int kc0 = 0; kc0 < nk_pad; kc0 += UNROLL) {
#pragma unroll
    for (int st = 0; st < UNROLL; ++st) {
      const int kc = kc0 + st;
      const LDS char* at = tiles[st % NT];
      // this step's loads, into the tile of chunk kc - 1 and the X slot of chunk kc - 4, both
      // free (the barrier that ended step kc - 1 follows every read of them).  The compiler
      // places them after the MFMAs, just before the wait; keeping them ahead was slower.
      load_a(tiles[(st + NT - 1) % NT], kc + NT - 1);
      load_x(xop[(st + NT) % UNROLL], kc + NT);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        bf16x8 aop[MB];
#pragma unroll
        for (int cb = 0; cb < MB; ++cb) {
          const LDS char* p = at + aoff[cb] + ks * 32 * RB;
          aop[cb] = join(tr_read(p), tr_read(p + 16 * RB));
        }
#pragma unroll
        for (int cb = 0; cb < MB; ++cb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            acc[nb][cb] = mfma16(aop[cb], __builtin_bit_cast(bf16x8, xop[st][nb][ks]),
                                 acc[nb][cb]);
      }
      wait_vm<3 * XN + 2 * NAW>();
      lds_barrier();
    }
  }

  // epilogue: acc[nb][cb] register j of lane (grp, col) is column 16 gcb + 4 grp + j of
  // token t0 + 16 nb + col.  Ranks are multiples of 8, so those four columns belong to one
  // agent; they are stored as one 8-byte write where that agent's layout allows it.
#pragma unroll
  for (int cb = 0; cb < MB; ++cb) {
    const int c0 = cb * 16 + 4 * grp;
    if (c0 >= R) continue;
    int a = 0;
    while (a + 1 < P->n_agents && P->col_start[a + 1] <= c0) ++a;
    bf16* Lp = (bf16*)P->Lout[a] + (c0 - P->col_start[a]);
    const int64_t ld = P->ldl[a];
    const bool vec = ((uintptr_t)Lp & 7) == 0 && (ld & 3) == 0;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int64_t t = t0 + nb * 16 + col;
      if (t >= T) continue;
      const f32x4 v = acc[nb][cb];
      if (vec) {
        *(bf16x4*)(Lp + t * ld) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) Lp[t * ld + j] = (bf16)v[j];
      }
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

// ---------------------------------------------------------------------------------------
// Decode-step append: the LR rows of a few new tokens, L_a[rows[t]] = x_t·A_a for every
// agent (the LR caches of PreLRShared kept current as tokens are generated).  The product
// is tiny in tokens and long in d_model, and at this size it is bound by memory latency, so
// d_model is split across workgroups and every X and A_cat element is read by exactly one
// of them (no workgroup re-reads another's data), in two passes over a caller workspace:
//
// pass 1 (lr_append_part_bf16): workgroup (slice s, token block tb, column block cb) with
//   64 tokens x 64 columns and the d_model values of slice s, in rounds of 256 values (eight
//   32-value chunks).  Wave (ts, kq) takes token sub-block ts (16 tokens), all 64 columns,
//   and chunks kq and kq + 4 of each round.  As in the precompute the product is computed
//   transposed with v_mfma_f32_16x16x32_bf16: the X rows are the B operand (straight from
//   memory); the [32 x 16] A_cat blocks of a round (chunk x column sub-block) pass through
//   LDS, rows permuted (a_k) for the transposing read, each loaded by one wave for the
//   four that use it.  The next round's loads are in flight during a round's MFMAs.  The
//   four k-quarters of a token sub-block meet in LDS and are added in a fixed order into the
//   slice's fp32 partial part[s][t][c].
// pass 2 (lr_append_sum_bf16): one thread per (token, column) adds the slices' partials in
//   slice order, rounds to bf16 and writes the token's cache row.
// Both passes add in a fixed order, so results are deterministic.
constexpr int kAppendRoundChunks = 8;         // 32-value chunks per round

__global__ __launch_bounds__(1024) void lr_append_part_bf16(const AppendArgs args) {
  const AppendArgs* AA = (const AppendArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const PrecomputeArgs* P = &AA->p;
  __shared__ __attribute__((aligned(16))) char tiles[4 * kAppendRoundChunks][1024];
  __shared__ float red[4][64][65];              // [k-quarter][token][column]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ts = wave & 3, kq = wave >> 2;
  const int grp = lane >> 4, col = lane & 15;
  const int s = blockIdx.x, tb = blockIdx.y, cb = blockIdx.z;
  const int64_t T = P->T, ldx = P->ldx, lda = P->lda;
  const int R = P->R;
  const int nk = (int)(P->d_model / 32);
  const int k_lo = s * AA->slice_chunks;                   // this slice's chunks
  const int k_hi = min(nk, k_lo + AA->slice_chunks);
  const int n_rounds = (k_hi - k_lo + kAppendRoundChunks - 1) / kAppendRoundChunks;

  // X: lane (grp, col) holds token 64 tb + 16 ts + col, d_model values 32 j + 8 grp .. + 8
  const int64_t t0 = (int64_t)tb * 64 + ts * 16;
  const int64_t left = T - t0;
  const int x_rows = left <= 0 ? 0 : (left < 16 ? (int)left : 16);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc((const char*)P->X + (x_rows ? t0 * ldx * 2 : 0),
                                              (int)(x_rows * ldx * 2));
  const int xoff = (int)(col * ldx * 2) + grp * 16;
  // A blocks: this wave loads blocks b = wave and wave + 16 of each round (chunk b / 4,
  // column sub-block b % 4); lane l loads 8 columns (64 cb + 16 (b % 4) + 8 (l & 1) ..) of
  // A_cat row 32 j + a_k(l / 2), which the LDS block keeps at row l / 2: offset 16 l
  const __amdgpu_buffer_rsrc_t ar = make_rsrc(P->A, (int)(P->d_model * lda * 2));
  int aoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c8 = cb * 64 + 16 * ((wave + 16 * i) & 3) + 8 * (lane & 1);
    aoff[i] = c8 < R ? (int)((a_k(lane >> 1) * lda + c8) * 2) : kOutOfRange;
  }
  const int a_chunk = (int)(32 * lda * 2);      // bytes of 32 A_cat rows
  // transposing read: lane (grp, e, q) points at block row 4 grp + e (then + 16), columns
  // 4 q .. + 4, and receives column col, d_model values 8 grp .. + 8 of the chunk
  const int toff = (4 * grp + (col >> 2)) * 32 + (col & 3) * 8;

  // chunks past the slice read zeros (soffset past every record)
  auto x_soff = [&](int r, int i) {
    const int j = k_lo + r * kAppendRoundChunks + kq + 4 * i;
    return __builtin_amdgcn_readfirstlane(r < n_rounds && j < k_hi ? j * 64 : kOutOfRange);
  };
  auto a_soff = [&](int r, int i) {
    const int j = k_lo + r * kAppendRoundChunks + ((wave + 16 * i) >> 2);
    return __builtin_amdgcn_readfirstlane(r < n_rounds && j < k_hi ? j * a_chunk : kOutOfRange);
  };
  u32x4 xq[2], aq[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    xq[i] = load_b128(xr, xoff, x_soff(0, i));
    aq[i] = load_b128(ar, aoff[i], a_soff(0, i));
  }
  f32x4 acc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
  for (int r = 0; r < n_rounds; ++r) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *(LDS u32x4*)((LDS char*)tiles[wave + 16 * i] + lane * 16) = aq[i];
    const u32x4 x0 = xq[0], x1 = xq[1];
    if (r + 1 < n_rounds) {                    // the next round's loads, during this one
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        xq[i] = load_b128(xr, xoff, x_soff(r + 1, i));
        aq[i] = load_b128(ar, aoff[i], a_soff(r + 1, i));
      }
    }
    lds_barrier();
#pragma unroll
    for (int cs = 0; cs < 4; ++cs) {
      const LDS char* t0b = (const LDS char*)tiles[4 * kq + cs];
      const LDS char* t1b = (const LDS char*)tiles[4 * (kq + 4) + cs];
      acc[cs] = mfma16(join(tr_read(t0b + toff), tr_read(t0b + toff + 16 * 32)),
                       __builtin_bit_cast(bf16x8, x0), acc[cs]);
      acc[cs] = mfma16(join(tr_read(t1b + toff), tr_read(t1b + toff + 16 * 32)),
                       __builtin_bit_cast(bf16x8, x1), acc[cs]);
    }
    lds_barrier();                             // the round's reads before the next stores
  }
  // acc[cs] register j of lane (grp, col): column 16 cs + 4 grp + j, token 16 ts + col
#pragma unroll
  for (int cs = 0; cs < 4; ++cs)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[kq][16 * ts + col][16 * cs + 4 * grp + j] = acc[cs][j];
  __syncthreads();
  float* part = AA->part + ((int64_t)s * AA->t_pad + tb * 64) * AA->r_pad + cb * 64;
  for (int e = tid; e < 64 * 64; e += 1024) {
    const int tl = e >> 6, cl = e & 63;
    part[(int64_t)tl * AA->r_pad + cl] =
        ((red[0][tl][cl] + red[1][tl][cl]) + red[2][tl][cl]) + red[3][tl][cl];
  }
}

// pass 2: thread (token t, columns 4 q .. 4 q + 3); the slices' partials (at most
// kAppendMaxSlices) are all requested before the first is added.  Ranks are multiples of 8,
// so the four columns belong to one agent.
__global__ __launch_bounds__(256) void lr_append_sum_bf16(const AppendArgs args) {
  const AppendArgs* AA = (const AppendArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const PrecomputeArgs* P = &AA->p;
  const int R4 = P->R / 4;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= P->T * R4) return;
  const int t = (int)(e / R4), c = 4 * (int)(e % R4);
  const f32x4* src = (const f32x4*)(AA->part + (int64_t)t * AA->r_pad + c);
  const int64_t stride = (int64_t)AA->t_pad * AA->r_pad / 4;
  const int n = AA->n_slices;
  f32x4 p[kAppendMaxSlices];
#pragma unroll
  for (int s = 0; s < kAppendMaxSlices; ++s) p[s] = s < n ? src[s * stride] : f32x4{};
  f32x4 v = p[0];
#pragma unroll
  for (int s = 1; s < kAppendMaxSlices; ++s) v += p[s];
  int a = 0;
  while (a + 1 < P->n_agents && P->col_start[a + 1] <= c) ++a;
  bf16* Lp = (bf16*)P->Lout[a] + (int64_t)AA->rows[t] * P->ldl[a] + (c - P->col_start[a]);
#pragma unroll
  for (int j = 0; j < 4; ++j) Lp[j] = (bf16)v[j];
}

// fp32 append: one thread per (token, column), a plain fp32 dot product over d_model.
__global__ __launch_bounds__(256) void lr_append_f32(const AppendArgs args) {
  const AppendArgs* AA = (const AppendArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const PrecomputeArgs* P = &AA->p;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= P->T * P->R) return;
  const int64_t t = e / P->R;
  const int c = (int)(e % P->R);
  const float* x = (const float*)P->X + t * P->ldx;
  const float* A = (const float*)P->A + c;
  float v = 0.f;
  for (int64_t k = 0; k < P->d_model; ++k) v = fmaf(x[k], A[k * P->lda], v);
  int a = 0;
  while (a + 1 < P->n_agents && P->col_start[a + 1] <= c) ++a;
  float* Lp = (float*)P->Lout[a];
  Lp[(int64_t)AA->rows[t] * P->ldl[a] + (c - P->col_start[a])] = v;
}

}  // namespace

hipError_t launch_precompute_bf16(const PrecomputeArgs& a, hipStream_t s) {
  const int tiles = (int)((a.T + TM - 1) / TM);
#define LRA_LAUNCH(NCB) \
  hipLaunchKernelGGL((lr_precompute_bf16<NCB>), dim3(tiles), dim3(256), 0, s, a)
  switch ((a.R + 63) / 64) {              // 64-column groups of A_cat
    case 1: LRA_LAUNCH(4); break;
    case 2: LRA_LAUNCH(8); break;
    case 3: LRA_LAUNCH(12); break;
    default: LRA_LAUNCH(16); break;
  }
#undef LRA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_precompute_f32(const PrecomputeArgs& a, hipStream_t s) {
  const int rt = (int)((a.T + 63) / 64);
  const int ct = (a.R + 63) / 64;
  hipLaunchKernelGGL(lr_precompute_f32, dim3(rt, ct), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append_bf16(const AppendArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)a.n_slices, (unsigned)(a.t_pad / 64), (unsigned)(a.r_pad / 64));
  hipLaunchKernelGGL(lr_append_part_bf16, grid, dim3(1024), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = a.p.T * (a.p.R / 4);
  hipLaunchKernelGGL(lr_append_sum_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_append_f32(const AppendArgs& a, hipStream_t s) {
  const int64_t n = a.p.T * a.p.R;
  hipLaunchKernelGGL(lr_append_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lra
