// Flash-LoRA-Attention prefill, bf16 storage / fp32 accumulation, for gfx950 (MI355X).
//
// Computes, per request and query row of agent a (LRAgent summary, section
// "3. Flash-LoRA-Attention"):
//     O = P·V_base + (P·L_a)·B_a,   P = causal softmax(Q·K_baseᵀ / sqrt(D))
// with ONE online softmax shared by both products; L_a stays r wide inside the key loop
// and B_a is applied once per tile of query rows, after the loop.
//
// A workgroup owns one kv head g of one request and a tile of 256 (query, head-in-group)
// rows, row = t*G + h_local, so all q heads that share K/V_base read each LDS tile
// (GQA-aware).  Each of its 8 waves owns 32 rows and keeps its scores TRANSPOSED,
// Sᵀ = K·Qᵀ: with v_mfma_f32_32x32x16_bf16 a lane then holds one query row's scores for
// 16 keys, the row max/sum need a single cross-half permlane32 swap, and the score
// accumulator is already laid out as the B operand of the next products
// Oᵀ += V_baseᵀ·Pᵀ and (P·L)ᵀ += Lᵀ·Pᵀ (keys are permuted identically on both sides).
// K, V_base and L tiles of 64 keys stream HBM -> LDS with direct buffer->LDS loads;
// K/V rows are XOR-swizzled in 16-byte chunks against LDS bank conflicts.  V_base and L
// are read with ds_read_b64_tr_b16, which transposes 4x16 blocks inside 16-lane groups,
// so the caches keep their natural token-major layout in HBM and LDS.
//
// When the planner splits a request's key range over several workgroups (to fill the
// 256 CUs), each applies B to its own partial state (B is linear) and writes
// (m, l, P·V_base + (P·L)·B) to the workspace; fla_combine_bf16 then merges the splits
// with their softmax weights.  The decode kernel (fla_decode.hip) writes the same partial
// state and shares the combine pass.
#include "lra_device.h"

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

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima, gfx9 encoding); as a
// builtin the compiler knows the wait happened and places no second one for the same loads
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): all but the N most recently issued vector-memory loads are done
template <int N>
__device__ __forceinline__ void wait_loads_but() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// LDS layouts of the 64-key tiles (rows are D*2 bytes; 16-byte chunk c of row k lives at
// position c ^ swz(k)).  K is read by 32 consecutive rows at one chunk (ds_read_b128), V by
// ds_read_b64_tr_b16 over 4 consecutive rows x 4 consecutive chunks per half-wave; each
// swizzle makes its own read pattern bank-conflict free on the 64 x 4-byte LDS banks.
template <int D>
__device__ __forceinline__ int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

// dword 3 of a raw buffer resource on gfx9: 32-bit data format.  Loads at offsets past
// the record count return zeros without touching memory.
constexpr int kBufferFlags = 0x00020000;
constexpr int kOutOfRange = 0x7ffffff0;   // a byte offset past every record count used here

// Direct buffer->LDS loads of 64-key tiles.  A tile's buffer resource starts at its first
// key row and covers only the rows inside the key range, so rows past the range (and LR
// columns past the rank, addressed out of range) land in LDS as zeros.  Each wave writes
// the 1 KB LDS units u = wave, wave+4, ...; unit i of a wave lies NW*RPU rows (K/V) or 32
// rows (L) below its unit 0 with the same swizzle, so one per-lane byte offset, fixed for
// the whole key loop, plus a uniform stride addresses them all.  K/V rows are D*2 bytes;
// LDS slot p of a row holds source chunk p ^ swz(row), with swz_k for K and swz_v for V_base
// and B_g (the loader of a wave takes the one its tiles need).  The LR tile is 64 x 64 bf16
// (128-byte rows) whose 64-byte halves are swapped on rows with bit 1 set.
template <int D, int NW = 4>
struct TileLoader {
  static constexpr int CPR = D / 8;          // 16-byte chunks per K/V row
  static constexpr int RPU = 64 / CPR;       // rows per 1 KB unit
  static constexpr int UPW = 64 / RPU / NW;  // K (and V) units per wave
  static constexpr int LPW = 8 / NW;         // LR units per wave
  int uoff, loff;                            // unit 0 of the wave (K or V layout; L)
  __device__ __forceinline__ TileLoader(int wave, int lane, bool v_layout, int row_bytes,
                                        int l_row_bytes, int rank) {
    const int row = wave * RPU + lane / CPR;
    const int swz = v_layout ? swz_v<D>(row) : swz_k<D>(row);
    uoff = row * row_bytes + (((lane % CPR) ^ swz) << 4);
    const int lrow = wave * 8 + (lane >> 3);
    const int c = (lane & 7) ^ (((lrow >> 1) & 1) * 4);
    loff = c * 8 < rank ? lrow * l_row_bytes + c * 16 : kOutOfRange;
  }
  // byte offsets of unit i (unsigned wrap keeps an out-of-range L offset out of range)
  __device__ __forceinline__ int unit(int i, int row_bytes) const {
    return uoff + i * (NW * RPU) * row_bytes;
  }
  __device__ __forceinline__ int lunit(int i, int l_row_bytes) const {
    return (int)((unsigned)loff + (unsigned)(i * NW * 8 * l_row_bytes));
  }
};

// Workgroup barrier for LDS operations issued by the waves themselves.  Unlike a
// workgroup fence it does not wait for direct buffer->LDS loads still in flight (those
// count in vmcnt): the issuing wave waits for them itself (wait_loads) before the barrier
// that publishes them.  The empty asm statements keep the compiler from moving memory
// operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int bytes) {
  // wave-uniform record count: readfirstlane keeps the resource in SGPRs
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}

__device__ __forceinline__ void load_unit(__amdgpu_buffer_rsrc_t r, LDS char* dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (LDS void*)dst, 16, voff, 0, 0, 0);
}

// B operand for key step st (16 keys) from the transposed score/probability block.
__device__ __forceinline__ bf16x8 pfrag(const f32x16& s, int half) {
  bf16x8 r;
#pragma unroll
  for (int q = 0; q < 8; ++q) r[q] = (bf16)s[half * 8 + q];
  return r;
}

// Per-lane LDS byte offsets of the MFMA operands, fixed for the whole key loop.
template <int D>
struct Offsets {
  static constexpr int KS = D / 16, DB = D / 32;
  int k[KS];     // K rows (A of Sᵀ=K·Qᵀ): + kb2 * 32 * D*2
  int v[DB];     // V tr reads (A of Oᵀ+=Vᵀ·Pᵀ): + key base * D*2
  int l[2];      // LR tr reads (A of (P·L)ᵀ+=Lᵀ·Pᵀ): + key base * 128
  __device__ __forceinline__ Offsets(int lane) {
    const int col = lane & 31, hi = lane >> 5, g16 = lane >> 4, jj = lane & 15;
    const int sk = swz_k<D>(col);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) k[ks] = col * (D * 2) + (((2 * ks + hi) ^ sk) << 4);
    const int e = jj >> 2;                       // key within the 4-row group
    const int krow = hi * 4 + e;                 // + multiple of 8 (immediate)
    const int cl = (g16 & 1) * 2 + ((jj & 3) >> 1);
    const int sub = (jj & 1) * 8;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      v[db] = krow * (D * 2) + (((db * 4 + cl) ^ swz_v<D>(krow)) << 4) + sub;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int rho = rb * 32 + (g16 & 1) * 16 + (jj & 3) * 4;
      l[rb] = krow * 128 + ((rho * 2) ^ (((krow >> 1) & 1) * 64));
    }
  }
};

template <int D>
__device__ __forceinline__ bf16x8 vfrag(const LDS char* tile, int off, int key0) {
  i16x4 lo = tr_read(tile + off + key0 * (D * 2));
  i16x4 hi = tr_read(tile + off + (key0 + 8) * (D * 2));
  return join(lo, hi);
}

__device__ __forceinline__ bf16x8 lfrag(const LDS char* tile, int off, int key0) {
  i16x4 lo = tr_read(tile + off + key0 * 128);
  i16x4 hi = tr_read(tile + off + (key0 + 8) * 128);
  return join(lo, hi);
}

// Threshold (log2 units) by which a row max may exceed the running max before the
// accumulators are rescaled; probabilities then stay below 2^8, which fp32 and bf16 hold
// exactly as well as values below 1.
constexpr float kRescaleSlack = 8.0f;

// LDS reads the prefill matrix phase issues before the first MFMA of its P·V part
constexpr int kPfReads = 18;

// ---------------------------------------------------------------------------------------
// Prefill kernel, ping-pong schedule (the default prefill path).
//
// One 8-wave workgroup per CU; the two halves of the workgroup, A = waves 0-3 and
// B = waves 4-7, run half a tile apart.  Every SIMD holds
// one A and one B wave.  Workgroup barriers cut time into phases; in each phase one group
// issues only matrix work (P·V_base and P·L of the previous tile, then Sᵀ = K·Qᵀ of the
// current one) while the other runs only the softmax of its current tile, so each SIMD's
// matrix core and vector ALU are busy at the same time:
//
//   phase      0      1      2      3      4     ...
//   group A   M(0)   V(0)   M(1)   V(1)   M(2)
//   group B    -     M(0)   V(0)   M(1)   V(1)
//
// M(j) = PV(j-1) + S(j), V(j) = softmax(j).  Tile j is read in phases 2j..2j+3, so three
// LDS buffers rotate.  Each group issues part of the direct loads in its softmax phase:
// group A the K rows, group B the V_base and L rows (see step).  The loop is unrolled by three so that every LDS access
// names its buffer statically.
//
// EX (the in-tile expansion comparator, not the regrouped path): group B expands every
// V_base tile to full width in LDS, V_tile + L_tile·B_g, at the start of its matrix phase
// M(j), and attention runs without an adapter term.  B then waits for V(j+1) at the end of
// its softmax phase (three phases of latency, like K), so the tile is complete when the
// expansion starts.
// One work item w (of request b) of the prefill; the three rotating tile buffers (and, for
// EX, the B_g tile) are the calling kernel's LDS, sized for at least this RB.
template <int D, int RB, bool EX>
__device__ __forceinline__ void prefill_item(const AttnArgs* A, const int w, const int b,
                                             LDS char* const buf0, LDS char* const buf1,
                                             LDS char* const buf2, LDS char* const btile) {
  constexpr int DB = D / 32;
  constexpr int KS = D / 16;
  constexpr int TILE_KV = 64 * D * 2;
  constexpr int TILE_L = 64 * 64 * 2;
  constexpr int BUF = 2 * TILE_KV + (RB ? TILE_L : 0);
  constexpr int RBA = EX ? 0 : RB;     // rank blocks of the attention's LR term
  constexpr int kRows = kPrefillRows;
  const ReqDesc& R = A->reqs[b];
  const int q_start = R.q_start, Lq = R.q_len, k_start = R.k_start, Lk = R.k_len;
  const int n_rt = R.n_rt, n_split = R.n_split;
  int local = w - R.work_start;
  const int rt = __builtin_amdgcn_readfirstlane(local % n_rt);
  local /= n_rt;
  const int sp = __builtin_amdgcn_readfirstlane(local % n_split);
  const int g = __builtin_amdgcn_readfirstlane(local / n_split);
  const int G = A->G, Hq = A->Hq, Hkv = A->Hkv;
  const AgentDesc& AG = A->agents[R.agent];
  const int rank = RB ? AG.rank : 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_b = wave >= 4;
  const int col = lane & 31, hi = lane >> 5;
  const int rows_total = Lq * G;
  const int row0 = rt * kRows;
  const int my_row = row0 + wave * 32 + col;
  const bool valid = my_row < rows_total;
  const int t = valid ? my_row / G : 0;
  const int hl = valid ? my_row - t * G : 0;
  const int pos = valid ? Lk - Lq + t : Lk - 1;
  const bool wave_active = row0 + wave * 32 < rows_total;

  const int last_row = min(row0 + kRows, rows_total) - 1;
  const int kend_causal = Lk - Lq + last_row / G + 1;
  const int kmask_from = Lk - Lq + row0 / G + 1;
  const int n_tiles_req = (Lk + kTileKeys - 1) / kTileKeys;
  const int tps = (n_tiles_req + n_split - 1) / n_split;
  const int kb = __builtin_amdgcn_readfirstlane(sp * tps * kTileKeys);
  const int ke = __builtin_amdgcn_readfirstlane(min(min(Lk, kb + tps * kTileKeys), kend_causal));
  const int n_tiles = ke > kb ? (ke - kb + kTileKeys - 1) / kTileKeys : 0;
  const int mask_from = min(kmask_from, ke);
  const int vis_last = min(pos, ke - 1) - hi * 4;

  const int64_t kv_stride = (int64_t)Hkv * D;
  const bf16* Kg = (const bf16*)A->K + ((int64_t)k_start * Hkv + g) * D;
  const bf16* Vg = (const bf16*)A->V + ((int64_t)k_start * Hkv + g) * D;
  const int64_t ldl = RB ? AG.ldl : 0;   // read once: kernel-argument loads in the loop stall
  const bf16* Lg = RB ? (const bf16*)AG.L + (int64_t)k_start * ldl : nullptr;

  bf16x8 qf[KS];
  {
    const bf16* qrow = (const bf16*)A->Q + ((int64_t)(q_start + t) * Hq + g * G + hl) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = valid ? *(const bf16x8*)(qrow + ks * 16 + hi * 8) : bf16x8{};
  }
  const Offsets<D> off(lane);

  const int row_bytes = (int)(kv_stride * 2), l_row_bytes = (int)(ldl * 2);
  // tile loads are split by part: group A (waves 0-3) loads K, group B (waves 4-7) loads
  // V_base and L, each during its own softmax phase (see step below)
  const TileLoader<D, 4> ld(wave & 3, lane, group_b, row_bytes, l_row_bytes, rank);
  constexpr int N_K = TileLoader<D, 4>::UPW;                       // K loads per A wave
  constexpr int N_V = TileLoader<D, 4>::UPW + (RB ? TileLoader<D, 4>::LPW : 0);   // per B wave
  auto tile_rows = [&](int k0) {
    return __builtin_amdgcn_readfirstlane(max(0, min(ke - k0, kTileKeys)));
  };
  auto load_k = [&](int k0, LDS char* dst) {   // this A wave's units of K rows k0..k0+63
    const auto kr = rows_rsrc(Kg + (int64_t)k0 * kv_stride, tile_rows(k0) * row_bytes);
#pragma unroll
    for (int i = 0; i < N_K; ++i) load_unit(kr, dst + ((wave & 3) + 4 * i) * 1024, ld.unit(i, row_bytes));
  };
  auto load_vl = [&](int k0, LDS char* dst) {  // this B wave's units of V_base and L rows
    const int rows = tile_rows(k0);
    const auto vr = rows_rsrc(Vg + (int64_t)k0 * kv_stride, rows * row_bytes);
#pragma unroll
    for (int i = 0; i < TileLoader<D, 4>::UPW; ++i)
      load_unit(vr, dst + TILE_KV + ((wave & 3) + 4 * i) * 1024, ld.unit(i, row_bytes));
    if (RB) {
      const auto lr = rows_rsrc(rank > 0 ? (const void*)(Lg + (int64_t)k0 * ldl) : (const void*)Kg,
                                rank > 0 ? rows * l_row_bytes : 0);
#pragma unroll
      for (int i = 0; i < TileLoader<D, 4>::LPW; ++i)
        load_unit(lr, dst + 2 * TILE_KV + ((wave & 3) + 4 * i) * 1024, ld.lunit(i, l_row_bytes));
    }
  };

  f32x16 accV[DB];
  f32x16 accL[RBA > 0 ? RBA : 1];
#pragma unroll
  for (int i = 0; i < DB; ++i) accV[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < (RBA > 0 ? RBA : 1); ++i) accL[i] = f32x16{};
  float m_run = kNegBig, l_run = 0.f;
  const float sl2 = A->scale_log2;
  f32x16 s[2];
  bf16x8 pf[4] = {};   // P of the previous tile as B operands, 16 keys each (tile -1: zero)

  // matrix phase M(j): PV(j-1) from vbuf, then Sᵀ(j) from kbuf.  Both parts run in every
  // step: step 0's P·V adds P = 0 times the zeroed rows of "tile -1", and the last step's
  // scores (j == n_tiles, from a stale K tile) are never used.  Without the conditions the
  // compiler keeps the LDS reads ahead of the MFMAs in all three unrolled steps (with them,
  // one step of the rank > 32 kernel waited on every read).
  auto mma_phase = [&](int j, const LDS char* kbuf, const LDS char* vbuf) {
    if (!wave_active) return;
    {
      const LDS char* vt = vbuf + TILE_KV;
      const LDS char* lt = vbuf + 2 * TILE_KV;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int key0 = (st >> 1) * 32 + (st & 1) * 16;
#pragma unroll
        for (int db = 0; db < DB; ++db) accV[db] = mfma32(vfrag<D>(vt, off.v[db], key0), pf[st], accV[db]);
#pragma unroll
        for (int rb = 0; rb < RBA; ++rb) accL[rb] = mfma32(lfrag(lt, off.l[rb], key0), pf[st], accL[rb]);
      }
      // scheduling: kPfReads LDS reads first, then one MFMA per two further reads, so each
      // MFMA's operands were requested several MFMAs earlier (the compiler's own order kept
      // only one fragment in flight and the MFMAs waited on LDS latency)
      constexpr int NR = 8 * DB + 8 * RBA, NM = 4 * DB + 4 * RBA;   // LDS reads, MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, kPfReads, 0);
#pragma unroll
      for (int i = 0; i < (NR - kPfReads) / 2; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NM - (NR - kPfReads) / 2, 0);
    }
    {
      // the two 32-key blocks alternate, so consecutive MFMAs are independent
      s[0] = f32x16{};
      s[1] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 k0f = *(const LDS bf16x8*)(kbuf + off.k[ks]);
        const bf16x8 k1f = *(const LDS bf16x8*)(kbuf + off.k[ks] + 32 * (D * 2));
        s[0] = mfma32(k0f, qf[ks], s[0]);
        s[1] = mfma32(k1f, qf[ks], s[1]);
      }
      // (the same pattern for the score part: 8 reads ahead)
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < KS - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, KS + 4, 0);
    }
  };
  // vector phase V(j): mask, online softmax, P(j) to bf16 fragments
  auto valu_phase = [&](int j) {
    if (!wave_active || j >= n_tiles) return;
    const int k0 = kb + j * kTileKeys;
    if (k0 + kTileKeys > mask_from) {
      // causal mask as an additive penalty, -inf where the key lies past the row's last
      // visible key (the sign of lim - key), else +0: pure vector arithmetic.  Written as
      // compares, the 32 lane masks are kept in scalar register pairs and push the kernel's
      // loop-carried scalars into VGPR-lane spills that every phase reloads.
      const int lim = vis_last - k0;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int d = lim - (kb2 * 32 + (e >> 2) * 8 + (e & 3));
          s[kb2][e] += __builtin_bit_cast(float, (d >> 31) & (int)0xff800000u);
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int e = 0; e < 16; e += 2) mx = fmaxf(mx, fmaxf(s[kb2][e], s[kb2][e + 1]));
    mx = half_max(mx) * sl2;
    if (__any(mx > m_run + kRescaleSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) accV[i] *= alpha;
#pragma unroll
      for (int i = 0; i < RBA; ++i) accL[i] *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb2][e], sl2, -m_run));
        s[kb2][e] = p;
        psum += p;
      }
    l_run += psum;
#pragma unroll
    for (int st = 0; st < 4; ++st) pf[st] = pfrag(s[st >> 1], st & 1);
  };
  // In-tile expansion of tile j (group B, EX): V_tile += L_tile·B_g as the MFMA product
  // (L·B_g)ᵀ = B_gᵀ·Lᵀ.  B_g sits in btile in the V tile layout, so vfrag reads B_gᵀ with the
  // same permuted k slots as the keys of Oᵀ += Vᵀ·Pᵀ; the L operand supplies ranks
  // r0 + hi*4 + (0..3) and r0 + 8 + hi*4 + (0..3) of one key row.  Units are (32-lane head
  // block, 32-key block); each B wave takes every fourth.
  auto expand_tile = [&](LDS char* vt, const LDS char* lt) {
    if (rank <= 0) return;
    for (int u = wave & 3; u < DB * 2; u += 4) {
      const int db = u % DB, key = (u / DB) * 32 + col;
      const int lswap = ((key >> 1) & 1) * 64;
      f32x16 c = f32x16{};
      for (int r0 = 0; r0 < rank; r0 += 16) {
        const i16x4 l0 = *(const LDS i16x4*)(lt + key * 128 + (((r0 + hi * 4) * 2) ^ lswap));
        const i16x4 l1 = *(const LDS i16x4*)(lt + key * 128 + (((r0 + 8 + hi * 4) * 2) ^ lswap));
        c = mfma32(vfrag<D>(btile, off.v[db], r0), join(l0, l1), c);
      }
      // lane holds key `key`, head lanes db*32 + 8*i + 4*hi .. +3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = db * 32 + i * 8 + hi * 4;
        LDS char* vp = vt + key * (D * 2) + (((d >> 3) ^ swz_v<D>(key)) << 4) + (d & 7) * 2;
        const bf16x4 vb = __builtin_bit_cast(bf16x4, *(LDS i16x4*)vp);
        bf16x4 o;
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) o[j2] = (bf16)((float)vb[j2] + c[i * 4 + j2]);
        *(LDS bf16x4*)vp = o;
      }
    }
  };
  // one step j of this wave's program (two barriers), buffers named statically.
  //  - K(t) is read in phases 2t and 2t+1; group A issues it as it enters V(t-2) (phase
  //    2t-3) and waits for it at the end of V(t-1): three phases of latency.
  //  - V_base(t) and L(t) are read in phases 2t+2 and 2t+3; group B issues them as it
  //    enters V(t-2) (phase 2t-2) and waits for them at the end of M(t): four phases.
  // Each wait leaves the next tile's loads in flight (vmcnt(N)), except where no next tile
  // was issued.  With the parts split, both softmax phases carry a share of the issue work.
  auto step = [&](int j, LDS char* kbuf, const LDS char* vbuf, LDS char* dma) {
    // the matrix phase runs at raised wave priority so the SIMD's arbiter serves its
    // MFMA and LDS issue ahead of the partner wave's softmax
    __builtin_amdgcn_s_setprio(2);
    if (EX && group_b && j < n_tiles) expand_tile(kbuf + TILE_KV, kbuf + 2 * TILE_KV);
    mma_phase(j, kbuf, vbuf);
    __builtin_amdgcn_s_setprio(0);
    if (!EX && group_b) {                // V(j) complete; V(j+1) may stay in flight
      if (j + 1 < n_tiles) wait_loads_but<N_V>();
      else wait_loads();
    }
    lds_barrier();
    if (j + 2 < n_tiles) {
      if (group_b) load_vl(kb + (j + 2) * kTileKeys, dma);
      else load_k(kb + (j + 2) * kTileKeys, dma);
    }
    valu_phase(j);
    if (!group_b) {                      // K(j+1) complete; K(j+2) may stay in flight
      if (j + 2 < n_tiles) wait_loads_but<N_K>();
      else wait_loads();
    } else if (EX) {                     // V(j+1) complete; V(j+2) may stay in flight
      if (j + 2 < n_tiles) wait_loads_but<N_V>();
      else wait_loads();
    }
    lds_barrier();
  };

  // the first step's P·V reads "tile -1" from buf2 with P = 0: its V and L rows are zeroed
  // (uninitialised LDS could hold NaN patterns)
  for (int o = tid * 16; o < BUF - TILE_KV; o += 512 * 16)
    *(LDS f32x4*)(buf2 + TILE_KV + o) = f32x4{0.f, 0.f, 0.f, 0.f};
  // prologue: K(0), K(1) and V(0) before phase 0; B issues V(1) in its extra phase 0
  if (!group_b) {
    if (n_tiles > 0) load_k(kb, buf0);
    if (n_tiles > 1) load_k(kb + kTileKeys, buf1);
    if (n_tiles > 1) wait_loads_but<N_K>();
    else wait_loads();
  } else {
    if (n_tiles > 0) load_vl(kb, buf0);
    if (EX && rank > 0) {             // B_g as a 64-row value tile, rows past the rank zero
      const auto br = rows_rsrc((const bf16*)AG.B + g * D, rank * row_bytes);
#pragma unroll
      for (int i = 0; i < TileLoader<D, 4>::UPW; ++i)
        load_unit(br, btile + ((wave & 3) + 4 * i) * 1024, ld.unit(i, row_bytes));
    }
    wait_loads();
  }
  lds_barrier();
  if (group_b) {               // B starts one phase late
    if (n_tiles > 1) load_vl(kb + kTileKeys, buf1);
    lds_barrier();
  }
  for (int j = 0; j <= n_tiles; j += 3) {
    step(j, buf0, buf2, buf2);
    if (j + 1 <= n_tiles) step(j + 1, buf1, buf0, buf0);
    if (j + 2 <= n_tiles) step(j + 2, buf2, buf1, buf1);
  }
  if (!group_b) lds_barrier();   // matches B's extra barrier at the start

  // ---- epilogue: acc = P·V_base + (P·L)·B_g with B applied once for the row tile; a
  // whole key range is normalised by l and stored as bf16 O, a key split stores its
  // unnormalised fp32 state (m, l, acc) for fla_combine_bf16.
  const float l_tot = half_sum(l_run);
  const float inv = n_split == 1 ? 1.f / l_tot : 1.f;
  if (n_split == 1) {
#pragma unroll
    for (int i = 0; i < DB; ++i) accV[i] *= inv;
  }
  if (RBA && rank > 0) {
    wait_loads();                 // nothing of the key loop is still in flight
    if (group_b) {
      const auto br = rows_rsrc((const bf16*)AG.B + g * D, rank * row_bytes);
#pragma unroll
      for (int i = 0; i < TileLoader<D, 4>::UPW; ++i)
        load_unit(br, buf0 + TILE_KV + ((wave & 3) + 4 * i) * 1024, ld.unit(i, row_bytes));
      wait_loads();
    }
    lds_barrier();
    if (wave_active) {
      const int nst = (rank + 15) / 16;
      for (int st = 0; st < nst; ++st) {
        const f32x16 lsc = accL[(RB > 1) ? (st >> 1) : 0] * inv;
        const bf16x8 p2 = pfrag(lsc, st & 1);
        const int key0 = (st >> 1) * 32 + (st & 1) * 16;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          accV[db] = mfma32(vfrag<D>(buf0 + TILE_KV, off.v[db], key0), p2, accV[db]);
      }
    }
  }
  if (!valid) return;
  if (n_split == 1) {
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
  } else {
    const int64_t pr = (int64_t)R.part_base + ((int64_t)sp * Lq + t) * Hq + g * G + hl;
    float* po = A->ws_o + pr * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *(f32x4*)(po + db * 32 + i * 8 + hi * 4) =
            f32x4{accV[db][i * 4], accV[db][i * 4 + 1], accV[db][i * 4 + 2], accV[db][i * 4 + 3]};
    if (hi == 0) *(float2*)(A->ws_ml + pr * 2) = float2{m_run, l_tot};
  }
}

// blockIdx -> work item: XCD-major for one request (grid_per_xcd > 0), else dealt in
// chunks of kDealChunk items round-robin over the XCDs
__device__ __forceinline__ int prefill_work_item(const AttnArgs* A) {
  const int bid = blockIdx.x;
  return A->grid_per_xcd > 0
             ? (bid & 7) * A->grid_per_xcd + (bid >> 3)
             : ((bid >> 3) / kDealChunk) * (8 * kDealChunk) + (bid & 7) * kDealChunk +
                   (bid >> 3) % kDealChunk;
}

template <int D, int RB, bool EX>
__global__ __launch_bounds__(512, 1) void fla_prefill_bf16(const AttnArgs args) {
  const AttnArgs* A = (const AttnArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int TILE_KV = 64 * D * 2;
  constexpr int BUF = 2 * TILE_KV + (RB ? 64 * 64 * 2 : 0);
  __shared__ __attribute__((aligned(1024))) char smem0[BUF];
  __shared__ __attribute__((aligned(1024))) char smem1[BUF];
  __shared__ __attribute__((aligned(1024))) char smem2[BUF];
  __shared__ __attribute__((aligned(1024))) char smemb[EX ? TILE_KV : 16];
  const int w = prefill_work_item(A);
  if (w >= A->n_work) return;
  prefill_item<D, RB, EX>(A, w, find_request(A, w), (LDS char*)smem0, (LDS char*)smem1,
                          (LDS char*)smem2, (LDS char*)smemb);
}

// A launch whose requests span LR widths (ranks 0, up to 32 and up to 64): each work item
// runs the loop of its own agent's width, so a rank-16 request next to rank-64 ones does
// not pay for the wider LR term (in one launch, without a second launch's tail).
template <int D>
__global__ __launch_bounds__(512, 1) void fla_prefill_mixed_bf16(const AttnArgs args) {
  const AttnArgs* A = (const AttnArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int BUF = 2 * 64 * D * 2 + 64 * 64 * 2;
  __shared__ __attribute__((aligned(1024))) char smem0[BUF];
  __shared__ __attribute__((aligned(1024))) char smem1[BUF];
  __shared__ __attribute__((aligned(1024))) char smem2[BUF];
  __shared__ __attribute__((aligned(1024))) char smemb[16];
  const int w = prefill_work_item(A);
  if (w >= A->n_work) return;
  const int b = find_request(A, w);
  const int rank = __builtin_amdgcn_readfirstlane(A->agents[A->reqs[b].agent].rank);
  LDS char* const b0 = (LDS char*)smem0;
  LDS char* const b1 = (LDS char*)smem1;
  LDS char* const b2 = (LDS char*)smem2;
  LDS char* const bt = (LDS char*)smemb;
  if (rank > 32) prefill_item<D, 2, false>(A, w, b, b0, b1, b2, bt);
  else if (rank > 0) prefill_item<D, 1, false>(A, w, b, b0, b1, b2, bt);
  else prefill_item<D, 0, false>(A, w, b, b0, b1, b2, bt);
}

// Merge the key-split states of one output row:
//   M = max m_s, w_s = 2^(m_s - M),   O = Σ w_s·acc_s / Σ w_s·l_s
// where acc_s = (P·V_base)_s + (P·L)_s·B_g already holds the up-projection (B is linear).
// D/VPT threads per row, each owning VPT consecutive output lanes; the splits are merged
// NB at a time with all of their loads in flight before the first is used.  The pass is
// bound by load latency: many rows (a split prefill) take VPT = 16, so that a wave keeps
// several KB of loads outstanding; few rows with many splits (decode) take VPT = 4 and
// NB = 8, so that the launch still spreads over the CUs.
template <int D, int VPT, int NB>
__global__ __launch_bounds__(256) void fla_combine_bf16(const AttnArgs args) {
  const AttnArgs* A = (const AttnArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int TPR = D / VPT, RPB = 256 / TPR;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  const int c0 = (threadIdx.x % TPR) * VPT;
  const int b = find_combine_request(A, min(row, A->n_comb - 1));   // whole wave
  if (row >= A->n_comb) return;
  const ReqDesc& R = A->reqs[b];
  const int Hq = A->Hq;
  const int local = row - R.comb_start;
  const int t = local / Hq, h = local - t * Hq;
  const int S = R.n_split;
  const int64_t p0 = (int64_t)R.part_base + (int64_t)t * Hq + h;
  const int64_t pstride = (int64_t)R.q_len * Hq;
  float M = kNegBig, l = 0.f;
  f32x4 o[VPT / 4] = {};
  for (int s0 = 0; s0 < S; s0 += NB) {
    float2 ml[NB];
    f32x4 v[NB][VPT / 4];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t pr = p0 + (int64_t)(s0 + i) * pstride;
      ml[i] = float2{kNegBig, 0.f};
#pragma unroll
      for (int k = 0; k < VPT / 4; ++k) v[i][k] = f32x4{};
      if (s0 + i < S) {
        ml[i] = *(const float2*)(A->ws_ml + pr * 2);
#pragma unroll
        for (int k = 0; k < VPT / 4; ++k) v[i][k] = *(const f32x4*)(A->ws_o + pr * D + c0 + 4 * k);
      }
    }
    float Mc = M;
#pragma unroll
    for (int i = 0; i < NB; ++i) Mc = fmaxf(Mc, ml[i].x);
    const float sc = __builtin_amdgcn_exp2f(M - Mc);
    l *= sc;
#pragma unroll
    for (int k = 0; k < VPT / 4; ++k) o[k] *= sc;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float w = __builtin_amdgcn_exp2f(ml[i].x - Mc);   // 0 for absent splits
      l += w * ml[i].y;
#pragma unroll
      for (int k = 0; k < VPT / 4; ++k) o[k] += w * v[i][k];
    }
    M = Mc;
  }
  const float inv = 1.f / l;
  bf16* orow = (bf16*)A->O + ((int64_t)(R.q_start + t) * Hq + h) * D + c0;
  if constexpr (VPT % 8 == 0) {   // 16-byte stores
#pragma unroll
    for (int k = 0; k < VPT / 4; k += 2) {
      bf16x8 ob;
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) {
        ob[j2] = (bf16)(o[k][j2] * inv);
        ob[4 + j2] = (bf16)(o[k + 1][j2] * inv);
      }
      *(bf16x8*)(orow + 4 * k) = ob;
    }
  } else {
#pragma unroll
    for (int k = 0; k < VPT / 4; ++k) {
      bf16x4 ob;
#pragma unroll
      for (int j2 = 0; j2 < 4; ++j2) ob[j2] = (bf16)(o[k][j2] * inv);
      *(bf16x4*)(orow + 4 * k) = ob;
    }
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnArgs& a, int head_dim, int max_rank, int n_grid,
                               hipStream_t s, bool expand, int min_rank) {
  const int rb = max_rank > 32 ? 2 : (max_rank > 0 ? 1 : 0);
  const int rb_lo = min_rank < 0 ? rb : (min_rank > 32 ? 2 : (min_rank > 0 ? 1 : 0));
  if (!expand && rb_lo != rb) {        // the launch spans LR widths
    if (head_dim == 128)
      hipLaunchKernelGGL((fla_prefill_mixed_bf16<128>), dim3(n_grid), dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((fla_prefill_mixed_bf16<64>), dim3(n_grid), dim3(512), 0, s, a);
    return hipGetLastError();
  }
#define LRA_LAUNCH(D, RB, EX) \
  hipLaunchKernelGGL((fla_prefill_bf16<D, RB, EX>), dim3(n_grid), dim3(512), 0, s, a)
  if (expand && rb > 0) {
    if (head_dim == 128) {
      if (rb == 1) LRA_LAUNCH(128, 1, true);
      else LRA_LAUNCH(128, 2, true);
    } else {
      if (rb == 1) LRA_LAUNCH(64, 1, true);
      else LRA_LAUNCH(64, 2, true);
    }
  } else if (head_dim == 128) {
    if (rb == 0) LRA_LAUNCH(128, 0, false);
    else if (rb == 1) LRA_LAUNCH(128, 1, false);
    else LRA_LAUNCH(128, 2, false);
  } else {
    if (rb == 0) LRA_LAUNCH(64, 0, false);
    else if (rb == 1) LRA_LAUNCH(64, 1, false);
    else LRA_LAUNCH(64, 2, false);
  }
#undef LRA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_combine_bf16(const AttnArgs& a, int head_dim, hipStream_t s) {
  // 16 values per thread once that still gives at least 256 blocks
  const bool wide = (int64_t)a.n_comb * (head_dim / 16) >= 256 * 256;
  const int rpb = 256 / (head_dim / (wide ? 16 : 4));   // rows per block
  const int grid = (a.n_comb + rpb - 1) / rpb;
#define LRA_COMBINE(D, VPT, NB) \
  hipLaunchKernelGGL((fla_combine_bf16<D, VPT, NB>), dim3(grid), dim3(kThreads), 0, s, a)
  if (head_dim == 128) {
    if (wide) LRA_COMBINE(128, 16, 4);
    else LRA_COMBINE(128, 4, 8);
  } else {
    if (wide) LRA_COMBINE(64, 16, 4);
    else LRA_COMBINE(64, 4, 8);
  }
#undef LRA_COMBINE
  return hipGetLastError();
}

}  // namespace lra
