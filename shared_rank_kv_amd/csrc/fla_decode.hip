// Flash-LoRA-Attention decode (one query token per request), bf16 storage / fp32
// accumulation, for gfx950 (MI355X).
//
// Same computation as the prefill kernel (LRAgent summary, section "3. Flash-LoRA-
// Attention": O = P·V_base + (P·L_a)·B_a with one online softmax), specialised for the
// HBM-bound decode shape: per (request, kv head) there are only G = Hq/Hkv query rows, so
// the work is streaming K/V_base/L rows at full bandwidth.
//
// A workgroup owns one (request, kv head, key split).  Each of its 4 waves streams its own
// interleaved 32-key tiles with an independent online-softmax state, so the loop has no
// workgroup barrier:
//  - K rows are loaded straight into v_mfma_f32_16x16x32_bf16 A-operand registers
//    (lane = key row, 8 consecutive d); scores are kept transposed, Sᵀ = K·Qᵀ, with the G
//    query rows as the 16 MFMA columns;
//  - V_base and L rows are staged through registers into a wave-private LDS tile and read
//    back with ds_read_b64_tr_b16 as the A operand of Oᵀ += V_baseᵀ·Pᵀ and
//    (P·L)ᵀ += Lᵀ·Pᵀ (the score accumulator is already the B operand);
//  - the next tile's K, V and L loads are in flight while the current tile computes.
// At the end the four wave states are merged through LDS, B_g is applied once
// (B is linear), and the key split's state (m, l, P·V_base + (P·L)·B) goes to the
// workspace for fla_combine_bf16, or O is written when the request has one split.
#include "lra_device.h"

namespace lra {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr float kNegBig = -1.0e30f;
constexpr float kRescaleSlack = 8.0f;      // log2 units (see the prefill kernel)
constexpr int kKeys = 32;                  // keys per wave tile

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

// max / sum over the four lanes l, l^16, l^32, l^48 that hold one query column
__device__ __forceinline__ float col_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float col_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// V tile swizzle: 16-byte chunk c of tile row k sits at chunk position c ^ vswz(k), which
// keeps the transposing reads (8 rows x 2 chunks per half-wave) bank-conflict free.
template <int D>
__device__ __forceinline__ int vswz(int k) { return D == 128 ? 2 * (k & 7) : 2 * ((k >> 1) & 3); }

// EX (the in-tile expansion comparator, not the regrouped path): every V_base tile is
// expanded to full width in LDS, V_tile + L_tile·B_g, before P·V, and attention then runs
// without an adapter term.  B_g stays in LDS for the whole work item; RB sizes its rank
// steps.
template <int D, int RB, bool EX>
__global__ __launch_bounds__(256, 2) void fla_decode_bf16(const AttnArgs args) {
  const AttnArgs* A = (const AttnArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  constexpr int DB = D / 16;                 // 16-row blocks of the transposed output
  constexpr int KS = D / 32;                 // k-steps of the score product
  constexpr int VT = kKeys * D * 2;          // V tile bytes (per wave)
  constexpr int LT = kKeys * 64 * 2;         // LR tile bytes (per wave, rank <= 64)
  constexpr int VLOADS = VT / 1024;          // 16-byte V loads per lane per tile
  constexpr int RBA = EX ? 0 : RB;           // rank blocks of the attention's LR term
  constexpr int NRB = RBA > 0 ? RBA * 2 : 1; // 16-column blocks of the LR accumulator
  constexpr int NL = RB == 2 ? 4 : 2;        // 16-byte L loads per lane per tile
  constexpr int NBU = D / 32;                // 16-byte units of a 64-row B tile per thread
  constexpr int BT = EX ? 32 * RB * D * 2 : 0;   // B_g tile (in-tile expansion)
  __shared__ __attribute__((aligned(1024))) char smem_raw[4 * (VT + LT) + BT];
  LDS char* smem = (LDS char*)smem_raw;

  const int bid = blockIdx.x;
  const int w = (bid & 7) * A->grid_per_xcd + (bid >> 3);
  if (w >= A->n_work) return;
  const int b = find_request(A, w);
  const ReqDesc& R = A->reqs[b];
  const int k_start = R.k_start, Lk = R.k_len, n_split = R.n_split;
  const int G = A->G, Hq = A->Hq, Hkv = A->Hkv;
  // the kv heads of one key split are adjacent work items: they share the split's L rows
  const int local = w - R.work_start;
  const int g = local % Hkv;
  const int sp = local / Hkv;
  const AgentDesc& AG = A->agents[R.agent];
  const int rank = RB ? AG.rank : 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop control
  const int col = lane & 15, grp = lane >> 4;

  // key range of this split, in 32-key tiles dealt round-robin to the 4 waves
  const int n_tiles_req = (Lk + kKeys - 1) / kKeys;
  const int tps = (n_tiles_req + n_split - 1) / n_split;
  const int kb = sp * tps * kKeys;
  const int ke = min(Lk, kb + tps * kKeys);
  const int n_tiles = ke > kb ? (ke - kb + kKeys - 1) / kKeys : 0;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0;

  const int64_t kv_stride = (int64_t)Hkv * D;
  const bf16* Kg = (const bf16*)A->K + ((int64_t)k_start * Hkv + g) * D;
  const bf16* Vg = (const bf16*)A->V + ((int64_t)k_start * Hkv + g) * D;
  const bf16* Lg = RB ? (const bf16*)AG.L + (int64_t)k_start * AG.ldl : nullptr;

  // Q (B operand of Sᵀ = K·Qᵀ): lane holds Q[head g*G + col][ks*32 + grp*8 .. +7]
  bf16x8 qf[KS];
  {
    const bf16* qrow = (const bf16*)A->Q + ((int64_t)R.q_start * Hq + g * G + col) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = col < G ? *(const bf16x8*)(qrow + ks * 32 + grp * 8) : bf16x8{};
  }

  LDS char* vt = smem + wave * (VT + LT);
  LDS char* lt = vt + VT;
  // LR tile: 32 rows x 64 bf16 (128-byte rows); columns past the rank stay zero
  if (RB) {
#pragma unroll
    for (int i = 0; i < LT / 1024; ++i) *(LDS u32x4*)(lt + i * 1024 + lane * 16) = u32x4{};
  }

  // per-lane load geometry, fixed for the loop:
  //  K: key row (kb2*16 + col), chunk (ks*4 + grp)  -> A operand of Sᵀ
  //  V: load i covers tile row i*(64/CPR) + lane/CPR, chunk lane%CPR
  //  L: 16-byte unit u = lane + 64*i of the 32 x rank tile: row u/(rank/8), chunk u%(rank/8)
  // Units past the tile (or all of them for a rank-0 agent, whose L may be null) load a
  // valid K row instead and store zeros into column chunk 7, which lies past the rank in
  // exactly those cases: loads and stores stay unconditional, so the loop has no branches.
  const int cpr_l = rank > 0 ? rank / 8 : 1;
  const bf16* l_src = rank > 0 ? Lg : Kg;
  const int64_t l_ld = rank > 0 ? AG.ldl : kv_stride;
  int l_row[NL], l_chunk[NL], l_dst[NL];
  bool l_ok[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int u = lane + 64 * i;
    const int r = u / cpr_l, c = u - r * cpr_l;
    l_ok[i] = rank > 0 && r < kKeys;
    l_row[i] = l_ok[i] ? r : 0;
    l_chunk[i] = l_ok[i] ? c : 0;
    l_dst[i] = l_ok[i] ? r * 128 + c * 16 : (u % kKeys) * 128 + 7 * 16;
  }
  u32x4 kreg[2][KS];
  u32x4 vreg[VLOADS];
  u32x4 lreg[NL];
  // Tiles past the wave's last one clamp to key ke-1: the loop prefetches without branches.
  auto tile_key = [&](int jt) { return kb + (wave + 4 * jt) * kKeys; };
  auto load_k = [&](int jt) {
    const int k0 = tile_key(jt);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int key = min(k0 + kb2 * 16 + col, ke - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kreg[kb2][ks] = *(const u32x4*)(Kg + (int64_t)key * kv_stride + (ks * 4 + grp) * 8);
    }
  };
  auto load_vl = [&](int jt) {
    const int k0 = tile_key(jt);
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int key = min(k0 + i * (64 / CPR) + lane / CPR, ke - 1);
      vreg[i] = *(const u32x4*)(Vg + (int64_t)key * kv_stride + (lane % CPR) * 8);
    }
    if (RB) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int key = min(k0 + l_row[i], ke - 1);
        lreg[i] = *(const u32x4*)(l_src + (int64_t)key * l_ld + l_chunk[i] * 8);
      }
    }
  };
  auto store_vl = [&]() {
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int row = i * (64 / CPR) + lane / CPR;
      const int c = (lane % CPR) ^ vswz<D>(row);
      *(LDS u32x4*)(vt + row * (D * 2) + c * 16) = vreg[i];
    }
    if (RB) {
#pragma unroll
      for (int i = 0; i < NL; ++i)
        *(LDS u32x4*)(lt + l_dst[i]) = l_ok[i] ? lreg[i] : u32x4{};
    }
  };

  // transposing-read offsets: lane (e = (lane&15)/4, q = lane&3) of group grp supplies
  // 4 bf16 of key row grp*4 + e (and 16 + grp*4 + e), columns 16-block + 4q
  int voff[DB];
  const int trow = grp * 4 + ((lane & 15) >> 2), tq = lane & 3;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int d = db * 16 + tq * 4;
    voff[db] = trow * (D * 2) + (((d >> 3) ^ vswz<D>(trow)) << 4) + (d & 7) * 2;
  }

  f32x4 acc[DB];
  f32x4 accl[NRB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x4{};
#pragma unroll
  for (int i = 0; i < NRB; ++i) accl[i] = f32x4{};
  float m_run = kNegBig, l_run = 0.f;
  const float sl2 = A->scale_log2;

  // In-tile expansion: B_g [32 RB rows (zero past the rank), D] in the V tile layout, read
  // back transposed as the A operand of (L·B_g)ᵀ = B_gᵀ·Lᵀ, whose k slots are then the same
  // permuted ranks as the keys of Oᵀ += Vᵀ·Pᵀ (see voff); the L operand supplies ranks
  // kr*32 + grp*4 + (0..3) and kr*32 + 16 + grp*4 + (0..3) of one key row.
  LDS char* bt = smem + 4 * (VT + LT);
  if (EX) {
    const bf16* Bg = rank > 0 ? (const bf16*)AG.B + g * D : nullptr;
    for (int u = tid; u < 32 * RB * CPR; u += 256) {
      const int row = u / CPR, c = u % CPR;
      const u32x4 v = row < rank ? *(const u32x4*)(Bg + (int64_t)row * kv_stride + c * 8) : u32x4{};
      *(LDS u32x4*)(bt + row * (D * 2) + ((c ^ vswz<D>(row)) << 4)) = v;
    }
    __syncthreads();
  }
  auto expand_tile = [&]() {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int key = kb2 * 16 + col;
      bf16x8 lf[RB > 0 ? RB : 1];
#pragma unroll
      for (int kr = 0; kr < RB; ++kr) {
        const LDS char* p = lt + key * 128 + (kr * 32 + grp * 4) * 2;
        lf[kr] = join(*(const LDS i16x4*)p, *(const LDS i16x4*)(p + 32));
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4 c = f32x4{};
#pragma unroll
        for (int kr = 0; kr < RB; ++kr)
          c = mfma16(join(tr_read(bt + voff[db] + kr * 32 * D * 2),
                          tr_read(bt + voff[db] + (kr * 32 + 16) * D * 2)), lf[kr], c);
        // lane holds key `key`, head lanes db*16 + 4*grp .. +3
        const int d = db * 16 + grp * 4;
        LDS char* vp = vt + key * (D * 2) + (((d >> 3) ^ vswz<D>(key)) << 4) + (d & 7) * 2;
        const i16x4 raw = *(LDS i16x4*)vp;
        const bf16x4 vb = __builtin_bit_cast(bf16x4, raw);
        bf16x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = (bf16)((float)vb[j] + c[j]);
        *(LDS bf16x4*)vp = o;
      }
    }
  };

  if (my_tiles > 0) {
    load_k(0);
    load_vl(0);
    store_vl();
    if (EX) expand_tile();
    load_vl(1);
    for (int jt = 0; jt < my_tiles; ++jt) {
      const int k0 = tile_key(jt);
      // Sᵀ = K·Qᵀ: 2 blocks of 16 keys x 16 query columns
      f32x4 s[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        s[kb2] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s[kb2] = mfma16(__builtin_bit_cast(bf16x8, kreg[kb2][ks]), qf[ks], s[kb2]);
      }
      load_k(jt + 1);
      // mask keys past the range; online softmax over the column's 32 keys
      const int lim = ke - 1 - k0 - grp * 4;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kb2 * 16 + j > lim) s[kb2][j] = -INFINITY;
      float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      mx = col_max(mx) * sl2;
      if (__any(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) acc[i] *= alpha;
#pragma unroll
        for (int i = 0; i < NRB; ++i) accl[i] *= alpha;
      }
      bf16x8 pf;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb2][j], sl2, -m_run));
          l_run += p;
          pf[kb2 * 4 + j] = (bf16)p;
        }
      // Oᵀ += V_baseᵀ·Pᵀ and (P·L)ᵀ += Lᵀ·Pᵀ; MFMA k slot i of lane group grp is key
      // grp*4 + i (i < 4) or 16 + grp*4 + i-4, the order of pf
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc[db] = mfma16(join(tr_read(vt + voff[db]), tr_read(vt + voff[db] + 16 * D * 2)), pf,
                         acc[db]);
      if (RBA) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const LDS char* p = lt + trow * 128 + (rb * 16 + tq * 4) * 2;
          accl[rb] = mfma16(join(tr_read(p), tr_read(p + 16 * 128)), pf, accl[rb]);
        }
      }
      // the next tile's V and L replace this one: this wave's LDS reads above precede the
      // writes in program order, and the LDS executes one wave's operations in order
      store_vl();
      if (EX) expand_tile();
      load_vl(jt + 2);
    }
  }

  // ---- merge the 4 wave states through LDS, apply B once, store
  const float l_col = col_sum(l_run);
  // B_g rows (rank x D, bf16) to registers now; their latency overlaps the merge
  u32x4 breg[NBU];
  if (RBA) {
    const bf16* Bg = (const bf16*)AG.B + g * D;
#pragma unroll
    for (int i = 0; i < NBU; ++i) {
      const int u = tid + 256 * i, row = u / CPR, c = u % CPR;
      breg[i] = row < rank ? *(const u32x4*)(Bg + (int64_t)row * kv_stride + c * 8) : u32x4{};
    }
  }
  __syncthreads();   // every wave is done with its tiles
  LDS float* sh = (LDS float*)smem;              // [wave][8 cols][D]   P·V_base
  LDS float* shl = sh + 4 * 8 * D;               // [wave][8 cols][64]  P·L
  LDS float* shm = shl + 4 * 8 * 64;             // [wave][8 cols][2]   (m, l)
  LDS char* bs = (LDS char*)(shm + 4 * 8 * 2);   // [64][D] bf16        B_g
  LDS float* sa = (LDS float*)(bs + 64 * D * 2); // [8 cols][64]        merged P·L
  if (col < G) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) sh[(wave * 8 + col) * D + db * 16 + grp * 4 + j] = acc[db][j];
    if (RBA) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j) shl[(wave * 8 + col) * 64 + rb * 16 + grp * 4 + j] = accl[rb][j];
    }
    if (grp == 0) {
      shm[(wave * 8 + col) * 2] = m_run;
      shm[(wave * 8 + col) * 2 + 1] = l_col;
    }
  }
  if (RBA) {
#pragma unroll
    for (int i = 0; i < NBU; ++i) *(LDS u32x4*)(bs + (tid + 256 * i) * 16) = breg[i];
  }
  __syncthreads();

  // softmax weights of the four wave states of query column c
  auto weights = [&](int c, float* wgt, float& M, float& l) {
    M = kNegBig;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) M = fmaxf(M, shm[(wv * 8 + c) * 2]);
    l = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) {
      wgt[wv] = __builtin_amdgcn_exp2f(shm[(wv * 8 + c) * 2] - M);
      l += wgt[wv] * shm[(wv * 8 + c) * 2 + 1];
    }
  };
  if (RBA) {
    // merged P·L of every (column, rank index), columns past the rank hold zeros
#pragma unroll
    for (int e = tid; e < 8 * 64; e += 256) {
      const int c = e / 64, rho = e % 64;
      if (c < G) {
        float wgt[4], M, l;
        weights(c, wgt, M, l);
        float v = 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) v += wgt[wv] * shl[(wv * 8 + c) * 64 + rho];
        sa[c * 64 + rho] = v;
      }
    }
    __syncthreads();
  }
  // outputs: thread -> column pair 2*dp of query columns c0, c0 + 256/(D/2), ...
  constexpr int TPC = D / 2;
  const int dp = tid % TPC;
#pragma unroll
  for (int c = tid / TPC; c < 8; c += 256 / TPC) {
    if (c >= G) break;
    float wgt[4], M, l;
    weights(c, wgt, M, l);
    float o0 = 0.f, o1 = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) {
      const f32x2 v = *(const LDS f32x2*)(sh + (wv * 8 + c) * D + 2 * dp);
      o0 += wgt[wv] * v[0];
      o1 += wgt[wv] * v[1];
    }
    if (RBA) {
#pragma unroll
      for (int rho = 0; rho < RBA * 32; rho += 4) {
        const f32x4 a = *(const LDS f32x4*)(sa + c * 64 + rho);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const bf16x2 bv = *(const LDS bf16x2*)(bs + ((rho + k) * D + 2 * dp) * 2);
          o0 += a[k] * (float)bv[0];
          o1 += a[k] * (float)bv[1];
        }
      }
    }
    const int h = g * G + c;
    if (n_split == 1) {
      const float inv = 1.f / l;
      bf16x2 ob = {(bf16)(o0 * inv), (bf16)(o1 * inv)};
      *(bf16x2*)((bf16*)A->O + ((int64_t)R.q_start * Hq + h) * D + 2 * dp) = ob;
    } else {
      const int64_t pr = (int64_t)R.part_base + (int64_t)sp * Hq + h;
      *(float2*)(A->ws_o + pr * D + 2 * dp) = float2{o0, o1};
      if (dp == 0) *(float2*)(A->ws_ml + pr * 2) = float2{M, l};
    }
  }
}

// ---------------------------------------------------------------------------------------
// Shared-context decode.  Requests of different agents that read the same base rows (one
// base cache shared by the agents: BaseShared in the LRAgent summary, section 2; with all
// LR caches aliased, BaseLRShared) form a unit of up to kMaxMembers requests.  A work item
// (unit, kv head, key split) streams each K/V_base tile once for every member: the
// members' query heads fill the 16 columns of the score tile (column c is member c / G,
// head c % G), so the one P·V_base product serves them all.  Only the LR term is per
// member: every tile, each member's L rows pass through the wave's LR tile in turn and
// (P·L_a)ᵀ += L_aᵀ·Pᵀ runs with P masked to that member's columns, so one accumulator
// holds, in every column, the product with that column's own agent.  B_a is applied per
// member when the wave states are merged.  Members may have seen different lengths of the
// context (same first row): the first member is the longest and sets the key range, and
// each column's scores are masked past its own member's length (a split past it leaves
// that member the empty state, which the combine pass weighs zero).
// (Ranks up to 32 keep two workgroups per CU, with a few registers spilled outside the key
// loop; rank 64 needs the register file of one.)
template <int D, int RB>
__global__ __launch_bounds__(256, RB == 2 ? 1 : 2) void fla_decode_shared_bf16(const AttnArgs args) {
  const AttnArgs* A = (const AttnArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  constexpr int CPR = D / 8;                 // 16-byte chunks per K/V row
  constexpr int DB = D / 16;                 // 16-row blocks of the transposed output
  constexpr int KS = D / 32;                 // k-steps of the score product
  constexpr int VT = kKeys * D * 2;          // V tile bytes (per wave)
  constexpr int LT = kKeys * 64 * 2;         // LR tile bytes (per wave, rank <= 64)
  constexpr int VLOADS = VT / 1024;          // 16-byte V loads per lane per tile
  constexpr int NRB = RB > 0 ? RB * 2 : 1;   // 16-column blocks of the LR accumulator
  constexpr int LCH = RB > 0 ? 4 * RB : 1;   // 16-byte chunks of the LR columns loaded per row
  constexpr int NL = RB > 0 ? kKeys * LCH / 64 : 0;   // 16-byte L loads per lane per member
  constexpr int NM = kMaxMembers;
  constexpr int LOOP_LDS = 4 * (VT + LT);
  constexpr int MERGE_LDS = (4 * 16 * D + 4 * 16 * 64 + 4 * 16 * 2 + 16 * 64) * 4;
  __shared__ __attribute__((aligned(1024)))
  char smem_raw[LOOP_LDS > MERGE_LDS ? LOOP_LDS : MERGE_LDS];
  LDS char* smem = (LDS char*)smem_raw;

  const int bid = blockIdx.x;
  const int w = (bid & 7) * A->grid_per_xcd + (bid >> 3);
  if (w >= A->n_work) return;
  const int b = find_unit(A, w);
  const ReqDesc& R = A->reqs[b];
  const int nm = __builtin_amdgcn_readfirstlane(R.n_members);
  const int k_start = R.k_start, Lk = R.k_len, n_split = R.n_split;
  const int G = A->G, Hq = A->Hq, Hkv = A->Hkv;
  const int local = w - R.work_start;
  const int g = local % Hkv;
  const int sp = local / Hkv;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop control
  const int col = lane & 15, grp = lane >> 4;
  const int mcol = col / G;                  // member of this lane's query column
  const bool col_ok = mcol < nm;
  // keys of this lane's member: the first member is the longest, the others see a prefix
  const int my_len = col_ok ? A->reqs[b + mcol].k_len : Lk;

  // key range of this split, in 32-key tiles dealt round-robin to the 4 waves
  const int n_tiles_req = (Lk + kKeys - 1) / kKeys;
  const int tps = (n_tiles_req + n_split - 1) / n_split;
  const int kb = sp * tps * kKeys;
  const int ke = min(Lk, kb + tps * kKeys);
  const int n_tiles = ke > kb ? (ke - kb + kKeys - 1) / kKeys : 0;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0;

  const int64_t kv_stride = (int64_t)Hkv * D;
  const bf16* Kg = (const bf16*)A->K + ((int64_t)k_start * Hkv + g) * D;
  const bf16* Vg = (const bf16*)A->V + ((int64_t)k_start * Hkv + g) * D;

  // Q (B operand of Sᵀ = K·Qᵀ): lane holds Q[head g*G + col%G of member col/G]
  bf16x8 qf[KS];
  {
    const int qs = col_ok ? A->reqs[b + mcol].q_start : 0;
    const bf16* qrow = (const bf16*)A->Q + ((int64_t)qs * Hq + g * G + col % G) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = col_ok ? *(const bf16x8*)(qrow + ks * 32 + grp * 8) : bf16x8{};
  }

  LDS char* vt = smem + wave * (VT + LT);
  LDS char* lt = vt + VT;

  // LR rows of every member slot through a buffer resource that covers exactly the
  // request's rows: reads past them, or of an empty slot, return zeros and never leave the
  // member's cache.  Chunks at or past a member's own rank are addressed out of range, so
  // they read zeros too: the row's padding (or the next row) never enters the shared LR
  // accumulator, where a non-finite value times another member's masked P (0·NaN) would
  // reach that member's columns.  Each load unit u = lane + 64 i covers row u / LCH,
  // 16-byte chunk u % LCH of the 32 x (32 RB) tile.
  __amdgpu_buffer_rsrc_t lrs[NM];
  int ldl_b[NM], rank_m[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    int bytes = 0;
    const void* base = A->K;
    ldl_b[m] = 0;
    rank_m[m] = 0;
    if (RB && m < nm) {
      const AgentDesc& AG = A->agents[A->reqs[b + m].agent];
      if (AG.rank > 0) {
        base = (const bf16*)AG.L + (int64_t)k_start * AG.ldl;
        bytes = (int)((int64_t)A->reqs[b + m].k_len * AG.ldl * 2);   // the member's own rows
        ldl_b[m] = (int)(AG.ldl * 2);
        rank_m[m] = AG.rank;
      }
    }
    ldl_b[m] = __builtin_amdgcn_readfirstlane(ldl_b[m]);
    rank_m[m] = __builtin_amdgcn_readfirstlane(rank_m[m]);
    lrs[m] = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0,
                                               __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
  }
  int l_row[NL > 0 ? NL : 1], l_dst[NL > 0 ? NL : 1];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int u = lane + 64 * i;
    l_row[i] = u / LCH;
    l_dst[i] = (u / LCH) * 128 + (u % LCH) * 16;
  }

  u32x4 kreg[2][KS];
  u32x4 vreg[VLOADS];
  u32x4 lreg[NM][NL > 0 ? NL : 1];
  // Tiles past the wave's last one clamp to key ke-1: the loop prefetches without branches.
  auto tile_key = [&](int jt) { return kb + (wave + 4 * jt) * kKeys; };
  auto load_k = [&](int jt) {
    const int k0 = tile_key(jt);
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const int key = min(k0 + kb2 * 16 + col, ke - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kreg[kb2][ks] = *(const u32x4*)(Kg + (int64_t)key * kv_stride + (ks * 4 + grp) * 8);
    }
  };
  auto load_v = [&](int jt) {
    const int k0 = tile_key(jt);
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int key = min(k0 + i * (64 / CPR) + lane / CPR, ke - 1);
      vreg[i] = *(const u32x4*)(Vg + (int64_t)key * kv_stride + (lane % CPR) * 8);
    }
  };
  // every member slot loads, unconditionally (empty slots read zeros without memory traffic)
  auto load_l = [&](int jt) {
    const int k0 = tile_key(jt);
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int key = min(k0 + l_row[i], ke - 1);
        const int c = (lane + 64 * i) % LCH;
        const int off = c * 8 < rank_m[m] ? key * ldl_b[m] + c * 16 : 0x7ffffff0;
        lreg[m][i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(lrs[m], off, 0, 0));
      }
  };
  auto store_v = [&]() {
#pragma unroll
    for (int i = 0; i < VLOADS; ++i) {
      const int row = i * (64 / CPR) + lane / CPR;
      const int c = (lane % CPR) ^ vswz<D>(row);
      *(LDS u32x4*)(vt + row * (D * 2) + c * 16) = vreg[i];
    }
  };

  // transposing-read offsets: lane (e = (lane&15)/4, q = lane&3) of group grp supplies
  // 4 bf16 of key row grp*4 + e (and 16 + grp*4 + e), columns 16-block + 4q
  int voff[DB];
  const int trow = grp * 4 + ((lane & 15) >> 2), tq = lane & 3;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int d = db * 16 + tq * 4;
    voff[db] = trow * (D * 2) + (((d >> 3) ^ vswz<D>(trow)) << 4) + (d & 7) * 2;
  }

  f32x4 acc[DB];
  f32x4 accl[NRB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x4{};
#pragma unroll
  for (int i = 0; i < NRB; ++i) accl[i] = f32x4{};
  float m_run = kNegBig, l_run = 0.f;
  const float sl2 = A->scale_log2;

  // K is loaded one tile ahead into registers, V two tiles ahead (registers, then the
  // wave's V tile), each member's L rows one tile ahead into registers.
  if (my_tiles > 0) {
    load_k(0);
    load_v(0);
    if (RB) load_l(0);
    store_v();
    load_v(1);
    for (int jt = 0; jt < my_tiles; ++jt) {
      const int k0 = tile_key(jt);
      f32x4 s[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        s[kb2] = f32x4{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s[kb2] = mfma16(__builtin_bit_cast(bf16x8, kreg[kb2][ks]), qf[ks], s[kb2]);
      }
      load_k(jt + 1);
      const int lim = min(ke, my_len) - 1 - k0 - grp * 4;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kb2 * 16 + j > lim) s[kb2][j] = -INFINITY;
      float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                       fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      mx = col_max(mx) * sl2;
      if (__any(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) acc[i] *= alpha;
#pragma unroll
        for (int i = 0; i < NRB; ++i) accl[i] *= alpha;
      }
      bf16x8 pf;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb2][j], sl2, -m_run));
          l_run += p;
          pf[kb2 * 4 + j] = (bf16)p;
        }
#pragma unroll
      for (int db = 0; db < DB; ++db)
        acc[db] = mfma16(join(tr_read(vt + voff[db]), tr_read(vt + voff[db] + 16 * D * 2)), pf,
                         acc[db]);
      if (RB) {
        // one member at a time through the LR tile: this wave's reads of member m precede
        // the writes of member m + 1 in program order, and the LDS executes one wave's
        // operations in order
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          if (m >= nm) break;
#pragma unroll
          for (int i = 0; i < NL; ++i) *(LDS u32x4*)(lt + l_dst[i]) = lreg[m][i];
          const bf16x8 pm = mcol == m ? pf : bf16x8{};
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) {
            const LDS char* p = lt + trow * 128 + (rb * 16 + tq * 4) * 2;
            accl[rb] = mfma16(join(tr_read(p), tr_read(p + 16 * 128)), pm, accl[rb]);
          }
        }
      }
      if (RB) load_l(jt + 1);
      // the next tile's V replaces this one: this wave's reads above precede the writes
      store_v();
      load_v(jt + 2);
    }
  }

  // ---- merge the 4 wave states through LDS, apply each member's B_a, store
  // Output mapping: thread (slot, dp) produces the d pair 2 dp of every query column of
  // member `slot` (its G heads), so it needs that member's B_a column pair only: the rank
  // rows go to registers now, before the merge, whose barriers hide their latency.
  constexpr int TPC = D / 2;                 // threads per d range
  constexpr int RMAX = RB > 0 ? 32 * RB : 1;
  const int dp = tid % TPC, slot = tid / TPC;
  bf16x2 bpre[RMAX];
  int brank = 0;
  if (RB && slot < nm) {
    const AgentDesc& AG = A->agents[A->reqs[b + slot].agent];
    brank = AG.rank;
    // rows past the rank read zeros (bounds of the resource), so the loads are unconditional
    const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const bf16*)AG.B + g * D), (short)0,
        (int)((int64_t)brank * kv_stride * 2), 0x00020000);
#pragma unroll
    for (int k = 0; k < RMAX; ++k)
      bpre[k] = __builtin_bit_cast(
          bf16x2, __builtin_amdgcn_raw_buffer_load_b32(br, (int)((k * kv_stride + 2 * dp) * 2),
                                                       0, 0));
  }
  const float l_col = col_sum(l_run);
  __syncthreads();   // every wave is done with its tiles
  LDS float* sh = (LDS float*)smem;              // [wave][16 cols][D]   P·V_base
  LDS float* shl = sh + 4 * 16 * D;              // [wave][16 cols][64]  P·L_a
  LDS float* shm = shl + 4 * 16 * 64;            // [wave][16 cols][2]   (m, l)
  LDS float* sa = shm + 4 * 16 * 2;              // [16 cols][64]        merged P·L_a
  if (col_ok) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) sh[(wave * 16 + col) * D + db * 16 + grp * 4 + j] = acc[db][j];
    if (RB) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          shl[(wave * 16 + col) * 64 + rb * 16 + grp * 4 + j] = accl[rb][j];
    }
    if (grp == 0) {
      shm[(wave * 16 + col) * 2] = m_run;
      shm[(wave * 16 + col) * 2 + 1] = l_col;
    }
  }
  __syncthreads();

  auto weights = [&](int c, float* wgt, float& M, float& l) {
    M = kNegBig;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) M = fmaxf(M, shm[(wv * 16 + c) * 2]);
    l = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) {
      wgt[wv] = __builtin_amdgcn_exp2f(shm[(wv * 16 + c) * 2] - M);
      l += wgt[wv] * shm[(wv * 16 + c) * 2 + 1];
    }
  };
  const int ncols = nm * G;
  if (RB) {
    // merged P·L_a of every (column, rank index) the outputs use
    for (int e = tid; e < 16 * RMAX; e += 256) {
      const int c = e / RMAX, rho = e % RMAX;
      if (c < ncols) {
        float wgt[4], M, l;
        weights(c, wgt, M, l);
        float v = 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) v += wgt[wv] * shl[(wv * 16 + c) * 64 + rho];
        sa[c * 64 + rho] = v;
      }
    }
    __syncthreads();
  }
  if (slot < nm) {
    const ReqDesc& Rm = A->reqs[b + slot];
    for (int hh = 0; hh < G; ++hh) {
      const int c = slot * G + hh;
      float wgt[4], M, l;
      weights(c, wgt, M, l);
      float o0 = 0.f, o1 = 0.f;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        const f32x2 v = *(const LDS f32x2*)(sh + (wv * 16 + c) * D + 2 * dp);
        o0 += wgt[wv] * v[0];
        o1 += wgt[wv] * v[1];
      }
      if (RB) {
        // columns of P·L_a at or past the member's rank are zero: skipped
#pragma unroll
        for (int k = 0; k < RMAX; ++k) {
          if (k < brank) {
            const float a = sa[c * 64 + k];
            o0 += a * (float)bpre[k][0];
            o1 += a * (float)bpre[k][1];
          }
        }
      }
      const int h = g * G + hh;
      if (n_split == 1) {
        const float inv = 1.f / l;
        bf16x2 ob = {(bf16)(o0 * inv), (bf16)(o1 * inv)};
        *(bf16x2*)((bf16*)A->O + ((int64_t)Rm.q_start * Hq + h) * D + 2 * dp) = ob;
      } else {
        const int64_t pr = (int64_t)Rm.part_base + (int64_t)sp * Hq + h;
        *(float2*)(A->ws_o + pr * D + 2 * dp) = float2{o0, o1};
        if (dp == 0) *(float2*)(A->ws_ml + pr * 2) = float2{M, l};
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_bf16(const AttnArgs& a, int head_dim, int max_rank, int n_grid,
                              hipStream_t s, bool expand) {
  const int rb = max_rank > 32 ? 2 : (max_rank > 0 ? 1 : 0);
#define LRA_LAUNCH(D, RB, EX) \
  hipLaunchKernelGGL((fla_decode_bf16<D, RB, EX>), dim3(n_grid), dim3(kThreads), 0, s, a)
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

hipError_t launch_decode_shared_bf16(const AttnArgs& a, int head_dim, int max_rank, int n_grid,
                                     hipStream_t s) {
  const int rb = max_rank > 32 ? 2 : (max_rank > 0 ? 1 : 0);
#define LRA_LAUNCH(D, RB) \
  hipLaunchKernelGGL((fla_decode_shared_bf16<D, RB>), dim3(n_grid), dim3(kThreads), 0, s, a)
  if (head_dim == 128) {
    if (rb == 0) LRA_LAUNCH(128, 0);
    else if (rb == 1) LRA_LAUNCH(128, 1);
    else LRA_LAUNCH(128, 2);
  } else {
    if (rb == 0) LRA_LAUNCH(64, 0);
    else if (rb == 1) LRA_LAUNCH(64, 1);
    else LRA_LAUNCH(64, 2);
  }
#undef LRA_LAUNCH
  return hipGetLastError();
}

}  // namespace lra
