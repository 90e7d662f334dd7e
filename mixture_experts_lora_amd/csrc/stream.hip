// Streamed grouped GEMMs: the four expert products of the layer
//   gate_up  G = X[tok] W_gu^T + (s X A_gu) B_gu,   H = silu(gate) * up
//   down     O = H W_dn^T + (s H A_dn) B_dn
//   dh       dH = w (dY[tok] W_dn + Q_dn A_dn^T),   dG = SwiGLU'(dH; G)
//   dx       dX_pair = dG W_gu + Q_gu A_gu^T
// over the ragged per-expert row segments (Unsloth faster-MoE page, "What is
// torch._grouped_mm?"), with the LoRA term kept split as a rank-r product
// added into the same accumulator ("Faster LoRA MoE training").
//
// One persistent workgroup per CU runs ONE pipeline over its whole work
// list: every step moves a k panel of each operand (320 rows of A, 256
// columns of B) from global memory straight into LDS (buffer_load_dwordx4
// ... lds).  The step stream runs through a tile's base K steps, then its
// rank-r steps, then on into the next tile, so the pipeline never drains
// between tiles: the next tile's first panels are in flight while the
// current tile's epilogue writes its outputs.
//
// A stage holds 64 k (MOE_SK; 32 k with a four-stage ring is the other
// depth the code supports) in a two-stage ring: every row of a
// row-contiguous panel is one whole 128-byte line per request, half the
// L1->L2 requests of 32-k stages for the same bytes.  The DMA offsets that
// are affine in the instruction index are held as one base per lane plus a
// uniform stride, which keeps the nine instructions per stage from
// spilling registers beside the accumulators.
//
//  - tile 320 x 256, 8 waves of 160 x 64, two per SIMD
//    (v_mfma_f32_32x32x16 on bf16 or fp16, fp32 accumulation, operands
//    swapped so a lane owns 4 consecutive columns): while one wave of a SIMD
//    waits to issue a memory instruction (the CU's queues fill with requests
//    that miss the L2), the other keeps the SIMD's MFMA unit busy;
//  - 320 rows, not 256: an expert's rows are tiled from its segment start,
//    and with about 256 +- 16 rows per expert a 256-row tile leaves half the
//    experts a short tail tile that streams the expert's whole weight panel
//    again for a few rows; 320 covers such an expert in one tile;
//  - row-contiguous panels are stored [rows][SK k] with the 16-byte chunk
//    of row r at position c ^ ((r >> 2) & 3) (32 k) or c ^ ((r >> 1) & 7)
//    (64 k), so that the 16 rows a quarter-wave of ds_read_b128 reads fall
//    on 16 distinct 16-byte bank groups;
//  - panels whose contraction index is the row index in memory (W_dn and
//    W_gu in the backward, B_dn and B_gu in the forward) are stored
//    [SK k][256 columns] with chunk c of row k at c ^ 4 (k & 3), and read
//    with ds_read_b64_tr_b16, which hands each lane 4 consecutive k of one
//    column: two of them make one MFMA operand;
//  - rows past a segment, columns past a matrix and k past the rank get an
//    out-of-range buffer offset and land in LDS as zeros;
//  - the gather indices (token of each sorted row) of the next tile are
//    DMA'd into LDS a whole tile ahead, so building the next tile's row
//    offsets needs no global load in the loop;
#include <algorithm>
#include <type_traits>

//
// The tile height (MOE_SBM: 320 or 256 rows) and the stage depth (MOE_SK: 64
// or 32 k) are build parameters: the library holds this file compiled once
// per combination, each in its own namespace (MOE_STILE), and the per-shape
// tile choice picks one per product.
#include "common.h"
#include "gemm_util.h"
#include "kernels.h"

#ifndef MOE_STILE
#define MOE_STILE t320k64
#endif

namespace moe {
inline namespace MOE_EL {
namespace MOE_STILE {
namespace {

#ifndef MOE_SBM
#define MOE_SBM 320
#endif
constexpr int SBM = MOE_SBM, SBN = 256;         // tile
constexpr int SWM = 2, SWN = 4;                 // wave grid
constexpr int SNW = SWM * SWN, SNT = 64 * SNW;  // 8 waves, two per SIMD
constexpr int STM = SBM / SWM, STN = SBN / SWN; // 160 x 64 per wave
constexpr int SFM = STM / 32, SFN = STN / 32;   // 5 x 2 fragments
#ifndef MOE_SK
#define MOE_SK 64
#endif
static_assert(MOE_SK == 32 || MOE_SK == 64, "stage depth");
constexpr int SK = MOE_SK;                      // k per ring stage
constexpr int SNS = SK == 64 ? 2 : 4;           // ring stages
constexpr int HK = SK / 16;                     // 16-k halves per stage
constexpr int CPR = SK / 8;                     // 16-byte chunks per K-panel row
constexpr int RPI = 1024 / (SK * 2);            // K-panel rows per DMA instruction
constexpr int APAN = SBM * SK, BPAN = SBN * SK;  // 16-bit elements of the A and B panels
constexpr int SSTAGE = APAN + BPAN;               // A panel then B panel
// One DMA instruction moves 1 KiB = RPI rows of SK k.  The B panel splits
// evenly over the waves; the A panel's AIN instructions go A_FULL to every
// wave and one more to each of the first A_REM waves.
constexpr int AIN = SBM / RPI, BIN = SBN / RPI;
constexpr int A_FULL = AIN / SNW, A_REM = AIN % SNW;
constexpr int NIA = A_FULL + (A_REM ? 1 : 0), NIB = BIN / SNW;
constexpr int PER_HI = NIA + NIB, PER_LO = A_FULL + NIB;  // per wave per stage
static_assert(SBM % 32 == 0 && BIN % SNW == 0, "panel split");
static_assert(SNS * SSTAGE * 2 <= 150 * 1024, "ring fits in LDS");
// gather indices of a tile, in whole 1 KiB DMA instructions (256 tokens)
constexpr int TOKB = (SBM + 255) / 256 * 256;

enum StreamKind { SK_GU = 0, SK_DN = 1, SK_DH = 2, SK_DX = 3 };

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

template <int KIND>
struct SP {
  static constexpr bool A_GATHER = KIND == SK_GU || KIND == SK_DH;
  static constexpr bool B_MAIN_MN = KIND == SK_DH || KIND == SK_DX;
  static constexpr bool B_LORA_MN = KIND == SK_GU || KIND == SK_DN;
  // operands whose DMA offsets are affine in the instruction index j (a
  // per-lane base plus j times a uniform stride): the rows of an ungathered
  // A panel, the rank-r A rows, and every MN panel.  Rows past a tile's
  // segment need no test there: the buffer's size ends at the segment.
  static constexpr bool A_MAIN_AFF = !A_GATHER;
  static constexpr bool B_MAIN_AFF = B_MAIN_MN;
  static constexpr bool B_LORA_AFF = B_LORA_MN;
};

template <int KIND>
__device__ __forceinline__ int s_ntn(const Layer& L) {
  return KIND == SK_GU ? cdiv(L.n, SBN / 2) : KIND == SK_DH ? cdiv(L.n, SBN) : cdiv(L.d, SBN);
}
template <int KIND>
__device__ __forceinline__ int s_kmain(const Layer& L) {
  return KIND == SK_GU || KIND == SK_DH ? L.d : KIND == SK_DN ? L.n : 2 * L.n;
}

// A work unit: a whole tile, or one column half of a tile.  With F tiles on
// G workgroups, a last round of r = F mod G <= G / 2 tiles would leave G - r
// workgroups idle; those r tiles run instead as 2 r half tiles (units nfull
// .. nfull + 2 r), columns [cb, ce) of the tile, so the last round is a full
// round of units that stream half the B panel each.
struct STile {
  int t, e, nt, row0, mrows, cb, ce;
};

__device__ __forceinline__ STile s_decode(const int* pre, const int* segst, int Et, int u, int ntn,
                                          int nfull) {
  STile T;
  T.t = u;
  int t = u;
  T.cb = 0;
  T.ce = SBN;
  if (u >= nfull) {
    const int v = u - nfull;
    t = nfull + (v >> 1);
    T.cb = __builtin_amdgcn_readfirstlane((v & 1) * (SBN / 2));
    T.ce = __builtin_amdgcn_readfirstlane(T.cb + SBN / 2);
  }
  T.e = __builtin_amdgcn_readfirstlane(find_expert(pre, Et, t, ntn));
  const int local = t - pre[T.e] * ntn;
  const int nm = pre[T.e + 1] - pre[T.e];
  T.nt = __builtin_amdgcn_readfirstlane(local / nm);
  const int mt = local - T.nt * nm;
  T.row0 = __builtin_amdgcn_readfirstlane(segst[T.e] + mt * SBM);
  T.mrows = __builtin_amdgcn_readfirstlane(min(SBM, segst[T.e + 1] - T.row0));
  return T;
}

__device__ __forceinline__ bool s_in(const STile& T, int c) { return c >= T.cb && c < T.ce; }

// Per-lane constants of the two panel layouts.
//  K panel, instruction j of wave w: row RPI (w + 8 j) + lane / CPR,
//  physical chunk lane % CPR holding logical chunk s_lck(j) = physical ^
//  the row's swizzle.
//  MN panel, instruction j of wave w: k row 2 (w + 8 j) + lane / 32, physical
//  chunk lane % 32 holding logical chunk lcm = (lane & 31) ^ fsw.
__device__ __forceinline__ int s_kswz(int r) { return SK == 32 ? (r >> 2) & 3 : (r >> 1) & 7; }
__device__ __forceinline__ int s_prow(int j) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  return RPI * (wid + j * SNW) + lane / CPR;
}
__device__ __forceinline__ int s_lck(int j) {
  const int lane = threadIdx.x & 63;
  return (lane % CPR) ^ s_kswz(s_prow(j));
}
__device__ __forceinline__ int s_lcm() {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  return (lane & 31) ^ ((2 * (wid & 1) + (lane >> 5)) * 4);
}
__device__ __forceinline__ int s_krow(int j) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  return 2 * (wid + j * SNW) + (lane >> 5);
}

// Issue cursor: the tile whose panels are being issued, its descriptors and
// per-lane offsets, and the next step to issue.
struct SIssue {
  int4v da_m, db_m, da_l, db_l;
  // per-instruction offsets; an affine operand keeps only element 0 and
  // adds j times its stride (xa_*, xb_*) when it issues instruction j
  uint32_t va_m[NIA], vb_m[NIB], va_l[NIA], vb_l[NIB];
  uint32_t xa_m, xb_m, xa_l, xb_l;
  uint32_t ldb_bm, ldb_bl;  // byte stride of the MN-panel sources (k rows)
  int step, smain, stot, rot;
};

template <int KIND, bool LORA>
__device__ __forceinline__ void s_setup(const Layer& L, const STile& T, const int* tok, SIssue& S) {
  const int n = L.n, d = L.d, rs = L.rs, ra = L.ra, r = L.r;
  const int lcm = s_lcm();
  const int e = T.e, row0 = T.row0, mrows = T.mrows;
  S.smain = s_kmain<KIND>(L) / SK;
  S.stot = S.smain + (LORA ? cdiv(rs, SK) : 0);
  S.step = 0;
  // Each tile starts its base K loop 64 e k into the contraction of its
  // expert e (wrapping round; 128 bytes of a row per expert, at either stage
  // depth): the tiles in flight at one moment then read different address
  // columns of their 4 KB-strided rows instead of all of them the same one.
  // Every tile of an expert keeps the same order, so the N tiles that share
  // an A panel still stream it in step.
  S.rot = __builtin_amdgcn_readfirstlane((T.e * (64 / SK)) % S.smain);
  S.ldb_bm = 0;
  S.ldb_bl = 0;
  // A main
  if constexpr (KIND == SK_GU || KIND == SK_DH) {
    S.da_m = make_desc(KIND == SK_GU ? L.x : L.dy, (int64_t)L.T * d * 2);
#pragma unroll
    for (int j = 0; j < NIA; ++j) {
      const int m = s_prow(j);
      S.va_m[j] = m < mrows ? (uint32_t)tok[m] * (uint32_t)(d * 2) + s_lck(j) * 16 : OOB;
    }
  } else {
    const int lda = KIND == SK_DN ? n : 2 * n;
    const bf16_t* src = KIND == SK_DN ? L.h : L.dg;
    S.da_m = make_desc(src + (int64_t)row0 * lda, (int64_t)mrows * lda * 2);
    S.va_m[0] = (uint32_t)s_prow(0) * (uint32_t)(lda * 2) + s_lck(0) * 16;
    S.xa_m = (uint32_t)(RPI * SNW) * (uint32_t)(lda * 2);
  }
  // A rank-r
  {
    const bf16_t* src = KIND == SK_GU ? L.xa : KIND == SK_DN ? L.ha : KIND == SK_DH ? L.qdn : L.qgu;
    S.da_l = make_desc(src + (int64_t)row0 * rs, (int64_t)mrows * rs * 2);
    S.va_l[0] = (uint32_t)s_prow(0) * (uint32_t)(rs * 2) + s_lck(0) * 16;
    S.xa_l = (uint32_t)(RPI * SNW) * (uint32_t)(rs * 2);
  }
  // B main and B rank-r
  if constexpr (KIND == SK_GU) {
    const int j0 = T.nt * (SBN / 2);
    S.db_m = make_desc(L.w_gu + (int64_t)e * 2 * n * d, (int64_t)2 * n * d * 2);
#pragma unroll
    for (int j = 0; j < NIB; ++j) {
      const int c = s_prow(j);
      const bool ok = j0 + (c >> 6) * 32 + (c & 31) < n && s_in(T, c);
      S.vb_m[j] = ok ? (uint32_t)gu_row(n, j0, c) * (uint32_t)(d * 2) + s_lck(j) * 16 : OOB;
    }
    S.db_l = make_desc(L.b_gu + (int64_t)e * r * 2 * n, (int64_t)r * 2 * n * 2);
    S.ldb_bl = 2 * n * 2;
    const int c = lcm * 8;  // tile column of this lane's chunk (8 columns, one gate/up group)
    const bool ok = j0 + (c >> 6) * 32 + (c & 31) < n && s_in(T, c);
    S.vb_l[0] = ok ? (uint32_t)s_krow(0) * S.ldb_bl + (uint32_t)gu_row(n, j0, c) * 2 : OOB;
    S.xb_l = (uint32_t)(2 * SNW) * S.ldb_bl;
  } else if constexpr (KIND == SK_DN) {
    const int c0 = T.nt * SBN;
    S.db_m = make_desc(L.w_dn + (int64_t)e * d * n, (int64_t)d * n * 2);
#pragma unroll
    for (int j = 0; j < NIB; ++j) {
      const int c = s_prow(j);
      S.vb_m[j] = c0 + c < d && s_in(T, c) ? (uint32_t)(c0 + c) * (uint32_t)(n * 2) + s_lck(j) * 16 : OOB;
    }
    S.db_l = make_desc(L.b_dn + (int64_t)e * r * d, (int64_t)r * d * 2);
    S.ldb_bl = d * 2;
    const int col = c0 + lcm * 8;
    const bool cin = s_in(T, lcm * 8);
    S.vb_l[0] = col < d && cin ? (uint32_t)s_krow(0) * S.ldb_bl + (uint32_t)col * 2 : OOB;
    S.xb_l = (uint32_t)(2 * SNW) * S.ldb_bl;
  } else if constexpr (KIND == SK_DH) {
    const int j0 = T.nt * SBN;
    S.db_m = make_desc(L.w_dn + (int64_t)e * d * n, (int64_t)d * n * 2);
    S.ldb_bm = n * 2;
    const int col = j0 + lcm * 8;
    const bool cin = s_in(T, lcm * 8);
    S.vb_m[0] = col < n && cin ? (uint32_t)s_krow(0) * S.ldb_bm + (uint32_t)col * 2 : OOB;
    S.xb_m = (uint32_t)(2 * SNW) * S.ldb_bm;
    S.db_l = make_desc(L.a_dn + (int64_t)e * n * ra, (int64_t)n * ra * 2);
#pragma unroll
    for (int j = 0; j < NIB; ++j) {
      const int c = s_prow(j);
      S.vb_l[j] = j0 + c < n && s_in(T, c) ? (uint32_t)(j0 + c) * (uint32_t)(ra * 2) + s_lck(j) * 16 : OOB;
    }
  } else {
    const int c0 = T.nt * SBN;
    S.db_m = make_desc(L.w_gu + (int64_t)e * 2 * n * d, (int64_t)2 * n * d * 2);
    S.ldb_bm = d * 2;
    const int col = c0 + lcm * 8;
    const bool cin = s_in(T, lcm * 8);
    S.vb_m[0] = col < d && cin ? (uint32_t)s_krow(0) * S.ldb_bm + (uint32_t)col * 2 : OOB;
    S.xb_m = (uint32_t)(2 * SNW) * S.ldb_bm;
    S.db_l = make_desc(L.a_gu + (int64_t)e * d * ra, (int64_t)d * ra * 2);
#pragma unroll
    for (int j = 0; j < NIB; ++j) {
      const int c = s_prow(j);
      S.vb_l[j] = c0 + c < d && s_in(T, c) ? (uint32_t)(c0 + c) * (uint32_t)(ra * 2) + s_lck(j) * 16 : OOB;
    }
  }
}

// Issue step `step` of the cursor's tile into the ring stage at LDS byte
// address `sb` (A panel, then B panel).
template <int KIND>
__device__ __forceinline__ void s_issue(const SIssue& S, int step, uint32_t sb, int rs, int r) {
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ma = sb, mb = sb + APAN * 2;
  // A instruction j exists for every wave below A_FULL, for the first A_REM
  // waves at A_FULL
  auto a_on = [&](int j) { return j < A_FULL || wid < A_REM; };
  if (step < S.smain) {
    int ks = step + S.rot;
    if (ks >= S.smain) ks -= S.smain;
    const int k0 = ks * SK;
#pragma unroll
    for (int j = 0; j < NIA; ++j)
      if (a_on(j))
        dma16(S.da_m, SP<KIND>::A_MAIN_AFF ? S.va_m[0] + (uint32_t)j * S.xa_m : S.va_m[j], (uint32_t)k0 * 2u,
              __builtin_amdgcn_readfirstlane(ma + (wid + j * SNW) * 1024));
#pragma unroll
    for (int j = 0; j < NIB; ++j)
      dma16(S.db_m, SP<KIND>::B_MAIN_AFF ? S.vb_m[0] + (uint32_t)j * S.xb_m : S.vb_m[j],
            SP<KIND>::B_MAIN_MN ? (uint32_t)k0 * S.ldb_bm : (uint32_t)k0 * 2u,
            __builtin_amdgcn_readfirstlane(mb + (wid + j * SNW) * 1024));
  } else {
    const int k0 = (step - S.smain) * SK;
#pragma unroll
    for (int j = 0; j < NIA; ++j)
      if (a_on(j))
        dma16(S.da_l, k0 + s_lck(0) * 8 < rs ? S.va_l[0] + (uint32_t)j * S.xa_l : OOB, (uint32_t)k0 * 2u,
              __builtin_amdgcn_readfirstlane(ma + (wid + j * SNW) * 1024));
#pragma unroll
    for (int j = 0; j < NIB; ++j) {
      if constexpr (SP<KIND>::B_LORA_MN)
        dma16(S.db_l, k0 + s_krow(j) < r ? S.vb_l[0] + (uint32_t)j * S.xb_l : OOB, (uint32_t)k0 * S.ldb_bl,
              __builtin_amdgcn_readfirstlane(mb + (wid + j * SNW) * 1024));
      else
        dma16(S.db_l, k0 + s_lck(j) * 8 < rs ? S.vb_l[j] : OOB, (uint32_t)k0 * 2u,
              __builtin_amdgcn_readfirstlane(mb + (wid + j * SNW) * 1024));
    }
  }
}

// Operand fragments of one k-half (16 k) of a ring stage: the wave's SFM A
// fragments (rows) and SFN B fragments (columns).
struct Frag {
  uint4 a[SFM], b[SFN];
};

// Every LDS read of this wave has returned (gfx9 s_waitcnt: lgkmcnt 0, vmcnt
// and expcnt left alone): a stage's slot is refilled right after the barrier
// that follows its last reads.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// A fragment fm, k-half kk: row-contiguous panel, chunk c of row r stored at
// c ^ ((r >> 2) & 3); lane L reads row wm 160 + fm 32 + L % 32, k 8 (2 kk +
// L / 32) .. + 8.
__device__ __forceinline__ uint4 s_read_a(const bf16_t* As, int kk, int fm) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / SWN, l = lane & 31;
  const char* ab = (const char*)As + (wm * STM + l) * (SK * 2);
  const int c = ((kk * 2 + (lane >> 5)) ^ s_kswz(l)) * 16;
  return *(const uint4*)(ab + fm * 32 * (SK * 2) + c);
}
// B fragment fn, k-half kk.  K panel: as A.  MN panel: 16-lane group g reads
// k rows 8 (g >> 1) + q (+4 in the second read) at columns 16 (g & 1) + 4 rr
// of the fragment; the transposing read gives lane (g, j) the 4 k values of
// column 16 (g & 1) + j.
template <bool BMN>
__device__ __forceinline__ uint4 s_read_b(const bf16_t* Bs, int kk, int fn) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wn = wid % SWN, l = lane & 31;
  if constexpr (!BMN) {
    const char* bb = (const char*)Bs + (wn * STN + l) * (SK * 2);
    const int c = ((kk * 2 + (lane >> 5)) ^ s_kswz(l)) * 16;
    return *(const uint4*)(bb + fn * 32 * (SK * 2) + c);
  } else {
    const int g = lane >> 4, q = (lane >> 2) & 3, rr = lane & 3;
    const int krow = kk * 16 + 8 * (g >> 1) + q;
    const int kx = (krow & 3) * 4;
    const int col = wn * STN + fn * 32 + 16 * (g & 1) + 4 * rr;
    const char* p = (const char*)Bs + krow * (SBN * 2) + (((col >> 3) ^ kx) * 16) + (col & 7) * 2;
    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * SBN * 2));
    return make_uint4((uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                      (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                      (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                      (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16));
  }
}

template <bool BMN>
__device__ __forceinline__ void s_read_half(const bf16_t* st, int kk, Frag& f) {
#pragma unroll
  for (int fm = 0; fm < SFM; ++fm) f.a[fm] = s_read_a(st, kk, fm);
#pragma unroll
  for (int fn = 0; fn < SFN; ++fn) f.b[fn] = s_read_b<BMN>(st + APAN, kk, fn);
}

// The MFMAs of the k-half held in f, and into f (as its fragments fall
// free) the reads of k-half kk of the stage at st, so that the LDS reads run
// under the MFMAs: the MFMAs of B fragment 0 with every A fragment, the read
// of the next B fragment 0, then those of B fragment 1 with each A fragment
// followed by the read of that A fragment, then the read of B fragment 1.
// The next half's first MFMA then waits only for the first two reads.
// (Padding rows are multiplied too: branching around fragments splits the
// accumulators' live ranges.)
static_assert(SFN == 2, "two column fragments per wave");
template <bool BMN_NEXT>
__device__ __forceinline__ void s_mfma_read(Frag& f, f32x16 (&acc)[SFM][SFN], const bf16_t* st, int kk) {
#pragma unroll
  for (int fm = 0; fm < SFM; ++fm) acc[fm][0] = mfma32(f.b[0], f.a[fm], acc[fm][0]);
  f.b[0] = s_read_b<BMN_NEXT>(st + APAN, kk, 0);
#pragma unroll
  for (int fm = 0; fm < SFM; ++fm) {
    acc[fm][1] = mfma32(f.b[1], f.a[fm], acc[fm][1]);
    f.a[fm] = s_read_a(st, kk, fm);
  }
  f.b[1] = s_read_b<BMN_NEXT>(st + APAN, kk, 1);
  constexpr int RB = BMN_NEXT ? 2 : 1;  // LDS reads per B fragment
  __builtin_amdgcn_sched_group_barrier(0x008, SFM, 0);
  __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);
#pragma unroll
  for (int fm = 0; fm < SFM; ++fm) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, RB, 0);
}

__device__ __forceinline__ void s_mfma(const Frag& f, f32x16 (&acc)[SFM][SFN]) {
#pragma unroll
  for (int fn = 0; fn < SFN; ++fn)
#pragma unroll
    for (int fm = 0; fm < SFM; ++fm) acc[fm][fn] = mfma32(f.b[fn], f.a[fm], acc[fm][fn]);
}

// Epilogue, through a private 4 KiB LDS staging area per wave.  The
// accumulators of a pair of neighbouring 32 x 32 fragments (fn = 2 pr, 2 pr
// + 1) are rounded to bf16 and written as rows of 64 values (128 bytes, the
// 16-byte chunk c of row m at c ^ (m & 7)); they are read back by rows, lane
// -> row (lane / 8) + 8 i, chunk lane % 8, so that each store instruction
// writes 8 whole 128-byte row segments.  Fragment (fm, fn) of the wave covers
// rows wm 128 + fm 32 + 0..31 and tile columns wn 128 + fn 32 + 0..31; lane l
// holds row l % 32, columns 8 g + 4 (l / 32) + 0..3 in elements 4 g + 0..3.
__device__ __forceinline__ void s_stage_pair(bf16_t* wl, const f32x16& v0, const f32x16& v1) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 31, h = lane >> 5;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const f32x16& v = f ? v1 : v0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = 4 * f + g;
      *(uint2*)(wl + m * 64 + ((c ^ (m & 7)) * 8) + 4 * h) =
          make_uint2(pack2(v[4 * g], v[4 * g + 1]), pack2(v[4 * g + 2], v[4 * g + 3]));
    }
  }
}
__device__ __forceinline__ uint4 s_unstage(const bf16_t* wl, int i) {
  const int lane = threadIdx.x & 63;
  const int r = (lane >> 3) + 8 * i, c = lane & 7;
  return *(const uint4*)(wl + r * 64 + ((c ^ (r & 7)) * 8));
}
__device__ __forceinline__ void s_store(rsrc_t r, uint32_t voff, uint4 v) {
  const v4u a = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(a, r, voff, 0, 0);
}
__device__ __forceinline__ float s_lo(uint32_t w) { return bf2f((bf16_t)(w & 0xffffu)); }
__device__ __forceinline__ float s_hi(uint32_t w) { return bf2f((bf16_t)(w >> 16)); }

// dh epilogue: dH (without the routing weight) of fragment pair (fm, pr) is
// staged as above and read back by rows: lane -> row (lane / 8) + 8 i,
// j = jb + 8 (lane % 8) + 0..7.  The SwiGLU backward needs gate and up of the
// same (row, j) from the saved G: those loads run one fragment pair ahead
// (the first one's wait also covers the next tile's panels already in
// flight; after that they overlap the previous pair's math and stores).
struct GUq {
  uint4 g[4], u[4];
  float w[4];
};
__device__ __forceinline__ void s_dh_load(const Layer& L, const STile& T, rsrc_t rg, rsrc_t rw, int q,
                                          GUq& o) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / SWN, wn = wid % SWN;
  const int fm = q / (SFN / 2), pr = q % (SFN / 2);
  const int n = L.n;
  const int j = T.nt * SBN + wn * STN + pr * 64 + (lane & 7) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = wm * STM + fm * 32 + (lane >> 3) + 8 * i;
    const bool ok = m < T.mrows && j < n && s_in(T, wn * STN);
    const uint32_t og = ok ? (uint32_t)(((int64_t)(T.row0 + m) * 2 * n + j) * 2) : OOB;
    const auto gq = __builtin_amdgcn_raw_buffer_load_b128(rg, og, 0, 0);
    const auto uq = __builtin_amdgcn_raw_buffer_load_b128(rg, ok ? og + (uint32_t)(n * 2) : OOB, 0, 0);
    o.g[i] = make_uint4(gq[0], gq[1], gq[2], gq[3]);
    o.u[i] = make_uint4(uq[0], uq[1], uq[2], uq[3]);
    o.w[i] = __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rw, ok ? (uint32_t)(T.row0 + m) * 4u : OOB, 0, 0));
  }
}
__device__ __forceinline__ void s_epilogue_dh(const Layer& L, const STile& T, f32x16 (&acc)[SFM][SFN], bf16_t* wl) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / SWN, wn = wid % SWN;
  const int n = L.n;
  const int64_t P = L.Ptot;
  const rsrc_t rg = make_rsrc(L.g, P * 2 * n * 2), rdg = make_rsrc(L.dg, P * 2 * n * 2);
  const rsrc_t rw = make_rsrc(L.wgt, P * 4);
  // <dH, H> of each row over each 64-column group, for the routing-weight
  // gradient; without a destination every such store falls out of range
  const int G = L.dw_groups;
  const rsrc_t rpart = make_rsrc(L.dw_part, L.dw_part ? P * G * 4 : 0);
  // with the tall tile's accumulators there is no room to hold a second pair
  constexpr bool AHEAD = SFM <= 4;
  GUq cur, nxt;
  if (AHEAD) s_dh_load(L, T, rg, rw, 0, cur);
#pragma unroll
  for (int q = 0; q < SFM * (SFN / 2); ++q) {
    const int fm = q / (SFN / 2), pr = q % (SFN / 2);
    if (AHEAD && q + 1 < SFM * (SFN / 2)) s_dh_load(L, T, rg, rw, q + 1, nxt);
    s_stage_pair(wl, acc[fm][2 * pr], acc[fm][2 * pr + 1]);
    // (the pair's accumulators are free once staged)
    if (!AHEAD) s_dh_load(L, T, rg, rw, q, cur);
    const int j = T.nt * SBN + wn * STN + pr * 64 + (lane & 7) * 8;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = s_unstage(wl, i);
      const uint32_t dw[4] = {v.x, v.y, v.z, v.w};
      const int m = wm * STM + fm * 32 + (lane >> 3) + 8 * i;
      const bool ok = m < T.mrows && j < n && s_in(T, wn * STN);
      const int64_t p = T.row0 + m;
      const uint32_t og = ok ? (uint32_t)((p * 2 * n + j) * 2) : OOB;
      const float w = cur.w[i];
      const uint32_t gw[4] = {cur.g[i].x, cur.g[i].y, cur.g[i].z, cur.g[i].w};
      const uint32_t uw[4] = {cur.u[i].x, cur.u[i].y, cur.u[i].z, cur.u[i].w};
      uint32_t dgt[4], dup[4];
      float hdot = 0.0f;  // this lane's 8 columns of <dH, H>, dH before w
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float rg2[2], ru2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float gv = hh ? s_hi(gw[e2]) : s_lo(gw[e2]);
          const float uv = hh ? s_hi(uw[e2]) : s_lo(uw[e2]);
          const float dhu = hh ? s_hi(dw[e2]) : s_lo(dw[e2]);
          const float dh = w * dhu;
          const float sg = sigmoid_f(gv);
          rg2[hh] = dh * uv * (sg * (1.0f + gv * (1.0f - sg)));
          ru2[hh] = dh * (gv * sg);
          hdot += dhu * (gv * sg * uv);
        }
        dgt[e2] = pack2(rg2[0], rg2[1]);
        dup[e2] = pack2(ru2[0], ru2[1]);
      }
      s_store(rdg, og, make_uint4(dgt[0], dgt[1], dgt[2], dgt[3]));
      s_store(rdg, ok ? og + (uint32_t)(n * 2) : OOB, make_uint4(dup[0], dup[1], dup[2], dup[3]));
      // the 8 lanes of a row hold its 64 columns of this pair
      hdot += __shfl_xor(hdot, 1, 64);
      hdot += __shfl_xor(hdot, 2, 64);
      hdot += __shfl_xor(hdot, 4, 64);
      const uint32_t od = ok && (lane & 7) == 0 ? (uint32_t)((p * G + (j >> 6)) * 4) : OOB;
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hdot), rpart, od, 0, 0);
    }
    if (AHEAD && q + 1 < SFM * (SFN / 2)) cur = nxt;
  }
}

template <int KIND>
__device__ __forceinline__ void s_epilogue(const Layer& L, const STile& T, f32x16 (&acc)[SFM][SFN], bf16_t* wl) {
  static_assert(KIND != SK_DH, "dh has its own epilogue");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / SWN, wn = wid % SWN;
  const int n = L.n, d = L.d;
  const int64_t P = L.Ptot;
  const rsrc_t rg = make_rsrc(L.g, P * 2 * n * 2), rh = make_rsrc(L.h, P * n * 2), ro = make_rsrc(L.o, P * d * 2);
#pragma unroll
  for (int fm = 0; fm < SFM; ++fm)
#pragma unroll
    for (int pr = 0; pr < SFN / 2; ++pr) {
      s_stage_pair(wl, acc[fm][2 * pr], acc[fm][2 * pr + 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = s_unstage(wl, i);
        const int m = wm * STM + fm * 32 + (lane >> 3) + 8 * i;
        const int64_t p = T.row0 + m;
        if constexpr (KIND == SK_GU) {
          // chunks 0..3 of the pair are gate(j), 4..7 up(j) for j = jb + 8
          // (chunk % 4) + 0..7: each lane stores its own chunk of G, and the
          // two lanes holding gate and up of the same j compute 4 h each
          const int c = lane & 7, up = c >> 2;
          const int j = T.nt * (SBN / 2) + (wn * (SFN / 2) + pr) * 32 + 8 * (c & 3);
          const bool ok = m < T.mrows && j < n && s_in(T, wn * STN);
          s_store(rg, ok ? (uint32_t)((p * 2 * n + (up ? n : 0) + j) * 2) : OOB, v);
          const uint32_t o[4] = {(uint32_t)__shfl_xor((int)v.x, 4, 64), (uint32_t)__shfl_xor((int)v.y, 4, 64),
                                 (uint32_t)__shfl_xor((int)v.z, 4, 64), (uint32_t)__shfl_xor((int)v.w, 4, 64)};
          const uint32_t mine[4] = {v.x, v.y, v.z, v.w};
          // lane with the gate chunk takes values 0..3, its partner 4..7
          uint32_t hw[2];
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const uint32_t gw = up ? o[2 * up + e2] : mine[e2];
            const uint32_t uw = up ? mine[2 * up + e2] : o[e2];
            hw[e2] = pack2(silu_f(s_lo(gw)) * s_lo(uw), silu_f(s_hi(gw)) * s_hi(uw));
          }
          const uint32_t oh = ok ? (uint32_t)((p * n + j + 4 * up) * 2) : OOB;
          __builtin_amdgcn_raw_buffer_store_b64((v2u){hw[0], hw[1]}, rh, oh, 0, 0);
        } else {
          const int c = T.nt * SBN + wn * STN + pr * 64 + (lane & 7) * 8;
          const bool ok = m < T.mrows && c < d && s_in(T, wn * STN);
          s_store(ro, ok ? (uint32_t)((p * d + c) * 2) : OOB, v);
        }
      }
    }
}

// LORA: the rank-r steps follow each tile's base steps (the split LoRA
// term); without them the kernel is the plain grouped GEMM, as the forward on
// merged weights uses it.
template <int KIND, bool LORA>
__global__ __launch_bounds__(SNT) __attribute__((amdgpu_waves_per_eu(SNW / 4, SNW / 4))) void k_stream(const Layer L) {
  __shared__ __attribute__((aligned(1024))) bf16_t ring[SNS * SSTAGE];
  __shared__ __attribute__((aligned(16))) int tokbuf[2][TOKB];
  __shared__ int pre[MAX_ET + 1];
  __shared__ int segst[MAX_ET + 1];
  __shared__ int sh[SNW];
  const int Et = L.Et;
  for (int e = threadIdx.x; e <= Et; e += SNT)
    segst[e] = e < L.E ? L.offsets[e] : e == L.E ? L.P : L.Ptot;
  __syncthreads();
  expert_prefix<SNT>(L, pre, sh, [&](int e) { return cdiv(segst[e + 1] - segst[e], SBM); });
  const int ntn = s_ntn<KIND>(L);
  const int G = gridDim.x;
  const int F = pre[Et] * ntn;  // tiles
  const int rlast = F % G;
  const int nsplit = rlast > 0 && 2 * rlast <= G ? rlast : 0;
  const int nfull = F - nsplit, total = F + nsplit;  // units
  int tc = first_tile();
  if (tc >= total) return;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rs = L.rs, r = L.r;
  const uint32_t ring_b = (uint32_t)(uintptr_t)ring;

  // issue cursor on the first tile; its gather indices come in directly
  STile ti = s_decode(pre, segst, Et, tc, ntn, nfull);
  if (SP<KIND>::A_GATHER) {
    for (int m = threadIdx.x; m < SBM; m += SNT)
      tokbuf[0][m] = ti.row0 + m < L.Ptot ? L.tok[ti.row0 + m] : 0;
    __syncthreads();
  }
  SIssue S;
  s_setup<KIND, LORA>(L, ti, tokbuf[0], S);
  int iord = 0;        // ordinal of the issue tile among this workgroup's tiles
  bool idone = false;  // no tile left to issue: repeat the last step
  // gather indices of the following tile, a whole tile ahead (wave 0, before
  // the step's panels, so the step's wait covers it)
  auto issue_tok = [&](int t_next, int slot) {
    if (!SP<KIND>::A_GATHER || wid != 0 || t_next >= total) return;
    const STile Tn = s_decode(pre, segst, Et, t_next, ntn, nfull);
    const int lane = threadIdx.x & 63;
    const int4v dt = make_desc(L.tok + Tn.row0, (int64_t)(L.Ptot - Tn.row0) * 4);
#pragma unroll
    for (int i = 0; i < TOKB / 256; ++i)
      dma16(dt, (uint32_t)(i * 256 + lane * 4) * 4u, 0,
            __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&tokbuf[slot][256 * i]));
  };
  issue_tok(tc + G, 1);
  // the next tile's gather indices must be in before the prologue's issues
  // can reach that tile
  wait_vmcnt<0>();
  __syncthreads();
  int gi = 0;  // global issue step (ring slot gi % SNS)
  auto issue_next = [&]() {
    if (S.step == S.stot) {
      const int tn = ti.t + G;
      if (!idone && tn < total) {
        ++iord;
        ti = s_decode(pre, segst, Et, tn, ntn, nfull);
        s_setup<KIND, LORA>(L, ti, tokbuf[iord & 1], S);
        issue_tok(tn + G, (iord + 1) & 1);
        // no scalar load of the switch stays pending into the step loop
        // (they return out of order, so a pending one would make every
        // fragment read wait for all the others)
        wait_lgkm0();
      } else {
        idone = true;
        S.step = S.stot - 1;
      }
    }
    s_issue<KIND>(S, S.step, ring_b + (uint32_t)(gi % SNS) * SSTAGE * 2, rs, r);
    if (!idone) ++S.step;
    ++gi;
  };
  // all SNS stages of the ring in flight before the first step
#pragma unroll 1
  for (int s = 0; s < SNS; ++s) issue_next();

  // compute: tiles in order, each its base steps then its rank-r steps.  A
  // step runs the MFMAs of its first k-half while reading its second; then
  // every wave waits for the next stage and meets the others at the step's
  // one barrier, after which the stage just read is free and is refilled;
  // then the second half's MFMAs run while the next stage's first half is
  // read.
  const int smain = s_kmain<KIND>(L) / SK;
  const int stot = smain + (LORA ? cdiv(rs, SK) : 0);
  int gc = 0;
  // The wait of step k: the stage after it must be in; younger than that
  // stage are the SNS - 2 stages issued after it.  In the first two steps of
  // every tile but the first, the previous tile's epilogue stores were issued
  // in between: those waits are full (vmcnt 0), so they never count on how
  // stores and loads retire relative to each other.
  constexpr int WAIT_HI = (SNS - 2) * PER_HI, WAIT_LO = (SNS - 2) * PER_LO;
  const bool hi = A_REM == 0 || wid < A_REM;  // this wave issues PER_HI per stage
  bool after_epi = false;
  auto ring_wait = [&](int k) {
    if (after_epi && k < 2) {
      wait_vmcnt<0>();
    } else {
      if (hi) wait_vmcnt<WAIT_HI>();
      else wait_vmcnt<WAIT_LO>();
    }
  };
  // first stage: the SNS - 1 later ones may still be in flight
  if (hi) wait_vmcnt<(SNS - 1) * PER_HI>();
  else wait_vmcnt<(SNS - 1) * PER_LO>();
  __syncthreads();
  Frag f;
  s_read_half<SP<KIND>::B_MAIN_MN>(ring, 0, f);
  constexpr bool MN_M = SP<KIND>::B_MAIN_MN, MN_L = SP<KIND>::B_LORA_MN;
#pragma unroll 1
  for (; tc < total; tc += G) {
    f32x16 acc[SFM][SFN];
#pragma unroll
    for (int fm = 0; fm < SFM; ++fm)
#pragma unroll
      for (int fn = 0; fn < SFN; ++fn) acc[fm][fn] = (f32x16)(0.0f);
    // one step: the MFMAs of its first k-half under the reads of its second,
    // the wait and barrier, the refill of the stage just read, the MFMAs of
    // the second half under the reads of the next stage's first half.  The
    // base steps, the step into the rank-r steps, and the rank-r steps are
    // separate straight-line loops (a branch inside one would split the
    // accumulators' live ranges).
    auto step = [&](auto mn_cur, auto mn_next, int k) {
      const bf16_t* st = ring + (gc % SNS) * SSTAGE;
#pragma unroll
      for (int kk = 1; kk < HK; ++kk) s_mfma_read<decltype(mn_cur)::value>(f, acc, st, kk);
      ring_wait(k);
      wait_lgkm0();
      __syncthreads();
      issue_next();
      s_mfma_read<decltype(mn_next)::value>(f, acc, ring + ((gc + 1) % SNS) * SSTAGE, 0);
      ++gc;
    };
    using BM = std::integral_constant<bool, MN_M>;
    using BL = std::integral_constant<bool, MN_L>;
    // the last step of the tile: its remaining halves, no refill
    auto last = [&](auto mn_cur) {
#pragma unroll
      for (int kk = 1; kk < HK; ++kk)
        s_mfma_read<decltype(mn_cur)::value>(f, acc, ring + (gc % SNS) * SSTAGE, kk);
      ring_wait(stot - 1);
      wait_lgkm0();
      __syncthreads();
      s_mfma(f, acc);
      ++gc;
    };
#pragma unroll 1
    for (int k = 0; k < smain - 1; ++k) step(BM{}, BM{}, k);
    if constexpr (LORA) {
      step(BM{}, BL{}, smain - 1);
#pragma unroll 1
      for (int k = smain; k < stot - 1; ++k) step(BL{}, BL{}, k);
      last(BL{});
    } else {
      last(BM{});
    }
    // the stage read last is not refilled until every wave has staged its
    // outputs through it
    const STile tcur = s_decode(pre, segst, Et, tc, ntn, nfull);
    if constexpr (KIND == SK_DH)
      s_epilogue_dh(L, tcur, acc, ring + ((gc + SNS - 1) % SNS) * SSTAGE + wid * 2048);
    else
      s_epilogue<KIND>(L, tcur, acc, ring + ((gc + SNS - 1) % SNS) * SSTAGE + wid * 2048);
    after_epi = true;
    __syncthreads();
    issue_next();
    // the next tile's first half (its stage is in: the last step waited for it)
    s_read_half<MN_M>(ring + (gc % SNS) * SSTAGE, 0, f);
  }
  wait_vmcnt<0>();
}

}  // namespace

template <int KIND, bool LORA>
static hipError_t launch_stream(const Layer& L, hipStream_t st, const char* name) {
  const int ntn = KIND == SK_GU ? cdiv(L.n, SBN / 2) : KIND == SK_DH ? cdiv(L.n, SBN) : cdiv(L.d, SBN);
  const int64_t tiles = (int64_t)(L.Ptot / SBM + L.Et) * ntn;
  int g = (int)std::min<int64_t>(tiles, L.ncu);
  g = std::max((g + 7) & ~7, 8);
  MOE_LAUNCH(name, (k_stream<KIND, LORA>), dim3(g), dim3(SNT), 0, st, L);
  return hipGetLastError();
}

// the forward products also run without the low-rank pass, on merged weights
hipError_t stream_gate_up(const Layer& L, hipStream_t st) {
  return L.lora ? launch_stream<SK_GU, true>(L, st, "gate_up")
                : launch_stream<SK_GU, false>(L, st, "gate_up_merged");
}
hipError_t stream_down(const Layer& L, hipStream_t st) {
  return L.lora ? launch_stream<SK_DN, true>(L, st, "down")
                : launch_stream<SK_DN, false>(L, st, "down_merged");
}
hipError_t stream_dx(const Layer& L, hipStream_t st) { return launch_stream<SK_DX, true>(L, st, "dx"); }
hipError_t stream_dh(const Layer& L, hipStream_t st) { return launch_stream<SK_DH, true>(L, st, "dh"); }

}  // namespace MOE_STILE
}  // inline namespace MOE_EL
}  // namespace moe
