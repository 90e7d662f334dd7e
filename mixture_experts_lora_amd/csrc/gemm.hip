// Grouped GEMMs of the MoE-LoRA layer on gfx950 MFMA.
//
// Every product of the layer is a GEMM over the ragged per-expert row
// segments of the sorted (token, expert) pairs, against that expert's slice of
// a stacked parameter (Unsloth faster-MoE page, "What is torch._grouped_mm?").
// The LoRA term stays split ("Faster LoRA MoE training"): the rank-r
// activation (X A_gu, H A_dn, dO B_dn^T, dG B_gu^T) comes from a skinny
// pre-pass, and its product with the other factor runs as a second, short
// MFMA pass into the SAME accumulator tile as the base product, so the
// adapter delta (A B)^T is never formed.
//
// Engine
//  - one workgroup = 4 waves = 256 threads; tile BM x BN, K step 64;
//  - v_mfma_f32_32x32x16_bf16, fp32 accumulation; the operands are swapped
//    (mfma(B, A)) so each lane owns 4 consecutive output columns of one row
//    and the epilogue writes 8-byte (bf16) or 16-byte (fp32) vectors;
//  - operands come in through buffer loads (buffer_load_dwordx4): rows
//    outside a segment and columns outside a matrix get a vector offset past
//    the buffer's range and read as zero in hardware, so the K loop has no
//    branches; for row-contiguous operands the K offset of a step is a scalar
//    register that only moves inside a row already range-checked;
//  - LDS holds both operands K-contiguous, rows padded to 72 elements, two
//    stages; global loads run two K steps ahead of the MFMAs (two register
//    stages);
//  - operands whose contraction index is the row index in memory (the weights
//    in the backward, the segment rows in the LoRA-gradient reductions) are
//    loaded as 4(k) x 8(mn) blocks and transposed in registers before the
//    LDS store;
//  - persistent grid; tile t of a round goes to the workgroup that shares an
//    XCD with tiles t-1 and t+1 (workgroups are dealt to the 8 XCDs round
//    robin), so the M-tiles of one expert's weight panel meet in one L2;
//  - the schedule is derived on the device from the routing offsets: no
//    host synchronisation, empty experts produce no tiles.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "gemm_util.h"
#include "kernels.h"

namespace moe {
inline namespace MOE_EL {

#ifndef MOE_PGR
#define MOE_PGR 2
#endif

constexpr int BK = 64;
constexpr int LDK = BK + 8;

// Tile configuration: BM x BN outputs per workgroup, WM x WN waves (64
// threads each), PGR register stages of global prefetch (1 or 2).
template <int BM_, int BN_, int WM_, int WN_, int PGR_ = MOE_PGR, int DMA_NS_ = 0, int DBK_ = 64,
          int OCC_ = 0>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WM_, WAVES_N = WN_, PGR = PGR_;
  // DMA_NS > 0: row-contiguous main-loop operands go global -> LDS directly
  // through a ring of DMA_NS stages of DBK k each (unpadded, XOR-swizzled rows)
  static constexpr int DMA_NS = DMA_NS_, DBK = DBK_;
  static constexpr int DMA_STAGE = (BM_ + BN_) * DBK_;   // bf16 elements per ring stage
  static constexpr int NW = WM_ * WN_, NT = 64 * NW;
  // waves per SIMD the register allocation must allow (default: two
  // workgroups of 4 waves, or one of 8, unless the wave tile is large)
  static constexpr int OCC = OCC_ ? OCC_ : (NW == 4 && (BM / WM_) * (BN / WN_) > 64 * 64) ? 1 : 2;
  static constexpr int TM = BM / WM_, TN = BN / WN_;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile at least 32x32");
  static_assert(DBK_ == 32 || DBK_ == 64, "DMA k step");
  static constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  // PGR 0: one LDS buffer, no prefetch (the short rank-r step of a DMA kernel)
  static constexpr int REG_LDS = (PGR_ == 0 ? 1 : 2) * STAGE;
  static constexpr int LDS_ELEMS = REG_LDS > DMA_NS_ * DMA_STAGE ? REG_LDS : DMA_NS_ * DMA_STAGE;
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t scale2(uint32_t w, float s) {
  return pack2(bf2f((bf16_t)(w & 0xffffu)) * s, bf2f((bf16_t)(w >> 16)) * s);
}
__device__ __forceinline__ uint4 scale8(uint4 v, float s) {
  return make_uint4(scale2(v.x, s), scale2(v.y, s), scale2(v.z, s), scale2(v.w, s));
}
__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------- operand panels

// R rows of a K-contiguous source; row r starts at byte rowoff(r) of the
// buffer (negative = a zero row).  Each thread moves 16-byte chunks; the K
// offset of a step goes in the scalar offset.  KCHECK masks chunks at or past
// kmax (narrow rank-r rows); SCALED multiplies each row by its own factor.
template <int R, int NT, bool KCHECK, bool SCALED, int NS = 3>
struct KOp {
  static constexpr int CH = R * (BK / 8);
  static constexpr int PER = (CH + NT - 1) / NT;
  rsrc_t rs;
  uint32_t voff[PER];
  float scl[PER];
  uint4 v[NS][PER];
  int kmax;

  template <class RowFn>
  __device__ KOp(rsrc_t r, RowFn rowoff, int kmax_) : rs(r), kmax(kmax_) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      float sc = 1.0f;
      int64_t o = -1;
      if (c < CH) o = rowoff(c >> 3, sc);
      voff[i] = o < 0 ? OOB : (uint32_t)o + (uint32_t)((c & 7) * 16);
      scl[i] = sc;
    }
  }
  template <int S>
  __device__ __forceinline__ void fetch(int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      uint32_t o = voff[i];
      if (KCHECK) {
        const int c = threadIdx.x + i * NT;
        if (k0 + (c & 7) * 8 >= kmax) o = OOB;
      }
      v[S][i] = bload16(rs, o, (uint32_t)k0 * 2u);
    }
  }
  template <int S>
  __device__ __forceinline__ void store(bf16_t* lds) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      if (CH % NT == 0 || c < CH) {
        uint4 w = v[S][i];
        if (SCALED) w = scale8(w, scl[i]);
        *(uint4*)(lds + (c >> 3) * LDK + (c & 7) * 8) = w;
      }
    }
  }
};

// Transposing store shared by the MN panels: a thread's 4(k) x 8(c) block
// goes to 8 LDS rows (one per column c) as 4 consecutive k values.  The lane
// mapping (kq fastest) puts a half-wave's 8-byte stores on distinct banks.
__device__ __forceinline__ void store_block_t(bf16_t* lds, int kq, int mg, const uint4 (&w)[4]) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int sh = (c & 1) * 16;
    const uint32_t e0 = (word_of(w[0], c >> 1) >> sh) & 0xffffu;
    const uint32_t e1 = (word_of(w[1], c >> 1) >> sh) & 0xffffu;
    const uint32_t e2 = (word_of(w[2], c >> 1) >> sh) & 0xffffu;
    const uint32_t e3 = (word_of(w[3], c >> 1) >> sh) & 0xffffu;
    *(uint2*)(lds + (mg * 8 + c) * LDK + kq * 4) = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
  }
}

// R columns of a source whose contraction index is its row index: element
// (k, c) at byte k*ldb + 2*col(c) of the buffer (the buffer starts at the
// first row of the contraction range and ends with its last row, so rows past
// the range read as zero).  8 consecutive columns are contiguous.  WROWS
// multiplies contraction row k by the fp32 weight at byte 4k of `rw`.
template <int R, int NT, int NS = 3, bool WROWS = false>
struct MNOp {
  static constexpr int NB = (BK / 4) * (R / 8);
  static constexpr int PER = (NB + NT - 1) / NT;
  rsrc_t rs, rw;
  uint32_t colb[PER];
  uint32_t ldb;
  uint4 v[NS][PER][4];
  uint4 wv[NS][PER];

  template <class ColFn>
  __device__ MNOp(rsrc_t r, ColFn colfn, uint32_t ldb_, rsrc_t rw_ = rsrc_t()) : rs(r), rw(rw_), ldb(ldb_) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int bi = threadIdx.x + i * NT;
      const int c = bi < NB ? colfn((bi >> 4) * 8) : -1;
      colb[i] = c < 0 ? OOB : (uint32_t)c * 2u;
    }
  }
  template <int S>
  __device__ __forceinline__ void fetch(int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int kq = (threadIdx.x + i * NT) & 15;
#pragma unroll
      for (int q = 0; q < 4; ++q)  // the row goes in the range-checked vector offset
        v[S][i][q] = bload16(rs, colb[i] + (uint32_t)(k0 + kq * 4 + q) * ldb, 0);
      if (WROWS) wv[S][i] = bload16(rw, (uint32_t)(k0 + kq * 4) * 4u, 0);
    }
  }
  template <int S>
  __device__ __forceinline__ void store(bf16_t* lds) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int bi = threadIdx.x + i * NT;
      if (NB % NT != 0 && bi >= NB) continue;
      uint4 w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = WROWS ? scale8(v[S][i][q], __uint_as_float(word_of(wv[S][i], q))) : v[S][i][q];
      store_block_t(lds, bi & 15, bi >> 4, w);
    }
  }
};

// As MNOp, but contraction row k is token tok[k] of a [T, ld] source (the
// hidden states or the upstream gradient), optionally scaled by wgt[k].  The
// gather indices of the next step are loaded one step ahead.
template <int R, int NT, bool SCALED, int NS = 3>
struct MNGather {
  static constexpr int NB = (BK / 4) * (R / 8);
  static constexpr int PER = (NB + NT - 1) / NT;
  rsrc_t rs, rtok, rwgt;
  uint32_t colb[PER];
  uint32_t ldb;
  int kmax;
  uint4 v[NS][PER][4];
  float scl[NS][PER][4];
  uint4 tn[PER], wn[PER];

  template <class ColFn>
  __device__ MNGather(rsrc_t r, rsrc_t rt, rsrc_t rw, ColFn colfn, uint32_t ldb_, int kmax_)
      : rs(r), rtok(rt), rwgt(rw), ldb(ldb_), kmax(kmax_) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int bi = threadIdx.x + i * NT;
      const int c = bi < NB ? colfn((bi >> 4) * 8) : -1;
      colb[i] = c < 0 ? OOB : (uint32_t)c * 2u;
      const uint32_t ro = (uint32_t)((bi & 15) * 4) * 4u;
      tn[i] = bload16(rtok, ro, 0);
      wn[i] = SCALED ? bload16(rwgt, ro, 0) : make_uint4(0, 0, 0, 0);
    }
  }
  template <int S>
  __device__ __forceinline__ void fetch(int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int kq = (threadIdx.x + i * NT) & 15;
      const uint4 t = tn[i], w = wn[i];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t tq = word_of(t, q);
        const uint32_t o = (k0 + kq * 4 + q < kmax) ? colb[i] + tq * ldb : OOB;
        v[S][i][q] = bload16(rs, o, 0);
        scl[S][i][q] = SCALED ? __uint_as_float(word_of(w, q)) : 1.0f;
      }
      const uint32_t ro = (uint32_t)(k0 + BK + kq * 4) * 4u;
      tn[i] = bload16(rtok, ro, 0);
      if (SCALED) wn[i] = bload16(rwgt, ro, 0);
    }
  }
  template <int S>
  __device__ __forceinline__ void store(bf16_t* lds) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int bi = threadIdx.x + i * NT;
      if (NB % NT != 0 && bi >= NB) continue;
      uint4 w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = SCALED ? scale8(v[S][i][q], scl[S][i][q]) : v[S][i][q];
      store_block_t(lds, bi & 15, bi >> 4, w);
    }
  }
};

// ---------------------------------------------------------------- MFMA main loop

template <class C>
__device__ __forceinline__ void mma_stage(const bf16_t* As, const bf16_t* Bs,
                                          f32x16 (&acc)[C::FM][C::FN], bool active) {
  if (!active) return;  // the wave's rows or columns are all padding
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / C::WAVES_N, wn = wid % C::WAVES_N;
  const bf16_t* ab = As + (wm * C::TM + (lane & 31)) * LDK + (lane >> 5) * 8;
  const bf16_t* bb = Bs + (wn * C::TN + (lane & 31)) * LDK + (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    uint4 a[C::FM], b[C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) a[fm] = *(const uint4*)(ab + fm * 32 * LDK + kk * 16);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) b[fn] = *(const uint4*)(bb + fn * 32 * LDK + kk * 16);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = mfma32(b[fn], a[fm], acc[fm][fn]);
  }
}

// One K step of the three-stage pipeline: register stage S (step kt) is free
// to take step kt+3, stage (S+1)%3 holds step kt+1 and goes to the other LDS
// buffer after the MFMAs.
template <class C, int S, class OA, class OB>
__device__ __forceinline__ void run_step3(bf16_t* lds, OA& oa, OB& ob, int kt, int nk, int klast,
                                          f32x16 (&acc)[C::FM][C::FN], bool active) {
  bf16_t* cur = lds + (kt & 1) * C::STAGE;
  bf16_t* nxt = lds + ((kt + 1) & 1) * C::STAGE;
  oa.template fetch<S>(min((kt + 3) * BK, klast));
  ob.template fetch<S>(min((kt + 3) * BK, klast));
  mma_stage<C>(cur, cur + C::A_ELEMS, acc, active);
  if (kt + 1 < nk) {
    oa.template store<(S + 1) % 3>(nxt);
    ob.template store<(S + 1) % 3>(nxt + C::A_ELEMS);
  }
  __syncthreads();
}

// Pipelined K loop over nk steps of 64.  Global loads run MOE_PGR steps ahead
// of the MFMAs, LDS is double-buffered, one barrier per step.  Ends with a
// barrier, so the LDS can be reused right after.
template <class C, class OA, class OB>
__device__ __forceinline__ void run_loop(bf16_t* lds, OA& oa, OB& ob, int nk,
                                         f32x16 (&acc)[C::FM][C::FN], bool active = true) {
  if (nk <= 0) return;
  if constexpr (C::PGR == 0) {
  for (int kt = 0; kt < nk; ++kt) {
    oa.template fetch<0>(kt * BK);
    ob.template fetch<0>(kt * BK);
    oa.template store<0>(lds);
    ob.template store<0>(lds + C::A_ELEMS);
    __syncthreads();
    mma_stage<C>(lds, lds + C::A_ELEMS, acc, active);
    __syncthreads();
  }
  } else if constexpr (C::PGR == 1) {
  oa.template fetch<0>(0);
  ob.template fetch<0>(0);
  oa.template store<0>(lds);
  ob.template store<0>(lds + C::A_ELEMS);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    bf16_t* cur = lds + (kt & 1) * C::STAGE;
    bf16_t* nxt = lds + ((kt + 1) & 1) * C::STAGE;
    if (kt + 1 < nk) {
      oa.template fetch<0>((kt + 1) * BK);
      ob.template fetch<0>((kt + 1) * BK);
    }
    mma_stage<C>(cur, cur + C::A_ELEMS, acc, active);
    if (kt + 1 < nk) {
      oa.template store<0>(nxt);
      ob.template store<0>(nxt + C::A_ELEMS);
    }
    __syncthreads();
  }
  } else if constexpr (C::PGR == 3) {
  // three register stages: stage s holds step kt+s while step kt computes
  const int klast = (nk - 1) * BK;
  oa.template fetch<0>(0);
  ob.template fetch<0>(0);
  oa.template fetch<1>(min(BK, klast));
  ob.template fetch<1>(min(BK, klast));
  oa.template fetch<2>(min(2 * BK, klast));
  ob.template fetch<2>(min(2 * BK, klast));
  oa.template store<0>(lds);
  ob.template store<0>(lds + C::A_ELEMS);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 6) {
    run_step3<C, 0>(lds, oa, ob, kt, nk, klast, acc, active);
    if (kt + 1 >= nk) break;
    run_step3<C, 1>(lds, oa, ob, kt + 1, nk, klast, acc, active);
    if (kt + 2 >= nk) break;
    run_step3<C, 2>(lds, oa, ob, kt + 2, nk, klast, acc, active);
    if (kt + 3 >= nk) break;
    run_step3<C, 0>(lds, oa, ob, kt + 3, nk, klast, acc, active);
    if (kt + 4 >= nk) break;
    run_step3<C, 1>(lds, oa, ob, kt + 4, nk, klast, acc, active);
    if (kt + 5 >= nk) break;
    run_step3<C, 2>(lds, oa, ob, kt + 5, nk, klast, acc, active);
  }
  } else {
  // Look-ahead fetches are issued unconditionally (past the last step they
  // re-read the last step's addresses and are never stored), so the compiler
  // can count outstanding loads exactly and waits only for the stage it needs.
  const int klast = (nk - 1) * BK;
  oa.template fetch<0>(0);
  ob.template fetch<0>(0);
  oa.template fetch<1>(min(BK, klast));
  ob.template fetch<1>(min(BK, klast));
  oa.template store<0>(lds);
  ob.template store<0>(lds + C::A_ELEMS);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += 2) {
    {  // step kt: buffer 0; register stage 1 holds kt+1
      bf16_t* nxt = lds + C::STAGE;
      oa.template fetch<0>(min((kt + 2) * BK, klast));
      ob.template fetch<0>(min((kt + 2) * BK, klast));
      mma_stage<C>(lds, lds + C::A_ELEMS, acc, active);
      if (kt + 1 < nk) {
        oa.template store<1>(nxt);
        ob.template store<1>(nxt + C::A_ELEMS);
      }
      __syncthreads();
    }
    if (kt + 1 >= nk) break;
    {  // step kt+1: buffer 1; register stage 0 holds kt+2
      bf16_t* cur = lds + C::STAGE;
      oa.template fetch<1>(min((kt + 3) * BK, klast));
      ob.template fetch<1>(min((kt + 3) * BK, klast));
      mma_stage<C>(cur, cur + C::A_ELEMS, acc, active);
      if (kt + 2 < nk) {
        oa.template store<0>(lds);
        ob.template store<0>(lds + C::A_ELEMS);
      }
      __syncthreads();
    }
  }
  }
}


// ---------------------------------------------------------------- LDS-DMA operands

// R rows x DBK k of a row-contiguous source, DMA'd into an unpadded swizzled
// LDS panel [R][DBK].  One instruction fills 1 KiB (1024 / (2 DBK) rows);
// the NW waves take the instructions in turn.  Row r starts at byte
// rowoff(r) of the buffer (negative = zero row); KCHECK zeroes chunks at or
// past kmax.
template <int R, int NW, bool KCHECK, int DBK>
struct KDma {
  static constexpr int CPR = DBK / 8, RPI = 64 / CPR;
  static constexpr int NI = R / (RPI * NW);
  static_assert(NI * RPI * NW == R, "rows must split evenly over the waves");
  int4v desc;
  uint32_t voff[NI];
  int kc[NI];
  int kmax;

  template <class RowFn>
  __device__ KDma(int4v d, RowFn rowoff, int kmax_) : desc(d), kmax(kmax_) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int row = RPI * (wid + j * NW) + lane / CPR;
      const int c = sw_chunk<DBK>(row, lane % CPR);
      const int64_t o = rowoff(row);
      voff[j] = o < 0 ? OOB : (uint32_t)o + (uint32_t)(c * 16);
      kc[j] = c * 8;
    }
  }
  // LDS byte address of the panel's row 0 is `base`
  __device__ __forceinline__ void issue(int k0, uint32_t base) {
    const int wid = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      uint32_t o = voff[j];
      if (KCHECK && k0 + kc[j] >= kmax) o = OOB;
      dma16(desc, o, (uint32_t)k0 * 2u, __builtin_amdgcn_readfirstlane(base + (wid + j * NW) * 1024));
    }
  }
};

// MFMAs of one ring stage over the wave's first NFM 32-row fragments (the
// rest of its rows are padding).  Fragment rows are 32-aligned, so the
// swizzle of a lane's row is the same in every fragment.
template <class C, int NFM>
__device__ __forceinline__ void mma_stage_sw(const bf16_t* As, const bf16_t* Bs,
                                             f32x16 (&acc)[C::FM][C::FN]) {
  if constexpr (NFM > 0) {
    constexpr int DBK = C::DBK;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int wm = wid / C::WAVES_N, wn = wid % C::WAVES_N;
    const int l = lane & 31;
    const bf16_t* ab = As + (wm * C::TM + l) * DBK;
    const bf16_t* bb = Bs + (wn * C::TN + l) * DBK;
#pragma unroll
    for (int kk = 0; kk < DBK / 16; ++kk) {
      const int c = sw_chunk<DBK>(l, kk * 2 + (lane >> 5)) * 8;
      uint4 a[NFM], b[C::FN];
#pragma unroll
      for (int fm = 0; fm < NFM; ++fm) a[fm] = *(const uint4*)(ab + fm * 32 * DBK + c);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) b[fn] = *(const uint4*)(bb + fn * 32 * DBK + c);
#pragma unroll
      for (int fm = 0; fm < NFM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn) acc[fm][fn] = mfma32(b[fn], a[fm], acc[fm][fn]);
    }
  }
}

// K loop over nk steps of DBK with both operands DMA'd through a ring of
// C::DMA_NS LDS stages, issued DMA_NS-1 steps ahead (past the last step the
// issue re-reads the last step into a stage nobody reads).  One barrier per
// step; ends with every DMA drained and a barrier, so the LDS can be reused.
template <class C, int NFM, class DA, class DB>
__device__ __forceinline__ void run_loop_dma(bf16_t* lds, DA& da, DB& db, int nk,
                                             f32x16 (&acc)[C::FM][C::FN]) {
  constexpr int NS = C::DMA_NS, PD = NS - 1, DBK = C::DBK;
  constexpr int PER_STAGE = DA::NI + DB::NI;  // DMA instructions per wave per stage
  if (nk <= 0) return;
  const uint32_t base = (uint32_t)(uintptr_t)lds;
  const int klast = (nk - 1) * DBK;
  auto issue = [&](int step, int slot) {
    const int k0 = min(step * DBK, klast);
    const uint32_t sb = base + (uint32_t)slot * C::DMA_STAGE * 2;
    da.issue(k0, sb);
    db.issue(k0, sb + C::BM * DBK * 2);
  };
#pragma unroll
  for (int s = 0; s < PD; ++s) issue(s, s);
  int slot = 0;
  for (int kt = 0; kt < nk; ++kt) {
    wait_vmcnt<(PD - 1) * PER_STAGE>();
    __syncthreads();
    issue(kt + PD, slot == 0 ? NS - 1 : slot - 1);
    const bf16_t* cur = lds + slot * C::DMA_STAGE;
    mma_stage_sw<C, NFM>(cur, cur + C::BM * DBK, acc);
    slot = slot + 1 == NS ? 0 : slot + 1;
  }
  wait_vmcnt<0>();
  __syncthreads();
}

// Calls f(std::integral_constant<int, v>) with v the wave's number of 32-row
// fragments holding valid rows (0 when its columns are all padding), rounded
// up to a multiple of STEP (2 for eight fragments, to bound code size).
template <int V, int STEP, class F>
__device__ __forceinline__ void nfm_dispatch(int nfm, F& f) {
  if constexpr (V <= 0) {
    f(std::integral_constant<int, 0>());
  } else {
    if (nfm > V - STEP) f(std::integral_constant<int, V>());
    else nfm_dispatch<V - STEP, STEP>(nfm, f);
  }
}
template <class C, class F>
__device__ __forceinline__ void with_nfm(int mrows, int ncols, F f) {
  const int wid = threadIdx.x >> 6;
  const int wm = wid / C::WAVES_N, wn = wid % C::WAVES_N;
  int nfm = wn * C::TN < ncols ? cdiv(mrows - wm * C::TM, 32) : 0;
  nfm = __builtin_amdgcn_readfirstlane(max(0, min(C::FM, nfm)));
  nfm_dispatch<C::FM, (C::FM > 4 ? 2 : 1)>(nfm, f);
}

template <class C>
__device__ __forceinline__ void zero_acc(f32x16 (&acc)[C::FM][C::FN]) {
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[fm][fn][i] = 0.0f;
}

// Visit the accumulator as (row, first col, 4 values): row/col inside the tile.
template <class C, class F>
__device__ __forceinline__ void for_each_quad(f32x16 (&acc)[C::FM][C::FN], F f) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / C::WAVES_N, wn = wid % C::WAVES_N;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = wm * C::TM + fm * 32 + (lane & 31);
        const int col = wn * C::TN + fn * 32 + g * 8 + (lane >> 5) * 4;
        f(row, col, acc[fm][fn][4 * g], acc[fm][fn][4 * g + 1], acc[fm][fn][4 * g + 2],
          acc[fm][fn][4 * g + 3]);
      }
}

// ---------------------------------------------------------------- forward

// Main-tile configurations (BM x BN, waves, prefetch depth); each of the four
// main GEMMs picks one at compile time.
template <int I> struct MainCfg;
template <> struct MainCfg<0> { using type = Cfg<128, 128, 2, 2, 2>; };  // 4 waves of 64x64
template <> struct MainCfg<1> { using type = Cfg<128, 256, 2, 4, 1>; };  // 8 waves of 64x64
template <> struct MainCfg<2> { using type = Cfg<256, 128, 4, 2, 1>; };  // 8 waves of 64x64
template <> struct MainCfg<3> { using type = Cfg<256, 256, 4, 2, 1>; };  // 8 waves of 64x128
template <> struct MainCfg<4> { using type = Cfg<128, 256, 2, 2, 1>; };  // 4 waves of 64x128
template <> struct MainCfg<5> { using type = Cfg<128, 128, 2, 2, 1>; };  // 4 waves of 64x64
template <> struct MainCfg<6> { using type = Cfg<256, 128, 4, 2, 2>; };  // 8 waves of 64x64
template <> struct MainCfg<7> { using type = Cfg<128, 256, 2, 4, 2>; };  // 8 waves of 64x64
template <> struct MainCfg<8> { using type = Cfg<128, 256, 2, 4, 3>; };  // 8 waves of 64x64
template <> struct MainCfg<9> { using type = Cfg<128, 128, 2, 2, 3>; };  // 4 waves of 64x64
template <> struct MainCfg<10> { using type = Cfg<256, 256, 2, 2, 1>; };  // 4 waves of 128x128
template <> struct MainCfg<11> { using type = Cfg<256, 128, 2, 2, 1>; };  // 4 waves of 128x64
// LDS-DMA main loops (forward GEMMs only): unpadded swizzled ring stages;
// the rank-r step runs unpipelined through one padded LDS buffer
template <> struct MainCfg<12> { using type = Cfg<256, 256, 2, 2, 0, 2, 64>; };     // 4 waves of 128x128
template <> struct MainCfg<13> { using type = Cfg<256, 128, 2, 2, 0, 3, 64>; };     // 4 waves of 128x64
template <> struct MainCfg<14> { using type = Cfg<128, 256, 1, 4, 0, 3, 64>; };     // 4 waves of 128x64
template <> struct MainCfg<15> { using type = Cfg<256, 256, 4, 2, 0, 4, 32>; };     // 8 waves of 64x128
template <> struct MainCfg<16> { using type = Cfg<256, 256, 4, 2, 0, 2, 64>; };     // 8 waves of 64x128
template <> struct MainCfg<17> { using type = Cfg<128, 256, 2, 2, 0, 3, 32, 2>; };  // 4 waves of 64x128, 2 WG/CU
template <> struct MainCfg<18> { using type = Cfg<256, 256, 2, 2, 0, 4, 32>; };     // 4 waves of 128x128
template <> struct MainCfg<19> { using type = Cfg<128, 256, 1, 4, 0, 4, 32>; };     // 4 waves of 128x64
template <> struct MainCfg<20> { using type = Cfg<128, 128, 2, 2, 0, 4, 32, 2>; };  // 4 waves of 64x64, 2 WG/CU
template <> struct MainCfg<21> { using type = Cfg<128, 256, 1, 4, 0, 3, 32, 2>; };  // 4 waves of 128x64, 2 WG/CU
template <> struct MainCfg<22> { using type = Cfg<256, 128, 4, 1, 0, 3, 32, 2>; };  // 4 waves of 64x128, 2 WG/CU
template <> struct MainCfg<23> { using type = Cfg<128, 256, 1, 4, 0, 6, 32>; };     // 4 waves of 128x64, deep ring
template <> struct MainCfg<24> { using type = Cfg<128, 256, 2, 2, 0, 6, 32>; };     // 4 waves of 64x128, deep ring
template <> struct MainCfg<25> { using type = Cfg<256, 128, 4, 1, 0, 6, 32>; };     // 4 waves of 64x128, deep ring
template <> struct MainCfg<26> { using type = Cfg<128, 256, 2, 4, 0, 6, 32>; };     // 8 waves of 64x64, deep ring
template <> struct MainCfg<27> { using type = Cfg<256, 256, 4, 2, 0, 4, 32>; };     // 8 waves of 64x128
// Which main products run on the streamed engine (stream.hip) by default:
// all four (its 320-row tiles cover a typical expert segment in one tile);
// the register-path kernels here remain the other engine of each product.
#ifndef MOE_STREAM_GU
#define MOE_STREAM_GU 1
#endif
#ifndef MOE_STREAM_DN
#define MOE_STREAM_DN 1
#endif
#ifndef MOE_STREAM_DX
#define MOE_STREAM_DX 1
#endif
#ifndef MOE_STREAM_DH
#define MOE_STREAM_DH 1
#endif
#ifndef MOE_CFG_GU
#define MOE_CFG_GU 7
#endif
#ifndef MOE_CFG_DN
#define MOE_CFG_DN 3
#endif
#ifndef MOE_CFG_DH
#define MOE_CFG_DH 7
#endif
#ifndef MOE_CFG_DX
#define MOE_CFG_DX 3
#endif
// Rank-r pre-passes: 128 rows x (64 | 128) rank columns, 4 waves.
template <int BN>
using CfgSkinny = Cfg<128, BN, 4, 1>;

#define MOE_GEMM_PROLOGUE(C)                                        \
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_ELEMS]; \
  __shared__ int pre[MAX_ET + 1];                                   \
  __shared__ int sh[C::NW];                                         \
  expert_prefix<C::NT>(L, pre, sh, [&](int e) { return cdiv(seg_count(L, e), C::BM); });

// true when this wave's rows [wm*TM, ..) start inside the tile's valid rows
// and its columns start inside the valid columns
template <class C>
__device__ __forceinline__ bool wave_active(int mrows, int ncols) {
  const int wid = threadIdx.x >> 6;
  return (wid / C::WAVES_N) * C::TM < mrows && (wid % C::WAVES_N) * C::TN < ncols;
}

// G = X W_gu^T + s (X A_gu) B_gu ; H = silu(gate) * up.   Tile: BM rows x BN/2 j.
template <class C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_gate_up(const Layer L) {
  MOE_GEMM_PROLOGUE(C)
  constexpr int JT = C::BN / 2;
  const int n = L.n, d = L.d, r = L.r, rs = L.rs;
  const int ntn = cdiv(n, JT);
  const int total = pre[L.Et] * ntn;
  const rsrc_t rx = make_rsrc(L.x, (int64_t)L.T * d * 2);
  for (int t = first_tile(); t < total; t += gridDim.x) {
    const MTile T = decode_m<C::BM>(L, pre, t, ntn);
    const int j0 = T.nt * JT;
    const bool act = wave_active<C>(T.mrows, 2 * (n - j0));
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    if constexpr (C::DMA_NS > 0) {
      const int32_t* tok = L.tok + T.row0;
      const int mrows = T.mrows;
      KDma<C::BM, C::NW, false, C::DBK> A(
          make_desc(L.x, (int64_t)L.T * d * 2),
          [&](int m) -> int64_t { return m < mrows ? (int64_t)tok[m] * d * 2 : -1; }, d);
      KDma<C::BN, C::NW, false, C::DBK> B(
          make_desc(L.w_gu + (int64_t)T.e * 2 * n * d, (int64_t)2 * n * d * 2),
          [&](int c) -> int64_t {
            return j0 + (c >> 6) * 32 + (c & 31) < n ? (int64_t)gu_row(n, j0, c) * d * 2 : -1;
          },
          d);
      with_nfm<C>(T.mrows, 2 * (n - j0), [&](auto NF) {
        run_loop_dma<C, decltype(NF)::value>(lds, A, B, d / C::DBK, acc);
      });
    } else {
      const int32_t* tok = L.tok + T.row0;
      const int mrows = T.mrows;
      KOp<C::BM, C::NT, false, false> A(
          rx, [&](int m, float&) -> int64_t { return m < mrows ? (int64_t)tok[m] * d * 2 : -1; }, d);
      KOp<C::BN, C::NT, false, false> B(
          make_rsrc(L.w_gu + (int64_t)T.e * 2 * n * d, (int64_t)2 * n * d * 2),
          [&](int c, float&) -> int64_t {
            const int row = gu_row(n, j0, c);
            return (row % n) < n && j0 + (c >> 6) * 32 + (c & 31) < n ? (int64_t)row * d * 2 : -1;
          },
          d);
      run_loop<C>(lds, A, B, d / BK, acc, act);
    }
    {
      KOp<C::BM, C::NT, true, false> A(make_rsrc(L.xa + (int64_t)T.row0 * rs, (int64_t)T.mrows * rs * 2),
                                       [&](int m, float&) -> int64_t { return (int64_t)m * rs * 2; }, rs);
      MNOp<C::BN, C::NT> B(make_rsrc(L.b_gu + (int64_t)T.e * r * 2 * n, (int64_t)r * 2 * n * 2),
                           [&](int c) {
                             return j0 + (c >> 6) * 32 + (c & 31) < n ? gu_row(n, j0, c) : -1;
                           },
                           2 * n * 2);
      run_loop<C>(lds, A, B, cdiv(rs, BK), acc, act);
    }
    // SwiGLU epilogue: a lane's fragments 2p (gate) and 2p+1 (up) cover the
    // same 32 j values.
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int wm = wid / C::WAVES_N, wn = wid % C::WAVES_N;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int m = wm * C::TM + fm * 32 + (lane & 31);
      if (m >= T.mrows) continue;
      const int64_t p = T.row0 + m;
      bf16_t* gr = L.g + p * 2 * n;
      bf16_t* hr = L.h + p * n;
#pragma unroll
      for (int pr = 0; pr < C::FN / 2; ++pr) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int j = j0 + (wn * (C::FN / 2) + pr) * 32 + g * 8 + (lane >> 5) * 4;
          if (j >= n) continue;
          float gv[4], uv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gv[q] = acc[fm][2 * pr][4 * g + q];
            uv[q] = acc[fm][2 * pr + 1][4 * g + q];
          }
          store_bf16x4(gr + j, gv[0], gv[1], gv[2], gv[3]);
          store_bf16x4(gr + n + j, uv[0], uv[1], uv[2], uv[3]);
          store_bf16x4(hr + j, silu_f(gv[0]) * uv[0], silu_f(gv[1]) * uv[1], silu_f(gv[2]) * uv[2],
                       silu_f(gv[3]) * uv[3]);
        }
      }
    }
  }
}

// O = H W_dn^T + s (H A_dn) B_dn.   Tile: BM rows x BN of d.
template <class C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_down(const Layer L) {
  MOE_GEMM_PROLOGUE(C)
  const int n = L.n, d = L.d, r = L.r, rs = L.rs;
  const int ntn = cdiv(d, C::BN);
  const int total = pre[L.Et] * ntn;
  for (int t = first_tile(); t < total; t += gridDim.x) {
    const MTile T = decode_m<C::BM>(L, pre, t, ntn);
    const int c0 = T.nt * C::BN;
    const bool act = wave_active<C>(T.mrows, d - c0);
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    if constexpr (C::DMA_NS > 0) {
      const int mrows = T.mrows;
      KDma<C::BM, C::NW, false, C::DBK> A(
          make_desc(L.h + (int64_t)T.row0 * n, (int64_t)T.mrows * n * 2),
          [&](int m) -> int64_t { return m < mrows ? (int64_t)m * n * 2 : -1; }, n);
      KDma<C::BN, C::NW, false, C::DBK> B(
          make_desc(L.w_dn + (int64_t)T.e * d * n, (int64_t)d * n * 2),
          [&](int c) -> int64_t { return c0 + c < d ? (int64_t)(c0 + c) * n * 2 : -1; }, n);
      with_nfm<C>(T.mrows, d - c0, [&](auto NF) {
        run_loop_dma<C, decltype(NF)::value>(lds, A, B, n / C::DBK, acc);
      });
    } else {
      KOp<C::BM, C::NT, false, false> A(make_rsrc(L.h + (int64_t)T.row0 * n, (int64_t)T.mrows * n * 2),
                                        [&](int m, float&) -> int64_t { return (int64_t)m * n * 2; }, n);
      KOp<C::BN, C::NT, false, false> B(make_rsrc(L.w_dn + (int64_t)T.e * d * n, (int64_t)d * n * 2),
                                        [&](int c, float&) -> int64_t {
                                          return c0 + c < d ? (int64_t)(c0 + c) * n * 2 : -1;
                                        },
                                        n);
      run_loop<C>(lds, A, B, n / BK, acc, act);
    }
    {
      KOp<C::BM, C::NT, true, false> A(make_rsrc(L.ha + (int64_t)T.row0 * rs, (int64_t)T.mrows * rs * 2),
                                       [&](int m, float&) -> int64_t { return (int64_t)m * rs * 2; }, rs);
      MNOp<C::BN, C::NT> B(make_rsrc(L.b_dn + (int64_t)T.e * r * d, (int64_t)r * d * 2),
                           [&](int c) { return c0 + c < d ? c0 + c : -1; }, d * 2);
      run_loop<C>(lds, A, B, cdiv(rs, BK), acc, act);
    }
    for_each_quad<C>(acc, [&](int m, int c, float v0, float v1, float v2, float v3) {
      if (m < T.mrows && c0 + c < d)
        store_bf16x4(L.o + (int64_t)(T.row0 + m) * d + c0 + c, v0, v1, v2, v3);
    });
  }
}

// ---------------------------------------------------------------- rank-r pre-passes

// out[p, 0:rs] = s * act(p) . F for the expert owning row p, where F is read
// column-wise from a [K, ra] factor (A_gu, A_dn) or row-wise from a [r, K]
// factor (B_dn, B_gu: out = act . F^T), and act is X[token], H, dY[token]
// (without the routing weight) or dG.  Columns in [r, rs) come out zero.
// Every consumer of these rank-r rows takes the LoRA scale from them.

// The contraction (d, n or 2n) can be split over `nsplit` workgroups per row
// tile: each writes an fp32 partial [split][Ptot][rs] that k_prepass_reduce
// sums in split order; with nsplit == 1 the tile writes bf16 directly.
template <int BN, int KIND>
__global__ __launch_bounds__(CfgSkinny<BN>::NT) __attribute__((amdgpu_waves_per_eu(2))) void k_rank_prepass(
    const Layer L, int nsplit) {
  using C = CfgSkinny<BN>;
  MOE_GEMM_PROLOGUE(C)
  const int n = L.n, d = L.d, r = L.r, rs = L.rs, ra = L.ra;
  const int K = KIND == PRE_XA || KIND == PRE_QDN ? d : KIND == PRE_HA ? n : 2 * n;
  const int kchunk = cdiv(K / BK, nsplit) * BK;
  const int total = pre[L.Et] * nsplit;
  const rsrc_t rx = make_rsrc(KIND == PRE_XA ? L.x : L.dy, (int64_t)L.T * d * 2);
  bf16_t* out = KIND == PRE_XA ? L.xa : KIND == PRE_HA ? L.ha : KIND == PRE_QDN ? L.qdn : L.qgu;
  for (int t = first_tile(); t < total; t += gridDim.x) {
    const int ks = t % nsplit;
    const MTile T = decode_m<C::BM>(L, pre, t / nsplit, 1);
    const int mrows = T.mrows;
    const int kb = ks * kchunk;
    const int kn = min(K - kb, kchunk);
    const bool act = wave_active<C>(mrows, rs) && kn > 0;
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    if (KIND == PRE_XA) {
      const int32_t* tok = L.tok + T.row0;
      KOp<C::BM, C::NT, false, false> A(
          rx,
          [&](int m, float&) -> int64_t { return m < mrows ? ((int64_t)tok[m] * d + kb) * 2 : -1; },
          kn);
      MNOp<C::BN, C::NT> B(make_rsrc(L.a_gu + ((int64_t)T.e * d + kb) * ra, (int64_t)kn * ra * 2),
                           [&](int c) { return c < rs ? c : -1; }, ra * 2);
      run_loop<C>(lds, A, B, kn / BK, acc, act);
    } else if (KIND == PRE_HA) {
      KOp<C::BM, C::NT, false, false> A(
          make_rsrc(L.h + (int64_t)T.row0 * n, (int64_t)mrows * n * 2),
          [&](int m, float&) -> int64_t { return ((int64_t)m * n + kb) * 2; }, kn);
      MNOp<C::BN, C::NT> B(make_rsrc(L.a_dn + ((int64_t)T.e * n + kb) * ra, (int64_t)kn * ra * 2),
                           [&](int c) { return c < rs ? c : -1; }, ra * 2);
      run_loop<C>(lds, A, B, kn / BK, acc, act);
    } else if (KIND == PRE_QDN) {
      const int32_t* tok = L.tok + T.row0;
      KOp<C::BM, C::NT, false, false> A(
          rx,
          [&](int m, float&) -> int64_t { return m < mrows ? ((int64_t)tok[m] * d + kb) * 2 : -1; },
          kn);
      KOp<C::BN, C::NT, false, false> B(
          make_rsrc(L.b_dn + (int64_t)T.e * r * d, (int64_t)r * d * 2),
          [&](int c, float&) -> int64_t { return c < r ? ((int64_t)c * d + kb) * 2 : -1; }, kn);
      run_loop<C>(lds, A, B, kn / BK, acc, act);
    } else {
      KOp<C::BM, C::NT, false, false> A(
          make_rsrc(L.dg + (int64_t)T.row0 * 2 * n, (int64_t)mrows * 2 * n * 2),
          [&](int m, float&) -> int64_t { return ((int64_t)m * 2 * n + kb) * 2; }, kn);
      KOp<C::BN, C::NT, false, false> B(
          make_rsrc(L.b_gu + (int64_t)T.e * r * 2 * n, (int64_t)r * 2 * n * 2),
          [&](int c, float&) -> int64_t { return c < r ? ((int64_t)c * 2 * n + kb) * 2 : -1; }, kn);
      run_loop<C>(lds, A, B, kn / BK, acc, act);
    }
    const float sc = L.s;
    if (nsplit == 1) {
      for_each_quad<C>(acc, [&](int m, int c, float v0, float v1, float v2, float v3) {
        if (m < mrows && c < rs)
          store_bf16x4(out + (int64_t)(T.row0 + m) * rs + c, sc * v0, sc * v1, sc * v2, sc * v3);
      });
    } else {
      float* part = L.pre_partial + (int64_t)ks * L.Ptot * rs;
      for_each_quad<C>(acc, [&](int m, int c, float v0, float v1, float v2, float v3) {
        if (m < mrows && c < rs)
          *(float4*)(part + (int64_t)(T.row0 + m) * rs + c) = make_float4(sc * v0, sc * v1, sc * v2, sc * v3);
      });
    }
  }
}

// out[p, c] = bf16(sum over splits of the fp32 partials), 4 columns a thread.
__global__ __launch_bounds__(256) void k_prepass_reduce(const Layer L, int kind, int nsplit) {
  bf16_t* out = kind == PRE_XA ? L.xa : kind == PRE_HA ? L.ha : kind == PRE_QDN ? L.qdn : L.qgu;
  const int64_t total4 = (int64_t)L.Ptot * L.rs / 4;
  const int64_t plane = (int64_t)L.Ptot * L.rs;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total4; i += (int64_t)gridDim.x * 256) {
    float4 a = *(const float4*)(L.pre_partial + 4 * i);
    for (int s = 1; s < nsplit; ++s) {
      const float4 b = *(const float4*)(L.pre_partial + s * plane + 4 * i);
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    store_bf16x4(out + 4 * i, a.x, a.y, a.z, a.w);
  }
}

// ---------------------------------------------------------------- backward, dX side

// dH = w * (dY[token] W_dn + Q_dn A_dn^T) with Q_dn = s dY[token] B_dn^T
// (dO = w dY[token] is the gradient of the expert output), then the SwiGLU
// backward: dgate = dH * up * silu'(gate), dup = dH * silu(gate).
template <class C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_dh(const Layer L) {
  MOE_GEMM_PROLOGUE(C)
  const int n = L.n, d = L.d, rs = L.rs, ra = L.ra;
  const int ntn = cdiv(n, C::BN);
  const int total = pre[L.Et] * ntn;
  const rsrc_t rdy = make_rsrc(L.dy, (int64_t)L.T * d * 2);
  for (int t = first_tile(); t < total; t += gridDim.x) {
    const MTile T = decode_m<C::BM>(L, pre, t, ntn);
    const int j0 = T.nt * C::BN;
    const bool act = wave_active<C>(T.mrows, n - j0);
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    {
      const int32_t* tok = L.tok + T.row0;
      const int mrows = T.mrows;
      KOp<C::BM, C::NT, false, false> A(
          rdy, [&](int m, float&) -> int64_t { return m < mrows ? (int64_t)tok[m] * d * 2 : -1; }, d);
      MNOp<C::BN, C::NT> B(make_rsrc(L.w_dn + (int64_t)T.e * d * n, (int64_t)d * n * 2),
                           [&](int c) { return j0 + c < n ? j0 + c : -1; }, n * 2);
      run_loop<C>(lds, A, B, d / BK, acc, act);
    }
    {
      KOp<C::BM, C::NT, true, false> A(make_rsrc(L.qdn + (int64_t)T.row0 * rs, (int64_t)T.mrows * rs * 2),
                                       [&](int m, float&) -> int64_t { return (int64_t)m * rs * 2; }, rs);
      KOp<C::BN, C::NT, true, false> B(make_rsrc(L.a_dn + (int64_t)T.e * n * ra, (int64_t)n * ra * 2),
                                       [&](int c, float&) -> int64_t {
                                         return j0 + c < n ? (int64_t)(j0 + c) * ra * 2 : -1;
                                       },
                                       rs);
      run_loop<C>(lds, A, B, cdiv(rs, BK), acc, act);
    }
    for_each_quad<C>(acc, [&](int m, int c, float v0, float v1, float v2, float v3) {
      const int j = j0 + c;
      if (m >= T.mrows || j >= n) return;
      const int64_t p = T.row0 + m;
      const uint2 gq = *(const uint2*)(L.g + p * 2 * n + j);
      const uint2 uq = *(const uint2*)(L.g + p * 2 * n + n + j);
      const float w = L.wgt[p];
      const float dh[4] = {w * v0, w * v1, w * v2, w * v3};
      const float gv[4] = {bf2f(gq.x & 0xffff), bf2f(gq.x >> 16), bf2f(gq.y & 0xffff), bf2f(gq.y >> 16)};
      const float uv[4] = {bf2f(uq.x & 0xffff), bf2f(uq.x >> 16), bf2f(uq.y & 0xffff), bf2f(uq.y >> 16)};
      float dgt[4], dup[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float sg = sigmoid_f(gv[q]);
        dgt[q] = dh[q] * uv[q] * (sg * (1.0f + gv[q] * (1.0f - sg)));
        dup[q] = dh[q] * (gv[q] * sg);
      }
      store_bf16x4(L.dg + p * 2 * n + j, dgt[0], dgt[1], dgt[2], dgt[3]);
      store_bf16x4(L.dg + p * 2 * n + n + j, dup[0], dup[1], dup[2], dup[3]);
    });
  }
}

// dX_pair = dG W_gu + s (dG B_gu^T) A_gu^T.   Tile: BM rows x BN of d.
template <class C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_dx(const Layer L) {
  MOE_GEMM_PROLOGUE(C)
  const int n = L.n, d = L.d, rs = L.rs, ra = L.ra;
  const int ntn = cdiv(d, C::BN);
  const int total = pre[L.Et] * ntn;
  for (int t = first_tile(); t < total; t += gridDim.x) {
    const MTile T = decode_m<C::BM>(L, pre, t, ntn);
    const int c0 = T.nt * C::BN;
    const bool act = wave_active<C>(T.mrows, d - c0);
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    {
      KOp<C::BM, C::NT, false, false> A(
          make_rsrc(L.dg + (int64_t)T.row0 * 2 * n, (int64_t)T.mrows * 2 * n * 2),
          [&](int m, float&) -> int64_t { return (int64_t)m * 2 * n * 2; }, 2 * n);
      MNOp<C::BN, C::NT> B(make_rsrc(L.w_gu + (int64_t)T.e * 2 * n * d, (int64_t)2 * n * d * 2),
                           [&](int c) { return c0 + c < d ? c0 + c : -1; }, d * 2);
      run_loop<C>(lds, A, B, 2 * n / BK, acc, act);
    }
    {
      KOp<C::BM, C::NT, true, false> A(make_rsrc(L.qgu + (int64_t)T.row0 * rs, (int64_t)T.mrows * rs * 2),
                                       [&](int m, float&) -> int64_t { return (int64_t)m * rs * 2; }, rs);
      KOp<C::BN, C::NT, true, false> B(make_rsrc(L.a_gu + (int64_t)T.e * d * ra, (int64_t)d * ra * 2),
                                       [&](int c, float&) -> int64_t {
                                         return c0 + c < d ? (int64_t)(c0 + c) * ra * 2 : -1;
                                       },
                                       rs);
      run_loop<C>(lds, A, B, cdiv(rs, BK), acc, act);
    }
    for_each_quad<C>(acc, [&](int m, int c, float v0, float v1, float v2, float v3) {
      if (m < T.mrows && c0 + c < d)
        store_bf16x4(L.o + (int64_t)(T.row0 + m) * d + c0 + c, v0, v1, v2, v3);
    });
  }
}

// ---------------------------------------------------------------- LoRA gradients

// out[e] (M x N, fp32) = sum over expert e's rows p of U(p, m) V(p, c); the
// LoRA scale s is already inside the rank-r rows (s X A_gu, s H A_dn, Q_dn,
// Q_gu).  Both operands are read with the row index p as contraction index.  A chunk
// of at most L.splitk rows makes one partial; an expert with a single
// chunk writes its result directly, otherwise into its partial slot for the
// fixed-order reduction.
enum GradKind { GR_DB_DN = 0, GR_DA_DN = 1, GR_DB_GU = 2, GR_DA_GU = 3 };

template <class C, int KIND>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::OCC))) void k_lora_grad(const Layer L) {
  constexpr int BM = C::BM, BN = C::BN, NT = C::NT;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_ELEMS];
  __shared__ int pre[MAX_ET + 1];
  __shared__ int sh[C::NW];
  expert_prefix<NT>(L, pre, sh, [&](int e) { return cdiv(seg_count(L, e), L.splitk); });
  const int n = L.n, d = L.d, rs = L.rs;
  int M, N;
  grad_shape(KIND, d, n, L.r, M, N);
  const int nmt = cdiv(M, BM), nnt = cdiv(N, BN);
  const int per_slot = nmt * nnt;
  const int total = pre[L.Et] * per_slot;
  float* outbase = KIND == GR_DB_DN ? L.db_dn : KIND == GR_DA_DN ? L.da_dn
                 : KIND == GR_DB_GU ? L.db_gu : L.da_gu;
  float* partial = L.partial + L.partial_off[KIND];
  const rsrc_t rx = make_rsrc(KIND == GR_DB_DN ? L.dy : L.x, (int64_t)L.T * d * 2);
  for (int t = first_tile(); t < total; t += gridDim.x) {
    const int slot = t / per_slot;
    const int rem = t - slot * per_slot;
    const int nt = rem / nmt, mt = rem - nt * nmt;
    const int e = find_expert(pre, L.Et, slot, 1);
    const int chunk = slot - pre[e];
    const int nchunk = pre[e + 1] - pre[e];
    const int kb = seg_start(L, e) + chunk * L.splitk;
    const int kn = min(seg_count(L, e) - chunk * L.splitk, L.splitk);
    const int m0 = mt * BM, c0 = nt * BN;
    const int nk = cdiv(kn, BK);
    const bool act = wave_active<C>(M - m0, N - c0);
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    const rsrc_t rtok = make_rsrc(L.tok + kb, (int64_t)kn * 4);
    const rsrc_t rwgt = make_rsrc(L.wgt + kb, (int64_t)kn * 4);
    if (KIND == GR_DB_DN) {  // (s H A_dn)^T (w dY[token]) : M = r, N = d
      MNOp<BM, NT> A(make_rsrc(L.ha + (int64_t)kb * rs, (int64_t)kn * rs * 2),
                     [&](int m) { return m0 + m < rs ? m0 + m : -1; }, rs * 2);
      MNGather<BN, NT, true> B(rx, rtok, rwgt, [&](int c) { return c0 + c < d ? c0 + c : -1; }, d * 2,
                               kn);
      run_loop<C>(lds, A, B, nk, acc, act);
    } else if (KIND == GR_DA_DN) {  // H^T (w Q_dn) : M = n, N = r
      MNOp<BM, NT> A(make_rsrc(L.h + (int64_t)kb * n, (int64_t)kn * n * 2),
                     [&](int m) { return m0 + m < n ? m0 + m : -1; }, n * 2);
      MNOp<BN, NT, 3, true> B(make_rsrc(L.qdn + (int64_t)kb * rs, (int64_t)kn * rs * 2),
                              [&](int c) { return c0 + c < rs ? c0 + c : -1; }, rs * 2, rwgt);
      run_loop<C>(lds, A, B, nk, acc, act);
    } else if (KIND == GR_DB_GU) {  // (s X A_gu)^T dG : M = r, N = 2n
      MNOp<BM, NT> A(make_rsrc(L.xa + (int64_t)kb * rs, (int64_t)kn * rs * 2),
                     [&](int m) { return m0 + m < rs ? m0 + m : -1; }, rs * 2);
      MNOp<BN, NT> B(make_rsrc(L.dg + (int64_t)kb * 2 * n, (int64_t)kn * 2 * n * 2),
                     [&](int c) { return c0 + c < 2 * n ? c0 + c : -1; }, 2 * n * 2);
      run_loop<C>(lds, A, B, nk, acc, act);
    } else {  // X^T Q_gu : M = d, N = r
      MNGather<BM, NT, false> A(rx, rtok, rwgt, [&](int m) { return m0 + m < d ? m0 + m : -1; }, d * 2,
                                kn);
      MNOp<BN, NT> B(make_rsrc(L.qgu + (int64_t)kb * rs, (int64_t)kn * rs * 2),
                     [&](int c) { return c0 + c < rs ? c0 + c : -1; }, rs * 2);
      run_loop<C>(lds, A, B, nk, acc, act);
    }
    const bool direct = nchunk == 1;
    float* out = direct ? outbase + (int64_t)e * M * N : partial + (int64_t)slot * M * N;
    for_each_quad<C>(acc, [&](int m, int c, float v0, float v1, float v2, float v3) {
      const int gm = m0 + m, gc = c0 + c;
      if (gm >= M) return;
      float* o = out + (int64_t)gm * N + gc;
      if ((N & 3) == 0) {
        if (gc < N) *(float4*)o = make_float4(v0, v1, v2, v3);
      } else {
        const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (gc + q < N) o[q] = vv[q];
      }
    });
  }
}

// For all four gradients at once (blockIdx.y = kind): out[e] = the sum of
// expert e's partials in chunk order when it has >= 2 chunks, zeros when it
// has no rows; single-chunk experts were written by the GEMM and are skipped.
// Every block builds the per-expert chunk prefix in LDS, walks the expert
// list and takes a grid-stride slice of each expert that needs it, so the
// launch costs little when none does.
constexpr int RED_NT = 256, RED_GX = 64;
__global__ __launch_bounds__(RED_NT) void k_grad_reduce(const Layer L) {
  const int kind = blockIdx.y;
  int M, N;
  grad_shape(kind, L.d, L.n, L.r, M, N);
  float* outbase = kind == GR_DB_DN ? L.db_dn : kind == GR_DA_DN ? L.da_dn
                 : kind == GR_DB_GU ? L.db_gu : L.da_gu;
  const float* partial = L.partial + L.partial_off[kind];
  const int64_t MN = (int64_t)M * N;
  // first partial slot of every expert (chunks of the experts before it)
  __shared__ int pre[MAX_ET + 1];
  __shared__ int sh[RED_NT / 64];
  expert_prefix<RED_NT>(L, pre, sh, [&](int e) { return cdiv(seg_count(L, e), L.splitk); });
  // usually every expert has exactly one chunk: then nothing is left to do
  int need = 0;
  for (int e = threadIdx.x; e < L.Et; e += RED_NT) need |= pre[e + 1] - pre[e] != 1;
  if (!__syncthreads_or(need)) return;
  for (int e = 0; e < L.Et; ++e) {
    const int slot0 = pre[e], nchunk = pre[e + 1] - slot0;
    if (nchunk == 1) continue;
    float* out = outbase + (int64_t)e * MN;
    for (int64_t i = (int64_t)blockIdx.x * RED_NT + threadIdx.x; i < MN; i += (int64_t)gridDim.x * RED_NT) {
      float acc = 0.0f;
      for (int c = 0; c < nchunk; ++c) acc += partial[(int64_t)(slot0 + c) * MN + i];
      out[i] = acc;
    }
  }
}

// ---------------------------------------------------------------- launchers

// Workgroups that fit on one CU at once, from the tile's LDS footprint.
template <class C>
constexpr int wg_per_cu() {
  return (C::LDS_ELEMS * 2 + 4096) * 2 <= 160 * 1024 ? 2 : 1;
}

static int grid_for(int max_tiles, int per_cu, int ncu) {
  int g = std::min(max_tiles, per_cu * ncu);
  g = std::max(g, 1);
  return (g + 7) & ~7;
}

static int mtiles_bound(const Layer& L, int BM) { return L.Ptot / BM + L.Et; }

#ifndef MOE_STREAM_PRE
#define MOE_STREAM_PRE 1
#endif

template <int KIND>
static void launch_prepass(const Layer& L, hipStream_t st, const char* name) {
  if ((L.engines & ENG_RANK_STREAM) && L.rs <= 64) {
    (void)stream_prepass(L, KIND, st);
    return;
  }
  const int mt = mtiles_bound(L, 128);
  const int K = KIND == PRE_XA || KIND == PRE_QDN ? L.d : KIND == PRE_HA ? L.n : 2 * L.n;
  const int nsplit = prepass_splits(L.Ptot, L.Et, K, L.ncu);
  if (L.rs <= 64) {
    using C = CfgSkinny<64>;
    MOE_LAUNCH(name, (k_rank_prepass<64, KIND>), dim3(grid_for(mt * nsplit, wg_per_cu<C>(), L.ncu)),
               dim3(C::NT), 0, st, L, nsplit);
  } else {
    using C = CfgSkinny<128>;
    MOE_LAUNCH(name, (k_rank_prepass<128, KIND>), dim3(grid_for(mt * nsplit, wg_per_cu<C>(), L.ncu)),
               dim3(C::NT), 0, st, L, nsplit);
  }
  if (nsplit > 1) {
    const int g = (int)std::min<int64_t>(cdiv64((int64_t)L.Ptot * L.rs / 4, 256), 4096);
    MOE_LAUNCH("prepass_reduce", k_prepass_reduce, dim3(g), dim3(256), 0, st, L, KIND, nsplit);
  }
}

// The streamed products in the tile configuration the layer's engine bits
// give each one (product p: 0 gate_up, 1 down, 2 dh, 3 dx): bit 5 + p =
// 256-row tiles, bit 9 + p = 32-k ring stages.
static int tile_cfg(const Layer& L, int p) {
  return (int)((L.engines >> (5 + p)) & 1u) | (int)(((L.engines >> (9 + p)) & 1u) << 1);
}
#define MOE_STREAM_DISPATCH(fn, p)                       \
  hipError_t fn(const Layer& L, hipStream_t st) {        \
    switch (tile_cfg(L, p)) {                            \
      case 1: return t256k64::fn(L, st);                 \
      case 2: return t320k32::fn(L, st);                 \
      case 3: return t256k32::fn(L, st);                 \
      default: return t320k64::fn(L, st);                \
    }                                                    \
  }
MOE_STREAM_DISPATCH(stream_gate_up, 0)
MOE_STREAM_DISPATCH(stream_down, 1)
MOE_STREAM_DISPATCH(stream_dh, 2)
MOE_STREAM_DISPATCH(stream_dx, 3)
#undef MOE_STREAM_DISPATCH

hipError_t gemm_gate_up(const Layer& L, hipStream_t st) {
  using C = MainCfg<MOE_CFG_GU>::type;
  // on merged weights: the streamed product without its low-rank pass
  if (!L.lora) return stream_gate_up(L, st);
  launch_prepass<PRE_XA>(L, st, "prepass_xa");
  if (L.engines & ENG_GU_STREAM) return stream_gate_up(L, st);
  const int tiles = mtiles_bound(L, C::BM) * cdiv(L.n, C::BN / 2);
  MOE_LAUNCH("gate_up", k_gate_up<C>, dim3(grid_for(tiles, wg_per_cu<C>(), L.ncu)), dim3(C::NT), 0,
             st, L);
  return hipGetLastError();
}

hipError_t gemm_down(const Layer& L, hipStream_t st) {
  using C = MainCfg<MOE_CFG_DN>::type;
  if (!L.lora) return stream_down(L, st);
  launch_prepass<PRE_HA>(L, st, "prepass_ha");
  if (L.engines & ENG_DN_STREAM) return stream_down(L, st);
  const int tiles = mtiles_bound(L, C::BM) * cdiv(L.d, C::BN);
  MOE_LAUNCH("down", k_down<C>, dim3(grid_for(tiles, wg_per_cu<C>(), L.ncu)), dim3(C::NT), 0, st, L);
  return hipGetLastError();
}

hipError_t gemm_dh(const Layer& L, hipStream_t st) {
  using C = MainCfg<MOE_CFG_DH>::type;
  launch_prepass<PRE_QDN>(L, st, "prepass_qdn");
  if (L.engines & ENG_DH_STREAM) return stream_dh(L, st);
  const int tiles = mtiles_bound(L, C::BM) * cdiv(L.n, C::BN);
  MOE_LAUNCH("dh", k_dh<C>, dim3(grid_for(tiles, wg_per_cu<C>(), L.ncu)), dim3(C::NT), 0, st, L);
  return hipGetLastError();
}

uint32_t default_engines() {
  return (MOE_STREAM_GU ? ENG_GU_STREAM : 0u) | (MOE_STREAM_DN ? ENG_DN_STREAM : 0u) |
         (MOE_STREAM_DH ? ENG_DH_STREAM : 0u) | (MOE_STREAM_DX ? ENG_DX_STREAM : 0u) |
         (MOE_STREAM_PRE ? ENG_RANK_STREAM : 0u);
}

bool prepass_writes_weighted_rows(const Layer& L) { return (L.engines & ENG_RANK_STREAM) && L.rs <= 64; }

hipError_t gemm_dx(const Layer& L, hipStream_t st) {
  using C = MainCfg<MOE_CFG_DX>::type;
  launch_prepass<PRE_QGU>(L, st, "prepass_qgu");
  if (L.engines & ENG_DX_STREAM) return stream_dx(L, st);
  const int tiles = mtiles_bound(L, C::BM) * cdiv(L.d, C::BN);
  MOE_LAUNCH("dx", k_dx<C>, dim3(grid_for(tiles, wg_per_cu<C>(), L.ncu)), dim3(C::NT), 0, st, L);
  return hipGetLastError();
}

template <class C, int KIND>
static void launch_grad(const Layer& L, hipStream_t st, const char* name) {
  int M, N;
  grad_shape(KIND, L.d, L.n, L.r, M, N);
  const int slots = L.Ptot / L.splitk + L.Et;
  const int tiles = slots * cdiv(M, C::BM) * cdiv(N, C::BN);
  MOE_LAUNCH(name, (k_lora_grad<C, KIND>), dim3(grid_for(tiles, wg_per_cu<C>(), L.ncu)), dim3(C::NT),
             0, st, L);
}

// LoRA-gradient tiles for rank <= 64: M = r (dB) or N = r (dA).
template <int I> struct GradCfgB;
template <> struct GradCfgB<0> { using type = Cfg<64, 128, 2, 2>; };
template <> struct GradCfgB<1> { using type = Cfg<64, 256, 1, 4>; };
template <> struct GradCfgB<2> { using type = Cfg<64, 256, 2, 4>; };
template <> struct GradCfgB<3> { using type = Cfg<64, 128, 1, 2, 2, 0, 64, 2>; };
template <> struct GradCfgB<4> { using type = Cfg<64, 128, 2, 2, 1>; };
template <int I> struct GradCfgA;
template <> struct GradCfgA<0> { using type = Cfg<128, 64, 4, 1>; };
template <> struct GradCfgA<1> { using type = Cfg<256, 64, 4, 1>; };
template <> struct GradCfgA<2> { using type = Cfg<256, 64, 4, 2>; };
template <> struct GradCfgA<3> { using type = Cfg<128, 64, 2, 1, 2, 0, 64, 2>; };
template <> struct GradCfgA<4> { using type = Cfg<128, 64, 4, 1, 1>; };
#ifndef MOE_GRAD_B
#define MOE_GRAD_B 0
#endif
#ifndef MOE_GRAD_A
#define MOE_GRAD_A 0
#endif


hipError_t gemm_lora_grads(const Layer& L, hipStream_t st) {
  if ((L.engines & ENG_RANK_STREAM) && L.rs <= 64) {
    const hipError_t e = dma_lora_grads(L, st);
    if (e != hipSuccess) return e;
  } else if (L.rs <= 64) {
    using CB = GradCfgB<MOE_GRAD_B>::type;
    using CA = GradCfgA<MOE_GRAD_A>::type;
    launch_grad<CB, GR_DB_DN>(L, st, "grad_db_dn");
    launch_grad<CA, GR_DA_DN>(L, st, "grad_da_dn");
    launch_grad<CB, GR_DB_GU>(L, st, "grad_db_gu");
    launch_grad<CA, GR_DA_GU>(L, st, "grad_da_gu");
  } else {
    launch_grad<Cfg<128, 128, 2, 2>, GR_DB_DN>(L, st, "grad_db_dn");
    launch_grad<Cfg<128, 128, 2, 2>, GR_DA_DN>(L, st, "grad_da_dn");
    launch_grad<Cfg<128, 128, 2, 2>, GR_DB_GU>(L, st, "grad_db_gu");
    launch_grad<Cfg<128, 128, 2, 2>, GR_DA_GU>(L, st, "grad_da_gu");
  }
  int64_t mn_max = 0;
  for (int kind = 0; kind < 4; ++kind) {
    int M, N;
    grad_shape(kind, L.d, L.n, L.r, M, N);
    mn_max = std::max<int64_t>(mn_max, (int64_t)M * N);
  }
  const int gx = (int)std::min<int64_t>(cdiv64(mn_max, RED_NT), RED_GX);
  MOE_LAUNCH("reduce_grads", k_grad_reduce, dim3(gx, 4), dim3(RED_NT), 0, st, L);
  return hipGetLastError();
}

}  // inline namespace MOE_EL
}  // namespace moe
