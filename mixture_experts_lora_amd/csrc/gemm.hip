// Grouped GEMMs of the MoE-LoRA layer on gfx950 MFMA.
//
// Every product of the layer is a GEMM over the ragged per-expert row
// segments of the sorted (token, expert) pairs, against that expert's slice of
// a stacked parameter (Unsloth faster-MoE page, "What is torch._grouped_mm?").
// The LoRA term stays split ("Faster LoRA MoE training"): the rank-r
// activation (X A, H A_dn, dO B_dn^T, dG B_gu^T) is produced by a skinny
// pre-pass, and its product with the other factor runs as a second, short
// MFMA pass into the SAME accumulator tile as the base product, so the
// adapter delta (A B)^T is never formed.
//
// Engine
//  - one workgroup = 4 waves = 256 threads; tile BM x BN, K step 64;
//  - v_mfma_f32_32x32x16_bf16, fp32 accumulation; the operands are swapped
//    (mfma(B, A)) so each lane owns 4 consecutive output columns of one row
//    and the epilogue writes 8-byte (bf16) or 16-byte (fp32) vectors;
//  - LDS holds both operands K-contiguous, rows padded to 72 elements, two
//    stages (global loads of step k+1 are in flight during the MFMAs of k);
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

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int NT = 256;
constexpr int BK = 64;
constexpr int LDK = BK + 8;
constexpr int MAX_ET = 512;

template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WM_, WAVES_N = WN_;
  static_assert(WM_ * WN_ == 4, "four waves");
  static constexpr int TM = BM / WM_, TN = BN / WN_;
  static constexpr int FM = TM / 32, FN = TN / 32;
  static_assert(FM >= 1 && FN >= 1, "wave tile at least 32x32");
  static constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LDS_ELEMS = 2 * STAGE;
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ int seg_start(const Layer& L, int e) {
  return e < L.E ? L.offsets[e] : L.P;
}
__device__ __forceinline__ int seg_count(const Layer& L, int e) {
  return e < L.E ? L.offsets[e + 1] - L.offsets[e] : L.T;
}
__device__ __forceinline__ int token_of(const Layer& L, int p) {
  return p < L.P ? L.sorted_pair[p] / L.k : p - L.P;
}
__device__ __forceinline__ float weight_of(const Layer& L, int p) {
  return p < L.P ? L.topk_w[L.sorted_pair[p]] : 1.0f;
}

// sorted position -> token / routing weight, small enough to capture by value
struct Rows {
  const int32_t* sp;
  const float* w;
  int k, P;
  __device__ __forceinline__ int token(int p) const { return p < P ? sp[p] / k : p - P; }
  __device__ __forceinline__ float weight(int p) const { return p < P ? w[sp[p]] : 1.0f; }
};
__device__ __forceinline__ Rows rows_of(const Layer& L) {
  Rows r;
  r.sp = L.sorted_pair;
  r.w = L.topk_w;
  r.k = L.k;
  r.P = L.P;
  return r;
}

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

// R rows of a K-contiguous source (row r at rowptr(r), K elements in a row);
// each thread moves 16-byte chunks.
template <int R, class RowFn>
struct KOperand {
  static constexpr int CH = R * (BK / 8);
  static constexpr int PER = (CH + NT - 1) / NT;
  const bf16_t* ptr[PER];
  float scl[PER];
  uint4 v[PER];
  int kmax;
  bool scaled;

  __device__ KOperand(RowFn rowfn, int kmax_, bool scaled_) : kmax(kmax_), scaled(scaled_) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      float sc = 1.0f;
      const bf16_t* p = nullptr;
      if (c < CH) p = rowfn(c >> 3, sc);
      ptr[i] = p ? p + (c & 7) * 8 : nullptr;
      scl[i] = sc;
    }
  }
  __device__ __forceinline__ void fetch(int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      if (ptr[i] && k0 + (c & 7) * 8 < kmax)
        v[i] = *(const uint4*)(ptr[i] + k0);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      if (CH % NT == 0 || c < CH) {
        uint4 w = v[i];
        if (scaled) w = scale8(w, scl[i]);
        *(uint4*)(lds + (c >> 3) * LDK + (c & 7) * 8) = w;
      }
    }
  }
};

// R columns of a source whose contraction index is the row index: element
// (k, c) at krow(k)[col(c)], 8 consecutive columns contiguous.  A thread
// loads a 4(k) x 8(c) block and writes it transposed into the K-contiguous
// LDS panel.  Lane mapping (kq fastest) keeps a half-wave's 8-byte LDS stores
// on distinct banks.
template <int R, class KRowFn>
struct MNOperand {
  static constexpr int NB = (BK / 4) * (R / 8);
  static constexpr int PER = (NB + NT - 1) / NT;
  int col[PER];  // element offset of the block's first column, -1 = outside
  uint4 v[PER][4];
  float scl[PER][4];
  KRowFn krow;
  int kbase, kmax;
  bool scaled;

  template <class ColFn>
  __device__ MNOperand(ColFn colfn, KRowFn krow_, int kbase_, int kmax_, bool scaled_)
      : krow(krow_), kbase(kbase_), kmax(kmax_), scaled(scaled_) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int bi = threadIdx.x + i * NT;
      col[i] = bi < NB ? colfn((bi >> 4) * 8) : -1;
    }
  }
  __device__ __forceinline__ void fetch(int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int kq = (threadIdx.x + i * NT) & 15;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kr = kbase + k0 + kq * 4 + q;
        float sc = 1.0f;
        const bf16_t* p = (col[i] >= 0 && kr < kmax) ? krow(kr, sc) : nullptr;
        v[i][q] = p ? *(const uint4*)(p + col[i]) : make_uint4(0, 0, 0, 0);
        scl[i][q] = sc;
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int bi = threadIdx.x + i * NT;
      if (NB % NT != 0 && bi >= NB) continue;
      const int kq = bi & 15, mg = bi >> 4;
      uint4 w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) w[q] = scaled ? scale8(v[i][q], scl[i][q]) : v[i][q];
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
  }
};

template <int R, class RowFn>
__device__ __forceinline__ KOperand<R, RowFn> kop(RowFn f, int kmax, bool scaled = false) {
  return KOperand<R, RowFn>(f, kmax, scaled);
}
template <int R, class ColFn, class KRowFn>
__device__ __forceinline__ MNOperand<R, KRowFn> mnop(ColFn c, KRowFn f, int kbase, int kmax,
                                                     bool scaled = false) {
  return MNOperand<R, KRowFn>(c, f, kbase, kmax, scaled);
}

// ---------------------------------------------------------------- MFMA main loop

template <class C>
__device__ __forceinline__ void mma_stage(const bf16_t* As, const bf16_t* Bs,
                                          f32x16 (&acc)[C::FM][C::FN]) {
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

// Pipelined K loop over nk steps of 64 (ends with a barrier, so the LDS can
// be reused right after).
template <class C, class OA, class OB>
__device__ __forceinline__ void run_loop(bf16_t* lds, OA& oa, OB& ob, int nk,
                                         f32x16 (&acc)[C::FM][C::FN]) {
  if (nk <= 0) return;
  oa.fetch(0);
  ob.fetch(0);
  oa.store(lds);
  ob.store(lds + C::A_ELEMS);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bf16_t* As = lds + (kt & 1) * C::STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      oa.fetch((kt + 1) * BK);
      ob.fetch((kt + 1) * BK);
    }
    mma_stage<C>(As, As + C::A_ELEMS, acc);
    if (more) {
      bf16_t* An = lds + ((kt + 1) & 1) * C::STAGE;
      oa.store(An);
      ob.store(An + C::A_ELEMS);
    }
    __syncthreads();
  }
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
        f(row, col, fn, acc[fm][fn][4 * g], acc[fm][fn][4 * g + 1], acc[fm][fn][4 * g + 2],
          acc[fm][fn][4 * g + 3]);
      }
}

__device__ __forceinline__ void store_bf16x4(bf16_t* p, float a, float b, float c, float d) {
  *(uint2*)p = make_uint2(pack2(a, b), pack2(c, d));
}

// ---------------------------------------------------------------- schedules

// Persistent loop order: round-robin XCD dealing -> contiguous logical tiles
// per XCD inside a round.
__device__ __forceinline__ int first_tile() {
  const int G = gridDim.x;
  return (G & 7) ? (int)blockIdx.x : (int)((blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3));
}

// Row-ragged schedule: tiles (e, nt, mt), mt fastest; BM rows of a segment.
struct MSched {
  int* pre;  // [Et+1] exclusive prefix of per-expert M-tile counts
  int Et;
  template <int BM>
  __device__ void init(const Layer& L, int* lds_pre, int* sh) {
    pre = lds_pre;
    Et = L.Et;
    const int e0 = 2 * threadIdx.x, e1 = e0 + 1;
    const int c0 = e0 < Et ? cdiv(seg_count(L, e0), BM) : 0;
    const int c1 = e1 < Et ? cdiv(seg_count(L, e1), BM) : 0;
    int tot;
    const int ex = block_excl_scan256(c0 + c1, sh, &tot);
    if (e0 < Et) pre[e0] = ex;
    if (e1 < Et) pre[e1] = ex + c0;
    if (threadIdx.x == 0) pre[Et] = tot;
    __syncthreads();
  }
  __device__ int total_m() const { return pre[Et]; }
  __device__ void decode(int t, int ntn, int& e, int& mt, int& nt) const {
    int lo = 0, hi = Et - 1;  // largest e with pre[e]*ntn <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] * ntn <= t) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int local = t - pre[e] * ntn;
    const int nm = pre[e + 1] - pre[e];
    nt = local / nm;
    mt = local - nt * nm;
  }
};

// Contraction-ragged schedule (LoRA gradients): per expert, the segment rows
// are split in chunks of SPLITK_ROWS; tiles (slot, nt, mt) with slot =
// pre[e] + chunk.
struct KSched {
  int* pre;
  int Et;
  __device__ void init(const Layer& L, int* lds_pre, int* sh) {
    pre = lds_pre;
    Et = L.Et;
    const int e0 = 2 * threadIdx.x, e1 = e0 + 1;
    const int c0 = e0 < Et ? cdiv(seg_count(L, e0), SPLITK_ROWS) : 0;
    const int c1 = e1 < Et ? cdiv(seg_count(L, e1), SPLITK_ROWS) : 0;
    int tot;
    const int ex = block_excl_scan256(c0 + c1, sh, &tot);
    if (e0 < Et) pre[e0] = ex;
    if (e1 < Et) pre[e1] = ex + c0;
    if (threadIdx.x == 0) pre[Et] = tot;
    __syncthreads();
  }
  __device__ int slots() const { return pre[Et]; }
  __device__ int expert_of_slot(int slot) const {
    int lo = 0, hi = Et - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= slot) lo = mid; else hi = mid - 1;
    }
    return lo;
  }
};

// ---------------------------------------------------------------- forward

// gate/up column interleave of the gate_up tile: 32-column groups alternate
// gate (rows j of W_gu) and up (rows n + j), so one lane holds gate and up of
// the same (row, j) in its two N fragments.
__device__ __forceinline__ int gu_row(int n, int j0, int c) {
  const int grp = c >> 5;
  return ((grp & 1) ? n : 0) + j0 + (grp >> 1) * 32 + (c & 31);
}

using CfgMain = Cfg<128, 128, 2, 2>;

// G = X W_gu^T + s (X A_gu) B_gu ; H = silu(gate) * up.   Tile: 128 rows x 64 j.
__global__ __launch_bounds__(NT) void k_gate_up(const Layer L) {
  using C = CfgMain;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_ELEMS];
  __shared__ int pre[MAX_ET + 1];
  __shared__ int sh[4];
  MSched sch;
  sch.init<C::BM>(L, pre, sh);
  const int ntn = L.n / 64;
  const int total = sch.total_m() * ntn;
  const int n = L.n, d = L.d;
  for (int t = first_tile(); t < total; t += gridDim.x) {
    int e, mt, nt;
    sch.decode(t, ntn, e, mt, nt);
    const int row0 = seg_start(L, e) + mt * C::BM;
    const int mrows = min(C::BM, seg_count(L, e) - mt * C::BM);
    const int j0 = nt * 64;
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    {
      auto A = kop<C::BM>(
          [&](int m, float&) -> const bf16_t* {
            return m < mrows ? L.x + (int64_t)token_of(L, row0 + m) * d : nullptr;
          },
          d);
      const bf16_t* wb = L.w_gu + (int64_t)e * 2 * n * d;
      auto B = kop<C::BN>(
          [&](int c, float&) -> const bf16_t* { return wb + (int64_t)gu_row(n, j0, c) * d; }, d);
      run_loop<C>(lds, A, B, d / BK, acc);
    }
    {
      auto A = kop<C::BM>(
          [&](int m, float&) -> const bf16_t* {
            return m < mrows ? L.xa + (int64_t)(row0 + m) * L.rs : nullptr;
          },
          L.rs);
      const bf16_t* bb = L.b_gu + (int64_t)e * L.r * 2 * n;
      const float s = L.s;
      auto B = mnop<C::BN>([&](int c) { return gu_row(n, j0, c); },
                           [=](int kr, float& sc) -> const bf16_t* {
                             sc = s;
                             return bb + (int64_t)kr * 2 * n;
                           },
                           0, L.r, s != 1.0f);
      run_loop<C>(lds, A, B, cdiv(L.rs, BK), acc);
    }
    // SwiGLU epilogue: the lane's fragments fn=0 (gate) and fn=1 (up) cover the
    // same 32 j values.
    {
      const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
      const int wm = wid / C::WAVES_N, wn = wid % C::WAVES_N;
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm) {
        const int m = wm * C::TM + fm * 32 + (lane & 31);
        if (m >= mrows) continue;
        const int64_t p = row0 + m;
        bf16_t* gr = L.g + p * 2 * n;
        bf16_t* hr = L.h + p * n;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int j = j0 + wn * 32 + g * 8 + (lane >> 5) * 4;
          const f32x16& ga = acc[fm][0];
          const f32x16& ua = acc[fm][1];
          float gv[4], uv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            gv[q] = ga[4 * g + q];
            uv[q] = ua[4 * g + q];
          }
          store_bf16x4(gr + j, gv[0], gv[1], gv[2], gv[3]);
          store_bf16x4(gr + n + j, uv[0], uv[1], uv[2], uv[3]);
          store_bf16x4(hr + j, silu_f(gv[0]) * uv[0], silu_f(gv[1]) * uv[1],
                       silu_f(gv[2]) * uv[2], silu_f(gv[3]) * uv[3]);
        }
      }
    }
  }
}

// O = H W_dn^T + s (H A_dn) B_dn.   Tile: 128 rows x 128 of d.
__global__ __launch_bounds__(NT) void k_down(const Layer L) {
  using C = CfgMain;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_ELEMS];
  __shared__ int pre[MAX_ET + 1];
  __shared__ int sh[4];
  MSched sch;
  sch.init<C::BM>(L, pre, sh);
  const int n = L.n, d = L.d;
  const int ntn = cdiv(d, C::BN);
  const int total = sch.total_m() * ntn;
  for (int t = first_tile(); t < total; t += gridDim.x) {
    int e, mt, nt;
    sch.decode(t, ntn, e, mt, nt);
    const int row0 = seg_start(L, e) + mt * C::BM;
    const int mrows = min(C::BM, seg_count(L, e) - mt * C::BM);
    const int c0 = nt * C::BN;
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    {
      auto A = kop<C::BM>(
          [&](int m, float&) -> const bf16_t* {
            return m < mrows ? L.h + (int64_t)(row0 + m) * n : nullptr;
          },
          n);
      const bf16_t* wb = L.w_dn + (int64_t)e * d * n;
      auto B = kop<C::BN>(
          [&](int c, float&) -> const bf16_t* {
            return c0 + c < d ? wb + (int64_t)(c0 + c) * n : nullptr;
          },
          n);
      run_loop<C>(lds, A, B, n / BK, acc);
    }
    {
      auto A = kop<C::BM>(
          [&](int m, float&) -> const bf16_t* {
            return m < mrows ? L.ha + (int64_t)(row0 + m) * L.rs : nullptr;
          },
          L.rs);
      const bf16_t* bb = L.b_dn + (int64_t)e * L.r * d;
      const float s = L.s;
      auto B = mnop<C::BN>([&](int c) { return c0 + c < d ? c0 + c : -1; },
                           [=](int kr, float& sc) -> const bf16_t* {
                             sc = s;
                             return bb + (int64_t)kr * d;
                           },
                           0, L.r, s != 1.0f);
      run_loop<C>(lds, A, B, cdiv(L.rs, BK), acc);
    }
    for_each_quad<C>(acc, [&](int m, int c, int, float v0, float v1, float v2, float v3) {
      if (m < mrows && c0 + c < d) store_bf16x4(L.o + (int64_t)(row0 + m) * d + c0 + c, v0, v1, v2, v3);
    });
  }
}

// ---------------------------------------------------------------- rank-r pre-passes

// out[p, 0:rs] = act(p) . F   where the [K x rs] factor F is read either
// column-wise from a [K, ra] array (A_gu, A_dn) or row-wise from a [r, K]
// array (B_dn, B_gu: out = act . F^T).  Columns >= r come out as zeros.
enum PrepassKind { PRE_XA = 0, PRE_HA = 1, PRE_QDN = 2, PRE_QGU = 3 };

template <int BN>
__global__ __launch_bounds__(NT) void k_rank_prepass(const Layer L, int kind) {
  using C = Cfg<128, BN, 4, 1>;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_ELEMS];
  __shared__ int pre[MAX_ET + 1];
  __shared__ int sh[4];
  MSched sch;
  sch.init<C::BM>(L, pre, sh);
  const int total = sch.total_m();
  const int n = L.n, d = L.d, r = L.r, rs = L.rs, ra = L.ra;
  for (int t = first_tile(); t < total; t += gridDim.x) {
    int e, mt, nt;
    sch.decode(t, 1, e, mt, nt);
    const int row0 = seg_start(L, e) + mt * C::BM;
    const int mrows = min(C::BM, seg_count(L, e) - mt * C::BM);
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    bf16_t* out;
    if (kind == PRE_XA) {
      out = L.xa;
      auto A = kop<C::BM>(
          [&](int m, float&) -> const bf16_t* {
            return m < mrows ? L.x + (int64_t)token_of(L, row0 + m) * d : nullptr;
          },
          d);
      const bf16_t* fb = L.a_gu + (int64_t)e * d * ra;
      auto B = mnop<C::BN>([&](int c) { return c < rs ? c : -1; },
                           [=](int kr, float&) -> const bf16_t* { return fb + (int64_t)kr * ra; },
                           0, d);
      run_loop<C>(lds, A, B, d / BK, acc);
    } else if (kind == PRE_HA) {
      out = L.ha;
      auto A = kop<C::BM>(
          [&](int m, float&) -> const bf16_t* {
            return m < mrows ? L.h + (int64_t)(row0 + m) * n : nullptr;
          },
          n);
      const bf16_t* fb = L.a_dn + (int64_t)e * n * ra;
      auto B = mnop<C::BN>([&](int c) { return c < rs ? c : -1; },
                           [=](int kr, float&) -> const bf16_t* { return fb + (int64_t)kr * ra; },
                           0, n);
      run_loop<C>(lds, A, B, n / BK, acc);
    } else if (kind == PRE_QDN) {
      out = L.qdn;
      auto A = kop<C::BM>(
          [&](int m, float& sc) -> const bf16_t* {
            if (m >= mrows) return nullptr;
            sc = weight_of(L, row0 + m);
            return L.dy + (int64_t)token_of(L, row0 + m) * d;
          },
          d, true);
      const bf16_t* fb = L.b_dn + (int64_t)e * r * d;
      auto B = kop<C::BN>(
          [&](int c, float&) -> const bf16_t* { return c < r ? fb + (int64_t)c * d : nullptr; }, d);
      run_loop<C>(lds, A, B, d / BK, acc);
    } else {
      out = L.qgu;
      auto A = kop<C::BM>(
          [&](int m, float&) -> const bf16_t* {
            return m < mrows ? L.dg + (int64_t)(row0 + m) * 2 * n : nullptr;
          },
          2 * n);
      const bf16_t* fb = L.b_gu + (int64_t)e * r * 2 * n;
      auto B = kop<C::BN>(
          [&](int c, float&) -> const bf16_t* {
            return c < r ? fb + (int64_t)c * 2 * n : nullptr;
          },
          2 * n);
      run_loop<C>(lds, A, B, 2 * n / BK, acc);
    }
    for_each_quad<C>(acc, [&](int m, int c, int, float v0, float v1, float v2, float v3) {
      if (m < mrows && c < rs) store_bf16x4(out + (int64_t)(row0 + m) * rs + c, v0, v1, v2, v3);
    });
  }
}

// ---------------------------------------------------------------- backward, dX side

// dH = dO W_dn + s (dO B_dn^T) A_dn^T with dO = w * dY[token], then the SwiGLU
// backward: dgate = dH * up * silu'(gate), dup = dH * silu(gate).
__global__ __launch_bounds__(NT) void k_dh(const Layer L) {
  using C = CfgMain;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_ELEMS];
  __shared__ int pre[MAX_ET + 1];
  __shared__ int sh[4];
  MSched sch;
  sch.init<C::BM>(L, pre, sh);
  const int n = L.n, d = L.d;
  const int ntn = cdiv(n, C::BN);
  const int total = sch.total_m() * ntn;
  for (int t = first_tile(); t < total; t += gridDim.x) {
    int e, mt, nt;
    sch.decode(t, ntn, e, mt, nt);
    const int row0 = seg_start(L, e) + mt * C::BM;
    const int mrows = min(C::BM, seg_count(L, e) - mt * C::BM);
    const int j0 = nt * C::BN;
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    {
      auto A = kop<C::BM>(
          [&](int m, float& sc) -> const bf16_t* {
            if (m >= mrows) return nullptr;
            sc = weight_of(L, row0 + m);
            return L.dy + (int64_t)token_of(L, row0 + m) * d;
          },
          d, true);
      const bf16_t* wb = L.w_dn + (int64_t)e * d * n;
      auto B = mnop<C::BN>([&](int c) { return j0 + c < n ? j0 + c : -1; },
                           [=](int kr, float&) -> const bf16_t* { return wb + (int64_t)kr * n; },
                           0, d);
      run_loop<C>(lds, A, B, d / BK, acc);
    }
    {
      auto A = kop<C::BM>(
          [&](int m, float&) -> const bf16_t* {
            return m < mrows ? L.qdn + (int64_t)(row0 + m) * L.rs : nullptr;
          },
          L.rs);
      const bf16_t* ab = L.a_dn + (int64_t)e * n * L.ra;
      const float s = L.s;
      auto B = kop<C::BN>(
          [&](int c, float& sc) -> const bf16_t* {
            sc = s;
            return j0 + c < n ? ab + (int64_t)(j0 + c) * L.ra : nullptr;
          },
          L.rs, s != 1.0f);
      run_loop<C>(lds, A, B, cdiv(L.rs, BK), acc);
    }
    for_each_quad<C>(acc, [&](int m, int c, int, float v0, float v1, float v2, float v3) {
      const int j = j0 + c;
      if (m >= mrows || j >= n) return;
      const int64_t p = row0 + m;
      const uint2 gq = *(const uint2*)(L.g + p * 2 * n + j);
      const uint2 uq = *(const uint2*)(L.g + p * 2 * n + n + j);
      const float dh[4] = {v0, v1, v2, v3};
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

// dX_pair = dG W_gu + s (dG B_gu^T) A_gu^T.   Tile: 128 rows x 128 of d.
__global__ __launch_bounds__(NT) void k_dx(const Layer L) {
  using C = CfgMain;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_ELEMS];
  __shared__ int pre[MAX_ET + 1];
  __shared__ int sh[4];
  MSched sch;
  sch.init<C::BM>(L, pre, sh);
  const int n = L.n, d = L.d;
  const int ntn = cdiv(d, C::BN);
  const int total = sch.total_m() * ntn;
  for (int t = first_tile(); t < total; t += gridDim.x) {
    int e, mt, nt;
    sch.decode(t, ntn, e, mt, nt);
    const int row0 = seg_start(L, e) + mt * C::BM;
    const int mrows = min(C::BM, seg_count(L, e) - mt * C::BM);
    const int c0 = nt * C::BN;
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    {
      auto A = kop<C::BM>(
          [&](int m, float&) -> const bf16_t* {
            return m < mrows ? L.dg + (int64_t)(row0 + m) * 2 * n : nullptr;
          },
          2 * n);
      const bf16_t* wb = L.w_gu + (int64_t)e * 2 * n * d;
      auto B = mnop<C::BN>([&](int c) { return c0 + c < d ? c0 + c : -1; },
                           [=](int kr, float&) -> const bf16_t* { return wb + (int64_t)kr * d; },
                           0, 2 * n);
      run_loop<C>(lds, A, B, 2 * n / BK, acc);
    }
    {
      auto A = kop<C::BM>(
          [&](int m, float&) -> const bf16_t* {
            return m < mrows ? L.qgu + (int64_t)(row0 + m) * L.rs : nullptr;
          },
          L.rs);
      const bf16_t* ab = L.a_gu + (int64_t)e * d * L.ra;
      const float s = L.s;
      auto B = kop<C::BN>(
          [&](int c, float& sc) -> const bf16_t* {
            sc = s;
            return c0 + c < d ? ab + (int64_t)(c0 + c) * L.ra : nullptr;
          },
          L.rs, s != 1.0f);
      run_loop<C>(lds, A, B, cdiv(L.rs, BK), acc);
    }
    for_each_quad<C>(acc, [&](int m, int c, int, float v0, float v1, float v2, float v3) {
      if (m < mrows && c0 + c < d) store_bf16x4(L.o + (int64_t)(row0 + m) * d + c0 + c, v0, v1, v2, v3);
    });
  }
}

// ---------------------------------------------------------------- LoRA gradients

// out[e] (M x N, fp32) = s * sum over expert e's rows p of U(p, m) V(p, c).
// Both operands are read with the row index p as contraction index.  A chunk
// of at most SPLITK_ROWS rows makes one partial; an expert with a single
// chunk writes its result directly, otherwise into partial[slot] for the
// fixed-order reduction.
enum GradKind { GR_DB_DN = 0, GR_DA_DN = 1, GR_DB_GU = 2, GR_DA_GU = 3 };

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(NT) void k_lora_grad(const Layer L, int kind, int M, int N) {
  using C = Cfg<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) bf16_t lds[C::LDS_ELEMS];
  __shared__ int pre[MAX_ET + 1];
  __shared__ int sh[4];
  KSched sch;
  sch.init(L, pre, sh);
  const int nmt = cdiv(M, BM), nnt = cdiv(N, BN);
  const int per_slot = nmt * nnt;
  const int total = sch.slots() * per_slot;
  const int n = L.n, d = L.d, rs = L.rs;
  float* outbase = kind == GR_DB_DN ? L.db_dn : kind == GR_DA_DN ? L.da_dn
                 : kind == GR_DB_GU ? L.db_gu : L.da_gu;
  for (int t = first_tile(); t < total; t += gridDim.x) {
    const int slot = t / per_slot;
    const int rem = t - slot * per_slot;
    const int nt = rem / nmt, mt = rem - nt * nmt;
    const int e = sch.expert_of_slot(slot);
    const int chunk = slot - pre[e];
    const int nchunk = pre[e + 1] - pre[e];
    const int kb = seg_start(L, e) + chunk * SPLITK_ROWS;
    const int ke = min(seg_start(L, e) + seg_count(L, e), kb + SPLITK_ROWS);
    const int m0 = mt * BM, c0 = nt * BN;
    const int nk = cdiv(ke - kb, BK);
    f32x16 acc[C::FM][C::FN];
    zero_acc<C>(acc);
    const Rows rw = rows_of(L);
    const bf16_t *ha = L.ha, *hh = L.h, *qdn = L.qdn, *xa = L.xa, *dg = L.dg, *qgu = L.qgu;
    const bf16_t *dy = L.dy, *xx = L.x;
    if (kind == GR_DB_DN) {  // s (H A_dn)^T dO : M = r, N = d
      auto A = mnop<BM>([&](int m) { return m0 + m < rs ? m0 + m : -1; },
                        [=](int p, float&) -> const bf16_t* { return ha + (int64_t)p * rs; },
                        kb, ke);
      auto B = mnop<BN>([&](int c) { return c0 + c < d ? c0 + c : -1; },
                        [=](int p, float& sc) -> const bf16_t* {
                          sc = rw.weight(p);
                          return dy + (int64_t)rw.token(p) * d;
                        },
                        kb, ke, true);
      run_loop<C>(lds, A, B, nk, acc);
    } else if (kind == GR_DA_DN) {  // s H^T Q_dn : M = n, N = r
      auto A = mnop<BM>([&](int m) { return m0 + m < n ? m0 + m : -1; },
                        [=](int p, float&) -> const bf16_t* { return hh + (int64_t)p * n; },
                        kb, ke);
      auto B = mnop<BN>([&](int c) { return c0 + c < rs ? c0 + c : -1; },
                        [=](int p, float&) -> const bf16_t* { return qdn + (int64_t)p * rs; },
                        kb, ke);
      run_loop<C>(lds, A, B, nk, acc);
    } else if (kind == GR_DB_GU) {  // s (X A_gu)^T dG : M = r, N = 2n
      auto A = mnop<BM>([&](int m) { return m0 + m < rs ? m0 + m : -1; },
                        [=](int p, float&) -> const bf16_t* { return xa + (int64_t)p * rs; },
                        kb, ke);
      auto B = mnop<BN>([&](int c) { return c0 + c < 2 * n ? c0 + c : -1; },
                        [=](int p, float&) -> const bf16_t* { return dg + (int64_t)p * 2 * n; },
                        kb, ke);
      run_loop<C>(lds, A, B, nk, acc);
    } else {  // s X^T Q_gu : M = d, N = r
      auto A = mnop<BM>([&](int m) { return m0 + m < d ? m0 + m : -1; },
                        [=](int p, float&) -> const bf16_t* {
                          return xx + (int64_t)rw.token(p) * d;
                        },
                        kb, ke);
      auto B = mnop<BN>([&](int c) { return c0 + c < rs ? c0 + c : -1; },
                        [=](int p, float&) -> const bf16_t* { return qgu + (int64_t)p * rs; },
                        kb, ke);
      run_loop<C>(lds, A, B, nk, acc);
    }
    const bool direct = nchunk == 1;
    float* out = direct ? outbase + (int64_t)e * M * N : L.partial + (int64_t)slot * M * N;
    const float s = direct ? L.s : 1.0f;
    for_each_quad<C>(acc, [&](int m, int c, int, float v0, float v1, float v2, float v3) {
      const int gm = m0 + m, gc = c0 + c;
      if (gm >= M) return;
      float* o = out + (int64_t)gm * N + gc;
      if ((N & 3) == 0) {
        if (gc < N) *(float4*)o = make_float4(s * v0, s * v1, s * v2, s * v3);
      } else {
        const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (gc + q < N) o[q] = s * vv[q];
      }
    });
  }
}

// out[e] = s * sum_chunks partial (experts with >= 2 chunks, summed in chunk
// order), zeros for experts without rows; single-chunk experts are already
// final.
__global__ __launch_bounds__(NT) void k_grad_reduce(const Layer L, int kind, int M, int N) {
  __shared__ int pre[MAX_ET + 1];
  __shared__ int sh[4];
  KSched sch;
  sch.init(L, pre, sh);
  float* outbase = kind == GR_DB_DN ? L.db_dn : kind == GR_DA_DN ? L.da_dn
                 : kind == GR_DB_GU ? L.db_gu : L.da_gu;
  const int64_t MN = (int64_t)M * N;
  const int e = blockIdx.y;
  const int nchunk = pre[e + 1] - pre[e];
  if (nchunk == 1) return;
  float* out = outbase + (int64_t)e * MN;
  for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < MN; i += (int64_t)gridDim.x * NT) {
    float acc = 0.0f;
    for (int c = 0; c < nchunk; ++c) acc += L.partial[(int64_t)(pre[e] + c) * MN + i];
    out[i] = L.s * acc;
  }
}

// ---------------------------------------------------------------- launchers

static int grid_for(int max_tiles, int per_cu, int ncu) {
  int g = std::min(max_tiles, per_cu * ncu);
  g = std::max(g, 1);
  return (g + 7) & ~7;
}

static int mtiles_bound(const Layer& L, int BM) { return L.Ptot / BM + L.Et; }

hipError_t gemm_gate_up(const Layer& L, hipStream_t st) {
  const int mt64 = mtiles_bound(L, 128);
  if (L.rs <= 64)
    MOE_LAUNCH("prepass_xa", k_rank_prepass<64>, dim3(grid_for(mt64, 2, L.ncu)), dim3(NT), 0, st, L,
                       (int)PRE_XA);
  else
    MOE_LAUNCH("prepass_xa", k_rank_prepass<128>, dim3(grid_for(mt64, 2, L.ncu)), dim3(NT), 0, st, L,
                       (int)PRE_XA);
  MOE_LAUNCH("gate_up", k_gate_up, dim3(grid_for(mt64 * (L.n / 64), 2, L.ncu)), dim3(NT), 0, st, L);
  return hipGetLastError();
}

hipError_t gemm_down(const Layer& L, hipStream_t st) {
  const int mt = mtiles_bound(L, 128);
  if (L.rs <= 64)
    MOE_LAUNCH("prepass_ha", k_rank_prepass<64>, dim3(grid_for(mt, 2, L.ncu)), dim3(NT), 0, st, L,
                       (int)PRE_HA);
  else
    MOE_LAUNCH("prepass_ha", k_rank_prepass<128>, dim3(grid_for(mt, 2, L.ncu)), dim3(NT), 0, st, L,
                       (int)PRE_HA);
  MOE_LAUNCH("down", k_down, dim3(grid_for(mt * cdiv(L.d, 128), 2, L.ncu)), dim3(NT), 0, st, L);
  return hipGetLastError();
}

hipError_t gemm_dh(const Layer& L, hipStream_t st) {
  const int mt = mtiles_bound(L, 128);
  if (L.rs <= 64)
    MOE_LAUNCH("prepass_qdn", k_rank_prepass<64>, dim3(grid_for(mt, 2, L.ncu)), dim3(NT), 0, st, L,
                       (int)PRE_QDN);
  else
    MOE_LAUNCH("prepass_qdn", k_rank_prepass<128>, dim3(grid_for(mt, 2, L.ncu)), dim3(NT), 0, st, L,
                       (int)PRE_QDN);
  MOE_LAUNCH("dh", k_dh, dim3(grid_for(mt * cdiv(L.n, 128), 2, L.ncu)), dim3(NT), 0, st, L);
  return hipGetLastError();
}

hipError_t gemm_dx(const Layer& L, hipStream_t st) {
  const int mt = mtiles_bound(L, 128);
  if (L.rs <= 64)
    MOE_LAUNCH("prepass_qgu", k_rank_prepass<64>, dim3(grid_for(mt, 2, L.ncu)), dim3(NT), 0, st, L,
                       (int)PRE_QGU);
  else
    MOE_LAUNCH("prepass_qgu", k_rank_prepass<128>, dim3(grid_for(mt, 2, L.ncu)), dim3(NT), 0, st, L,
                       (int)PRE_QGU);
  MOE_LAUNCH("dx", k_dx, dim3(grid_for(mt * cdiv(L.d, 128), 2, L.ncu)), dim3(NT), 0, st, L);
  return hipGetLastError();
}

static const char* const kGradNames[4] = {"grad_db_dn", "grad_da_dn", "grad_db_gu", "grad_da_gu"};
static const char* const kReduceNames[4] = {"reduce_db_dn", "reduce_da_dn", "reduce_db_gu",
                                            "reduce_da_gu"};

template <int BM, int BN, int WM, int WN>
static void launch_grad(const Layer& L, int kind, int M, int N, hipStream_t st) {
  const int slots = L.Ptot / SPLITK_ROWS + L.Et;
  const int tiles = slots * cdiv(M, BM) * cdiv(N, BN);
  MOE_LAUNCH(kGradNames[kind], (k_lora_grad<BM, BN, WM, WN>), dim3(grid_for(tiles, 2, L.ncu)), dim3(NT), 0,
                     st, L, kind, M, N);
  const int64_t MN = (int64_t)M * N;
  const int gx = (int)std::min<int64_t>(cdiv64(MN, NT), 64);
  MOE_LAUNCH(kReduceNames[kind], k_grad_reduce, dim3(gx, L.Et), dim3(NT), 0, st, L, kind, M, N);
}

hipError_t gemm_lora_grads(const Layer& L, hipStream_t st) {
  const int r = L.r, n = L.n, d = L.d;
  if (L.rs <= 64) {
    launch_grad<64, 128, 2, 2>(L, GR_DB_DN, r, d, st);
    launch_grad<128, 64, 4, 1>(L, GR_DA_DN, n, r, st);
    launch_grad<64, 128, 2, 2>(L, GR_DB_GU, r, 2 * n, st);
    launch_grad<128, 64, 4, 1>(L, GR_DA_GU, d, r, st);
  } else {
    launch_grad<128, 128, 2, 2>(L, GR_DB_DN, r, d, st);
    launch_grad<128, 128, 2, 2>(L, GR_DA_DN, n, r, st);
    launch_grad<128, 128, 2, 2>(L, GR_DB_GU, r, 2 * n, st);
    launch_grad<128, 128, 2, 2>(L, GR_DA_GU, d, r, st);
  }
  return hipGetLastError();
}

}  // namespace moe
