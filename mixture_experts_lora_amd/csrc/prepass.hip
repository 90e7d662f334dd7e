// Rank-r pre-passes of the split LoRA term ("Faster LoRA MoE training": the
// low-rank path is (X A) B, never B A^T merged into W):
//   X A_gu     out[p] = s X[tok p] A_gu[e]      (contraction d)
//   H A_dn     out[p] = s H[p] A_dn[e]          (contraction n)
//   Q_dn       out[p] = s dY[tok p] B_dn[e]^T   (contraction d), and with it
//              w Q_dn and w (s H A_dn), the weighted rows the down module's
//              LoRA gradients contract with (w = routing weight of row p)
//   Q_gu       out[p] = s dG[p] B_gu[e]^T       (contraction 2n)
// for the expert e owning sorted row p; columns [r, rs) come out zero.
//
// These products have only r <= 64 columns, so they are streams: every
// activation row is read once and the MFMA work is small beside it.  One
// workgroup takes a block of at most 160 rows of one expert (an expert's
// rows are cut into near-equal blocks), five waves of one 32-row fragment
// row and all 64 columns each, and runs the whole contraction through a ring
// of four LDS stages of 64 k, filled by buffer_load_dwordx4 ... lds: each
// row's 64 k are one 128-byte line.  Activation panels are row-contiguous
// [160 rows][64 k] with the 16-byte chunk c of row m at c ^ (m & 7); the
// factor panel is k-major [64 k][64 columns] (A_gu, A_dn: read with
// ds_read_b64_tr_b16) or row-contiguous like the activations (B_dn, B_gu).
#include <algorithm>

#include "common.h"
#include "gemm_util.h"
#include "kernels.h"

namespace moe {
inline namespace MOE_EL {
namespace {

constexpr int QB = 160;                    // rows of a block at most
constexpr int QW = QB / 32, QNT = 64 * QW;  // five waves, one fragment row each
constexpr int QK = 64;                     // k per ring stage
constexpr int QNS = 4;                     // ring stages
constexpr int QA = QB * QK;                // bf16 elements of the activation panel
constexpr int QF = 64 * QK;                // bf16 elements of the factor panel
constexpr int QSTAGE = QA + QF;
constexpr int QNA = QA * 2 / 1024 / QW;    // activation DMA instructions per wave and stage
constexpr int QNF = QF * 2 / 1024 / 4;     // factor instructions of waves 0..3
static_assert(QNA * QW * 1024 == QA * 2 && QNF * 4 * 1024 == QF * 2, "panel split");

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef unsigned v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float s_lo(uint32_t w) { return bf2f((bf16_t)(w & 0xffffu)); }
__device__ __forceinline__ float s_hi(uint32_t w) { return bf2f((bf16_t)(w >> 16)); }

template <int KIND>
struct QP {
  static constexpr bool GATHER = KIND == PRE_XA || KIND == PRE_QDN;  // X[tok], dY[tok]
  static constexpr bool F_KMAJOR = KIND == PRE_XA || KIND == PRE_HA;  // factor [K, ra]
};

// 16 k of one row of a row-contiguous panel (128-byte rows, swizzled)
__device__ __forceinline__ uint4 q_row_frag(const char* panel, int row, int kk) {
  const int lane = threadIdx.x & 63;
  const int c = (2 * kk + (lane >> 5)) ^ (row & 7);
  return *(const uint4*)(panel + row * (QK * 2) + c * 16);
}

// 16 k of column cb + lane % 32 of the k-major factor panel: 16-lane group g
// reads k rows 8 (g >> 1) + q (+4) at columns 16 (g & 1) + 4 rr; the
// transposing read gives lane (g, j) the 4 k values of column 16 (g & 1) + j.
// Chunk c of k row kr sits at c ^ 4 ((kr >> 1) & 1).
__device__ __forceinline__ uint4 q_col_frag(const char* panel, int kk, int cb) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, q = (lane >> 2) & 3, rr = lane & 3;
  const int krow = kk * 16 + 8 * (g >> 1) + q;
  const int col = cb + 16 * (g & 1) + 4 * rr;
  const char* p = panel + krow * 128 + (((col >> 3) ^ (((krow >> 1) & 1) * 4)) * 16) + (col & 7) * 2;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * 128));
  return make_uint4((uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                    (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                    (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                    (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16));
}

template <int KIND>
__global__ __launch_bounds__(QNT) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_rank_stream(const Layer L) {
  using P = QP<KIND>;
  __shared__ __attribute__((aligned(1024))) bf16_t ring[QNS * QSTAGE];
  __shared__ int tokb[QB];
  __shared__ int pre[MAX_ET + 1];
  __shared__ int sh[QW];
  expert_prefix<QNT>(L, pre, sh, [&](int e) { return cdiv(seg_count(L, e), QB); });
  const int total = pre[L.Et];
  const int n = L.n, d = L.d, r = L.r, rs = L.rs, ra = L.ra;
  const int K = KIND == PRE_XA || KIND == PRE_QDN ? d : KIND == PRE_HA ? n : 2 * n;
  const int nk = K / QK;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t ring_b = (uint32_t)(uintptr_t)ring;
  // row-contiguous panels: instruction j of a wave covers 8 rows, lane i row
  // 8 (...) + i / 8, physical chunk i % 8 holding logical chunk lc
  const int lc = (lane & 7) ^ (lane >> 3);
  // k-major factor panel: k row 8 (...) + i / 8, physical chunk i % 8
  // holding logical chunk lf
  const int lf = (lane & 7) ^ (((lane >> 4) & 1) * 4);
  bf16_t* out = KIND == PRE_XA ? L.xa : KIND == PRE_HA ? L.ha : KIND == PRE_QDN ? L.qdn : L.qgu;
  const rsrc_t ro = make_rsrc(out, (int64_t)L.Ptot * rs * 2);
  const rsrc_t rqw = make_rsrc(L.qw, (int64_t)L.Ptot * rs * 2);
  const rsrc_t rhw = make_rsrc(L.hw, (int64_t)L.Ptot * rs * 2);
  const rsrc_t rha = make_rsrc(L.ha, (int64_t)L.Ptot * rs * 2);
  const float sc = L.s;

#pragma unroll 1
  for (int t = blockIdx.x; t < total; t += gridDim.x) {
    const int e = __builtin_amdgcn_readfirstlane(find_expert(pre, L.Et, t, 1));
    const int cnt = seg_count(L, e);
    const int nb = pre[e + 1] - pre[e], b = t - pre[e];
    const int hb = cdiv(cnt, nb);
    const int row0 = __builtin_amdgcn_readfirstlane(seg_start(L, e) + b * hb);
    const int h = __builtin_amdgcn_readfirstlane(min(hb, cnt - b * hb));
    if (h <= 0) continue;  // the earlier blocks already cover the expert's rows
    if (P::GATHER) {
      for (int m = threadIdx.x; m < QB; m += QNT) tokb[m] = m < h ? L.tok[row0 + m] : 0;
      __syncthreads();
    }
    // activation panel operands
    int4v da;
    uint32_t va[QNA];
    if constexpr (P::GATHER) {
      da = make_desc(KIND == PRE_XA ? L.x : L.dy, (int64_t)L.T * d * 2);
#pragma unroll
      for (int j = 0; j < QNA; ++j) {
        const int m = 8 * (wid + QW * j) + (lane >> 3);
        va[j] = m < h ? (uint32_t)tokb[m] * (uint32_t)(d * 2) + lc * 16 : OOB;
      }
    } else {
      const int ld = KIND == PRE_HA ? n : 2 * n;
      da = make_desc((KIND == PRE_HA ? L.h : L.dg) + (int64_t)row0 * ld, (int64_t)h * ld * 2);
#pragma unroll
      for (int j = 0; j < QNA; ++j) {
        const int m = 8 * (wid + QW * j) + (lane >> 3);
        va[j] = m < h ? (uint32_t)m * (uint32_t)(ld * 2) + lc * 16 : OOB;
      }
    }
    // factor panel operands (waves 0..3)
    int4v df;
    uint32_t vf[QNF];
    uint32_t fstep;  // source bytes per ring stage
    if constexpr (P::F_KMAJOR) {
      df = make_desc((KIND == PRE_XA ? L.a_gu : L.a_dn) + (int64_t)e * K * ra, (int64_t)K * ra * 2);
      fstep = (uint32_t)QK * (uint32_t)(ra * 2);
#pragma unroll
      for (int j = 0; j < QNF; ++j) {
        const int kr = 8 * (wid + 4 * j) + (lane >> 3);
        vf[j] = lf * 8 < ra ? (uint32_t)kr * (uint32_t)(ra * 2) + lf * 16 : OOB;
      }
    } else {
      df = make_desc((KIND == PRE_QDN ? L.b_dn : L.b_gu) + (int64_t)e * r * K, (int64_t)r * K * 2);
      fstep = QK * 2;
#pragma unroll
      for (int j = 0; j < QNF; ++j) {
        const int c = 8 * (wid + 4 * j) + (lane >> 3);
        vf[j] = c < r ? (uint32_t)c * (uint32_t)(K * 2) + lc * 16 : OOB;
      }
    }
    // stage s (the last one again past the end, so every wave issues the
    // same number of instructions per step) into slot s % QNS
    auto issue = [&](int s) {
      const int ks = s < nk ? s : nk - 1;
      const uint32_t sb = ring_b + (uint32_t)(s % QNS) * QSTAGE * 2;
      const uint32_t soa = (uint32_t)ks * QK * 2;
#pragma unroll
      for (int j = 0; j < QNA; ++j) dma16(da, va[j], soa, sb + (uint32_t)(wid + QW * j) * 1024u);
      if (wid < 4) {
#pragma unroll
        for (int j = 0; j < QNF; ++j)
          dma16(df, vf[j], (uint32_t)ks * fstep, sb + QA * 2 + (uint32_t)(wid + 4 * j) * 1024u);
      }
    };
    f32x16 acc0 = (f32x16)(0.0f), acc1 = (f32x16)(0.0f);
#pragma unroll 1
    for (int s = 0; s < QNS - 1; ++s) issue(s);
#pragma unroll 1
    for (int k = 0; k < nk; ++k) {
      // stage k in: younger are stages k + 1 .. k + QNS - 2
      if (wid < 4) wait_vmcnt<(QNS - 2) * (QNA + QNF)>();
      else wait_vmcnt<(QNS - 2) * QNA>();
      __syncthreads();
      issue(k + QNS - 1);  // into the slot of stage k - 1, which every wave is done with
      const char* st = (const char*)(ring + (k % QNS) * QSTAGE);
      const char* fp = st + QA * 2;
      const int row = 32 * wid + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < QK / 16; ++kk) {
        const uint4 a = q_row_frag(st, row, kk);
        uint4 b0, b1;
        if constexpr (P::F_KMAJOR) {
          b0 = q_col_frag(fp, kk, 0);
          b1 = q_col_frag(fp, kk, 32);
        } else {
          b0 = q_row_frag(fp, lane & 31, kk);
          b1 = q_row_frag(fp, 32 + (lane & 31), kk);
        }
        acc0 = mfma32(b0, a, acc0);
        acc1 = mfma32(b1, a, acc1);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with the ring before the next block refills it
    // lane: row 32 wid + lane % 32, columns 32 f + 8 g + 4 (lane / 32) + 0..3
    const int m = 32 * wid + (lane & 31);
    const int64_t p = row0 + m;
    // Q_dn also leaves the weighted rank-r rows of the down module's LoRA
    // gradients: w Q_dn and w (s H A_dn), each rounded from the bf16 row
    float wr = 0.0f;
    if constexpr (KIND == PRE_QDN) wr = m < h ? L.wgt[p] : 0.0f;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const f32x16& v = f ? acc1 : acc0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = 32 * f + 8 * g + 4 * (lane >> 5);
        const uint32_t o = m < h && c < rs ? (uint32_t)((p * rs + c) * 2) : OOB;
        const v2u w = {pack2(sc * v[4 * g], sc * v[4 * g + 1]), pack2(sc * v[4 * g + 2], sc * v[4 * g + 3])};
        __builtin_amdgcn_raw_buffer_store_b64(w, ro, o, 0, 0);
        if constexpr (KIND == PRE_QDN) {
          const v2u qw = {pack2(wr * s_lo(w[0]), wr * s_hi(w[0])), pack2(wr * s_lo(w[1]), wr * s_hi(w[1]))};
          __builtin_amdgcn_raw_buffer_store_b64(qw, rqw, o, 0, 0);
          const v2u ha = __builtin_amdgcn_raw_buffer_load_b64(rha, o, 0, 0);
          const v2u hw = {pack2(wr * s_lo(ha[0]), wr * s_hi(ha[0])), pack2(wr * s_lo(ha[1]), wr * s_hi(ha[1]))};
          __builtin_amdgcn_raw_buffer_store_b64(hw, rhw, o, 0, 0);
        }
      }
    }
  }
}

}  // namespace

template <int KIND>
static hipError_t launch_rank_stream(const Layer& L, hipStream_t st, const char* name) {
  // blocks: sum over experts of ceil(rows / 160) <= P_tot / 160 + E_tot
  const int64_t blocks = (int64_t)L.Ptot / QB + L.Et;
  const int g = (int)std::min<int64_t>(blocks, L.ncu);
  MOE_LAUNCH(name, k_rank_stream<KIND>, dim3(std::max(g, 1)), dim3(QNT), 0, st, L);
  return hipGetLastError();
}

hipError_t stream_prepass(const Layer& L, int kind, hipStream_t st) {
  switch (kind) {
    case PRE_XA: return launch_rank_stream<PRE_XA>(L, st, "prepass_xa");
    case PRE_HA: return launch_rank_stream<PRE_HA>(L, st, "prepass_ha");
    case PRE_QDN: return launch_rank_stream<PRE_QDN>(L, st, "prepass_qdn");
    default: return launch_rank_stream<PRE_QGU>(L, st, "prepass_qgu");
  }
}

}  // inline namespace MOE_EL
}  // namespace moe
