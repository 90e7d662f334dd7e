// LoRA-factor gradients of the expert layer ("Faster LoRA MoE training":
// only the adapters A, B train, the base W stays frozen):
//   dB_dn[e] = (w s H A_dn)^T dY[tok]      [r, d]
//   dA_dn[e] = H^T (w Q_dn)                [n, r]
//   dB_gu[e] = (s X A_gu)^T dG             [r, 2n]
//   dA_gu[e] = X[tok]^T Q_gu               [d, r]
// Each is a product over the rows of the expert's segment: C = U^T V with U
// [rows, M] and V [rows, N] both row-major, so the contraction index is the
// row index of both operands.
//
// Both operands move global -> LDS with buffer_load_dwordx4 ... lds as
// k-major panels (32 segment rows x the tile's columns, whole 16-byte row
// chunks, the chunk XOR-swizzled by row), through a three-stage ring, and
// the MFMA operands come out of LDS with ds_read_b64_tr_b16 (each lane gets 4
// consecutive rows of one column).  Token-gathered operands (dY, X) take their
// row offsets from the segment chunk's gather indices, staged in LDS at tile
// start.  Tiles are 64 (the rank side) x 256, 4 waves of 64 x 64, and the
// four kinds share one persistent launch; segments longer than L.splitk
// are split into chunks whose fp32 partials k_grad_reduce sums in chunk
// order.
#include <algorithm>

#include "common.h"
#include "gemm_util.h"
#include "kernels.h"

namespace moe {
inline namespace MOE_EL {
namespace {

constexpr int GK = 32;               // segment rows per ring stage
constexpr int GNS = 3, GPD = 2;      // ring stages, issue distance
constexpr int GNW = 4, GNT = 64 * GNW;
constexpr int GLONG = 256, GRANK = 64;

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

enum GKind { G_DB_DN = 0, G_DA_DN = 1, G_DB_GU = 2, G_DA_GU = 3 };

template <int KIND>
struct GP {
  static constexpr bool DB = KIND == G_DB_DN || KIND == G_DB_GU;  // M = rank side
  static constexpr int BM = DB ? GRANK : GLONG, BN = DB ? GLONG : GRANK;
  static constexpr int WM = DB ? 1 : 4, WN = DB ? 4 : 1;          // wave grid
  static constexpr bool U_GATHER = KIND == G_DA_GU;               // X[tok]
  static constexpr bool V_GATHER = KIND == G_DB_DN;               // dY[tok]
  static constexpr int NIU = GK * BM * 2 / 1024 / GNW, NIV = GK * BN * 2 / 1024 / GNW;
  static constexpr int PER = NIU + NIV;
  static constexpr int STAGE = GK * (BM + BN);  // bf16 elements
};

// chunk swizzle of a k-major panel row of C columns (C / 8 chunks): the
// 16-lane groups of a transposing read hit distinct 16-byte bank groups
template <int C>
__device__ __forceinline__ int g_sw(int k) {
  static_assert(C == 256 || C == 64, "panel width");
  return C == 256 ? (k & 3) * 4 : ((k >> 1) & 1) * 4;
}

// One operand panel: GK rows x C columns starting at column c0 of a
// row-major [rows, ld] source.  Instruction j of wave w covers rows
// RPI (w + 4 j) .. + RPI, lane i row RPI (w + 4 j) + i / CPR, physical chunk
// i % CPR holding logical chunk (i % CPR) ^ sw(row).
template <int C, bool GATHER>
struct GPanel {
  static constexpr int CPR = C / 8, RPI = 64 / CPR, NI = GK * C * 2 / 1024 / GNW;
  int4v desc;
  uint32_t colb;   // byte offset of this lane's chunk within a source row
  uint32_t ldb;    // source row stride, bytes
  int rows;        // valid rows of the chunk
  bool colok;

  __device__ GPanel(const bf16_t* base, int64_t bytes, int ld, int c0, int ncols, int rows_) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    desc = make_desc(base, bytes);
    ldb = (uint32_t)ld * 2u;
    rows = rows_;
    // the logical chunk is the same for every instruction of this lane:
    // RPI (w + 4 j) keeps row & 3 (C = 256) and (row >> 1) & 1 (C = 64)
    const int row0 = RPI * wid + lane / CPR;
    const int lc = (lane % CPR) ^ g_sw<C>(row0);
    colok = c0 + lc * 8 < ncols;
    colb = (uint32_t)(c0 + lc * 8) * 2u;
  }
  // rows k0 .. k0 + GK of the chunk into the panel at LDS byte address sb;
  // tok = the chunk's gather indices (GATHER) in LDS
  __device__ __forceinline__ void issue(int k0, uint32_t sb, const int* tok) const {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int row = RPI * (wid + j * GNW) + lane / CPR;
      const int k = k0 + row;
      uint32_t o = OOB;
      if (colok && k < rows) o = GATHER ? (uint32_t)tok[k] * ldb + colb : (uint32_t)row * ldb + colb;
      dma16(desc, o, GATHER ? 0u : (uint32_t)k0 * ldb,
            __builtin_amdgcn_readfirstlane(sb + (wid + j * GNW) * 1024));
    }
  }
};

// The MFMA operand of 32 columns (cb .. cb + 32) for k = kk*16 .. + 16 from
// a k-major panel of C columns: lane L holds column cb + L % 32 and rows
// 8 (L / 32) + 0..7.
template <int C>
__device__ __forceinline__ uint4 g_frag(const char* panel, int kk, int cb) {
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4, q = (lane >> 2) & 3, rr = lane & 3;
  const int krow = kk * 16 + 8 * (g >> 1) + q;
  const int col = cb + 16 * (g & 1) + 4 * rr;
  const char* p = panel + krow * (C * 2) + (((col >> 3) ^ g_sw<C>(krow)) * 16) + (col & 7) * 2;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)p);
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p + 4 * C * 2));
  return make_uint4((uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16),
                    (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16),
                    (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16),
                    (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16));
}

// Shape of a kind's tile list: tiles per segment chunk (M tiles x N tiles).
template <int KIND>
__device__ __forceinline__ int grad_per_slot(const Layer& L) {
  using P = GP<KIND>;
  int M, N;
  grad_shape(KIND, L.d, L.n, L.r, M, N);
  return cdiv(M, P::BM) * cdiv(N, P::BN);
}

// Tile t of kind KIND: C tile of dB / dA over one segment chunk, through the
// workgroup's ring and gather-index buffer.
template <int KIND>
__device__ __forceinline__ void grad_tile(const Layer& L, int t, bf16_t* ring, int* tokbuf,
                                          const int* pre) {
  using P = GP<KIND>;
  const int n = L.n, d = L.d, rs = L.rs;
  int M, N;
  grad_shape(KIND, d, n, L.r, M, N);
  const int nmt = cdiv(M, P::BM), nnt = cdiv(N, P::BN);
  const int per_slot = nmt * nnt;
  (void)nnt;
  float* outbase = KIND == G_DB_DN ? L.db_dn : KIND == G_DA_DN ? L.da_dn : KIND == G_DB_GU ? L.db_gu : L.da_gu;
  float* partial = L.partial + L.partial_off[KIND];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int wm = wid / P::WN, wn = wid % P::WN;
  const uint32_t ring_b = (uint32_t)(uintptr_t)ring;
  const int slot = t / per_slot;
  const int rem = t - slot * per_slot;
  const int nt = rem / nmt, mt = rem - nt * nmt;
  // tile scalars are wave-uniform: keep them in scalar registers (the DMA
  // descriptors built from them must be)
  const int e = __builtin_amdgcn_readfirstlane(find_expert(pre, L.Et, slot, 1));
  const int chunk = __builtin_amdgcn_readfirstlane(slot - pre[e]);
  const int nchunk = __builtin_amdgcn_readfirstlane(pre[e + 1] - pre[e]);
  const int kb = __builtin_amdgcn_readfirstlane(seg_start(L, e) + chunk * L.splitk);
  const int kn = __builtin_amdgcn_readfirstlane(min(seg_count(L, e) - chunk * L.splitk, L.splitk));
  const int m0 = mt * P::BM, c0 = nt * P::BN;
  if (P::U_GATHER || P::V_GATHER) {
    for (int i = threadIdx.x; i < kn; i += GNT) tokbuf[i] = L.tok[kb + i];
    __syncthreads();
  }
  // U: [rows, M] source, V: [rows, N] source, both from row kb on
  const bf16_t* ub;
  int64_t ubytes;
  int uld;
  if constexpr (KIND == G_DB_DN) { ub = L.hw + (int64_t)kb * rs; ubytes = (int64_t)kn * rs * 2; uld = rs; }
  else if constexpr (KIND == G_DA_DN) { ub = L.h + (int64_t)kb * n; ubytes = (int64_t)kn * n * 2; uld = n; }
  else if constexpr (KIND == G_DB_GU) { ub = L.xa + (int64_t)kb * rs; ubytes = (int64_t)kn * rs * 2; uld = rs; }
  else { ub = L.x; ubytes = (int64_t)L.T * d * 2; uld = d; }
  const bf16_t* vb;
  int64_t vbytes;
  int vld;
  if constexpr (KIND == G_DB_DN) { vb = L.dy; vbytes = (int64_t)L.T * d * 2; vld = d; }
  else if constexpr (KIND == G_DA_DN) { vb = L.qw + (int64_t)kb * rs; vbytes = (int64_t)kn * rs * 2; vld = rs; }
  else if constexpr (KIND == G_DB_GU) { vb = L.dg + (int64_t)kb * 2 * n; vbytes = (int64_t)kn * 2 * n * 2; vld = 2 * n; }
  else { vb = L.qgu + (int64_t)kb * rs; vbytes = (int64_t)kn * rs * 2; vld = rs; }
  const GPanel<P::BM, P::U_GATHER> U(ub, ubytes, uld, m0, M, kn);
  const GPanel<P::BN, P::V_GATHER> V(vb, vbytes, vld, c0, N, kn);
  const int nk = cdiv(kn, GK);
  auto issue = [&](int s) {
    const int sc = min(s, max(nk - 1, 0));
    const uint32_t sb = ring_b + (uint32_t)(s % GNS) * P::STAGE * 2;
    U.issue(sc * GK, sb, tokbuf);
    V.issue(sc * GK, sb + GK * P::BM * 2, tokbuf);
  };
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16)(0.0f);
#pragma unroll
  for (int s = 0; s < GPD; ++s) issue(s);
  for (int s = 0; s < nk; ++s) {
    wait_vmcnt<(GPD - 1) * P::PER>();
    __syncthreads();
    issue(s + GPD);
    const char* st = (const char*)(ring + (s % GNS) * P::STAGE);
#pragma unroll
    for (int kk = 0; kk < GK / 16; ++kk) {
      uint4 a[2], b[2];
#pragma unroll
      for (int f = 0; f < 2; ++f) a[f] = g_frag<P::BM>(st, kk, wm * 64 + f * 32);
#pragma unroll
      for (int f = 0; f < 2; ++f) b[f] = g_frag<P::BN>(st + GK * P::BM * 2, kk, wn * 64 + f * 32);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(b[j], a[i], acc[i][j]);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();  // ring and gather indices free for the next tile
  const bool direct = nchunk == 1;
  float* out = direct ? outbase + (int64_t)e * M * N : partial + (int64_t)slot * M * N;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gm = m0 + wm * 64 + i * 32 + (lane & 31);
        const int gc = c0 + wn * 64 + j * 32 + g * 8 + (lane >> 5) * 4;
        if (gm >= M) continue;
        float* o = out + (int64_t)gm * N + gc;
        const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1], v2 = acc[i][j][4 * g + 2],
                    v3 = acc[i][j][4 * g + 3];
        if ((N & 3) == 0) {
          if (gc < N) *(float4*)o = make_float4(v0, v1, v2, v3);
        } else {
          const float vv[4] = {v0, v1, v2, v3};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (gc + q < N) o[q] = vv[q];
        }
      }
}

constexpr int GSTAGE = GP<0>::STAGE;
static_assert(GP<1>::STAGE == GSTAGE && GP<2>::STAGE == GSTAGE && GP<3>::STAGE == GSTAGE,
              "one ring for every kind");

// All four kinds in one persistent launch (from K0 on): their tile lists one
// after the other, so no kind's last partial round of tiles leaves CUs idle.
template <int K0>
__global__ __launch_bounds__(GNT) __attribute__((amdgpu_waves_per_eu(2))) void k_grad_all(const Layer L) {
  __shared__ __attribute__((aligned(1024))) bf16_t ring[GNS * GSTAGE];
  __shared__ __attribute__((aligned(16))) int tokbuf[SPLITK_MAX];
  __shared__ int pre[MAX_ET + 1];
  __shared__ int sh[GNW];
  expert_prefix<GNT>(L, pre, sh, [&](int e) { return cdiv(seg_count(L, e), L.splitk); });
  const int slots = pre[L.Et];
  const int c1 = K0 <= 0 ? slots * grad_per_slot<0>(L) : 0;
  const int c2 = c1 + (K0 <= 1 ? slots * grad_per_slot<1>(L) : 0);
  const int c3 = c2 + slots * grad_per_slot<2>(L);
  const int total = c3 + slots * grad_per_slot<3>(L);
  for (int t = first_tile(); t < total; t += gridDim.x) {
    if (t < c1) grad_tile<0>(L, t, ring, tokbuf, pre);
    else if (t < c2) grad_tile<1>(L, t - c1, ring, tokbuf, pre);
    else if (t < c3) grad_tile<2>(L, t - c2, ring, tokbuf, pre);
    else grad_tile<3>(L, t - c3, ring, tokbuf, pre);
  }
}

// dst[p, :] = w[p] * src[p, :] over [Ptot, rs] (the weighted rank-r rows).
__global__ __launch_bounds__(256) void k_weight_rows(const Layer L, const bf16_t* __restrict__ src,
                                                     bf16_t* __restrict__ dst) {
  const int rs8 = L.rs / 8;
  const int64_t total = (int64_t)L.Ptot * rs8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t p = i / rs8;
    const float w = L.wgt[p];
    const uint4 v = *(const uint4*)(src + i * 8);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack2(w * bf2f((bf16_t)(u[q] & 0xffffu)), w * bf2f((bf16_t)(u[q] >> 16)));
    *(uint4*)(dst + i * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

hipError_t dma_lora_grads(const Layer& L, hipStream_t st) {
  if (!prepass_writes_weighted_rows(L)) {
    const int g = std::min<int64_t>(cdiv64((int64_t)L.Ptot * L.rs / 8, 256), 2048);
    MOE_LAUNCH("weight_rows", k_weight_rows, dim3(g), dim3(256), 0, st, L, L.ha, L.hw);
    MOE_LAUNCH("weight_rows", k_weight_rows, dim3(g), dim3(256), 0, st, L, L.qdn, L.qw);
  }
  // upper bound of the merged tile list (slots per expert <= rows / chunk + 1)
  const int64_t slots = L.Ptot / L.splitk + L.Et;
  int64_t tiles = 0;
  for (int kind = 0; kind < 4; ++kind) {
    int M, N;
    grad_shape(kind, L.d, L.n, L.r, M, N);
    const bool db = kind == G_DB_DN || kind == G_DB_GU;
    tiles += slots * cdiv(M, db ? GRANK : GLONG) * cdiv(N, db ? GLONG : GRANK);
  }
  int g = (int)std::min<int64_t>(tiles, 2 * L.ncu);
  g = std::max((g + 7) & ~7, 8);
  MOE_LAUNCH("lora_grads", k_grad_all<0>, dim3(g), dim3(GNT), 0, st, L);
  return hipGetLastError();
}

}  // inline namespace MOE_EL
}  // namespace moe
