// Device helpers shared by the grouped-GEMM kernels: buffer resources and
// range-checked loads, LDS-DMA, the per-expert tile schedule.
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {
inline namespace MOE_EL {

constexpr int MAX_ET = 512;  // experts (routed + shared) a schedule prefix can hold

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t OOB = 0x80000000u;  // offset past every buffer: reads as zero

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t cap = 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < cap ? bytes : cap), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ int seg_start(const Layer& L, int e) {
  return e < L.E ? L.offsets[e] : L.P;
}
__device__ __forceinline__ int seg_count(const Layer& L, int e) {
  return e < L.E ? L.offsets[e + 1] - L.offsets[e] : L.T;
}

// Buffer descriptor as four scalar registers (base, 16-bit stride 0,
// num_records, the gfx9 raw-buffer word).
typedef int int4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int4v make_desc(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const int64_t cap = 0x7fffffff;
  int4v d;
  d.x = (int)(uint32_t)(a & 0xffffffffu);
  d.y = (int)(uint32_t)((a >> 32) & 0xffffu);
  d.z = (int)(bytes < cap ? bytes : cap);
  d.w = 0x00020000;
  return d;
}

// One buffer_load_dwordx4 ... lds: every lane's 16 bytes land in LDS at
// lds_addr + 16 * lane (out-of-range lanes write zeros).  Issued from inline
// asm so the compiler does not serialise LDS reads behind it; completion is
// tracked with explicit vmcnt waits by the pipeline.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(int4v desc, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  // the scalar operands are wave-uniform by contract; readfirstlane keeps the
  // compiler from handing a VGPR copy of one to an "s" constraint
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(desc),
                 "s"(__builtin_amdgcn_readfirstlane(soff))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// vmcnt wait with the other counters left alone (gfx9 s_waitcnt encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// XOR swizzle of the 16-byte chunk position inside an LDS row of DBK bf16:
// the 16 rows one ds_read_b128 quarter-wave touches (same chunk) land on 16
// distinct 16-byte bank groups of the 256-byte bank window.
template <int DBK>
__device__ __forceinline__ int sw_chunk(int row, int c) {
  constexpr int CPR = DBK / 8, RP = 256 / (DBK * 2);  // chunks per row, rows per window
  return c ^ ((row / RP) & (CPR - 1));
}

__device__ __forceinline__ void store_bf16x4(bf16_t* p, float a, float b, float c, float d) {
  *(uint2*)p = make_uint2(pack2(a, b), pack2(c, d));
}

// Persistent loop order: round-robin XCD dealing -> contiguous logical tiles
// per XCD inside a round.
__device__ __forceinline__ int first_tile() {
  const int G = gridDim.x;
  return (G & 7) ? (int)blockIdx.x : (int)((blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3));
}

// Exclusive scan of one int per thread over a block of NW waves (all threads
// must call); `sh` holds NW ints.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[wid] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = sh[w];
    if (w < wid) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

// Per-expert counts of a schedule unit (M tiles, or split-K chunks) and their
// exclusive prefix over experts, in LDS.  Each thread takes EP consecutive
// experts.
template <int NT, class CountFn>
__device__ __forceinline__ void expert_prefix(const Layer& L, int* pre, int* sh, CountFn cnt) {
  constexpr int EP = (MAX_ET + NT - 1) / NT;
  const int Et = L.Et;
  int c[EP], sum = 0;
#pragma unroll
  for (int i = 0; i < EP; ++i) {
    const int e = EP * threadIdx.x + i;
    c[i] = e < Et ? cnt(e) : 0;
    sum += c[i];
  }
  int tot;
  int ex = block_excl_scan<NT / 64>(sum, sh, &tot);
#pragma unroll
  for (int i = 0; i < EP; ++i) {
    const int e = EP * threadIdx.x + i;
    if (e < Et) pre[e] = ex;
    ex += c[i];
  }
  if (threadIdx.x == 0) pre[Et] = tot;
  __syncthreads();
}

// largest e in [0, Et) with pre[e] * mul <= t
__device__ __forceinline__ int find_expert(const int* pre, int Et, int t, int mul) {
  int lo = 0, hi = Et - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] * mul <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Row-ragged tile (e, nt, mt), mt fastest.
struct MTile {
  int e, mt, nt, row0, mrows;
};
template <int BM>
__device__ __forceinline__ MTile decode_m(const Layer& L, const int* pre, int t, int ntn) {
  MTile T;
  T.e = find_expert(pre, L.Et, t, ntn);
  const int local = t - pre[T.e] * ntn;
  const int nm = pre[T.e + 1] - pre[T.e];
  T.nt = local / nm;
  T.mt = local - T.nt * nm;
  T.row0 = seg_start(L, T.e) + T.mt * BM;
  T.mrows = min(BM, seg_count(L, T.e) - T.mt * BM);
  return T;
}

// gate/up column interleave of the gate_up tile: 32-column groups alternate
// gate (rows j of W_gu) and up (rows n + j), so one lane holds gate and up of
// the same (row, j) in two neighbouring N fragments.
__device__ __forceinline__ int gu_row(int n, int j0, int c) {
  const int grp = c >> 5;
  return ((grp & 1) ? n : 0) + j0 + (grp >> 1) * 32 + (c & 31);
}

}  // inline namespace MOE_EL
}  // namespace moe
