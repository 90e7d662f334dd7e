// Routing: top-k softmax and the one-pass grouping of (token, slot) pairs by
// expert (article on Unsloth x NVIDIA training optimisations, section
// "Optimisation 3: MoE routing grouped once": flatten, stable sort by expert
// id, one bincount, offsets from counts, slice by offset, gather).
//
// Two kernels, no host round trip:
//   1. route_select  at most 256 workgroups, each a contiguous block of
//      tokens taken 16 at a time; a token is one 16-lane DPP row.  Its
//      logits become 64-bit keys (order-preserving bits of the value, then
//      the complement of the expert id), so "largest logit, ties to the
//      lower id" is one unsigned maximum; pick j is the row maximum of the
//      keys below pick j-1, reduced over the row with DPP rotations.  Softmax
//      over the picks.  An LDS-private per-expert token bitmask (16 bits per
//      round of 16 tokens) gives, by popcount, every pair's rank among the
//      block's earlier pairs of its expert (a token never picks an expert
//      twice, so that rank is the number of earlier tokens that picked it:
//      the sort stays stable without atomics deciding any order) and the
//      block's histogram row.
//   2. route_scatter  at most 64 workgroups of 1024 threads.  Each sums the
//      histogram columns (the bincount: totals, and the part below its own
//      range of blocks), scans the totals into the exclusive offsets, then
//      places every pair of its range: dest = offsets[e] + (pairs of e in
//      earlier blocks) + rank.  It writes sorted_pair, its inverse pair_pos,
//      and the gather table of the sorted rows (token and routing weight of
//      each row; the shared expert's rows P + t are token t with weight 1).
#include "common.h"
#include "gemm_util.h"
#include "kernels.h"

namespace moe {

constexpr int RS_TOK = 16;              // tokens per round of route_select (one 16-lane row each)
constexpr int RS_THREADS = RS_TOK * 16;
constexpr int RS_MAXBLK = 256;          // route_select workgroups at most
constexpr int SC_THREADS = 1024;        // route_scatter workgroup
constexpr int SC_MAXBLK = 64;           // route_scatter workgroups at most
constexpr int SC_BPB = RS_MAXBLK / SC_MAXBLK;  // histogram rows per route_scatter workgroup at most

struct RouteGeom {
  int spb;    // rounds of 16 tokens per route_select workgroup
  int nblk;   // route_select workgroups (histogram rows)
  int bpb2;   // histogram rows per route_scatter workgroup
  int nblk2;  // route_scatter workgroups
};

static RouteGeom route_geom(int64_t T) {
  RouteGeom g;
  const int nsub = (int)cdiv64(T, RS_TOK);
  const int nb = nsub < RS_MAXBLK ? nsub : RS_MAXBLK;
  g.spb = cdiv(nsub, nb);
  g.nblk = cdiv(nsub, g.spb);
  g.bpb2 = cdiv(g.nblk, SC_MAXBLK);
  g.nblk2 = cdiv(g.nblk, g.bpb2);
  return g;
}

// Order-preserving unsigned image of a logit: larger value -> larger image,
// -0 and +0 equal, NaN below every other value (-inf included).
__device__ __forceinline__ uint32_t rt_ord(float v) {
  uint32_t u = __float_as_uint(v);
  if (v != v) return 0u;
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// inverse of rt_ord (the NaN image 0 maps back to a NaN)
__device__ __forceinline__ float rt_val(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// DPP row_ror:N (rotate within each 16-lane row) of a 32-bit value
template <int N>
__device__ __forceinline__ uint32_t ror_row(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x120 | N, 0xf, 0xf, false);
}
template <int N>
__device__ __forceinline__ uint64_t ror_row64(uint64_t x) {
  return ((uint64_t)ror_row<N>((uint32_t)(x >> 32)) << 32) | ror_row<N>((uint32_t)x);
}
// maximum / sum over the 16 lanes of a row; every lane of the row gets the
// same result (rotations by 8, 4, 2, 1 pair each lane with lanes whose
// partial results equal its own, so even the float sum is bitwise the same)
__device__ __forceinline__ uint64_t row_max64(uint64_t x) {
  uint64_t y;
  y = ror_row64<8>(x); x = y > x ? y : x;
  y = ror_row64<4>(x); x = y > x ? y : x;
  y = ror_row64<2>(x); x = y > x ? y : x;
  y = ror_row64<1>(x); x = y > x ? y : x;
  return x;
}
__device__ __forceinline__ float row_sum(float x) {
  x += __uint_as_float(ror_row<8>(__float_as_uint(x)));
  x += __uint_as_float(ror_row<4>(__float_as_uint(x)));
  x += __uint_as_float(ror_row<2>(__float_as_uint(x)));
  x += __uint_as_float(ror_row<1>(__float_as_uint(x)));
  return x;
}

__device__ __forceinline__ uint64_t max64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// NV keys per lane (the smallest power of two with 16 NV >= E)
template <int NV>
__global__ __launch_bounds__(RS_THREADS) void route_select(
    const float* __restrict__ logits, int T, int E, int k, int spb, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int32_t* __restrict__ blk_counts, int32_t* __restrict__ local_rank) {
  extern __shared__ __attribute__((aligned(8))) unsigned char rs_smem[];
  uint64_t* sel = (uint64_t*)rs_smem;  // [RS_TOK][k] picked keys
  __shared__ uint32_t mask[256];       // tokens of this round that picked expert e
  __shared__ int cnt[256];             // pairs of expert e in earlier rounds of the block
  const int tl = threadIdx.x >> 4, sub = threadIdx.x & 15;
  for (int e = threadIdx.x; e < E; e += RS_THREADS) {
    mask[e] = 0u;
    cnt[e] = 0;
  }
  __syncthreads();
#pragma unroll 1
  for (int s = 0; s < spb; ++s) {
    const int64_t t0 = ((int64_t)blockIdx.x * spb + s) * RS_TOK;
    if (t0 >= T) break;  // uniform over the workgroup
    const int64_t t = t0 + tl;
    const bool valid = t < T;
    // lane sub keeps the keys of experts sub, sub + 16, ...; absent ones are 0
    float lv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = sub + 16 * i;
      lv[i] = valid && e < E ? logits[t * E + e] : 0.0f;
    }
    uint64_t key[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = sub + 16 * i;
      key[i] = valid && e < E ? ((uint64_t)rt_ord(lv[i]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)e) : 0;
    }
    uint64_t prev = ~(uint64_t)0;
#pragma unroll 1
    for (int j = 0; j < k; ++j) {
      // the lane's largest key below the previous pick: independent
      // candidates, then a tree of maxima
      uint64_t c[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) c[i] = key[i] < prev ? key[i] : 0;
#pragma unroll
      for (int w = NV / 2; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) c[i] = max64(c[i], c[i + w]);
      const uint64_t best = row_max64(c[0]);
      prev = best;
      if (sub == (j & 15)) sel[tl * k + j] = best;
    }
    __syncthreads();
    // softmax of the k picked logits, relative to the largest
    const float v0 = rt_val((uint32_t)(sel[tl * k] >> 32));
    float part = 0.0f;
    for (int j = sub; j < k; j += 16) part += expf(rt_val((uint32_t)(sel[tl * k + j] >> 32)) - v0);
    const float inv = 1.0f / row_sum(part);
    if (valid) {
      for (int j = sub; j < k; j += 16) {
        const uint64_t kk = sel[tl * k + j];
        const int id = (int)(0xffffffffu - (uint32_t)kk);
        topk_ids[t * k + j] = id;
        topk_w[t * k + j] = expf(rt_val((uint32_t)(kk >> 32)) - v0) * inv;
        atomicOr(&mask[id], 1u << tl);
      }
    }
    __syncthreads();
    if (valid) {
      for (int j = sub; j < k; j += 16) {
        const int id = (int)(0xffffffffu - (uint32_t)sel[tl * k + j]);
        local_rank[t * k + j] = cnt[id] + __popc(mask[id] & ((1u << tl) - 1u));
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += RS_THREADS) {
      cnt[e] += __popc(mask[e]);
      mask[e] = 0u;
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < E; e += RS_THREADS) blk_counts[(int64_t)blockIdx.x * E + e] = cnt[e];
}

constexpr int SC_PRE = 4;                 // pairs per thread whose inputs load with the histogram
constexpr int SC_COL = 32;                // histogram rows per load batch of the column sums

__global__ __launch_bounds__(SC_THREADS) void route_scatter(
    const int32_t* __restrict__ topk_ids, const float* __restrict__ topk_w,
    const int32_t* __restrict__ blk_counts, const int32_t* __restrict__ local_rank, int T, int E, int k,
    int S, int spb, int nblk, int bpb2, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos, int32_t* __restrict__ row_token,
    float* __restrict__ row_weight) {
  __shared__ int part_lo[SC_THREADS];   // [group][expert] histogram rows below this range
  __shared__ int part_tot[SC_THREADS];  // [group][expert] all histogram rows
  __shared__ int base[SC_BPB][256];     // offsets[e] + pairs of e in rows before row q of the range
  __shared__ int sh[SC_THREADS / 64];
  const int tid = threadIdx.x;
  const int bfirst = blockIdx.x * bpb2, blast = min(nblk, bfirst + bpb2);
  const int64_t tok_per_blk = (int64_t)spb * RS_TOK;
  const int64_t ta = bfirst * tok_per_blk, tb = min((int64_t)T, blast * tok_per_blk);
  const int64_t i_end = tb * k;
  // Every global load the placement needs is issued here, before any result
  // is used: the thread's first SC_PRE pairs, its histogram column chunk and
  // (threads e < E) expert e's entries in the range's rows.
  int p_id[SC_PRE], p_rank[SC_PRE];
  float p_w[SC_PRE];
#pragma unroll
  for (int q = 0; q < SC_PRE; ++q) {
    const int64_t i = ta * k + tid + (int64_t)q * SC_THREADS;
    const bool ok = i < i_end;
    p_id[q] = ok ? topk_ids[i] : 0;
    p_rank[q] = ok ? local_rank[i] : 0;
    p_w[q] = ok ? topk_w[i] : 0.0f;
  }
  // column sums of the histogram: rows split over ng groups of E threads
  const int ng = SC_THREADS / E;
  const int g = tid / E, e = tid - g * E;
  // (nblk <= 256 rows and ng >= 8 groups for E <= 128: one batch; two at E = 256)
  const int ch = cdiv(nblk, ng);
  const int r0 = g * ch, r1 = g < ng ? min(nblk, r0 + ch) : r0;
  int rowc[SC_BPB];
#pragma unroll
  for (int q = 0; q < SC_BPB; ++q)
    rowc[q] = tid < E && bfirst + q < blast ? blk_counts[(int64_t)(bfirst + q) * E + tid] : 0;
  int lo = 0, tot = 0;
  for (int rb = r0; rb < r1; rb += SC_COL) {
    int c[SC_COL];
#pragma unroll
    for (int q = 0; q < SC_COL; ++q) c[q] = rb + q < r1 ? blk_counts[(int64_t)(rb + q) * E + e] : 0;
#pragma unroll
    for (int q = 0; q < SC_COL; ++q) {
      tot += c[q];
      lo += rb + q < bfirst ? c[q] : 0;
    }
  }
  part_lo[tid] = lo;
  part_tot[tid] = tot;
  __syncthreads();
  int c_e = 0, below = 0;
  if (tid < E) {
    for (int gg = 0; gg < ng; ++gg) {
      below += part_lo[gg * E + tid];
      c_e += part_tot[gg * E + tid];
    }
  }
  int total;
  const int o = block_excl_scan<SC_THREADS / 64>(c_e, sh, &total);
  if (tid < E) {
    // first sorted position of expert e's pairs in each histogram row of the range
    int run = o + below;
#pragma unroll
    for (int q = 0; q < SC_BPB; ++q) {
      base[q][tid] = run;
      run += rowc[q];
    }
    if (blockIdx.x == 0) {
      counts[tid] = c_e;
      offsets[tid] = o;
    }
  }
  if (tid == 0 && blockIdx.x == 0) offsets[E] = total;
  __syncthreads();
  auto place = [&](int64_t i, int id, int rank, float w) {
    const int64_t t = i / k;
    const int q = (int)(t / tok_per_blk) - bfirst;
    const int dest = base[q][id] + rank;
    sorted_pair[dest] = (int32_t)i;
    pair_pos[i] = dest;
    row_token[dest] = (int32_t)t;
    row_weight[dest] = w;
  };
#pragma unroll
  for (int q = 0; q < SC_PRE; ++q) {
    const int64_t i = ta * k + tid + (int64_t)q * SC_THREADS;
    if (i < i_end) place(i, p_id[q], p_rank[q], p_w[q]);
  }
  for (int64_t i = ta * k + tid + (int64_t)SC_PRE * SC_THREADS; i < i_end; i += SC_THREADS)
    place(i, topk_ids[i], local_rank[i], topk_w[i]);
  if (S) {
    const int64_t P = (int64_t)T * k;
    for (int64_t t = ta + tid; t < tb; t += SC_THREADS) {
      row_token[P + t] = (int32_t)t;
      row_weight[P + t] = 1.0f;
    }
  }
}

size_t route_ws_bytes(int64_t T, int E, int k) {
  const RouteGeom g = route_geom(T);
  size_t a = (size_t)g.nblk * E * sizeof(int32_t);
  a = (a + 255) & ~(size_t)255;
  return a + (size_t)T * k * sizeof(int32_t);
}

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int S, int32_t* ids, float* w,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                        int32_t* row_token, float* row_weight, void* ws, hipStream_t st) {
  const RouteGeom g = route_geom(T);
  size_t a = (size_t)g.nblk * E * sizeof(int32_t);
  a = (a + 255) & ~(size_t)255;
  int32_t* blk = (int32_t*)ws;
  int32_t* rank = (int32_t*)((char*)ws + a);
  const size_t lds = (size_t)RS_TOK * k * sizeof(uint64_t);
  const int nv = (E + 15) / 16;
  auto sel = nv <= 1 ? route_select<1> : nv <= 2 ? route_select<2> : nv <= 4 ? route_select<4>
             : nv <= 8 ? route_select<8> : route_select<16>;
  MOE_LAUNCH("route_select", sel, dim3(g.nblk), dim3(RS_THREADS), lds, st, logits, (int)T, E, k, g.spb, ids,
             w, blk, rank);
  MOE_LAUNCH("route_scatter", route_scatter, dim3(g.nblk2), dim3(SC_THREADS), 0, st, ids, w, blk, rank,
             (int)T, E, k, S, g.spb, g.nblk, g.bpb2, counts, offsets, sorted_pair, pair_pos, row_token,
             row_weight);
  return hipGetLastError();
}

}  // namespace moe
