// Routing: top-k softmax and the one-pass grouping of (token, slot) pairs by
// expert (article on Unsloth x NVIDIA training optimisations, section
// "Optimisation 3: MoE routing grouped once": flatten, stable sort by expert
// id, one bincount, offsets from counts, slice by offset).
//
// Three kernels, no host round trip:
//   1. route_topk_hist  one workgroup per block of 64 tokens: top-k + softmax,
//      then an LDS-private per-expert token bitmask (64 bits = the block's
//      tokens).  Popcounts of the bitmask give the block's histogram row and
//      every pair's rank among the block's earlier pairs of the same expert
//      (a token never picks an expert twice, so rank within the block equals
//      the number of earlier tokens that picked it: the sort stays stable
//      without atomics deciding any order).
//   2. route_scan_blocks  one workgroup per expert: exclusive scan of that
//      expert's histogram column over blocks (-> block bases) and its total
//      (-> counts, the bincount).
//   3. route_permute  exclusive scan of counts (-> offsets, E+1 entries), then
//      dest = offsets[e] + base[block][e] + rank; sorted_pair[dest] = i and
//      pair_pos[i] = dest.
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int RT_TOK = 64;     // tokens per routing block
constexpr int RT_THREADS = 256;

__host__ __device__ inline int route_lds_stride(int E) { return ((E + 7) / 8) * 8 + 4; }

__global__ __launch_bounds__(RT_THREADS) void route_topk_hist(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int32_t* __restrict__ blk_counts, int32_t* __restrict__ local_rank) {
  extern __shared__ float Ls[];  // [RT_TOK][stride]
  __shared__ uint32_t mask[2 * 256];
  const int stride = route_lds_stride(E);
  const int b = blockIdx.x;
  const int t0 = b * RT_TOK;
  const int ntok = min(RT_TOK, T - t0);
  const float* src = logits + (int64_t)t0 * E;
  for (int idx = threadIdx.x; idx < ntok * E; idx += RT_THREADS) {
    int tl = idx / E, e = idx - tl * E;
    Ls[tl * stride + e] = src[idx];
  }
  for (int i = threadIdx.x; i < 2 * E; i += RT_THREADS) mask[i] = 0u;
  __syncthreads();

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int tl = wid * 16 + (lane >> 2);
  const int sub = lane & 3;
  const bool valid = tl < ntok;
  const int t = t0 + tl;
  const float* row = Ls + tl * stride;

  // Repeated selection in the total order (value descending, id ascending):
  // pick j is the best element strictly after pick j-1.
  float pv = INFINITY;
  int pe = -1;
  float v0 = 0.f, sum = 0.f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
    if (valid) {
      for (int e = sub; e < E; e += 4) {
        float v = row[e];
        bool after = (v < pv) || (v == pv && e > pe);
        bool better = (be == 0x7fffffff) || (v > bv) || (v == bv && e < be);
        if (after && better) { bv = v; be = e; }
      }
    }
#pragma unroll
    for (int m = 1; m < 4; m <<= 1) {
      float ov = __shfl_xor(bv, m, 64);
      int oe = __shfl_xor(be, m, 64);
      bool take = (oe != 0x7fffffff) &&
                  ((be == 0x7fffffff) || (ov > bv) || (ov == bv && oe < be));
      if (take) { bv = ov; be = oe; }
    }
    if (j == 0) v0 = bv;
    sum += expf(bv - v0);
    pv = bv;
    pe = be;
    if (valid && (j & 3) == sub) topk_ids[(int64_t)t * k + j] = be;
  }
  if (valid) {
    const float inv = 1.0f / sum;
    for (int j = sub; j < k; j += 4) {
      int id = topk_ids[(int64_t)t * k + j];  // written above by this thread
      topk_w[(int64_t)t * k + j] = expf(row[id] - v0) * inv;
      atomicOr(&mask[2 * id + (tl >> 5)], 1u << (tl & 31));
    }
  }
  __syncthreads();
  if (valid) {
    for (int j = sub; j < k; j += 4) {
      int id = topk_ids[(int64_t)t * k + j];
      uint32_t lo = mask[2 * id], hi = mask[2 * id + 1];
      int rank = tl < 32 ? __popc(lo & ((1u << tl) - 1u))
                         : __popc(lo) + __popc(hi & ((1u << (tl - 32)) - 1u));
      local_rank[(int64_t)t * k + j] = rank;
    }
  }
  for (int e = threadIdx.x; e < E; e += RT_THREADS)
    blk_counts[(int64_t)b * E + e] = __popc(mask[2 * e]) + __popc(mask[2 * e + 1]);
}

__global__ __launch_bounds__(RT_THREADS) void route_scan_blocks(int32_t* __restrict__ blk,
                                                                int nblk, int E,
                                                                int32_t* __restrict__ counts) {
  __shared__ int sh[4];
  const int e = blockIdx.x;
  const int per = (nblk + RT_THREADS - 1) / RT_THREADS;
  const int b0 = threadIdx.x * per, b1 = min(nblk, b0 + per);
  int s = 0;
  for (int b = b0; b < b1; ++b) s += blk[(int64_t)b * E + e];
  int total;
  int base = block_excl_scan256(s, sh, &total);
  for (int b = b0; b < b1; ++b) {
    int c = blk[(int64_t)b * E + e];
    blk[(int64_t)b * E + e] = base;
    base += c;
  }
  if (threadIdx.x == 0) counts[e] = total;
}

__global__ __launch_bounds__(RT_THREADS) void route_permute(
    const int32_t* __restrict__ topk_ids, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ bases, const int32_t* __restrict__ local_rank, int T, int E, int k,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos) {
  __shared__ int offs[256 + 1];
  __shared__ int bb[256];
  __shared__ int sh[4];
  const int b = blockIdx.x;
  const int e = threadIdx.x;
  int c = e < E ? counts[e] : 0;
  int total;
  int o = block_excl_scan256(c, sh, &total);
  if (e < E) {
    offs[e] = o;
    bb[e] = bases[(int64_t)b * E + e];
  }
  if (e == 0) offs[E] = total;
  if (b == 0) {
    if (e < E) offsets[e] = o;
    if (e == 0) offsets[E] = total;
  }
  __syncthreads();
  const int64_t i0 = (int64_t)b * RT_TOK * k;
  const int64_t i1 = min((int64_t)T, (int64_t)(b + 1) * RT_TOK) * k;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += RT_THREADS) {
    int id = topk_ids[i];
    int dest = offs[id] + bb[id] + local_rank[i];
    sorted_pair[dest] = (int32_t)i;
    pair_pos[i] = dest;
  }
}

size_t route_ws_bytes(int64_t T, int E, int k) {
  const int64_t nblk = cdiv64(T, RT_TOK);
  size_t a = (size_t)nblk * E * sizeof(int32_t);
  a = (a + 255) & ~(size_t)255;
  return a + (size_t)T * k * sizeof(int32_t);
}

hipError_t launch_route(const float* logits, int64_t T, int E, int k, int32_t* ids, float* w,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_pair,
                        int32_t* pair_pos, void* ws, hipStream_t st) {
  const int nblk = (int)cdiv64(T, RT_TOK);
  size_t a = (size_t)nblk * E * sizeof(int32_t);
  a = (a + 255) & ~(size_t)255;
  int32_t* blk = (int32_t*)ws;
  int32_t* rank = (int32_t*)((char*)ws + a);
  const size_t lds = (size_t)RT_TOK * route_lds_stride(E) * sizeof(float);
  if (lds > 65536) {
    static std::atomic<int> raised{0};
    if (!raised.exchange(1))
      (void)hipFuncSetAttribute((const void*)route_topk_hist,
                                hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
  }
  MOE_LAUNCH("route_topk_hist", route_topk_hist, dim3(nblk), dim3(RT_THREADS), lds, st, logits, (int)T, E, k,
                     ids, w, blk, rank);
  MOE_LAUNCH("route_scan_blocks", route_scan_blocks, dim3(E), dim3(RT_THREADS), 0, st, blk, nblk, E, counts);
  MOE_LAUNCH("route_permute", route_permute, dim3(nblk), dim3(RT_THREADS), 0, st, ids, counts, blk, rank,
                     (int)T, E, k, offsets, sorted_pair, pair_pos);
  return hipGetLastError();
}

}  // namespace moe
