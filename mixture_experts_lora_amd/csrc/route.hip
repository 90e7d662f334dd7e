// Routing: top-k softmax and the one-pass grouping of (token, slot) pairs by
// expert (article on Unsloth x NVIDIA training optimisations, section
// "Optimisation 3: MoE routing grouped once": flatten, stable sort by expert
// id, one bincount, offsets from counts, slice by offset).
//
// Three kernels, no host round trip:
//   1. route_topk_hist  one workgroup per block of 16 tokens (16 lanes per
//      token, logits in registers): top-k + softmax, then an LDS-private
//      per-expert token bitmask (16 bits = the block's tokens).  Popcounts of the bitmask give the block's histogram row and
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
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int RT_TOK = 16;      // tokens per routing block
constexpr int RT_LANES = 16;    // lanes per token; each holds up to 16 logits
constexpr int RT_THREADS = RT_TOK * RT_LANES;
constexpr int SCAN_THREADS = 256;
constexpr int PERM_BLOCKS = 4;  // routing blocks per permute workgroup
constexpr int PERM_THREADS = 256;

// (v, e) comes strictly before (bv, be) in the order value descending, id
// ascending; be < 0 marks "nothing yet"
__device__ __forceinline__ bool rt_before(float v, int e, float bv, int be) {
  return be < 0 || v > bv || (v == bv && e < be);
}

// One workgroup per block of 16 tokens, 16 lanes per token.  A lane keeps its
// token's logits e = lane, lane+16, ... in registers; pick j is the best
// element strictly after pick j-1, found by a register scan and a 16-lane
// shuffle reduction.  The picks go to LDS, then the softmax weights, the
// block's per-expert token bitmask (16 bits), the in-block ranks and the
// histogram row follow from there.
__global__ __launch_bounds__(RT_THREADS) void route_topk_hist(
    const float* __restrict__ logits, int T, int E, int k, int32_t* __restrict__ topk_ids,
    float* __restrict__ topk_w, int32_t* __restrict__ blk_counts, int32_t* __restrict__ local_rank) {
  extern __shared__ unsigned char rt_smem[];
  int* sel_id = (int*)rt_smem;                    // [RT_TOK][k]
  float* sel_v = (float*)(sel_id + RT_TOK * k);  // [RT_TOK][k]
  __shared__ uint32_t mask[256];
  const int b = blockIdx.x;
  const int t0 = b * RT_TOK;
  const int ntok = min(RT_TOK, T - t0);
  const int tl = threadIdx.x / RT_LANES;
  const int sub = threadIdx.x % RT_LANES;
  const bool valid = tl < ntok;
  const int t = t0 + tl;
  for (int i = threadIdx.x; i < E; i += RT_THREADS) mask[i] = 0u;

  float v[16];
  const float* row = logits + (int64_t)t * E;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = sub + RT_LANES * i;
    v[i] = (valid && e < E) ? row[e] : -INFINITY;
  }
  float pv = INFINITY;
  int pe = -1;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = -1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = sub + RT_LANES * i;
      const bool after = (v[i] < pv) || (v[i] == pv && e > pe);
      if (e < E && after && rt_before(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int m = 1; m < RT_LANES; m <<= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oe = __shfl_xor(be, m, 64);
      if (oe >= 0 && rt_before(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    pv = bv;
    pe = be;
    if (sub == 0) {
      sel_id[tl * k + j] = be;
      sel_v[tl * k + j] = bv;
    }
  }
  __syncthreads();
  if (valid) {
    const float v0 = sel_v[tl * k];
    float sum = 0.0f;
    for (int j = 0; j < k; ++j) sum += expf(sel_v[tl * k + j] - v0);
    const float inv = 1.0f / sum;
    for (int j = sub; j < k; j += RT_LANES) {
      const int id = sel_id[tl * k + j];
      topk_ids[(int64_t)t * k + j] = id;
      topk_w[(int64_t)t * k + j] = expf(sel_v[tl * k + j] - v0) * inv;
      atomicOr(&mask[id], 1u << tl);
    }
  }
  __syncthreads();
  if (valid) {
    for (int j = sub; j < k; j += RT_LANES) {
      const int id = sel_id[tl * k + j];
      local_rank[(int64_t)t * k + j] = __popc(mask[id] & ((1u << tl) - 1u));
    }
  }
  for (int e = threadIdx.x; e < E; e += RT_THREADS)
    blk_counts[(int64_t)b * E + e] = __popc(mask[e]);
}

__global__ __launch_bounds__(SCAN_THREADS) void route_scan_blocks(int32_t* __restrict__ blk,
                                                                  int nblk, int E,
                                                                  int32_t* __restrict__ counts) {
  __shared__ int sh[4];
  const int e = blockIdx.x;
  const int per = (nblk + SCAN_THREADS - 1) / SCAN_THREADS;
  const int b0 = threadIdx.x * per, b1 = min(nblk, b0 + per);
  int s = 0;
  for (int b = b0; b < b1; ++b) s += blk[(int64_t)b * E + e];
  int total;
  int base = block_excl_scan256(s, sh, &total);
  for (int b = b0; b < b1; ++b) {
    const int c = blk[(int64_t)b * E + e];
    blk[(int64_t)b * E + e] = base;
    base += c;
  }
  if (threadIdx.x == 0) counts[e] = total;
}

__global__ __launch_bounds__(PERM_THREADS) void route_permute(
    const int32_t* __restrict__ topk_ids, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ bases, const int32_t* __restrict__ local_rank, int T, int E, int k,
    int nblk, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos) {
  __shared__ int offs[256 + 1];
  __shared__ int bb[PERM_BLOCKS][256];
  __shared__ int sh[4];
  const int pb = blockIdx.x;
  const int e = threadIdx.x;
  const int c = e < E ? counts[e] : 0;
  int total;
  const int o = block_excl_scan256(c, sh, &total);
  if (e < E) {
    offs[e] = o;
#pragma unroll
    for (int q = 0; q < PERM_BLOCKS; ++q) {
      const int b = pb * PERM_BLOCKS + q;
      bb[q][e] = b < nblk ? bases[(int64_t)b * E + e] : 0;
    }
  }
  if (e == 0) offs[E] = total;
  if (pb == 0) {
    if (e < E) offsets[e] = o;
    if (e == 0) offsets[E] = total;
  }
  __syncthreads();
  const int64_t tok0 = (int64_t)pb * PERM_BLOCKS * RT_TOK;
  const int64_t i0 = tok0 * k;
  const int64_t i1 = min((int64_t)T, tok0 + PERM_BLOCKS * RT_TOK) * k;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += PERM_THREADS) {
    const int id = topk_ids[i];
    const int q = (int)((i / k - tok0) / RT_TOK);
    const int dest = offs[id] + bb[q][id] + local_rank[i];
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
  const size_t lds = (size_t)RT_TOK * k * (sizeof(int) + sizeof(float));
  MOE_LAUNCH("route_topk_hist", route_topk_hist, dim3(nblk), dim3(RT_THREADS), lds, st, logits, (int)T, E, k,
                     ids, w, blk, rank);
  MOE_LAUNCH("route_scan_blocks", route_scan_blocks, dim3(E), dim3(SCAN_THREADS), 0, st, blk, nblk, E,
             counts);
  MOE_LAUNCH("route_permute", route_permute, dim3(cdiv(nblk, PERM_BLOCKS)), dim3(PERM_THREADS), 0, st,
             ids, counts, blk, rank, (int)T, E, k, nblk, offsets, sorted_pair, pair_pos);
  return hipGetLastError();
}

}  // namespace moe
