// Weighted gather-combine of the per-pair outputs into token rows (the
// faster-MoE page's per-token sum over the k selected experts), forward
// (weighted by the routing weights) and backward (unweighted).
#include "common.h"
#include "kernels.h"

namespace moe {
inline namespace MOE_EL {

// dst[t] = sum_j w[t,j] * src[pair_pos[t*k+j]]  (+ src[P + t] for the shared
// expert), fp32 sum in slot order; w = 1 when not weighted (the backward,
// where the routing weight already entered through dO).
__global__ __launch_bounds__(256) void k_combine(const Layer L, int weighted,
                                                 const bf16_t* __restrict__ src,
                                                 bf16_t* __restrict__ dst) {
  const int t = blockIdx.x;
  const int d = L.d, k = L.k;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    auto add = [&](const uint4& v, float w) {
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += w * bf2f((bf16_t)(u[q] & 0xffffu));
        acc[2 * q + 1] += w * bf2f((bf16_t)(u[q] >> 16));
      }
    };
    // four slots' rows in flight at once, added in slot order
    int j = 0;
    for (; j + 4 <= k; j += 4) {
      uint4 v[4];
      float w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t i = (int64_t)t * k + j + q;
        w[q] = weighted ? L.topk_w[i] : 1.0f;
        v[q] = *(const uint4*)(src + (int64_t)L.pair_pos[i] * d + c);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) add(v[q], w[q]);
    }
    for (; j < k; ++j) {
      const int64_t i = (int64_t)t * k + j;
      add(*(const uint4*)(src + (int64_t)L.pair_pos[i] * d + c), weighted ? L.topk_w[i] : 1.0f);
    }
    if (L.S) {
      const uint4 v = *(const uint4*)(src + ((int64_t)L.P + t) * d + c);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf2f((bf16_t)(u[q] & 0xffffu));
        acc[2 * q + 1] += bf2f((bf16_t)(u[q] >> 16));
      }
    }
    *(uint4*)(dst + (int64_t)t * d + c) =
        make_uint4(pack2(acc[0], acc[1]), pack2(acc[2], acc[3]), pack2(acc[4], acc[5]),
                   pack2(acc[6], acc[7]));
  }
}

hipError_t launch_combine(const Layer& L, bool weighted, const bf16_t* src, bf16_t* dst,
                          hipStream_t st) {
  MOE_LAUNCH(weighted ? "combine_y" : "combine_dx", k_combine, dim3(L.T), dim3(256), 0, st, L, weighted ? 1 : 0, src, dst);
  return hipGetLastError();
}

}  // inline namespace MOE_EL
}  // namespace moe
