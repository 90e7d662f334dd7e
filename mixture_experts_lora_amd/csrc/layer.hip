// LoRA-factor packing, router gradients and buffer layouts
// (nothing here depends on the element type).
#include <atomic>

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

WsLayout ws_layout(int64_t T, int d, int n, int E, int k, int r, int S) {
  const int64_t Ptot = T * k + (int64_t)S * T;
  const int64_t Et = E + S;
  const int64_t rs = (r + 7) / 8 * 8;
  WsLayout w;
  size_t off = 0;
  w.o = off;        off += align256((size_t)Ptot * d * 2);
  w.dg = off;       off += align256((size_t)Ptot * 2 * n * 2);
  w.qdn = off;      off += align256((size_t)Ptot * rs * 2);
  w.qgu = off;      off += align256((size_t)Ptot * rs * 2);
  w.hw = off;       off += align256((size_t)Ptot * rs * 2);
  w.qw = off;       off += align256((size_t)Ptot * rs * 2);
  w.dw_part = off;  off += align256((size_t)Ptot * (n / 64) * 4);
  // partial slots for the smallest split-K chunk any engine setting uses
  const int64_t slots = Ptot / SPLITK_MIN + Et;
  int64_t pf = 0;
  for (int kind = 0; kind < 4; ++kind) {
    int M, N;
    grad_shape(kind, d, n, r, M, N);
    w.partial_off[kind] = pf;
    pf += (slots * M * N + 63) / 64 * 64;
  }
  w.partial = off;  off += align256((size_t)pf * 4);
  w.pre_partial = off; off += align256((size_t)PREPASS_MAX_SPLIT * Ptot * rs * 4);
  const bool pack = (r % 8) != 0;
  w.a_gu_pack = off; off += pack ? align256((size_t)(Et * d * rs * 2)) : 0;
  w.a_dn_pack = off; off += pack ? align256((size_t)(Et * n * rs * 2)) : 0;
  w.total = off;
  return w;
}

SavedLayout saved_layout(int64_t T, int d, int n, int E, int k, int r, int S) {
  (void)d;
  (void)E;
  const int64_t Ptot = T * k + (int64_t)S * T;
  const int64_t rs = (r + 7) / 8 * 8;
  SavedLayout s;
  size_t off = 0;
  s.g = off;  off += align256((size_t)Ptot * 2 * n * 2);
  s.h = off;  off += align256((size_t)Ptot * n * 2);
  s.xa = off; off += align256((size_t)Ptot * rs * 2);
  s.ha = off; off += align256((size_t)Ptot * rs * 2);
  s.total = off;
  return s;
}

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int cu = 0;
  if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
    cu = 256;
  if (dev < 64) cache[dev].store(cu, std::memory_order_relaxed);
  return cu;
}

// [rows, r] -> [rows, rs] with zero padding, for ranks that are not a
// multiple of 8 (16-byte vector loads need 8-element rows).
__global__ void k_pack_rank(const bf16_t* __restrict__ src, bf16_t* __restrict__ dst, int64_t rows,
                            int r, int rs) {
  const int64_t total = rows * rs;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / rs;
    const int c = (int)(i - row * rs);
    dst[i] = c < r ? src[row * r + c] : (bf16_t)0;
  }
}

hipError_t launch_pack_a(const Layer& L, const bf16_t* a_gu_src, const bf16_t* a_dn_src,
                         bf16_t* a_gu_dst, bf16_t* a_dn_dst, hipStream_t st) {
  const int64_t rows_gu = (int64_t)L.Et * L.d, rows_dn = (int64_t)L.Et * L.n;
  const int gb = (int)std::min<int64_t>(cdiv64(rows_gu * L.rs, 256), 4096);
  const int gd = (int)std::min<int64_t>(cdiv64(rows_dn * L.rs, 256), 4096);
  MOE_LAUNCH("pack_a", k_pack_rank, dim3(gb), dim3(256), 0, st, a_gu_src, a_gu_dst, rows_gu, L.r, L.rs);
  MOE_LAUNCH("pack_a", k_pack_rank, dim3(gd), dim3(256), 0, st, a_dn_src, a_dn_dst, rows_dn, L.r, L.rs);
  return hipGetLastError();
}

// Gradients that reach the router (for a model that trains it; the layer's
// own backward leaves the router frozen, "Faster LoRA MoE training").  Y[t]
// is linear in the routing weights, so d w[t, j] = <dY[t], O(t, j)>, which
// equals <dH, H> over the pair's row with dH taken before the routing weight
// (the dh epilogue leaves those dot products per 64-column group in
// dw_part).  Through the softmax over the k selected logits:
// d logit[t, id_j] = w_j (dw_j - sum_i w_i dw_i); the other logits get 0.
// One wave per token; sums run in a fixed order.
__global__ __launch_bounds__(64) void k_router_grad(const Layer L, float* __restrict__ d_topk_w,
                                                    float* __restrict__ d_logits) {
  __shared__ float row[256];  // E <= 256 (validated at the boundary), k <= E
  __shared__ float dwv[256];
  const int t = blockIdx.x, lane = threadIdx.x;
  const int k = L.k, E = L.E, G = L.dw_groups;
  float part = 0.0f;
  for (int j = lane; j < k; j += 64) {
    const int64_t p = L.pair_pos[(int64_t)t * k + j];
    const float* src = L.dw_part + p * G;
    float sdw = 0.0f;
    for (int g = 0; g < G; ++g) sdw += src[g];
    dwv[j] = sdw;
    if (d_topk_w) d_topk_w[(int64_t)t * k + j] = sdw;
    part += L.topk_w[(int64_t)t * k + j] * sdw;
  }
  if (!d_logits) return;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
  for (int e = lane; e < E; e += 64) row[e] = 0.0f;
  __syncthreads();
  for (int j = lane; j < k; j += 64) {
    const float w = L.topk_w[(int64_t)t * k + j];
    row[L.topk_ids[(int64_t)t * k + j]] = w * (dwv[j] - part);
  }
  __syncthreads();
  for (int e = lane; e < E; e += 64) d_logits[(int64_t)t * E + e] = row[e];
}

hipError_t launch_router_grad(const Layer& L, float* d_topk_w, float* d_logits, hipStream_t st) {
  MOE_LAUNCH("router_grad", k_router_grad, dim3(L.T), dim3(64), 0, st, L, d_topk_w, d_logits);
  return hipGetLastError();
}

}  // namespace moe
