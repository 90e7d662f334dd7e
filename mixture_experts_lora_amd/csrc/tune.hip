// Engine choice per layer shape, and the one-time autotune that makes it
// (the faster-MoE page's kernels pick their configurations by a start-up
// autotune, "Unsloth MoE Triton kernels"; here the choice is between the two
// engines every grouped product has: the register-path kernels of gemm.hip
// and the streamed LDS-DMA kernels of stream.hip / prepass.hip / grads.hip).
#include <string.h>

#include <algorithm>
#include <array>
#include <map>
#include <mutex>

#include "../../include/moe_lora.h"
#include "kernels.h"

namespace moe {

namespace {
std::mutex g_mu;
std::map<std::array<int, 7>, uint32_t> g_table;
}  // namespace

uint32_t lookup_engines(int d, int n, int E, int k, int r, int S, int f16) {
  std::lock_guard<std::mutex> lock(g_mu);
  const auto it = g_table.find({d, n, E, k, r, S, f16});
  return it == g_table.end() ? default_engines() : it->second;
}

void record_engines(int d, int n, int E, int k, int r, int S, int f16, uint32_t engines) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_table[{d, n, E, k, r, S, f16}] = engines;
}

}  // namespace moe

using namespace moe;

namespace {

size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

// Buffers of one route + forward + backward, carved from the scratch block.
struct TuneBufs {
  moe_routing rt;
  void *route_ws, *saved, *ws;
  moe_bf16 *y, *dx;
  float *da_gu, *db_gu, *da_dn, *db_dn;
  size_t route_ws_bytes, saved_bytes, ws_bytes, total;
};

TuneBufs carve(const moe_dims* dm, char* base) {
  TuneBufs b{};
  const size_t T = (size_t)dm->T, k = dm->k, E = dm->E, d = dm->d, n = dm->n, r = dm->r;
  const size_t Et = E + dm->n_shared, P = T * k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += a256(bytes);
    return p;
  };
  b.rt.topk_ids = (int32_t*)take(P * 4);
  b.rt.topk_w = (float*)take(P * 4);
  b.rt.counts = (int32_t*)take(E * 4);
  b.rt.offsets = (int32_t*)take((E + 1) * 4);
  b.rt.sorted_pair = (int32_t*)take(P * 4);
  b.rt.pair_pos = (int32_t*)take(P * 4);
  b.rt.row_token = (int32_t*)take((P + dm->n_shared * T) * 4);
  b.rt.row_weight = (float*)take((P + dm->n_shared * T) * 4);
  b.route_ws_bytes = moe_route_workspace_bytes(dm);
  b.saved_bytes = moe_forward_saved_bytes(dm);
  b.ws_bytes = moe_workspace_bytes(dm);
  b.route_ws = take(b.route_ws_bytes);
  b.saved = take(b.saved_bytes);
  b.ws = take(b.ws_bytes);
  b.y = (moe_bf16*)take(T * d * 2);
  b.dx = (moe_bf16*)take(T * d * 2);
  b.da_gu = (float*)take(Et * d * r * 4);
  b.db_gu = (float*)take(Et * r * 2 * n * 4);
  b.da_dn = (float*)take(Et * n * r * 4);
  b.db_dn = (float*)take(Et * r * d * 4);
  b.total = off;
  return b;
}

moe_status run_layer(const moe_dims* dm, const float* logits, const moe_bf16* x, const moe_bf16* dy,
                     const moe_weights* w, TuneBufs& b, void* stream) {
  moe_status st = moe_route(dm, logits, &b.rt, b.route_ws, b.route_ws_bytes, stream);
  if (st == MOE_SUCCESS)
    st = moe_lora_forward(dm, x, &b.rt, w, b.y, b.saved, b.saved_bytes, b.ws, b.ws_bytes, stream);
  if (st == MOE_SUCCESS)
    st = moe_lora_backward(dm, dy, x, &b.rt, w, b.saved, b.saved_bytes, b.dx, b.da_gu, b.db_gu,
                           b.da_dn, b.db_dn, nullptr, nullptr, b.ws, b.ws_bytes, stream);
  return st;
}

// Milliseconds per step of each product under the current engines: gate_up,
// down, dh, dx, and the rank-r group (pre-passes, weighted rows, gradients).
moe_status time_products(const moe_dims* dm, const float* logits, const moe_bf16* x,
                         const moe_bf16* dy, const moe_weights* w, TuneBufs& b, void* stream,
                         double (&t)[5]) {
  constexpr int STEPS = 3, NAME = 64, MAXN = 64;
  moe_status st = run_layer(dm, logits, x, dy, w, b, stream);  // warm up
  if (st != MOE_SUCCESS) return st;
  if ((st = moe_timing_enable(1)) != MOE_SUCCESS) return st;
  for (int i = 0; i < STEPS && st == MOE_SUCCESS; ++i) st = run_layer(dm, logits, x, dy, w, b, stream);
  static char names[MAXN * NAME];
  float ms[MAXN];
  int launches[MAXN];
  const int cnt = moe_timing_report(names, NAME, ms, launches, MAXN);
  moe_timing_enable(0);
  if (st != MOE_SUCCESS) return st;
  if (cnt < 0) return MOE_ERROR_LAUNCH;
  static const char* const rank_group[] = {"prepass_xa", "prepass_ha", "prepass_qdn", "prepass_qgu",
                                           "prepass_reduce", "weight_rows", "lora_grads",
                                           "grad_db_dn", "grad_da_dn", "grad_db_gu", "grad_da_gu",
                                           "reduce_grads"};
  for (double& v : t) v = 0.0;
  for (int i = 0; i < cnt; ++i) {
    const char* nm = names + i * NAME;
    const double per_step = ms[i] / STEPS;
    if (!strcmp(nm, "gate_up")) t[0] += per_step;
    else if (!strcmp(nm, "down")) t[1] += per_step;
    else if (!strcmp(nm, "dh")) t[2] += per_step;
    else if (!strcmp(nm, "dx")) t[3] += per_step;
    else
      for (const char* g : rank_group)
        if (!strcmp(nm, g)) t[4] += per_step;
  }
  return MOE_SUCCESS;
}

}  // namespace

extern "C" {

moe_status moe_set_engines(const moe_dims* dm, unsigned engines) {
  if (!dm || (engines & ~(unsigned)ENG_ALL)) return MOE_ERROR_INVALID_VALUE;
  record_engines(dm->d, dm->n, dm->E, dm->k, dm->r, dm->n_shared, dm->dtype == MOE_F16, engines);
  return MOE_SUCCESS;
}

unsigned moe_get_engines(const moe_dims* dm) {
  if (!dm) return default_engines();
  return lookup_engines(dm->d, dm->n, dm->E, dm->k, dm->r, dm->n_shared, dm->dtype == MOE_F16);
}

size_t moe_autotune_scratch_bytes(const moe_dims* dm) {
  if (!moe_workspace_bytes(dm)) return 0;
  return carve(dm, nullptr).total;
}

moe_status moe_autotune(const moe_dims* dm, const float* logits, const moe_bf16* x,
                        const moe_bf16* dy, const moe_weights* w, void* scratch,
                        size_t scratch_bytes, void* stream, unsigned* engines_out) {
  if (!moe_workspace_bytes(dm)) return MOE_ERROR_INVALID_VALUE;
  if (!scratch || ((uintptr_t)scratch & 255)) return MOE_ERROR_INVALID_VALUE;
  if (scratch_bytes < moe_autotune_scratch_bytes(dm)) return MOE_ERROR_WORKSPACE;
  TuneBufs b = carve(dm, (char*)scratch);
  const unsigned before = moe_get_engines(dm);
  // each setting twice, alternating, best of the two per product: the first
  // timed runs of a process can be slower while the clocks settle
  double ts[5], tr[5], t[5];
  for (int i = 0; i < 5; ++i) ts[i] = tr[i] = 1e30;
  moe_status st = MOE_SUCCESS;
  for (int round = 0; round < 2 && st == MOE_SUCCESS; ++round)
    for (int streamed = 1; streamed >= 0 && st == MOE_SUCCESS; --streamed) {
      moe_set_engines(dm, streamed ? ENG_ALL : 0u);
      st = time_products(dm, logits, x, dy, w, b, stream, t);
      double* best = streamed ? ts : tr;
      for (int i = 0; i < 5; ++i) best[i] = std::min(best[i], t[i]);
    }
  if (st != MOE_SUCCESS) {
    moe_set_engines(dm, before);
    return st;
  }
  const uint32_t bits[5] = {ENG_GU_STREAM, ENG_DN_STREAM, ENG_DH_STREAM, ENG_DX_STREAM,
                            ENG_RANK_STREAM};
  unsigned chosen = 0;
  for (int i = 0; i < 5; ++i)
    if (ts[i] <= tr[i]) chosen |= bits[i];
  moe_set_engines(dm, chosen);
  if (engines_out) *engines_out = chosen;
  return MOE_SUCCESS;
}

}  // extern "C"
