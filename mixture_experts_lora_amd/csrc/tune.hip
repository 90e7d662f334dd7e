// Engine and tile choice per layer shape, and the one-time autotune that
// makes it (the faster-MoE page's kernels pick their configurations by a
// start-up autotune, "Unsloth MoE Triton kernels").  Per grouped product the
// choice is the register-path kernel of gemm.hip or the streamed kernel of
// stream.hip in one of its four tile configurations (320- or 256-row tiles,
// 64- or 32-k ring stages); for the rank-r group (pre-passes and LoRA
// gradients) the register path or the streamed one with 2048-, 1024- or
// 4096-row split-K chunks.
#include <string.h>

#include <algorithm>
#include <array>
#include <initializer_list>
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
  char names[MAXN * NAME];  // per call: concurrent autotunes on other threads keep their own
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
  if (!dm || !engines_valid(engines)) return MOE_ERROR_INVALID_VALUE;
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
  // the settings timed: each sets every product alike; per product the
  // fastest setting wins (a product's kernels do not depend on the others')
  constexpr uint32_t ALL4 = 15u;  // the four products' bits of a tile field
  constexpr int NSET = 7, REG = 4;
  const uint32_t settings[NSET] = {
      ENG_ALL,                                                 // 0: streamed, 320 rows, 64-k (default)
      ENG_ALL | (ALL4 << 5),                                   // 1: 256-row tiles
      ENG_ALL | (ALL4 << 9),                                   // 2: 32-k stages
      ENG_ALL | (ALL4 << 5) | (ALL4 << 9),                     // 3: both
      0u,                                                      // 4: register path
      ENG_ALL | (1u << ENG_SPLITK_SHIFT),                      // 5: 1024-row split-K chunks
      ENG_ALL | (2u << ENG_SPLITK_SHIFT)};                     // 6: 4096-row split-K chunks
  // each setting twice, alternating, best of the two per product: the first
  // timed runs of a process can be slower while the clocks settle
  double best[NSET][5], t[5];
  for (auto& row : best)
    for (double& v : row) v = 1e30;
  moe_status st = MOE_SUCCESS;
  for (int round = 0; round < 2 && st == MOE_SUCCESS; ++round)
    for (int i = 0; i < NSET && st == MOE_SUCCESS; ++i) {
      moe_set_engines(dm, settings[i]);
      st = time_products(dm, logits, x, dy, w, b, stream, t);
      for (int p = 0; p < 5; ++p) best[i][p] = std::min(best[i][p], t[p]);
    }
  if (st != MOE_SUCCESS) {
    moe_set_engines(dm, before);
    return st;
  }
  // a setting other than the default has to win by more than 1 % (run-to-run
  // noise is about that size)
  auto pick = [&](int p, std::initializer_list<int> cands) {
    int w = 0;
    for (int i : cands)
      if (best[i][p] < best[w][p] && best[i][p] < 0.99 * best[0][p]) w = i;
    return w;
  };
  unsigned chosen = 0;
  for (int p = 0; p < 4; ++p) {
    const int w = pick(p, {1, 2, 3, REG});
    if (w != REG) chosen |= (1u << p) | (settings[w] & (((1u << 5) | (1u << 9)) << p));
  }
  const int wr = pick(4, {REG, 5, 6});
  if (wr != REG) chosen |= ENG_RANK_STREAM | (settings[wr] & ENG_SPLITK_MASK);
  moe_set_engines(dm, chosen);
  if (engines_out) *engines_out = chosen;
  return MOE_SUCCESS;
}

}  // extern "C"
