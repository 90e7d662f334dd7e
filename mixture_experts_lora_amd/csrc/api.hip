// C ABI: argument validation, buffer carving and the launch sequence of each
// entry point (declared and documented in include/moe_lora.h).
#include <math.h>

#include "../../include/moe_lora.h"
#include "kernels.h"

using namespace moe;

namespace {

bool aligned16(const void* p) { return p && (((uintptr_t)p) & 15u) == 0; }

moe_status check_dims(const moe_dims* dm) {
  if (!dm) return MOE_ERROR_INVALID_VALUE;
  if (dm->T < 1 || dm->d < 1 || dm->n < 1 || dm->E < 1 || dm->r < 1) return MOE_ERROR_INVALID_VALUE;
  if (dm->k < 1 || dm->k > dm->E) return MOE_ERROR_INVALID_VALUE;
  if (dm->n_shared != 0 && dm->n_shared != 1) return MOE_ERROR_INVALID_VALUE;
  if (!isfinite(dm->lora_scale)) return MOE_ERROR_INVALID_VALUE;
  if (dm->dtype != MOE_BF16 && dm->dtype != MOE_F16) return MOE_ERROR_INVALID_VALUE;
  if (dm->d % 64 || dm->n % 64 || dm->E > 256 || dm->r > 128) return MOE_ERROR_UNSUPPORTED;
  const int64_t ptot = dm->T * (int64_t)dm->k + (int64_t)dm->n_shared * dm->T;
  if (ptot >= ((int64_t)1 << 31)) return MOE_ERROR_UNSUPPORTED;
  // Buffer resources take 32-bit byte offsets below 2^31 (0x80000000 is the
  // out-of-range marker), so every buffer the kernels address that way must
  // stay below 2 GiB: the widest per-row buffers are [P_tot, max(2n, d)]
  // 16-bit (O, dX per pair, G, dG); H, the rank-r rows (r <= 128 < 2n), the
  // per-row tables and the router partials are narrower per row, and [T, d]
  // has fewer rows.  One expert's [2n, d] weight is addressed the same way.
  const int64_t lim = (int64_t)1 << 31;
  const int64_t widest = 2 * (int64_t)(2 * dm->n > dm->d ? 2 * dm->n : dm->d);
  if (ptot * widest >= lim) return MOE_ERROR_UNSUPPORTED;
  if ((int64_t)2 * dm->n * dm->d * 2 >= lim) return MOE_ERROR_UNSUPPORTED;
  return MOE_SUCCESS;
}

Layer make_layer(const moe_dims* dm) {
  Layer L = {};
  L.T = (int)dm->T;
  L.d = dm->d;
  L.n = dm->n;
  L.E = dm->E;
  L.k = dm->k;
  L.r = dm->r;
  L.S = dm->n_shared;
  L.Et = dm->E + dm->n_shared;
  L.rs = (dm->r + 7) / 8 * 8;
  L.ra = (dm->r % 8) ? L.rs : dm->r;
  L.P = L.T * L.k;
  L.Ptot = L.P + L.S * L.T;
  L.s = dm->lora_scale;
  L.ncu = device_cu_count();
  L.f16 = dm->dtype == MOE_F16;
  L.lora = 1;
  L.engines = lookup_engines(dm->d, dm->n, dm->E, dm->k, dm->r, dm->n_shared, L.f16);
  L.splitk = splitk_rows(L.engines);
  return L;
}

moe_status check_routing_in(const moe_routing* rt) {
  if (!rt) return MOE_ERROR_INVALID_VALUE;
  if (!aligned16(rt->topk_ids) || !aligned16(rt->topk_w) || !aligned16(rt->offsets) ||
      !aligned16(rt->sorted_pair) || !aligned16(rt->pair_pos) || !aligned16(rt->row_token) ||
      !aligned16(rt->row_weight))
    return MOE_ERROR_INVALID_VALUE;
  return MOE_SUCCESS;
}

moe_status check_weights(const moe_weights* w) {
  if (!w) return MOE_ERROR_INVALID_VALUE;
  if (!aligned16(w->w_gate_up) || !aligned16(w->w_down) || !aligned16(w->a_gate_up) ||
      !aligned16(w->b_gate_up) || !aligned16(w->a_down) || !aligned16(w->b_down))
    return MOE_ERROR_INVALID_VALUE;
  return MOE_SUCCESS;
}

moe_status launched(hipError_t e) { return e == hipSuccess ? MOE_SUCCESS : MOE_ERROR_LAUNCH; }

// The element-type-dependent launchers of the layer's type.
#define EL(L, fn, ...) ((L).f16 ? ::moe::el_f16::fn(__VA_ARGS__) : ::moe::el_bf16::fn(__VA_ARGS__))

void attach_common(Layer& L, const moe_routing* rt, const moe_weights* w, const moe_dims* dm,
                   void* ws) {
  L.topk_ids = rt->topk_ids;
  L.topk_w = rt->topk_w;
  L.offsets = rt->offsets;
  L.sorted_pair = rt->sorted_pair;
  L.pair_pos = rt->pair_pos;
  L.tok = rt->row_token;
  L.wgt = rt->row_weight;
  L.w_gu = w->w_gate_up;
  L.w_dn = w->w_down;
  L.b_gu = w->b_gate_up;
  L.b_dn = w->b_down;
  const WsLayout wl = ws_layout(dm->T, dm->d, dm->n, dm->E, dm->k, dm->r, dm->n_shared);
  char* base = (char*)ws;
  if (dm->r % 8) {
    L.a_gu = (const bf16_t*)(base + wl.a_gu_pack);
    L.a_dn = (const bf16_t*)(base + wl.a_dn_pack);
  } else {
    L.a_gu = w->a_gate_up;
    L.a_dn = w->a_down;
  }
  L.o = (bf16_t*)(base + wl.o);
  L.dg = (bf16_t*)(base + wl.dg);
  L.qdn = (bf16_t*)(base + wl.qdn);
  L.qgu = (bf16_t*)(base + wl.qgu);
  L.hw = (bf16_t*)(base + wl.hw);
  L.qw = (bf16_t*)(base + wl.qw);
  L.dw_part = nullptr;  // set by backward when router gradients are requested
  L.dw_groups = dm->n / 64;
  L.partial = (float*)(base + wl.partial);
  L.pre_partial = (float*)(base + wl.pre_partial);
  for (int i = 0; i < 4; ++i) L.partial_off[i] = wl.partial_off[i];
}

void attach_saved(Layer& L, const moe_dims* dm, void* saved) {
  const SavedLayout sl = saved_layout(dm->T, dm->d, dm->n, dm->E, dm->k, dm->r, dm->n_shared);
  char* base = (char*)saved;
  L.g = (bf16_t*)(base + sl.g);
  L.h = (bf16_t*)(base + sl.h);
  L.xa = (bf16_t*)(base + sl.xa);
  L.ha = (bf16_t*)(base + sl.ha);
}

hipError_t maybe_pack(const Layer& L, const moe_weights* w, hipStream_t st) {
  if (L.r % 8 == 0) return hipSuccess;
  return launch_pack_a(L, w->a_gate_up, w->a_down, (bf16_t*)L.a_gu, (bf16_t*)L.a_dn, st);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_SUCCESS: return "MOE_SUCCESS";
    case MOE_ERROR_INVALID_VALUE: return "MOE_ERROR_INVALID_VALUE";
    case MOE_ERROR_UNSUPPORTED: return "MOE_ERROR_UNSUPPORTED";
    case MOE_ERROR_WORKSPACE: return "MOE_ERROR_WORKSPACE";
    case MOE_ERROR_LAUNCH: return "MOE_ERROR_LAUNCH";
  }
  return "MOE_UNKNOWN_STATUS";
}

size_t moe_route_workspace_bytes(const moe_dims* dm) {
  if (check_dims(dm) != MOE_SUCCESS) return 0;
  return route_ws_bytes(dm->T, dm->E, dm->k);
}

size_t moe_forward_saved_bytes(const moe_dims* dm) {
  if (check_dims(dm) != MOE_SUCCESS) return 0;
  return saved_layout(dm->T, dm->d, dm->n, dm->E, dm->k, dm->r, dm->n_shared).total;
}

size_t moe_workspace_bytes(const moe_dims* dm) {
  if (check_dims(dm) != MOE_SUCCESS) return 0;
  return ws_layout(dm->T, dm->d, dm->n, dm->E, dm->k, dm->r, dm->n_shared).total;
}

moe_status moe_route(const moe_dims* dm, const float* logits, const moe_routing* out, void* ws,
                     size_t ws_bytes, void* stream) {
  moe_status st = check_dims(dm);
  if (st != MOE_SUCCESS) return st;
  if (!aligned16(logits) || !out || !aligned16(out->counts) || check_routing_in(out) != MOE_SUCCESS ||
      !aligned16(ws))
    return MOE_ERROR_INVALID_VALUE;
  if (ws_bytes < route_ws_bytes(dm->T, dm->E, dm->k)) return MOE_ERROR_WORKSPACE;
  return launched(launch_route(logits, dm->T, dm->E, dm->k, dm->n_shared, out->topk_ids, out->topk_w,
                               out->counts, out->offsets, out->sorted_pair, out->pair_pos,
                               out->row_token, out->row_weight, ws, (hipStream_t)stream));
}

moe_status moe_lora_forward(const moe_dims* dm, const moe_bf16* x, const moe_routing* rt,
                            const moe_weights* w, moe_bf16* y, void* saved, size_t saved_bytes,
                            void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_dims(dm);
  if (st != MOE_SUCCESS) return st;
  if ((st = check_routing_in(rt)) != MOE_SUCCESS) return st;
  if ((st = check_weights(w)) != MOE_SUCCESS) return st;
  if (!aligned16(x) || !aligned16(y) || !aligned16(saved) || !aligned16(ws))
    return MOE_ERROR_INVALID_VALUE;
  if (saved_bytes < moe_forward_saved_bytes(dm) || ws_bytes < moe_workspace_bytes(dm))
    return MOE_ERROR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  Layer L = make_layer(dm);
  attach_common(L, rt, w, dm, ws);
  attach_saved(L, dm, saved);
  L.x = x;
  L.y = y;
  hipError_t e = maybe_pack(L, w, s);
  if (e == hipSuccess) e = EL(L, gemm_gate_up, L, s);
  if (e == hipSuccess) e = EL(L, gemm_down, L, s);
  if (e == hipSuccess) e = EL(L, launch_combine, L, true, L.o, L.y, s);
  return launched(e);
}

moe_status moe_merge_lora(const moe_dims* dm, const moe_weights* w, moe_bf16* w_gate_up_merged,
                          moe_bf16* w_down_merged, void* stream) {
  moe_status st = check_dims(dm);
  if (st != MOE_SUCCESS) return st;
  if ((st = check_weights(w)) != MOE_SUCCESS) return st;
  if (!aligned16(w_gate_up_merged) || !aligned16(w_down_merged)) return MOE_ERROR_INVALID_VALUE;
  Layer L = make_layer(dm);
  L.w_gu = w->w_gate_up;
  L.w_dn = w->w_down;
  L.b_gu = w->b_gate_up;
  L.b_dn = w->b_down;
  return launched(EL(L, merge_lora, L, w->a_gate_up, w->a_down, w_gate_up_merged, w_down_merged,
                     (hipStream_t)stream));
}

moe_status moe_forward_merged(const moe_dims* dm, const moe_bf16* x, const moe_routing* rt,
                              const moe_bf16* w_gate_up_merged, const moe_bf16* w_down_merged,
                              moe_bf16* y, void* saved, size_t saved_bytes, void* ws,
                              size_t ws_bytes, void* stream) {
  moe_status st = check_dims(dm);
  if (st != MOE_SUCCESS) return st;
  if ((st = check_routing_in(rt)) != MOE_SUCCESS) return st;
  if (!aligned16(x) || !aligned16(y) || !aligned16(saved) || !aligned16(ws) ||
      !aligned16(w_gate_up_merged) || !aligned16(w_down_merged))
    return MOE_ERROR_INVALID_VALUE;
  if (saved_bytes < moe_forward_saved_bytes(dm) || ws_bytes < moe_workspace_bytes(dm))
    return MOE_ERROR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  // the low-rank factor slots are never read with the low-rank pass off
  const moe_weights mw = {w_gate_up_merged, w_down_merged, w_gate_up_merged, w_gate_up_merged,
                          w_down_merged, w_down_merged};
  Layer L = make_layer(dm);
  L.lora = 0;
  attach_common(L, rt, &mw, dm, ws);
  attach_saved(L, dm, saved);
  L.x = x;
  L.y = y;
  hipError_t e = EL(L, gemm_gate_up, L, s);
  if (e == hipSuccess) e = EL(L, gemm_down, L, s);
  if (e == hipSuccess) e = EL(L, launch_combine, L, true, L.o, L.y, s);
  return launched(e);
}

moe_status moe_lora_backward(const moe_dims* dm, const moe_bf16* dy, const moe_bf16* x,
                             const moe_routing* rt, const moe_weights* w, const void* saved,
                             size_t saved_bytes, moe_bf16* dx, float* da_gate_up,
                             float* db_gate_up, float* da_down, float* db_down,
                             float* d_topk_w, float* d_logits, void* ws, size_t ws_bytes,
                             void* stream) {
  moe_status st = check_dims(dm);
  if (st != MOE_SUCCESS) return st;
  if ((st = check_routing_in(rt)) != MOE_SUCCESS) return st;
  if ((st = check_weights(w)) != MOE_SUCCESS) return st;
  if (!aligned16(dy) || !aligned16(x) || !aligned16(saved) || !aligned16(dx) ||
      !aligned16(da_gate_up) || !aligned16(db_gate_up) || !aligned16(da_down) ||
      !aligned16(db_down) || !aligned16(ws))
    return MOE_ERROR_INVALID_VALUE;
  if ((d_topk_w && !aligned16(d_topk_w)) || (d_logits && !aligned16(d_logits)))
    return MOE_ERROR_INVALID_VALUE;
  const bool router = d_topk_w || d_logits;
  if (saved_bytes < moe_forward_saved_bytes(dm) || ws_bytes < moe_workspace_bytes(dm))
    return MOE_ERROR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  Layer L = make_layer(dm);
  attach_common(L, rt, w, dm, ws);
  attach_saved(L, dm, (void*)saved);
  L.x = x;
  L.dy = dy;
  L.dx = dx;
  L.da_gu = da_gate_up;
  L.db_gu = db_gate_up;
  L.da_dn = da_down;
  L.db_dn = db_down;
  if (router) {
    // the <dH, H> partials come from the streamed dh's epilogue
    L.engines |= ENG_DH_STREAM;
    L.dw_part = (float*)((char*)ws + ws_layout(dm->T, dm->d, dm->n, dm->E, dm->k, dm->r,
                                               dm->n_shared).dw_part);
  }
  hipError_t e = maybe_pack(L, w, s);
  if (e == hipSuccess) e = EL(L, gemm_dh, L, s);
  if (e == hipSuccess && router) e = launch_router_grad(L, d_topk_w, d_logits, s);
  if (e == hipSuccess) e = EL(L, gemm_dx, L, s);
  if (e == hipSuccess) e = EL(L, launch_combine, L, false, L.o, L.dx, s);
  if (e == hipSuccess) e = EL(L, gemm_lora_grads, L, s);
  return launched(e);
}

}  // extern "C"
