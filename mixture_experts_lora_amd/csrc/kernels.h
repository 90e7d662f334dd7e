// Internal interface between the C ABI (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifndef MOE_EL
#ifdef MOE_F16
#define MOE_EL el_f16
#else
#define MOE_EL el_bf16
#endif
#endif

namespace moe {

typedef uint16_t bf16_t;

// Everything one forward or backward call touches.  Device pointers only.
// Rows of every grouped GEMM are "sorted positions" p in [0, P_tot): routed
// pairs in expert order p < P (expert e owns [offsets[e], offsets[e+1])),
// then the shared expert's T rows p = P + t.
// Engine of each product (bit set = streamed / one-launch LDS-DMA engine,
// clear = register-path engine); the choice is made per layer shape.
enum EngineBits : uint32_t {
  ENG_GU_STREAM = 1u << 0,    // gate_up grouped GEMM
  ENG_DN_STREAM = 1u << 1,    // down
  ENG_DH_STREAM = 1u << 2,    // dh (+ SwiGLU backward); router-gradient partials need it
  ENG_DX_STREAM = 1u << 3,    // dX per pair
  ENG_RANK_STREAM = 1u << 4,  // rank-r pre-passes and LoRA gradients (rank <= 64)
  ENG_ALL = 31u,
  // tile configuration of each streamed product (product p = 0 gate_up,
  // 1 down, 2 dh, 3 dx): bit 5 + p set = 256-row tiles (else 320), bit 9 + p
  // set = 32-k ring stages (else 64-k)
  ENG_TILE256 = 1u << 5,
  ENG_STAGE32 = 1u << 9,
  // rows per split-K chunk of the LoRA gradients: field value 0 = 2048,
  // 1 = 1024, 2 = 4096
  ENG_SPLITK_SHIFT = 13,
  ENG_SPLITK_MASK = 3u << 13,
  ENG_VALID = (1u << 15) - 1
};
constexpr int SPLITK_MIN = 1024, SPLITK_MAX = 4096;
inline int splitk_rows(uint32_t engines) {
  const uint32_t f = (engines & ENG_SPLITK_MASK) >> ENG_SPLITK_SHIFT;
  return f == 1 ? 1024 : f == 2 ? 4096 : 2048;
}
inline bool engines_valid(uint32_t engines) {
  return (engines & ~(uint32_t)ENG_VALID) == 0 && (engines & ENG_SPLITK_MASK) != ENG_SPLITK_MASK;
}

struct Layer {
  int T, d, n, E, k, r, S, Et;
  int f16;           // elements are fp16 (else bf16)
  int lora;          // the split low-rank pass runs (0: forward on merged weights)
  uint32_t engines;  // EngineBits
  int rs;       // row stride of the rank-r activations (r rounded up to 8)
  int ra;       // row stride used to read A_gu / A_dn (r, or rs for the packed copies)
  int P, Ptot;  // routed pairs, all rows
  int splitk;   // rows per split-K chunk of the LoRA gradients (splitk_rows(engines))
  float s;      // LoRA scale
  int ncu;      // compute units of the device (persistent grid sizing)
  // routing
  const int32_t* topk_ids;
  const float* topk_w;
  const int32_t* offsets;
  const int32_t* sorted_pair;
  const int32_t* pair_pos;
  // weights
  const bf16_t* w_gu;  // [Et, 2n, d]
  const bf16_t* w_dn;  // [Et, d, n]
  const bf16_t* a_gu;  // [Et, d, ra]
  const bf16_t* b_gu;  // [Et, r, 2n]
  const bf16_t* a_dn;  // [Et, n, ra]
  const bf16_t* b_dn;  // [Et, r, d]
  // activations
  const bf16_t* x;   // [T, d]
  const bf16_t* dy;  // [T, d]
  bf16_t* g;         // [Ptot, 2n]  saved
  bf16_t* h;         // [Ptot, n]   saved
  bf16_t* xa;        // [Ptot, rs]  saved
  bf16_t* ha;        // [Ptot, rs]  saved
  bf16_t* o;         // [Ptot, d]   forward: O; backward: dX per pair
  bf16_t* dg;        // [Ptot, 2n]
  bf16_t* qdn;       // [Ptot, rs]
  bf16_t* qgu;       // [Ptot, rs]
  bf16_t* hw;        // [Ptot, rs]  w * s H A_dn (dB_dn operand)
  bf16_t* qw;        // [Ptot, rs]  w * Q_dn (dA_dn operand)
  float* dw_part;    // [Ptot, n / 64] partial <dH, H> per 64-column group, or null
  int dw_groups;     // n / 64
  bf16_t* y;         // [T, d]
  bf16_t* dx;        // [T, d]
  float* da_gu;      // [Et, d, r]
  float* db_gu;      // [Et, r, 2n]
  float* da_dn;      // [Et, n, r]
  float* db_dn;      // [Et, r, d]
  float* partial;    // split-K partial sums of the LoRA gradients
  float* pre_partial;  // split-K partial sums of the rank-r pre-passes [split][Ptot][rs]
  int64_t partial_off[4];  // float offset of each gradient's partial slots
  const int32_t* tok;      // [Ptot] token of each sorted row (routing's gather table)
  const float* wgt;        // [Ptot] routing weight of each sorted row (1 for shared)
};

// Shape (M x N) of the four LoRA gradients: 0 dB_dn [r,d], 1 dA_dn [n,r],
// 2 dB_gu [r,2n], 3 dA_gu [d,r].
__host__ __device__ inline void grad_shape(int kind, int d, int n, int r, int& M, int& N) {
  M = kind == 0 ? r : kind == 1 ? n : kind == 2 ? r : d;
  N = kind == 0 ? d : kind == 1 ? r : kind == 2 ? 2 * n : r;
}

// Workspace carving shared by the size query and the launchers.
struct WsLayout {
  size_t o, dg, qdn, qgu, hw, qw, dw_part, partial, pre_partial, a_gu_pack, a_dn_pack, total;
  int64_t partial_off[4];
};
struct SavedLayout {
  size_t g, h, xa, ha, total;
};
WsLayout ws_layout(int64_t T, int d, int n, int E, int k, int r, int S);
SavedLayout saved_layout(int64_t T, int d, int n, int E, int k, int r, int S);

size_t route_ws_bytes(int64_t T, int E, int k);
hipError_t launch_route(const float* logits, int64_t T, int E, int k, int S, int32_t* ids, float* w,
                        int32_t* counts, int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos,
                        int32_t* row_token, float* row_weight, void* ws, hipStream_t st);

// Rank-r pre-pass kinds: s X A_gu, s H A_dn, s dY B_dn^T, s dG B_gu^T.
enum PrepassKind { PRE_XA = 0, PRE_HA = 1, PRE_QDN = 2, PRE_QGU = 3 };

// Launchers that depend on the element type, declared for both builds (the
// sources are compiled once with bf16 and once with fp16 elements, into
// moe::el_bf16 and moe::el_f16; code of one build calls its own unqualified).
#define MOE_ELEMENT_LAUNCHERS                                                                     \
  /* grouped GEMMs with their rank-r pre-pass (gemm.hip) */                                       \
  hipError_t gemm_gate_up(const Layer& L, hipStream_t st);    /* G, H (+ X A_gu) */                \
  hipError_t gemm_down(const Layer& L, hipStream_t st);       /* O (+ H A_dn) */                   \
  hipError_t gemm_dh(const Layer& L, hipStream_t st);         /* dG (+ dO B_dn^T) */               \
  hipError_t gemm_dx(const Layer& L, hipStream_t st);         /* dX per pair (+ dG B_gu^T) */      \
  hipError_t gemm_lora_grads(const Layer& L, hipStream_t st); /* dA, dB of both modules */         \
  uint32_t default_engines(); /* the engines used when none was chosen for a shape */             \
  /* whether the Q_dn pre-pass also writes w Q_dn and w (s H A_dn) (the streamed one does) */     \
  bool prepass_writes_weighted_rows(const Layer& L);                                              \
  /* streamed products without their pre-pass, in the tile configuration   */                    \
  /* the layer's engine bits choose (gemm.hip, over the builds of stream.hip) */                   \
  hipError_t stream_gate_up(const Layer& L, hipStream_t st);                                      \
  hipError_t stream_down(const Layer& L, hipStream_t st);                                         \
  hipError_t stream_dx(const Layer& L, hipStream_t st);                                           \
  hipError_t stream_dh(const Layer& L, hipStream_t st);                                           \
  /* streamed rank-r pre-passes, rs <= 64 (prepass.hip) */                                        \
  hipError_t stream_prepass(const Layer& L, int kind, hipStream_t st);                            \
  /* LDS-DMA LoRA gradients, rank <= 64 (grads.hip) */                                            \
  hipError_t dma_lora_grads(const Layer& L, hipStream_t st);                                      \
  /* W + s (A B)^T of every expert, both modules (merge.hip) */                                   \
  hipError_t merge_lora(const Layer& L, const bf16_t* a_gu, const bf16_t* a_dn, bf16_t* w_gu_out,   \
                        bf16_t* w_dn_out, hipStream_t st);                                          \
  /* weighted gather-combine of per-pair rows into token rows (combine.hip) */                   \
  hipError_t launch_combine(const Layer& L, bool weighted, const bf16_t* src, bf16_t* dst,        \
                            hipStream_t st);

// stream.hip, built once per tile height x stage depth
#define MOE_STREAM_LAUNCHERS                                    \
  hipError_t stream_gate_up(const Layer& L, hipStream_t st);    \
  hipError_t stream_down(const Layer& L, hipStream_t st);       \
  hipError_t stream_dx(const Layer& L, hipStream_t st);         \
  hipError_t stream_dh(const Layer& L, hipStream_t st);
#define MOE_STREAM_TILES             \
  namespace t320k64 { MOE_STREAM_LAUNCHERS } \
  namespace t256k64 { MOE_STREAM_LAUNCHERS } \
  namespace t320k32 { MOE_STREAM_LAUNCHERS } \
  namespace t256k32 { MOE_STREAM_LAUNCHERS }

inline namespace MOE_EL {
MOE_ELEMENT_LAUNCHERS
MOE_STREAM_TILES
}
#ifdef MOE_F16
namespace el_bf16 {
MOE_ELEMENT_LAUNCHERS
MOE_STREAM_TILES
}
#else
namespace el_f16 {
MOE_ELEMENT_LAUNCHERS
MOE_STREAM_TILES
}
#endif

// Kernels that do not depend on the element type (layer.hip).
hipError_t launch_pack_a(const Layer& L, const bf16_t* a_gu_src, const bf16_t* a_dn_src,
                         bf16_t* a_gu_dst, bf16_t* a_dn_dst, hipStream_t st);
// Routing-weight and logit gradients from the dh epilogue's partials.
hipError_t launch_router_grad(const Layer& L, float* d_topk_w, float* d_logits, hipStream_t st);
// Shape -> engines table (tune.hip): a recorded choice, else default_engines().
uint32_t lookup_engines(int d, int n, int E, int k, int r, int S, int f16);
void record_engines(int d, int n, int E, int k, int r, int S, int f16, uint32_t engines);

int device_cu_count();

// Kernel launch through the optional event-timing recorder (timing.hip).
void timing_pre(const char* name, hipStream_t st);
void timing_post(hipStream_t st);
#define MOE_LAUNCH(name, kernel, grid, block, lds, stream, ...)              \
  do {                                                                       \
    ::moe::timing_pre(name, stream);                                         \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);       \
    ::moe::timing_post(stream);                                              \
  } while (0)

constexpr int PREPASS_MAX_SPLIT = 4;

// Contraction splits of a rank-r pre-pass: enough row tiles x splits to give
// every CU about two workgroups, at most PREPASS_MAX_SPLIT, each split at
// least 4 K steps of 64.
inline int prepass_splits(int Ptot, int Et, int K, int ncu) {
  const int mt = Ptot / 128 + Et;
  // split only when the row tiles alone would leave most CUs idle
  if (mt * 2 >= ncu) return 1;
  int s = (2 * ncu + mt - 1) / mt;
  s = s < 1 ? 1 : s > PREPASS_MAX_SPLIT ? PREPASS_MAX_SPLIT : s;
  while (s > 1 && (K / 64) / s < 4) --s;
  return s;
}

}  // namespace moe
