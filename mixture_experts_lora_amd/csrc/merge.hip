// Merged LoRA weights, the path split LoRA avoids (faster-MoE page, "Faster
// LoRA MoE training" and "MoE LoRA changes things": PEFT forms the adapter
// delta of every expert and adds it to the base weight before the grouped
// product).  For each expert e:
//   W'_gu[e] = W_gu[e] + s (A_gu[e] B_gu[e])^T    [2n, d]
//   W'_dn[e] = W_dn[e] + s (A_dn[e] B_dn[e])^T    [d, n]
// i.e. W'[row][col] = W[row][col] + s sum_q B[q][row] A[col][q], rounded once
// to the element type.
//
// The pass is a stream of W (read once, written once).  One workgroup takes
// a strip of 128 columns of one expert: the strip's slice of A ([col][q]) goes
// to LDS once, then the strip runs down its rows 64 at a time.  For each row
// tile the B slice ([row][q]) is transposed into LDS, four waves form the
// 64 x 128 delta with v_mfma_f32_32x32x16 (K = r padded to 16 with zeros) and
// stage s * delta in LDS, and W is read, updated and written as whole
// 16-byte row chunks.  The next row tile's W and B chunks are loaded into
// registers while the current tile computes.
#include "common.h"
#include "kernels.h"

namespace moe {
inline namespace MOE_EL {
namespace {

constexpr int MR = 64, MC = 128, MNT = 256;       // row tile, column strip, threads
constexpr int MWC = MR * MC / 8 / MNT;            // 16-byte W chunks per thread and row tile (4)
constexpr int MBC = 128 * MR / 8 / MNT;           // 16-byte B chunks per thread and row tile, r <= 128 (4)

__global__ __launch_bounds__(MNT) void k_merge(const bf16_t* __restrict__ W, const bf16_t* __restrict__ B,
                                               const bf16_t* __restrict__ A, bf16_t* __restrict__ Wo,
                                               int R, int C, int r, float s) {
  extern __shared__ __attribute__((aligned(16))) unsigned char mg_smem[];
  const int rp = (r + 15) & ~15;  // K padded to the MFMA depth
  const int ld = rp + 8;          // LDS row length of the factor slices (16-byte aligned rows)
  bf16_t* as = (bf16_t*)mg_smem;                // [MC][ld]  A[col0 + col][q]
  bf16_t* bs = as + MC * ld;                    // [MR][ld]  B[q][row0 + row]
  float* dl = (float*)(bs + MR * ld);           // [MR][MC + 4]  s * delta
  constexpr int DLD = MC + 4;
  const int e = blockIdx.y;
  const int col0 = blockIdx.x * MC;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const bf16_t* we = W + (int64_t)e * R * C;
  bf16_t* wo = Wo + (int64_t)e * R * C;
  const bf16_t* be = B + (int64_t)e * r * R;
  const bf16_t* ae = A + (int64_t)e * C * r;

  // the strip's A slice, once (16-byte loads when A's rows are 16-byte aligned)
  if ((r & 7) == 0) {
    const int cpr = rp / 8;
    for (int i = tid; i < MC * cpr; i += MNT) {
      const int col = i / cpr, q8 = (i - col * cpr) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (q8 < r && col0 + col < C) v = *(const uint4*)(ae + (int64_t)(col0 + col) * r + q8);
      *(uint4*)(as + col * ld + q8) = v;
    }
  } else {
    for (int i = tid; i < MC * rp; i += MNT) {
      const int col = i / rp, q = i - col * rp;
      as[col * ld + q] = (q < r && col0 + col < C) ? ae[(int64_t)(col0 + col) * r + q] : (bf16_t)0;
    }
  }

  // chunk j of a thread: W chunk tid + j MNT = (row, 8 columns); B chunk
  // tid + j MNT = (q, 8 rows)
  uint4 wv[MWC], bv[MBC];
  auto load = [&](int row0) {
#pragma unroll
    for (int j = 0; j < MWC; ++j) {
      const int c = tid + j * MNT, row = c / (MC / 8), c8 = (c % (MC / 8)) * 8;
      const bool ok = row0 + row < R && col0 + c8 < C;
      wv[j] = ok ? *(const uint4*)(we + (int64_t)(row0 + row) * C + col0 + c8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < MBC; ++j) {
      const int c = tid + j * MNT, q = c / (MR / 8), r8 = (c % (MR / 8)) * 8;
      const bool ok = q < r && row0 + r8 < R;
      bv[j] = ok ? *(const uint4*)(be + (int64_t)q * R + row0 + r8) : make_uint4(0, 0, 0, 0);
    }
  };
  const int wm = wid >> 1, wn = wid & 1;  // wave: rows 32 wm, columns 64 wn
  load(0);
#pragma unroll 1
  for (int row0 = 0; row0 < R; row0 += MR) {
    // B slice of this tile, transposed into [row][q]
#pragma unroll
    for (int j = 0; j < MBC; ++j) {
      const int c = tid + j * MNT, q = c / (MR / 8), r8 = (c % (MR / 8)) * 8;
      if (q < rp) {
        const uint32_t u[4] = {bv[j].x, bv[j].y, bv[j].z, bv[j].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          bs[(r8 + 2 * h) * ld + q] = (bf16_t)(u[h] & 0xffffu);
          bs[(r8 + 2 * h + 1) * ld + q] = (bf16_t)(u[h] >> 16);
        }
      }
    }
    uint4 wcur[MWC];
#pragma unroll
    for (int j = 0; j < MWC; ++j) wcur[j] = wv[j];
    __syncthreads();
    if (row0 + MR < R) load(row0 + MR);  // the next tile's chunks, under this tile's work
    f32x16 acc[2] = {(f32x16)(0.0f), (f32x16)(0.0f)};
    for (int k0 = 0; k0 < rp; k0 += 16) {
      const int kq = k0 + 8 * (lane >> 5);
      const uint4 a = *(const uint4*)(bs + (32 * wm + (lane & 31)) * ld + kq);
#pragma unroll
      for (int fn = 0; fn < 2; ++fn) {
        const uint4 b = *(const uint4*)(as + (64 * wn + 32 * fn + (lane & 31)) * ld + kq);
        acc[fn] = mfma32(b, a, acc[fn]);
      }
    }
    // lane: row 32 wm + lane % 32, columns 64 wn + 32 fn + 8 g + 4 (lane / 32) + 0..3
#pragma unroll
    for (int fn = 0; fn < 2; ++fn)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          dl[(32 * wm + (lane & 31)) * DLD + 64 * wn + 32 * fn + 8 * g + 4 * (lane >> 5) + j] = s * acc[fn][4 * g + j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < MWC; ++j) {
      const int c = tid + j * MNT, row = c / (MC / 8), c8 = (c % (MC / 8)) * 8;
      if (row0 + row >= R || col0 + c8 >= C) continue;
      const uint32_t u[4] = {wcur[j].x, wcur[j].y, wcur[j].z, wcur[j].w};
      const float* dr = dl + row * DLD + c8;
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = pack2(bf2f((bf16_t)(u[q] & 0xffffu)) + dr[2 * q], bf2f((bf16_t)(u[q] >> 16)) + dr[2 * q + 1]);
      *(uint4*)(wo + (int64_t)(row0 + row) * C + col0 + c8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    __syncthreads();  // bs and dl are rewritten by the next tile
  }
}

hipError_t merge_one(const bf16_t* W, const bf16_t* B, const bf16_t* A, bf16_t* Wo, int Et, int R, int C,
                     int r, float s, const char* name, hipStream_t st) {
  const int ld = ((r + 15) & ~15) + 8;
  const size_t lds = (size_t)(MC + MR) * ld * 2 + (size_t)MR * (MC + 4) * 4;
  MOE_LAUNCH(name, k_merge, dim3(cdiv(C, MC), Et), dim3(MNT), lds, st, W, B, A, Wo, R, C, r, s);
  return hipGetLastError();
}

}  // namespace

hipError_t merge_lora(const Layer& L, const bf16_t* a_gu, const bf16_t* a_dn, bf16_t* w_gu_out,
                      bf16_t* w_dn_out, hipStream_t st) {
  hipError_t e = merge_one(L.w_gu, L.b_gu, a_gu, w_gu_out, L.Et, 2 * L.n, L.d, L.r, L.s, "merge_gate_up", st);
  if (e == hipSuccess) e = merge_one(L.w_dn, L.b_dn, a_dn, w_dn_out, L.Et, L.d, L.n, L.r, L.s, "merge_down", st);
  return e;
}

}  // inline namespace MOE_EL
}  // namespace moe
