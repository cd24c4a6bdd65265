// General matrix-core GEMM tile shared by the projection GEMMs of the
// attention (gemm.hip) and the MLP of the full block (block.hip): 128 rows x BN
// columns of A * Wt^T, K in steps of 32, operands staged through padded LDS with
// a register prefetch of the next step.
//
// "Boost Vision Transformer with GPU-Friendly Sparsity and Quantization",
// Section 3.2 / Figure 3: the Q, K, V and output projections and the
// feed-forward layers of the transformer block are GEMMs.
#pragma once

#include "common.hpp"

namespace swin {

constexpr int kBM = 128;     // rows per workgroup (4 waves x 32 rows)
constexpr int kBK = 32;      // K per step = one 16x16x32 operand slice
constexpr int kThreads = 256;

template <typename T, int BN>
struct GemmSmem {
  static constexpr int LD = kBK + 16 / (int)sizeof(T);  // row pitch, padded by 16 bytes
  T a[kBM * LD];
  T b[BN * LD];
};

// acc[i][j] += A[m0 + wave*32 + 16i .., :] * Wt[n0 + 16j .., :]^T over all K.
// A row r is token src_token(r) of A when GATHER, else row r.  Rows >= rows are
// clamped to the last valid row (computed, never stored).
template <typename T, int BN, bool GATHER>
__device__ __forceinline__ void gemm_tile(const T* __restrict__ A, const Geom& g, int rows, int m0,
                                          const T* __restrict__ Wt, int n0, int K,
                                          GemmSmem<T, BN>& sm, f32x4 (&acc)[2][BN / 16]) {
  constexpr int E = sizeof(T);
  constexpr int LD = GemmSmem<T, BN>::LD;
  constexpr int CPR = kBK * E / 16;  // 16-byte chunks per row per K step
  constexpr int RPP = kThreads / CPR;
  constexpr int APASS = kBM / RPP;
  constexpr int BPASS = (BN + RPP - 1) / RPP;
  constexpr int EPC = 16 / E;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int cr = tid / CPR, cc = tid % CPR;

  const T* arow[APASS];
#pragma unroll
  for (int p = 0; p < APASS; ++p) {
    int r = m0 + cr + p * RPP;
    if (r >= rows) r = rows - 1;
    int64_t src = GATHER ? src_token(g, r) : (int64_t)r;
    arow[p] = A + src * K + cc * EPC;
  }
  const T* brow[BPASS];
  bool bval[BPASS];
#pragma unroll
  for (int p = 0; p < BPASS; ++p) {
    int n = cr + p * RPP;
    bval[p] = n < BN;
    brow[p] = Wt + (int64_t)(n0 + (bval[p] ? n : 0)) * K + cc * EPC;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < BN / 16; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 ra[APASS], rb[BPASS];
#pragma unroll
  for (int p = 0; p < APASS; ++p) ra[p] = *reinterpret_cast<const uint4*>(arow[p]);
#pragma unroll
  for (int p = 0; p < BPASS; ++p)
    if (bval[p]) rb[p] = *reinterpret_cast<const uint4*>(brow[p]);

  for (int k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < APASS; ++p)
      *reinterpret_cast<uint4*>(&sm.a[(cr + p * RPP) * LD + cc * EPC]) = ra[p];
#pragma unroll
    for (int p = 0; p < BPASS; ++p)
      if (bval[p]) *reinterpret_cast<uint4*>(&sm.b[(cr + p * RPP) * LD + cc * EPC]) = rb[p];
    __syncthreads();
    if (k0 + kBK < K) {
#pragma unroll
      for (int p = 0; p < APASS; ++p)
        ra[p] = *reinterpret_cast<const uint4*>(arow[p] + k0 + kBK);
#pragma unroll
      for (int p = 0; p < BPASS; ++p)
        if (bval[p]) rb[p] = *reinterpret_cast<const uint4*>(brow[p] + k0 + kBK);
    }
    vec8<T> af[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      af[i] = load8(&sm.a[(wave * 32 + i * 16 + (lane & 15)) * LD + (lane >> 4) * 8]);
#pragma unroll
    for (int j = 0; j < BN / 16; ++j) {
      vec8<T> bf = load8(&sm.b[(j * 16 + (lane & 15)) * LD + (lane >> 4) * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i) acc[i][j] = mma_16x16x32(af[i], bf, acc[i][j]);
    }
  }
}

}  // namespace swin
