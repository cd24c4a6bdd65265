// QKV projection and output projection GEMMs on the gfx950 matrix cores.
//
// "Boost Vision Transformer with GPU-Friendly Sparsity and Quantization",
// Section 3.2 / Figure 3: the Q, K, V projections and the output projection of
// the attention module are GEMMs.  "Boosting Swin Transformer Speed", Inference
// Optimization: the QKV GEMM carries its bias and no transposes are left; the
// shift / partition / reverse index maps are fused into the neighbouring ops.
//
// Both GEMMs compute rows of tokens times nn.Linear weights ([out, in], K
// contiguous on both sides).  The QKV GEMM reads its A rows through the cyclic
// shift + window partition map (each row is one contiguous token vector in x),
// and stores q, k, v per (window, head) block, so the attention kernel reads
// contiguous [N, 32] tiles.  The projection GEMM writes each window-order row
// back to its un-shifted position.
#include "gemm_core.hpp"
#include "launch.hpp"

namespace swin {

// ---------------------------------------------------------------------------
// QKV projection.  Output tile 128 tokens x 96 channels; 3C is a multiple of 96
// because C is a multiple of 32.  Each 32-column group is one head of one of
// q / k / v, so the V2 per-head L2 norm is a 16-lane reduction.
// ---------------------------------------------------------------------------
template <typename T, typename QT>
__global__ __launch_bounds__(kThreads) void qkv_gemm_kernel(FwdParams p) {
  constexpr int BN = 96;
  __shared__ GemmSmem<T, BN> sm;
  const Geom g = p.g;
  const int rows = g.B * g.H * g.W;
  const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * BN;
  const int C = g.C;
  f32x4 acc[2][BN / 16];
  gemm_tile<T, BN, true>(static_cast<const T*>(p.x), g, rows, m0, static_cast<const T*>(p.w_qkv),
                         n0, C, sm, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const T* bq = static_cast<const T*>(p.b_qkv);
#pragma unroll
  for (int j = 0; j < BN / 16; ++j) {
    float bias = bq ? (float)bq[n0 + j * 16 + (lane & 15)] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] += bias;
  }
#pragma unroll
  for (int jp = 0; jp < BN / 32; ++jp) {
    const int col0 = n0 + jp * 32;
    const int part = col0 / C;  // 0 = q, 1 = k, 2 = v
    const int h = (col0 - part * C) >> 5;
    float mult[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) mult[i][r] = 1.0f;
    if (part < 2 && p.v2) {
      // "Swin Transformer V2" summary, How It Works: cosine similarity of q and
      // k scaled by 1/tau (tau clipped at tau_min); the 1/tau and log2(e) of the
      // base-2 softmax are folded into q.
      const float qm = kLog2e / fmaxf(p.tau[h], p.tau_min);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float a0 = acc[i][2 * jp][r], a1 = acc[i][2 * jp + 1][r];
          float ss = a0 * a0 + a1 * a1;
          ss += __shfl_xor(ss, 1);
          ss += __shfl_xor(ss, 2);
          ss += __shfl_xor(ss, 4);
          ss += __shfl_xor(ss, 8);
          float inv = 1.0f / fmaxf(sqrtf(ss), p.eps);
          mult[i][r] = part == 0 ? inv * qm : inv;
        }
    } else if (part == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) mult[i][r] = p.q_mult;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wave * 32 + i * 16 + (lane >> 4) * 4 + r;
        if (row >= rows) continue;
        const int w = row / g.N;
        const int t = row - w * g.N;
        const int64_t base = ((int64_t)(w * g.heads + h) * g.N + t) * 32 + (lane & 15);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          float v = acc[i][2 * jp + jj][r] * mult[i][r];
          if (part == 0)
            static_cast<QT*>(p.buf.q)[base + 16 * jj] = from_f32<QT>(v);
          else if (part == 1)
            static_cast<QT*>(p.buf.k)[base + 16 * jj] = from_f32<QT>(v);
          else
            static_cast<T*>(p.buf.v)[base + 16 * jj] = from_f32<T>(v);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Output projection; the store is the window reverse + inverse shift.
// ---------------------------------------------------------------------------
template <typename T, int BN>
__global__ __launch_bounds__(kThreads) void proj_gemm_kernel(FwdParams p) {
  __shared__ GemmSmem<T, BN> sm;
  const Geom g = p.g;
  const int rows = g.B * g.H * g.W;
  const int m0 = blockIdx.x * kBM, n0 = blockIdx.y * BN;
  const int C = g.C;
  f32x4 acc[2][BN / 16];
  gemm_tile<T, BN, false>(static_cast<const T*>(p.buf.o), g, rows, m0,
                          static_cast<const T*>(p.w_proj), n0, C, sm, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const T* bp = static_cast<const T*>(p.b_proj);
  T* y = static_cast<T*>(p.y);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wave * 32 + i * 16 + (lane >> 4) * 4 + r;
      if (row >= rows) continue;
      const int64_t dst = src_token(g, row) * C;
#pragma unroll
      for (int j = 0; j < BN / 16; ++j) {
        const int col = n0 + j * 16 + (lane & 15);
        float bias = bp ? (float)bp[col] : 0.0f;
        y[dst + col] = from_f32<T>(acc[i][j][r] + bias);
      }
    }
}

template <typename T>
static hipError_t qkv_dispatch(const FwdParams& p, hipStream_t st) {
  const int rows = p.g.B * p.g.H * p.g.W;
  dim3 grid((rows + kBM - 1) / kBM, 3 * p.g.C / 96);
  if (p.qk == kF16)
    hipLaunchKernelGGL((qkv_gemm_kernel<T, h16>), grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((qkv_gemm_kernel<T, T>), grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_qkv_gemm(const FwdParams& p, hipStream_t st) {
  switch (p.io) {
    case kF32: return qkv_dispatch<float>(p, st);
    case kF16: return qkv_dispatch<h16>(p, st);
    default: return qkv_dispatch<b16>(p, st);
  }
}

template <typename T>
static hipError_t proj_dispatch(const FwdParams& p, hipStream_t st) {
  const int rows = p.g.B * p.g.H * p.g.W;
  const int C = p.g.C;
  const int gx = (rows + kBM - 1) / kBM;
  if (C % 128 == 0)
    hipLaunchKernelGGL((proj_gemm_kernel<T, 128>), dim3(gx, C / 128), dim3(kThreads), 0, st, p);
  else if (C % 96 == 0)
    hipLaunchKernelGGL((proj_gemm_kernel<T, 96>), dim3(gx, C / 96), dim3(kThreads), 0, st, p);
  else if (C % 64 == 0)
    hipLaunchKernelGGL((proj_gemm_kernel<T, 64>), dim3(gx, C / 64), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL((proj_gemm_kernel<T, 32>), dim3(gx, C / 32), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_proj_gemm(const FwdParams& p, hipStream_t st) {
  switch (p.io) {
    case kF32: return proj_dispatch<float>(p, st);
    case kF16: return proj_dispatch<h16>(p, st);
    default: return proj_dispatch<b16>(p, st);
  }
}

}  // namespace swin
