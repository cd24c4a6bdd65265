// FP8 (OCP E4M3) linear layers for the QKV and projection GEMMs: per-row
// quantisation of an activation or weight matrix, and the scaled product on
// the 8-bit float matrix cores.
//
// Pages: "Boosting Swin Transformer Speed", Inference Optimization (the QKV and
// projection GEMMs run in 8 bits with per-channel scales; here the MI355X's
// native 8-bit float takes the place of the 8-bit integers).
//
// Format: E4M3 with exponent bias 7, 3 mantissa bits, largest finite 448,
// subnormals k * 2^-9, no infinities.  Quantisation of a row: amax = max |x|,
// scale = amax / 448, inv = 448 / amax (1 and 1 for a zero row), code =
// E4M3(x * inv) rounded to nearest, ties to even, after clamping to +-448; the
// sign bit is set exactly when x * inv < 0.  All of it in float32.
#include "launch.hpp"

namespace swin {

namespace {

// E4M3 code of v (clamped to +-448), to nearest, ties to even.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const float a = fminf(fabsf(v), 448.0f);
  uint32_t c;
  if (a < 0.015625f) {
    // Below 2^-6: multiples of 2^-9 (code 8 is 2^-6, the smallest normal).
    c = (uint32_t)rintf(a * 512.0f);
  } else {
    // Round the 23-bit mantissa to 3 bits (ties to even); a carry moves into
    // the exponent.  Exponent field = float exponent - 127 + 7.
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    c = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  }
  return v < 0.0f ? (c | 0x80u) : c;
}

// One wave per row: the row's absolute maximum, then its codes.
template <typename T>
__global__ __launch_bounds__(256) void fp8_quant_kernel(const T* __restrict__ x, int rows, int K,
                                                        uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // no workgroup barrier below
  const T* xr = x + (int64_t)row * K;
  float m = 0.f;
  for (int k = lane; k < K; k += 64) m = fmaxf(m, fabsf((float)xr[k]));
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
  const float scale = m > 0.f ? m / 448.0f : 1.0f;
  const float inv = m > 0.f ? 448.0f / m : 1.0f;
  uint8_t* cr = codes + (int64_t)row * K;
  for (int k = lane; k < K; k += 64) cr[k] = (uint8_t)e4m3_code((float)xr[k] * inv);
  if (lane == 0) scales[row] = scale;
}

// Y[r][n] = (sum_k A[r][k] W[n][k]) * sa[r] * sw[n] + bias[n], A and W as E4M3
// codes with K contiguous.  64 x 64 tile per workgroup of 4 waves, 32 x 32 per
// wave; each 16 x 16 tile is a chain of 16x16x32 8-bit float products whose
// fragments (lane l: row l % 16, k = 8 (l/16) .. +7, 8 bytes) load straight
// from memory.
template <typename TO>
__global__ __launch_bounds__(256) void fp8_linear_kernel(Fp8Linear p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32;
  const int n0 = blockIdx.x * 64 + (wave & 1) * 32;
  const int64_t ra[2] = {m0 + i16, m0 + 16 + i16};
  const int nb[2] = {n0 + i16, n0 + 16 + i16};
  const uint8_t* ap[2];
  const uint8_t* wp[2];
  bool aok[2], wok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    aok[i] = ra[i] < p.rows;
    wok[i] = nb[i] < p.N;
    ap[i] = p.a + (aok[i] ? ra[i] : 0) * p.K + 8 * g4;
    wp[i] = p.w + (int64_t)(wok[i] ? nb[i] : 0) * p.K + 8 * g4;
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < p.K; k += 32) {
    long af[2], wf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      af[i] = aok[i] ? *reinterpret_cast<const long*>(ap[i] + k) : 0L;
      wf[i] = wok[i] ? *reinterpret_cast<const long*>(wp[i] + k) : 0L;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(af[i], wf[j], acc[i][j], 0, 0, 0);
  }
  // Lane l holds column l % 16 of rows 4 (l / 16) .. +3 of each tile.
  TO* y = static_cast<TO*>(p.y);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = nb[j];
    if (n >= p.N) continue;
    const float sw = p.sw[n];
    const float b = p.bias ? ld_any(p.bias, p.bias_type, n) : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + 16 * i + 4 * g4 + r;
        if (m >= p.rows) continue;
        y[m * p.N + n] = from_f32<TO>(acc[i][j][r] * p.sa[m] * sw + b);
      }
  }
}

}  // namespace

hipError_t launch_fp8_quant(const void* x, int io, int rows, int K, uint8_t* codes, float* scales,
                            hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4), block(256);
  if (io == kF32)
    hipLaunchKernelGGL(fp8_quant_kernel<float>, grid, block, 0, st, static_cast<const float*>(x),
                       rows, K, codes, scales);
  else if (io == kF16)
    hipLaunchKernelGGL(fp8_quant_kernel<h16>, grid, block, 0, st, static_cast<const h16*>(x), rows,
                       K, codes, scales);
  else
    hipLaunchKernelGGL(fp8_quant_kernel<b16>, grid, block, 0, st, static_cast<const b16*>(x), rows,
                       K, codes, scales);
  return hipGetLastError();
}

hipError_t launch_fp8_linear(const Fp8Linear& p, int out_io, hipStream_t st) {
  if (p.rows <= 0) return hipSuccess;
  if (p.K % 32) return hipErrorInvalidValue;
  const dim3 grid((p.N + 63) / 64, (unsigned)((p.rows + 63) / 64)), block(256);
  if (out_io == kF32)
    hipLaunchKernelGGL(fp8_linear_kernel<float>, grid, block, 0, st, p);
  else if (out_io == kF16)
    hipLaunchKernelGGL(fp8_linear_kernel<h16>, grid, block, 0, st, p);
  else
    hipLaunchKernelGGL(fp8_linear_kernel<b16>, grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace swin
