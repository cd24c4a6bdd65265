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

// The same with 8 elements per lane and step (K % 8 == 0, x 16-byte and codes
// 8-byte aligned): 16- or 32-byte loads, 8-byte code stores.
template <typename T>
__global__ __launch_bounds__(256) void fp8_quant8_kernel(const T* __restrict__ x, int rows, int K,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // no workgroup barrier below
  const T* xr = x + (int64_t)row * K;
  auto load = [&](int c, float (&v)[8]) {
    if constexpr (sizeof(T) == 4) {
      const float4 a = *reinterpret_cast<const float4*>(xr + 8 * c);
      const float4 b = *reinterpret_cast<const float4*>(xr + 8 * c + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      const vec8<T> a = gload8(xr + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (float)a[e];
    }
  };
  const int nc = K / 8;
  float m = 0.f;
  for (int c = lane; c < nc; c += 64) {
    float v[8];
    load(c, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
  const float scale = m > 0.f ? m / 448.0f : 1.0f;
  const float inv = m > 0.f ? 448.0f / m : 1.0f;
  uint8_t* cr = codes + (int64_t)row * K;
  for (int c = lane; c < nc; c += 64) {
    float v[8];
    load(c, v);
    uint2 packed = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      packed.x |= e4m3_code(v[e] * inv) << (8 * e);
      packed.y |= e4m3_code(v[4 + e] * inv) << (8 * e);
    }
    *reinterpret_cast<uint2*>(cr + 8 * c) = packed;
  }
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

// The same product for K a multiple of 128 on the gfx950 16x16x128 8-bit
// float products (unit block scales).  128 x 128 tile per workgroup of 4
// waves (64 x 64 each, 16 accumulator tiles); K in steps of 128 through LDS
// (rows padded to 144 bytes), the next step's 16-byte chunks loaded into
// registers during the current step.  A lane's fragment is 32 consecutive
// bytes of one row; A and W use the same placement, so each product pairs
// equal k.
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kF8T = 128, kF8K = 128, kF8P = 144;

template <typename TO>
__global__ __launch_bounds__(256) void fp8_linear_tiled_kernel(Fp8Linear p) {
  __shared__ __attribute__((aligned(16))) uint8_t as[kF8T * kF8P];
  __shared__ __attribute__((aligned(16))) uint8_t ws[kF8T * kF8P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g4 = lane >> 4;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int64_t m0 = (int64_t)blockIdx.y * kF8T;
  const int n0 = blockIdx.x * kF8T;
  // Staging: chunk c = tid + 256 i (i < 4) is row c / 8, bytes 16 (c % 8).
  uint4 ra[4], rw[4];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, cc = c & 7;
      const int64_t m = m0 + row;
      const int n = n0 + row;
      ra[i] = m < p.rows ? *reinterpret_cast<const uint4*>(p.a + m * p.K + kb + 16 * cc)
                         : uint4{0u, 0u, 0u, 0u};
      rw[i] = n < p.N ? *reinterpret_cast<const uint4*>(p.w + (int64_t)n * p.K + kb + 16 * cc)
                      : uint4{0u, 0u, 0u, 0u};
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i, row = c >> 3, cc = c & 7;
      *reinterpret_cast<uint4*>(&as[row * kF8P + 16 * cc]) = ra[i];
      *reinterpret_cast<uint4*>(&ws[row * kF8P + 16 * cc]) = rw[i];
    }
  };
  auto frag = [&](const uint8_t* base, int row) {
    const uint4 lo = *reinterpret_cast<const uint4*>(base + row * kF8P + 32 * g4);
    const uint4 hi = *reinterpret_cast<const uint4*>(base + row * kF8P + 32 * g4 + 16);
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  fetch(0);
  stage();
  __syncthreads();
  for (int kb = 0; kb < p.K; kb += kF8K) {
    const bool more = kb + kF8K < p.K;
    if (more) fetch(kb + kF8K);
    i32x8 af[4], wf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      af[t] = frag(as, wm + 16 * t + i16);
      wf[t] = frag(ws, wn + 16 * t + i16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], wf[j], acc[i][j], 0, 0,
                                                                     0, 127, 0, 127);
    __syncthreads();  // every wave done reading this step
    if (more) {
      stage();
      __syncthreads();
    }
  }
  TO* y = static_cast<TO*>(p.y);
  float sa[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + wm + 16 * i + 4 * g4 + r;
      sa[i][r] = m < p.rows ? p.sa[m] : 0.f;
    }
  if constexpr (sizeof(TO) == 2) {
    // 16-bit output: the wave's 64 x 64 tile goes through LDS (rows of 144
    // bytes; waves 0, 1 in the A buffer, 2, 3 in the W buffer; every read of
    // both ended at the loop's last barrier) and leaves as 16-byte row chunks.
    uint8_t* tile = (wave < 2 ? as : ws) + (wave & 1) * 64 * kF8P;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + 16 * j + i16;
      const float sw = n < p.N ? p.sw[n] : 0.f;
      const float b = (p.bias && n < p.N) ? ld_any(p.bias, p.bias_type, n) : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<TO*>(&tile[(16 * i + 4 * g4 + r) * kF8P + 2 * (16 * j + i16)]) =
              from_f32<TO>(acc[i][j][r] * sa[i][r] * sw + b);
    }
    asm volatile("" ::: "memory");  // the wave's tile writes before its reads
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int c = lane + 64 * q, row = c >> 3, cc = c & 7;
      const int64_t m = m0 + wm + row;
      const int n = n0 + wn + 8 * cc;
      if (m >= p.rows || n >= p.N) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(&tile[row * kF8P + 16 * cc]);
      if (n + 8 <= p.N && (reinterpret_cast<uintptr_t>(y + m * p.N + n) & 15) == 0) {
        *reinterpret_cast<uint4*>(y + m * p.N + n) = v;
      } else {
        const TO* e = reinterpret_cast<const TO*>(&v);
        for (int k = 0; k < 8 && n + k < p.N; ++k) y[m * p.N + n + k] = e[k];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn + 16 * j + i16;
      if (n >= p.N) continue;
      const float sw = p.sw[n];
      const float b = p.bias ? ld_any(p.bias, p.bias_type, n) : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t m = m0 + wm + 16 * i + 4 * g4 + r;
          if (m >= p.rows) continue;
          y[m * p.N + n] = from_f32<TO>(acc[i][j][r] * sa[i][r] * sw + b);
        }
    }
  }
}

}  // namespace

hipError_t launch_fp8_quant(const void* x, int io, int rows, int K, uint8_t* codes, float* scales,
                            hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((rows + 3) / 4), block(256);
  if (K % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(codes) & 7) == 0) {
    if (io == kF32)
      hipLaunchKernelGGL(fp8_quant8_kernel<float>, grid, block, 0, st,
                         static_cast<const float*>(x), rows, K, codes, scales);
    else if (io == kF16)
      hipLaunchKernelGGL(fp8_quant8_kernel<h16>, grid, block, 0, st, static_cast<const h16*>(x),
                         rows, K, codes, scales);
    else
      hipLaunchKernelGGL(fp8_quant8_kernel<b16>, grid, block, 0, st, static_cast<const b16*>(x),
                         rows, K, codes, scales);
    return hipGetLastError();
  }
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
  if (fp8_tiled_supported(p)) return launch_fp8_tiled(p, out_io, st);
  if (p.K % kF8K == 0) {
    const dim3 grid((p.N + kF8T - 1) / kF8T, (unsigned)((p.rows + kF8T - 1) / kF8T)), block(256);
    if (out_io == kF32)
      hipLaunchKernelGGL(fp8_linear_tiled_kernel<float>, grid, block, 0, st, p);
    else if (out_io == kF16)
      hipLaunchKernelGGL(fp8_linear_tiled_kernel<h16>, grid, block, 0, st, p);
    else
      hipLaunchKernelGGL(fp8_linear_tiled_kernel<b16>, grid, block, 0, st, p);
    return hipGetLastError();
  }
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
